"""Host logic of bench.py on the CPU: the counter reductions behind the
roofline's `traffic`, the choice of the roofline kernel, and the refusal of
more than one GPU."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

ATTN = "_ZN6vitenc12_GLOBAL__N_120attention_lds_kernelIDF16bLi64ELi4ELi4EEEvPKT_(args)"
UP = "_ZN6vitenc12_GLOBAL__N_115gemm_lds_kernelIDF16bLi256ELi256ELi2ELi4ELi8ELi2ELi32ELi1ELb0EEEvPKT_(args)"
RESID = "_ZN6vitenc12_GLOBAL__N_115gemm_lds_kernelIDF16bLi128ELi128ELi2ELi2ELi16ELi2ELi32ELi2ELb0EEEvPKT_(args)"
COPY = "__amd_rocclr_copyBuffer"
TORCH_COPY = "void at::native::elementwise_kernel<copy, float, int>(args)"
SMALL_COPY = "void at::native::elementwise_kernel<copy, bf16>(args)"


def _write_csv(path, counter, seq):
    """rocprofv3 counter_collection.csv rows: one per (dispatch, counter)."""
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                                           "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for i, (k, v) in enumerate(seq):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": k, "Counter_Name": counter, "Counter_Value": v,
                        "Start_Timestamp": 1000 * i, "End_Timestamp": 1000 * i + 500})


# two layers (attention, out, up, down), a copy between dispatches, then the
# back-to-back launches of the shared kernel alone (an odd number of them),
# then one more layer: only dispatches right after attention count as out,
# only those right after the up projection as down
SEQ = [(ATTN, 1.0), (RESID, 10.0), (UP, 2.0), (RESID, 100.0),
       (ATTN, 1.0), (COPY, 5.0), (RESID, 12.0), (UP, 2.0), (COPY, 5.0), (RESID, 102.0),
       (RESID, 999.0), (RESID, 999.0), (RESID, 999.0),
       (ATTN, 1.0), (RESID, 14.0), (UP, 2.0), (RESID, 104.0)]


def test_counter_means_by_predecessor(tmp_path):
    p = tmp_path / "c.csv"
    _write_csv(p, "FETCH_SIZE", SEQ)
    out = bench.counter_means(str(p), "FETCH_SIZE", bench.SHARED_DISPATCH["out_gemm"])
    down = bench.counter_means(str(p), "FETCH_SIZE", bench.SHARED_DISPATCH["down_gemm"])
    assert out[RESID] == (12.0, 3)
    assert down[RESID] == (102.0, 3)
    every = bench.counter_means(str(p), "FETCH_SIZE")
    assert every[RESID][1] == 9 and every[ATTN] == (1.0, 3)
    # every second dispatch of the shared kernel would have mixed them up
    resid = [v for k, v in SEQ if k == RESID]
    assert sum(resid[1::2]) / len(resid[1::2]) != 102.0


def _counters(tmp_path, fetch_kib, write_kib, copy_fetch_kib, copy_write_kib):
    f, w = tmp_path / "fetch.csv", tmp_path / "write.csv"
    layer = lambda v: [(ATTN, 3.0), (RESID, 1.0), (UP, 4.0), (RESID, v)]
    _write_csv(f, "FETCH_SIZE", layer(fetch_kib) * 3 + [(TORCH_COPY, copy_fetch_kib), (SMALL_COPY, 7.0), (TORCH_COPY, copy_fetch_kib)])
    _write_csv(w, "WRITE_SIZE", layer(write_kib) * 3 + [(TORCH_COPY, copy_write_kib)])
    out = tmp_path / "down_gemm_unit_counters.txt"
    bench.write_counters("down_gemm", str(f), str(w), str(out))
    return out


def test_traffic_from_counter_summary(tmp_path):
    copy_kib = bench.COPY_BYTES / 1024
    # the calibration copy (the copy kernel with the largest reading) reads half its
    # bytes on FETCH_SIZE (factor 2) and all of them on WRITE_SIZE
    out = _counters(tmp_path, 1000.0, 300.0, copy_kib / 2, copy_kib)
    t = bench.read_traffic("down_gemm", "unit", path=str(out))
    assert t == pytest.approx((2 * 1000.0 + 300.0) * 1024)


def test_traffic_null_when_sources_changed(tmp_path):
    copy_kib = bench.COPY_BYTES / 1024
    out = _counters(tmp_path, 1000.0, 300.0, copy_kib / 2, copy_kib)
    text = out.read_text()
    h = bench.sources_hash(bench.KERNEL_SOURCES["down_gemm"][1])
    assert f"source_sha256_16: {h}" in text
    out.write_text(text.replace(h, "0" * 16))
    assert bench.read_traffic("down_gemm", "unit", path=str(out)) is None
    assert bench.read_traffic("down_gemm", "no_such_workload") is None


def test_roofline_takes_the_largest_alone_time():
    # name: (ms in the layer sequence, flops, bytes, ms alone)
    bd = {"layernorm": (0.008, 0.0, 25.2e6, 0.030),   # twice per layer: 0.060
          "attention": (0.049, 34.36e9, 33.5e6, 0.047),
          "down_gemm": (0.050, 34.36e9, 75.5e6, 0.046)}
    roof = bench.roofline_of(bd, "no_such_workload")
    assert roof["kernel"] == "layernorm" and roof["bound"] == "hbm"
    assert roof["achieved"] == pytest.approx(25.2e6 / 0.030e-3 / 1e9, rel=1e-3)
    del bd["layernorm"]
    roof = bench.roofline_of(bd, "no_such_workload")
    assert roof["kernel"] == "attention" and roof["bound"] == "mfma"
    assert roof["avg_launch_ms"] == pytest.approx(0.047) and roof["in_layer_ms"] == pytest.approx(0.049)
    assert roof["achieved"] == pytest.approx(34.36e9 / 0.047e-3 / 1e12, rel=1e-3)
    assert roof["frac"] == pytest.approx(roof["achieved"] / bench.PEAK_BF16_TFLOPS, rel=1e-3)
    assert roof["traffic"] is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
