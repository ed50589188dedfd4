"""Throughput of the ViT encoder forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--graph] [--no-cpu-baseline]
                    [--part all|encoder|predictor|head|variants|configs|weights8]
    python bench.py --write-counters KERNEL FETCH.csv WRITE.csv OUT.txt


A step is one vitenc_encode call over one batch: the V-JEPA-2-style ViT-L
video encoder, 2 clips x 16 frames x 3 x 256 x 256 -> 2 x 2048 tokens, 24
layers, bf16 with fp32 accumulation, synthetic seeded inputs resident in HBM.
Prints one JSON line.  The roofline object is measured for the dominant
kernel by timing its step entry point (the same kernel and launch
configuration encode uses) with HIP events on the stream it is launched on:
its launches back to back between one event pair, weights rotating over the
layers, which is what a rocprofv3 kernel trace of `--only KERNEL` measures
(`in_layer_ms` is the time of one launch bracketed by its own event pair
inside the layer sequence, dispatch latency included).
The line's `predictor` object times the masked-latent predictor that follows
the encoder (one vitenc_predict call per step) the same way, with its own
roofline and oracle baseline; `head` does the same for the attentive-pool
classifier head (one vitenc_head_forward call per step); `variants` times
encoder options on their own inputs (a resampled position table, the one-frame
image tokenizer with hierarchical outputs); `all_configs` times every encoder
workload; `weights8` compares 8-bit block weights with bf16 weights on the
ViT-L/16 image encoder.  `--part NAME` prints that object alone (the counter
runs of their kernels use it).

Its `traffic` figure comes from a committed counter summary (written by the
--write-counters mode from two rocprofv3 --pmc runs of this script: one
collecting FETCH_SIZE, one WRITE_SIZE).  Each counter is scaled by what it
reads for a plain 256 MiB device copy timed in the same run, and the figure is
reported only while the kernel's sources still hash to what was profiled.
"""
from __future__ import annotations

import argparse
import csv
import re
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# Peaks, recomputed from the device's reported CU count and peak clock by
# device_peaks(): dense bf16 MFMA 4096 flop per clock per CU (256 CU x 2.4 GHz
# x 4096 = 2516.6 TFLOP/s on MI355X), fp32 256 flop per clock per CU
# (157.3 TFLOP/s); HBM3E 8 TB/s as published (not derivable from attributes).
BF16_FLOP_PER_CLK_CU = 4096
FP32_FLOP_PER_CLK_CU = 256
PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0
PEAK_FP32_TFLOPS = 157.3
PEAK_SOURCE = {"cus": 256, "clock_ghz": 2.4, "from": "published MI355X figures"}
# hipDeviceAttribute_t values of the HIP runtime API (hip_runtime_api.h)
_HIP_ATTR_CLOCK_RATE_KHZ = 5
_HIP_ATTR_CU_COUNT = 63


def device_peaks():
    """Set the MFMA peaks from the device's CU count and peak clock (HIP
    device attributes) and return the figures used."""
    global PEAK_BF16_TFLOPS, PEAK_FP32_TFLOPS, PEAK_SOURCE
    import ctypes
    import torch
    torch.cuda.init()
    hip = ctypes.CDLL("libamdhip64.so")
    dev = torch.cuda.current_device()
    clk, cus = ctypes.c_int(0), ctypes.c_int(0)
    if (hip.hipDeviceGetAttribute(ctypes.byref(clk), _HIP_ATTR_CLOCK_RATE_KHZ, dev) != 0 or
            hip.hipDeviceGetAttribute(ctypes.byref(cus), _HIP_ATTR_CU_COUNT, dev) != 0 or clk.value <= 0):
        return PEAK_SOURCE
    ghz = clk.value / 1e6
    PEAK_BF16_TFLOPS = round(cus.value * BF16_FLOP_PER_CLK_CU * ghz / 1e3, 1)
    PEAK_FP32_TFLOPS = round(cus.value * FP32_FLOP_PER_CLK_CU * ghz / 1e3, 1)
    PEAK_SOURCE = {"cus": cus.value, "clock_ghz": ghz, "bf16_flop_per_clk_per_cu": BF16_FLOP_PER_CLK_CU,
                   "fp32_flop_per_clk_per_cu": FP32_FLOP_PER_CLK_CU, "from": "hipDeviceGetAttribute (peak clock)"}
    return PEAK_SOURCE


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None
COPY_BYTES = 256 << 20        # plain device copy used to calibrate the HBM byte counters
CSRC = os.path.join(ROOT, "vision_transformer_amd", "csrc")
# kernel-breakdown name -> (pattern of its device kernel's mangled name, sources it is compiled from).
# The GEMM epilogue is the second-to-last template argument of gemm_lds_kernel (STORE 0, GELU 1,
# RESID 2, PATCH 3, QKV 4; the last one is the 8-bit weight flag); the out and down projections
# share the RESID instantiation.
KERNEL_SOURCES = {
    "attention": (r"attention_lds_kernel", ["attention.hip", "common.h", "launch.h"]),
    "qkv_gemm": (r"gemm_lds_kernel.*Li4ELb0EEEv", ["gemm.hip", "common.h", "launch.h"]),
    "up_gemm": (r"gemm_lds_kernel.*Li1ELb0EEEv", ["gemm.hip", "common.h", "launch.h"]),
    "down_gemm": (r"gemm_lds_kernel.*Li2ELb0EEEv", ["gemm.hip", "common.h", "launch.h"]),
    "out_gemm": (r"gemm_lds_kernel.*Li2ELb0EEEv", ["gemm.hip", "common.h", "launch.h"]),
    "layernorm": (r"layernorm", ["elementwise.hip", "common.h", "launch.h"]),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--graph", action="store_true", help="replay the step as a captured HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--only", metavar="KERNEL", default=None,
                    help="launch only this kernel of the encoder layer (a kernel-breakdown name) --kernel-reps "
                         "times at the headline shape and exit (for counter runs)")
    ap.add_argument("--part", choices=("all", "encoder", "predictor", "head", "variants", "configs", "weights8"),
                    default="all",
                    help="what to time: the encoder (the headline line), the predictor or the attentive-pool "
                         "head (reported in the line's `predictor` / `head` objects), or all three")
    ap.add_argument("--sq-summary", metavar="COUNTER_CSV", default=None,
                    help="print per-kernel MFMA / VALU / LDS utilisation from a rocprofv3 --pmc pass over the "
                         "SQ counters of this script")
    ap.add_argument("--workload", default=None,
                    help="with --part configs: time only the encoder workload of this name")
    ap.add_argument("--write-counters", nargs=4, metavar=("KERNEL", "FETCH_CSV", "WRITE_CSV", "OUT_TXT"),
                    help="summarise two rocprofv3 --pmc counter_collection.csv files of this script "
                         "for KERNEL (a kernel-breakdown name)")
    return ap.parse_args()


def sources_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# kernels that share one device instantiation: the kernel whose dispatch comes right before each
# of theirs (copies aside) in a layer: the out projection follows attention, the down projection
# follows the up projection (dispatches after anything else, such as the back-to-back launches
# of one kernel alone, are left out)
SHARED_DISPATCH = {"out_gemm": r"attention_lds_kernel", "down_gemm": r"gemm_lds_kernel.*Li1ELb0EEEv"}


def counter_means(path, counter, follows=None):
    """{kernel name: (mean counter value, dispatches)} from a rocprofv3 counter csv; with
    `follows` (a pattern) only the dispatches whose preceding dispatch, copies aside, is of a
    kernel matching it."""
    seq = []
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] == counter:
                seq.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    seq.sort()
    out, prev = {}, None
    for _, k, v in seq:
        if follows is None or (prev is not None and re.search(follows, prev.split("(")[0])):
            out.setdefault(k, []).append(v)
        if "copy" not in k.split("(")[0].lower():
            prev = k
    return {k: (sum(v) / len(v), len(v)) for k, v in out.items()}


SQ_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_INSTS_VALU",
               "SQ_INSTS_MFMA", "SQ_INSTS_VALU_TRANS_F32", "SQ_LDS_BANK_CONFLICT", "SQ_BUSY_CYCLES")


def sq_summary(csv_path, clock_ghz=2.4, cus=256, simds=1024):
    """Per-kernel utilisation from one rocprofv3 --pmc pass over SQ_COUNTERS
    (+ GRBM_GUI_ACTIVE) of this script: means per dispatch of the MFMA-busy
    cycles over all SIMDs, the VALU- and LDS-active cycles summed over waves
    (quad-cycles, scaled by 4) per CU, and the instruction counts, each
    against the dispatch's duration at the quoted clock."""
    import collections
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    dur = collections.defaultdict(dict)
    with open(csv_path) as fh:
        for r in csv.DictReader(fh):
            k = r["Kernel_Name"]
            vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
            dur[k][r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    lines = ["kernel           dispatches  us    mfma_busy  valu_active  lds_active   valu_insts  mfma_insts"
             "  trans_insts  lds_bank_conflicts"]
    for name, (pattern, _) in KERNEL_SOURCES.items():
        if name == "out_gemm":
            continue
        ks = [k for k in vals if re.search(pattern, k.split("(")[0])]
        if not ks:
            continue
        c, d = vals[ks[0]], dur[ks[0]]
        mean = lambda n: sum(c[n]) / len(c[n])
        ns = sum(d.values()) / len(d)
        cyc = ns * clock_ghz
        label = "out+down_gemm" if name == "down_gemm" else name
        lines.append(f"{label:16s} {len(d):10d} {ns / 1000:5.1f} {mean('SQ_VALU_MFMA_BUSY_CYCLES') / (simds * cyc):10.3f}"
                     f" {4 * mean('SQ_ACTIVE_INST_VALU') / (cus * cyc):12.3f}"
                     f" {4 * mean('SQ_ACTIVE_INST_LDS') / (cus * cyc):11.3f}"
                     f" {mean('SQ_INSTS_VALU'):12.4g} {mean('SQ_INSTS_MFMA'):11.4g}"
                     f" {mean('SQ_INSTS_VALU_TRANS_F32'):12.4g} {mean('SQ_LDS_BANK_CONFLICT'):19.4g}")
    print("\n".join(lines))


def write_counters(dominant, fetch_csv, write_csv, out_txt):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the dominant kernel and of
    the calibration copy, plus the hash of the kernel's sources."""
    pattern, files = KERNEL_SOURCES[dominant]
    lines = [f"kernel: {dominant}", f"device_kernel_pattern: {pattern}", f"sources: {' '.join(files)}",
             f"source_sha256_16: {sources_hash(files)}", f"copy_bytes: {COPY_BYTES}"]
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        means = counter_means(path, counter)
        shared = counter_means(path, counter, SHARED_DISPATCH.get(dominant))
        kern = [(k, shared[k]) for k in shared if re.search(pattern, k.split("(")[0])]
        copy = [(k, v) for k, v in means.items() if "copy" in k.split("(")[0].lower()]
        if not kern or not copy:
            raise SystemExit(f"{path}: no {pattern} or copy dispatches with {counter}")
        # the copy with the largest reading is the 256 MiB calibration copy
        ck, (cv, cn) = max(copy, key=lambda kv: kv[1][0])
        if len(kern) > 1:
            raise SystemExit(f"{path}: {pattern} matches {len(kern)} kernels")
        kk, (kv, kn) = kern[0]
        lines += [f"{counter}_KiB_per_dispatch: {kv:.1f}", f"{counter}_dispatches: {kn}",
                  f"{counter}_kernel: {kk.split('(')[0][:160]}",
                  f"copy_{counter}_KiB_per_dispatch: {cv:.1f}", f"copy_{counter}_dispatches: {cn}"]
    with open(out_txt, "a") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def read_traffic(dominant, workload, path=None):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary (or the summary at `path`), or None if there is none or the
    kernel changed since."""
    path = path or os.path.join(ROOT, "profiles", f"{dominant}_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    _, files = KERNEL_SOURCES[dominant]
    if kv.get("kernel") != dominant or kv.get("source_sha256_16") != sources_hash(files):
        return None
    total = 0.0
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        scale = float(kv["copy_bytes"]) / (float(kv[f"copy_{c}_KiB_per_dispatch"]) * 1024.0)
        total += float(kv[f"{c}_KiB_per_dispatch"]) * 1024.0 * scale
    return total


def kernel_breakdown(cfg, enc, reps, stream, busy, only=None):
    """The kernels of one encoder layer, launched in encode's order through
    their C-ABI entry points at the encode shapes, each bracketed by a pair of
    HIP events on `stream`.  Repetition r uses the weights of layer r mod L,
    so that, as inside encode, each launch streams weights the previous ones
    did not; the RoPE table is filled once, as encode does.  `busy()` queues a
    few full encode steps first so that the GPU is still working while the
    host queues the layer sequences: each event pair then brackets the kernel
    alone.  Returns {name: (ms per launch in the layer sequence, flops, bytes,
    ms per launch alone)}."""
    import torch
    from vision_transformer_amd import vitenc as V
    B, N, D, F, H = cfg.batch, cfg.n_tokens, cfg.embed_dim, cfg.ffn_dim, cfg.n_head
    hd = D // H
    M = B * N
    dt = cfg.dtype
    td = V.torch_dtype(dt)
    dev = "cuda"
    g = torch.Generator(device=dev).manual_seed(0)
    Z = torch.randn((M, D), device=dev, generator=g)
    Y = torch.empty((M, D), device=dev, dtype=td)
    O = torch.empty((M, D), device=dev, dtype=td)
    U = torch.empty((M, F), device=dev, dtype=td)
    blk0 = enc.blocks[0]
    tab = V.op_rope_table(hd, cfg.grid, cfg.rope_layout, cfg.rope_interpolate, cfg.rope_ref_grid, cfg.rope_theta)
    Q, K, Vt = V.op_qkv_rope(dt, Y.normal_(generator=g), blk0["qkv_w"], blk0["qkv_b"], B, N, H, rope=cfg.rope,
                             grid=cfg.grid, n_prefix=cfg.n_prefix,
                             outs=(torch.empty((B, H, N, hd), dtype=td, device=dev),
                                   torch.empty((B, H, N, hd), dtype=td, device=dev),
                                   torch.zeros((B, H, hd, (N + 63) // 64 * 64), dtype=td, device=dev), tab),
                             table_ready=True)
    torch.cuda.synchronize()
    es = 2
    pairs = cfg.visible_pairs() * B * H
    work = {
        "layernorm": (0.0, M * D * (4 + es) + 8 * D),
        "qkv_gemm": (2.0 * M * D * 3 * D, (M * D + 3 * D * D + 3 * M * D) * es),
        "attention": (4.0 * hd * pairs, 4 * M * D * es),
        "out_gemm": (2.0 * M * D * D, (M * D + D * D) * es + 8 * M * D),
        "up_gemm": (2.0 * M * D * F, (M * D + F * D + M * F) * es),
        "down_gemm": (2.0 * M * F * D, (M * F + D * F) * es + 8 * M * D),
    }

    def layer(blk):
        return [
            ("layernorm", lambda: V.op_layernorm(Z, blk["ln1_w"], blk["ln1_b"], cfg.ln_eps, dt, out=Y)),
            ("qkv_gemm", lambda: V.op_qkv_rope(dt, Y, blk["qkv_w"], blk["qkv_b"], B, N, H, rope=cfg.rope,
                                               grid=cfg.grid, n_prefix=cfg.n_prefix, outs=(Q, K, Vt, tab),
                                               table_ready=True)),
            ("attention", lambda: V.op_attention(dt, Q, K, Vt, cfg.attn_mode, cfg.n_prefix,
                                                 cfg.grid[1] * cfg.grid[2], out=O)),
            ("out_gemm", lambda: V.op_linear_residual(dt, O, blk["out_w"], blk["out_b"], Z, ls=blk.get("ls1"))),
            ("layernorm", lambda: V.op_layernorm(Z, blk["ln2_w"], blk["ln2_b"], cfg.ln_eps, dt, out=Y)),
            ("up_gemm", lambda: V.op_linear_gelu(dt, Y, blk["up_w"], blk["up_b"], out=U)),
            ("down_gemm", lambda: V.op_linear_residual(dt, U, blk["down_w"], blk["down_b"], Z, ls=blk.get("ls2"))),
        ]

    seqs = [layer(enc.blocks[r % len(enc.blocks)]) for r in range(reps)]
    if only is not None:
        busy()
        for seq in seqs:
            for name, fn in seq:
                if name == only:
                    fn()
        torch.cuda.synchronize()
        return {}
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in seq] for seq in seqs]
    first, last = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    busy()
    first.record(stream)
    for seq, evs in zip(seqs, ev):
        for (name, fn), (e0, e1) in zip(seq, evs):
            e0.record(stream)
            fn()
            e1.record(stream)
    last.record(stream)
    torch.cuda.synchronize()
    acc, cnt = {}, {}
    for seq, evs in zip(seqs, ev):
        for (name, _), (e0, e1) in zip(seq, evs):
            acc[name] = acc.get(name, 0.0) + e0.elapsed_time(e1)
            cnt[name] = cnt.get(name, 0) + 1
    log(f"[bench] layer sequence: kernels {sum(acc.values()):.3f} ms of {first.elapsed_time(last):.3f} ms span "
        f"over {reps} layers")
    res = {name: (acc[name] / cnt[name],) + work[name] for name in acc}
    # Each kernel also alone: its `reps` launches back to back (weights of
    # layer r mod L, as above) between one event pair, which is what a
    # rocprofv3 kernel trace of `--only NAME` measures.  The event pairs
    # around single launches above also hold each launch's dispatch latency.
    alone = {}
    for name in res:
        fns = [fn for seq in seqs for nm, fn in seq if nm == name][:reps]
        busy()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        for fn in fns:
            fn()
        a1.record(stream)
        torch.cuda.synchronize()
        alone[name] = a0.elapsed_time(a1) / len(fns)
    log("[bench] each kernel alone, back to back (ms): " + ", ".join(f"{k}={v:.4f}" for k, v in alone.items()))
    res = {name: v + (alone[name],) for name, v in res.items()}
    # calibration for the HBM byte counters: a plain device copy of known size
    # (fp32 -> int32 keeps the element size, so torch launches its own copy kernel)
    src = torch.empty(COPY_BYTES // 4, device=dev, dtype=torch.float32).fill_(1.0)
    dst = torch.empty(COPY_BYTES // 4, device=dev, dtype=torch.int32)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    return res


def cpu_baseline(cfg, wl, layers=None):
    """The oracle (unchanged, float64 numpy) on one clip through `layers`
    layers (default: all of them), scaled to the full depth if fewer."""
    import oracle
    cores = _oracle_cores()
    layers = layers or cfg.n_layer
    one = cfg.replace(batch=1)
    px = wl.pixels[:1]
    t0 = time.perf_counter()
    Z = oracle.embed(one, wl.weights, px)
    t1 = time.perf_counter()
    rope_pos, vis = oracle.rope_and_mask(one, px.shape)
    for blk in wl.weights.blocks[:layers]:
        Z = oracle.encoder_block(Z, blk, one, rope_pos, vis)
    t2 = time.perf_counter()
    out = oracle.layer_norm(Z, wl.weights.norm_w, wl.weights.norm_b, one.ln_eps)
    t3 = time.perf_counter()
    per_clip = (t1 - t0) + (t2 - t1) * cfg.n_layer / layers + (t3 - t2)
    return {"value": round(one.n_tokens / per_clip, 3), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"1 of {cfg.batch} clips ({one.n_tokens} tokens), patch embed + {layers} of {cfg.n_layer} "
                      f"layers + final norm, {t3 - t0:.1f} s"}


class PredictorShape:
    """The predictor's blocks as kernel_breakdown sees them: B items of
    n_ctx + n_tgt tokens, full attention, 3-D RoPE on the grid, no prefix."""

    def __init__(self, cfg):
        self.name, self.batch, self.n_tokens = cfg.name, cfg.batch, cfg.n_tokens
        self.embed_dim, self.ffn_dim, self.n_head, self.dtype = cfg.embed_dim, cfg.ffn_dim, cfg.n_head, cfg.dtype
        self.grid, self.rope_layout, self.rope_theta, self.ln_eps = cfg.grid, cfg.rope_layout, cfg.rope_theta, cfg.ln_eps
        self.rope, self.rope_interpolate, self.rope_ref_grid, self.n_prefix, self.attn_mode = 1, 0, 0, 0, 0
        # the timed step ops put the tokens at the grid positions in order, which needs a full grid
        assert cfg.n_tokens == cfg.n_grid

    def visible_pairs(self):
        return self.n_tokens * self.n_tokens


def cpu_baseline_predictor(cfg, wl):
    """The predictor oracle (unchanged) on the whole workload: every item
    through every block (a few seconds of float64 work)."""
    import oracle
    cores = _oracle_cores()
    t0 = time.perf_counter()
    oracle.predictor_forward(cfg.hparams(), wl.weights, wl.enc_tokens, wl.ctx_ids, wl.tgt_ids, cfg.mask_index)
    dt = time.perf_counter() - t0
    return {"value": round(cfg.batch * cfg.n_tokens / dt, 3), "unit": "tokens/s", "cores": int(cores),
            "cpu_model": cpu_model(),
            "kind": "oracle", "sample": f"the whole workload ({cfg.batch} items x {cfg.n_tokens} tokens, "
                                        f"{cfg.n_layer} blocks), {dt:.1f} s"}


def _oracle_cores():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return os.cpu_count() or 1


def roofline_of(bd, workload):
    """The roofline object of the kernel that takes the most time in one
    forward (layernorm runs twice per block), timed alone: its launches back
    to back between one event pair, as a rocprofv3 kernel trace of
    `bench.py --only KERNEL` measures it; the time of each launch inside the
    layer sequence (with its dispatch latency) is reported beside it."""
    weight = {"layernorm": 2}
    dom = max(bd, key=lambda k: bd[k][3] * weight.get(k, 1))
    in_layer_ms, d_flops, d_bytes, d_ms = bd[dom]
    if d_flops > 0:
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(d_flops / (d_ms * 1e-3) / 1e12, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(d_bytes / (d_ms * 1e-3) / 1e9, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["avg_launch_ms"] = round(d_ms, 5)
    roof["timing"] = "launches back to back, weights of layer r mod L"
    roof["in_layer_ms"] = round(in_layer_ms, 5)
    traffic = read_traffic(dom, workload)
    roof["traffic"] = None if traffic is None else round(traffic / 1e6, 2)
    roof["traffic_unit"] = "MB per launch"
    roof["algorithmic_bytes"] = round(d_bytes / 1e6, 2)
    return roof


def time_steps(step, steps, warmup, stream, per_call=None):
    """Mean ms per step over `steps` back-to-back steps bracketed by one
    event pair (and the host wall time).  With per_call a list, an event pair
    also brackets every call on the same stream and the list receives each
    call's ms (their median and minimum are reported beside the mean)."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)] \
        if per_call is not None else None
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        if evs:
            evs[i][0].record(stream)
        step()
        if evs:
            evs[i][1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    if evs:
        per_call.extend(e0.elapsed_time(e1) for e0, e1 in evs)
    return start.elapsed_time(end) / steps, t_wall * 1e3 / steps


def bench_predictor(args, stream):
    """One vitenc_predict call per step on the full predictor shape: 2 items x
    (1024 context + 1024 target) tokens of the 8 x 16 x 16 grid, 12 blocks of
    width 384, bf16; ids and encoder features resident on the device."""
    import torch
    from vision_transformer_amd import vitenc as V
    from vision_transformer_amd import workloads as W
    cfg = W.PREDICTOR
    log(f"[bench] predictor {cfg.name}: B={cfg.batch} ctx={cfg.n_ctx} tgt={cfg.n_tgt} D={cfg.embed_dim} "
        f"L={cfg.n_layer}")
    wl = W.make_predictor_workload(cfg)
    pred = V.Predictor.from_workload(wl)
    V.check_pred_ids(wl.ctx_ids, wl.tgt_ids, cfg.n_grid)
    enc = torch.from_numpy(wl.enc_tokens).cuda()
    ctx = torch.from_numpy(wl.ctx_ids).cuda()
    tgt = torch.from_numpy(wl.tgt_ids).cuda()
    ws, out = pred.alloc(cfg.batch, cfg.n_ctx, cfg.n_tgt)

    def step():
        pred.predict_into(enc, ctx, tgt, ws, out, cfg.mask_index, stream, check_ids=False)

    ms, wall = time_steps(step, args.steps, args.warmup, stream)
    tflops = cfg.flops() / (ms * 1e-3) / 1e12
    log(f"[bench] predictor {ms:.3f} ms/call, {tflops:.1f} TFLOP/s (wall {wall:.3f} ms/call)")

    def busy():
        for _ in range(8):
            step()

    bd = kernel_breakdown(PredictorShape(cfg), pred, args.kernel_reps, stream, busy)
    log("[bench] predictor per-kernel (ms): " + ", ".join(f"{k}={v[0]:.4f}" for k, v in bd.items()))
    res = {"workload": cfg.name, "ms_per_call": round(ms, 4),
           "tokens_per_s": round(cfg.batch * cfg.n_tokens / ms * 1e3, 1),
           "target_tokens_per_s": round(cfg.batch * cfg.n_tgt / ms * 1e3, 1),
           "tflops": round(tflops, 2), "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
           "config": {"global_batch": cfg.batch, "n_ctx": cfg.n_ctx, "n_tgt": cfg.n_tgt, "grid": list(cfg.grid),
                      "embed_dim": cfg.embed_dim, "enc_dim": cfg.enc_dim, "layers": cfg.n_layer,
                      "heads": cfg.n_head},
           "kernels_ms_per_layer": {k: round(v[0], 5) for k, v in bd.items()},
           "kernels_ms_alone": {k: round(v[3], 5) for k, v in bd.items()},
           "roofline": roofline_of(bd, cfg.name), "cpu_baseline": None}
    if not args.no_cpu_baseline:
        log("[bench] predictor cpu baseline (oracle) ...")
        res["cpu_baseline"] = cpu_baseline_predictor(cfg, wl)
        log(f"[bench] predictor cpu baseline {res['cpu_baseline']}")
    pred.close()
    return res


class HeadShape:
    """The attentive-pool head's pooler blocks as kernel_breakdown sees them:
    B items of N tokens, full attention, no RoPE, no prefix."""

    def __init__(self, cfg):
        self.name, self.batch, self.n_tokens = cfg.name, cfg.batch, cfg.n_tokens
        self.embed_dim, self.ffn_dim, self.n_head, self.dtype = cfg.embed_dim, cfg.ffn_dim, cfg.n_head, cfg.dtype
        self.ln_eps = cfg.ln_eps
        self.grid, self.rope_layout, self.rope_theta = (1, 1, 1), 0, 10000.0
        self.rope, self.rope_interpolate, self.rope_ref_grid, self.n_prefix, self.attn_mode = 0, 0, 0, 0, 0

    def visible_pairs(self):
        return self.n_tokens * self.n_tokens


def head_xattn_bytes(cfg):
    """Algorithmic HBM bytes of the cross-attention and the tail: the tokens
    read twice (scores, then weighted sums), the q, k, v, fc1, fc2 and
    classifier weights once, the pooled and logit outputs."""
    B, N, D, F, C = cfg.batch, cfg.n_tokens, cfg.embed_dim, cfg.ffn_dim, cfg.n_classes
    es = 4 if cfg.dtype == 0 else 2
    return 2 * B * N * D * 4 + (3 * D * D + 2 * D * F + C * D) * es + B * (D + C) * 4


def cpu_baseline_head(cfg, wl):
    """The head oracle (unchanged) on the whole workload."""
    import oracle
    cores = _oracle_cores()
    t0 = time.perf_counter()
    oracle.attentive_pool_forward(cfg.hparams(), wl.weights, wl.tokens)
    dt = time.perf_counter() - t0
    return {"value": round(cfg.batch * cfg.n_tokens / dt, 3), "unit": "tokens/s", "cores": int(cores),
            "cpu_model": cpu_model(),
            "kind": "oracle", "sample": f"the whole workload ({cfg.batch} items x {cfg.n_tokens} tokens, "
                                        f"{cfg.n_pool_layers} pooler blocks + cross-attention + classifier), "
                                        f"{dt:.1f} s"}


def bench_head(args, stream):
    """One vitenc_head_forward call per step on the V-JEPA 2 ViT-L classifier
    head over the 2 x 2048 output tokens of two clips (3 pooler blocks, 174
    classes, bf16).  The cross-attention and tail are also timed alone (a
    second handle without pooler blocks over the same weights)."""
    import torch
    from vision_transformer_amd import vitenc as V
    from vision_transformer_amd import workloads as W
    cfg = W.HEAD
    log(f"[bench] head {cfg.name}: B={cfg.batch} N={cfg.n_tokens} D={cfg.embed_dim} L={cfg.n_pool_layers} "
        f"classes={cfg.n_classes}")
    wl = W.make_head_workload(cfg)
    head = V.Head.from_workload(wl)
    bare = V.Head(dict(head.hp, n_pool_layers=0), head.tensors, [])
    tok = torch.from_numpy(wl.tokens).cuda()
    ws, pooled, logits = head.alloc(cfg.batch, cfg.n_tokens)
    ws0, pooled0, logits0 = bare.alloc(cfg.batch, cfg.n_tokens)

    def step():
        head.forward_into(tok, ws, pooled, logits, stream)

    def step_bare():
        bare.forward_into(tok, ws0, pooled0, logits0, stream)

    ms, wall = time_steps(step, args.steps, args.warmup, stream)
    ms_x, _ = time_steps(step_bare, args.steps, args.warmup, stream)
    tflops = cfg.flops() / (ms * 1e-3) / 1e12
    log(f"[bench] head {ms:.3f} ms/call ({ms_x * 1e3:.1f} us without pooler blocks), {tflops:.1f} TFLOP/s")

    def busy():
        for _ in range(4):
            step()

    bd = kernel_breakdown(HeadShape(cfg), head, args.kernel_reps, stream, busy)
    log("[bench] head per-kernel (ms): " + ", ".join(f"{k}={v[0]:.4f}" for k, v in bd.items()))
    xb = head_xattn_bytes(cfg)
    xroof = {"part": "cross-attention + MLP + classifier", "bound": "hbm",
             "achieved": round(xb / (ms_x * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "algorithmic_bytes": round(xb / 1e6, 2), "ms": round(ms_x, 5)}
    xroof["frac"] = round(xroof["achieved"] / PEAK_HBM_GBS, 4)
    res = {"workload": cfg.name, "ms_per_call": round(ms, 4),
           "tokens_per_s": round(cfg.batch * cfg.n_tokens / ms * 1e3, 1),
           "tflops": round(tflops, 2), "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
           "config": {"global_batch": cfg.batch, "tokens_per_item": cfg.n_tokens, "embed_dim": cfg.embed_dim,
                      "pool_layers": cfg.n_pool_layers, "heads": cfg.n_head, "classes": cfg.n_classes},
           "kernels_ms_per_layer": {k: round(v[0], 5) for k, v in bd.items()},
           "kernels_ms_alone": {k: round(v[3], 5) for k, v in bd.items()},
           "roofline": roofline_of(bd, cfg.name), "xattn_roofline": xroof, "cpu_baseline": None}
    if not args.no_cpu_baseline:
        log("[bench] head cpu baseline (oracle) ...")
        res["cpu_baseline"] = cpu_baseline_head(cfg, wl)
        log(f"[bench] head cpu baseline {res['cpu_baseline']}")
    bare.close()
    head.close()
    return res


def bench_variants(args, stream):
    """Encoder options on their own inputs, each one encode call per step:
    the ViT-L image encoder at 256x256 with its 14x14 sincos table resampled
    bicubically (batch 8), and a V-JEPA 2.1 ViT-g image at 384x384 through the
    one-frame tokenizer with four hierarchical outputs (batch 4).  The
    resampling step is also timed alone against HBM bandwidth."""
    import torch
    from vision_transformer_amd import vitenc as V
    from vision_transformer_amd import workloads as W
    cases = [
        W.CONFIGS[1].replace(name="ijepa_vit_l_256_resampled", height=256, width=256,
                             pos_interp=W.POS_INTERP_BICUBIC, pos_grid=(1, 14, 14)),
        W.CONFIGS[3].replace(name="vjepa21_vit_g_image_384_hier4", frames=1, batch=4, image_patch_embed=1,
                             hier_layers=(9, 19, 29, 39)),
    ]
    res = {}
    for cfg in cases:
        log(f"[bench] variant {cfg.name}: B={cfg.batch} grid={cfg.grid} L={cfg.n_layer}")
        wl = W.make_workload(cfg)
        enc = V.Encoder.from_workload(wl)
        px = torch.from_numpy(wl.pixels).cuda()
        ws, out, pooled = enc.alloc(cfg.batch, cfg.frames, cfg.height, cfg.width)
        hier = None
        if cfg.hier_layers:
            hier = torch.empty((len(cfg.hier_layers),) + tuple(out.shape), dtype=torch.float32, device="cuda")
        ms, _ = time_steps(lambda: enc.encode_into(px, ws, out, pooled, stream, hier=hier), max(5, args.steps // 2),
                           args.warmup, stream)
        tokens = cfg.batch * cfg.n_tokens
        r = {"ms_per_step": round(ms, 4), "tokens_per_s": round(tokens / ms * 1e3, 1),
             "tflops": round(cfg.flops() / (ms * 1e-3) / 1e12, 2),
             "config": {"global_batch": cfg.batch, "grid": list(cfg.grid), "layers": cfg.n_layer,
                        "embed_dim": cfg.embed_dim, "table_grid": list(cfg.table_grid) if cfg.pos_interp else None,
                        "hier_layers": list(cfg.hier_layers)}}
        if cfg.pos_interp:
            tab = torch.from_numpy(wl.weights.pos).cuda()
            dst = torch.empty((cfg.n_tokens, cfg.embed_dim), dtype=torch.float32, device="cuda")
            reps = 50
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            V.op_pos_resample(tab, cfg.n_prefix, cfg.table_grid, cfg.grid, cfg.pos_interp, out=dst)
            e0.record(stream)
            for _ in range(reps):
                V.op_pos_resample(tab, cfg.n_prefix, cfg.table_grid, cfg.grid, cfg.pos_interp, out=dst)
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / reps * 1e3
            nbytes = (tab.numel() + dst.numel()) * 4
            r["pos_resample"] = {"us": round(us, 2), "bound": "hbm", "algorithmic_bytes": nbytes,
                                 "achieved_GBs": round(nbytes / (us * 1e-6) / 1e9, 1), "peak_GBs": PEAK_HBM_GBS}
        res[cfg.name] = r
        log(f"[bench] variant {cfg.name}: {r}")
        enc.close()
    # the small fp32 ViT-Ti image (257 tokens, about 90 short kernels): eager
    # calls against replays of the call captured once into a HIP graph
    cfg = W.CONFIGS[0]
    wl = W.make_workload(cfg)
    enc = V.Encoder.from_workload(wl)
    px = torch.from_numpy(wl.pixels).cuda()
    ws, out, pooled = enc.alloc(cfg.batch, cfg.frames, cfg.height, cfg.width)
    eager, _ = time_steps(lambda: enc.encode_into(px, ws, out, pooled, stream), args.steps, args.warmup, stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        enc.encode_into(px, ws, out, pooled)
    replay, _ = time_steps(g.replay, args.steps, args.warmup, stream)
    res[cfg.name + "_graph"] = {"eager_ms": round(eager, 4), "graph_replay_ms": round(replay, 4),
                                "tokens_per_s_graph": round(cfg.batch * cfg.n_tokens / replay * 1e3, 1),
                                "tflops_fp32_graph": round(cfg.flops() / (replay * 1e-3) / 1e12, 2)}
    log(f"[bench] variant {cfg.name} graph: {res[cfg.name + '_graph']}")
    enc.close()
    return res


def bench_weights8(args, stream):
    """8-bit block weights against bf16 weights on the ViT-L/16 image encoder
    (the regime the pages quantise for: small image batches, where the
    weights are a large part of the bytes a forward moves), batch 8 and
    batch 1: one encode call per step, and the up and down projections alone
    at the encode shapes (weights rotated over the 24 layers, so every launch
    reads its weights from HBM) with their algorithmic bytes per launch."""
    import torch
    from vision_transformer_amd import vitenc as V
    from vision_transformer_amd import workloads as W
    res = {}
    for batch in (8, 1):
        row = {}
        encs = {}
        for fmt, wf in (("bf16", W.WEIGHTS_PLAIN), ("mxfp8", W.WEIGHTS_MXFP8)):
            cfg = W.CONFIGS[1].replace(batch=batch, weight_format=wf)
            wl = W.make_workload(cfg)
            enc = V.Encoder.from_workload(wl)
            px = torch.from_numpy(wl.pixels).cuda()
            ws, out, pooled = enc.alloc(cfg.batch, cfg.frames, cfg.height, cfg.width)
            ms, _ = time_steps(lambda: enc.encode_into(px, ws, out, pooled, stream), max(10, args.steps),
                               args.warmup, stream)
            M, D, F = cfg.batch * cfg.n_tokens, cfg.embed_dim, cfg.ffn_dim
            wb = 1 + 1 / 32 if wf == W.WEIGHTS_MXFP8 else 2   # weight bytes per weight
            Y = torch.randn((M, D), device="cuda").to(torch.bfloat16)
            Uo = torch.randn((M, F), device="cuda").to(torch.bfloat16)
            Z = torch.zeros((M, D), device="cuda")
            L = len(enc.blocks)
            reps = 3 * L

            def up(i):
                b = enc.blocks[i % L]
                if wf == W.WEIGHTS_MXFP8:
                    V.op_linear_mxfp8(1, Y, b["up_w"], b["up_s"], b["up_b"], Uo)
                else:
                    V.op_linear_gelu(W.DTYPE_BF16, Y, b["up_w"], b["up_b"], out=Uo)

            def down(i):
                b = enc.blocks[i % L]
                if wf == W.WEIGHTS_MXFP8:
                    V.op_linear_mxfp8(0, Uo, b["down_w"], b["down_s"], b["down_b"], Z)
                else:
                    V.op_linear_residual(W.DTYPE_BF16, Uo, b["down_w"], b["down_b"], Z)

            gem = {}
            for name, fn, flops, nbytes in (
                    ("up_gemm", up, 2.0 * M * D * F, M * D * 2 + F * D * wb + M * F * 2),
                    ("down_gemm", down, 2.0 * M * F * D, M * F * 2 + D * F * wb + 8 * M * D)):
                for i in range(L):
                    fn(i)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for i in range(reps):
                    fn(i)
                e1.record(stream)
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) / reps * 1e3
                gem[name] = {"us": round(us, 2), "tflops": round(flops / (us * 1e-6) / 1e12, 1),
                             "mfma_frac": round(flops / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
                             "algorithmic_MB": round(nbytes / 1e6, 2),
                             "hbm_GBs": round(nbytes / (us * 1e-6) / 1e9, 1),
                             "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
            row[fmt] = {"ms_per_step": round(ms, 4), "tokens_per_s": round(cfg.batch * cfg.n_tokens / ms * 1e3, 1),
                        "tflops": round(cfg.flops() / (ms * 1e-3) / 1e12, 2),
                        "weight_MB_per_forward": round(cfg.n_layer * (4 * D * D + 2 * D * F) * wb / 1e6, 1),
                        **gem}
            log(f"[bench] weights8 batch {batch} {fmt}: {row[fmt]}")
            enc.close()
            del wl, px, ws, out, pooled, Y, Uo, Z
            torch.cuda.empty_cache()
        row["speedup"] = round(row["bf16"]["ms_per_step"] / row["mxfp8"]["ms_per_step"], 3)
        res[f"vit_l16_image_batch{batch}"] = row
    return res


def bench_configs(args, stream):
    """Every encoder workload at its own shape (the five the metric's
    configuration list names), one encode call per step: throughput and the
    fraction of the MFMA peak of its arithmetic type."""
    import torch
    from vision_transformer_amd import vitenc as V
    from vision_transformer_amd import workloads as W
    res = {}
    names = [c.name for c in W.CONFIGS]
    if args.workload is not None and args.workload not in names:
        raise SystemExit(f"unknown workload {args.workload!r}; one of {names}")
    for cfg in W.CONFIGS:
        if args.workload is not None and cfg.name != args.workload:
            continue
        wl = W.make_workload(cfg)
        enc = V.Encoder.from_workload(wl)
        px = torch.from_numpy(wl.pixels).cuda()
        ws, out, pooled = enc.alloc(cfg.batch, cfg.frames, cfg.height, cfg.width)
        steps = 3 if cfg.n_tokens * cfg.batch > 10000 else max(5, args.steps // 2)
        ms, _ = time_steps(lambda: enc.encode_into(px, ws, out, pooled, stream), steps, 1, stream)
        tf = cfg.flops() / (ms * 1e-3) / 1e12
        peak = PEAK_FP32_TFLOPS if cfg.dtype == W.DTYPE_F32 else PEAK_BF16_TFLOPS
        res[cfg.name] = {"ms_per_step": round(ms, 4), "tokens_per_s": round(cfg.batch * cfg.n_tokens / ms * 1e3, 1),
                         "tflops": round(tf, 2), "peak_tflops": peak, "mfma_frac": round(tf / peak, 4),
                         "dtype": "f32" if cfg.dtype == W.DTYPE_F32 else "bf16", "steps": steps}
        log(f"[bench] config {cfg.name}: {res[cfg.name]}")
        enc.close()
        del wl, px, ws, out, pooled
        torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.sq_summary:
        sq_summary(args.sq_summary)
        return
    if args.write_counters:
        write_counters(*args.write_counters)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(items are independent: N GPUs would each encode their own batch).", file=sys.stderr)
        sys.exit(2)
    import torch
    from vision_transformer_amd import vitenc as V
    from vision_transformer_amd import workloads as W

    peak_source = device_peaks()
    log(f"[bench] peaks: bf16 {PEAK_BF16_TFLOPS} TFLOP/s, fp32 {PEAK_FP32_TFLOPS} TFLOP/s from {peak_source}")
    stream = torch.cuda.current_stream()
    if args.part == "predictor":
        print(json.dumps({"predictor": bench_predictor(args, stream)}), flush=True)
        return
    if args.part == "head":
        print(json.dumps({"head": bench_head(args, stream)}), flush=True)
        return
    if args.part == "variants":
        print(json.dumps({"variants": bench_variants(args, stream)}), flush=True)
        return
    if args.part == "configs":
        print(json.dumps({"configs": bench_configs(args, stream)}), flush=True)
        return
    if args.part == "weights8":
        print(json.dumps({"weights8": bench_weights8(args, stream)}), flush=True)
        return
    cfg = W.HEADLINE
    log(f"[bench] workload {cfg.name}: B={cfg.batch} N={cfg.n_tokens} D={cfg.embed_dim} L={cfg.n_layer}")
    wl = W.make_workload(cfg)
    enc = V.Encoder.from_workload(wl)
    if args.only:
        def warm():
            # library GEMMs (kernels of other names) queued ahead, so that the
            # kernel's launches run on a busy GPU, as in the layer-sequence timing
            a = torch.randn((4096, 4096), device="cuda", dtype=torch.bfloat16)
            for _ in range(100):
                torch.matmul(a, a)

        kernel_breakdown(cfg, enc, args.kernel_reps, stream, warm, only=args.only)
        print(json.dumps({"only": args.only, "launches": args.kernel_reps}), flush=True)
        return
    px = torch.from_numpy(wl.pixels).cuda()
    ws, out, pooled = enc.alloc(cfg.batch, cfg.frames, cfg.height, cfg.width)

    step = lambda: enc.encode_into(px, ws, out, pooled, stream)
    if args.graph:
        step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            enc.encode_into(px, ws, out, pooled)
        step = graph.replay
    calls = []
    ms, wall = time_steps(step, args.steps, args.warmup, stream, per_call=calls)
    tokens = cfg.batch * cfg.n_tokens
    tflops = cfg.flops() / (ms * 1e-3) / 1e12
    med, mn = float(np.median(calls)), float(np.min(calls))
    log(f"[bench] {ms:.3f} ms/step, {tokens / ms * 1e3:.0f} tokens/s, {tflops:.1f} TFLOP/s "
        f"(wall {wall:.3f} ms/step; per call median {med:.3f} min {mn:.3f} ms)")

    def busy():
        for _ in range(4):
            enc.encode_into(px, ws, out, pooled, stream)

    bd = kernel_breakdown(cfg, enc, args.kernel_reps, stream, busy)
    per_layer = {k: v[0] for k, v in bd.items()}
    log("[bench] per-kernel (ms): " + ", ".join(f"{k}={v:.4f}" for k, v in per_layer.items()))
    roof = roofline_of(bd, cfg.name)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        cpu = cpu_baseline(cfg, wl)
        log(f"[bench] cpu baseline {cpu}")
    enc.close()
    pred = bench_predictor(args, stream) if args.part == "all" else None
    head = bench_head(args, stream) if args.part == "all" else None
    variants = bench_variants(args, stream) if args.part == "all" else None
    configs = bench_configs(args, stream) if args.part == "all" else None
    weights8 = bench_weights8(args, stream) if args.part == "all" else None

    line = {
        "metric": "encoder tokens/sec + MFMA TFLOP/s fraction of peak (ViT-L video, bf16, 1 GPU)",
        "value": round(tokens / ms * 1e3, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) pixels, N(0,0.02) weights)",
        "tflops": round(tflops, 2), "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "per_call": {"median_ms": round(med, 4), "min_ms": round(mn, 4), "max_ms": round(float(np.max(calls)), 4),
                     "calls": len(calls), "tokens_per_s_median": round(tokens / med * 1e3, 1),
                     "tflops_median": round(cfg.flops() / (med * 1e-3) / 1e12, 2),
                     "mfma_frac_median": round(cfg.flops() / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
        "peak": {"bf16_tflops": PEAK_BF16_TFLOPS, "fp32_tflops": PEAK_FP32_TFLOPS, "hbm_gbs": PEAK_HBM_GBS,
                 **peak_source},
        "config": {"workload": cfg.name, "global_batch": cfg.batch, "tokens_per_item": cfg.n_tokens,
                   "embed_dim": cfg.embed_dim, "layers": cfg.n_layer, "heads": cfg.n_head,
                   "graph": bool(args.graph)},
        "kernels_ms_per_layer": {k: round(v, 5) for k, v in per_layer.items()},
        "kernels_ms_alone": {k: round(v[3], 5) for k, v in bd.items()},
        "roofline": roof,
        "cpu_baseline": cpu,
        "predictor": pred,
        "head": head,
        "variants": variants,
        "all_configs": configs,
        "weights8": weights8,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
