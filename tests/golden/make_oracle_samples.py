"""Writes the oracle's full-depth outputs of the five encoder workloads at
sampled token rows (plus the pooled feature) to tests/golden/oracle_<name>.npz,
and those of the ViT-L/16 image workload with its block matrices in the 8-bit
block format (items 0 and 7, quantised by oracle/quant.py) to
tests/golden/oracle_<name>_mxfp8.npz.

    python tests/golden/make_oracle_samples.py [name ...]   (name_mxfp8 for the latter)

Calls only oracle/ and the seeded workload generator; nothing here comes from
the GPU path.  The full forwards take from seconds (ViT-Ti) to most of an
hour (the 18432-token ViT-g clip) on a few CPU cores, which is why the GPU
tests read the stored samples instead of recomputing them.
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from vision_transformer_amd import workloads as W  # noqa: E402

N_SAMPLED = 96


def sample_rows(cfg):
    """Prefix rows, frame boundaries, the last row and seeded random rows."""
    N = cfg.n_tokens
    gt, gh, gw = cfg.grid
    S = gh * gw
    p = cfg.n_prefix
    fixed = [0, 1, 2, p + S - 1, p + S, N // 2, N - 2, N - 1]
    rng = np.random.default_rng(12345)
    rows = np.concatenate([fixed, rng.integers(0, N, N_SAMPLED)])
    return np.unique(np.clip(rows, 0, N - 1))


def main(names):
    for cfg in W.CONFIGS:
        if names and cfg.name not in names:
            continue
        t0 = time.time()
        wl = W.make_workload(cfg)
        out, pooled = oracle.encoder_forward(cfg, wl.weights, wl.pixels)
        rows = sample_rows(cfg)
        path = os.path.join(HERE, f"oracle_{cfg.name}.npz")
        np.savez_compressed(path, rows=rows, tokens=out[:, rows].astype(np.float64), pooled=pooled,
                            n_layer=cfg.n_layer, seed=cfg.seed)
        print(f"{cfg.name}: {time.time() - t0:.1f} s -> {path}", flush=True)
    cfg = W.CONFIGS[1].replace(weight_format=W.WEIGHTS_MXFP8)
    name = cfg.name + "_mxfp8"
    if not names or name in names:
        t0 = time.time()
        wl = W.make_workload(cfg)
        items = [0, 7]
        w = oracle.quant.dequantized_weights(wl.weights)
        out, pooled = oracle.encoder_forward(cfg.replace(batch=len(items)), w, wl.pixels[items])
        rows = sample_rows(cfg)
        path = os.path.join(HERE, f"oracle_{name}.npz")
        np.savez_compressed(path, items=np.array(items), rows=rows, tokens=out[:, rows].astype(np.float64),
                            pooled=pooled, n_layer=cfg.n_layer, seed=cfg.seed)
        print(f"{name}: {time.time() - t0:.1f} s -> {path}", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:])
