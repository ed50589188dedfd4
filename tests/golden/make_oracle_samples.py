"""Writes the oracle's full-depth outputs of the five encoder workloads at
sampled token rows (plus the pooled feature) to tests/golden/oracle_<name>.npz.

    python tests/golden/make_oracle_samples.py [name ...]

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


if __name__ == "__main__":
    main(sys.argv[1:])
