"""V-JEPA 2.1 encoder options on the GPU against the oracle: hierarchical
outputs (vitenc_encode_hier: block outputs through their own norms) on video
clips, and one-frame images through the separate image tokenizer with the
image modality vector.  Gates as the encoder's, on every output."""
import numpy as np
import pytest

import oracle
from vision_transformer_amd import workloads as W

from gpu_util import gates_ok, say, to_np

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

BASE = W.CONFIGS[3].replace(frames=4, height=64, width=48, n_layer=12, image_patch_embed=1,
                            hier_layers=(2, 5, 8, 11))


def _run(cfg):
    from vision_transformer_amd.vitenc import Encoder
    say(f"encode {cfg.name} frames={cfg.frames} grid={cfg.grid} L={cfg.n_layer} hier={cfg.hier_layers} "
        f"dtype={cfg.dtype}")
    wl = W.make_workload(cfg)
    enc = Encoder.from_workload(wl)
    px = torch.from_numpy(wl.pixels).cuda()
    ws, out, pooled = enc.alloc(cfg.batch, cfg.frames, cfg.height, cfg.width)
    hier = torch.empty((len(cfg.hier_layers),) + tuple(out.shape), dtype=torch.float32, device="cuda")
    enc.encode_into(px, ws, out, pooled, hier=hier)
    # the plain entry point gives the same tokens
    out2 = torch.empty_like(out)
    enc.encode_into(px, ws, out2, None)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    ro, rp, rh = oracle.encoder_forward(cfg, wl.weights, wl.pixels, return_hier=True)
    pairs = [("tokens", to_np(out), ro), ("pooled", to_np(pooled), rp)]
    pairs += [(f"hier{k}", to_np(hier[k]), rh[k]) for k in range(len(cfg.hier_layers))]
    for name, g, r in pairs:
        st = oracle.compare(g, r)
        say(f"  {name} {st}")
        assert gates_ok(cfg, st), (name, st)
    enc.close()


def _short(cfg, dtype):
    # the bf16 recipe's own error grows with depth on these small clips (as in
    # the encoder's small-clip tests): four blocks there
    if dtype == W.DTYPE_F32:
        return cfg
    return cfg.replace(n_layer=4, hier_layers=(0, 1, 3))


@pytest.mark.parametrize("dtype", [W.DTYPE_F32, W.DTYPE_BF16])
def test_video_hierarchical_outputs(gpu_lib, dtype):
    _run(_short(BASE.replace(name="vjepa21_hier_video", dtype=dtype), dtype))


@pytest.mark.parametrize("dtype", [W.DTYPE_F32, W.DTYPE_BF16])
def test_image_tokenizer(gpu_lib, dtype):
    """One frame at 96x80: the 1x16x16 tokenizer, the image modality vector,
    RoPE on a one-frame grid with interpolation, hierarchical outputs."""
    cfg = BASE.replace(name="vjepa21_image", frames=1, height=96, width=80, batch=2, dtype=dtype)
    if dtype == W.DTYPE_F32:
        cfg = cfg.replace(std_tok=1.0)
    _run(_short(cfg, dtype))
