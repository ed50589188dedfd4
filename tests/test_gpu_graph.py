"""The C-ABI calls captured into a HIP graph (torch.cuda.CUDAGraph on the
calling stream) and replayed: every replay, with eager work and
synchronisations between them, must give the eager call's result bit for bit
(the kernels are deterministic and the library allocates nothing, so a
captured call is the same launch sequence on the same buffers)."""
import numpy as np
import pytest

from vision_transformer_amd import workloads as W

from gpu_util import say

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _replays_match(run, outs, n=3):
    """run(): enqueue the call on the current stream.  outs: its outputs."""
    run()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    scratch = torch.randn(512, 512, device="cuda")
    for r in range(n):
        for o in outs:
            o.fill_(float("nan"))
        scratch = scratch @ scratch.T / 512.0      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b), f"replay {r} differs"
    say(f"  {n} replays match the eager call")


@pytest.mark.parametrize("cfg", [W.CONFIGS[0], W.CONFIGS[2].replace(frames=4, height=64, width=64, n_layer=3)],
                         ids=["vit_ti_fp32", "video_bf16"])
def test_encode_graph_replay(gpu_lib, cfg):
    from vision_transformer_amd.vitenc import Encoder
    say(f"graph encode {cfg.name} L={cfg.n_layer}")
    wl = W.make_workload(cfg)
    enc = Encoder.from_workload(wl)
    px = torch.from_numpy(wl.pixels).cuda()
    ws, out, pooled = enc.alloc(cfg.batch, cfg.frames, cfg.height, cfg.width)
    _replays_match(lambda: enc.encode_into(px, ws, out, pooled), [out, pooled])
    enc.close()


def test_predict_graph_replay(gpu_lib):
    from vision_transformer_amd.vitenc import Predictor
    cfg = W.PREDICTOR.replace(n_layer=2, grid=(2, 8, 8), n_ctx=60, n_tgt=50)
    say(f"graph predict {cfg.name} L={cfg.n_layer}")
    wl = W.make_predictor_workload(cfg)
    p = Predictor.from_workload(wl)
    enc = torch.from_numpy(wl.enc_tokens).cuda()
    ctx = torch.from_numpy(wl.ctx_ids).cuda()
    tgt = torch.from_numpy(wl.tgt_ids).cuda()
    ws, out = p.alloc(cfg.batch, cfg.n_ctx, cfg.n_tgt)
    _replays_match(lambda: p.predict_into(enc, ctx, tgt, ws, out, 1, check_ids=False), [out])
    p.close()


def test_head_graph_replay(gpu_lib):
    from vision_transformer_amd.vitenc import Head
    cfg = W.HEAD.replace(n_pool_layers=1, n_tokens=300, embed_dim=256, n_head=4, ffn_dim=512)
    say(f"graph head {cfg.name}")
    wl = W.make_head_workload(cfg)
    h = Head.from_workload(wl)
    tok = torch.from_numpy(wl.tokens).cuda()
    ws, pooled, logits = h.alloc(cfg.batch, cfg.n_tokens)
    _replays_match(lambda: h.forward_into(tok, ws, pooled, logits), [pooled, logits])
    h.close()
