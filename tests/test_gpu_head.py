"""The attentive-pool head and classifier on the GPU (vitenc_head_forward
through the C ABI) against the CPU oracle (oracle.attentive_pool_forward):
the V-JEPA 2 ViT-L classifier shape on the tokens of two 16-frame clips, small
ragged shapes in fp32 / bf16 / f16, a sensitised variant (a large query and
q/k weights make the attention peaked; random LayerNorm parameters tell the
two norms apart), no pooler blocks, one token, more items than one
matrix-vector launch takes, no classifier, and a ViT-g width (22 heads, two
head groups in every pass).  Gates as the encoder's on both outputs."""
import numpy as np
import pytest

import oracle
from vision_transformer_amd import workloads as W

from gpu_util import gates_ok, say, to_np

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

SMALL = W.HEAD.replace(name="head_small_f32", embed_dim=128, n_head=4, ffn_dim=256, n_pool_layers=2, n_classes=10,
                       batch=3, n_tokens=37, dtype=W.DTYPE_F32)


def run_head(wl, device="cuda"):
    from vision_transformer_amd.vitenc import Head
    head = Head.from_workload(wl, device)
    tok = torch.from_numpy(wl.tokens).to(device)
    pooled, logits = head.forward(tok)
    torch.cuda.synchronize()
    res = to_np(pooled), to_np(logits)
    head.close()
    return res


def _parity(cfg, wl=None):
    wl = wl or W.make_head_workload(cfg)
    say(f"head {cfg.name} L={cfg.n_pool_layers} B={cfg.batch} N={cfg.n_tokens} D={cfg.embed_dim} H={cfg.n_head} "
        f"classes={cfg.n_classes} dtype={cfg.dtype}")
    pooled, logits = run_head(wl)
    rp, rl = oracle.attentive_pool_forward(cfg.hparams(), wl.weights, wl.tokens)
    st = oracle.compare(pooled, rp)
    say(f"  pooled {st}")
    assert gates_ok(cfg, st), st
    if cfg.n_classes:
        st = oracle.compare(logits, rl)
        say(f"  logits {st}")
        assert gates_ok(cfg, st), st
    return pooled, rp


def test_head_full_shape(gpu_lib):
    """3 pooler blocks, 16 heads of 64, 174 classes over 2 x 2048 tokens, bf16."""
    _parity(W.HEAD)


@pytest.mark.parametrize("dtype", [W.DTYPE_F32, W.DTYPE_BF16, W.DTYPE_F16])
def test_head_small(gpu_lib, dtype):
    _parity(SMALL.replace(dtype=dtype))


def test_head_sensitised_fp32(gpu_lib):
    cfg = SMALL.replace(name="head_sensitised", std_query=1.0, std_qk=0.2, ln_random=True, n_tokens=300)
    _parity(cfg)


def test_head_no_pooler_blocks_hd64(gpu_lib):
    _parity(SMALL.replace(name="head_xattn_only", n_pool_layers=0, embed_dim=256, n_head=4, n_tokens=1000,
                          std_query=1.0, std_qk=0.2))


def test_head_one_token(gpu_lib):
    _parity(SMALL.replace(name="head_one_token", n_tokens=1, n_pool_layers=1))


def test_head_many_items(gpu_lib):
    """Ten items: two matrix-vector launches per step of the tail."""
    _parity(SMALL.replace(name="head_ten_items", batch=10, n_tokens=9, n_pool_layers=1))


def test_head_without_classifier(gpu_lib):
    _parity(SMALL.replace(name="head_no_classes", n_classes=0))


def test_head_vit_g_width(gpu_lib):
    """D 1408, 22 heads of 64: the scores pass stages two head groups and the
    weighted sums run two passes of 16 and 6 heads; ragged token count."""
    _parity(SMALL.replace(name="head_vit_g", embed_dim=1408, n_head=22, ffn_dim=512, n_pool_layers=1, n_tokens=45,
                          batch=2, std_query=1.0, std_qk=0.2))


def test_head_narrow_width(gpu_lib):
    """D 96 (3 heads of 32): a quarter of a wave's float4 lanes hold a row."""
    _parity(SMALL.replace(name="head_narrow", embed_dim=96, n_head=3, ffn_dim=64, n_pool_layers=1, n_tokens=70))
