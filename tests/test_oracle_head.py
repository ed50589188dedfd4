"""Pins of the attentive-pool head oracle (oracle/head.py) against a library
special case (torch's multi-head attention and Transformer encoder layer in
float64), brute force, closed forms and invariants."""
import math

import numpy as np
import pytest

import oracle
from vision_transformer_amd import workloads as W

torch = pytest.importorskip("torch")
F = torch.nn.functional

TINY = W.HeadConfig("tiny_head", embed_dim=48, n_head=3, ffn_dim=96, n_pool_layers=2, n_classes=7, batch=2,
                    n_tokens=11, dtype=W.DTYPE_F32, std_w=0.1, std_query=1.0, std_qk=0.3, ln_random=True, seed=5)


def _wl(cfg=TINY):
    return W.make_head_workload(cfg)


def _t(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


def _torch_head(cfg, w, tokens, n_layers):
    """The head from torch modules: TransformerEncoderLayer (pre-LN, GELU,
    eps) for the pooler blocks, MultiheadAttention with an identity output
    projection for the cross-attention (query not normalised, keys and
    values normalised), the MLP and the classifier as linear layers."""
    D, H = cfg.embed_dim, cfg.n_head
    x = _t(tokens)
    with torch.no_grad():
        for blk in w.blocks[:n_layers]:
            layer = torch.nn.TransformerEncoderLayer(D, H, dim_feedforward=cfg.ffn_dim, dropout=0.0,
                                                     activation="gelu", layer_norm_eps=cfg.ln_eps,
                                                     batch_first=True, norm_first=True, dtype=torch.float64)
            layer.self_attn.in_proj_weight.copy_(_t(blk.qkv_w)); layer.self_attn.in_proj_bias.copy_(_t(blk.qkv_b))
            layer.self_attn.out_proj.weight.copy_(_t(blk.out_w)); layer.self_attn.out_proj.bias.copy_(_t(blk.out_b))
            layer.linear1.weight.copy_(_t(blk.up_w)); layer.linear1.bias.copy_(_t(blk.up_b))
            layer.linear2.weight.copy_(_t(blk.down_w)); layer.linear2.bias.copy_(_t(blk.down_b))
            layer.norm1.weight.copy_(_t(blk.ln1_w)); layer.norm1.bias.copy_(_t(blk.ln1_b))
            layer.norm2.weight.copy_(_t(blk.ln2_w)); layer.norm2.bias.copy_(_t(blk.ln2_b))
            layer.eval()
            x = layer(x)
        mha = torch.nn.MultiheadAttention(D, H, bias=True, batch_first=True, dtype=torch.float64)
        mha.in_proj_weight.copy_(torch.cat([_t(w.q_w), _t(w.k_w), _t(w.v_w)]))
        mha.in_proj_bias.copy_(torch.cat([_t(w.q_b), _t(w.k_b), _t(w.v_b)]))
        mha.out_proj.weight.copy_(torch.eye(D, dtype=torch.float64))
        mha.out_proj.bias.zero_()
        kv = F.layer_norm(x, (D,), _t(w.ln_kv_w), _t(w.ln_kv_b), cfg.ln_eps)
        q0 = _t(w.query)[None, None, :].expand(x.shape[0], 1, D)
        a, _ = mha(q0, kv, kv, need_weights=False)
        y = q0 + a
        h = F.layer_norm(y, (D,), _t(w.ln2_w), _t(w.ln2_b), cfg.ln_eps)
        y = y + F.linear(F.gelu(F.linear(h, _t(w.up_w), _t(w.up_b))), _t(w.down_w), _t(w.down_b))
        logits = F.linear(y, _t(w.cls_w), _t(w.cls_b))
    return y[:, 0].numpy(), logits[:, 0].numpy()


@pytest.mark.parametrize("n_layers", [0, 2])
def test_head_matches_torch_modules(n_layers):
    wl = _wl()
    pooled, logits = oracle.attentive_pool_forward(TINY.hparams(), wl.weights, wl.tokens, n_layers=n_layers)
    tp, tl = _torch_head(TINY, wl.weights, wl.tokens, n_layers)
    assert np.abs(pooled - tp).max() < 1e-12 * max(1.0, np.abs(tp).max())
    assert np.abs(logits - tl).max() < 1e-12 * max(1.0, np.abs(tl).max())


def test_cross_attention_brute_force():
    """Explicit loops over heads, keys and dims (math.exp), tiny shapes."""
    cfg = TINY.replace(n_tokens=5, embed_dim=12, n_head=2, ffn_dim=8, n_pool_layers=0, batch=1)
    wl = _wl(cfg)
    w, x = wl.weights, wl.tokens.astype(np.float64)[0]
    D, H, hd, eps = 12, 2, 6, cfg.ln_eps
    kv = []
    for j in range(5):
        mu = sum(x[j]) / D
        var = sum((x[j][c] - mu) ** 2 for c in range(D)) / D
        kv.append([(x[j][c] - mu) / math.sqrt(var + eps) * w.ln_kv_w[c] + w.ln_kv_b[c] for c in range(D)])
    q = [sum(float(w.q_w[r][c]) * float(w.query[c]) for c in range(D)) + float(w.q_b[r]) for r in range(D)]
    k = [[sum(float(w.k_w[r][c]) * kv[j][c] for c in range(D)) + float(w.k_b[r]) for r in range(D)] for j in range(5)]
    v = [[sum(float(w.v_w[r][c]) * kv[j][c] for c in range(D)) + float(w.v_b[r]) for r in range(D)] for j in range(5)]
    y = [0.0] * D
    for h in range(H):
        s = [sum(q[h * hd + i] * k[j][h * hd + i] for i in range(hd)) / math.sqrt(hd) for j in range(5)]
        m = max(s)
        e = [math.exp(t - m) for t in s]
        z = sum(e)
        for i in range(hd):
            y[h * hd + i] = float(w.query[h * hd + i]) + sum(e[j] / z * v[j][h * hd + i] for j in range(5))
    y = np.array(y)
    ref = oracle.cross_attention_pool(cfg.hparams(), w, wl.tokens[:1])[0]
    mu, var = y.mean(), y.var()
    hln = (y - mu) / math.sqrt(var + eps) * w.ln2_w + w.ln2_b
    u = np.array([sum(float(w.up_w[r][c]) * hln[c] for c in range(D)) + float(w.up_b[r]) for r in range(8)])
    g = np.array([0.5 * t * (1.0 + math.erf(t / math.sqrt(2.0))) for t in u])
    f = np.array([sum(float(w.down_w[r][c]) * g[c] for c in range(8)) + float(w.down_b[r]) for r in range(D)])
    assert np.abs(ref - (y + f)).max() < 1e-12


def _closed_form_uniform(cfg, w, token):
    """query + v(LN_kv(token)), then the MLP residual: the head's output when
    every token equals `token` (every key scores the same)."""
    f64 = lambda a: np.asarray(a, dtype=np.float64)
    kv = oracle.layer_norm(f64(token), w.ln_kv_w, w.ln_kv_b, cfg.ln_eps)
    y = f64(w.query) + f64(w.v_w) @ kv + f64(w.v_b)
    u = f64(w.up_w) @ oracle.layer_norm(y, w.ln2_w, w.ln2_b, cfg.ln_eps) + f64(w.up_b)
    g = 0.5 * u * (1.0 + np.array([math.erf(t / math.sqrt(2.0)) for t in u]))
    return y + f64(w.down_w) @ g + f64(w.down_b)


def test_identical_tokens_give_uniform_attention():
    """All tokens equal: every key scores the same, so the attention output
    is v(token) whatever the query and the key weights."""
    cfg = TINY.replace(n_pool_layers=0, batch=1)
    wl = _wl(cfg)
    tok = np.repeat(wl.tokens[:, :1], cfg.n_tokens, axis=1)
    w = wl.weights
    a = oracle.cross_attention_pool(cfg.hparams(), w, tok)
    assert np.abs(a[0] - _closed_form_uniform(cfg, w, tok[0, 0])).max() < 1e-12
    w.k_w = w.k_w * 3.0
    w.query = -w.query
    b = oracle.cross_attention_pool(cfg.hparams(), w, tok)
    assert np.abs(b[0] - _closed_form_uniform(cfg, w, tok[0, 0])).max() < 1e-12
    assert np.abs(a - b).max() > 1e-3


def test_pooled_is_invariant_to_token_order():
    wl = _wl()
    perm = np.random.default_rng(0).permutation(TINY.n_tokens)
    a, la = oracle.attentive_pool_forward(TINY.hparams(), wl.weights, wl.tokens)
    b, lb = oracle.attentive_pool_forward(TINY.hparams(), wl.weights, wl.tokens[:, perm])
    assert np.abs(a - b).max() < 1e-12 and np.abs(la - lb).max() < 1e-12


def test_query_is_not_normalised_and_keys_are():
    """Scaling the tokens leaves the keys and values unchanged (they pass
    through a LayerNorm; eps 0 makes that exact), so with no pooler blocks
    the output is unchanged; scaling the query changes it."""
    cfg = TINY.replace(n_pool_layers=0, ln_eps=0.0)
    wl = _wl(cfg)
    a = oracle.cross_attention_pool(cfg.hparams(), wl.weights, wl.tokens)
    b = oracle.cross_attention_pool(cfg.hparams(), wl.weights, wl.tokens * 8.0)
    assert np.abs(a - b).max() < 1e-9
    w2 = W.make_head_workload(cfg).weights
    w2.query = w2.query * 2.0
    c = oracle.cross_attention_pool(cfg.hparams(), w2, wl.tokens)
    assert np.abs(a - c).max() > 1e-3
