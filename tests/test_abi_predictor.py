"""The predictor's C ABI on the CPU: creation, workspace planning and every
refusal of vitenc_predict happen before any device work, so they are checked
here with fake (never dereferenced) pointers; plus the host-side id check of
the binding.  No kernel is launched by any test here."""
import ctypes
import os

import numpy as np
import pytest

from vision_transformer_amd import vitenc as V
from vision_transformer_amd import workloads as W

pytestmark = pytest.mark.skipif(not os.path.exists(V.LIB_PATH), reason="libvitenc.so not built")

FAKE = 0x1000


def _hp(**kw):
    hp = V.Predictor.hparams_of(W.PREDICTOR)
    hp.update(kw)
    h = V.PredHparams()
    for name, _ in V.PredHparams._fields_:
        setattr(h, name, hp[name])
    return h


def _weights(n_layer, blank=None, blank_block=None):
    bw = (V.BlockWeights * n_layer)()
    for i in range(n_layer):
        for f in V.BLOCK_FIELDS:
            if f not in ("ls1", "ls2"):
                setattr(bw[i], f, FAKE)
    if blank_block:
        setattr(bw[n_layer - 1], blank_block, None)
    w = V.PredWeights(FAKE, FAKE, FAKE, ctypes.cast(bw, ctypes.POINTER(V.BlockWeights)), FAKE, FAKE, FAKE, FAKE)
    if blank:
        setattr(w, blank, None)
    return w, bw


def _create(hp, w):
    h = ctypes.c_void_p()
    return V.lib().vitenc_predictor_create(ctypes.byref(hp), ctypes.byref(w), ctypes.byref(h)), h


def _text():
    return V.lib().vitenc_error_text().decode()


@pytest.fixture
def pred():
    hp = _hp()
    w, bw = _weights(hp.n_layer)
    st, h = _create(hp, w)
    assert st == 0, _text()
    yield h
    V.lib().vitenc_predictor_destroy(h)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(embed_dim=0), 1, "embed_dim"),
    (dict(enc_dim=0), 1, "enc_dim"),
    (dict(n_layer=0), 1, "n_layer"),
    (dict(n_head=0), 1, "n_head"),
    (dict(ffn_dim=0), 1, "ffn_dim"),
    (dict(n_mask_tokens=0), 1, "n_mask_tokens"),
    (dict(ln_eps=-1.0), 1, "ln_eps"),
    (dict(rope_theta=0.0), 1, "rope_theta"),
    (dict(rope_layout=2), 1, "rope_layout"),
    (dict(grid_t=0), 1, "grid"),
    (dict(grid_w=1024), 1, "grid"),
    (dict(dtype=7), 1, "dtype"),
    (dict(n_head=5), 1, "divisible"),
    (dict(n_head=3), 6, "head_dim"),
    (dict(embed_dim=8192, n_head=128), 6, "embed_dim"),
])
def test_predictor_hparam_refusals(kw, status, needle):
    hp = _hp(**kw)
    w, bw = _weights(max(1, hp.n_layer))
    st, h = _create(hp, w)
    assert st == status and needle in _text(), (st, _text())
    assert not h.value


@pytest.mark.parametrize("blank", ["embed_w", "embed_b", "mask_tokens", "norm_w", "proj_w", "proj_b"])
def test_predictor_null_weight_refused(blank):
    hp = _hp()
    w, bw = _weights(hp.n_layer, blank=blank)
    st, h = _create(hp, w)
    assert st == 3 and not h.value


def test_predictor_null_block_tensor_refused():
    hp = _hp()
    w, bw = _weights(hp.n_layer, blank_block="down_w")
    st, h = _create(hp, w)
    assert st == 3 and "block 11" in _text()


def test_predictor_workspace_and_shape_refusals(pred):
    L = V.lib()
    n = ctypes.c_size_t()
    assert L.vitenc_predict_workspace_size(pred, 2, 1024, 1024, ctypes.byref(n)) == 0
    cfg = W.PREDICTOR
    M, D, F = 2 * 2048, cfg.embed_dim, cfg.ffn_dim
    # at least the residual stream, five activations in bf16, the FFN hidden and the split context rows
    assert n.value >= M * D * 4 + 5 * M * D * 2 + M * F * 2 + 2 * 1024 * 2 * cfg.enc_dim * 2
    assert n.value < 2 * (M * D * 4 + 5 * M * D * 2 + M * F * 2 + 2 * 1024 * 2 * cfg.enc_dim * 2 + 2 * 1024 * D * 4)
    for args, needle in [((0, 4, 4), "at least 1"), ((1, 0, 4), "at least 1"), ((1, 4, 0), "at least 1"),
                         ((1, 1024, 1025), "exceeds")]:
        assert L.vitenc_predict_workspace_size(pred, *args, ctypes.byref(n)) == 2
        assert needle in _text()


def test_predict_refusals_before_any_launch(pred):
    L = V.lib()
    n = ctypes.c_size_t()
    assert L.vitenc_predict_workspace_size(pred, 1, 8, 8, ctypes.byref(n)) == 0
    ws = 0x10000  # 256-byte aligned fake
    good = dict(enc=FAKE, B=1, n_enc=2048, ctx=FAKE, nc=8, tgt=FAKE, nt=8, mi=1, ws=ws, wsb=n.value, out=FAKE)

    def call(**kw):
        a = dict(good)
        a.update(kw)
        return L.vitenc_predict(pred, a["enc"], a["B"], a["n_enc"], a["ctx"], a["nc"], a["tgt"], a["nt"], a["mi"],
                                a["ws"], a["wsb"], a["out"], None)

    assert call(enc=None) == 3
    assert call(ctx=None) == 3
    assert call(out=None) == 3
    assert call(n_enc=2047) == 2 and "n_enc" in _text()
    assert call(mi=10) == 1 and "mask_index" in _text()
    assert call(mi=-1) == 1
    assert call(ws=None) == 3
    assert call(ws=ws + 8) == 4
    assert call(wsb=n.value - 1) == 4
    assert call(nt=0) == 2


def test_host_id_check():
    ctx = np.array([[0, 3, 5]], np.int32)
    V.check_pred_ids(ctx, np.array([[1, 2, 9]], np.int32), 10)
    with pytest.raises(ValueError, match="overlap"):
        V.check_pred_ids(ctx, np.array([[1, 3, 9]], np.int32), 10)
    with pytest.raises(ValueError, match="increasing"):
        V.check_pred_ids(np.array([[0, 5, 3]], np.int32), np.array([[1, 2, 9]], np.int32), 10)
    with pytest.raises(ValueError, match="outside"):
        V.check_pred_ids(ctx, np.array([[1, 2, 10]], np.int32), 10)
    with pytest.raises(ValueError, match="outside"):
        V.check_pred_ids(np.array([[-1, 3, 5]], np.int32), np.array([[1, 2, 9]], np.int32), 10)


def test_predictor21_option_tensors_are_required():
    """Each V-JEPA 2.1 option needs its tensors; out_dim, n_hier_in and
    embed_hidden are range-checked; out_ctx needs the context projection."""
    import ctypes
    from vision_transformer_amd import vitenc as V
    L = V.lib()
    base = dict(embed_dim=64, enc_dim=32, n_layer=1, n_head=2, ffn_dim=128, n_mask_tokens=2, ln_eps=1e-6,
                rope_theta=1e4, rope_layout=1, grid_t=2, grid_h=3, grid_w=4, dtype=0)
    fake = 0x1000

    def create(extra_hp=None, extra_w=None):
        hp = V.PredHparams(**dict(base, **(extra_hp or {})))
        bw = (V.BlockWeights * 1)()
        for n in V.BLOCK_FIELDS:
            if n not in ("ls1", "ls2"):
                setattr(bw[0], n, fake)
        w = V.PredWeights(fake, fake, fake, ctypes.cast(bw, ctypes.POINTER(V.BlockWeights)), fake, fake, fake, fake)
        for k, v in (extra_w or {}).items():
            setattr(w, k, v)
        h = ctypes.c_void_p()
        st = L.vitenc_predictor_create(ctypes.byref(hp), ctypes.byref(w), ctypes.byref(h))
        if st == 0:
            L.vitenc_predictor_destroy(h)
        return st

    assert create() == 0
    assert create({"n_hier_in": 4, "embed_hidden": 96}) == 3                     # ENULL: embed2
    assert create({"n_hier_in": 4, "embed_hidden": 96}, {"embed2_w": fake, "embed2_b": fake}) == 0
    assert create({"n_hier_in": 4, "embed_hidden": 0}, {"embed2_w": fake, "embed2_b": fake}) == 1
    assert create({"n_hier_in": 99}) == 1
    assert create({"modality_embed": 1}) == 3
    assert create({"modality_embed": 1}, {"mod_embed_img": fake, "mod_embed_video": fake}) == 0
    assert create({"context_proj": 1}) == 3
    assert create({"context_proj": 1}, {"proj_ctx_w": fake, "proj_ctx_b": fake}) == 0
    assert create({"out_dim": -3}) == 1
    assert create({"out_dim": 1664}) == 0
