"""The attentive-pool head's C ABI on the CPU: creation, workspace planning
and every refusal of vitenc_head_forward happen before any device work, so
they are checked here with fake (never dereferenced) pointers.  No kernel is
launched by any test here."""
import ctypes
import os

import pytest

from vision_transformer_amd import vitenc as V
from vision_transformer_amd import workloads as W

pytestmark = pytest.mark.skipif(not os.path.exists(V.LIB_PATH), reason="libvitenc.so not built")

FAKE = 0x1000       # 16-byte aligned, never dereferenced


def _hp(**kw):
    hp = W.HEAD.hparams()
    hp.update(kw)
    h = V.HeadHparams()
    for name, _ in V.HeadHparams._fields_:
        setattr(h, name, hp[name])
    return h


def _weights(n_layer, blank=None, blank_block=None, **ptr):
    bw = (V.BlockWeights * max(1, n_layer))()
    for i in range(n_layer):
        for f in V.BLOCK_FIELDS:
            if f not in ("ls1", "ls2"):
                setattr(bw[i], f, FAKE)
    if blank_block:
        setattr(bw[n_layer - 1], blank_block, None)
    w = V.HeadWeights(ctypes.cast(bw, ctypes.POINTER(V.BlockWeights)), *[FAKE] * len(V.HEAD_FIELDS))
    if blank:
        setattr(w, blank, None)
    for k, v in ptr.items():
        setattr(w, k, v)
    return w, bw


def _create(hp, w):
    h = ctypes.c_void_p()
    return V.lib().vitenc_head_create(ctypes.byref(hp), ctypes.byref(w), ctypes.byref(h)), h


def _text():
    return V.lib().vitenc_error_text().decode()


@pytest.fixture
def head():
    hp = _hp()
    w, bw = _weights(hp.n_pool_layers)
    st, h = _create(hp, w)
    assert st == 0, _text()
    yield h
    V.lib().vitenc_head_destroy(h)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(embed_dim=0), 1, "embed_dim"),
    (dict(n_head=0), 1, "n_head"),
    (dict(ffn_dim=0), 1, "ffn_dim"),
    (dict(n_pool_layers=-1), 1, "n_pool_layers"),
    (dict(n_classes=-1), 1, "n_classes"),
    (dict(ln_eps=float("inf")), 1, "ln_eps"),
    (dict(dtype=3), 1, "dtype"),
    (dict(n_head=7), 1, "divisible"),
    (dict(embed_dim=8192, n_head=128), 6, "embed_dim"),
    (dict(embed_dim=1026, n_head=9), 6, "multiple of 4"),
    (dict(n_head=8), 6, "head_dim"),
])
def test_head_hparam_refusals(kw, status, needle):
    hp = _hp(**kw)
    w, bw = _weights(max(0, hp.n_pool_layers))
    st, h = _create(hp, w)
    assert st == status and needle in _text(), (st, _text())
    assert not h.value


def test_head_width_is_free_without_pooler_blocks():
    hp = _hp(n_head=8, n_pool_layers=0)
    w, bw = _weights(0, blocks=None)
    st, h = _create(hp, w)
    assert st == 0, _text()
    V.lib().vitenc_head_destroy(h)


@pytest.mark.parametrize("blank", ["query", "ln_kv_w", "q_w", "k_b", "v_w", "ln2_b", "up_w", "down_b", "cls_w"])
def test_head_null_weight_refused(blank):
    hp = _hp()
    w, bw = _weights(hp.n_pool_layers, blank=blank)
    st, h = _create(hp, w)
    assert st == 3 and not h.value


def test_classifier_weights_optional_without_classes():
    hp = _hp(n_classes=0)
    w, bw = _weights(hp.n_pool_layers, cls_w=None, cls_b=None)
    st, h = _create(hp, w)
    assert st == 0, _text()
    V.lib().vitenc_head_destroy(h)


def test_head_misaligned_norm_refused():
    hp = _hp()
    w, bw = _weights(hp.n_pool_layers, ln_kv_w=FAKE + 4)
    st, h = _create(hp, w)
    assert st == 1 and "aligned" in _text()


def test_head_null_block_tensor_refused():
    hp = _hp()
    w, bw = _weights(hp.n_pool_layers, blank_block="qkv_w")
    st, h = _create(hp, w)
    assert st == 3 and "block 2" in _text()


def test_head_workspace_and_forward_refusals(head):
    L = V.lib()
    n = ctypes.c_size_t()
    assert L.vitenc_head_workspace_size(head, 2, 2048, ctypes.byref(n)) == 0
    M, D, F = 4096, 1024, 4096
    assert n.value >= M * D * 4 + 5 * M * D * 2 + M * F * 2
    for args in [(0, 8), (1, 0), (1, (1 << 22) + 1)]:
        assert L.vitenc_head_workspace_size(head, *args, ctypes.byref(n)) == 2
    assert L.vitenc_head_workspace_size(head, 1, 16, ctypes.byref(n)) == 0
    ws = 0x10000

    def call(tokens=FAKE, B=1, N=16, w=ws, wb=n.value, pooled=FAKE, logits=FAKE):
        return L.vitenc_head_forward(head, tokens, B, N, w, wb, pooled, logits, None)

    assert call(tokens=None) == 3
    assert call(pooled=None) == 3
    assert call(tokens=FAKE + 4) == 1 and "aligned" in _text()
    assert call(w=None) == 3
    assert call(w=ws + 16) == 4
    assert call(wb=n.value - 1) == 4
    assert call(N=0) == 2
