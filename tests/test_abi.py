"""The C ABI on the CPU: the library loads, exports every symbol the header
declares, and refuses bad input by name before any device work (refusal,
never clamping: jepa.cpp "Architecture", section "Robustness").  No kernel
is launched by any test here."""
import ctypes
import os
import re
import threading

import pytest

from vision_transformer_amd import vitenc as V
from vision_transformer_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vitenc.h")

pytestmark = pytest.mark.skipif(not os.path.exists(V.LIB_PATH), reason="libvitenc.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vitenc_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = V.lib()
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(V.SIGNATURES), "binding and header disagree"
    assert L.vitenc_abi_version() == 5


FAKE = 0x1000  # a non-NULL pointer that is never dereferenced: creation only validates


def _hp(**kw):
    cfg = W.CONFIGS[2]
    hp = cfg.hparams()
    hp["pos_rows"] = 0
    hp.update(kw)
    return V.make_hparams(hp)


def _weights(n_layer, ls=False, blank=None):
    bw = (V.BlockWeights * n_layer)()
    for i in range(n_layer):
        for f in V.BLOCK_FIELDS:
            if f in ("ls1", "ls2") and not ls:
                continue
            setattr(bw[i], f, FAKE)
    if blank:
        setattr(bw[0], blank, None)
    w = V.Weights(FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.cast(bw, ctypes.POINTER(V.BlockWeights)), FAKE, FAKE)
    return w, bw


def _create(hp, w):
    h = ctypes.c_void_p()
    st = V.lib().vitenc_model_create(ctypes.byref(hp), ctypes.byref(w), ctypes.byref(h))
    return st, h


def _text():
    return V.lib().vitenc_error_text().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(embed_dim=0), 1, "embed_dim"),
    (dict(embed_dim=70000), 1, "embed_dim"),
    (dict(n_layer=0), 1, "n_layer"),
    (dict(n_head=0), 1, "n_head"),
    (dict(ffn_dim=0), 1, "ffn_dim"),
    (dict(patch_size=0), 1, "patch_size"),
    (dict(tubelet_size=2000), 1, "tubelet_size"),
    (dict(in_chans=0), 1, "in_chans"),
    (dict(ln_eps=float("nan")), 1, "ln_eps"),
    (dict(ln_eps=2.0), 1, "ln_eps"),
    (dict(dtype=7), 1, "dtype"),
    (dict(pos_type=5), 1, "pos_type"),
    (dict(rope=3), 1, "rope"),
    (dict(rope_layout=4), 1, "rope_layout"),
    (dict(attn_mode=9), 1, "attn_mode"),
    (dict(embed_dim=1000, n_head=16), 1, "divisible"),
    (dict(embed_dim=65, n_head=1), 1, "odd"),
    (dict(rope_theta=0.0), 1, "rope_theta"),
    (dict(rope_interpolate=1, rope_ref_grid=0), 1, "rope_ref_grid"),
    (dict(rope=0, attn_mode=1), 1, "block_causal"),
    (dict(rope=0, rope_interpolate=1, rope_ref_grid=16), 1, "rope_interpolate"),
    (dict(pos_type=1, pos_rows=0), 1, "pos_rows"),
    (dict(pos_type=1, pos_rows=197, pos_interp=3), 1, "pos_interp"),
    (dict(pos_type=0, pos_interp=1, pos_grid_t=1, pos_grid_h=14, pos_grid_w=14), 1, "without a position table"),
    (dict(pos_type=1, pos_rows=197, pos_interp=1, pos_grid_t=1, pos_grid_h=0, pos_grid_w=14), 1, "table grid"),
    (dict(pos_type=1, pos_rows=197, pos_interp=1, pos_grid_t=1, pos_grid_h=14, pos_grid_w=14), 1, "makes 196"),
    (dict(pos_type=1, pos_rows=392, pos_interp=1, pos_grid_t=2, pos_grid_h=14, pos_grid_w=14), 1, "one-frame"),
    (dict(embed_dim=1024, n_head=8), 6, "head_dim"),
    (dict(embed_dim=8192, n_head=128), 6, "embed_dim"),
])
def test_hparam_refusals(kw, status, needle):
    w, _keep = _weights(24)
    st, h = _create(_hp(**kw), w)
    assert st == status, _text()
    assert needle in _text()
    assert not h.value


@pytest.mark.parametrize("blank", ["qkv_w", "ln2_b", "down_b"])
def test_null_weight_refused(blank):
    w, _keep = _weights(24, blank=blank)
    st, h = _create(_hp(), w)
    assert st == 3 and "block 0" in _text()


def test_layer_scale_pointers_required():
    w, _keep = _weights(24, ls=False)
    st, _ = _create(_hp(layer_scale=1), w)
    assert st == 3 and "ls1" in _text()
    w2, _keep2 = _weights(24, ls=True)
    st, h = _create(_hp(layer_scale=1), w2)
    assert st == 0
    V.lib().vitenc_model_destroy(h)


@pytest.fixture()
def model():
    w, keep = _weights(24)
    st, h = _create(_hp(), w)
    assert st == 0, _text()
    yield h
    V.lib().vitenc_model_destroy(h)


def test_workspace_size_and_shape_refusals(model):
    L = V.lib()
    n = ctypes.c_size_t()
    assert L.vitenc_workspace_size(model, 2, 16, 256, 256, ctypes.byref(n)) == 0
    ws_c3 = n.value
    # Z fp32 + Y, Q, K, Vt, O bf16 [M, D] + U bf16 [M, F] + patch rows, at least
    M, D, F = 4096, 1024, 4096
    assert ws_c3 >= M * D * 4 + 5 * M * D * 2 + M * F * 2
    assert L.vitenc_workspace_size(model, 1, 16, 256, 256, ctypes.byref(n)) == 0 and n.value < ws_c3
    for shape, needle in [((0, 16, 256, 256), "non-positive"), ((2, 15, 256, 256), "tubelet"),
                          ((2, 16, 250, 256), "patch_size"), ((1, 2, 16 * 1024, 16), "grid"),
                          ((1, 2048, 16 * 600, 16 * 600), "grid")]:
        st = L.vitenc_workspace_size(model, *shape, ctypes.byref(n))
        assert st == 2 and needle in _text(), (shape, _text())


def test_token_limit_refused():
    w, keep = _weights(1)
    st, h = _create(_hp(n_layer=1, patch_size=1, tubelet_size=1), w)
    assert st == 0
    n = ctypes.c_size_t()
    st = V.lib().vitenc_workspace_size(h, 1, 5, 1000, 1000, ctypes.byref(n))
    assert st == 2 and "2^22" in _text()
    V.lib().vitenc_model_destroy(h)


def test_pos_table_rows_must_match_tokens():
    w, keep = _weights(24)
    st, h = _create(_hp(pos_type=1, pos_rows=197, rope=0, tubelet_size=1), w)
    assert st == 0
    n = ctypes.c_size_t()
    assert V.lib().vitenc_workspace_size(h, 1, 1, 224, 224, ctypes.byref(n)) == 2
    assert "position table" in _text()
    V.lib().vitenc_model_destroy(h)


def test_resampled_table_accepts_other_grids():
    """A 14x14 table with bicubic resampling encodes any one-frame grid, and
    refuses a multi-frame one; trilinear takes any grid."""
    w, keep = _weights(24)
    L = V.lib()
    n = ctypes.c_size_t()
    st, h = _create(_hp(pos_type=1, pos_rows=196, rope=0, tubelet_size=1, pos_interp=1, pos_grid_t=1, pos_grid_h=14,
                        pos_grid_w=14), w)
    assert st == 0, _text()
    assert L.vitenc_workspace_size(h, 1, 1, 224, 224, ctypes.byref(n)) == 0
    base = n.value
    assert L.vitenc_workspace_size(h, 1, 1, 256, 320, ctypes.byref(n)) == 0
    assert n.value > base
    assert L.vitenc_workspace_size(h, 1, 2, 224, 224, ctypes.byref(n)) == 2 and "bicubic" in _text()
    L.vitenc_model_destroy(h)
    st, h = _create(_hp(pos_type=1, pos_rows=8 * 14 * 14, rope=0, tubelet_size=2, pos_interp=2, pos_grid_t=8,
                        pos_grid_h=14, pos_grid_w=14), w)
    assert st == 0, _text()
    assert L.vitenc_workspace_size(h, 1, 8, 256, 256, ctypes.byref(n)) == 0
    L.vitenc_model_destroy(h)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(image_patch_embed=2), 1, "image_patch_embed"),
    (dict(n_hier=9), 1, "n_hier"),
    (dict(n_hier=2, hier_layers=(5, 5)), 1, "strictly increase"),
    (dict(n_hier=1, hier_layers=(24,)), 1, "strictly increase"),
])
def test_hier_and_image_refusals(kw, status, needle):
    w, _keep = _weights(24)
    st, h = _create(_hp(**kw), w)
    assert st == status and needle in _text(), _text()


def test_image_tokenizer_and_hier_norm_pointers_required():
    w, _keep = _weights(24)
    st, _ = _create(_hp(image_patch_embed=1), w)
    assert st == 3 and "patch_img_w" in _text()
    w.patch_img_w = w.patch_img_b = 0x1000
    st, _ = _create(_hp(image_patch_embed=1, modality_embed=1), w)
    assert st == 3 and "mod_embed_img" in _text()
    st, _ = _create(_hp(n_hier=2, hier_layers=(3, 7)), w)
    assert st == 3 and "hier norm 0" in _text()
    w.hier_norm_w[0] = w.hier_norm_b[0] = w.hier_norm_w[1] = w.hier_norm_b[1] = 0x1000
    st, h = _create(_hp(n_hier=2, hier_layers=(3, 7), image_patch_embed=1), w)
    assert st == 0, _text()
    n = ctypes.c_size_t()
    # one frame goes through the image tokenizer; a tubelet-2 model without one refuses it
    assert V.lib().vitenc_workspace_size(h, 1, 1, 256, 256, ctypes.byref(n)) == 0
    V.lib().vitenc_model_destroy(h)
    st, h = _create(_hp(), w)
    assert st == 0
    assert V.lib().vitenc_workspace_size(h, 1, 1, 256, 256, ctypes.byref(n)) == 2 and "tubelet" in _text()
    V.lib().vitenc_model_destroy(h)


def test_pos_resample_op_refusals():
    L = V.lib()
    FAKE = 0x1000
    assert L.vitenc_op_pos_resample(None, 0, 8, 1, 4, 4, 1, 5, 5, 1, FAKE, None) == 3
    assert L.vitenc_op_pos_resample(FAKE, 0, 8, 1, 4, 4, 1, 5, 5, 7, FAKE, None) == 1
    assert L.vitenc_op_pos_resample(FAKE, 0, 8, 2, 4, 4, 1, 5, 5, 1, FAKE, None) == 2
    assert L.vitenc_op_pos_resample(FAKE, 0, 0, 1, 4, 4, 1, 5, 5, 2, FAKE, None) == 2


def test_encode_refusals_before_any_launch(model):
    L = V.lib()
    n = ctypes.c_size_t()
    assert L.vitenc_workspace_size(model, 2, 16, 256, 256, ctypes.byref(n)) == 0
    need = n.value
    args = lambda ws, nbytes, px=FAKE, out=FAKE: (model, px, 2, 16, 256, 256, ws, nbytes, out, None, None)
    assert L.vitenc_encode(*args(None, need)) == 3
    assert L.vitenc_encode(*args(4096, need - 1)) == 4 and "needed" in _text()
    assert L.vitenc_encode(*args(4096 + 8, need)) == 4 and "aligned" in _text()
    assert L.vitenc_encode(*args(4096, need, px=None)) == 3
    assert L.vitenc_encode(*args(4096, need, out=None)) == 3
    assert L.vitenc_encode(None, FAKE, 2, 16, 256, 256, 4096, need, FAKE, None, None) == 3
    assert L.vitenc_encode(model, FAKE, 2, 16, 255, 256, 4096, need, FAKE, None, None) == 2


def test_step_entry_point_refusals():
    L = V.lib()
    assert L.vitenc_op_layernorm(9, FAKE, FAKE, FAKE, 1e-6, 4, 64, FAKE, None) == 1
    assert L.vitenc_op_layernorm(0, None, FAKE, FAKE, 1e-6, 4, 64, FAKE, None) == 3
    assert L.vitenc_op_layernorm(0, FAKE, FAKE, FAKE, 1e-6, 4, 5000, FAKE, None) == 6
    assert L.vitenc_op_attention(1, FAKE, FAKE, FAKE, 1, 64, 2, 48, 0, 0, 0, None, FAKE, None) == 6
    assert L.vitenc_op_attention(1, FAKE, FAKE, FAKE, 1, 64, 2, 64, 1, 0, 0, None, FAKE, None) == 2
    assert L.vitenc_op_attention(1, FAKE, FAKE, FAKE, 1, 64, 2, 64, 0, 64, 0, None, FAKE, None) == 2
    S = L.vitenc_attention_scratch_floats
    # (dtype, B, N, heads, hd, attn_mode, n_prefix, tokens_per_frame)
    # prefix rows need the scratch (8 heads, 9 runs of 256 keys, 64 + 2 floats each)
    assert S(1, 1, 2049, 8, 64, 0, 1, 0) == 8 * 9 * 66
    assert S(1, 1, 2048, 8, 64, 0, 0, 0) == 0
    # in fp32 every row when the query tiles make fewer than 16 workgroups (3 heads x 2 tiles)
    assert S(0, 1, 257, 3, 64, 0, 1, 0) == 3 * 257 * 2 * 66
    assert S(0, 1, 256, 3, 64, 0, 0, 0) == 3 * 256 * 1 * 66
    assert S(1, 1, 257, 3, 64, 0, 1, 0) == 3 * 1 * 2 * 66          # 16-bit: the prefix row only
    assert S(0, 1, 257, 3, 64, 1, 1, 64) == 3 * 1 * 2 * 66          # fp32 block-causal: no row split
    # block-causal 16-bit calls with a small grid split the late query tiles:
    # 16 frames of 256 tokens after a CLS, 16 heads -> 32 query tiles of 128;
    # tile qt walks 4 (qt // 2 + 1) + 1 key tiles of 64 (the CLS shifts the
    # frames by one key), largest 65; those above 65 / 3 (25 and up: qt >= 10)
    # are split: 22 tiles x 128 rows x 2 halves x (64 + 4) floats per head,
    # after the prefix row's 17 runs x 66 floats (a multiple of 4 already)
    pre = 16 * 17 * 66
    assert S(1, 1, 4097, 16, 64, 1, 1, 256) == pre + 16 * 22 * 128 * 2 * 68
    assert S(2, 1, 4097, 16, 64, 1, 1, 256) == pre + 16 * 22 * 128 * 2 * 68   # fp16 alike
    assert S(1, 1, 4097, 16, 64, 0, 1, 256) == pre                  # full attention: none
    assert S(1, 2, 4097, 16, 64, 1, 1, 256) == 2 * (pre + 16 * 22 * 128 * 2 * 68)  # 1024 workgroups
    assert S(1, 3, 4097, 16, 64, 1, 1, 256) == 3 * pre              # 1536 workgroups: not split
    # 3 heads: the prefix area (3 x 17 x 66 = 3366 floats) is padded to 3368
    assert S(1, 1, 4097, 3, 64, 1, 1, 256) == 3368 + 3 * 22 * 128 * 2 * 68
    assert S(1, 1, 4097, 16, 64, 1, 1, 4096) == pre                 # one frame: nothing to balance
    # full attention beyond the 768 resident workgroups with a last round less
    # than half full: the last k query tiles of every head run as halves, k the
    # fewest that leave only halves in the last round
    assert S(1, 1, 2048, 49, 64, 0, 0, 0) == 49 * 1 * 128 * 2 * 68       # 784 tiles: 16 over, k = 1
    assert S(1, 1, 2048, 49, 32, 0, 0, 0) == 49 * 1 * 128 * 2 * 36       # hd 32 alike
    assert S(1, 1, 18432, 22, 64, 0, 0, 0) == 22 * 5 * 128 * 2 * 68      # 3168 tiles: 96 over, k = 5
    assert S(1, 1, 2048, 48, 64, 0, 0, 0) == 0                           # 768 tiles: whole rounds
    assert S(1, 1, 2048, 73, 64, 0, 0, 0) == 0                           # 1168: last round 400 of 768
    assert S(1, 2, 2048, 16, 64, 0, 0, 0) == 0                           # the headline: one round
    # with a CLS row: the prefix area (25 x 17 x 66 = 28050 floats, padded to 28052), then the halves
    assert S(1, 1, 4097, 25, 64, 0, 1, 0) == 28052 + 25 * 2 * 128 * 2 * 68
    assert S(7, 1, 64, 1, 64, 0, 0, 0) == -1 and S(1, 1, 64, 1, 64, 2, 0, 0) == -1
    assert S(1, 1, 64, 1, 64, 1, 0, 0) == -1
    assert L.vitenc_op_attention(1, FAKE, FAKE, FAKE, 1, 257, 2, 64, 0, 1, 0, None, FAKE, None) == 3
    assert L.vitenc_op_attention(1, FAKE, FAKE, FAKE, 1, 64, 2, 64, 2, 0, 0, None, FAKE, None) == 1   # attn_mode
    # the scratch must be 16-byte aligned when the call needs one (the split tiles' float4 partials)
    assert L.vitenc_op_attention(1, FAKE, FAKE, FAKE, 1, 257, 2, 64, 0, 1, 0, FAKE + 4, FAKE, None) == 1
    assert L.vitenc_op_qkv_rope(1, FAKE, FAKE, FAKE, 1, 17, 64, 1, 1, 2, 2, 2, 0,
                                FAKE, FAKE, FAKE, FAKE, None) == 2          # 8 patches + 0 prefix != 17
    assert L.vitenc_op_qkv_rope(1, FAKE, FAKE, FAKE, 1, 8, 64, 1, 1, 2, 2, 2, 0,
                                None, FAKE, FAKE, FAKE, None) == 3          # RoPE without a table
    assert L.vitenc_op_rope_table(63, 0, 0, 0, 1e4, 2, 2, 2, FAKE, None) == 1   # odd head width
    assert L.vitenc_op_rope_table(64, 0, 1, 0, 1e4, 2, 2, 2, FAKE, None) == 1   # interpolate, no ref grid
    assert L.vitenc_op_rope_table(64, 0, 0, 0, 1e4, 2, 0, 2, FAKE, None) == 2   # empty grid
    assert L.vitenc_op_rope_table(64, 0, 0, 0, 1e4, 2, 2, 2, None, None) == 3
    assert L.vitenc_op_embed(1, FAKE, 1, 3, 1, 30, 32, 1, 16, FAKE, FAKE, None, None, None, 64, FAKE, FAKE,
                             None) == 2
    assert L.vitenc_op_pool(FAKE, 1, 4, 8, 0, 4, FAKE, None) == 2


def test_error_text_is_thread_local(model):
    L = V.lib()
    n = ctypes.c_size_t()
    assert L.vitenc_workspace_size(model, 0, 16, 256, 256, ctypes.byref(n)) == 2
    seen = {}

    def other():
        seen["text"] = L.vitenc_error_text().decode()

    t = threading.Thread(target=other)
    t.start(); t.join()
    assert seen["text"] == ""
    assert "non-positive" in _text()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(weight_format=2), 1, "weight_format"),
    (dict(weight_format=1, dtype=0), 6, "BF16"),
    (dict(weight_format=1, dtype=2), 6, "BF16"),
    (dict(weight_format=1, ffn_dim=4000), 1, "multiples of 64"),
])
def test_weight_format_refusals(kw, status, needle):
    w, _keep = _weights(24)
    st, h = _create(_hp(**kw), w)
    assert st == status and needle in _text(), _text()


def test_8bit_block_scales_and_alignment_required():
    w, bw = _weights(24)
    st, h = _create(_hp(weight_format=1), w)
    assert st == 0, _text()
    V.lib().vitenc_model_destroy(h)
    bw[3].up_s = None
    st, _ = _create(_hp(weight_format=1), w)
    assert st == 3 and "block 3" in _text() and "scale" in _text()
    bw[3].up_s = FAKE
    bw[5].down_w = FAKE + 8
    st, _ = _create(_hp(weight_format=1), w)
    assert st == 1 and "block 5" in _text() and "16-byte" in _text()
    # plain weights ignore the scale pointers
    bw[5].down_w = FAKE
    bw[0].qkv_s = None
    st, h = _create(_hp(), w)
    assert st == 0
    V.lib().vitenc_model_destroy(h)


def test_8bit_entry_point_refusals():
    L = V.lib()
    assert L.vitenc_quantize_mxfp8(None, 8, 64, FAKE, FAKE, None) == 3
    assert L.vitenc_quantize_mxfp8(FAKE, 8, 96, FAKE, FAKE, None) == 2 and "64" in _text()
    assert L.vitenc_quantize_mxfp8(FAKE, 0, 64, FAKE, FAKE, None) == 2
    assert L.vitenc_quantize_mxfp8(FAKE + 4, 8, 64, FAKE, FAKE, None) == 1 and "aligned" in _text()
    assert L.vitenc_op_linear_mxfp8(2, FAKE, FAKE, FAKE, FAKE, None, 4, 8, 64, FAKE, None) == 1
    assert L.vitenc_op_linear_mxfp8(0, FAKE, FAKE, None, FAKE, None, 4, 8, 64, FAKE, None) == 3
    assert L.vitenc_op_linear_mxfp8(0, FAKE, FAKE, FAKE, FAKE, None, 4, 8, 96, FAKE, None) == 2
    assert L.vitenc_op_linear_mxfp8(1, FAKE, FAKE, FAKE, FAKE, None, 4, 12, 64, FAKE, None) == 2
    assert L.vitenc_op_linear_mxfp8(1, FAKE + 2, FAKE, FAKE, FAKE, None, 4, 8, 64, FAKE, None) == 1
