"""ctypes binding of libvitenc.so (include/vitenc.h).

Argument marshalling only: every step of the encoder runs in the library's
HIP kernels.  PyTorch provides device memory and the stream.  If the library
has not been built, lib() raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libvitenc.so")

c_i32, c_f32, c_vp, c_size = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t

F32, BF16, F16 = 0, 1, 2
MAX_HIER = 8
STATUS = {0: "OK", 1: "EINVAL", 2: "ESHAPE", 3: "ENULL", 4: "EWORKSPACE", 5: "EDEVICE", 6: "EUNSUPPORTED"}


class VitencError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(f"vitenc {STATUS.get(status, status)}: {text}")
        self.status = status
        self.text = text


class Hparams(ctypes.Structure):
    _fields_ = [(n, c_i32) for n in ("embed_dim", "n_layer", "n_head", "ffn_dim", "patch_size",
                                      "tubelet_size", "in_chans")] + \
               [("ln_eps", c_f32), ("rope_theta", c_f32)] + \
               [(n, c_i32) for n in ("pos_type", "pos_rows", "rope", "rope_layout", "rope_interpolate",
                                      "rope_ref_grid", "cls_token", "modality_embed", "layer_scale",
                                      "attn_mode", "dtype", "pos_interp", "pos_grid_t", "pos_grid_h",
                                      "pos_grid_w", "image_patch_embed", "n_hier")] + \
               [("hier_layers", c_i32 * MAX_HIER), ("weight_format", c_i32)]


BLOCK_FIELDS = ("ln1_w", "ln1_b", "qkv_w", "qkv_b", "out_w", "out_b", "ln2_w", "ln2_b", "up_w", "up_b",
                "down_w", "down_b", "ls1", "ls2", "qkv_s", "out_s", "up_s", "down_s")
WEIGHTS_PLAIN, WEIGHTS_MXFP8 = 0, 1
QUANT_MATRICES = ("qkv_w", "out_w", "up_w", "down_w")   # stored in 8 bits with WEIGHTS_MXFP8


class BlockWeights(ctypes.Structure):
    _fields_ = [(n, c_vp) for n in BLOCK_FIELDS]


class Weights(ctypes.Structure):
    _fields_ = [("patch_w", c_vp), ("patch_b", c_vp), ("pos_embed", c_vp), ("cls_token", c_vp),
                ("mod_embed", c_vp), ("blocks", ctypes.POINTER(BlockWeights)), ("norm_w", c_vp),
                ("norm_b", c_vp), ("patch_img_w", c_vp), ("patch_img_b", c_vp), ("mod_embed_img", c_vp),
                ("hier_norm_w", c_vp * MAX_HIER), ("hier_norm_b", c_vp * MAX_HIER)]


class PredHparams(ctypes.Structure):
    _fields_ = [(n, c_i32) for n in ("embed_dim", "enc_dim", "n_layer", "n_head", "ffn_dim", "n_mask_tokens")] + \
               [("ln_eps", c_f32), ("rope_theta", c_f32)] + \
               [(n, c_i32) for n in ("rope_layout", "grid_t", "grid_h", "grid_w", "dtype", "out_dim", "n_hier_in",
                                     "embed_hidden", "modality_embed", "context_proj")]


class PredWeights(ctypes.Structure):
    _fields_ = [("embed_w", c_vp), ("embed_b", c_vp), ("mask_tokens", c_vp),
                ("blocks", ctypes.POINTER(BlockWeights)), ("norm_w", c_vp), ("norm_b", c_vp),
                ("proj_w", c_vp), ("proj_b", c_vp), ("embed2_w", c_vp), ("embed2_b", c_vp),
                ("mod_embed_img", c_vp), ("mod_embed_video", c_vp), ("proj_ctx_w", c_vp), ("proj_ctx_b", c_vp)]


class HeadHparams(ctypes.Structure):
    _fields_ = [(n, c_i32) for n in ("embed_dim", "n_head", "ffn_dim", "n_pool_layers", "n_classes")] + \
               [("ln_eps", c_f32), ("dtype", c_i32)]


HEAD_FIELDS = ("query", "ln_kv_w", "ln_kv_b", "q_w", "q_b", "k_w", "k_b", "v_w", "v_b", "ln2_w", "ln2_b",
               "up_w", "up_b", "down_w", "down_b", "cls_w", "cls_b")


class HeadWeights(ctypes.Structure):
    _fields_ = [("blocks", ctypes.POINTER(BlockWeights))] + [(n, c_vp) for n in HEAD_FIELDS]


_LIB = None

# exported symbol -> (restype, argtypes)
SIGNATURES = {
    "vitenc_abi_version": (c_i32, []),
    "vitenc_error_text": (ctypes.c_char_p, []),
    "vitenc_model_create": (c_i32, [ctypes.POINTER(Hparams), ctypes.POINTER(Weights), ctypes.POINTER(c_vp)]),
    "vitenc_model_destroy": (None, [c_vp]),
    "vitenc_workspace_size": (c_i32, [c_vp, c_i32, c_i32, c_i32, c_i32, ctypes.POINTER(c_size)]),
    "vitenc_encode": (c_i32, [c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_size, c_vp, c_vp, c_vp]),
    "vitenc_encode_hier": (c_i32, [c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_size, c_vp, c_vp, c_vp, c_vp]),
    "vitenc_op_embed": (c_i32, [c_i32, c_vp] + [c_i32] * 7 + [c_vp] * 5 + [c_i32, c_vp, c_vp, c_vp]),
    "vitenc_op_layernorm": (c_i32, [c_i32, c_vp, c_vp, c_vp, c_f32, c_i32, c_i32, c_vp, c_vp]),
    "vitenc_op_rope_table": (c_i32, [c_i32] * 4 + [c_f32] + [c_i32] * 3 + [c_vp, c_vp]),
    "vitenc_op_qkv_rope": (c_i32, [c_i32, c_vp, c_vp, c_vp] + [c_i32] * 9 + [c_vp] * 5),
    "vitenc_rope_table_floats": (ctypes.c_int64, [c_i32] * 4),
    "vitenc_op_pos_resample": (c_i32, [c_vp] + [c_i32] * 9 + [c_vp, c_vp]),
    "vitenc_op_attention": (c_i32, [c_i32, c_vp, c_vp, c_vp] + [c_i32] * 7 + [c_vp, c_vp, c_vp]),
    "vitenc_op_attention_noalloc": (c_i32, [c_i32, c_vp, c_vp, c_vp] + [c_i32] * 7 + [c_vp, c_vp]),
    "vitenc_attention_scratch_floats": (ctypes.c_int64, [c_i32] * 8),
    "vitenc_op_linear_residual": (c_i32, [c_i32, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_vp, c_vp]),
    "vitenc_op_linear_gelu": (c_i32, [c_i32, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_vp, c_vp]),
    "vitenc_op_pool": (c_i32, [c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp]),
    "vitenc_op_linear_mxfp8": (c_i32, [c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_vp, c_vp]),
    "vitenc_quantize_mxfp8": (c_i32, [c_vp, c_i32, c_i32, c_vp, c_vp, c_vp]),
    "vitenc_predictor_create": (c_i32, [ctypes.POINTER(PredHparams), ctypes.POINTER(PredWeights),
                                        ctypes.POINTER(c_vp)]),
    "vitenc_predictor_destroy": (None, [c_vp]),
    "vitenc_predict_workspace_size": (c_i32, [c_vp, c_i32, c_i32, c_i32, ctypes.POINTER(c_size)]),
    "vitenc_predict": (c_i32, [c_vp, c_vp, c_i32, c_i32, c_vp, c_i32, c_vp, c_i32, c_i32, c_vp, c_size, c_vp,
                               c_vp]),
    "vitenc_predict_all": (c_i32, [c_vp, c_vp, c_i32, c_i32, c_vp, c_i32, c_vp, c_i32, c_i32, c_vp, c_size, c_vp,
                                   c_vp, c_vp]),
    "vitenc_head_create": (c_i32, [ctypes.POINTER(HeadHparams), ctypes.POINTER(HeadWeights), ctypes.POINTER(c_vp)]),
    "vitenc_head_destroy": (None, [c_vp]),
    "vitenc_head_workspace_size": (c_i32, [c_vp, c_i32, c_i32, ctypes.POINTER(c_size)]),
    "vitenc_head_forward": (c_i32, [c_vp, c_vp, c_i32, c_i32, c_vp, c_size, c_vp, c_vp, c_vp]),
}


def lib():
    """The loaded library.  torch is imported first so that the library binds
    to the HIP runtime torch already loaded."""
    global _LIB
    if _LIB is None:
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m vision_transformer_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def check(status: int):
    if status != 0:
        raise VitencError(status, lib().vitenc_error_text().decode())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def torch_dtype(dtype: int):
    import torch
    return {F32: torch.float32, BF16: torch.bfloat16, F16: torch.float16}[dtype]


def to_device(arr: np.ndarray, dtype: int, device="cuda"):
    """Upload a weight matrix held as device-storage numpy (bf16 bits as
    uint16, f16, or f32)."""
    import torch
    if dtype == BF16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    if dtype == F16:
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float16)).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def f32_to_device(arr, device="cuda"):
    import torch
    if arr is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def make_hparams(hp: Dict) -> Hparams:
    h = Hparams()
    for name, _ in Hparams._fields_:
        if name == "hier_layers":
            layers = list(hp.get("hier_layers", ()) or ())
            h.hier_layers[:] = (layers + [0] * MAX_HIER)[:MAX_HIER]
        else:
            setattr(h, name, hp.get(name, 0))
    return h


class Encoder:
    """A model handle over device-resident weights."""

    def __init__(self, hp: Dict, tensors: Dict, blocks):
        self.hp = dict(hp)
        self.tensors = tensors            # keeps device memory alive
        self.blocks = blocks
        L = lib()
        self._hp = make_hparams(self.hp)
        self._bw = (BlockWeights * len(blocks))()
        for i, b in enumerate(blocks):
            for n in BLOCK_FIELDS:
                setattr(self._bw[i], n, _ptr(b.get(n)))
        hw = list(tensors.get("hier_norm_w", []))
        hb = list(tensors.get("hier_norm_b", []))
        self._w = Weights(_ptr(tensors["patch_w"]), _ptr(tensors["patch_b"]), _ptr(tensors.get("pos")),
                          _ptr(tensors.get("cls")), _ptr(tensors.get("mod")),
                          ctypes.cast(self._bw, ctypes.POINTER(BlockWeights)), _ptr(tensors["norm_w"]),
                          _ptr(tensors["norm_b"]), _ptr(tensors.get("patch_img_w")),
                          _ptr(tensors.get("patch_img_b")), _ptr(tensors.get("mod_img")),
                          (c_vp * MAX_HIER)(*([_ptr(t) for t in hw] + [None] * (MAX_HIER - len(hw)))),
                          (c_vp * MAX_HIER)(*([_ptr(t) for t in hb] + [None] * (MAX_HIER - len(hb)))))
        h = c_vp()
        check(L.vitenc_model_create(ctypes.byref(self._hp), ctypes.byref(self._w), ctypes.byref(h)))
        self.handle = h

    @classmethod
    def from_workload(cls, wl, device="cuda") -> "Encoder":
        cfg, w = wl.cfg, wl.weights
        dt = cfg.dtype
        hp = cfg.hparams()
        hp["pos_rows"] = 0 if w.pos is None else w.pos.shape[0]
        t = {"patch_w": to_device(w.store["patch_w"], dt, device), "patch_b": f32_to_device(w.patch_b, device),
             "pos": f32_to_device(w.pos, device), "cls": f32_to_device(w.cls, device),
             "mod": f32_to_device(w.mod, device), "norm_w": f32_to_device(w.norm_w, device),
             "norm_b": f32_to_device(w.norm_b, device)}
        if getattr(w, "patch_img_w", None) is not None:
            t["patch_img_w"] = to_device(w.store["patch_img_w"], dt, device)
            t["patch_img_b"] = f32_to_device(w.patch_img_b, device)
            t["mod_img"] = f32_to_device(w.mod_img, device)
        t["hier_norm_w"] = [f32_to_device(x, device) for x in getattr(w, "hier_norm_w", [])]
        t["hier_norm_b"] = [f32_to_device(x, device) for x in getattr(w, "hier_norm_b", [])]
        blocks = []
        wq = hp.get("weight_format", WEIGHTS_PLAIN) == WEIGHTS_MXFP8
        for b in w.blocks:
            d = {}
            for n in QUANT_MATRICES:
                if wq:
                    # fp32 matrices quantised on the device into codes and block scales
                    d[n], d[n[:-2] + "_s"] = quantize_mxfp8(f32_to_device(b.store[n], device))
                else:
                    d[n] = to_device(b.store[n], dt, device)
            for n in ("qkv_b", "out_b", "up_b", "down_b", "ln1_w", "ln1_b", "ln2_w", "ln2_b", "ls1", "ls2"):
                d[n] = f32_to_device(getattr(b, n), device)
            blocks.append(d)
        return cls(hp, t, blocks)

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            lib().vitenc_model_destroy(self.handle)
            self.handle = c_vp()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_bytes(self, B, T, H, W) -> int:
        n = c_size()
        check(lib().vitenc_workspace_size(self.handle, B, T, H, W, ctypes.byref(n)))
        return n.value

    def tokens(self, T, H, W) -> int:
        hp = self.hp
        tub = 1 if (hp.get("image_patch_embed") and T == 1) else hp["tubelet_size"]
        return (T // tub) * (H // hp["patch_size"]) * (W // hp["patch_size"]) + (1 if hp["cls_token"] else 0)

    def alloc(self, B, T, H, W, device="cuda"):
        """Workspace and outputs for a [B, C, T, H, W] input."""
        import torch
        ws = torch.empty(self.workspace_bytes(B, T, H, W), dtype=torch.uint8, device=device)
        N = self.tokens(T, H, W)
        D = self.hp["embed_dim"]
        out = torch.empty((B, N, D), dtype=torch.float32, device=device)
        pooled = torch.empty((B, D), dtype=torch.float32, device=device)
        return ws, out, pooled

    def encode_into(self, pixels, ws, out, pooled=None, stream=None, hier=None):
        """hier: None, or fp32 [n_hier, B, N, D] for the hierarchical outputs."""
        B, C, T, H, W = pixels.shape
        if hier is None:
            check(lib().vitenc_encode(self.handle, pixels.data_ptr(), B, T, H, W, ws.data_ptr(), ws.numel(),
                                      out.data_ptr(), _ptr(pooled), _stream(stream)))
        else:
            check(lib().vitenc_encode_hier(self.handle, pixels.data_ptr(), B, T, H, W, ws.data_ptr(), ws.numel(),
                                           out.data_ptr(), _ptr(pooled), hier.data_ptr(), _stream(stream)))

    def encode(self, pixels, stream=None):
        B, C, T, H, W = pixels.shape
        ws, out, pooled = self.alloc(B, T, H, W, device=pixels.device)
        self.encode_into(pixels, ws, out, pooled, stream)
        return out, pooled


def check_pred_ids(ctx_ids, tgt_ids, n_enc):
    """The id contract of vitenc_predict, checked on the host: per item each
    list strictly increasing, within [0, n_enc), and the two disjoint."""
    c = np.asarray(ctx_ids.cpu() if hasattr(ctx_ids, "cpu") else ctx_ids)
    t = np.asarray(tgt_ids.cpu() if hasattr(tgt_ids, "cpu") else tgt_ids)
    if c.ndim != 2 or t.ndim != 2 or c.shape[0] != t.shape[0]:
        raise ValueError("ctx_ids / tgt_ids must be [B, n] with the same B")
    for name, a in (("ctx_ids", c), ("tgt_ids", t)):
        if a.size and (a.min() < 0 or a.max() >= n_enc):
            raise ValueError(f"{name} outside [0, {n_enc})")
        if a.shape[1] > 1 and not (np.diff(a, axis=1) > 0).all():
            raise ValueError(f"{name} not strictly increasing within an item")
    for b in range(c.shape[0]):
        if np.intersect1d(c[b], t[b]).size:
            raise ValueError(f"item {b}: context and target ids overlap")


class Predictor:
    """A masked-latent predictor handle over device-resident weights."""

    def __init__(self, hp: Dict, tensors: Dict, blocks):
        self.hp = dict(hp)
        self.tensors = tensors
        self.blocks = blocks
        L = lib()
        self._hp = PredHparams()
        for name, _ in PredHparams._fields_:
            setattr(self._hp, name, self.hp.get(name, 0))
        self._bw = (BlockWeights * len(blocks))()
        for i, b in enumerate(blocks):
            for n in BLOCK_FIELDS:
                setattr(self._bw[i], n, _ptr(b.get(n)))
        opt = lambda n: _ptr(tensors.get(n))
        self._w = PredWeights(_ptr(tensors["embed_w"]), _ptr(tensors["embed_b"]), _ptr(tensors["mask_tokens"]),
                              ctypes.cast(self._bw, ctypes.POINTER(BlockWeights)), _ptr(tensors["norm_w"]),
                              _ptr(tensors["norm_b"]), _ptr(tensors["proj_w"]), _ptr(tensors["proj_b"]),
                              opt("embed2_w"), opt("embed2_b"), opt("mod_embed_img"), opt("mod_embed_video"),
                              opt("proj_ctx_w"), opt("proj_ctx_b"))
        h = c_vp()
        check(L.vitenc_predictor_create(ctypes.byref(self._hp), ctypes.byref(self._w), ctypes.byref(h)))
        self.handle = h

    @staticmethod
    def hparams_of(cfg) -> Dict:
        hp = cfg.hparams()
        gt, gh, gw = hp.pop("grid")
        hp.update(grid_t=gt, grid_h=gh, grid_w=gw)
        return hp

    @classmethod
    def from_workload(cls, wl, device="cuda") -> "Predictor":
        cfg, w = wl.cfg, wl.weights
        dt = cfg.dtype
        t = {"embed_w": to_device(w.store["embed_w"], dt, device), "embed_b": f32_to_device(w.embed_b, device),
             "mask_tokens": f32_to_device(w.mask_tokens, device), "norm_w": f32_to_device(w.norm_w, device),
             "norm_b": f32_to_device(w.norm_b, device), "proj_w": to_device(w.store["proj_w"], dt, device),
             "proj_b": f32_to_device(w.proj_b, device)}
        if w.embed2_w is not None:
            t["embed2_w"] = to_device(w.store["embed2_w"], dt, device)
            t["embed2_b"] = f32_to_device(w.embed2_b, device)
        if w.mod_img is not None:
            t["mod_embed_img"] = f32_to_device(w.mod_img, device)
            t["mod_embed_video"] = f32_to_device(w.mod_video, device)
        if w.proj_ctx_w is not None:
            t["proj_ctx_w"] = to_device(w.store["proj_ctx_w"], dt, device)
            t["proj_ctx_b"] = f32_to_device(w.proj_ctx_b, device)
        blocks = []
        for b in w.blocks:
            d = {n: to_device(b.store[n], dt, device) for n in QUANT_MATRICES}
            for n in ("qkv_b", "out_b", "up_b", "down_b", "ln1_w", "ln1_b", "ln2_w", "ln2_b"):
                d[n] = f32_to_device(getattr(b, n), device)
            blocks.append(d)
        return cls(cls.hparams_of(cfg), t, blocks)

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            lib().vitenc_predictor_destroy(self.handle)
            self.handle = c_vp()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_bytes(self, B, n_ctx, n_tgt) -> int:
        n = c_size()
        check(lib().vitenc_predict_workspace_size(self.handle, B, n_ctx, n_tgt, ctypes.byref(n)))
        return n.value

    def out_width(self) -> int:
        return self.hp.get("out_dim") or self.hp["enc_dim"]

    def alloc(self, B, n_ctx, n_tgt, device="cuda"):
        import torch
        ws = torch.empty(self.workspace_bytes(B, n_ctx, n_tgt), dtype=torch.uint8, device=device)
        out = torch.empty((B, n_tgt, self.out_width()), dtype=torch.float32, device=device)
        return ws, out

    def predict_into(self, enc_tokens, ctx_ids, tgt_ids, ws, out, mask_index=1, stream=None, check_ids=True,
                     out_ctx=None):
        """enc_tokens fp32 [B, n_enc, enc_dim] ([n_hier_in, B, n_enc, enc_dim]),
        ctx_ids / tgt_ids int32 [B, n] on the device.  check_ids copies the ids
        to the host (a synchronisation) to check their contract before the
        call.  out_ctx: None, or fp32 [B, n_ctx, out_dim] for the projected
        context rows."""
        B, n_enc = enc_tokens.shape[-3], enc_tokens.shape[-2]
        if check_ids:
            check_pred_ids(ctx_ids, tgt_ids, n_enc)
        check(lib().vitenc_predict_all(self.handle, enc_tokens.data_ptr(), B, n_enc, ctx_ids.data_ptr(),
                                       ctx_ids.shape[1], tgt_ids.data_ptr(), tgt_ids.shape[1], mask_index,
                                       ws.data_ptr(), ws.numel(), out.data_ptr(), _ptr(out_ctx), _stream(stream)))

    def predict(self, enc_tokens, ctx_ids, tgt_ids, mask_index=1, stream=None, return_context=False):
        import torch
        B = enc_tokens.shape[-3]
        ws, out = self.alloc(B, ctx_ids.shape[1], tgt_ids.shape[1], device=enc_tokens.device)
        out_ctx = None
        if return_context:
            out_ctx = torch.empty((B, ctx_ids.shape[1], self.out_width()), dtype=torch.float32,
                                  device=enc_tokens.device)
        self.predict_into(enc_tokens, ctx_ids, tgt_ids, ws, out, mask_index, stream, out_ctx=out_ctx)
        return (out, out_ctx) if return_context else out


class Head:
    """An attentive-pool head (+ classifier) handle over device-resident
    weights."""

    def __init__(self, hp: Dict, tensors: Dict, blocks):
        self.hp = dict(hp)
        self.tensors = tensors
        self.blocks = blocks
        L = lib()
        self._hp = HeadHparams()
        for name, _ in HeadHparams._fields_:
            setattr(self._hp, name, self.hp.get(name, 0))
        self._bw = (BlockWeights * max(1, len(blocks)))()
        for i, b in enumerate(blocks):
            for n in BLOCK_FIELDS:
                setattr(self._bw[i], n, _ptr(b.get(n)))
        self._w = HeadWeights(ctypes.cast(self._bw, ctypes.POINTER(BlockWeights)),
                              *[_ptr(tensors.get(n)) for n in HEAD_FIELDS])
        h = c_vp()
        check(L.vitenc_head_create(ctypes.byref(self._hp), ctypes.byref(self._w), ctypes.byref(h)))
        self.handle = h

    @classmethod
    def from_workload(cls, wl, device="cuda") -> "Head":
        cfg, w = wl.cfg, wl.weights
        dt = cfg.dtype
        t = {n: f32_to_device(getattr(w, n), device) for n in ("query", "ln_kv_w", "ln_kv_b", "q_b", "k_b", "v_b",
                                                                 "ln2_w", "ln2_b", "up_b", "down_b", "cls_b")}
        for n in ("q_w", "k_w", "v_w", "up_w", "down_w", "cls_w"):
            t[n] = to_device(w.store[n], dt, device)
        blocks = []
        for b in w.blocks:
            d = {n: to_device(b.store[n], dt, device) for n in QUANT_MATRICES}
            for n in ("qkv_b", "out_b", "up_b", "down_b", "ln1_w", "ln1_b", "ln2_w", "ln2_b"):
                d[n] = f32_to_device(getattr(b, n), device)
            blocks.append(d)
        return cls(cfg.hparams(), t, blocks)

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            lib().vitenc_head_destroy(self.handle)
            self.handle = c_vp()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_bytes(self, B, N) -> int:
        n = c_size()
        check(lib().vitenc_head_workspace_size(self.handle, B, N, ctypes.byref(n)))
        return n.value

    def alloc(self, B, N, device="cuda"):
        import torch
        ws = torch.empty(self.workspace_bytes(B, N), dtype=torch.uint8, device=device)
        pooled = torch.empty((B, self.hp["embed_dim"]), dtype=torch.float32, device=device)
        logits = torch.empty((B, max(1, self.hp["n_classes"])), dtype=torch.float32, device=device)
        return ws, pooled, logits

    def forward_into(self, tokens, ws, pooled, logits=None, stream=None):
        B, N, _ = tokens.shape
        check(lib().vitenc_head_forward(self.handle, tokens.data_ptr(), B, N, ws.data_ptr(), ws.numel(),
                                        pooled.data_ptr(), _ptr(logits), _stream(stream)))

    def forward(self, tokens, stream=None):
        B, N, _ = tokens.shape
        ws, pooled, logits = self.alloc(B, N, device=tokens.device)
        self.forward_into(tokens, ws, pooled, logits if self.hp["n_classes"] > 0 else None, stream)
        return pooled, logits[:, :self.hp["n_classes"]]


# ---------------------------------------------------------------------------
# step entry points (one kernel or fused pair each)
# ---------------------------------------------------------------------------
def op_embed(dtype, pixels, tubelet, patch, patch_w, patch_b, pos=None, cls=None, mod=None, stream=None):
    import torch
    B, C, T, H, W = pixels.shape
    D = patch_w.shape[0]
    Np = (T // tubelet) * (H // patch) * (W // patch)
    K = C * tubelet * patch * patch
    lda = (K + 7) // 8 * 8
    scratch = torch.empty(B * Np * 2 * lda, dtype=torch_dtype(dtype), device=pixels.device)
    Z = torch.empty((B, Np + (1 if cls is not None else 0), D), dtype=torch.float32, device=pixels.device)
    check(lib().vitenc_op_embed(dtype, pixels.data_ptr(), B, C, T, H, W, tubelet, patch, patch_w.data_ptr(),
                                patch_b.data_ptr(), _ptr(pos), _ptr(cls), _ptr(mod), D, scratch.data_ptr(),
                                Z.data_ptr(), _stream(stream)))
    return Z


def op_layernorm(x, w, b, eps, out_dtype, stream=None, out=None):
    import torch
    M, D = x.shape
    y = torch.empty((M, D), dtype=torch_dtype(out_dtype), device=x.device) if out is None else out
    check(lib().vitenc_op_layernorm(out_dtype, x.data_ptr(), w.data_ptr(), b.data_ptr(), eps, M, D, y.data_ptr(),
                                    _stream(stream)))
    return y


def op_rope_table(head_dim, grid, rope_layout=0, rope_interpolate=0, rope_ref_grid=0, rope_theta=10000.0,
                  stream=None, out=None, device="cuda"):
    import torch
    tab = out if out is not None else torch.empty(max(lib().vitenc_rope_table_floats(head_dim, *grid), 1),
                                                  dtype=torch.float32, device=device)
    check(lib().vitenc_op_rope_table(head_dim, rope_layout, rope_interpolate, rope_ref_grid, rope_theta, grid[0],
                                     grid[1], grid[2], tab.data_ptr(), _stream(stream)))
    return tab


def op_qkv_rope(dtype, Y, qkv_w, qkv_b, B, N, n_head, rope=0, rope_layout=0, rope_interpolate=0,
                rope_ref_grid=0, rope_theta=10000.0, grid=(1, 1, 1), n_prefix=0, stream=None, outs=None,
                table_ready=False):
    """outs: optional preallocated (Q, K, Vt, rope_table).  The RoPE table is
    filled first (vitenc_op_rope_table) unless table_ready says outs[3]
    already holds it."""
    import torch
    D = Y.shape[1]
    hd = D // n_head
    ldv = (N + 63) // 64 * 64
    td = torch_dtype(dtype)
    if outs is None:
        Q = torch.empty((B, n_head, N, hd), dtype=td, device=Y.device)
        K = torch.empty((B, n_head, N, hd), dtype=td, device=Y.device)
        Vt = torch.zeros((B, n_head, hd, ldv), dtype=td, device=Y.device)
        nt = lib().vitenc_rope_table_floats(hd, *grid)
        tab = torch.empty(max(nt, 1), dtype=torch.float32, device=Y.device)
    else:
        Q, K, Vt, tab = outs
    if rope and not table_ready:
        op_rope_table(hd, grid, rope_layout, rope_interpolate, rope_ref_grid, rope_theta, stream=stream, out=tab)
    check(lib().vitenc_op_qkv_rope(dtype, Y.data_ptr(), qkv_w.data_ptr(), qkv_b.data_ptr(), B, N, D, n_head, rope,
                                   grid[0], grid[1], grid[2], n_prefix, tab.data_ptr() if rope else None,
                                   Q.data_ptr(), K.data_ptr(), Vt.data_ptr(), _stream(stream)))
    return Q, K, Vt


def op_pos_resample(pos, prefix, src_grid, dst_grid, mode, stream=None, out=None):
    """pos fp32 [prefix + prod(src_grid), D] -> [prefix + prod(dst_grid), D]."""
    import torch
    D = pos.shape[1]
    rows = prefix + dst_grid[0] * dst_grid[1] * dst_grid[2]
    if out is None:
        out = torch.empty((rows, D), dtype=torch.float32, device=pos.device)
    check(lib().vitenc_op_pos_resample(pos.data_ptr(), prefix, D, *src_grid, *dst_grid, mode, out.data_ptr(),
                                       _stream(stream)))
    return out


def op_attention(dtype, Q, K, Vt, attn_mode=0, n_prefix=0, tokens_per_frame=0, stream=None, out=None,
                 scratch=None):
    """scratch: None (allocated here when the prefix rows need it) or fp32
    with at least vitenc_attention_scratch_floats() elements."""
    import torch
    B, H, N, hd = Q.shape
    O = torch.empty((B, N, H * hd), dtype=torch_dtype(dtype), device=Q.device) if out is None else out
    nf = lib().vitenc_attention_scratch_floats(dtype, B, N, H, hd, attn_mode, n_prefix, tokens_per_frame)
    if scratch is None and nf > 0:
        scratch = torch.empty(nf, dtype=torch.float32, device=Q.device)
    check(lib().vitenc_op_attention(dtype, Q.data_ptr(), K.data_ptr(), Vt.data_ptr(), B, N, H, hd, attn_mode,
                                    n_prefix, tokens_per_frame, _ptr(scratch), O.data_ptr(), _stream(stream)))
    return O


def op_attention_noalloc(dtype, Q, K, Vt, attn_mode=0, n_prefix=0, tokens_per_frame=0, stream=None, out=None):
    """vitenc_op_attention_noalloc: the partials in the library's fixed array."""
    import torch
    B, H, N, hd = Q.shape
    O = torch.empty((B, N, H * hd), dtype=torch_dtype(dtype), device=Q.device) if out is None else out
    check(lib().vitenc_op_attention_noalloc(dtype, Q.data_ptr(), K.data_ptr(), Vt.data_ptr(), B, N, H, hd, attn_mode,
                                            n_prefix, tokens_per_frame, O.data_ptr(), _stream(stream)))
    return O


def op_linear_residual(dtype, A, W, b, Z, ls=None, stream=None):
    M, K = A.shape
    Nout = W.shape[0]
    check(lib().vitenc_op_linear_residual(dtype, A.data_ptr(), W.data_ptr(), b.data_ptr(), _ptr(ls), M, Nout, K,
                                          Z.data_ptr(), _stream(stream)))
    return Z


def op_linear_gelu(dtype, A, W, b, stream=None, out=None):
    import torch
    M, K = A.shape
    Nout = W.shape[0]
    U = torch.empty((M, Nout), dtype=torch_dtype(dtype), device=A.device) if out is None else out
    check(lib().vitenc_op_linear_gelu(dtype, A.data_ptr(), W.data_ptr(), b.data_ptr(), M, Nout, K, U.data_ptr(),
                                      _stream(stream)))
    return U


def quantize_mxfp8(w, stream=None):
    """fp32 device matrix [rows, cols] -> (codes uint8 [rows, cols], scale
    bytes uint8 [cols/64, rows, 2]) in the format of vitenc_quantize_mxfp8."""
    import torch
    rows, cols = w.shape
    w = w.contiguous()
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=w.device)
    scales = torch.empty((cols // 64, rows, 2), dtype=torch.uint8, device=w.device)
    check(lib().vitenc_quantize_mxfp8(w.data_ptr(), rows, cols, codes.data_ptr(), scales.data_ptr(),
                                      _stream(stream)))
    return codes, scales


def op_linear_mxfp8(epi, A, codes, scales, b, out, ls=None, stream=None):
    """epi 0: out (fp32 Z) += ls * (A W^T + b); epi 1: out (bf16) = GELU(A W^T + b)."""
    M, K = A.shape
    Nout = codes.shape[0]
    check(lib().vitenc_op_linear_mxfp8(epi, A.data_ptr(), codes.data_ptr(), scales.data_ptr(), b.data_ptr(),
                                       _ptr(ls), M, Nout, K, out.data_ptr(), _stream(stream)))
    return out


def op_pool(X, cls, n_prefix, stream=None):
    import torch
    B, N, D = X.shape
    pooled = torch.empty((B, D), dtype=torch.float32, device=X.device)
    check(lib().vitenc_op_pool(X.data_ptr(), B, N, D, int(cls), n_prefix, pooled.data_ptr(), _stream(stream)))
    return pooled
