"""Encoder configurations and seeded synthetic inputs.

This module is shared by the HIP path's tests/benchmark and by the CPU oracle's
tests.  It holds no step of the encoder's arithmetic: only shapes, random
draws, the bf16 storage rounding of the drawn weights, and the construction of
the position *table* that the sincos2d family receives as an input (that table
is a converter-side product, not a step of the encoder forward; see
jepa.cpp "GGUF schema (v1)", section "Encoder tensors", and jepa.cpp
"Converter", section "common.py").

Workload shapes follow the five encoder families described on the pages:
hfvit ViT-Ti/14 (jepa.cpp "GGUF schema (v1)", family note "hfvit" / "lewm"),
I-JEPA ViT-L/16 (family "ijepa"), V-JEPA 2 ViT-L video (jepa.cpp
"Architecture", family matrix "vjepa2"), V-JEPA 2.1 ViT-g video ("vjepa2_1")
and LeVJEPA ViT-L block-causal video (family note "levjepa").

Draw order for one config (seed = 1000 + config index):
  1. pixels  [B, C, T, H, W] fp32 ~ N(0, 1)
  2. patch_w [D, C*t*P*P], patch_b [D]                 ~ N(0, std_w)
  3. pos table (learned: N(0, std_w); sincos2d: deterministic), cls [D],
     mod [D], in that order, each only when the config has it
  4. per block: qkv_w, qkv_b, out_w, out_b, up_w, up_b, down_w, down_b,
     then ls1, ls2 when layer_scale is set (N(1, 0.1));
     LayerNorm gamma = 1, beta = 0 (no draw)
  5. final norm gamma = 1, beta = 0 (no draw)
Because blocks are drawn in order, a config truncated to its first k layers
receives exactly the first k blocks of the full config.

Matrices of bf16/f16 configs are rounded to that type with round-to-nearest-
even; the rounded values (held exactly in fp32) are what both the GPU and the
oracle consume.  Vectors, norms and tables stay fp32.  With weight_format 1
(8-bit block weights) the four block matrices stay fp32 and each side
quantises them with its own quantiser.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

DTYPE_F32, DTYPE_BF16, DTYPE_F16 = 0, 1, 2
POS_NONE, POS_TABLE = 0, 1
POS_INTERP_NONE, POS_INTERP_BICUBIC, POS_INTERP_TRILINEAR = 0, 1, 2
ROPE_NONE, ROPE_3D = 0, 1
LAYOUT_TILED, LAYOUT_INTERLEAVED = 0, 1
ATTN_FULL, ATTN_BLOCK_CAUSAL = 0, 1
WEIGHTS_PLAIN, WEIGHTS_MXFP8 = 0, 1


@dataclass
class EncoderConfig:
    """Hyperparameters of one encoder plus the input clip geometry."""
    name: str
    embed_dim: int
    n_layer: int
    n_head: int
    ffn_dim: int
    patch_size: int
    tubelet_size: int
    in_chans: int = 3
    ln_eps: float = 1e-6
    rope_theta: float = 10000.0
    pos_type: int = POS_NONE
    pos_kind: str = ""            # "learned" | "sincos2d" (table contents only)
    pos_interp: int = POS_INTERP_NONE
    pos_grid: Optional[tuple] = None  # the table's (t, h, w) grid; None: the input grid
    image_patch_embed: int = 0        # a separate one-frame tokenizer (and modality vector) for images
    hier_layers: tuple = ()           # blocks whose outputs are also returned, each with its own norm
    rope: int = ROPE_NONE
    rope_layout: int = LAYOUT_TILED
    rope_interpolate: int = 0
    rope_ref_grid: int = 0
    cls_token: int = 0
    modality_embed: int = 0
    layer_scale: int = 0
    attn_mode: int = ATTN_FULL
    dtype: int = DTYPE_BF16
    weight_format: int = 0            # 1: the four block matrices in the 8-bit block format
    # input geometry
    batch: int = 1
    frames: int = 1
    height: int = 224
    width: int = 224
    # synthetic-value scales
    std_w: float = 0.02
    std_qk: Optional[float] = None   # sensitised variants: std of the q and k rows of qkv_w
    std_tok: Optional[float] = None  # sensitised variants: std of cls / mod vectors
    seed: int = 1000

    # ---- derived geometry -------------------------------------------------
    @property
    def head_dim(self) -> int:
        return self.embed_dim // self.n_head

    @property
    def is_image(self) -> bool:
        """An image input through the separate one-frame tokenizer."""
        return bool(self.image_patch_embed) and self.frames == 1

    @property
    def input_tubelet(self) -> int:
        return 1 if self.is_image else self.tubelet_size

    @property
    def grid(self):
        return (self.frames // self.input_tubelet, self.height // self.patch_size,
                self.width // self.patch_size)

    @property
    def n_patches(self) -> int:
        gt, gh, gw = self.grid
        return gt * gh * gw

    @property
    def n_prefix(self) -> int:
        return 1 if self.cls_token else 0

    @property
    def n_tokens(self) -> int:
        return self.n_patches + self.n_prefix

    @property
    def table_grid(self):
        """The (t, h, w) grid the position table was built for."""
        return tuple(self.pos_grid) if self.pos_grid is not None else self.grid

    @property
    def pos_grid_t(self) -> int:
        return self.table_grid[0] if self.pos_interp else 0

    @property
    def pos_grid_h(self) -> int:
        return self.table_grid[1] if self.pos_interp else 0

    @property
    def pos_grid_w(self) -> int:
        return self.table_grid[2] if self.pos_interp else 0

    @property
    def pos_rows(self) -> int:
        if self.pos_type != POS_TABLE:
            return 0
        t, h, w = self.table_grid
        return t * h * w + self.n_prefix

    @property
    def patch_k(self) -> int:
        return self.in_chans * self.input_tubelet * self.patch_size * self.patch_size

    def replace(self, **kw) -> "EncoderConfig":
        return dataclasses.replace(self, **kw)

    def hparams(self) -> Dict[str, float]:
        """The fields that form the library's hyperparameter struct."""
        keys = ["embed_dim", "n_layer", "n_head", "ffn_dim", "patch_size", "tubelet_size",
                "in_chans", "ln_eps", "rope_theta", "pos_type", "rope", "rope_layout",
                "rope_interpolate", "rope_ref_grid", "cls_token", "modality_embed",
                "layer_scale", "attn_mode", "dtype", "pos_interp"]
        hp = {k: getattr(self, k) for k in keys}
        hp["pos_rows"] = self.pos_rows
        hp["image_patch_embed"] = self.image_patch_embed
        hp["n_hier"] = len(self.hier_layers)
        hp["hier_layers"] = tuple(self.hier_layers)
        hp["pos_grid_t"], hp["pos_grid_h"], hp["pos_grid_w"] = self.table_grid if self.pos_interp else (0, 0, 0)
        hp["weight_format"] = self.weight_format
        return hp

    def flops(self) -> float:
        """Algorithmic FLOPs of one forward: 2*M*N*K per GEMM plus 4*D per
        visible (query, key) pair per layer (softmax, LN, GELU not counted)."""
        B, N, D, F, L = self.batch, self.n_tokens, self.embed_dim, self.ffn_dim, self.n_layer
        Np = self.n_patches
        f = 2.0 * B * Np * self.patch_k * D
        M = B * N
        f += L * 2.0 * M * D * (3 * D + D + 2 * F)
        f += L * 4.0 * D * B * self.visible_pairs()
        return f

    def visible_pairs(self) -> int:
        """Visible (query, key) pairs of one item's attention (closed form)."""
        N = self.n_tokens
        if self.attn_mode == ATTN_FULL:
            return N * N
        p = self.n_prefix
        gt, gh, gw = self.grid
        S = gh * gw
        # prefix rows see all N keys; a patch query of frame f sees (f+1)*S patch keys
        return p * N + S * S * sum(f + 1 for f in range(gt))


def _configs() -> List[EncoderConfig]:
    c1 = EncoderConfig(name="vit_ti14_hfvit_image", embed_dim=192, n_layer=12, n_head=3, ffn_dim=768,
                       patch_size=14, tubelet_size=1, pos_type=POS_TABLE, pos_kind="learned",
                       cls_token=1, dtype=DTYPE_F32, batch=1, frames=1, height=224, width=224,
                       seed=1000)
    c2 = EncoderConfig(name="vit_l16_ijepa_image", embed_dim=1024, n_layer=24, n_head=16, ffn_dim=4096,
                       patch_size=16, tubelet_size=1, pos_type=POS_TABLE, pos_kind="sincos2d",
                       dtype=DTYPE_BF16, batch=8, frames=1, height=224, width=224, seed=1001)
    c3 = EncoderConfig(name="vjepa2_vit_l_video", embed_dim=1024, n_layer=24, n_head=16, ffn_dim=4096,
                       patch_size=16, tubelet_size=2, rope=ROPE_3D, rope_layout=LAYOUT_TILED,
                       dtype=DTYPE_BF16, batch=2, frames=16, height=256, width=256, seed=1002)
    c4 = EncoderConfig(name="vjepa21_vit_g_video", embed_dim=1408, n_layer=40, n_head=22, ffn_dim=6144,
                       patch_size=16, tubelet_size=2, rope=ROPE_3D, rope_layout=LAYOUT_INTERLEAVED,
                       rope_interpolate=1, rope_ref_grid=256 // 16, modality_embed=1,
                       dtype=DTYPE_BF16, batch=1, frames=64, height=384, width=384, seed=1003)
    c5 = EncoderConfig(name="levjepa_vit_l_blockcausal", embed_dim=1024, n_layer=24, n_head=16,
                       ffn_dim=4096, patch_size=16, tubelet_size=1, rope=ROPE_3D,
                       rope_layout=LAYOUT_TILED, cls_token=1, attn_mode=ATTN_BLOCK_CAUSAL,
                       dtype=DTYPE_BF16, batch=1, frames=16, height=256, width=256, seed=1004)
    return [c1, c2, c3, c4, c5]


CONFIGS: List[EncoderConfig] = _configs()
BY_NAME: Dict[str, EncoderConfig] = {c.name: c for c in CONFIGS}
# the headline workload: V-JEPA-2-style ViT-L video encoder, 2 clips x 2048 tokens
HEADLINE = CONFIGS[2]


def sensitised(cfg: EncoderConfig, std_qk: float = 0.2, std_tok: float = 1.0) -> EncoderConfig:
    """Variant whose attention is far from uniform (large q/k rows) and whose
    prefix / modality vectors are large, so that position, mask and token-
    assembly mistakes become visible at the parity gates."""
    return cfg.replace(name=cfg.name + "_sensitised", std_qk=std_qk, std_tok=std_tok)


# ---------------------------------------------------------------------------
# storage rounding (not a step of the method: it defines the weight values)
# ---------------------------------------------------------------------------
def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = np.isnan(x)
    r = ((u.astype(np.uint64) + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def quantise(x: np.ndarray, dtype: int):
    """Returns (storage array for the device, exact fp32 values)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == DTYPE_F32:
        return x, x
    if dtype == DTYPE_BF16:
        b = round_bf16(x)
        return b, bf16_bits_to_f32(b)
    if dtype == DTYPE_F16:
        h = x.astype(np.float16)
        return h, h.astype(np.float32)
    raise ValueError(dtype)


def sincos2d_table(gh: int, gw: int, dim: int, w_first: bool = True) -> np.ndarray:
    """2-D sine-cosine position table [gh*gw, dim] (the standard MAE-style
    construction: dim/2 columns per axis, each [sin | cos] over dim/4
    frequencies 10000^(-k/(dim/4))).  With w_first the w-axis half comes
    first, as in the I-JEPA checkpoint table described on the schema page."""
    assert dim % 4 == 0
    q = dim // 4
    omega = 1.0 / 10000.0 ** (np.arange(q, dtype=np.float64) / q)

    def axis(pos):
        a = np.outer(pos, omega)
        return np.concatenate([np.sin(a), np.cos(a)], axis=1)

    hh, ww = np.meshgrid(np.arange(gh, dtype=np.float64), np.arange(gw, dtype=np.float64),
                         indexing="ij")
    eh, ew = axis(hh.reshape(-1)), axis(ww.reshape(-1))
    t = np.concatenate([ew, eh] if w_first else [eh, ew], axis=1)
    return t.astype(np.float32)


# ---------------------------------------------------------------------------
# weights
# ---------------------------------------------------------------------------
@dataclass
class Block:
    qkv_w: np.ndarray
    qkv_b: np.ndarray
    out_w: np.ndarray
    out_b: np.ndarray
    up_w: np.ndarray
    up_b: np.ndarray
    down_w: np.ndarray
    down_b: np.ndarray
    ln1_w: np.ndarray
    ln1_b: np.ndarray
    ln2_w: np.ndarray
    ln2_b: np.ndarray
    ls1: Optional[np.ndarray] = None
    ls2: Optional[np.ndarray] = None
    # device storage of the matrices (bf16 bits / f16 / f32)
    store: Dict[str, np.ndarray] = field(default_factory=dict)


@dataclass
class Weights:
    patch_w: np.ndarray
    patch_b: np.ndarray
    pos: Optional[np.ndarray]
    cls: Optional[np.ndarray]
    mod: Optional[np.ndarray]
    blocks: List[Block]
    norm_w: np.ndarray
    norm_b: np.ndarray
    store: Dict[str, np.ndarray] = field(default_factory=dict)
    # the separate one-frame tokenizer and its modality vector
    patch_img_w: Optional[np.ndarray] = None
    patch_img_b: Optional[np.ndarray] = None
    mod_img: Optional[np.ndarray] = None
    # one norm per hierarchical output
    hier_norm_w: List[np.ndarray] = field(default_factory=list)
    hier_norm_b: List[np.ndarray] = field(default_factory=list)


@dataclass
class Workload:
    cfg: EncoderConfig
    pixels: np.ndarray        # fp32 [B, C, T, H, W]
    weights: Weights


def _normal(rng, shape, std):
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


def make_workload(cfg: EncoderConfig, seed: Optional[int] = None) -> Workload:
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    B, C, T, H, W = cfg.batch, cfg.in_chans, cfg.frames, cfg.height, cfg.width
    D, F = cfg.embed_dim, cfg.ffn_dim
    dt = cfg.dtype
    pixels = rng.standard_normal((B, C, T, H, W), dtype=np.float32)

    wstore = {}
    kvid = cfg.in_chans * cfg.tubelet_size * cfg.patch_size * cfg.patch_size
    pw_s, pw = quantise(_normal(rng, (D, kvid), cfg.std_w), dt)
    wstore["patch_w"] = pw_s
    pb = _normal(rng, (D,), cfg.std_w)

    pos = cls = mod = None
    std_tok = cfg.std_w if cfg.std_tok is None else cfg.std_tok
    if cfg.pos_type == POS_TABLE:
        # the table is built for its own grid (the input grid unless pos_grid says otherwise)
        if cfg.pos_kind == "sincos2d":
            gt, gh, gw = cfg.table_grid
            assert gt == 1 and not cfg.cls_token
            pos = sincos2d_table(gh, gw, D, w_first=True)
        else:
            pos = _normal(rng, (cfg.pos_rows, D), cfg.std_w)
    if cfg.cls_token:
        cls = _normal(rng, (D,), std_tok)
    if cfg.modality_embed:
        mod = _normal(rng, (D,), std_tok)

    ones = np.ones(D, np.float32)
    zeros = np.zeros(D, np.float32)
    blocks = []
    # 8-bit block weights are quantised from the fp32 draws (by each side's own
    # quantiser), so those four matrices keep their fp32 values here
    mdt = DTYPE_F32 if cfg.weight_format == WEIGHTS_MXFP8 else dt
    for _ in range(cfg.n_layer):
        st = {}
        qkv = _normal(rng, (3 * D, D), cfg.std_w)
        if cfg.std_qk is not None:
            qkv[: 2 * D] *= np.float32(cfg.std_qk / cfg.std_w)
        st["qkv_w"], qkv_w = quantise(qkv, mdt)
        qkv_b = _normal(rng, (3 * D,), cfg.std_w)
        st["out_w"], out_w = quantise(_normal(rng, (D, D), cfg.std_w), mdt)
        out_b = _normal(rng, (D,), cfg.std_w)
        st["up_w"], up_w = quantise(_normal(rng, (F, D), cfg.std_w), mdt)
        up_b = _normal(rng, (F,), cfg.std_w)
        st["down_w"], down_w = quantise(_normal(rng, (D, F), cfg.std_w), mdt)
        down_b = _normal(rng, (D,), cfg.std_w)
        ls1 = ls2 = None
        if cfg.layer_scale:
            ls1 = (1.0 + 0.1 * rng.standard_normal(D, dtype=np.float32)).astype(np.float32)
            ls2 = (1.0 + 0.1 * rng.standard_normal(D, dtype=np.float32)).astype(np.float32)
        blocks.append(Block(qkv_w, qkv_b, out_w, out_b, up_w, up_b, down_w, down_b,
                            ones, zeros, ones, zeros, ls1, ls2, st))
    w = Weights(pw, pb, pos, cls, mod, blocks, ones, zeros, wstore)
    # drawn last, so that the draws above do not depend on these options
    if cfg.image_patch_embed:
        kimg = cfg.in_chans * cfg.patch_size * cfg.patch_size
        wstore["patch_img_w"], w.patch_img_w = quantise(_normal(rng, (D, kimg), cfg.std_w), dt)
        w.patch_img_b = _normal(rng, (D,), cfg.std_w)
        if cfg.modality_embed:
            w.mod_img = _normal(rng, (D,), std_tok)
    for _ in cfg.hier_layers:
        w.hier_norm_w.append((1.0 + 0.1 * rng.standard_normal(D, dtype=np.float32)).astype(np.float32))
        w.hier_norm_b.append((0.1 * rng.standard_normal(D, dtype=np.float32)).astype(np.float32))
    return Workload(cfg, pixels, w)


# ---------------------------------------------------------------------------
# masked predictor (the V-JEPA 2 latent predictor that follows the encoder)
# ---------------------------------------------------------------------------
@dataclass
class PredictorConfig:
    """A masked-latent predictor: context encoder features are projected to
    embed_dim, joined by a mask token at every target position, put in token
    order, run through n_layer pre-LN blocks with 3-D RoPE on the token
    positions, normalised, and the target rows projected back to enc_dim."""
    name: str
    embed_dim: int = 384
    enc_dim: int = 1024
    n_layer: int = 12
    n_head: int = 12
    ffn_dim: int = 1536
    n_mask_tokens: int = 10
    ln_eps: float = 1e-6
    rope_theta: float = 10000.0
    rope_layout: int = LAYOUT_TILED
    grid: tuple = (8, 16, 16)
    batch: int = 2
    n_ctx: int = 1024
    n_tgt: int = 1024
    mask_index: int = 1
    dtype: int = DTYPE_BF16
    std_w: float = 0.02
    std_tok: float = 0.02
    seed: int = 2000
    # V-JEPA 2.1 options: output width (0: enc_dim), hierarchical encoder
    # levels concatenated into a 2-layer embed MLP of embed_hidden units,
    # modality vectors, and the projection of the context rows
    out_dim: int = 0
    n_hier_in: int = 1
    embed_hidden: int = 0
    modality_embed: int = 0
    context_proj: int = 0

    @property
    def head_dim(self) -> int:
        return self.embed_dim // self.n_head

    @property
    def n_grid(self) -> int:
        return self.grid[0] * self.grid[1] * self.grid[2]

    @property
    def n_tokens(self) -> int:
        return self.n_ctx + self.n_tgt

    def replace(self, **kw) -> "PredictorConfig":
        d = dict(self.__dict__)
        d.update(kw)
        return PredictorConfig(**d)

    def hparams(self) -> Dict:
        return dict(embed_dim=self.embed_dim, enc_dim=self.enc_dim, n_layer=self.n_layer, n_head=self.n_head,
                    ffn_dim=self.ffn_dim, n_mask_tokens=self.n_mask_tokens, ln_eps=self.ln_eps,
                    rope_theta=self.rope_theta, rope_layout=self.rope_layout, grid=tuple(self.grid),
                    dtype=self.dtype, out_dim=self.out_width, n_hier_in=self.n_hier_in,
                    embed_hidden=self.embed_hidden, modality_embed=self.modality_embed,
                    context_proj=self.context_proj)

    @property
    def out_width(self) -> int:
        return self.out_dim or self.enc_dim

    def flops(self) -> float:
        M, D, F, De = self.batch * self.n_tokens, self.embed_dim, self.ffn_dim, self.enc_dim
        per_layer = 2.0 * M * D * (3 * D + D + 2 * F) + 4.0 * D * self.batch * self.n_tokens ** 2
        if self.n_hier_in > 1:
            embed = 2.0 * self.batch * self.n_ctx * (self.n_hier_in * De * self.embed_hidden + self.embed_hidden * D)
        else:
            embed = 2.0 * self.batch * self.n_ctx * De * D
        proj = 2.0 * self.batch * (self.n_tgt + (self.n_ctx if self.context_proj else 0)) * D * self.out_width
        return embed + self.n_layer * per_layer + proj


# V-JEPA 2 ViT-L predictor shape: 12 blocks of width 384, 12 heads of 32, on the
# 8 x 16 x 16 token grid of a 16-frame 256-px clip, half the tokens as context
PREDICTOR = PredictorConfig("vjepa2_predictor")
# V-JEPA 2.1 predictor shapes (8 mask tokens, interleaved RoPE, modality
# vectors, the projection of the context rows, out_dim the teacher's width):
# after a ViT-L encoder (one hierarchical level) and after a ViT-g encoder
# (four levels of width 1408 concatenated into a 2-layer embed MLP), on the
# 8 x 16 x 16 grid of a 16-frame 256-px clip and the 8 x 24 x 24 grid of a
# 16-frame 384-px clip
PREDICTOR_21_L = PredictorConfig("vjepa21_predictor_vit_l", n_mask_tokens=8, rope_layout=LAYOUT_INTERLEAVED,
                                 out_dim=1664, modality_embed=1, context_proj=1, mask_index=0, seed=2100)
PREDICTOR_21_G = PredictorConfig("vjepa21_predictor_vit_g", enc_dim=1408, n_mask_tokens=8,
                                 rope_layout=LAYOUT_INTERLEAVED, out_dim=1664, n_hier_in=4, embed_hidden=1536,
                                 modality_embed=1, context_proj=1, mask_index=0, grid=(8, 24, 24), n_ctx=1152,
                                 n_tgt=1152, batch=1, seed=2101)


@dataclass
class PredictorWeights:
    embed_w: np.ndarray          # [embed_dim, enc_dim]
    embed_b: np.ndarray
    mask_tokens: np.ndarray      # [n_mask_tokens, embed_dim]
    blocks: List[Block]
    norm_w: np.ndarray
    norm_b: np.ndarray
    proj_w: np.ndarray           # [out_dim, embed_dim]
    proj_b: np.ndarray
    store: Dict[str, np.ndarray] = field(default_factory=dict)
    # V-JEPA 2.1 options (None when off); with n_hier_in > 1, embed_w / embed_b
    # are the first MLP layer [embed_hidden, n_hier_in * enc_dim]
    embed2_w: Optional[np.ndarray] = None   # [embed_dim, embed_hidden]
    embed2_b: Optional[np.ndarray] = None
    mod_img: Optional[np.ndarray] = None    # [embed_dim]
    mod_video: Optional[np.ndarray] = None
    proj_ctx_w: Optional[np.ndarray] = None  # [out_dim, embed_dim]
    proj_ctx_b: Optional[np.ndarray] = None


@dataclass
class PredictorWorkload:
    cfg: PredictorConfig
    enc_tokens: np.ndarray       # fp32 [B, n_grid, enc_dim] ([n_hier_in, B, n_grid, enc_dim]), unit scale
    ctx_ids: np.ndarray          # int32 [B, n_ctx], strictly increasing
    tgt_ids: np.ndarray          # int32 [B, n_tgt], strictly increasing, disjoint from ctx_ids
    weights: PredictorWeights


def make_predictor_workload(cfg: PredictorConfig, seed: Optional[int] = None) -> PredictorWorkload:
    """Draw order: encoder features, per item a permutation of the grid (the
    first n_ctx ids are the context, the next n_tgt the targets), embed
    weight and bias, mask tokens, the blocks (as the encoder's), proj; then,
    for the V-JEPA 2.1 options that are on, the further hierarchical levels of
    the encoder features, the second embed layer, the image and video
    modality vectors and the context projection (so that configurations
    without them draw exactly what they did before the options existed)."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    B, Ng, De, D, F = cfg.batch, cfg.n_grid, cfg.enc_dim, cfg.embed_dim, cfg.ffn_dim
    assert cfg.n_ctx + cfg.n_tgt <= Ng
    dt = cfg.dtype
    enc = rng.standard_normal((B, Ng, De), dtype=np.float32)
    ctx, tgt = [], []
    for _ in range(B):
        perm = rng.permutation(Ng)
        ctx.append(np.sort(perm[:cfg.n_ctx]))
        tgt.append(np.sort(perm[cfg.n_ctx:cfg.n_ctx + cfg.n_tgt]))
    ctx_ids = np.stack(ctx).astype(np.int32).reshape(B, cfg.n_ctx)
    tgt_ids = np.stack(tgt).astype(np.int32).reshape(B, cfg.n_tgt)
    st = {}
    Hd = cfg.embed_hidden if cfg.n_hier_in > 1 else D
    st["embed_w"], embed_w = quantise(_normal(rng, (Hd, cfg.n_hier_in * De), cfg.std_w), dt)
    embed_b = _normal(rng, (Hd,), cfg.std_w)
    mask_tokens = _normal(rng, (cfg.n_mask_tokens, D), cfg.std_tok)
    ones = np.ones(D, np.float32)
    zeros = np.zeros(D, np.float32)
    blocks = []
    for _ in range(cfg.n_layer):
        bs = {}
        bs["qkv_w"], qkv_w = quantise(_normal(rng, (3 * D, D), cfg.std_w), dt)
        qkv_b = _normal(rng, (3 * D,), cfg.std_w)
        bs["out_w"], out_w = quantise(_normal(rng, (D, D), cfg.std_w), dt)
        out_b = _normal(rng, (D,), cfg.std_w)
        bs["up_w"], up_w = quantise(_normal(rng, (F, D), cfg.std_w), dt)
        up_b = _normal(rng, (F,), cfg.std_w)
        bs["down_w"], down_w = quantise(_normal(rng, (D, F), cfg.std_w), dt)
        down_b = _normal(rng, (D,), cfg.std_w)
        blocks.append(Block(qkv_w, qkv_b, out_w, out_b, up_w, up_b, down_w, down_b,
                            ones, zeros, ones, zeros, None, None, bs))
    Do = cfg.out_width
    st["proj_w"], proj_w = quantise(_normal(rng, (Do, D), cfg.std_w), dt)
    proj_b = _normal(rng, (Do,), cfg.std_w)
    w = PredictorWeights(embed_w, embed_b, mask_tokens, blocks, ones, zeros, proj_w, proj_b, st)
    if cfg.n_hier_in > 1:
        more = rng.standard_normal((cfg.n_hier_in - 1, B, Ng, De), dtype=np.float32)
        enc = np.concatenate([enc[None], more], axis=0)
        st["embed2_w"], w.embed2_w = quantise(_normal(rng, (D, Hd), cfg.std_w), dt)
        w.embed2_b = _normal(rng, (D,), cfg.std_w)
    if cfg.modality_embed:
        w.mod_img = _normal(rng, (D,), cfg.std_tok)
        w.mod_video = _normal(rng, (D,), cfg.std_tok)
    if cfg.context_proj:
        st["proj_ctx_w"], w.proj_ctx_w = quantise(_normal(rng, (Do, D), cfg.std_w), dt)
        w.proj_ctx_b = _normal(rng, (Do,), cfg.std_w)
    return PredictorWorkload(cfg, enc, ctx_ids, tgt_ids, w)


# ---------------------------------------------------------------------------
# attentive-pool head + classifier (jepa.cpp "GGUF schema (v1)", "Head
# (jepa.head.*)"; SkyVision.cpp README, V-JEPA 2 backend notes, the pooler
# and classifier heads)
# ---------------------------------------------------------------------------
@dataclass
class HeadConfig:
    """n_pool_layers self-attention blocks over the encoder's output tokens
    (the encoder block without RoPE or mask), then one learned query attends
    over them (LayerNorm on keys and values only, no output projection), the
    query residual and an MLP, and a linear classifier on the pooled token."""
    name: str
    embed_dim: int = 1024
    n_head: int = 16
    ffn_dim: int = 4096
    n_pool_layers: int = 3
    n_classes: int = 174
    ln_eps: float = 1e-6
    batch: int = 2
    n_tokens: int = 2048
    dtype: int = DTYPE_BF16
    std_w: float = 0.02
    std_query: float = 0.02
    std_qk: float = 0.02         # the cross-attention's q and k weights (sensitised variants raise it)
    ln_random: bool = False      # draw the cross-attention's two LayerNorms instead of (1, 0)
    seed: int = 3000

    @property
    def head_dim(self) -> int:
        return self.embed_dim // self.n_head

    def replace(self, **kw) -> "HeadConfig":
        d = dict(self.__dict__)
        d.update(kw)
        return HeadConfig(**d)

    def hparams(self) -> Dict:
        return dict(embed_dim=self.embed_dim, n_head=self.n_head, ffn_dim=self.ffn_dim,
                    n_pool_layers=self.n_pool_layers, n_classes=self.n_classes, ln_eps=self.ln_eps,
                    dtype=self.dtype)

    def flops(self) -> float:
        """Blocks as GEMMs and attention; the cross-attention as the head
        computes it (the key and value projections folded into the learned
        query: one pass of dot products for the scores and one weighted sum of
        the normalised tokens per head); the MLP and classifier as matrix-
        vector products."""
        B, N, D, F = self.batch, self.n_tokens, self.embed_dim, self.ffn_dim
        M = B * N
        blocks = self.n_pool_layers * (2.0 * M * D * (3 * D + D + 2 * F) + 4.0 * D * B * N * N)
        xattn = 2.0 * D * D * 2 + 2.0 * M * D * self.n_head * 2 + 2.0 * B * D * D
        tail = 2.0 * B * (2 * D * F + D * self.n_classes)
        return blocks + xattn + tail


# the attentive-pool classifier of a V-JEPA 2 ViT-L video model (3 pooler
# blocks, 16 heads of 64, 174 classes) on the 2 x 2048 tokens of two clips
HEAD = HeadConfig("vjepa2_attentive_pool")


@dataclass
class HeadWeights:
    blocks: List[Block]
    query: np.ndarray            # [embed_dim]
    ln_kv_w: np.ndarray
    ln_kv_b: np.ndarray
    q_w: np.ndarray              # [embed_dim, embed_dim]
    q_b: np.ndarray
    k_w: np.ndarray
    k_b: np.ndarray
    v_w: np.ndarray
    v_b: np.ndarray
    ln2_w: np.ndarray
    ln2_b: np.ndarray
    up_w: np.ndarray             # [ffn_dim, embed_dim]
    up_b: np.ndarray
    down_w: np.ndarray           # [embed_dim, ffn_dim]
    down_b: np.ndarray
    cls_w: np.ndarray            # [n_classes, embed_dim]
    cls_b: np.ndarray
    store: Dict[str, np.ndarray] = field(default_factory=dict)


@dataclass
class HeadWorkload:
    cfg: HeadConfig
    tokens: np.ndarray           # fp32 [B, n_tokens, embed_dim]: the encoder's output features
    weights: HeadWeights


def make_head_workload(cfg: HeadConfig, seed: Optional[int] = None) -> HeadWorkload:
    """Draw order: the input tokens ~N(0, 1) (the encoder's final-LayerNorm
    output is unit-scale per token); per pooler block as the encoder's; the
    query; the cross-attention's q, k, v weights and biases; the MLP; the
    classifier; last, the two LayerNorms' (gamma, beta) when ln_random."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    B, N, D, F, C = cfg.batch, cfg.n_tokens, cfg.embed_dim, cfg.ffn_dim, cfg.n_classes
    dt = cfg.dtype
    tokens = rng.standard_normal((B, N, D), dtype=np.float32)
    ones = np.ones(D, np.float32)
    zeros = np.zeros(D, np.float32)
    blocks = []
    for _ in range(cfg.n_pool_layers):
        bs = {}
        bs["qkv_w"], qkv_w = quantise(_normal(rng, (3 * D, D), cfg.std_w), dt)
        qkv_b = _normal(rng, (3 * D,), cfg.std_w)
        bs["out_w"], out_w = quantise(_normal(rng, (D, D), cfg.std_w), dt)
        out_b = _normal(rng, (D,), cfg.std_w)
        bs["up_w"], up_w = quantise(_normal(rng, (F, D), cfg.std_w), dt)
        up_b = _normal(rng, (F,), cfg.std_w)
        bs["down_w"], down_w = quantise(_normal(rng, (D, F), cfg.std_w), dt)
        down_b = _normal(rng, (D,), cfg.std_w)
        blocks.append(Block(qkv_w, qkv_b, out_w, out_b, up_w, up_b, down_w, down_b,
                            ones, zeros, ones, zeros, None, None, bs))
    st = {}
    query = _normal(rng, (D,), cfg.std_query)
    st["q_w"], q_w = quantise(_normal(rng, (D, D), cfg.std_qk), dt)
    q_b = _normal(rng, (D,), cfg.std_w)
    st["k_w"], k_w = quantise(_normal(rng, (D, D), cfg.std_qk), dt)
    k_b = _normal(rng, (D,), cfg.std_w)
    st["v_w"], v_w = quantise(_normal(rng, (D, D), cfg.std_w), dt)
    v_b = _normal(rng, (D,), cfg.std_w)
    st["up_w"], up_w = quantise(_normal(rng, (F, D), cfg.std_w), dt)
    up_b = _normal(rng, (F,), cfg.std_w)
    st["down_w"], down_w = quantise(_normal(rng, (D, F), cfg.std_w), dt)
    down_b = _normal(rng, (D,), cfg.std_w)
    st["cls_w"], cls_w = quantise(_normal(rng, (C, D), cfg.std_w), dt)
    cls_b = _normal(rng, (C,), cfg.std_w)
    ln = [ones, zeros, ones, zeros]
    if cfg.ln_random:
        ln = [np.float32(1) + _normal(rng, (D,), 0.2), _normal(rng, (D,), 0.2),
              np.float32(1) + _normal(rng, (D,), 0.2), _normal(rng, (D,), 0.2)]
    w = HeadWeights(blocks, query, ln[0], ln[1], q_w, q_b, k_w, k_b, v_w, v_b, ln[2], ln[3],
                    up_w, up_b, down_w, down_b, cls_w, cls_b, st)
    return HeadWorkload(cfg, tokens, w)
