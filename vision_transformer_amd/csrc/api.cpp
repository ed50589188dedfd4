// C ABI of the encoder (include/vitenc.h): validation, workspace planning and
// the launch sequence of one forward.  Every refusal happens here, before any
// device work is enqueued; the kernels assume the shapes validated here.
#include "vitenc.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>
#include <vector>

#include "launch.h"

using namespace vitenc;

struct vitenc_model {
    vitenc_hparams hp;
    vitenc_weights w;
    std::vector<vitenc_block_weights> blocks;
};

namespace {
thread_local std::string g_error;
} // namespace

namespace vitenc {
vitenc_status fail(vitenc_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return st;
}
void clear_error() { g_error.clear(); }

vitenc_status device_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return VITENC_OK;
    return fail(VITENC_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}
} // namespace vitenc

namespace {

constexpr int64_t kMaxTokens = int64_t(1) << 22;   // per item, as the pages' loader limit
constexpr int kMaxGrid = 1023;                     // per axis (packed 10-bit positions)
constexpr int kMaxEmbed = 4096;                    // LayerNorm keeps a row in one wave's registers

bool in_range(int64_t v, int64_t lo, int64_t hi) { return v >= lo && v <= hi; }
bool valid_dtype(int dt) { return dt == VITENC_F32 || dt == VITENC_BF16 || dt == VITENC_F16; }
int64_t rup(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

vitenc_status validate_hparams(const vitenc_hparams *hp) {
    if (!hp) return fail(VITENC_ENULL, "hparams is NULL");
    if (!in_range(hp->embed_dim, 1, 65536)) return fail(VITENC_EINVAL, "embed_dim %d outside 1..65536", hp->embed_dim);
    if (!in_range(hp->n_layer, 1, 1024)) return fail(VITENC_EINVAL, "n_layer %d outside 1..1024", hp->n_layer);
    if (!in_range(hp->n_head, 1, 1024)) return fail(VITENC_EINVAL, "n_head %d outside 1..1024", hp->n_head);
    if (!in_range(hp->ffn_dim, 1, 1 << 20)) return fail(VITENC_EINVAL, "ffn_dim %d outside 1..2^20", hp->ffn_dim);
    if (!in_range(hp->patch_size, 1, 1024)) return fail(VITENC_EINVAL, "patch_size %d outside 1..1024", hp->patch_size);
    if (!in_range(hp->tubelet_size, 1, 1024))
        return fail(VITENC_EINVAL, "tubelet_size %d outside 1..1024", hp->tubelet_size);
    if (!in_range(hp->in_chans, 1, 1024)) return fail(VITENC_EINVAL, "in_chans %d outside 1..1024", hp->in_chans);
    if (!std::isfinite(hp->ln_eps) || hp->ln_eps < 0.0f || hp->ln_eps > 1.0f)
        return fail(VITENC_EINVAL, "ln_eps %g not a finite value in [0, 1]", (double)hp->ln_eps);
    if (!valid_dtype(hp->dtype)) return fail(VITENC_EINVAL, "unknown dtype %d", hp->dtype);
    if (hp->pos_type != VITENC_POS_NONE && hp->pos_type != VITENC_POS_TABLE)
        return fail(VITENC_EINVAL, "unknown pos_type %d", hp->pos_type);
    if (hp->rope != VITENC_ROPE_NONE && hp->rope != VITENC_ROPE_3D) return fail(VITENC_EINVAL, "unknown rope %d", hp->rope);
    if (hp->rope_layout != VITENC_ROPE_TILED && hp->rope_layout != VITENC_ROPE_INTERLEAVED)
        return fail(VITENC_EINVAL, "unknown rope_layout %d", hp->rope_layout);
    if (hp->attn_mode != VITENC_ATTN_FULL && hp->attn_mode != VITENC_ATTN_BLOCK_CAUSAL)
        return fail(VITENC_EINVAL, "unknown attn_mode %d", hp->attn_mode);
    if (hp->embed_dim % hp->n_head != 0)
        return fail(VITENC_EINVAL, "embed_dim %d not divisible by n_head %d", hp->embed_dim, hp->n_head);
    const int hd = hp->embed_dim / hp->n_head;
    if (hp->rope == VITENC_ROPE_3D) {
        if (!std::isfinite(hp->rope_theta) || hp->rope_theta <= 0.0f)
            return fail(VITENC_EINVAL, "rope_theta %g must be finite and > 0", (double)hp->rope_theta);
        if (hd % 2 != 0) return fail(VITENC_EINVAL, "head_dim %d is odd; 3-D RoPE rotates pairs", hd);
        if (2 * ((hd / 3) / 2) < 2) return fail(VITENC_EINVAL, "head_dim %d leaves no rotated pair per axis", hd);
        if (hp->rope_interpolate && hp->rope_ref_grid <= 0)
            return fail(VITENC_EINVAL, "rope_interpolate without a rope_ref_grid to rescale from");
    } else if (hp->rope_interpolate) {
        return fail(VITENC_EINVAL, "rope_interpolate set on a model without 3-D RoPE");
    }
    if (hp->attn_mode == VITENC_ATTN_BLOCK_CAUSAL && hp->rope != VITENC_ROPE_3D)
        return fail(VITENC_EINVAL, "block_causal attention on a model without a frame grid (rope3d)");
    if (hp->pos_type == VITENC_POS_TABLE && hp->pos_rows <= 0)
        return fail(VITENC_EINVAL, "pos_type TABLE with pos_rows %d", hp->pos_rows);
    if (hp->pos_interp != VITENC_POS_INTERP_NONE && hp->pos_interp != VITENC_POS_INTERP_BICUBIC &&
        hp->pos_interp != VITENC_POS_INTERP_TRILINEAR)
        return fail(VITENC_EINVAL, "unknown pos_interp %d", hp->pos_interp);
    if (hp->pos_interp != VITENC_POS_INTERP_NONE) {
        if (hp->pos_type != VITENC_POS_TABLE) return fail(VITENC_EINVAL, "pos_interp set without a position table");
        if (!in_range(hp->pos_grid_t, 1, kMaxGrid) || !in_range(hp->pos_grid_h, 1, kMaxGrid) ||
            !in_range(hp->pos_grid_w, 1, kMaxGrid))
            return fail(VITENC_EINVAL, "position table grid %dx%dx%d outside 1..%d per axis", hp->pos_grid_t,
                        hp->pos_grid_h, hp->pos_grid_w, kMaxGrid);
        const int64_t rows = (int64_t)hp->pos_grid_t * hp->pos_grid_h * hp->pos_grid_w + (hp->cls_token ? 1 : 0);
        if (rows != hp->pos_rows)
            return fail(VITENC_EINVAL, "pos_rows %d but the table grid %dx%dx%d%s makes %lld", hp->pos_rows,
                        hp->pos_grid_t, hp->pos_grid_h, hp->pos_grid_w, hp->cls_token ? " + CLS" : "",
                        (long long)rows);
        if (hp->pos_interp == VITENC_POS_INTERP_BICUBIC && hp->pos_grid_t != 1)
            return fail(VITENC_EINVAL, "bicubic position resampling needs a one-frame table");
    }
    if (hp->image_patch_embed != 0 && hp->image_patch_embed != 1)
        return fail(VITENC_EINVAL, "image_patch_embed %d is not 0 or 1", hp->image_patch_embed);
    if (!in_range(hp->n_hier, 0, VITENC_MAX_HIER))
        return fail(VITENC_EINVAL, "n_hier %d outside 0..%d", hp->n_hier, VITENC_MAX_HIER);
    for (int k = 0; k < hp->n_hier; ++k) {
        if (!in_range(hp->hier_layers[k], 0, hp->n_layer - 1) || (k > 0 && hp->hier_layers[k] <= hp->hier_layers[k - 1]))
            return fail(VITENC_EINVAL, "hier_layers must strictly increase within [0, n_layer): entry %d is %d", k,
                        hp->hier_layers[k]);
    }
    if (hp->weight_format != VITENC_WEIGHTS_PLAIN && hp->weight_format != VITENC_WEIGHTS_MXFP8)
        return fail(VITENC_EINVAL, "unknown weight_format %d", hp->weight_format);
    if (hp->weight_format == VITENC_WEIGHTS_MXFP8) {
        if (hp->dtype != VITENC_BF16) return fail(VITENC_EUNSUPPORTED, "8-bit weights run with dtype BF16 only");
        if (hp->embed_dim % 64 || hp->ffn_dim % 64)
            return fail(VITENC_EINVAL, "8-bit weights need embed_dim and ffn_dim multiples of 64 (got %d, %d)",
                        hp->embed_dim, hp->ffn_dim);
    }
    if (hd != 64 && hd != 32)
        return fail(VITENC_EUNSUPPORTED, "head_dim %d: the attention kernel implements 64 and 32", hd);
    if (hp->embed_dim > kMaxEmbed)
        return fail(VITENC_EUNSUPPORTED, "embed_dim %d above %d", hp->embed_dim, kMaxEmbed);
    return VITENC_OK;
}

struct Plan {
    bool image;
    int tub;
    int B, C, T, H, W;
    int gt, gh, gw, Np, p, N;
    int64_t M;
    int D, F, nh, hd, K, lda, ldv;
    size_t off_Z, off_Y, off_Q, off_K, off_V, off_O, off_U, off_A, off_rope, off_tok, off_pos, off_attn, total;
    size_t off_skp;           // split-K partials (sk_floats == 0: none)
    int64_t sk_floats;
    bool resample;
};

vitenc_status make_plan(const vitenc_model *m, int32_t B, int32_t T, int32_t H, int32_t W, Plan &pl) {
    const vitenc_hparams &hp = m->hp;
    if (B <= 0 || T <= 0 || H <= 0 || W <= 0)
        return fail(VITENC_ESHAPE, "non-positive input shape B=%d T=%d H=%d W=%d", B, T, H, W);
    // a one-frame input of a model with an image tokenizer goes through it
    pl.image = hp.image_patch_embed && T == 1;
    pl.tub = pl.image ? 1 : hp.tubelet_size;
    if (T % pl.tub) return fail(VITENC_ESHAPE, "T=%d not a multiple of tubelet_size %d", T, pl.tub);
    if (H % hp.patch_size || W % hp.patch_size)
        return fail(VITENC_ESHAPE, "H=%d / W=%d not multiples of patch_size %d", H, W, hp.patch_size);
    pl.B = B; pl.C = hp.in_chans; pl.T = T; pl.H = H; pl.W = W;
    pl.gt = T / pl.tub; pl.gh = H / hp.patch_size; pl.gw = W / hp.patch_size;
    if (pl.gt > kMaxGrid || pl.gh > kMaxGrid || pl.gw > kMaxGrid)
        return fail(VITENC_ESHAPE, "token grid %dx%dx%d exceeds %d per axis", pl.gt, pl.gh, pl.gw, kMaxGrid);
    const int64_t np = (int64_t)pl.gt * pl.gh * pl.gw;
    pl.p = hp.cls_token ? 1 : 0;
    if (np + pl.p > kMaxTokens) return fail(VITENC_ESHAPE, "%lld tokens per item exceed 2^22", (long long)(np + pl.p));
    pl.Np = (int)np;
    pl.N = pl.Np + pl.p;
    pl.M = (int64_t)B * pl.N;
    if (pl.M > (int64_t(1) << 30)) return fail(VITENC_ESHAPE, "B*N = %lld rows exceed 2^30", (long long)pl.M);
    pl.resample = hp.pos_interp != VITENC_POS_INTERP_NONE &&
                  (hp.pos_grid_t != pl.gt || hp.pos_grid_h != pl.gh || hp.pos_grid_w != pl.gw);
    if (hp.pos_type == VITENC_POS_TABLE && !pl.resample && hp.pos_rows != pl.N)
        return fail(VITENC_ESHAPE, "position table has %d rows but the input makes %d tokens", hp.pos_rows, pl.N);
    if (pl.resample && hp.pos_interp == VITENC_POS_INTERP_BICUBIC && pl.gt != 1)
        return fail(VITENC_ESHAPE, "bicubic position resampling of a %d-frame token grid", pl.gt);
    pl.D = hp.embed_dim; pl.F = hp.ffn_dim; pl.nh = hp.n_head; pl.hd = pl.D / pl.nh;
    pl.K = hp.in_chans * pl.tub * hp.patch_size * hp.patch_size;
    pl.lda = embed_lda(hp.dtype, pl.K);
    pl.ldv = (int)rup(pl.N, 64);
    const size_t es = (size_t)dtype_size(hp.dtype);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = (size_t)rup((int64_t)(off + bytes), 256);
        return o;
    };
    pl.off_Z = take((size_t)pl.M * pl.D * 4);
    pl.off_Y = take((size_t)pl.M * pl.D * es);
    pl.off_Q = take((size_t)pl.M * pl.D * es);
    pl.off_K = take((size_t)pl.M * pl.D * es);
    pl.off_V = take((size_t)B * pl.nh * pl.hd * pl.ldv * es);
    pl.off_O = take((size_t)pl.M * pl.D * es);
    pl.off_U = take((size_t)pl.M * pl.F * es);
    pl.off_A = take((size_t)B * pl.Np * pl.lda * es);
    const int d = 2 * ((pl.hd / 3) / 2);
    pl.off_rope = take((size_t)(pl.gt + pl.gh + pl.gw) * d * 2 * 4);
    pl.off_tok = take((size_t)pl.Np * 4);
    pl.off_pos = pl.resample ? take((size_t)pl.N * pl.D * 4) : 0;
    pl.off_attn = take(
        (size_t)attention_scratch_floats(hp.dtype, B, pl.N, pl.nh, pl.hd, hp.attn_mode, pl.p, pl.gh * pl.gw) * 4);
    // split-K scratch for the GEMMs whose tiles leave most CUs idle (small inputs)
    {
        const bool wq = hp.weight_format == VITENC_WEIGHTS_MXFP8;
        const int Kp = pl.lda == 2 * pl.K ? 2 * pl.K : pl.K, Mi = (int)pl.M;
        pl.sk_floats = std::max<int64_t>({gemm_splitk_floats(hp.dtype, EPI_PATCH, B * pl.Np, pl.D, Kp, false),
                                          gemm_splitk_floats(hp.dtype, EPI_QKV, Mi, 3 * pl.D, pl.D, wq),
                                          gemm_splitk_floats(hp.dtype, EPI_RESID, Mi, pl.D, pl.D, wq),
                                          gemm_splitk_floats(hp.dtype, EPI_GELU, Mi, pl.F, pl.D, wq),
                                          gemm_splitk_floats(hp.dtype, EPI_RESID, Mi, pl.D, pl.F, wq)});
    }
    pl.off_skp = pl.sk_floats ? take((size_t)pl.sk_floats * 4) : 0;
    pl.total = off;
    return VITENC_OK;
}

#define CHECK_DEV(expr, what)                                                                                     \
    do {                                                                                                          \
        vitenc_status st_ = device_status((expr), what);                                                          \
        if (st_ != VITENC_OK) return st_;                                                                         \
    } while (0)

} // namespace

extern "C" {

int32_t vitenc_abi_version(void) { return VITENC_ABI_VERSION; }

const char *vitenc_error_text(void) { return g_error.c_str(); }

vitenc_status vitenc_model_create(const vitenc_hparams *hp, const vitenc_weights *w, vitenc_model **out) {
    g_error.clear();
    if (!out) return fail(VITENC_ENULL, "out is NULL");
    *out = nullptr;
    vitenc_status st = validate_hparams(hp);
    if (st != VITENC_OK) return st;
    if (!w) return fail(VITENC_ENULL, "weights is NULL");
    if (!w->patch_w || !w->patch_b) return fail(VITENC_ENULL, "patch_w / patch_b is NULL");
    if (hp->pos_type == VITENC_POS_TABLE && !w->pos_embed) return fail(VITENC_ENULL, "pos_embed is NULL");
    if (hp->cls_token && !w->cls_token) return fail(VITENC_ENULL, "cls_token is NULL");
    if (hp->modality_embed && !w->mod_embed) return fail(VITENC_ENULL, "mod_embed is NULL");
    if (!w->norm_w || !w->norm_b) return fail(VITENC_ENULL, "norm_w / norm_b is NULL");
    if (!w->blocks) return fail(VITENC_ENULL, "blocks is NULL");
    for (int i = 0; i < hp->n_layer; ++i) {
        const vitenc_block_weights &b = w->blocks[i];
        const void *req[] = {b.ln1_w, b.ln1_b, b.qkv_w, b.qkv_b, b.out_w, b.out_b,
                             b.ln2_w, b.ln2_b, b.up_w, b.up_b, b.down_w, b.down_b};
        for (const void *p : req)
            if (!p) return fail(VITENC_ENULL, "block %d: a required tensor is NULL", i);
        if (hp->layer_scale && (!b.ls1 || !b.ls2)) return fail(VITENC_ENULL, "block %d: ls1 / ls2 is NULL", i);
        if (hp->weight_format == VITENC_WEIGHTS_MXFP8) {
            if (!b.qkv_s || !b.out_s || !b.up_s || !b.down_s)
                return fail(VITENC_ENULL, "block %d: a block scale pointer is NULL (8-bit weights)", i);
            for (const void *c : {b.qkv_w, b.out_w, b.up_w, b.down_w})
                if (reinterpret_cast<uintptr_t>(c) % 16)
                    return fail(VITENC_EINVAL, "block %d: 8-bit weight codes must be 16-byte aligned", i);
        }
    }
    if (hp->image_patch_embed) {
        if (!w->patch_img_w || !w->patch_img_b) return fail(VITENC_ENULL, "patch_img_w / patch_img_b is NULL");
        if (hp->modality_embed && !w->mod_embed_img) return fail(VITENC_ENULL, "mod_embed_img is NULL");
    }
    for (int k = 0; k < hp->n_hier; ++k)
        if (!w->hier_norm_w[k] || !w->hier_norm_b[k]) return fail(VITENC_ENULL, "hier norm %d is NULL", k);
    vitenc_model *m = new vitenc_model;
    m->hp = *hp;
    m->w = *w;
    m->blocks.assign(w->blocks, w->blocks + hp->n_layer);
    m->w.blocks = m->blocks.data();
    *out = m;
    return VITENC_OK;
}

void vitenc_model_destroy(vitenc_model *m) { delete m; }

vitenc_status vitenc_workspace_size(const vitenc_model *m, int32_t B, int32_t T, int32_t H, int32_t W,
                                    size_t *bytes) {
    g_error.clear();
    if (!m || !bytes) return fail(VITENC_ENULL, "model / bytes is NULL");
    Plan pl;
    vitenc_status st = make_plan(m, B, T, H, W, pl);
    if (st != VITENC_OK) return st;
    *bytes = pl.total;
    return VITENC_OK;
}

vitenc_status vitenc_encode(const vitenc_model *m, const float *pixels, int32_t B, int32_t T, int32_t H, int32_t W,
                            void *workspace, size_t ws_bytes, float *out_tokens, float *out_pooled, void *stream) {
    return vitenc_encode_hier(m, pixels, B, T, H, W, workspace, ws_bytes, out_tokens, out_pooled, nullptr, stream);
}

vitenc_status vitenc_encode_hier(const vitenc_model *m, const float *pixels, int32_t B, int32_t T, int32_t H,
                                 int32_t W, void *workspace, size_t ws_bytes, float *out_tokens, float *out_pooled,
                                 float *out_hier, void *stream) {
    g_error.clear();
    if (!m) return fail(VITENC_ENULL, "model is NULL");
    if (!pixels || !out_tokens) return fail(VITENC_ENULL, "pixels / out_tokens is NULL");
    Plan pl;
    vitenc_status st = make_plan(m, B, T, H, W, pl);
    if (st != VITENC_OK) return st;
    if (!workspace) return fail(VITENC_ENULL, "workspace is NULL");
    if ((uintptr_t)workspace % 256) return fail(VITENC_EWORKSPACE, "workspace not 256-byte aligned");
    if (ws_bytes < pl.total)
        return fail(VITENC_EWORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, pl.total);

    const vitenc_hparams &hp = m->hp;
    const int dt = hp.dtype;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    float *Z = reinterpret_cast<float *>(ws + pl.off_Z);
    void *Y = ws + pl.off_Y, *Q = ws + pl.off_Q, *Kb = ws + pl.off_K, *Vt = ws + pl.off_V;
    void *O = ws + pl.off_O, *U = ws + pl.off_U, *A = ws + pl.off_A;
    float *rope_tab = reinterpret_cast<float *>(ws + pl.off_rope);
    int *tok_pos = reinterpret_cast<int *>(ws + pl.off_tok);
    const int M = (int)pl.M, D = pl.D, F = pl.F;

    // the position table, resampled to this input's grid when it was built for another
    const float *pos = hp.pos_type == VITENC_POS_TABLE ? m->w.pos_embed : nullptr;
    if (pl.resample) {
        float *pbuf = reinterpret_cast<float *>(ws + pl.off_pos);
        CHECK_DEV(launch_pos_resample(pos, pl.p, D, hp.pos_grid_t, hp.pos_grid_h, hp.pos_grid_w, pl.gt, pl.gh, pl.gw,
                                      hp.pos_interp, pbuf, s),
                  "position resampling");
        pos = pbuf;
    }

    float *sk_part = pl.sk_floats ? reinterpret_cast<float *>(ws + pl.off_skp) : nullptr;
    auto with_splitk = [&](EpiArgs &ep) {
        ep.sk_part = sk_part;
        ep.sk_part_floats = pl.sk_floats;
    };

    // a1-a3: tokens
    CHECK_DEV(launch_patchify(dt, pixels, B, pl.C, T, H, W, pl.tub, hp.patch_size, A, pl.lda, s), "patchify");
    const float *mod = !hp.modality_embed ? nullptr : pl.image ? m->w.mod_embed_img : m->w.mod_embed;
    {
        EpiArgs ep;
        ep.bias = pl.image ? m->w.patch_img_b : m->w.patch_b;
        ep.Z = Z;
        ep.ldz = D;
        ep.pos = pos;
        ep.mod = mod;
        ep.Np = pl.Np;
        ep.Ntok = pl.N;
        ep.prefix = pl.p;
        const bool split = pl.lda == 2 * pl.K;
        ep.kwrap = split ? pl.K : 0;
        with_splitk(ep);
        CHECK_DEV(launch_gemm(dt, EPI_PATCH, A, pl.lda, pl.image ? m->w.patch_img_w : m->w.patch_w, pl.K, B * pl.Np, D,
                              split ? 2 * pl.K : pl.K, ep, s),
                  "patch GEMM");
    }
    if (pl.p)
        CHECK_DEV(launch_prefix_rows(m->w.cls_token, pos,
                                     mod,
                                     B, pl.N, D, Z, s),
                  "prefix rows");
    if (hp.rope)
        CHECK_DEV(launch_rope_table(pl.hd, hp.rope_layout, hp.rope_interpolate, hp.rope_ref_grid, hp.rope_theta, pl.gt,
                                    pl.gh, pl.gw, rope_tab, tok_pos, s),
                  "rope tables");

    BlockGeom g;
    g.dtype = dt; g.B = B; g.N = pl.N; g.D = D; g.F = F; g.n_head = pl.nh; g.head_dim = pl.hd; g.ldv = pl.ldv;
    g.prefix = pl.p; g.attn_mode = hp.attn_mode; g.tokens_per_frame = pl.gh * pl.gw; g.layer_scale = hp.layer_scale;
    g.wq = hp.weight_format == VITENC_WEIGHTS_MXFP8;
    g.eps = hp.ln_eps;
    g.rope = hp.rope; g.gt = pl.gt; g.gh = pl.gh; g.gw = pl.gw; g.rope_tab = rope_tab; g.tok_pos = tok_pos;
    BlockBufs bb;
    bb.Z = Z; bb.Y = Y; bb.Q = Q; bb.K = Kb; bb.Vt = Vt; bb.O = O; bb.U = U;
    bb.attn_scratch = reinterpret_cast<float *>(ws + pl.off_attn);
    bb.sk_part = sk_part;
    bb.sk_part_floats = pl.sk_floats;
    int k_hier = 0;
    for (int l = 0; l < hp.n_layer; ++l) {
        const char *what = "block";
        const hipError_t e = run_block(g, bb, m->blocks[l], s, &what);
        CHECK_DEV(e, what);
        if (k_hier < hp.n_hier && hp.hier_layers[k_hier] == l) {
            if (out_hier)
                CHECK_DEV(launch_layernorm(DT_F32, Z, m->w.hier_norm_w[k_hier], m->w.hier_norm_b[k_hier], hp.ln_eps, M,
                                           D, out_hier + (int64_t)k_hier * M * D, s),
                          "hierarchical norm");
            ++k_hier;
        }
    }
    CHECK_DEV(launch_layernorm(DT_F32, Z, m->w.norm_w, m->w.norm_b, hp.ln_eps, M, D, out_tokens, s), "final norm");
    if (out_pooled) CHECK_DEV(launch_pool(out_tokens, B, pl.N, D, hp.cls_token, pl.p, out_pooled, s), "pool");
    return VITENC_OK;
}

} // extern "C"
