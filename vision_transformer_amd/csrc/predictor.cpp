// C ABI of the masked-latent predictor (include/vitenc.h): validation,
// workspace planning and the launch sequence (SkyVision.cpp README, V-JEPA 2
// backend notes, "masked-latent predictor"; jepa.cpp "GGUF schema (v1)",
// "Predictor (jepa.pred.*)").  Every refusal happens before device work.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <vector>

#include "launch.h"

using namespace vitenc;

struct vitenc_predictor {
    vitenc_pred_hparams hp;
    vitenc_pred_weights w;
    std::vector<vitenc_block_weights> blocks;
};

namespace {

constexpr int kMaxGrid = 1023;   // per axis (packed 10-bit positions)
constexpr int kMaxEmbed = 4096;  // LayerNorm keeps a row in one wave's registers

bool in_range(int64_t v, int64_t lo, int64_t hi) { return v >= lo && v <= hi; }
int64_t rup(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

vitenc_status validate(const vitenc_pred_hparams *hp) {
    if (!hp) return fail(VITENC_ENULL, "hparams is NULL");
    if (!in_range(hp->embed_dim, 1, 65536)) return fail(VITENC_EINVAL, "embed_dim %d outside 1..65536", hp->embed_dim);
    if (!in_range(hp->enc_dim, 1, 65536)) return fail(VITENC_EINVAL, "enc_dim %d outside 1..65536", hp->enc_dim);
    if (!in_range(hp->n_layer, 1, 1024)) return fail(VITENC_EINVAL, "n_layer %d outside 1..1024", hp->n_layer);
    if (!in_range(hp->n_head, 1, 1024)) return fail(VITENC_EINVAL, "n_head %d outside 1..1024", hp->n_head);
    if (!in_range(hp->ffn_dim, 1, 1 << 20)) return fail(VITENC_EINVAL, "ffn_dim %d outside 1..2^20", hp->ffn_dim);
    if (!in_range(hp->n_mask_tokens, 1, 1 << 16))
        return fail(VITENC_EINVAL, "n_mask_tokens %d outside 1..65536", hp->n_mask_tokens);
    if (!std::isfinite(hp->ln_eps) || hp->ln_eps < 0.0f || hp->ln_eps > 1.0f)
        return fail(VITENC_EINVAL, "ln_eps %g not a finite value in [0, 1]", (double)hp->ln_eps);
    if (!std::isfinite(hp->rope_theta) || hp->rope_theta <= 0.0f)
        return fail(VITENC_EINVAL, "rope_theta %g must be finite and > 0", (double)hp->rope_theta);
    if (hp->rope_layout != VITENC_ROPE_TILED && hp->rope_layout != VITENC_ROPE_INTERLEAVED)
        return fail(VITENC_EINVAL, "unknown rope_layout %d", hp->rope_layout);
    if (!in_range(hp->grid_t, 1, kMaxGrid) || !in_range(hp->grid_h, 1, kMaxGrid) || !in_range(hp->grid_w, 1, kMaxGrid))
        return fail(VITENC_EINVAL, "token grid %dx%dx%d outside 1..%d per axis", hp->grid_t, hp->grid_h, hp->grid_w,
                    kMaxGrid);
    if ((int64_t)hp->grid_t * hp->grid_h * hp->grid_w > (int64_t(1) << 22))
        return fail(VITENC_EINVAL, "token grid of more than 2^22 tokens");
    if (hp->dtype != VITENC_F32 && hp->dtype != VITENC_BF16 && hp->dtype != VITENC_F16)
        return fail(VITENC_EINVAL, "unknown dtype %d", hp->dtype);
    if (hp->out_dim != 0 && !in_range(hp->out_dim, 1, 65536))
        return fail(VITENC_EINVAL, "out_dim %d outside 1..65536 (0: enc_dim)", hp->out_dim);
    if (!in_range(hp->n_hier_in, 0, VITENC_MAX_HIER))
        return fail(VITENC_EINVAL, "n_hier_in %d outside 0..%d", hp->n_hier_in, VITENC_MAX_HIER);
    if (hp->n_hier_in > 1 && !in_range(hp->embed_hidden, 1, 65536))
        return fail(VITENC_EINVAL, "embed_hidden %d outside 1..65536 (needed with n_hier_in > 1)", hp->embed_hidden);
    if ((int64_t)(hp->n_hier_in > 1 ? hp->n_hier_in : 1) * hp->enc_dim > 65536)
        return fail(VITENC_EINVAL, "n_hier_in x enc_dim above 65536");
    if (hp->modality_embed != 0 && hp->modality_embed != 1)
        return fail(VITENC_EINVAL, "modality_embed %d is not 0 or 1", hp->modality_embed);
    if (hp->context_proj != 0 && hp->context_proj != 1)
        return fail(VITENC_EINVAL, "context_proj %d is not 0 or 1", hp->context_proj);
    if (hp->embed_dim % hp->n_head)
        return fail(VITENC_EINVAL, "embed_dim %d not divisible by n_head %d", hp->embed_dim, hp->n_head);
    const int hd = hp->embed_dim / hp->n_head;
    if (hd != 64 && hd != 32)
        return fail(VITENC_EUNSUPPORTED, "head_dim %d: the attention kernel implements 64 and 32", hd);
    if (hp->embed_dim > kMaxEmbed) return fail(VITENC_EUNSUPPORTED, "embed_dim %d above %d", hp->embed_dim, kMaxEmbed);
    return VITENC_OK;
}

struct PredPlan {
    int B, nc, nt, N, M, D, De, F, nh, hd, ldv, lda_e;
    int nh_in, Ke, Do, Hd; // hierarchical levels, embed input width, output width, embed MLP hidden width
    bool split;
    size_t off_Z, off_Y, off_Q, off_K, off_V, off_O, off_U, off_A, off_Zt, off_rctx, off_rtgt, off_tok, off_rope,
        off_attn, off_Ue, total;
};

vitenc_status make_plan(const vitenc_predictor *p, int B, int nc, int nt, PredPlan &pl) {
    const vitenc_pred_hparams &hp = p->hp;
    if (B < 1 || nc < 1 || nt < 1)
        return fail(VITENC_ESHAPE, "B=%d n_ctx=%d n_tgt=%d: each must be at least 1", B, nc, nt);
    const int64_t n_grid = (int64_t)hp.grid_t * hp.grid_h * hp.grid_w;
    if ((int64_t)nc + nt > n_grid)
        return fail(VITENC_ESHAPE, "n_ctx + n_tgt = %lld exceeds the grid's %lld tokens", (long long)nc + nt,
                    (long long)n_grid);
    if ((int64_t)B * (nc + nt) > (int64_t(1) << 30))
        return fail(VITENC_ESHAPE, "B*(n_ctx+n_tgt) rows exceed 2^30");
    pl.B = B; pl.nc = nc; pl.nt = nt; pl.N = nc + nt; pl.M = B * pl.N;
    pl.D = hp.embed_dim; pl.De = hp.enc_dim; pl.F = hp.ffn_dim; pl.nh = hp.n_head; pl.hd = pl.D / pl.nh;
    pl.ldv = (int)rup(pl.N, 64);
    pl.nh_in = hp.n_hier_in > 1 ? hp.n_hier_in : 1;
    pl.Ke = pl.nh_in * pl.De;
    pl.Do = hp.out_dim ? hp.out_dim : pl.De;
    pl.Hd = pl.nh_in > 1 ? hp.embed_hidden : 0;
    pl.lda_e = embed_lda(hp.dtype, pl.Ke);
    pl.split = pl.lda_e == 2 * pl.Ke;
    const size_t es = (size_t)dtype_size(hp.dtype);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = (size_t)rup((int64_t)(off + bytes), 256);
        return o;
    };
    const size_t M = (size_t)pl.M, D = (size_t)pl.D;
    pl.off_Z = take(M * D * 4);
    pl.off_Y = take(M * D * es);
    pl.off_Q = take(M * D * es);
    pl.off_K = take(M * D * es);
    pl.off_V = take((size_t)B * pl.nh * pl.hd * pl.ldv * es);
    pl.off_O = take(M * D * es);
    pl.off_U = take(M * (size_t)pl.F * es);
    pl.off_A = take((size_t)B * nc * pl.lda_e * es);
    // target rows, then (context projection) the context rows, of the norm
    pl.off_Zt = take((size_t)B * std::max(nc, nt) * D * 4);
    pl.off_Ue = pl.Hd ? take((size_t)B * nc * pl.Hd * es) : 0;
    pl.off_rctx = take((size_t)B * nc * 4);
    pl.off_rtgt = take((size_t)B * nt * 4);
    pl.off_tok = take(M * 4);
    const int d = 2 * ((pl.hd / 3) / 2);
    pl.off_rope = take((size_t)(hp.grid_t + hp.grid_h + hp.grid_w) * d * 2 * 4);
    // attention keeps no prefix rows here, but a small grid splits every row over runs of keys
    pl.off_attn =
        take((size_t)attention_scratch_floats(hp.dtype, B, pl.N, pl.nh, pl.hd, VITENC_ATTN_FULL, 0, 0) * 4);
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

vitenc_status vitenc_predictor_create(const vitenc_pred_hparams *hp, const vitenc_pred_weights *w,
                                      vitenc_predictor **out) {
    clear_error();
    if (!out) return fail(VITENC_ENULL, "out is NULL");
    *out = nullptr;
    vitenc_status st = validate(hp);
    if (st != VITENC_OK) return st;
    if (!w) return fail(VITENC_ENULL, "weights is NULL");
    if (!w->embed_w || !w->embed_b || !w->mask_tokens || !w->norm_w || !w->norm_b || !w->proj_w || !w->proj_b)
        return fail(VITENC_ENULL, "a required predictor tensor is NULL");
    if (!w->blocks) return fail(VITENC_ENULL, "blocks is NULL");
    if (hp->n_hier_in > 1 && (!w->embed2_w || !w->embed2_b))
        return fail(VITENC_ENULL, "n_hier_in > 1 needs embed2_w / embed2_b");
    if (hp->modality_embed && (!w->mod_embed_img || !w->mod_embed_video))
        return fail(VITENC_ENULL, "modality_embed needs mod_embed_img / mod_embed_video");
    if (hp->context_proj && (!w->proj_ctx_w || !w->proj_ctx_b))
        return fail(VITENC_ENULL, "context_proj needs proj_ctx_w / proj_ctx_b");
    for (int i = 0; i < hp->n_layer; ++i) {
        const vitenc_block_weights &b = w->blocks[i];
        const void *req[] = {b.ln1_w, b.ln1_b, b.qkv_w, b.qkv_b, b.out_w, b.out_b,
                             b.ln2_w, b.ln2_b, b.up_w, b.up_b, b.down_w, b.down_b};
        for (const void *q : req)
            if (!q) return fail(VITENC_ENULL, "block %d: a required tensor is NULL", i);
    }
    vitenc_predictor *p = new vitenc_predictor;
    p->hp = *hp;
    p->w = *w;
    p->blocks.assign(w->blocks, w->blocks + hp->n_layer);
    p->w.blocks = p->blocks.data();
    *out = p;
    return VITENC_OK;
}

void vitenc_predictor_destroy(vitenc_predictor *p) { delete p; }

vitenc_status vitenc_predict_workspace_size(const vitenc_predictor *p, int32_t B, int32_t n_ctx, int32_t n_tgt,
                                            size_t *bytes) {
    clear_error();
    if (!p || !bytes) return fail(VITENC_ENULL, "predictor / bytes is NULL");
    PredPlan pl;
    vitenc_status st = make_plan(p, B, n_ctx, n_tgt, pl);
    if (st != VITENC_OK) return st;
    *bytes = pl.total;
    return VITENC_OK;
}

vitenc_status vitenc_predict(const vitenc_predictor *p, const float *enc_tokens, int32_t B, int32_t n_enc,
                             const int32_t *ctx_ids, int32_t n_ctx, const int32_t *tgt_ids, int32_t n_tgt,
                             int32_t mask_index, void *workspace, size_t ws_bytes, float *out, void *stream) {
    return vitenc_predict_all(p, enc_tokens, B, n_enc, ctx_ids, n_ctx, tgt_ids, n_tgt, mask_index, workspace,
                              ws_bytes, out, nullptr, stream);
}

vitenc_status vitenc_predict_all(const vitenc_predictor *p, const float *enc_tokens, int32_t B, int32_t n_enc,
                                 const int32_t *ctx_ids, int32_t n_ctx, const int32_t *tgt_ids, int32_t n_tgt,
                                 int32_t mask_index, void *workspace, size_t ws_bytes, float *out, float *out_ctx,
                                 void *stream) {
    clear_error();
    if (!p) return fail(VITENC_ENULL, "predictor is NULL");
    if (!enc_tokens || !ctx_ids || !tgt_ids || !out) return fail(VITENC_ENULL, "enc_tokens / ids / out is NULL");
    PredPlan pl;
    vitenc_status st = make_plan(p, B, n_ctx, n_tgt, pl);
    if (st != VITENC_OK) return st;
    const vitenc_pred_hparams &hp = p->hp;
    const int n_grid = hp.grid_t * hp.grid_h * hp.grid_w;
    if (n_enc != n_grid)
        return fail(VITENC_ESHAPE, "n_enc %d differs from the grid's %d tokens", n_enc, n_grid);
    if (mask_index < 0 || mask_index >= hp.n_mask_tokens)
        return fail(VITENC_EINVAL, "mask_index %d outside [0, %d)", mask_index, hp.n_mask_tokens);
    if (out_ctx && !hp.context_proj)
        return fail(VITENC_EINVAL, "out_ctx given to a predictor without a context projection");
    if (!workspace) return fail(VITENC_ENULL, "workspace is NULL");
    if ((uintptr_t)workspace % 256) return fail(VITENC_EWORKSPACE, "workspace not 256-byte aligned");
    if (ws_bytes < pl.total) return fail(VITENC_EWORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, pl.total);

    const int dt = hp.dtype;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    float *Z = reinterpret_cast<float *>(ws + pl.off_Z);
    void *Y = ws + pl.off_Y, *A = ws + pl.off_A;
    float *Zt = reinterpret_cast<float *>(ws + pl.off_Zt);
    int *row_ctx = reinterpret_cast<int *>(ws + pl.off_rctx);
    int *row_tgt = reinterpret_cast<int *>(ws + pl.off_rtgt);
    int *tok_pos = reinterpret_cast<int *>(ws + pl.off_tok);
    float *rope_tab = reinterpret_cast<float *>(ws + pl.off_rope);
    const int D = pl.D, De = pl.De, Ke = pl.Ke, Do = pl.Do;
    // the modality vector: image for a one-frame grid, video otherwise
    const float *mod = !hp.modality_embed ? nullptr : hp.grid_t == 1 ? p->w.mod_embed_img : p->w.mod_embed_video;

    // token order: the Z row of every context and target token, and the
    // position of every Z row
    CHECK_DEV(launch_pred_order(ctx_ids, n_ctx, tgt_ids, n_tgt, B, hp.grid_t, hp.grid_h, hp.grid_w, row_ctx, row_tgt,
                                tok_pos, s),
              "token order");
    // context rows: the encoder features of the context ids, the levels of a
    // hierarchical input side by side (level l in columns [l De, (l+1) De) of
    // each half of a split row)
    for (int l = 0; l < pl.nh_in; ++l) {
        const float *src = enc_tokens + (int64_t)l * B * n_enc * De;
        void *dst = static_cast<char *>(A) + (size_t)l * De * dtype_size(dt);
        CHECK_DEV(launch_gather_rows(dt, src, De, nullptr, ctx_ids, n_ctx, n_enc, B * n_ctx, De, pl.split, dst,
                                     pl.lda_e, s, Ke),
                  "context gather");
    }
    {
        const bool mlp = pl.nh_in > 1;
        EpiArgs ep;
        ep.bias = p->w.embed_b;
        ep.kwrap = pl.split ? Ke : 0;
        if (mlp) {
            // embed.0 + GELU into the hidden rows, then embed.2 below
            ep.out = ws + pl.off_Ue;
            ep.ldo = pl.Hd;
            CHECK_DEV(launch_gemm(dt, EPI_GELU, A, pl.lda_e, p->w.embed_w, Ke, B * n_ctx, pl.Hd,
                                  pl.split ? 2 * Ke : Ke, ep, s),
                      "embed MLP GEMM");
        } else {
            ep.Z = Z;
            ep.ldz = D;
            ep.row_map = row_ctx;
            ep.mod = mod;
            CHECK_DEV(launch_gemm(dt, EPI_PATCH, A, pl.lda_e, p->w.embed_w, Ke, B * n_ctx, D, pl.split ? 2 * Ke : Ke,
                                  ep, s),
                      "embed GEMM");
        }
        if (mlp) {
            EpiArgs e2;
            e2.bias = p->w.embed2_b;
            e2.Z = Z;
            e2.ldz = D;
            e2.row_map = row_ctx;
            e2.mod = mod;
            CHECK_DEV(launch_gemm(dt, EPI_PATCH, ws + pl.off_Ue, pl.Hd, p->w.embed2_w, pl.Hd, B * n_ctx, D, pl.Hd, e2,
                                  s),
                      "embed MLP output GEMM");
        }
    }
    // target rows: the mask token (+ the modality vector)
    CHECK_DEV(launch_fill_rows(p->w.mask_tokens + (int64_t)mask_index * D, mod, row_tgt, B * n_tgt, D, Z, s),
              "mask rows");
    CHECK_DEV(launch_rope_table(pl.hd, hp.rope_layout, 0, 0, hp.rope_theta, hp.grid_t, hp.grid_h, hp.grid_w, rope_tab,
                                nullptr, s),
              "rope table");

    BlockGeom g;
    g.dtype = dt; g.B = B; g.N = pl.N; g.D = D; g.F = pl.F; g.n_head = pl.nh; g.head_dim = pl.hd; g.ldv = pl.ldv;
    g.prefix = 0; g.attn_mode = VITENC_ATTN_FULL; g.tokens_per_frame = hp.grid_h * hp.grid_w; g.layer_scale = 0;
    g.eps = hp.ln_eps;
    g.rope = VITENC_ROPE_3D; g.gt = hp.grid_t; g.gh = hp.grid_h; g.gw = hp.grid_w;
    g.rope_tab = rope_tab; g.tok_pos = tok_pos; g.tok_pos_stride = pl.N;
    BlockBufs bb;
    bb.Z = Z; bb.Y = Y; bb.Q = ws + pl.off_Q; bb.K = ws + pl.off_K; bb.Vt = ws + pl.off_V; bb.O = ws + pl.off_O;
    bb.U = ws + pl.off_U;
    bb.attn_scratch = reinterpret_cast<float *>(ws + pl.off_attn);
    for (int l = 0; l < hp.n_layer; ++l) {
        const char *what = "block";
        const hipError_t e = run_block(g, bb, p->blocks[l], s, &what);
        CHECK_DEV(e, what);
    }
    // rows in the order of an id list -> norm -> projection (out = 0 + proj)
    auto project = [&](const int *rows, int n, const void *pw, const float *pb, float *dst,
                       const char *what) -> vitenc_status {
        CHECK_DEV(launch_gather_rows(DT_F32, Z, D, rows, nullptr, 1, 1, B * n, D, false, Zt, D, s), what);
        CHECK_DEV(launch_layernorm(dt, Zt, p->w.norm_w, p->w.norm_b, hp.ln_eps, B * n, D, Y, s), what);
        CHECK_DEV(launch_zero(dst, (int64_t)B * n * Do, s), what);
        EpiArgs ep;
        ep.bias = pb;
        ep.Z = dst;
        ep.ldz = Do;
        CHECK_DEV(launch_gemm(dt, EPI_RESID, Y, D, pw, D, B * n, Do, D, ep, s), what);
        return VITENC_OK;
    };
    st = project(row_tgt, n_tgt, p->w.proj_w, p->w.proj_b, out, "target projection");
    if (st != VITENC_OK) return st;
    if (out_ctx) {
        st = project(row_ctx, n_ctx, p->w.proj_ctx_w, p->w.proj_ctx_b, out_ctx, "context projection");
        if (st != VITENC_OK) return st;
    }
    return VITENC_OK;
}

} // extern "C"
