// C ABI of the attentive-pool head and classifier (include/vitenc.h):
// validation, workspace planning and the launch sequence (jepa.cpp "GGUF
// schema (v1)", "Head (jepa.head.*)"; SkyVision.cpp README, V-JEPA 2 backend
// notes, the pooler and classifier heads).  Every refusal happens before any
// device work.
#include <hip/hip_runtime.h>

#include <cmath>
#include <vector>

#include "launch.h"

using namespace vitenc;

struct vitenc_head {
    vitenc_head_hparams hp;
    vitenc_head_weights w;
    std::vector<vitenc_block_weights> blocks;
};

namespace {

constexpr int kMaxEmbed = 4096; // LayerNorm rows live in one wave's registers

bool in_range(int64_t v, int64_t lo, int64_t hi) { return v >= lo && v <= hi; }
int64_t rup(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
bool aligned16(const void *p) { return (uintptr_t)p % 16 == 0; }

vitenc_status validate(const vitenc_head_hparams *hp) {
    if (!hp) return fail(VITENC_ENULL, "hparams is NULL");
    if (!in_range(hp->embed_dim, 1, 65536)) return fail(VITENC_EINVAL, "embed_dim %d outside 1..65536", hp->embed_dim);
    if (!in_range(hp->n_head, 1, 1024)) return fail(VITENC_EINVAL, "n_head %d outside 1..1024", hp->n_head);
    if (!in_range(hp->ffn_dim, 1, 1 << 20)) return fail(VITENC_EINVAL, "ffn_dim %d outside 1..2^20", hp->ffn_dim);
    if (!in_range(hp->n_pool_layers, 0, 1024))
        return fail(VITENC_EINVAL, "n_pool_layers %d outside 0..1024", hp->n_pool_layers);
    if (!in_range(hp->n_classes, 0, 1 << 20)) return fail(VITENC_EINVAL, "n_classes %d outside 0..2^20", hp->n_classes);
    if (!std::isfinite(hp->ln_eps) || hp->ln_eps < 0.0f || hp->ln_eps > 1.0f)
        return fail(VITENC_EINVAL, "ln_eps %g not a finite value in [0, 1]", (double)hp->ln_eps);
    if (hp->dtype != VITENC_F32 && hp->dtype != VITENC_BF16 && hp->dtype != VITENC_F16)
        return fail(VITENC_EINVAL, "unknown dtype %d", hp->dtype);
    if (hp->embed_dim % hp->n_head)
        return fail(VITENC_EINVAL, "embed_dim %d not divisible by n_head %d", hp->embed_dim, hp->n_head);
    if (hp->embed_dim > kMaxEmbed) return fail(VITENC_EUNSUPPORTED, "embed_dim %d above %d", hp->embed_dim, kMaxEmbed);
    if (hp->embed_dim % 4)
        return fail(VITENC_EUNSUPPORTED, "embed_dim %d not a multiple of 4 (16-byte token rows)", hp->embed_dim);
    const int hd = hp->embed_dim / hp->n_head;
    if (hp->n_pool_layers > 0 && hd != 64 && hd != 32)
        return fail(VITENC_EUNSUPPORTED, "head_dim %d: the attention kernel implements 64 and 32", hd);
    return VITENC_OK;
}

struct HeadPlan {
    int B, N, M, D, F, H, hd, ldv, NC, C;
    size_t off_Z, off_Y, off_Q, off_K, off_V, off_O, off_U;
    size_t off_q, off_u, off_ub, off_s, off_stats, off_P, off_ybar, off_y, off_h, off_f, off_attn, total;
};

vitenc_status make_plan(const vitenc_head *hd, int B, int N, HeadPlan &pl) {
    const vitenc_head_hparams &hp = hd->hp;
    if (B < 1 || N < 1) return fail(VITENC_ESHAPE, "B=%d N=%d: each must be at least 1", B, N);
    if (N > (1 << 22)) return fail(VITENC_ESHAPE, "%d tokens per item exceed 2^22", N);
    if ((int64_t)B * N > (int64_t(1) << 30)) return fail(VITENC_ESHAPE, "B*N rows exceed 2^30");
    pl.B = B; pl.N = N; pl.M = B * N;
    pl.D = hp.embed_dim; pl.F = hp.ffn_dim; pl.H = hp.n_head; pl.hd = pl.D / pl.H;
    pl.ldv = (int)rup(N, 64);
    pl.NC = xattn_chunks(N);
    pl.C = hp.n_classes;
    const size_t es = (size_t)dtype_size(hp.dtype);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = (size_t)rup((int64_t)(off + bytes), 256);
        return o;
    };
    const size_t M = (size_t)pl.M, D = (size_t)pl.D, H = (size_t)pl.H;
    pl.off_Z = pl.off_Y = pl.off_Q = pl.off_K = pl.off_V = pl.off_O = pl.off_U = 0;
    if (hp.n_pool_layers > 0) {
        pl.off_Z = take(M * D * 4);
        pl.off_Y = take(M * D * es);
        pl.off_Q = take(M * D * es);
        pl.off_K = take(M * D * es);
        pl.off_V = take((size_t)B * H * pl.hd * pl.ldv * es);
        pl.off_O = take(M * D * es);
        pl.off_U = take(M * (size_t)pl.F * es);
    }
    // the pooler blocks' attention has no prefix rows, but a small grid splits every row over runs of keys
    pl.off_attn = hp.n_pool_layers > 0
                      ? take((size_t)attention_scratch_floats(hp.dtype, B, N, H, pl.hd, VITENC_ATTN_FULL, 0, 0) * 4)
                      : 0;
    pl.off_q = take(D * 4);
    pl.off_u = take(H * D * 4);
    pl.off_ub = take(H * 4);
    pl.off_s = take((size_t)B * H * N * 4);
    pl.off_stats = take(M * 8);
    pl.off_P = take((size_t)B * pl.NC * H * D * 4);
    pl.off_ybar = take((size_t)B * H * D * 4);
    pl.off_y = take((size_t)B * D * 4);
    pl.off_h = take((size_t)B * D * 4);
    pl.off_f = take((size_t)B * pl.F * 4);
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

vitenc_status vitenc_head_create(const vitenc_head_hparams *hp, const vitenc_head_weights *w, vitenc_head **out) {
    clear_error();
    if (!out) return fail(VITENC_ENULL, "out is NULL");
    *out = nullptr;
    vitenc_status st = validate(hp);
    if (st != VITENC_OK) return st;
    if (!w) return fail(VITENC_ENULL, "weights is NULL");
    const void *req[] = {w->query, w->ln_kv_w, w->ln_kv_b, w->q_w, w->q_b, w->k_w, w->k_b, w->v_w, w->v_b,
                         w->ln2_w, w->ln2_b, w->up_w, w->up_b, w->down_w, w->down_b};
    for (const void *p : req)
        if (!p) return fail(VITENC_ENULL, "a required head tensor is NULL");
    if (hp->n_classes > 0 && (!w->cls_w || !w->cls_b)) return fail(VITENC_ENULL, "cls_w / cls_b is NULL");
    if (!aligned16(w->ln_kv_w) || !aligned16(w->ln_kv_b))
        return fail(VITENC_EINVAL, "ln_kv_w / ln_kv_b not 16-byte aligned");
    if (hp->n_pool_layers > 0) {
        if (!w->blocks) return fail(VITENC_ENULL, "blocks is NULL");
        for (int i = 0; i < hp->n_pool_layers; ++i) {
            const vitenc_block_weights &b = w->blocks[i];
            const void *breq[] = {b.ln1_w, b.ln1_b, b.qkv_w, b.qkv_b, b.out_w, b.out_b,
                                  b.ln2_w, b.ln2_b, b.up_w, b.up_b, b.down_w, b.down_b};
            for (const void *p : breq)
                if (!p) return fail(VITENC_ENULL, "block %d: a required tensor is NULL", i);
        }
    }
    vitenc_head *h = new vitenc_head;
    h->hp = *hp;
    h->w = *w;
    if (hp->n_pool_layers > 0) h->blocks.assign(w->blocks, w->blocks + hp->n_pool_layers);
    h->w.blocks = h->blocks.data();
    *out = h;
    return VITENC_OK;
}

void vitenc_head_destroy(vitenc_head *h) { delete h; }

vitenc_status vitenc_head_workspace_size(const vitenc_head *h, int32_t B, int32_t N, size_t *bytes) {
    clear_error();
    if (!h || !bytes) return fail(VITENC_ENULL, "head / bytes is NULL");
    HeadPlan pl;
    vitenc_status st = make_plan(h, B, N, pl);
    if (st != VITENC_OK) return st;
    *bytes = pl.total;
    return VITENC_OK;
}

vitenc_status vitenc_head_forward(const vitenc_head *h, const float *tokens, int32_t B, int32_t N, void *workspace,
                                  size_t ws_bytes, float *pooled, float *logits, void *stream) {
    clear_error();
    if (!h) return fail(VITENC_ENULL, "head is NULL");
    if (!tokens || !pooled) return fail(VITENC_ENULL, "tokens / pooled is NULL");
    HeadPlan pl;
    vitenc_status st = make_plan(h, B, N, pl);
    if (st != VITENC_OK) return st;
    if (!aligned16(tokens)) return fail(VITENC_EINVAL, "tokens not 16-byte aligned");
    if (!workspace) return fail(VITENC_ENULL, "workspace is NULL");
    if ((uintptr_t)workspace % 256) return fail(VITENC_EWORKSPACE, "workspace not 256-byte aligned");
    if (ws_bytes < pl.total) return fail(VITENC_EWORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, pl.total);

    const vitenc_head_hparams &hp = h->hp;
    const vitenc_head_weights &w = h->w;
    const int dt = hp.dtype, D = pl.D, F = pl.F, H = pl.H;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    auto f32 = [&](size_t off) { return reinterpret_cast<float *>(ws + off); };

    // pooler blocks over the whole token stream
    const float *X = tokens;
    if (hp.n_pool_layers > 0) {
        float *Z = f32(pl.off_Z);
        CHECK_DEV(hipMemcpyAsync(Z, tokens, (size_t)pl.M * D * sizeof(float), hipMemcpyDeviceToDevice, s),
                  "token copy");
        BlockGeom g;
        g.dtype = dt; g.B = B; g.N = N; g.D = D; g.F = F; g.n_head = H; g.head_dim = pl.hd; g.ldv = pl.ldv;
        g.prefix = 0; g.attn_mode = VITENC_ATTN_FULL; g.tokens_per_frame = N; g.layer_scale = 0;
        g.eps = hp.ln_eps; g.rope = 0;
        BlockBufs bb;
        bb.Z = Z; bb.Y = ws + pl.off_Y; bb.Q = ws + pl.off_Q; bb.K = ws + pl.off_K; bb.Vt = ws + pl.off_V;
        bb.O = ws + pl.off_O; bb.U = ws + pl.off_U;
        bb.attn_scratch = reinterpret_cast<float *>(ws + pl.off_attn);
        for (int l = 0; l < hp.n_pool_layers; ++l) {
            const char *what = "pooler block";
            const hipError_t e = run_block(g, bb, h->blocks[l], s, &what);
            CHECK_DEV(e, what);
        }
        X = Z;
    }
    // the query, and the key projection folded into it
    float *q = f32(pl.off_q), *u = f32(pl.off_u), *ub = f32(pl.off_ub);
    CHECK_DEV(launch_gemv(dt, w.q_w, D, w.q_b, w.query, 0, D, 0, 1, D, D, false, nullptr, 0, q, D, s), "query GEMV");
    CHECK_DEV(launch_xattn_fold(dt, w.k_w, w.k_b, q, D, H, u, ub, s), "key fold");
    // scores over the normalised tokens, softmax, weighted sums per head
    float *sc = f32(pl.off_s), *P = f32(pl.off_P), *ybar = f32(pl.off_ybar);
    float2 *stats = reinterpret_cast<float2 *>(ws + pl.off_stats);
    CHECK_DEV(launch_xattn_scores(X, B, N, D, w.ln_kv_w, w.ln_kv_b, hp.ln_eps, u, ub, H, sc, stats, s), "scores");
    CHECK_DEV(launch_xattn_softmax(sc, stats, B, N, H, s), "softmax");
    CHECK_DEV(launch_xattn_pool(X, stats, sc, B, N, D, H, w.ln_kv_w, w.ln_kv_b, P, ybar, s), "weighted sums");
    // y = query + Wv ybar_h + bv (no output projection); pooled = y + MLP(LN2(y))
    float *y = f32(pl.off_y), *hn = f32(pl.off_h), *f = f32(pl.off_f);
    CHECK_DEV(launch_gemv(dt, w.v_w, D, w.v_b, ybar, (int64_t)H * D, pl.hd, D, B, D, D, false, w.query, 0, y, D, s),
              "value GEMV");
    CHECK_DEV(launch_layernorm(DT_F32, y, w.ln2_w, w.ln2_b, hp.ln_eps, B, D, hn, s), "head ln2");
    CHECK_DEV(launch_gemv(dt, w.up_w, D, w.up_b, hn, D, F, 0, B, F, D, true, nullptr, 0, f, F, s), "head fc1");
    CHECK_DEV(launch_gemv(dt, w.down_w, F, w.down_b, f, F, D, 0, B, D, F, false, y, D, pooled, D, s), "head fc2");
    if (logits && pl.C > 0)
        CHECK_DEV(launch_gemv(dt, w.cls_w, D, w.cls_b, pooled, D, pl.C, 0, B, pl.C, D, false, nullptr, 0, logits, pl.C,
                              s),
                  "classifier");
    return VITENC_OK;
}

} // extern "C"
