// The launch sequence of one pre-LN block (jepa.cpp "Architecture", "The
// shared ViT graph"):  x += ls1 * out(attn(rope(qkv(ln1(x)))));
// x += ls2 * down(gelu(up(ln2(x)))).  Shared by the encoder and the predictor.
// With g.wq the four matrices are 8-bit codes whose block scales come from
// the block weights' *_s pointers (the GEMM expands them to bf16 exactly).
#include "launch.h"

namespace vitenc {

hipError_t run_block(const BlockGeom &g, const BlockBufs &b, const vitenc_block_weights &w, hipStream_t s,
                     const char **what) {
    const int M = g.B * g.N, D = g.D, F = g.F;
    hipError_t e;
    auto splitk = [&](EpiArgs &ep) {
        ep.sk_part = b.sk_part;
        ep.sk_part_floats = b.sk_part_floats;
    };
#define STEP(expr, name)                                                                                          \
    do {                                                                                                          \
        e = (expr);                                                                                               \
        if (e != hipSuccess) {                                                                                    \
            *what = name;                                                                                         \
            return e;                                                                                             \
        }                                                                                                         \
    } while (0)
    // A one-item call whose prefix (CLS) rows add a row block to the GEMMs
    // (4097 = 4096 patch tokens + CLS) computes the patch rows of the out, up
    // and down projections on the tile grid and their prefix rows apart
    // (launch_gemm_rows).  QKV keeps every row: its transposed V stores need
    // token runs aligned to 8, and its extra row block costs little (24 more
    // tiles on top of 768).
    const int pre = g.B == 1 && g.prefix > 0 && g.prefix <= kGemmRowsMax && g.dtype != DT_F32 && !g.wq &&
                            (M - g.prefix + 127) / 128 < (M + 127) / 128
                        ? g.prefix
                        : 0;
    const int64_t es = dtype_size(g.dtype);
    auto gemm = [&](int epi, const void *A, int64_t lda, const void *W, int N, int K, EpiArgs ep) {
        if (pre == 0) return launch_gemm(g.dtype, epi, A, lda, W, K, M, N, K, ep, s);
        EpiArgs em = ep;
        if (em.out) em.out = static_cast<char *>(em.out) + pre * em.ldo * es;
        if (em.Z) em.Z += pre * em.ldz;
        if (pre == 1) {
            // a single prefix row rides along in the tile kernel, which holds
            // every weight slab in LDS anyway (where its configuration has that
            // path; otherwise the row kernel below)
            EpiArgs ef = em;
            ef.pre_a = A;
            ef.pre_out = ep.out;
            ef.pre_z = ep.Z;
            const hipError_t e1 = launch_gemm(g.dtype, epi, static_cast<const char *>(A) + lda * es, lda, W, K,
                                              M - 1, N, K, ef, s);
            if (e1 != hipErrorNotSupported) return e1;
        }
        // the prefix rows first: their kernel reads the whole weight matrix
        // once, which leaves it in the last-level cache for the tile grid
        hipError_t e2 = launch_gemm_rows(g.dtype, epi, A, lda, W, K, pre, N, K, ep, s);
        if (e2 != hipSuccess) return e2;
        return launch_gemm(g.dtype, epi, static_cast<const char *>(A) + pre * lda * es, lda, W, K, M - pre, N, K, em,
                           s);
    };
    STEP(launch_layernorm(g.dtype, b.Z, w.ln1_w, w.ln1_b, g.eps, M, D, b.Y, s), "ln1");
    {
        EpiArgs ep;
        ep.bias = w.qkv_b;
        ep.Q = b.Q; ep.K = b.K; ep.Vt = b.Vt;
        ep.D = D; ep.head_dim = g.head_dim; ep.ldv = g.ldv;
        ep.Ntok = g.N; ep.prefix = g.prefix;
        ep.rope = g.rope;
        ep.d_rot = 2 * ((g.head_dim / 3) / 2);
        ep.rope_tab = g.rope_tab; ep.tok_pos = g.tok_pos; ep.tok_pos_stride = g.tok_pos_stride;
        ep.rope_tab_pairs = (g.gt + g.gh + g.gw) * ep.d_rot;
        ep.gt = g.gt; ep.gh = g.gh;
        if (g.wq) ep.wscale = w.qkv_s;
        splitk(ep);
        STEP(launch_gemm(g.dtype, EPI_QKV, b.Y, D, w.qkv_w, D, M, 3 * D, D, ep, s), "qkv GEMM");
    }
    STEP(launch_attention(g.dtype, b.Q, b.K, b.Vt, g.B, g.N, g.n_head, g.head_dim, g.ldv, g.attn_mode, g.prefix,
                          g.tokens_per_frame, b.attn_scratch, b.O, s),
         "attention");
    {
        EpiArgs ep;
        ep.bias = w.out_b; ep.Z = b.Z; ep.ldz = D;
        ep.ls = g.layer_scale ? w.ls1 : nullptr;
        if (g.wq) ep.wscale = w.out_s;
        splitk(ep);
        STEP(gemm(EPI_RESID, b.O, D, w.out_w, D, D, ep), "out GEMM");
    }
    STEP(launch_layernorm(g.dtype, b.Z, w.ln2_w, w.ln2_b, g.eps, M, D, b.Y, s), "ln2");
    {
        EpiArgs ep;
        ep.bias = w.up_b; ep.out = b.U; ep.ldo = F;
        if (g.wq) ep.wscale = w.up_s;
        splitk(ep);
        STEP(gemm(EPI_GELU, b.Y, D, w.up_w, F, D, ep), "up GEMM");
    }
    {
        EpiArgs ep;
        ep.bias = w.down_b; ep.Z = b.Z; ep.ldz = D;
        ep.ls = g.layer_scale ? w.ls2 : nullptr;
        if (g.wq) ep.wscale = w.down_s;
        splitk(ep);
        STEP(gemm(EPI_RESID, b.U, F, w.down_w, D, F, ep), "down GEMM");
    }
#undef STEP
    return hipSuccess;
}

} // namespace vitenc
