// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vitenc.h"

namespace vitenc {

// thread-local refusal text behind vitenc_error_text()
vitenc_status fail(vitenc_status st, const char *fmt, ...);
void clear_error();
// VITENC_OK, or EDEVICE with "what: <HIP error text>"
vitenc_status device_status(hipError_t e, const char *what);

enum Dtype { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };
inline int dtype_size(int dt) { return dt == DT_F32 ? 4 : 2; }
inline int dtype_chunk_elems(int dt) { return dt == DT_F32 ? 4 : 8; }

enum EpiKind { EPI_STORE = 0, EPI_GELU = 1, EPI_RESID = 2, EPI_PATCH = 3, EPI_QKV = 4 };

// Everything an epilogue may need; unused fields are ignored.
struct EpiArgs {
    const float *bias = nullptr;     // [N]
    // STORE / GELU: out T [M, ldo]
    void *out = nullptr;
    int64_t ldo = 0;
    // RESID: Z fp32 [M, ldz] += ls * v ; PATCH: Z fp32 token rows
    float *Z = nullptr;
    int64_t ldz = 0;
    const float *ls = nullptr;
    // PATCH: GEMM row m = b*Np + n -> token row b*Ntok + prefix + n, or
    // row_map[m] when row_map is set (then pos must be null; mod is added)
    const float *pos = nullptr;      // fp32 [Ntok, ldz] or null
    const float *mod = nullptr;      // fp32 [ldz] or null
    int Np = 0, Ntok = 0, prefix = 0;
    const int *row_map = nullptr;
    // QKV: GEMM row m = b*Ntok + tok; column c in [0, 3D)
    void *Q = nullptr, *K = nullptr, *Vt = nullptr;
    int D = 0, head_dim = 0, ldv = 0;
    int rope = 0, d_rot = 0;
    const float *rope_tab = nullptr; // cos / signed sin pairs per (axis, position, j)
    int rope_tab_pairs = 0;          // number of (cos, signed sin) pairs in rope_tab
    const int *tok_pos = nullptr;    // packed (t, h, w) per patch token
    int tok_pos_stride = 0;          // 0: one position list for all items; else per item
    int gt = 0, gh = 0;              // axis offsets into rope_tab
    // A has 2*kwrap columns whose second half pairs with W's columns again
    // (the split-pixel patch embedding); 0: A and W share K
    int kwrap = 0;
    // 8-bit weights (bf16 GEMMs only): when set, W holds E4M3 codes [N, K]
    // (ldw in bytes) and wscale the E8M0 exponent byte of every 32-weight
    // block, laid out [K/64][N][2] (the two blocks of a 64-column slab of a
    // row side by side); needs K % 64 == 0, N % 8 == 0, no kwrap
    const uint8_t *wscale = nullptr;
    // split-K scratch: when sk_part is set the launcher may split K over S
    // workgroups per tile (STORE, GELU and RESID epilogues); each writes its
    // raw fp32 partial [M, N] to sk_part + split * M * N and a second kernel
    // adds the S partials in split order and applies the epilogue.
    float *sk_part = nullptr;
    int64_t sk_part_floats = 0;
    int splits = 1; // set by the launcher
    // One prefix row (a CLS token) beside the tile grid: when pre_a is set,
    // the tile kernel also forms pre_a [K] times W^T.  Its workgroups split
    // the N columns, each adding its share from the weight slabs it holds in
    // LDS anyway, and the row goes through the same GELU / residual epilogue
    // into pre_out / pre_z (the output / residual row of the prefix token).
    // RESID and GELU only, on the 256 x 256 and the 128-deep 128 x 128
    // configurations, unsplit, K <= 4096; otherwise the launcher returns
    // hipErrorNotSupported and launches nothing.
    const void *pre_a = nullptr;
    void *pre_out = nullptr;
    float *pre_z = nullptr;
};

// Split-K scratch floats a GEMM of this shape can use (0: it does not split;
// the launcher splits only when the tiles leave most of the CUs idle).
int64_t gemm_splitk_floats(int dtype, int epi, int M, int N, int K, bool wq);

// Patch embedding in a 16-bit type with K a multiple of 64 stores each pixel
// as two values, hi = round(x) and lo = round(x - hi), in the two halves of a
// row of 2K columns, and runs the patch GEMM over both halves against the
// same weights: the pixels then enter the embedding with about 16 significant
// bits instead of 8.  Returns the A row length (elements) of a patch row.
inline int embed_lda(int dtype, int K) {
    if (dtype != DT_F32 && K % 64 == 0) return 2 * K;
    return (K + 7) / 8 * 8;
}

hipError_t launch_gemm(int dtype, int epi, const void *A, int64_t lda, const void *W, int64_t ldw,
                       int M, int N, int K, const EpiArgs &ep, hipStream_t s);

// The same GEMM and epilogue (STORE, GELU or RESID) for R <= kGemmRowsMax
// rows, A's rows lda apart: a dot product per output, for the few prefix rows
// of a one-item call whose patch rows then fill the tile grid of launch_gemm
// exactly.  16-bit types, K % 8 == 0.
constexpr int kGemmRowsMax = 4;
hipError_t launch_gemm_rows(int dtype, int epi, const void *A, int64_t lda, const void *W, int64_t ldw, int R,
                            int N, int K, const EpiArgs &ep, hipStream_t s);

// codes [rows, cols] E4M3 and scales [cols/64][rows][2] E8M0 of the fp32
// matrix w [rows, cols] (cols % 64 == 0; w and codes 16-byte aligned)
hipError_t launch_mxfp8_quantize(const float *w, int rows, int cols, uint8_t *codes, uint8_t *scales,
                                 hipStream_t s);

hipError_t launch_layernorm(int out_dtype, const float *x, const float *w, const float *b, float eps,
                            int M, int D, void *y, hipStream_t s);

// lda == 2K selects the split (hi, lo) representation (embed_lda)
hipError_t launch_patchify(int dtype, const float *px, int B, int C, int T, int H, int W, int tub,
                           int P, void *A, int64_t lda, hipStream_t s);

hipError_t launch_prefix_rows(const float *cls, const float *pos, const float *mod, int B, int Ntok,
                              int D, float *Z, hipStream_t s);

// out [prefix + dt*dh*dw, D] = the position table pos [prefix + st*sh*sw, D]
// resampled from grid (st, sh, sw) to (dt, dh, dw); mode 1 bicubic (one-frame
// tables), 2 trilinear; prefix rows copied
hipError_t launch_pos_resample(const float *pos, int prefix, int D, int st, int sh, int sw, int dt, int dh, int dw,
                               int mode, float *out, hipStream_t s);

// fills rope_tab (cos, signed sin) for the three axes and tok_pos for every patch token
hipError_t launch_rope_table(int head_dim, int layout, int interpolate, int ref_grid, float theta,
                             int gt, int gh, int gw, float *rope_tab, int *tok_pos, hipStream_t s);

// masked predictor: merge the sorted context and target id lists of each item
// into position order (row_ctx / row_tgt: the Z row of each, b*(nc+nt) + rank)
// and write the packed (t, h, w) of every position-ordered token to tok_pos
// [B*(nc+nt)]
hipError_t launch_pred_order(const int *ctx_ids, int nc, const int *tgt_ids, int nt, int B, int gt, int gh, int gw,
                             int *row_ctx, int *row_tgt, int *tok_pos, hipStream_t s);
// out row r (dtype out_dtype, stride ldo) = fp32 src row rows[r] when rows is
// set, else row ids[r] of item r / per_item (src_rows rows per item), D
// columns; split (16-bit out only): rounded value in [0, D), remainder in
// [lo_off, lo_off + D) of the out row (lo_off < 0: D)
hipError_t launch_gather_rows(int out_dtype, const float *src, int64_t lds, const int *rows, const int *ids,
                              int per_item, int src_rows, int R, int D, bool split, void *out, int64_t ldo,
                              hipStream_t s, int64_t lo_off = -1);
// Z row rows[r] = vec (+ add when set, D fp32 each) for r in [0, R)
hipError_t launch_fill_rows(const float *vec, const float *add, const int *rows, int R, int D, float *Z,
                            hipStream_t s);
hipError_t launch_zero(float *x, int64_t n, hipStream_t s);

// attentive-pool head: matrix-vector products for nb <= any items
// out[b*ldo + r] = act(W[r, :C] . x_{b,r} + bias[r]) + res[b*ldr + r],
// x_{b,r} = x + b*ldx + (r / rpg)*ldg; W in `dtype`, x, bias, res, out fp32
hipError_t launch_gemv(int dtype, const void *W, int64_t ldw, const float *bias, const float *x, int64_t ldx, int rpg,
                       int64_t ldg, int nb, int R, int C, bool gelu, const float *res, int64_t ldr, float *out,
                       int64_t ldo, hipStream_t s);
// u [H, D] = (Wk_h^T q_h) / sqrt(hd), ub [H] = (q_h . bk_h) / sqrt(hd)
hipError_t launch_xattn_fold(int dtype, const void *Wk, const float *bk, const float *q, int D, int H, float *u,
                             float *ub, hipStream_t s);
// s [B, H, N] = u_h . LN(z_j) + ub[h]; stats [B*N] = (mean, rstd) of each row; D % 4 == 0, D <= 4096
hipError_t launch_xattn_scores(const float *Z, int B, int N, int D, const float *ln_w, const float *ln_b, float eps,
                               const float *u, const float *ub, int H, float *s, float2 *stats, hipStream_t st);
// s -> p * rstd in place (softmax over each (item, head) row)
hipError_t launch_xattn_softmax(float *s, const float2 *stats, int B, int N, int H, hipStream_t st);
// ybar [B, H, D] = sum_j p_j LN(z_j) per head, through partials P [B, xattn_chunks(N), H, D]
int xattn_chunks(int N);
hipError_t launch_xattn_pool(const float *Z, const float2 *stats, const float *w, int B, int N, int D, int H,
                             const float *ln_w, const float *ln_b, float *P, float *ybar, hipStream_t st);

// scratch: fp32, 16-byte aligned, attention_scratch_floats(...) floats (partial
// results of the prefix rows, of rows split over runs of keys and of query
// tiles split over halves of their keys); may be NULL when that is 0
int64_t attention_scratch_floats(int dtype, int B, int N, int H, int head_dim, int attn_mode, int n_prefix,
                                 int tokens_per_frame);
hipError_t launch_attention(int dtype, const void *Q, const void *K, const void *Vt, int B, int N,
                            int H, int head_dim, int ldv, int attn_mode, int n_prefix,
                            int tokens_per_frame, float *scratch, void *O, hipStream_t s);

hipError_t launch_pool(const float *X, int B, int N, int D, int cls, int n_prefix, float *pooled,
                       hipStream_t s);

// One pre-LN block over the fp32 residual stream Z of B items of N tokens
// (jepa.cpp "Architecture", "The shared ViT graph"): the encoder and the
// predictor run the same sequence of launches.
struct BlockGeom {
    int dtype = 0, B = 0, N = 0, D = 0, F = 0, n_head = 0, head_dim = 0, ldv = 0;
    int prefix = 0, attn_mode = 0, tokens_per_frame = 0, layer_scale = 0;
    float eps = 0.0f;
    int rope = 0, gt = 0, gh = 0, gw = 0;
    const float *rope_tab = nullptr;
    const int *tok_pos = nullptr;
    int tok_pos_stride = 0;          // 0: tok_pos shared by all items
    int wq = 0;                      // the four block matrices are 8-bit codes with block scales
};
struct BlockBufs {
    float *Z = nullptr;              // fp32 [B*N, D]
    void *Y = nullptr, *Q = nullptr, *K = nullptr, *Vt = nullptr, *O = nullptr, *U = nullptr;
    float *attn_scratch = nullptr;   // attention_scratch_floats(...) floats when prefix > 0
    float *sk_part = nullptr;        // split-K scratch (EpiArgs::sk_part), or none
    int64_t sk_part_floats = 0;
};
// *what names the failing launch
hipError_t run_block(const BlockGeom &g, const BlockBufs &b, const vitenc_block_weights &w, hipStream_t s,
                     const char **what);

} // namespace vitenc
