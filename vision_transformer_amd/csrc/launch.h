// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vitenc.h"

namespace vitenc {

// thread-local refusal text behind vitenc_error_text()
vitenc_status fail(vitenc_status st, const char *fmt, ...);
void clear_error();

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
    // PATCH: GEMM row m = b*Np + n -> token row b*Ntok + prefix + n
    const float *pos = nullptr;      // fp32 [Ntok, ldz] or null
    const float *mod = nullptr;      // fp32 [ldz] or null
    int Np = 0, Ntok = 0, prefix = 0;
    // QKV: GEMM row m = b*Ntok + tok; column c in [0, 3D)
    void *Q = nullptr, *K = nullptr, *Vt = nullptr;
    int D = 0, head_dim = 0, ldv = 0;
    int rope = 0, d_rot = 0;
    const float *rope_tab = nullptr; // cos / signed sin pairs per (axis, position, j)
    int rope_tab_pairs = 0;          // number of (cos, signed sin) pairs in rope_tab
    const int *tok_pos = nullptr;    // packed (t, h, w) per patch token
    int gt = 0, gh = 0;              // axis offsets into rope_tab
    // A has 2*kwrap columns whose second half pairs with W's columns again
    // (the split-pixel patch embedding); 0: A and W share K
    int kwrap = 0;
};

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

hipError_t launch_layernorm(int out_dtype, const float *x, const float *w, const float *b, float eps,
                            int M, int D, void *y, hipStream_t s);

// lda == 2K selects the split (hi, lo) representation (embed_lda)
hipError_t launch_patchify(int dtype, const float *px, int B, int C, int T, int H, int W, int tub,
                           int P, void *A, int64_t lda, hipStream_t s);

hipError_t launch_prefix_rows(const float *cls, const float *pos, const float *mod, int B, int Ntok,
                              int D, float *Z, hipStream_t s);

// fills rope_tab (cos, signed sin) for the three axes and tok_pos for every patch token
hipError_t launch_rope_table(int head_dim, int layout, int interpolate, int ref_grid, float theta,
                             int gt, int gh, int gw, float *rope_tab, int *tok_pos, hipStream_t s);

hipError_t launch_attention(int dtype, const void *Q, const void *K, const void *Vt, int B, int N,
                            int H, int head_dim, int ldv, int attn_mode, int n_prefix,
                            int tokens_per_frame, void *O, hipStream_t s);

hipError_t launch_pool(const float *X, int B, int N, int D, int cls, int n_prefix, float *pooled,
                       hipStream_t s);

} // namespace vitenc
