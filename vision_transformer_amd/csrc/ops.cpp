// Step entry points of include/vitenc.h: one step of the encoder graph each,
// running the same launchers as vitenc_encode.
#include "vitenc.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "launch.h"

using namespace vitenc;

namespace {

#define op_fail vitenc::fail

vitenc_status op_dev(hipError_t e, const char *what) {
    if (e == hipSuccess) return VITENC_OK;
    return op_fail(VITENC_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool dtype_ok(int dt) { return dt == VITENC_F32 || dt == VITENC_BF16 || dt == VITENC_F16; }

} // namespace

extern "C" {

vitenc_status vitenc_op_embed(int32_t dtype, const float *pixels, int32_t B, int32_t C, int32_t T, int32_t H,
                              int32_t W, int32_t tubelet, int32_t patch, const void *patch_w, const float *patch_b,
                              const float *pos, const float *cls, const float *mod, int32_t D, void *scratch,
                              float *Z, void *stream) {
    clear_error();
    if (!dtype_ok(dtype)) return op_fail(VITENC_EINVAL, "unknown dtype %d", dtype);
    if (!pixels || !patch_w || !patch_b || !scratch || !Z) return op_fail(VITENC_ENULL, "a required pointer is NULL");
    if (B <= 0 || C <= 0 || T <= 0 || H <= 0 || W <= 0 || tubelet <= 0 || patch <= 0 || D <= 0)
        return op_fail(VITENC_ESHAPE, "non-positive size");
    if (T % tubelet || H % patch || W % patch) return op_fail(VITENC_ESHAPE, "input not divisible into patches");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int Np = (T / tubelet) * (H / patch) * (W / patch);
    const int K = C * tubelet * patch * patch;
    const int lda = embed_lda(dtype, K);
    const bool split = lda == 2 * K;
    const int p = cls ? 1 : 0;
    vitenc_status st = op_dev(launch_patchify(dtype, pixels, B, C, T, H, W, tubelet, patch, scratch, lda, s), "patchify");
    if (st) return st;
    EpiArgs ep;
    ep.bias = patch_b; ep.Z = Z; ep.ldz = D; ep.pos = pos; ep.mod = mod;
    ep.Np = Np; ep.Ntok = Np + p; ep.prefix = p;
    ep.kwrap = split ? K : 0;
    st = op_dev(launch_gemm(dtype, EPI_PATCH, scratch, lda, patch_w, K, B * Np, D, split ? 2 * K : K, ep, s),
                "patch GEMM");
    if (st) return st;
    if (p) return op_dev(launch_prefix_rows(cls, pos, mod, B, Np + p, D, Z, s), "prefix rows");
    return VITENC_OK;
}

vitenc_status vitenc_op_layernorm(int32_t out_dtype, const float *x, const float *w, const float *b, float eps,
                                  int32_t M, int32_t D, void *y, void *stream) {
    clear_error();
    if (!dtype_ok(out_dtype)) return op_fail(VITENC_EINVAL, "unknown dtype %d", out_dtype);
    if (!x || !w || !b || !y) return op_fail(VITENC_ENULL, "a required pointer is NULL");
    if (M < 0 || D <= 0) return op_fail(VITENC_ESHAPE, "bad size M=%d D=%d", M, D);
    if (D > 4096) return op_fail(VITENC_EUNSUPPORTED, "D=%d above 4096", D);
    return op_dev(launch_layernorm(out_dtype, x, w, b, eps, M, D, y, reinterpret_cast<hipStream_t>(stream)),
                  "layernorm");
}

vitenc_status vitenc_op_pos_resample(const float *pos, int32_t prefix, int32_t D, int32_t st, int32_t sh,
                                     int32_t sw, int32_t dt, int32_t dh, int32_t dw, int32_t mode, float *out,
                                     void *stream) {
    clear_error();
    if (!pos || !out) return op_fail(VITENC_ENULL, "pos / out is NULL");
    if (mode != VITENC_POS_INTERP_BICUBIC && mode != VITENC_POS_INTERP_TRILINEAR)
        return op_fail(VITENC_EINVAL, "unknown resampling mode %d", mode);
    if (prefix < 0 || prefix > 1 || D <= 0 || st <= 0 || sh <= 0 || sw <= 0 || dt <= 0 || dh <= 0 || dw <= 0 ||
        st > 1023 || sh > 1023 || sw > 1023 || dt > 1023 || dh > 1023 || dw > 1023)
        return op_fail(VITENC_ESHAPE, "bad resampling sizes");
    if (mode == VITENC_POS_INTERP_BICUBIC && (st != 1 || dt != 1))
        return op_fail(VITENC_ESHAPE, "bicubic resampling needs one-frame grids");
    return op_dev(launch_pos_resample(pos, prefix, D, st, sh, sw, dt, dh, dw, mode, out,
                                      reinterpret_cast<hipStream_t>(stream)),
                  "position resampling");
}

int64_t vitenc_rope_table_floats(int32_t head_dim, int32_t gt, int32_t gh, int32_t gw) {
    const int d = 2 * ((head_dim / 3) / 2);
    return (int64_t)(gt + gh + gw) * d * 2 + (int64_t)gt * gh * gw; // cos/sin pairs, then packed positions
}

vitenc_status vitenc_op_rope_table(int32_t head_dim, int32_t rope_layout, int32_t rope_interpolate,
                                  int32_t rope_ref_grid, float rope_theta, int32_t gt, int32_t gh, int32_t gw,
                                  float *rope_table, void *stream) {
    clear_error();
    if (!rope_table) return op_fail(VITENC_ENULL, "rope_table is NULL");
    if (head_dim <= 0 || head_dim % 2) return op_fail(VITENC_EINVAL, "head_dim %d (RoPE needs an even one)", head_dim);
    if (gt <= 0 || gh <= 0 || gw <= 0 || gt > 1023 || gh > 1023 || gw > 1023)
        return op_fail(VITENC_ESHAPE, "grid %dx%dx%d", gt, gh, gw);
    if (rope_interpolate && rope_ref_grid <= 0) return op_fail(VITENC_EINVAL, "interpolate without ref grid");
    const int d = 2 * ((head_dim / 3) / 2);
    int *tok = reinterpret_cast<int *>(rope_table + (int64_t)(gt + gh + gw) * d * 2);
    return op_dev(launch_rope_table(head_dim, rope_layout, rope_interpolate, rope_ref_grid, rope_theta, gt, gh, gw,
                                    rope_table, tok, reinterpret_cast<hipStream_t>(stream)),
                  "rope tables");
}

vitenc_status vitenc_op_qkv_rope(int32_t dtype, const void *Y, const void *qkv_w, const float *qkv_b, int32_t B,
                                 int32_t N, int32_t D, int32_t n_head, int32_t rope, int32_t gt, int32_t gh,
                                 int32_t gw, int32_t n_prefix, const float *rope_table, void *Q, void *K, void *Vt,
                                 void *stream) {
    clear_error();
    if (!dtype_ok(dtype)) return op_fail(VITENC_EINVAL, "unknown dtype %d", dtype);
    if (!Y || !qkv_w || !qkv_b || !Q || !K || !Vt) return op_fail(VITENC_ENULL, "a required pointer is NULL");
    if (B <= 0 || N <= 0 || D <= 0 || n_head <= 0 || D % n_head) return op_fail(VITENC_ESHAPE, "bad sizes");
    const int hd = D / n_head;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    EpiArgs ep;
    ep.bias = qkv_b; ep.Q = Q; ep.K = K; ep.Vt = Vt;
    ep.D = D; ep.head_dim = hd; ep.ldv = (N + 63) / 64 * 64;
    ep.Ntok = N; ep.prefix = n_prefix;
    ep.rope = rope;
    if (rope) {
        if (!rope_table) return op_fail(VITENC_ENULL, "rope_table is NULL");
        if (hd % 2) return op_fail(VITENC_EINVAL, "odd head_dim with RoPE");
        if (gt <= 0 || gh <= 0 || gw <= 0 || gt > 1023 || gh > 1023 || gw > 1023 ||
            (int64_t)gt * gh * gw + n_prefix != N)
            return op_fail(VITENC_ESHAPE, "grid %dx%dx%d + %d prefix does not make %d tokens", gt, gh, gw, n_prefix, N);
        const int d = 2 * ((hd / 3) / 2);
        ep.d_rot = d; ep.rope_tab = rope_table;
        ep.tok_pos = reinterpret_cast<const int *>(rope_table + (int64_t)(gt + gh + gw) * d * 2);
        ep.gt = gt; ep.gh = gh;
        ep.rope_tab_pairs = (gt + gh + gw) * d;
    }
    return op_dev(launch_gemm(dtype, EPI_QKV, Y, D, qkv_w, D, B * N, 3 * D, D, ep, s), "qkv GEMM");
}

int64_t vitenc_attention_scratch_floats(int32_t dtype, int32_t B, int32_t N, int32_t n_head, int32_t head_dim,
                                        int32_t attn_mode, int32_t n_prefix, int32_t tokens_per_frame) {
    if (!dtype_ok(dtype) || B <= 0 || N <= 0 || n_head <= 0 || head_dim <= 0 || n_prefix < 0 || n_prefix > N ||
        (attn_mode != 0 && attn_mode != 1) || (attn_mode == 1 && tokens_per_frame <= 0))
        return -1;
    return attention_scratch_floats(dtype, B, N, n_head, head_dim, attn_mode, n_prefix, tokens_per_frame);
}

vitenc_status vitenc_op_attention(int32_t dtype, const void *Q, const void *K, const void *Vt, int32_t B, int32_t N,
                                  int32_t n_head, int32_t head_dim, int32_t attn_mode, int32_t n_prefix,
                                  int32_t tokens_per_frame, float *scratch, void *O, void *stream) {
    clear_error();
    if (!dtype_ok(dtype)) return op_fail(VITENC_EINVAL, "unknown dtype %d", dtype);
    if (!Q || !K || !Vt || !O) return op_fail(VITENC_ENULL, "a required pointer is NULL");
    if (B <= 0 || N <= 0 || n_head <= 0) return op_fail(VITENC_ESHAPE, "bad sizes");
    if (head_dim != 64 && head_dim != 32) return op_fail(VITENC_EUNSUPPORTED, "head_dim %d", head_dim);
    if (n_prefix < 0 || n_prefix >= N) return op_fail(VITENC_ESHAPE, "n_prefix %d outside [0, N)", n_prefix);
    if (attn_mode == 1 && tokens_per_frame <= 0) return op_fail(VITENC_ESHAPE, "block-causal geometry");
    if (attn_mode != 0 && attn_mode != 1) return op_fail(VITENC_EINVAL, "unknown attn_mode %d", attn_mode);
    if (attention_scratch_floats(dtype, B, N, n_head, head_dim, attn_mode, n_prefix, tokens_per_frame) > 0) {
        if (!scratch) return op_fail(VITENC_ENULL, "scratch is NULL but this call needs it");
        if (reinterpret_cast<uintptr_t>(scratch) % 16 != 0) return op_fail(VITENC_EINVAL, "scratch must be 16-byte aligned");
    }
    return op_dev(launch_attention(dtype, Q, K, Vt, B, N, n_head, head_dim, (N + 63) / 64 * 64, attn_mode, n_prefix,
                                   tokens_per_frame, scratch, O, reinterpret_cast<hipStream_t>(stream)),
                  "attention");
}

vitenc_status vitenc_op_linear_residual(int32_t dtype, const void *A, const void *W, const float *b, const float *ls,
                                        int32_t M, int32_t Nout, int32_t K, float *Z, void *stream) {
    clear_error();
    if (!dtype_ok(dtype)) return op_fail(VITENC_EINVAL, "unknown dtype %d", dtype);
    if (!A || !W || !b || !Z) return op_fail(VITENC_ENULL, "a required pointer is NULL");
    if (M < 0 || Nout <= 0 || K <= 0) return op_fail(VITENC_ESHAPE, "bad sizes");
    EpiArgs ep;
    ep.bias = b; ep.ls = ls; ep.Z = Z; ep.ldz = Nout;
    return op_dev(launch_gemm(dtype, EPI_RESID, A, K, W, K, M, Nout, K, ep, reinterpret_cast<hipStream_t>(stream)),
                  "linear residual");
}

vitenc_status vitenc_op_linear_gelu(int32_t dtype, const void *A, const void *W, const float *b, int32_t M,
                                    int32_t Nout, int32_t K, void *U, void *stream) {
    clear_error();
    if (!dtype_ok(dtype)) return op_fail(VITENC_EINVAL, "unknown dtype %d", dtype);
    if (!A || !W || !b || !U) return op_fail(VITENC_ENULL, "a required pointer is NULL");
    if (M < 0 || Nout <= 0 || K <= 0) return op_fail(VITENC_ESHAPE, "bad sizes");
    EpiArgs ep;
    ep.bias = b; ep.out = U; ep.ldo = Nout;
    return op_dev(launch_gemm(dtype, EPI_GELU, A, K, W, K, M, Nout, K, ep, reinterpret_cast<hipStream_t>(stream)),
                  "linear gelu");
}

vitenc_status vitenc_op_linear_mxfp8(int32_t epi, const void *A, const uint8_t *codes, const uint8_t *scales,
                                     const float *b, const float *ls, int32_t M, int32_t Nout, int32_t K, void *out,
                                     void *stream) {
    clear_error();
    if (epi != 0 && epi != 1) return op_fail(VITENC_EINVAL, "unknown epilogue %d", epi);
    if (!A || !codes || !scales || !b || !out) return op_fail(VITENC_ENULL, "a required pointer is NULL");
    if (M < 0 || Nout <= 0 || K <= 0) return op_fail(VITENC_ESHAPE, "bad sizes");
    if (K % 64 || Nout % 8) return op_fail(VITENC_ESHAPE, "8-bit weights need K %% 64 == 0 and Nout %% 8 == 0");
    if (reinterpret_cast<uintptr_t>(A) % 16 || reinterpret_cast<uintptr_t>(codes) % 16)
        return op_fail(VITENC_EINVAL, "A and codes must be 16-byte aligned");
    EpiArgs ep;
    ep.bias = b;
    ep.wscale = scales;
    if (epi == 0) {
        ep.ls = ls; ep.Z = reinterpret_cast<float *>(out); ep.ldz = Nout;
    } else {
        ep.out = out; ep.ldo = Nout;
    }
    return op_dev(launch_gemm(VITENC_BF16, epi == 0 ? EPI_RESID : EPI_GELU, A, K, codes, K, M, Nout, K, ep,
                              reinterpret_cast<hipStream_t>(stream)),
                  "linear (8-bit weights)");
}

vitenc_status vitenc_quantize_mxfp8(const float *w, int32_t rows, int32_t cols, uint8_t *codes, uint8_t *scales,
                                    void *stream) {
    clear_error();
    if (!w || !codes || !scales) return op_fail(VITENC_ENULL, "a required pointer is NULL");
    if (rows <= 0 || cols <= 0 || cols % 64) return op_fail(VITENC_ESHAPE, "need rows > 0 and cols a multiple of 64");
    if (reinterpret_cast<uintptr_t>(w) % 16 || reinterpret_cast<uintptr_t>(codes) % 16)
        return op_fail(VITENC_EINVAL, "w and codes must be 16-byte aligned");
    return op_dev(launch_mxfp8_quantize(w, rows, cols, codes, scales, reinterpret_cast<hipStream_t>(stream)),
                  "quantize");
}

vitenc_status vitenc_op_pool(const float *X, int32_t B, int32_t N, int32_t D, int32_t cls, int32_t n_prefix,
                             float *pooled, void *stream) {
    clear_error();
    if (!X || !pooled) return op_fail(VITENC_ENULL, "a required pointer is NULL");
    if (B <= 0 || N <= 0 || D <= 0 || n_prefix < 0 || (!cls && n_prefix >= N))
        return op_fail(VITENC_ESHAPE, "bad sizes");
    return op_dev(launch_pool(X, B, N, D, cls, n_prefix, pooled, reinterpret_cast<hipStream_t>(stream)), "pool");
}

} // extern "C"
