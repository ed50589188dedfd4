// Memory-bound steps of the encoder: patch rearrangement, LayerNorm, prefix
// (CLS) rows, the 3-D RoPE tables, and the pooled feature.
#include "common.h"
#include "launch.h"

namespace vitenc {

namespace {

// ---------------------------------------------------------------------------
// a1 rearrange NCTHW pixels into patch rows (jepa.cpp "Architecture", "The
// shared ViT graph"; "GGUF schema (v1)", "Encoder tensors": C-T-H-W order;
// "Token order": T-major, then H, then W).
//   A[b*Np + n, f] = X[b, c, t'*t + dt, h'*P + dh, w'*P + dw]
//   n = (t'*gh + h')*gw + w',  f = ((c*t + dt)*P + dh)*P + dw
// Columns f in [K, lda) are zero padding.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void patchify_kernel(const float *__restrict__ X, int C, int T_, int H,
                                                       int W, int tub, int P, int gh, int gw, int Np,
                                                       int K, int64_t lda, int64_t total, T *__restrict__ A) {
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t m = idx / lda;
        const int f0 = (int)(idx - m * lda);
        // split rows (lda == 2K): columns [K, 2K) hold x - round(x) of column f - K
        const bool lo = lda == 2 * (int64_t)K && f0 >= K;
        const int f = lo ? f0 - K : f0;
        float v = 0.0f;
        if (f < K) {
            const int b = (int)(m / Np), n = (int)(m - (int64_t)b * Np);
            const int tt = n / (gh * gw), hh = (n / gw) % gh, ww = n % gw;
            const int dw = f % P, dh = (f / P) % P, dt = (f / (P * P)) % tub, c = f / (P * P * tub);
            const int64_t src = ((((int64_t)b * C + c) * T_ + (tt * tub + dt)) * H + (hh * P + dh)) * W +
                                (ww * P + dw);
            v = X[src];
        }
        const T h = from_f32<T>(v);
        A[idx] = lo ? from_f32<T>(v - to_f32(h)) : h;
    }
}

// Row form of the same rearrangement: one thread moves one patch row, the P
// consecutive pixels of one (channel, frame, pixel row) of one token, which are
// P consecutive elements of A.  With P a multiple of 4 and W a multiple of 4 the
// row is read with 16-byte loads; bf16/f16 rows of 16 are written as two 16-byte
// chunks.  The thread that owns a token's last row also zeroes the pad columns.
template <typename T, int P, bool VEC, bool SPLIT>
__global__ __launch_bounds__(256) void patchify_rows_kernel(const float *__restrict__ X, int C, int T_, int H,
                                                            int W, int tub, int gh, int gw, int Np, int R, int K,
                                                            int lda, uint32_t total, T *__restrict__ A) {
    const uint32_t r = blockIdx.x * 256u + threadIdx.x;
    if (r >= total) return;
    const uint32_t m = r / (uint32_t)R, q = r - m * (uint32_t)R;
    const int dh = (int)(q % P), dt = (int)((q / P) % (uint32_t)tub), c = (int)(q / (P * (uint32_t)tub));
    const int b = (int)(m / (uint32_t)Np), n = (int)(m - (uint32_t)b * (uint32_t)Np);
    const int S = gh * gw;
    const int tt = n / S, hw = n - tt * S, hh = hw / gw, ww = hw - hh * gw;
    const float *src = X + ((((int64_t)b * C + c) * T_ + (tt * tub + dt)) * H + (hh * P + dh)) * (int64_t)W + ww * P;
    T *dst = A + (int64_t)m * lda + (int64_t)q * P;
    float v[P];
    if constexpr (VEC) {
#pragma unroll
        for (int i = 0; i < P / 4; ++i) {
            const float4 f = reinterpret_cast<const float4 *>(src)[i];
            v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < P; ++i) v[i] = src[i];
    }
    if constexpr (SPLIT && !(VEC && P % 8 == 0)) {
        // hi = round(x) in the first K columns, lo = round(x - hi) in the next K
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const T h = from_f32<T>(v[i]);
            dst[i] = h;
            dst[K + i] = from_f32<T>(v[i] - to_f32(h));
        }
        return;
    } else if constexpr (SPLIT) {
        static_assert(sizeof(T) == 2, "split rows are 16-bit");
#pragma unroll
        for (int i = 0; i < P / 8; ++i) {
            Chunk hi, lo;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float a = v[8 * i + 2 * j], b = v[8 * i + 2 * j + 1];
                const T ha = from_f32<T>(a), hb = from_f32<T>(b);
                hi.w[j] = bits16(ha) | (bits16(hb) << 16);
                lo.w[j] = pack2<T>(a - to_f32(ha), b - to_f32(hb));
            }
            store_chunk(dst + 8 * i, hi);
            store_chunk(dst + K + 8 * i, lo);
        }
        return;
    } else if constexpr (VEC && sizeof(T) == 2 && P % 8 == 0) {
#pragma unroll
        for (int i = 0; i < P / 8; ++i) {
            Chunk ch;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                ch.w[j] = pack2<T>(v[8 * i + 2 * j], v[8 * i + 2 * j + 1]);
            store_chunk(dst + 8 * i, ch);
        }
    } else if constexpr (VEC && sizeof(T) == 4) {
#pragma unroll
        for (int i = 0; i < P / 4; ++i)
            reinterpret_cast<float4 *>(dst)[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
    } else {
#pragma unroll
        for (int i = 0; i < P; ++i) dst[i] = from_f32<T>(v[i]);
    }
    if (q == (uint32_t)R - 1)
        for (int f = K; f < lda; ++f) A[(int64_t)m * lda + f] = from_f32<T>(0.0f);
}

// ---------------------------------------------------------------------------
// a4 LayerNorm: one wave per row, the row held in registers, centred
// two-pass population variance, eps inside the root ("GGUF schema (v1)",
// jepa.enc.ln_eps; "Architecture", "Attention and precision").
// When D is a multiple of 4 (and the rows 16-byte aligned) each lane moves 4
// consecutive elements per access (16-byte loads, 8-byte bf16 stores);
// otherwise element-wise.
// ---------------------------------------------------------------------------
template <typename TO>
__device__ __forceinline__ void store4(TO *dst, float a, float b, float c, float d) {
    if constexpr (sizeof(TO) == 4) {
        *reinterpret_cast<float4 *>(dst) = make_float4(a, b, c, d);
    } else {
        uint2 u;
        u.x = pack2<TO>(a, b);
        u.y = pack2<TO>(c, d);
        *reinterpret_cast<uint2 *>(dst) = u;
    }
}

template <typename TO, int NE>
__global__ __launch_bounds__(256) void layernorm_vec4_kernel(const float *__restrict__ x, const float *__restrict__ w,
                                                             const float *__restrict__ b, float eps, int M, int D,
                                                             TO *__restrict__ y) {
    const int lane = threadIdx.x & 63;
    // wave-uniform (scalar) row, so that the buffer resources below are scalar
    const int row = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= M) return;
    const int D4 = D >> 2;
    // the row, the scale and the shift are all requested before the first
    // reduction, so the three loads overlap; columns past D read as zero
    const uint32_t rb = (uint32_t)D * 4u;
    const __amdgpu_buffer_rsrc_t rx = buf_rsrc(x + (int64_t)row * D, rb);
    const __amdgpu_buffer_rsrc_t rw = buf_rsrc(w, rb), rbb = buf_rsrc(b, rb);
    float4 v[NE], ww[NE], bb[NE];
#pragma unroll
    for (int i = 0; i < NE; ++i) {
        const uint32_t off = (uint32_t)(lane + 64 * i) * 16u;
        v[i] = buf_f32x4(rx, off);
        ww[i] = buf_f32x4(rw, off);
        bb[i] = buf_f32x4(rbb, off);
    }
    // keep the scale and shift loads here, ahead of the reductions (the
    // scheduler would otherwise sink them to their use, a second round trip)
    __builtin_amdgcn_sched_barrier(0);
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < NE; ++i) s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    const float mean = wave_sum(s) / (float)D;
    float q = 0.0f;
#pragma unroll
    for (int i = 0; i < NE; ++i) {
        const float a = v[i].x - mean, c = v[i].y - mean, d = v[i].z - mean, e = v[i].w - mean;
        const float t = (a * a + c * c) + (d * d + e * e);
        q += lane + 64 * i < D4 ? t : 0.0f;
    }
    const float rstd = 1.0f / sqrtf(wave_sum(q) / (float)D + eps);
    TO *yr = y + (int64_t)row * D;
#pragma unroll
    for (int i = 0; i < NE; ++i) {
        const int c4 = lane + 64 * i;
        if (c4 < D4)
            store4<TO>(yr + 4 * c4, (v[i].x - mean) * rstd * ww[i].x + bb[i].x,
                       (v[i].y - mean) * rstd * ww[i].y + bb[i].y, (v[i].z - mean) * rstd * ww[i].z + bb[i].z,
                       (v[i].w - mean) * rstd * ww[i].w + bb[i].w);
    }
}

template <typename TO, int NE>
__global__ __launch_bounds__(256) void layernorm_kernel(const float *__restrict__ x, const float *__restrict__ w,
                                                        const float *__restrict__ b, float eps, int M, int D,
                                                        TO *__restrict__ y) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M) return;
    const float *xr = x + (int64_t)row * D;
    float v[NE];
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < NE; ++i) {
        const int c = lane + 64 * i;
        v[i] = c < D ? xr[c] : 0.0f;
        s += v[i];
    }
    const float mean = wave_sum(s) / (float)D;
    float q = 0.0f;
#pragma unroll
    for (int i = 0; i < NE; ++i) {
        const int c = lane + 64 * i;
        const float d = v[i] - mean;
        q += c < D ? d * d : 0.0f;
    }
    const float var = wave_sum(q) / (float)D;
    const float rstd = 1.0f / sqrtf(var + eps);
    TO *yr = y + (int64_t)row * D;
#pragma unroll
    for (int i = 0; i < NE; ++i) {
        const int c = lane + 64 * i;
        if (c < D) yr[c] = from_f32<TO>((v[i] - mean) * rstd * w[c] + b[c]);
    }
}

// ---------------------------------------------------------------------------
// a3 prefix rows: Z[b, 0] = cls (+ pos row 0) (+ mod)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prefix_rows_kernel(const float *__restrict__ cls, const float *__restrict__ pos,
                                                          const float *__restrict__ mod, int B, int Ntok, int D,
                                                          float *__restrict__ Z) {
    const int d = blockIdx.x * blockDim.x + threadIdx.x;
    const int b = blockIdx.y;
    if (d >= D || b >= B) return;
    float v = cls[d];
    if (pos) v += pos[d];
    if (mod) v += mod[d];
    Z[(int64_t)b * Ntok * D + d] = v;
}

// ---------------------------------------------------------------------------
// Position table resampled to another token grid (jepa.cpp "GGUF schema
// (v1)", "Encoder tensors": tables are built for the training grid and the
// runtime bicubic / trilinear-interpolates them for other grids).  Output
// row r < prefix copies input row r; patch row n = (t*dh + h)*dw + w reads
// source coordinate c = (o + 1/2) * n_in / n_out - 1/2 on each axis:
//   mode 1 (bicubic, one-frame tables): four taps floor(c) - 1 .. floor(c) + 2
//     per spatial axis, indices clamped to the axis, with the cubic-
//     convolution weights (Keys' kernel, a = -0.75) of t = c - floor(c);
//   mode 2 (trilinear): c clamped below at 0, taps floor(c) and floor(c) + 1
//     (clamped to the axis) with weights 1 - t and t, on every axis.
// Coordinates and weights are formed in fp64; the weighted sum in fp32.
// One workgroup per output row, four columns per thread.
// ---------------------------------------------------------------------------
__device__ __forceinline__ double cubic_w(double s) {
    constexpr double a = -0.75;
    s = fabs(s);
    if (s <= 1.0) return ((a + 2.0) * s - (a + 3.0)) * s * s + 1.0;
    if (s < 2.0) return ((a * s - 5.0 * a) * s + 8.0 * a) * s - 4.0 * a;
    return 0.0;
}

// taps (index, weight) of output sample o on an axis of n_in -> n_out
template <int MODE>
__device__ __forceinline__ void axis_taps(int o, int n_in, int n_out, int *idx, float *wt) {
    double c = ((double)o + 0.5) * (double)n_in / (double)n_out - 0.5;
    if constexpr (MODE == 1) {
        const double f = floor(c), t = c - f;
        const int i = (int)f;
        const double w[4] = {cubic_w(1.0 + t), cubic_w(t), cubic_w(1.0 - t), cubic_w(2.0 - t)};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            idx[k] = min(max(i - 1 + k, 0), n_in - 1);
            wt[k] = (float)w[k];
        }
    } else {
        c = fmax(c, 0.0);
        const double f = floor(c), t = c - f;
        const int i = (int)f;
        idx[0] = min(i, n_in - 1);
        idx[1] = min(i + 1, n_in - 1);
        wt[0] = (float)(1.0 - t);
        wt[1] = (float)t;
    }
}

template <int MODE>
__global__ __launch_bounds__(256) void pos_resample_kernel(const float *__restrict__ pos, int prefix, int D, int st,
                                                           int sh, int sw, int dt, int dh, int dw,
                                                           float *__restrict__ out) {
    const int r = blockIdx.x;
    float *o = out + (int64_t)r * D;
    if (r < prefix) {
        for (int c = threadIdx.x; c < D; c += blockDim.x) o[c] = pos[(int64_t)r * D + c];
        return;
    }
    const int n = r - prefix;
    const int w = n % dw, h = (n / dw) % dh, t = n / (dw * dh);
    constexpr int NT = MODE == 1 ? 4 : 2;
    int it[NT], ih[NT], iw[NT];
    float wt_t[NT], wt_h[NT], wt_w[NT];
    if constexpr (MODE == 1) {
        // one-frame table: no temporal taps
        it[0] = 0; wt_t[0] = 1.0f;
#pragma unroll
        for (int k = 1; k < NT; ++k) { it[k] = 0; wt_t[k] = 0.0f; }
    } else {
        axis_taps<MODE>(t, st, dt, it, wt_t);
    }
    axis_taps<MODE>(h, sh, dh, ih, wt_h);
    axis_taps<MODE>(w, sw, dw, iw, wt_w);
    const float *src = pos + (int64_t)prefix * D;
    for (int c = threadIdx.x; c < D; c += blockDim.x) {
        float acc = 0.0f;
#pragma unroll
        for (int a = 0; a < (MODE == 1 ? 1 : NT); ++a)
#pragma unroll
            for (int b = 0; b < NT; ++b)
#pragma unroll
                for (int e = 0; e < NT; ++e) {
                    const int64_t row = ((int64_t)it[a] * sh + ih[b]) * sw + iw[e];
                    acc = fmaf(wt_t[a] * wt_h[b] * wt_w[e], src[row * D + c], acc);
                }
        o[c] = acc;
    }
}

// ---------------------------------------------------------------------------
// a6 tables of the 3-D RoPE ("Architecture", "3-D RoPE"): for axis a in
// (t, h, w), position p and rotated element j in [0, d):
//   angle = pos_a(p) * omega_k,  omega_k = theta^(-2k/d),
//   k = j mod (d/2) (tiled) or j / 2 (interleaved),
//   pos_a(p) = p, or p * (ref - 1)/(g - 1) on h and w under interpolate_rope
// stored as (cos, sign_j * sin) with sign -1 on even j and +1 on odd j, so the
// rotation of element j is x_j * cos + x_{j^1} * signed_sin (rotate90 of the
// pair (y1, y2) is (-y2, y1)).  Also the packed (t, h, w) of each patch token
// (i = t*gh*gw + h*gw + w, "GGUF schema (v1)", "Token order").
// Angles are formed in fp64 and rounded once.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rope_table_kernel(int d, int layout, int interpolate, int ref_grid,
                                                         double theta, int gt, int gh, int gw,
                                                         float *__restrict__ tab, int *__restrict__ tok_pos) {
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    const int n_tab = (gt + gh + gw) * d;
    if (idx < n_tab) {
        const int p_all = idx / d, j = idx - p_all * d;
        int axis, p, g;
        if (p_all < gt) { axis = 0; p = p_all; g = gt; }
        else if (p_all < gt + gh) { axis = 1; p = p_all - gt; g = gh; }
        else { axis = 2; p = p_all - gt - gh; g = gw; }
        double pos = (double)p;
        if (interpolate && axis > 0 && g > 1) pos = pos * (double)(ref_grid - 1) / (double)(g - 1);
        const int k = layout == 0 ? (j % (d / 2)) : (j / 2);
        const double omega = pow(theta, -2.0 * (double)k / (double)d);
        const double ang = pos * omega;
        tab[2 * idx] = (float)cos(ang);
        tab[2 * idx + 1] = (float)((j & 1) ? sin(ang) : -sin(ang));
    }
    const int np = gt * gh * gw;
    if (tok_pos && idx < np) {
        const int t = idx / (gh * gw), h = (idx / gw) % gh, w = idx % gw;
        tok_pos[idx] = t | (h << 10) | (w << 20);
    }
}

// ---------------------------------------------------------------------------
// a11 pooled feature: the CLS row, or the mean of the patch rows.
// 1024 threads: 64 columns x 16 row groups, partial sums combined in LDS in a
// fixed order (deterministic).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void pool_kernel(const float *__restrict__ X, int N, int D, int cls,
                                                    int n_prefix, float *__restrict__ pooled) {
    // 16 columns x 64 row groups per block: enough blocks to spread one clip's
    // rows over the chip, each row group reading 64 contiguous bytes per row
    __shared__ float part[64][16];
    const int cx = threadIdx.x & 15, rg = threadIdx.x >> 4;
    const int d = blockIdx.x * 16 + cx;
    const int b = blockIdx.y;
    const float *xb = X + (int64_t)b * N * D;
    float s = 0.0f;
    if (d < D) {
        if (cls) {
            s = rg == 0 ? xb[d] : 0.0f;
        } else {
            // four independent partial sums, so that four row loads are in
            // flight per step (fixed order: deterministic)
            float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
            int n = n_prefix + rg;
            for (; n + 192 < N; n += 256) {
                s0 += xb[(int64_t)n * D + d];
                s1 += xb[(int64_t)(n + 64) * D + d];
                s2 += xb[(int64_t)(n + 128) * D + d];
                s3 += xb[(int64_t)(n + 192) * D + d];
            }
            for (; n < N; n += 64) s0 += xb[(int64_t)n * D + d];
            s = (s0 + s1) + (s2 + s3);
        }
    }
    part[rg][cx] = s;
    __syncthreads();
    if (rg == 0 && d < D) {
        float t = 0.0f;
        for (int r = 0; r < 64; ++r) t += part[r][cx];
        pooled[(int64_t)b * D + d] = cls ? t : t / (float)(N - n_prefix);
    }
}

template <typename TO>
hipError_t launch_ln_t(const float *x, const float *w, const float *b, float eps, int M, int D, TO *y,
                       hipStream_t s) {
    dim3 grid((unsigned)cdiv(M, 4)), block(256);
    const bool vec = D % 4 == 0 && (uintptr_t)x % 16 == 0 && (uintptr_t)w % 16 == 0 && (uintptr_t)b % 16 == 0 &&
                     (uintptr_t)y % 16 == 0;
    if (vec) {
        const int ne = (int)cdiv(D / 4, 64);
#define VITENC_LN4(NE_)                                                                                  \
    if (ne <= NE_) {                                                                                     \
        hipLaunchKernelGGL((layernorm_vec4_kernel<TO, NE_>), grid, block, 0, s, x, w, b, eps, M, D, y);  \
        return hipGetLastError();                                                                        \
    }
        VITENC_LN4(1)
        VITENC_LN4(2)
        VITENC_LN4(3)
        VITENC_LN4(4)
        VITENC_LN4(6)
        VITENC_LN4(8)
        VITENC_LN4(12)
        VITENC_LN4(16)
#undef VITENC_LN4
    }
    const int ne = (int)cdiv(D, 64);
#define VITENC_LN(NE_)                                                                                   \
    if (ne <= NE_) {                                                                                     \
        hipLaunchKernelGGL((layernorm_kernel<TO, NE_>), grid, block, 0, s, x, w, b, eps, M, D, y);       \
        return hipGetLastError();                                                                        \
    }
    VITENC_LN(4)
    VITENC_LN(8)
    VITENC_LN(16)
    VITENC_LN(24)
    VITENC_LN(32)
    VITENC_LN(48)
    VITENC_LN(64)
#undef VITENC_LN
    return hipErrorInvalidValue;
}

} // namespace

namespace {
template <typename T>
hipError_t launch_patchify_t(const float *px, int B, int C, int T_, int H, int W, int tub, int P, T *A,
                             int64_t lda, hipStream_t s) {
    const int gt = T_ / tub, gh = H / P, gw = W / P, Np = gt * gh * gw;
    const int K = C * tub * P * P;
    const int R = C * tub * P;
    const int64_t rows = (int64_t)B * Np * R;
    const bool aligned = W % 4 == 0 && (uintptr_t)px % 16 == 0 && (uintptr_t)A % 16 == 0 &&
                         (lda * (int64_t)sizeof(T)) % 16 == 0;
    const bool split = lda == 2 * (int64_t)K;
    if (rows < (int64_t(1) << 31) && lda < (int64_t(1) << 31) && (P == 16 || P == 14)) {
        const unsigned blocks = (unsigned)cdiv(rows, 256);
        if (split) {
            if constexpr (sizeof(T) == 2) {
                if (P == 16 && aligned)
                    hipLaunchKernelGGL((patchify_rows_kernel<T, 16, true, true>), dim3(blocks), dim3(256), 0, s, px,
                                       C, T_, H, W, tub, gh, gw, Np, R, K, (int)lda, (uint32_t)rows, A);
                else if (P == 16)
                    hipLaunchKernelGGL((patchify_rows_kernel<T, 16, false, true>), dim3(blocks), dim3(256), 0, s, px,
                                       C, T_, H, W, tub, gh, gw, Np, R, K, (int)lda, (uint32_t)rows, A);
                else
                    hipLaunchKernelGGL((patchify_rows_kernel<T, 14, false, true>), dim3(blocks), dim3(256), 0, s, px,
                                       C, T_, H, W, tub, gh, gw, Np, R, K, (int)lda, (uint32_t)rows, A);
            }
        } else if (P == 16 && aligned)
            hipLaunchKernelGGL((patchify_rows_kernel<T, 16, true, false>), dim3(blocks), dim3(256), 0, s, px, C, T_,
                               H, W, tub, gh, gw, Np, R, K, (int)lda, (uint32_t)rows, A);
        else if (P == 16)
            hipLaunchKernelGGL((patchify_rows_kernel<T, 16, false, false>), dim3(blocks), dim3(256), 0, s, px, C,
                               T_, H, W, tub, gh, gw, Np, R, K, (int)lda, (uint32_t)rows, A);
        else
            hipLaunchKernelGGL((patchify_rows_kernel<T, 14, false, false>), dim3(blocks), dim3(256), 0, s, px, C,
                               T_, H, W, tub, gh, gw, Np, R, K, (int)lda, (uint32_t)rows, A);
        return hipGetLastError();
    }
    const int64_t total = (int64_t)B * Np * lda;
    const unsigned blocks = (unsigned)std::min<int64_t>(cdiv(total, 256), 65535 * 8);
    hipLaunchKernelGGL(patchify_kernel<T>, dim3(blocks), dim3(256), 0, s, px, C, T_, H, W, tub, P, gh, gw, Np, K,
                       lda, total, A);
    return hipGetLastError();
}
} // namespace

hipError_t launch_patchify(int dtype, const float *px, int B, int C, int T, int H, int W, int tub, int P,
                           void *A, int64_t lda, hipStream_t s) {
    if ((int64_t)B * (T / tub) * (H / P) * (W / P) == 0) return hipSuccess;
    switch (dtype) {
    case DT_F32: return launch_patchify_t(px, B, C, T, H, W, tub, P, reinterpret_cast<float *>(A), lda, s);
    case DT_BF16: return launch_patchify_t(px, B, C, T, H, W, tub, P, reinterpret_cast<bf16_t *>(A), lda, s);
    case DT_F16: return launch_patchify_t(px, B, C, T, H, W, tub, P, reinterpret_cast<f16_t *>(A), lda, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_layernorm(int out_dtype, const float *x, const float *w, const float *b, float eps, int M, int D,
                            void *y, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    switch (out_dtype) {
    case DT_F32: return launch_ln_t<float>(x, w, b, eps, M, D, reinterpret_cast<float *>(y), s);
    case DT_BF16: return launch_ln_t<bf16_t>(x, w, b, eps, M, D, reinterpret_cast<bf16_t *>(y), s);
    case DT_F16: return launch_ln_t<f16_t>(x, w, b, eps, M, D, reinterpret_cast<f16_t *>(y), s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_prefix_rows(const float *cls, const float *pos, const float *mod, int B, int Ntok, int D,
                              float *Z, hipStream_t s) {
    dim3 grid((unsigned)cdiv(D, 256), (unsigned)B);
    hipLaunchKernelGGL(prefix_rows_kernel, grid, dim3(256), 0, s, cls, pos, mod, B, Ntok, D, Z);
    return hipGetLastError();
}

hipError_t launch_pos_resample(const float *pos, int prefix, int D, int st, int sh, int sw, int dt, int dh, int dw,
                               int mode, float *out, hipStream_t s) {
    const int rows = prefix + dt * dh * dw;
    if (rows <= 0) return hipSuccess;
    if (mode == 1)
        hipLaunchKernelGGL(pos_resample_kernel<1>, dim3((unsigned)rows), dim3(256), 0, s, pos, prefix, D, st, sh, sw, dt,
                           dh, dw, out);
    else if (mode == 2)
        hipLaunchKernelGGL(pos_resample_kernel<2>, dim3((unsigned)rows), dim3(256), 0, s, pos, prefix, D, st, sh, sw, dt,
                           dh, dw, out);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_rope_table(int head_dim, int layout, int interpolate, int ref_grid, float theta, int gt, int gh,
                             int gw, float *rope_tab, int *tok_pos, hipStream_t s) {
    const int d = 2 * ((head_dim / 3) / 2);
    const int n = std::max((gt + gh + gw) * d, gt * gh * gw);
    hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, d, layout, interpolate,
                       ref_grid, (double)theta, gt, gh, gw, rope_tab, tok_pos);
    return hipGetLastError();
}

hipError_t launch_pool(const float *X, int B, int N, int D, int cls, int n_prefix, float *pooled, hipStream_t s) {
    dim3 grid((unsigned)cdiv(D, 16), (unsigned)B);
    hipLaunchKernelGGL(pool_kernel, grid, dim3(1024), 0, s, X, N, D, cls, n_prefix, pooled);
    return hipGetLastError();
}

} // namespace vitenc
