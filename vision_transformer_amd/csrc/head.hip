// The attentive-pool head and its classifier after the pooler blocks
// (jepa.cpp "GGUF schema (v1)", "Head (jepa.head.*)"; SkyVision.cpp README,
// V-JEPA 2 backend notes, the pooler and classifier heads): one learned
// query attends over LayerNorm(tokens) with no output projection, then the
// query residual, an MLP with its own LayerNorm and residual, and a linear
// classifier.
//
// A single query makes the key and value projections foldable.  For head h,
//   q_h . k_j = q_h . (Wk_h y_j + bk_h) = (Wk_h^T q_h) . y_j + q_h . bk_h
// so the scores need one D-vector u_h = Wk_h^T q_h per head instead of the
// [N, D] key matrix, and, since the weights p_j of a head sum to one,
//   sum_j p_j (Wv_h y_j + bv_h) = Wv_h (sum_j p_j y_j) + bv_h,
// so the values need one weighted sum of the normalised tokens per head and
// one matrix-vector product.  The N x D x D key and value GEMMs become two
// passes over the tokens; what remains is bandwidth-bound.  With
// y_j = (z_j - mu_j) rstd_j gamma + beta and sum_j p_j = 1,
//   sum_j p_j y_j = gamma * sum_j (p_j rstd_j) (z_j - mu_j) + beta,
// so the second pass reads the raw tokens and the per-row statistics of the
// first.  Everything here is fp32 arithmetic on the model's weights.
#include "common.h"
#include "launch.h"

namespace vitenc {

namespace {

constexpr int kGemvBatch = 8;    // items per matrix-vector launch
constexpr int kWsumHeads = 16;   // heads per weighted-sum pass (accumulators per lane: 4 per head)
constexpr int kWsumRows = 256;   // tokens per weighted-sum workgroup
constexpr int kWsumGroups = 16;  // row groups of a weighted-sum workgroup (16 threads of 4 columns each)

// Sum of 64 values over the 64 lanes of a wave for 64 outputs at once: on
// entry every lane holds a partial of each output v[0..64); on exit lane l
// returns the total of output l.  Each butterfly step halves the outputs a
// lane keeps (the half selected by the lane's bit), so 63 shuffles serve all
// 64 outputs instead of 6 per output.  (One template level per step keeps
// every index a compile-time constant, so v stays in registers.)
template <int M>
__device__ __forceinline__ void butterfly_step(float (&v)[64], int lane) {
    const bool up = (lane & M) != 0;
#pragma unroll
    for (int i = 0; i < M; ++i) {
        const float send = up ? v[i] : v[i + M];
        const float keep = up ? v[i + M] : v[i];
        v[i] = keep + __shfl_xor(send, M, 64);
    }
    if constexpr (M > 1) butterfly_step<M / 2>(v, lane);
}
__device__ __forceinline__ float transpose_reduce64(float (&v)[64], int lane) {
    butterfly_step<32>(v, lane);
    return v[0];
}

constexpr int pow2_floor(int x) { return x >= 16 ? 16 : x >= 8 ? 8 : x >= 4 ? 4 : x >= 2 ? 2 : 1; }

template <typename T> __device__ __forceinline__ void unpack(const Chunk &c, float *v);
template <> __device__ __forceinline__ void unpack<float>(const Chunk &c, float *v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = __builtin_bit_cast(float, c.w[e]);
}
template <> __device__ __forceinline__ void unpack<bf16_t>(const Chunk &c, float *v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[2 * e] = __builtin_bit_cast(float, c.w[e] << 16);
        v[2 * e + 1] = __builtin_bit_cast(float, c.w[e] & 0xffff0000u);
    }
}
template <> __device__ __forceinline__ void unpack<f16_t>(const Chunk &c, float *v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[2 * e] = (float)__builtin_bit_cast(f16_t, (uint16_t)(c.w[e] & 0xffffu));
        v[2 * e + 1] = (float)__builtin_bit_cast(f16_t, (uint16_t)(c.w[e] >> 16));
    }
}

// out[b*ldo + r] = act(W[r, 0:C] . x_{b,r} + bias[r]) + res[b*ldr + r] for
// b < nb, with x_{b,r} = x + b*ldx + (r / rpg)*ldg (rows of one group share
// an input vector).  One wave per output row; each weight row is read once,
// in 16-byte loads (VEC: W, x and their strides allow them).
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void gemv_kernel(const T *__restrict__ W, int64_t ldw, const float *__restrict__ bias,
                                                   const float *__restrict__ x, int64_t ldx, int rpg, int64_t ldg,
                                                   int nb, int R, int C, int gelu, const float *__restrict__ res,
                                                   int64_t ldr, float *__restrict__ out, int64_t ldo) {
    constexpr int E = 16 / (int)sizeof(T); // weights per 16-byte load
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= R) return;
    const T *w = W + (int64_t)r * ldw;
    const float *xr = x + (int64_t)(r / rpg) * ldg;
    float acc[kGemvBatch];
#pragma unroll
    for (int b = 0; b < kGemvBatch; ++b) acc[b] = 0.0f;
    // four weight chunks in flight per lane before they are used
    constexpr int U = 4;
    for (int c0 = lane * E; c0 < C; c0 += U * 64 * E) {
        Chunk wc[U];
        if (VEC) {
#pragma unroll
            for (int k = 0; k < U; ++k) {
                const int c = c0 + k * 64 * E;
                wc[k] = c + E <= C ? load_chunk(w + c) : zero_chunk();
            }
        }
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const int c = c0 + k * 64 * E;
        if (c >= C) break;
        float wv[E];
        const bool full = c + E <= C;
        if (VEC && full) {
            unpack<T>(wc[k], wv);
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) wv[e] = c + e < C ? to_f32(w[c + e]) : 0.0f;
        }
#pragma unroll
        for (int b = 0; b < kGemvBatch; ++b) {
            if (b >= nb) break;
            const float *xb = xr + (int64_t)b * ldx + c;
            if (VEC && full) {
#pragma unroll
                for (int e = 0; e < E; e += 4) {
                    const float4 xv = *reinterpret_cast<const float4 *>(xb + e);
                    acc[b] = fmaf(wv[e], xv.x, acc[b]);
                    acc[b] = fmaf(wv[e + 1], xv.y, acc[b]);
                    acc[b] = fmaf(wv[e + 2], xv.z, acc[b]);
                    acc[b] = fmaf(wv[e + 3], xv.w, acc[b]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if (c + e < C) acc[b] = fmaf(wv[e], xb[e], acc[b]);
            }
        }
    }
    }
#pragma unroll
    for (int b = 0; b < kGemvBatch; ++b) {
        if (b >= nb) break;
        float v = wave_sum(acc[b]);
        if (lane == 0) {
            if (bias) v += bias[r];
            if (gelu) v = gelu_erf(v);
            if (res) v += res[(int64_t)b * ldr + r];
            out[(int64_t)b * ldo + r] = v;
        }
    }
}

// u[h*D + c] = scale * sum_i Wk[h*hd + i, c] q[h*hd + i] and
// ub[h] = scale * sum_i q[h*hd + i] bk[h*hd + i]: the key projection folded
// into the query.  Workgroup (column block of 64, head); four row groups per
// column, summed in a fixed order.
template <typename T>
__global__ __launch_bounds__(256) void fold_kernel(const T *__restrict__ Wk, int64_t ldw, const float *__restrict__ bk,
                                                   const float *__restrict__ q, int D, int hd, float scale,
                                                   float *__restrict__ u, float *__restrict__ ub) {
    __shared__ float red[4][64];
    const int lane = threadIdx.x & 63, g = threadIdx.x >> 6, h = blockIdx.y;
    const int c = blockIdx.x * 64 + lane;
    float acc = 0.0f;
    if (c < D)
#pragma unroll 8
        for (int i = g; i < hd; i += 4) acc = fmaf(to_f32(Wk[(int64_t)(h * hd + i) * ldw + c]), q[h * hd + i], acc);
    red[g][lane] = acc;
    __syncthreads();
    if (g == 0 && c < D) u[(int64_t)h * D + c] = scale * (((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane]);
    if (g == 0 && blockIdx.x == 0) {
        float t = 0.0f;
        for (int i = lane; i < hd; i += 64) t = fmaf(q[h * hd + i], bk[h * hd + i], t);
        t = wave_sum(t);
        if (lane == 0) ub[h] = scale * t;
    }
}

// First pass: per token row the key/value LayerNorm in registers (fp32,
// centred two-pass), then the scores of the workgroup's heads
// s[(b*H + h)*N + j] = u_h . y_j + ub[h] with u in LDS; head group 0 also
// stores the row's (mean, rstd).  A wave takes RB = 64/HP rows at a time,
// keeps one partial per (row, head) in each lane, and reduces all 64 of them
// over the wave in one transposed butterfly.  NE float4s per lane cover
// D <= 256*NE; HP is a power of two covering the HG heads of a group.
template <int NE, int HP>
__global__ __launch_bounds__(256) void xattn_scores_kernel(const float *__restrict__ Z, int M, int N, int D,
                                                           const float *__restrict__ ln_w,
                                                           const float *__restrict__ ln_b, float eps,
                                                           const float *__restrict__ u, const float *__restrict__ ub,
                                                           int H, int HG, float *__restrict__ s,
                                                           float2 *__restrict__ stats) {
    constexpr int RB = 64 / HP;
    extern __shared__ float su[]; // [HG][D]
    const int h0 = blockIdx.y * HG, nh = min(HG, H - h0);
    {
        // eight 16-byte loads in flight per thread before their LDS stores
        const float4 *u4 = reinterpret_cast<const float4 *>(u + (int64_t)h0 * D);
        float4 *s4 = reinterpret_cast<float4 *>(su);
        const int n4 = nh * D / 4;
        for (int i0 = threadIdx.x; i0 < n4; i0 += 8 * 256) {
            float4 a[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int i = i0 + k * 256;
                a[k] = i < n4 ? u4[i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (i0 + k * 256 < n4) s4[i0 + k * 256] = a[k];
        }
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int D4 = D / 4;
    const float4 *g4 = reinterpret_cast<const float4 *>(ln_w), *b4 = reinterpret_cast<const float4 *>(ln_b);
    const int row0 = (blockIdx.x * 4 + wave) * RB;
    float part[64];
#pragma unroll
    for (int i = 0; i < 64; ++i) part[i] = 0.0f;
    // PF rows at a time: their loads all in flight, each normalised in
    // registers, then every u fragment read from LDS serves all PF rows
    constexpr int PF = pow2_floor(RB < 16 / NE ? RB : (16 / NE > 0 ? 16 / NE : 1)); // divides RB
#pragma unroll
    for (int g0 = 0; g0 < RB; g0 += PF) {
        float4 y[PF][NE];
#pragma unroll
        for (int k = 0; k < PF; ++k) {
            const int row = row0 + g0 + k;
            const float4 *z = reinterpret_cast<const float4 *>(Z + (int64_t)min(row, M - 1) * D);
#pragma unroll
            for (int i = 0; i < NE; ++i) {
                const int c4 = lane + 64 * i;
                y[k][i] = c4 < D4 ? z[c4] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            }
        }
#pragma unroll
        for (int k = 0; k < PF; ++k) {
            const int row = row0 + g0 + k;
            float sum = 0.0f;
#pragma unroll
            for (int i = 0; i < NE; ++i) sum += (y[k][i].x + y[k][i].y) + (y[k][i].z + y[k][i].w);
            const float mean = wave_sum(sum) / (float)D;
            float sq = 0.0f;
#pragma unroll
            for (int i = 0; i < NE; ++i) {
                if (lane + 64 * i < D4) {
                    const float a = y[k][i].x - mean, b = y[k][i].y - mean, c = y[k][i].z - mean,
                                d = y[k][i].w - mean;
                    sq += (a * a + b * b) + (c * c + d * d);
                }
            }
            const float rstd = 1.0f / sqrtf(wave_sum(sq) / (float)D + eps);
#pragma unroll
            for (int i = 0; i < NE; ++i) {
                const int c4 = lane + 64 * i;
                if (c4 < D4) {
                    const float4 gw = g4[c4], gb = b4[c4];
                    y[k][i] = make_float4((y[k][i].x - mean) * rstd * gw.x + gb.x,
                                          (y[k][i].y - mean) * rstd * gw.y + gb.y,
                                          (y[k][i].z - mean) * rstd * gw.z + gb.z,
                                          (y[k][i].w - mean) * rstd * gw.w + gb.w);
                }
            }
            if (blockIdx.y == 0 && lane == 0 && row < M) stats[row] = make_float2(mean, rstd);
        }
#pragma unroll
        for (int h = 0; h < HP; ++h) {
            if (h < nh) {
                const float4 *uh = reinterpret_cast<const float4 *>(su + h * D);
                float d[PF];
#pragma unroll
                for (int k = 0; k < PF; ++k) d[k] = 0.0f;
#pragma unroll
                for (int i = 0; i < NE; ++i) {
                    const int c4 = lane + 64 * i;
                    if (c4 < D4) {
                        const float4 w4 = uh[c4];
#pragma unroll
                        for (int k = 0; k < PF; ++k) {
                            d[k] = fmaf(w4.x, y[k][i].x, d[k]);
                            d[k] = fmaf(w4.y, y[k][i].y, d[k]);
                            d[k] = fmaf(w4.z, y[k][i].z, d[k]);
                            d[k] = fmaf(w4.w, y[k][i].w, d[k]);
                        }
                    }
                }
#pragma unroll
                for (int k = 0; k < PF; ++k) part[(g0 + k) * HP + h] = d[k];
            }
        }
    }
    const float tot = transpose_reduce64(part, lane);
    const int r = lane / HP, h = lane - r * HP, row = row0 + r;
    if (row < M && h < nh) {
        const int b = row / N, j = row - b * N;
        s[((int64_t)b * H + h0 + h) * N + j] = tot + ub[h0 + h];
    }
}

// Softmax of each (item, head) row of scores, turned in place into the
// weights of the second pass: w_j = p_j * rstd_j.
__global__ __launch_bounds__(256) void xattn_softmax_kernel(float *__restrict__ s, const float2 *__restrict__ stats,
                                                            int N, int H) {
    __shared__ float red[4];
    const int bh = blockIdx.x, b = bh / H;
    float *row = s + (int64_t)bh * N;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float m = -INFINITY;
#pragma unroll 8
    for (int j = threadIdx.x; j < N; j += 256) m = fmaxf(m, row[j]);
    m = wave_max(m);
    if (lane == 0) red[wave] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float t = 0.0f;
#pragma unroll 8
    for (int j = threadIdx.x; j < N; j += 256) t += expf(row[j] - m);
    t = wave_sum(t);
    if (lane == 0) red[wave] = t;
    __syncthreads();
    const float inv = 1.0f / (((red[0] + red[1]) + red[2]) + red[3]);
#pragma unroll 8
    for (int j = threadIdx.x; j < N; j += 256) row[j] = expf(row[j] - m) * inv * stats[(int64_t)b * N + j].y;
}

// Second pass: P[((b*NC + ch)*H + h)*D + c] = sum over the chunk's tokens j
// of w[(b*H + h)*N + j] * (Z[b*N + j, c] - mean_j), for up to kWsumHeads
// heads.  A workgroup takes 64 columns (16 float4 columns) of kWsumRows
// tokens: 16 row groups stride over the tokens, and their partials are summed
// in LDS in a fixed order.
__global__ __launch_bounds__(256) void xattn_wsum_kernel(const float *__restrict__ Z, const float2 *__restrict__ stats,
                                                         const float *__restrict__ w, int N, int D, int H, int NC,
                                                         int n_hg, float *__restrict__ P) {
    __shared__ float sw[kWsumHeads][kWsumRows];
    __shared__ float smu[kWsumRows];
    __shared__ float4 red[kWsumGroups][kWsumHeads][16];
    const int b = blockIdx.z / n_hg, h0 = (blockIdx.z % n_hg) * kWsumHeads;
    const int nh = min(kWsumHeads, H - h0);
    const int ch = blockIdx.y, j0 = ch * kWsumRows, nj = min(kWsumRows, N - j0);
    for (int t = threadIdx.x; t < kWsumHeads * kWsumRows; t += 256) {
        const int h = t / kWsumRows, jj = t - h * kWsumRows;
        sw[h][jj] = (h < nh && jj < nj) ? w[((int64_t)b * H + h0 + h) * N + j0 + jj] : 0.0f;
    }
    for (int t = threadIdx.x; t < kWsumRows; t += 256) smu[t] = t < nj ? stats[(int64_t)b * N + j0 + t].x : 0.0f;
    __syncthreads();
    const int D4 = D / 4;
    const int cq = threadIdx.x & 15, rg = threadIdx.x >> 4;
    const int c4 = blockIdx.x * 16 + cq;
    float4 acc[kWsumHeads];
#pragma unroll
    for (int h = 0; h < kWsumHeads; ++h) acc[h] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (c4 < D4) {
        const float4 *z = reinterpret_cast<const float4 *>(Z + ((int64_t)b * N + j0) * D) + c4;
        // eight rows' loads in flight per thread, then their updates
        constexpr int U = 8;
        for (int j0r = rg; j0r < nj; j0r += U * kWsumGroups) {
            float4 d[U];
#pragma unroll
            for (int k = 0; k < U; ++k) {
                const int jj = j0r + k * kWsumGroups;
                d[k] = jj < nj ? z[(int64_t)jj * D4] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            }
#pragma unroll
            for (int k = 0; k < U; ++k) {
                const int jj = j0r + k * kWsumGroups;
                if (jj < nj) {
                    const float mu = smu[jj];
                    d[k].x -= mu; d[k].y -= mu; d[k].z -= mu; d[k].w -= mu;
#pragma unroll
                    for (int h = 0; h < kWsumHeads; ++h) {
                        const float p = sw[h][jj];
                        acc[h].x = fmaf(p, d[k].x, acc[h].x);
                        acc[h].y = fmaf(p, d[k].y, acc[h].y);
                        acc[h].z = fmaf(p, d[k].z, acc[h].z);
                        acc[h].w = fmaf(p, d[k].w, acc[h].w);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int h = 0; h < kWsumHeads; ++h) red[rg][h][cq] = acc[h];
    __syncthreads();
    const int h = threadIdx.x >> 4, q = threadIdx.x & 15;
    float4 t = red[0][h][q];
#pragma unroll
    for (int g = 1; g < kWsumGroups; ++g) {
        const float4 x = red[g][h][q];
        t.x += x.x; t.y += x.y; t.z += x.z; t.w += x.w;
    }
    const int c4o = blockIdx.x * 16 + q;
    if (h < nh && c4o < D4) reinterpret_cast<float4 *>(P + (((int64_t)b * NC + ch) * H + h0 + h) * D)[c4o] = t;
}

// ybar[(b*H + h)*D + c] = gamma_c * sum_ch P[((b*NC + ch)*H + h)*D + c] + beta_c
__global__ __launch_bounds__(256) void xattn_reduce_kernel(const float *__restrict__ P, int B, int NC, int H, int D,
                                                           const float *__restrict__ ln_w,
                                                           const float *__restrict__ ln_b, float *__restrict__ ybar) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t HD = (int64_t)H * D;
    if (i >= B * HD) return;
    const int b = (int)(i / HD);
    const int64_t hc = i - b * HD;
    const int c = (int)(hc % D);
    float t = 0.0f;
    for (int ch = 0; ch < NC; ++ch) t += P[((int64_t)b * NC + ch) * HD + hc];
    ybar[i] = ln_w[c] * t + ln_b[c];
}

template <typename T>
hipError_t gemv_t(const void *W, int64_t ldw, const float *bias, const float *x, int64_t ldx, int rpg, int64_t ldg,
                  int nb, int R, int C, bool gelu, const float *res, int64_t ldr, float *out, int64_t ldo,
                  hipStream_t s) {
    constexpr int E = 16 / (int)sizeof(T);
    const bool vec = ldw % E == 0 && (uintptr_t)W % 16 == 0 && (uintptr_t)x % 16 == 0 && ldx % 4 == 0 &&
                     ldg % 4 == 0;
    const T *w = reinterpret_cast<const T *>(W);
    for (int b0 = 0; b0 < nb; b0 += kGemvBatch) {
        const int n = std::min(kGemvBatch, nb - b0);
        const float *xb = x + (int64_t)b0 * ldx;
        const float *rb = res ? res + (int64_t)b0 * ldr : nullptr;
        float *ob = out + (int64_t)b0 * ldo;
        const dim3 grid((unsigned)cdiv(R, 4));
        if (vec)
            hipLaunchKernelGGL((gemv_kernel<T, true>), grid, dim3(256), 0, s, w, ldw, bias, xb, ldx, rpg, ldg, n, R, C,
                               (int)gelu, rb, ldr, ob, ldo);
        else
            hipLaunchKernelGGL((gemv_kernel<T, false>), grid, dim3(256), 0, s, w, ldw, bias, xb, ldx, rpg, ldg, n, R,
                               C, (int)gelu, rb, ldr, ob, ldo);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int NE>
hipError_t scores_t(const float *Z, int M, int N, int D, const float *ln_w, const float *ln_b, float eps,
                    const float *u, const float *ub, int H, float *s, float2 *stats, hipStream_t st) {
    // u of HG heads (at most 16 and 64 KB of LDS) per workgroup
    const int HG = std::max(1, std::min(std::min(H, 16), 16384 / D));
    const dim3 block(256);
    if (HG <= 4) {
        const dim3 grid((unsigned)cdiv(M, 4 * 16), (unsigned)cdiv(H, HG));
        hipLaunchKernelGGL((xattn_scores_kernel<NE, 4>), grid, block, (size_t)HG * D * sizeof(float), st, Z, M, N, D,
                           ln_w, ln_b, eps, u, ub, H, HG, s, stats);
    } else {
        const dim3 grid((unsigned)cdiv(M, 4 * 4), (unsigned)cdiv(H, HG));
        hipLaunchKernelGGL((xattn_scores_kernel<NE, 16>), grid, block, (size_t)HG * D * sizeof(float), st, Z, M, N,
                           D, ln_w, ln_b, eps, u, ub, H, HG, s, stats);
    }
    return hipGetLastError();
}

} // namespace

hipError_t launch_gemv(int dtype, const void *W, int64_t ldw, const float *bias, const float *x, int64_t ldx, int rpg,
                       int64_t ldg, int nb, int R, int C, bool gelu, const float *res, int64_t ldr, float *out,
                       int64_t ldo, hipStream_t s) {
    if (nb <= 0 || R <= 0) return hipSuccess;
    switch (dtype) {
    case DT_F32: return gemv_t<float>(W, ldw, bias, x, ldx, rpg, ldg, nb, R, C, gelu, res, ldr, out, ldo, s);
    case DT_BF16: return gemv_t<bf16_t>(W, ldw, bias, x, ldx, rpg, ldg, nb, R, C, gelu, res, ldr, out, ldo, s);
    case DT_F16: return gemv_t<f16_t>(W, ldw, bias, x, ldx, rpg, ldg, nb, R, C, gelu, res, ldr, out, ldo, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_xattn_fold(int dtype, const void *Wk, const float *bk, const float *q, int D, int H, float *u,
                             float *ub, hipStream_t s) {
    const int hd = D / H;
    const float scale = 1.0f / sqrtf((float)hd);
    const dim3 grid((unsigned)cdiv(D, 64), (unsigned)H);
    switch (dtype) {
    case DT_F32:
        hipLaunchKernelGGL(fold_kernel<float>, grid, dim3(256), 0, s, reinterpret_cast<const float *>(Wk), (int64_t)D,
                           bk, q, D, hd, scale, u, ub);
        break;
    case DT_BF16:
        hipLaunchKernelGGL(fold_kernel<bf16_t>, grid, dim3(256), 0, s, reinterpret_cast<const bf16_t *>(Wk),
                           (int64_t)D, bk, q, D, hd, scale, u, ub);
        break;
    case DT_F16:
        hipLaunchKernelGGL(fold_kernel<f16_t>, grid, dim3(256), 0, s, reinterpret_cast<const f16_t *>(Wk), (int64_t)D,
                           bk, q, D, hd, scale, u, ub);
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_xattn_scores(const float *Z, int B, int N, int D, const float *ln_w, const float *ln_b, float eps,
                               const float *u, const float *ub, int H, float *s, float2 *stats, hipStream_t st) {
    const int M = B * N;
    switch (cdiv(D, 256)) {
    case 1: return scores_t<1>(Z, M, N, D, ln_w, ln_b, eps, u, ub, H, s, stats, st);
    case 2: return scores_t<2>(Z, M, N, D, ln_w, ln_b, eps, u, ub, H, s, stats, st);
    case 3: return scores_t<3>(Z, M, N, D, ln_w, ln_b, eps, u, ub, H, s, stats, st);
    case 4: return scores_t<4>(Z, M, N, D, ln_w, ln_b, eps, u, ub, H, s, stats, st);
    case 5: case 6: return scores_t<6>(Z, M, N, D, ln_w, ln_b, eps, u, ub, H, s, stats, st);
    case 7: case 8: return scores_t<8>(Z, M, N, D, ln_w, ln_b, eps, u, ub, H, s, stats, st);
    case 9: case 10: case 11: case 12: return scores_t<12>(Z, M, N, D, ln_w, ln_b, eps, u, ub, H, s, stats, st);
    case 13: case 14: case 15: case 16: return scores_t<16>(Z, M, N, D, ln_w, ln_b, eps, u, ub, H, s, stats, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_xattn_softmax(float *s, const float2 *stats, int B, int N, int H, hipStream_t st) {
    hipLaunchKernelGGL(xattn_softmax_kernel, dim3((unsigned)(B * H)), dim3(256), 0, st, s, stats, N, H);
    return hipGetLastError();
}

int xattn_chunks(int N) { return (int)cdiv(N, kWsumRows); }

hipError_t launch_xattn_pool(const float *Z, const float2 *stats, const float *w, int B, int N, int D, int H,
                             const float *ln_w, const float *ln_b, float *P, float *ybar, hipStream_t st) {
    const int NC = xattn_chunks(N), n_hg = (int)cdiv(H, kWsumHeads);
    const dim3 grid((unsigned)cdiv(D / 4, 16), (unsigned)NC, (unsigned)(B * n_hg));
    hipLaunchKernelGGL(xattn_wsum_kernel, grid, dim3(256), 0, st, Z, stats, w, N, D, H, NC, n_hg, P);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)B * H * D;
    hipLaunchKernelGGL(xattn_reduce_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, st, P, B, NC, H, D, ln_w, ln_b,
                       ybar);
    return hipGetLastError();
}

} // namespace vitenc
