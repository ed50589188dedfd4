// Fused attention O = softmax(Q K^T / sqrt(hd) + mask) V per item and head
// (jepa.cpp "Architecture", "The shared ViT graph" and "Block-causal
// attention"), an online-softmax ("flash") reorganisation of the exact
// softmax: nothing of size N^2 is ever stored.
//
// Work split: one 256-thread workgroup per (item, head, 128 queries); each of
// its 4 waves owns 32 queries.  Key/value tiles of 64 keys are staged through
// LDS (double-buffered, fetched into registers one tile ahead) and shared by
// the 4 waves.
//
// The score tile is computed transposed, S^T = K Q^T, with 32x32 MFMAs: then
// the accumulator of lane l holds 16 keys of query (l % 32), and the other
// half of that query's keys sits in lane l ^ 32, so the row max and row sum
// are in-lane reductions plus one cross-lane exchange.  P^T stays in
// registers and feeds O^T += V^T P^T directly as the B operand; V arrives
// already transposed per head (the QKV epilogue writes it that way).  In LDS
// each 16-key group of a V^T row is stored as [k0-3, k8-11 | k4-7, k12-15],
// so the 8 keys a lane group contributes to one 32x32x16 MFMA are one
// 16-byte read.  LDS chunk indices are XOR-swizzled by row (common.h).
//
// Mask: query i sees the keys [lo(i), hi(i)):
//   full attention                 lo = 0, hi = N
//   block-causal, prefix row i<p   lo = 0, hi = N        (the CLS row is open)
//   block-causal, patch row        lo = p, hi = p + (frame(i) + 1) * S
// with S patch tokens per frame and frame(i) = (i - p) / S.  This is the
// pages' rule (key j visible iff frame(i) >= frame(j); no patch row sees the
// CLS column) written as an interval, evaluated per element in registers
// only on tiles that straddle an interval bound; tiles wholly outside every
// query's interval are skipped.
#include "common.h"
#include "launch.h"

namespace vitenc {

namespace {

constexpr int kThreads = 256;
constexpr int BQ = 128;   // queries per workgroup
constexpr int BKV = 64;   // keys per tile

__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = min(v, __shfl_xor(v, off, 64));
    return v;
}
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = max(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ __forceinline__ void key_interval(int q, int N, int causal, int p, int S, int &lo, int &hi) {
    if (!causal || q < p) {
        lo = 0;
        hi = N;
    } else {
        lo = p;
        hi = min(N, p + ((q - p) / S + 1) * S);
    }
}

template <typename T, int HD>
__global__ __launch_bounds__(kThreads, 2) void attention_kernel(const T *__restrict__ Q, const T *__restrict__ K,
                                                                const T *__restrict__ Vt, int N, int H, int ldv,
                                                                int causal, int p, int S, float scale_log2,
                                                                T *__restrict__ O) {
    constexpr int KPC = Elem<T>::kPerChunk;
    constexpr int QCH = HD / KPC;     // 16-byte chunks per q/k row
    constexpr int KCH = BKV / KPC;    // 16-byte chunks per V^T row of a tile
    constexpr int K_PER = BKV * QCH / kThreads;
    constexpr int V_PER = HD * KCH / kThreads;
    constexpr int NDB = HD / 32;      // 32-row blocks of O^T
    static_assert(K_PER >= 1 && V_PER >= 1, "tile too small");

    __shared__ Chunk sK[2][BKV][QCH];
    __shared__ Chunk sV[2][HD][KCH];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, l32 = lane & 31;
    const int bh = blockIdx.x;                 // item * H + head
    const int b = bh / H, head = bh - b * H;
    const int qt = gridDim.y - 1 - blockIdx.y; // heavy (late-frame) tiles first
    const int q0 = qt * BQ;
    const int D = H * HD;

    const T *Qb = Q + (int64_t)bh * N * HD;
    const T *Kb = K + (int64_t)bh * N * HD;
    const T *Vb = Vt + (int64_t)bh * HD * ldv;

    // this lane's query and its visible key interval
    const int qrow = q0 + wave * 32 + l32;
    int lo, hi;
    key_interval(min(qrow, N - 1), N, causal, p, S, lo, hi);
    const int w_lo = wave_min_i(lo), w_hi = wave_max_i(hi);
    const int w_full_lo = wave_max_i(lo), w_full_hi = wave_min_i(hi);

    // workgroup key range (intervals are monotone in the query index)
    int wg_lo, wg_hi, tmp;
    key_interval(q0, N, causal, p, S, wg_lo, tmp);
    key_interval(min(q0 + BQ - 1, N - 1), N, causal, p, S, tmp, wg_hi);
    if (q0 < p) wg_hi = N;
    const int kt_begin = wg_lo / BKV, kt_end = (int)cdiv(wg_hi, BKV);

    // Q fragment (B operand of S^T = K Q^T): chunks 2s + g of this lane's query row
    Chunk qf[QCH / 2];
#pragma unroll
    for (int s = 0; s < QCH / 2; ++s)
        qf[s] = qrow < N ? load_chunk(Qb + (int64_t)qrow * HD + (2 * s + g) * KPC) : zero_chunk();

    Chunk rk[K_PER], rv[V_PER];
    auto gload = [&](int kt) {
        const int kb = kt * BKV;
#pragma unroll
        for (int i = 0; i < K_PER; ++i) {
            const int e = tid + kThreads * i;
            const int r = e / QCH, c = e % QCH;
            const int key = kb + r;
            rk[i] = key < N ? load_chunk(Kb + (int64_t)key * HD + c * KPC) : zero_chunk();
        }
#pragma unroll
        for (int i = 0; i < V_PER; ++i) {
            const int e = tid + kThreads * i;
            const int r = e / KCH, c = e % KCH;
            const int key = kb + c * KPC;
            const T *src = Vb + (int64_t)r * ldv + key;
            if (key + KPC <= N) {
                rv[i] = load_chunk(src);
            } else {
                Chunk z = zero_chunk();
                if constexpr (KPC == 4) {
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2)
                        if (key + e2 < N) z.w[e2] = __builtin_bit_cast(uint32_t, src[e2]);
                } else {
#pragma unroll
                    for (int e2 = 0; e2 < 8; ++e2)
                        if (key + e2 < N) z.w[e2 >> 1] |= bits16(src[e2]) << (16 * (e2 & 1));
                }
                rv[i] = z;
            }
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < K_PER; ++i) {
            const int e = tid + kThreads * i;
            const int r = e / QCH, c = e % QCH;
            sK[buf][r][c ^ swz<QCH>(r)] = rk[i];
        }
#pragma unroll
        for (int i = 0; i < V_PER; ++i) {
            const int e = tid + kThreads * i;
            const int r = e / KCH, c = e % KCH;
            if constexpr (KPC == 8) {
                // chunk c holds keys 8c..8c+7 = 16u + 8h + (0..7): its halves go to
                // logical slots 2u (keys +0..3) and 2u+1 (keys +4..7), at byte 8h
                const int u = c >> 1, h = c & 1;
                uint2 *row = reinterpret_cast<uint2 *>(&sV[buf][r][0]);
                row[2 * ((2 * u) ^ swz<KCH>(r)) + h] = make_uint2(rv[i].w[0], rv[i].w[1]);
                row[2 * ((2 * u + 1) ^ swz<KCH>(r)) + h] = make_uint2(rv[i].w[2], rv[i].w[3]);
            } else {
                sV[buf][r][c ^ swz<KCH>(r)] = rv[i];
            }
        }
    };

    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;

    if (kt_begin < kt_end) {
        gload(kt_begin);
        sstore(0);
    }
    __syncthreads();
    for (int kt = kt_begin; kt < kt_end; ++kt) {
        const int cur = (kt - kt_begin) & 1;
        const int kb = kt * BKV;
        if (kt + 1 < kt_end) gload(kt + 1);

        const bool active = kb < w_hi && kb + BKV > w_lo;
        if (active) {
            const bool need_mask = !(kb >= w_full_lo && kb + BKV <= w_full_hi);
            // ---- S^T for two 32-key blocks
            f32x16 sc[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
#pragma unroll
                for (int i = 0; i < 16; ++i) sc[j][i] = 0.0f;
                const int r = 32 * j + l32;
#pragma unroll
                for (int s = 0; s < QCH / 2; ++s) {
                    const Chunk a = sK[cur][r][(2 * s + g) ^ swz<QCH>(r)];
                    mfma_chunk<T>(sc[j], a, qf[s]);
                }
            }
            // ---- scale, mask, running max
            float mx = -INFINITY;
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float x = sc[j][i] * scale_log2;
                    if (need_mask) {
                        const int key = kb + 32 * j + acc_row(i, g);
                        if (key < lo || key >= hi) x = -INFINITY;
                    }
                    sc[j][i] = x;
                    mx = fmaxf(mx, x);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float m_new = fmaxf(m_run, mx);
            const float m_use = m_new == -INFINITY ? 0.0f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
            // ---- P = exp2(S - m), row sums, O^T += V^T P^T
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                float pv[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    pv[i] = __builtin_amdgcn_exp2f(sc[j][i] - m_use);
                    l_run += pv[i];
                }
                if constexpr (KPC == 8) {
                    // one 32x32x16 MFMA per 8 P values: slot e of lane group g is
                    // key 32j + 16st + 8*(e/4) + 4g + e%4 (accumulator slot 8st + e)
#pragma unroll
                    for (int st = 0; st < 2; ++st) {
                        Chunk pb;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            pb.w[e] = bits16(from_f32<T>(pv[8 * st + 2 * e])) |
                                      (bits16(from_f32<T>(pv[8 * st + 2 * e + 1])) << 16);
#pragma unroll
                        for (int db = 0; db < NDB; ++db) {
                            const int r = db * 32 + l32;
                            const int slot = 2 * (2 * j + st) + g;
                            mfma_chunk<T>(o[db], sV[cur][r][slot ^ swz<KCH>(r)], pb);
                        }
                    }
                } else {
                    // fp32: four 32x32x2 MFMAs per chunk of 4 consecutive keys
                    // 32j + 8*q4 + 4g + (0..3) (accumulator slots 4*q4 + 0..3)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        Chunk pb;
#pragma unroll
                        for (int e = 0; e < 4; ++e) pb.w[e] = __builtin_bit_cast(uint32_t, pv[4 * q4 + e]);
#pragma unroll
                        for (int db = 0; db < NDB; ++db) {
                            const int r = db * 32 + l32;
                            const int c = 8 * j + 2 * q4 + g;
                            mfma_chunk<T>(o[db], sV[cur][r][c ^ swz<KCH>(r)], pb);
                        }
                    }
                }
            }
        }
        if (kt + 1 < kt_end) sstore(cur ^ 1);
        __syncthreads();
    }

    // ---- normalise and store O[b, q, head*HD + d]
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    if (qrow < N) {
        T *orow = O + ((int64_t)b * N + qrow) * D + head * HD;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) orow[db * 32 + acc_row(i, g)] = from_f32<T>(o[db][i] * inv);
    }
}

template <typename T, int HD>
hipError_t launch_t(const void *Q, const void *K, const void *Vt, int B, int N, int H, int ldv, int causal, int p,
                    int S, void *O, hipStream_t s) {
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)HD);
    dim3 grid((unsigned)(B * H), (unsigned)cdiv(N, BQ));
    hipLaunchKernelGGL((attention_kernel<T, HD>), grid, dim3(kThreads), 0, s, reinterpret_cast<const T *>(Q),
                       reinterpret_cast<const T *>(K), reinterpret_cast<const T *>(Vt), N, H, ldv, causal, p, S,
                       scale_log2, reinterpret_cast<T *>(O));
    return hipGetLastError();
}

template <typename T>
hipError_t launch_hd(int head_dim, const void *Q, const void *K, const void *Vt, int B, int N, int H, int ldv,
                     int causal, int p, int S, void *O, hipStream_t s) {
    if (head_dim == 64) return launch_t<T, 64>(Q, K, Vt, B, N, H, ldv, causal, p, S, O, s);
    if (head_dim == 32) return launch_t<T, 32>(Q, K, Vt, B, N, H, ldv, causal, p, S, O, s);
    return hipErrorInvalidValue;
}

} // namespace

hipError_t launch_attention(int dtype, const void *Q, const void *K, const void *Vt, int B, int N, int H,
                            int head_dim, int ldv, int attn_mode, int n_prefix, int tokens_per_frame, void *O,
                            hipStream_t s) {
    if (B <= 0 || N <= 0) return hipSuccess;
    const int causal = attn_mode == 1;
    const int S = tokens_per_frame > 0 ? tokens_per_frame : 1;
    switch (dtype) {
    case DT_F32: return launch_hd<float>(head_dim, Q, K, Vt, B, N, H, ldv, causal, n_prefix, S, O, s);
    case DT_BF16: return launch_hd<bf16_t>(head_dim, Q, K, Vt, B, N, H, ldv, causal, n_prefix, S, O, s);
    case DT_F16: return launch_hd<f16_t>(head_dim, Q, K, Vt, B, N, H, ldv, causal, n_prefix, S, O, s);
    }
    return hipErrorInvalidValue;
}

} // namespace vitenc
