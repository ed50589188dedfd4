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
constexpr float kRescale = 8.0f; // log2 headroom before the running max moves
// LDS ring depth of the direct-to-LDS kernel: at hd 64 three stages (48 KB,
// so three workgroups fit a CU where the grid has that many: measured 4.1 %
// faster on the 18432-token clip, 0.8 % on the block-causal 4097-token clip and
// 0.3 % on 2 x 2048 tokens against four stages), at hd 32 four (the 8 KB
// stages never limit occupancy; three measured 1.2 % slower per predictor call)
template <int HD> constexpr int kStages = HD == 64 ? 3 : 4;
// key count from which the tile loads come from inline assembly: at hd 64 from
// 4096 keys (below that the builtin loads measured 1 % faster per encode), at
// hd 32 always (the predictor's 2048-key calls 0.7 % faster per call)
template <int HD> constexpr int kDeepKeys = HD == 64 ? 4096 : 0;
constexpr int kLdsWaves = 4; // waves (32 queries each) per workgroup, hd 64

// acc + lo + hi of a dword holding two 16-bit values (one packed dot product
// with (1, 1), fp32 accumulation)
template <typename T> __device__ __forceinline__ float sum2(uint32_t pk, float acc);
template <> __device__ __forceinline__ float sum2<bf16_t>(uint32_t pk, float acc) {
    const bf16x2_t one = {(bf16_t)1.0f, (bf16_t)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk), one, acc, false);
}
template <> __device__ __forceinline__ float sum2<f16_t>(uint32_t pk, float acc) {
    const f16x2_t one = {(f16_t)1.0f, (f16_t)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pk), one, acc, false);
}

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

__host__ __device__ __forceinline__ void key_interval(int q, int N, int causal, int p, int S, int &lo, int &hi) {
    if (!causal || q < p) {
        lo = 0;
        hi = N;
    } else {
        lo = p;
        const int end = p + ((q - p) / S + 1) * S;
        hi = end < N ? end : N;
    }
}

template <typename T, int HD>
__global__ __launch_bounds__(kThreads, 2) void attention_kernel(const T *__restrict__ Q, const T *__restrict__ K,
                                                                const T *__restrict__ Vt, int N, int H, int ldv,
                                                                int causal, int p, int S, int q_begin,
                                                                float scale_log2, T *__restrict__ O) {
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
    const int q0 = q_begin + qt * BQ;
    const int D = H * HD;

    const T *Qb = Q + (int64_t)bh * N * HD;
    const T *Kb = K + (int64_t)bh * N * HD;
    const T *Vb = Vt + (int64_t)bh * HD * ldv;

    // this lane's query and its visible key interval
    const int qrow = q0 + wave * 32 + l32;
    int lo, hi;
    key_interval(min(qrow, N - 1), N, causal, p, S, lo, hi);
    // a wave whose queries all lie past the end (in the last, partial query
    // tile) takes an empty interval: it joins the tile loads and barriers but
    // computes nothing
    const bool live = q0 + wave * 32 < N;
    const int w_lo = live ? wave_min_i(lo) : N, w_hi = live ? wave_max_i(hi) : 0;
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
    // A tile wholly inside [0, N) is fetched without per-chunk bounds checks
    // (the branch is uniform); the last, ragged tile zero-fills past N.
    auto gload_k = [&](int kt) {
        const int kb = kt * BKV;
#pragma unroll
        for (int i = 0; i < K_PER; ++i) {
            const int e = tid + kThreads * i;
            const int r = e / QCH, c = e % QCH;
            const int key = kb + r;
            rk[i] = (kb + BKV <= N || key < N) ? load_chunk(Kb + (int64_t)key * HD + c * KPC) : zero_chunk();
        }
    };
    auto gload_v = [&](int kt) {
        const int kb = kt * BKV;
        if (kb + BKV <= N) {
#pragma unroll
            for (int i = 0; i < V_PER; ++i) {
                const int e = tid + kThreads * i;
                const int r = e / KCH, c = e % KCH;
                rv[i] = load_chunk(Vb + (int64_t)r * ldv + kb + c * KPC);
            }
            return;
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
    auto sstore_k = [&](int buf) {
#pragma unroll
        for (int i = 0; i < K_PER; ++i) {
            const int e = tid + kThreads * i;
            const int r = e / QCH, c = e % QCH;
            sK[buf][r][c ^ swz<QCH>(r)] = rk[i];
        }
    };
    auto sstore_v = [&](int buf) {
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
    // S^T of one tile: two 32-key blocks of this wave's 32 queries
    auto scores = [&](f32x16 (&sc)[2], int buf) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
            for (int i = 0; i < 16; ++i) sc[j][i] = 0.0f;
            const int r = 32 * j + l32;
#pragma unroll
            for (int s2 = 0; s2 < QCH / 2; ++s2) {
                const Chunk a = sK[buf][r][(2 * s2 + g) ^ swz<QCH>(r)];
                mfma_chunk<T>(sc[j], a, qf[s2]);
            }
        }
    };
    auto tile_active = [&](int kt) { return kt * BKV < w_hi && kt * BKV + BKV > w_lo; };

    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;

    // Register-staged double buffer: tile t+1 is fetched into registers
    // while tile t is computed out of LDS, then stored into the other buffer.
    f32x16 sc[2];
    if (kt_begin < kt_end) {
        gload_k(kt_begin);
        gload_v(kt_begin);
        sstore_k(0);
        sstore_v(0);
    }
    __syncthreads();
    for (int kt = kt_begin; kt < kt_end; ++kt) {
        const int cur = (kt - kt_begin) & 1;
        const int kb = kt * BKV;
        if (kt + 1 < kt_end) {
            gload_k(kt + 1);
            gload_v(kt + 1);
        }
        if (tile_active(kt)) scores(sc, cur);

        if (tile_active(kt)) {
            const bool need_mask = !(kb >= w_full_lo && kb + BKV <= w_full_hi);
            // ---- mask, tile max of the raw scores (the scale is positive)
            float mx = -INFINITY;
            if (need_mask) {
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = kb + 32 * j + acc_row(i, g);
                        if (key < lo || key >= hi) sc[j][i] = -INFINITY;
                    }
            }
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[j][i]);
            mx *= scale_log2;
            // Lazy rescaling: the running max m_run (log2 units) moves only
            // when a score exceeds it by more than kRescale, so most tiles skip
            // the O rescale; exponents stay <= kRescale, and O / l is the same
            // for any m_run.  A query's scores sit in a lane pair (l, l ^ 32):
            // either lane's own maximum decides whether the pair's moves, and
            // the pair maximum is formed only on the rescaling tiles.
            if (__ballot(mx > m_run + kRescale)) {
                mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
                const bool grow = mx > m_run + kRescale;
                // lanes that do not grow keep their state (alpha 1): their
                // m_run may still be -inf, and exp2(-inf - -inf) is NaN
                const float m_new = grow ? mx : m_run;
                const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f; // 0 on the first tile
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
            }
            const float neg_m = m_run == -INFINITY ? 0.0f : -m_run;
            // ---- P = exp2(S - m), row sums, O^T += V^T P^T
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                float pv[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) pv[i] = __builtin_amdgcn_exp2f(fmaf(sc[j][i], scale_log2, neg_m));
                if constexpr (KPC == 8) {
                    // one 32x32x16 MFMA per 8 P values: slot e of lane group g is
                    // key 32j + 16st + 8*(e/4) + 4g + e%4 (accumulator slot 8st + e)
#pragma unroll
                    for (int st = 0; st < 2; ++st) {
                        Chunk pb;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            pb.w[e] = pack2<T>(pv[8 * st + 2 * e], pv[8 * st + 2 * e + 1]);
                            // the row sum adds the rounded weights the MFMA uses
                            l_run = sum2<T>(pb.w[e], l_run);
                        }
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
                        for (int e = 0; e < 4; ++e) {
                            pb.w[e] = __builtin_bit_cast(uint32_t, pv[4 * q4 + e]);
                            l_run += pv[4 * q4 + e];
                        }
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
        if (kt + 1 < kt_end) {
            sstore_k(cur ^ 1);
            sstore_v(cur ^ 1);
        }
        __syncthreads();
    }

    // ---- normalise and store O[b, q, head*HD + d]
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    if (qrow < N) {
        T *orow = O + ((int64_t)b * N + qrow) * D + head * HD;
        // accumulator slots 4u..4u+3 are 4 consecutive dims: one 8-byte store
        // (16 bytes for fp32) per group
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                T *dst = orow + db * 32 + acc_row(4 * u, g);
                const float a0 = o[db][4 * u] * inv, a1 = o[db][4 * u + 1] * inv;
                const float a2 = o[db][4 * u + 2] * inv, a3 = o[db][4 * u + 3] * inv;
                if constexpr (sizeof(T) == 4) {
                    *reinterpret_cast<float4 *>(dst) = make_float4(a0, a1, a2, a3);
                } else {
                    *reinterpret_cast<uint2 *>(dst) = make_uint2(pack2<T>(a0, a1), pack2<T>(a2, a3));
                }
            }
    }
}

// Direct-to-LDS form for 16-bit types: the K and V^T tiles are fetched from
// HBM straight into a ring of STAGES LDS stages with buffer loads, so up to
// STAGES - 1 tiles are in flight while one is computed.  The K rows of each
// 16-key group are stored with bits 2 and 3 of the row index swapped: the
// score accumulator row R then holds key pi(R), and the 8 probabilities a lane
// group feeds one P.V MFMA are 8 consecutive keys, matching a plain 16-byte
// read of a V^T row.  Loads past the end of K read zeros (buffer range
// check); the V^T columns of the ragged last tile are zeroed in LDS.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rs, Chunk *dst, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)dst, 16, voff, soff, 0, 0);
}
// The same load from inline assembly (M0 carries the LDS address; nothing
// else in the kernel keeps a value in M0).  The compiler does not count
// these loads: with them and a compiler-visible wait for the Q fragments
// before the key loop, the loop carries no wait of the compiler's own, only
// the kernel's vm_wait for the tile it is about to read.  (With the builtin
// the compiler cannot tell the ring stages apart and waits for every load in
// flight, the newest tile's included, before each tile's first fragment
// reads.)
__device__ __forceinline__ void load_lds16_asm(__amdgpu_buffer_rsrc_t rs, Chunk *dst, uint32_t voff, uint32_t soff) {
    const uint32_t lds = (uint32_t)(uintptr_t)(const lds_void_t *)dst;
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds), "v"(voff), "s"(rs),
                 "s"(soff)
                 : "memory");
}
__device__ __forceinline__ int key_perm(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Prefix (CLS) query rows.  They see every key in both masks (the CLS row is
// open), and a tile of 32*NWV queries holding a single prefix query would
// cost as much as a full tile, so the tiled kernels start at the first patch
// query and the prefix rows are computed here, split over the keys: one
// workgroup per (prefix row, head, run of kPrefixKeys keys) stores the
// fp32 scores of its keys (16-byte K row loads) in LDS, turns them into
// weights against the run's own max, and multiplies them into V (each thread
// one output dim of one key group, 16-byte runs of V^T); the partial
// (max, sum, o[HD]) goes to scratch, and a merge kernel combines the runs of
// a row in order (online-softmax rescaling).  In 16-bit calls these
// workgroups are the last ones of the tiled kernel's own grid (short jobs
// that fill the CUs the heavy tiles leave idle at the end), not a launch of
// their own.
constexpr int kPrefixThreads = 256;
constexpr int kPrefixKeys = 256;

// QR query rows of one (item, head) per workgroup (the rows of a row-split
// call share their K and V^T reads; a prefix call has QR = 1): thread k of the
// run scores key k against each row, the weights go through LDS, and thread
// (group, d) accumulates output dim d over its key group for each row.
// Rows pq0 .. pq0 + nq - 1 of (item, head) bh, keys of run `run` of `runs`;
// smem: prefix_smem_floats<HD, QR>() floats of LDS.  Every thread of the
// workgroup (kPrefixThreads) calls it.
template <int HD, int QR> constexpr int prefix_smem_floats() {
    return QR * kPrefixKeys + QR * HD + 2 * QR * (kPrefixThreads / 64) + QR * (kPrefixThreads / HD) * HD;
}
template <typename T, int HD, int QR>
__device__ __forceinline__ void prefix_run(const T *__restrict__ Q, const T *__restrict__ K,
                                           const T *__restrict__ Vt, int N, int ldv, int p, float scale_log2,
                                           float *__restrict__ part, int bh, int pq0, int nq, int run, int runs,
                                           float *smem) {
    constexpr int KPC = Elem<T>::kPerChunk;
    constexpr int NW = kPrefixThreads / 64;
    constexpr int G = kPrefixThreads / HD;   // key groups of the PV step
    constexpr int VE = 16 / (int)sizeof(T);  // keys per 16-byte V^T load
    static_assert(kPrefixKeys <= kPrefixThreads, "one key per thread");
    static_assert(QR * HD <= kPrefixThreads, "one query element per thread");
    float(*ss)[kPrefixKeys] = reinterpret_cast<float(*)[kPrefixKeys]>(smem);
    float(*sq)[HD] = reinterpret_cast<float(*)[HD]>(smem + QR * kPrefixKeys);
    float(*red)[QR][NW] = reinterpret_cast<float(*)[QR][NW]>(smem + QR * kPrefixKeys + QR * HD);
    float(*so)[G][HD] = reinterpret_cast<float(*)[G][HD]>(smem + QR * kPrefixKeys + QR * HD + 2 * QR * NW);
    const int c0 = run * kPrefixKeys, n = min(kPrefixKeys, N - c0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int d = tid % HD, grp = tid / HD;
    if (tid < QR * HD) {
        const int q = tid / HD;
        sq[q][d] = q < nq ? to_f32(Q[((int64_t)bh * N + pq0 + q) * HD + d]) * scale_log2 : 0.0f;
    }
    __syncthreads();
    float sc[QR];
#pragma unroll
    for (int q = 0; q < QR; ++q) sc[q] = -INFINITY;
    if (tid < n) {
#pragma unroll
        for (int q = 0; q < QR; ++q) sc[q] = 0.0f;
        const T *kr = K + ((int64_t)bh * N + c0 + tid) * HD;
#pragma unroll
        for (int c = 0; c < HD / KPC; ++c) {
            const Chunk ch = load_chunk(kr + c * KPC);
            const T *e = reinterpret_cast<const T *>(&ch);
#pragma unroll
            for (int u = 0; u < KPC; ++u) {
                const float kv = to_f32(e[u]);
#pragma unroll
                for (int q = 0; q < QR; ++q) sc[q] = fmaf(sq[q][c * KPC + u], kv, sc[q]);
            }
        }
    }
#pragma unroll
    for (int q = 0; q < QR; ++q) {
        const float mw = wave_max(sc[q]);
        if (lane == 0) red[0][q][wave] = mw;
    }
    __syncthreads();
    float m[QR];
#pragma unroll
    for (int q = 0; q < QR; ++q) {
        m[q] = red[0][q][0];
#pragma unroll
        for (int w = 1; w < NW; ++w) m[q] = fmaxf(m[q], red[0][q][w]);
        const float wgt = tid < n ? __builtin_amdgcn_exp2f(sc[q] - m[q]) : 0.0f;
        ss[q][tid] = wgt;
        const float lw = wave_sum(wgt);
        if (lane == 0) red[1][q][wave] = lw;
    }
    __syncthreads();
    const T *vrow = Vt + ((int64_t)bh * HD + d) * ldv + c0;
    float acc[QR];
#pragma unroll
    for (int q = 0; q < QR; ++q) acc[q] = 0.0f;
    const int full = n / VE * VE;
    for (int k = grp * VE; k < full; k += G * VE) {
        const Chunk ch = load_chunk(vrow + k);
        const T *e = reinterpret_cast<const T *>(&ch);
#pragma unroll
        for (int u = 0; u < VE; ++u) {
            const float vv = to_f32(e[u]);
#pragma unroll
            for (int q = 0; q < QR; ++q) acc[q] = fmaf(ss[q][k + u], vv, acc[q]);
        }
    }
    for (int k = full + grp; k < n; k += G) {
        const float vv = to_f32(vrow[k]);
#pragma unroll
        for (int q = 0; q < QR; ++q) acc[q] = fmaf(ss[q][k], vv, acc[q]);
    }
#pragma unroll
    for (int q = 0; q < QR; ++q) so[q][grp][d] = acc[q];
    __syncthreads();
    if (tid < QR * HD) {
        const int q = tid / HD;
        if (q < nq) {
            float t = 0.0f;
#pragma unroll
            for (int g2 = 0; g2 < G; ++g2) t += so[q][g2][d];
            float *out = part + (((int64_t)bh * p + pq0 + q) * runs + run) * (HD + 2);
            out[2 + d] = t;
            if (d == 0) {
                float l = 0.0f;
#pragma unroll
                for (int w = 0; w < NW; ++w) l += red[1][q][w];
                out[0] = m[q];
                out[1] = l;
            }
        }
    }
}

// Order in which the workgroups of the direct-to-LDS kernel take the query
// tiles, and which tiles are computed as two workgroups over halves of their
// keys.  With the block-causal mask a late frame's query tile sees up to
// (frames) times the keys of frame 0's; when the grid is one or two rounds of
// workgroups over the CUs, the late tiles alone then set the kernel's time.
// When the largest key count is at least twice the smallest, a tile is split
// in two when its key tiles exceed a third of the largest count: each half
// writes its unnormalised partial (o, running max, running sum) to scratch and
// merge_kernel combines the two.  Tiles of equal cost (no mask, or a single
// frame) split the same way when their grid leaves a last round of
// workgroups less than half full: the last tiles of every (item, head) then
// run as halves, so the last round holds half tiles.  Jobs run largest
// first.  n = 0: no split, tiles in reverse order (the heaviest last tiles
// first), one workgroup each.
constexpr int kMaxJobs = 480;
constexpr int kSplitMaxWorkgroups = 1024; // block-causal: above this the dispatcher balances the tiles by itself
constexpr int kSplitMinKeyTiles = 8;
struct TileOrder {
    int n;      // jobs (the grid's y extent), 0 when nothing is split
    int qs;     // the query tiles qs .. T-1 are split
    int nslots; // T - qs
    uint16_t job[kMaxJobs]; // bits 0-13 query tile; bits 14-15: 0 all keys, 1 first half, 2 second half
};

// DEEP: the tile loads from inline assembly (load_lds16_asm), for long key
// sequences, where the ring then keeps STAGES - 1 tiles in flight.
template <typename T, int HD, int STAGES, int NWV, bool DEEP>
__global__ __launch_bounds__(64 * NWV, 2) void attention_lds_kernel(const T *__restrict__ Q, const T *__restrict__ K,
                                                                    const T *__restrict__ Vt, int N, int H, int ldv,
                                                                    int causal, int p, int S, int q_begin,
                                                                    float scale_log2, const TileOrder order,
                                                                    float *__restrict__ part, int pre_y0,
                                                                    float *__restrict__ pre_part, T *__restrict__ O) {
    static_assert(sizeof(T) == 2, "16-bit types");
    constexpr int KPC = 8;
    constexpr int QCH = HD / KPC;              // chunks per K row (8 or 4)
    constexpr int VCH = BKV / KPC;             // chunks per V^T row of a tile (8)
    constexpr int KRI = 64 / QCH;              // K rows per load instruction
    constexpr int VRI = 64 / VCH;              // V^T rows per load instruction
    constexpr int NW = NWV;
    constexpr int kThreadsL = 64 * NWV, BQL = 32 * NWV; // threads, queries per workgroup
    constexpr int K_INST = BKV / (KRI * NW);   // per wave and tile
    constexpr int V_INST = HD / (VRI * NW);
    constexpr int PER = K_INST + V_INST;
    constexpr int NDB = HD / 32;
    static_assert(K_INST >= 1 && V_INST >= 1 && K_INST * KRI * NW == BKV && V_INST * VRI * NW == HD, "tile");
    static_assert(STAGES >= 2 && STAGES <= 4 && (STAGES - 2) * PER <= 63, "vmcnt range");

    __shared__ Chunk sK[STAGES][BKV][QCH];
    __shared__ Chunk sV[STAGES][HD][VCH];

    if ((int)blockIdx.y >= pre_y0) {
        // a run of keys of one prefix row (rows q_begin of every (item, head))
        static_assert(kThreadsL == kPrefixThreads && prefix_smem_floats<HD, 1>() * 4 <= (int)sizeof(sK), "prefix job");
        const int runs = (int)cdiv(N, kPrefixKeys), y = (int)blockIdx.y - pre_y0;
        const int pq = y / runs;
        prefix_run<T, HD, 1>(Q, K, Vt, N, ldv, q_begin, scale_log2, pre_part, (int)blockIdx.x, pq, 1, y - pq * runs,
                             runs, reinterpret_cast<float *>(&sK[0][0][0]));
        return;
    }

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, l32 = lane & 31;
    const int bh = blockIdx.x;
    const int b = bh / H, head = bh - b * H;
    int qt = pre_y0 - 1 - blockIdx.y, piece = 0; // heavy (late-frame) tiles first
    if (order.n > 0) {
        const int j = order.job[blockIdx.y];
        qt = j & 0x3FFF;
        piece = j >> 14;
    }
    const int q0 = q_begin + qt * BQL;
    const int D = H * HD;

    const T *Qb = Q + (int64_t)bh * N * HD;
    const T *Kb = K + (int64_t)bh * N * HD;
    const T *Vb = Vt + (int64_t)bh * HD * ldv;
    const __amdgpu_buffer_rsrc_t rsk =
        __builtin_amdgcn_make_buffer_rsrc((void *)Kb, 0, (int)((int64_t)N * HD * sizeof(T)), 0x00020000);
    const __amdgpu_buffer_rsrc_t rsv =
        __builtin_amdgcn_make_buffer_rsrc((void *)Vb, 0, (int)((int64_t)HD * ldv * sizeof(T)), 0x00020000);

    const int qrow = q0 + wave * 32 + l32;
    int lo, hi;
    key_interval(min(qrow, N - 1), N, causal, p, S, lo, hi);
    // a wave whose queries all lie past the end (in the last, partial query
    // tile) takes an empty interval: it joins the tile loads and barriers but
    // computes nothing
    const bool live = q0 + wave * 32 < N;
    const int w_lo = live ? wave_min_i(lo) : N, w_hi = live ? wave_max_i(hi) : 0;
    const int w_full_lo = wave_max_i(lo), w_full_hi = wave_min_i(hi);
    int wg_lo, wg_hi, tmp;
    key_interval(q0, N, causal, p, S, wg_lo, tmp);
    key_interval(min(q0 + BQL - 1, N - 1), N, causal, p, S, tmp, wg_hi);
    if (q0 < p) wg_hi = N;
    int kt_begin = wg_lo / BKV, kt_end = (int)cdiv(wg_hi, BKV);
    if (piece) {
        const int mid = kt_begin + (kt_end - kt_begin) / 2;
        if (piece == 1) kt_end = mid;
        else kt_begin = mid;
    }
    const int ntiles = kt_end - kt_begin;

    Chunk qf[QCH / 2];
#pragma unroll
    for (int s2 = 0; s2 < QCH / 2; ++s2)
        qf[s2] = qrow < N ? load_chunk(Qb + (int64_t)qrow * HD + (2 * s2 + g) * KPC) : zero_chunk();
    if constexpr (DEEP) __builtin_amdgcn_s_waitcnt(0xF70); // vmcnt(0): the Q fragments have landed

    // per-lane byte offsets of the tile loads (the tile's key offset goes in
    // the scalar offset)
    uint32_t vk[K_INST], vv[V_INST];
#pragma unroll
    for (int j = 0; j < K_INST; ++j) {
        const int r = (wave * K_INST + j) * KRI + lane / QCH, c = lane % QCH;
        vk[j] = (uint32_t)((key_perm(r) * HD + (c ^ swz<QCH>(r)) * KPC) * sizeof(T));
    }
#pragma unroll
    for (int j = 0; j < V_INST; ++j) {
        const int r = (wave * V_INST + j) * VRI + lane / VCH, c = lane % VCH;
        vv[j] = (uint32_t)(((int64_t)r * ldv + (c ^ swz<VCH>(r)) * KPC) * sizeof(T));
    }
    auto issue = [&](int stage, int kt) {
        const uint32_t koff = (uint32_t)(kt * BKV) * HD * (uint32_t)sizeof(T);
        const uint32_t voff = (uint32_t)(kt * BKV) * (uint32_t)sizeof(T);
#pragma unroll
        for (int j = 0; j < K_INST; ++j) {
            if constexpr (DEEP) load_lds16_asm(rsk, &sK[stage][(wave * K_INST + j) * KRI][0], vk[j], koff);
            else load_lds16(rsk, &sK[stage][(wave * K_INST + j) * KRI][0], vk[j], koff);
        }
#pragma unroll
        for (int j = 0; j < V_INST; ++j) {
            if constexpr (DEEP) load_lds16_asm(rsv, &sV[stage][(wave * V_INST + j) * VRI][0], vv[j], voff);
            else load_lds16(rsv, &sV[stage][(wave * V_INST + j) * VRI][0], vv[j], voff);
        }
    };
    auto wait_tile = [&](int later) {
        if (later >= 2) vm_wait<(STAGES > 3 ? 2 * PER : 0)>();
        else if (later == 1) vm_wait<(STAGES > 2 ? PER : 0)>();
        else vm_wait<0>();
        __syncthreads();
    };

    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;
    // Row sums: with hd 64 a lane adds its rounded weights with packed dot
    // products (VALU); with hd 32, where the softmax's VALU work outweighs
    // the MFMAs twice over, an MFMA of the weights against a block of ones
    // forms them (every accumulator slot of a lane then holds its query's
    // sum over all the keys of both lane groups).
    constexpr bool kMfmaSum = HD == 32;
    f32x16 lsum;
#pragma unroll
    for (int i = 0; i < 16; ++i) lsum[i] = 0.0f;
    Chunk ones;
#pragma unroll
    for (int i = 0; i < 4; ++i) ones.w[i] = pack2<T>(1.0f, 1.0f);

#pragma unroll
    for (int s2 = 0; s2 < STAGES - 1; ++s2)
        if (s2 < ntiles) issue(s2, kt_begin + s2);

    // Lane byte offsets of the fragment reads within a stage (the swizzle
    // depends on the row's low 4 bits only, so rows 32 apart share it); with
    // the loop unrolled over the ring, the stage and the 32-row block are
    // immediate offsets of the reads.  They pass through an empty asm once per
    // tile, so that the compiler keeps one register per offset instead of a
    // sum per stage.
    uint32_t kofs[QCH / 2], vofs[4];
#pragma unroll
    for (int s2 = 0; s2 < QCH / 2; ++s2)
        kofs[s2] = (uint32_t)(l32 * QCH + ((2 * s2 + g) ^ swz<QCH>(l32))) * (uint32_t)sizeof(Chunk);
#pragma unroll
    for (int c = 0; c < 4; ++c)
        vofs[c] = (uint32_t)(l32 * VCH + ((2 * c + g) ^ swz<VCH>(l32))) * (uint32_t)sizeof(Chunk);
    auto lds_chunk = [](const void *base, uint32_t off) __attribute__((always_inline)) {
        return *reinterpret_cast<const Chunk *>(reinterpret_cast<const char *>(base) + off);
    };
    auto tile_step = [&](auto pos, int t) __attribute__((always_inline)) {
        constexpr int stg = decltype(pos)::value;
        const int kt = kt_begin + t, kb = kt * BKV;
#pragma unroll
        for (int i = 0; i < QCH / 2; ++i) asm("" : "+v"(kofs[i]));
#pragma unroll
        for (int i = 0; i < 4; ++i) asm("" : "+v"(vofs[i]));
        // tiles issued so far: 0 .. min(t + STAGES - 2, ntiles - 1)
        wait_tile(min(t + STAGES - 2, ntiles - 1) - t);
        // every wave is past tile t-1, so its stage can be refilled
        if (t + STAGES - 1 < ntiles) issue((stg + STAGES - 1) % STAGES, kt + STAGES - 1);
        if (kb + BKV > N) {
            // ragged last tile: V^T columns of keys >= N hold whatever follows
            // the last token in memory; make them zero
            for (int e = tid; e < HD * BKV; e += kThreadsL) {
                const int d = e / BKV, key = e % BKV;
                if (kb + key >= N) {
                    T *row = reinterpret_cast<T *>(&sV[stg][d][0]);
                    row[((key / KPC) ^ swz<VCH>(d)) * KPC + key % KPC] = from_f32<T>(0.0f);
                }
            }
            __syncthreads();
        }
        if (!(kb < w_hi && kb + BKV > w_lo)) return;
        const bool need_mask = !(kb >= w_full_lo && kb + BKV <= w_full_hi);

        f32x16 sc[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
            for (int i = 0; i < 16; ++i) sc[j][i] = 0.0f;
            const int r = 32 * j + l32;
#pragma unroll
            for (int s2 = 0; s2 < QCH / 2; ++s2)
                mfma_chunk<T>(sc[j], lds_chunk(&sK[stg][32 * j][0], kofs[s2]), qf[s2]);
        }
        float mx = -INFINITY;
        if (need_mask) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = kb + 32 * j + key_perm(acc_row(i, g));
                    if (key < lo || key >= hi) sc[j][i] = -INFINITY;
                }
        }
        // Each query's scores sit in a lane pair (l, l ^ 32).  The pair's
        // maximum is needed only when the running max moves, which happens
        // iff either lane's own maximum exceeds m_run + kRescale: the lane
        // maxima decide that without the cross-lane exchange, and the pair
        // maximum is taken only on the (rare) rescaling tiles.
        {
            float m0 = sc[0][0], m1 = sc[1][0];
#pragma unroll
            for (int i = 1; i < 16; ++i) {
                m0 = fmaxf(m0, sc[0][i]);
                m1 = fmaxf(m1, sc[1][i]);
            }
            mx = fmaxf(m0, m1) * scale_log2;
        }
        if (__ballot(mx > m_run + kRescale)) {
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const bool grow = mx > m_run + kRescale;
            // lanes that do not grow keep their state: a lane whose keys in
            // this half of a split tile are all masked still has m_run = -inf,
            // and exp2(-inf - -inf) would be NaN
            const float m_new = grow ? mx : m_run;
            const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
            m_run = m_new;
            l_run *= alpha;
            if constexpr (kMfmaSum) {
#pragma unroll
                for (int i = 0; i < 16; ++i) lsum[i] *= alpha;
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
        }
        const float neg_m = m_run == -INFINITY ? 0.0f : -m_run;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                // accumulator slots 8st .. 8st+7 of lane group g are keys
                // 32j + 16st + 8g + (0..7)
                Chunk pb;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[j][8 * st + 2 * e], scale_log2, neg_m));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[j][8 * st + 2 * e + 1], scale_log2, neg_m));
                    pb.w[e] = pack2<T>(p0, p1);
                    if constexpr (!kMfmaSum) l_run = sum2<T>(pb.w[e], l_run); // the rounded weights
                }
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    mfma_chunk<T>(o[db], lds_chunk(&sV[stg][32 * db][0], vofs[2 * j + st]), pb);
                if constexpr (kMfmaSum) mfma_chunk<T>(lsum, ones, pb);
            }
        }
    };
    static_assert(STAGES == 3 || STAGES == 4, "one copy of the tile step per ring stage");
    for (int t = 0; t < ntiles; t += STAGES) {
        tile_step(std::integral_constant<int, 0>{}, t);
        if (t + 1 >= ntiles) break;
        tile_step(std::integral_constant<int, 1>{}, t + 1);
        if (t + 2 >= ntiles) break;
        tile_step(std::integral_constant<int, 2>{}, t + 2);
        if constexpr (STAGES == 4) {
            if (t + 3 >= ntiles) break;
            tile_step(std::integral_constant<int, 3 % STAGES>{}, t + 3);
        }
    }

    const float l_tot = kMfmaSum ? lsum[0] : l_run + __shfl_xor(l_run, 32, 64);
    if (piece) {
        // half of the keys: the unnormalised partial, [HD] o then (max, sum)
        if (qrow < N) {
            const int64_t prow = ((int64_t)bh * order.nslots + (qt - order.qs)) * BQL + (qrow - q0);
            float *dst = part + (prow * 2 + piece - 1) * (HD + 4);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    *reinterpret_cast<float4 *>(dst + db * 32 + acc_row(4 * u, g)) =
                        make_float4(o[db][4 * u], o[db][4 * u + 1], o[db][4 * u + 2], o[db][4 * u + 3]);
            if (g == 0) *reinterpret_cast<float2 *>(dst + HD) = make_float2(m_run, l_tot);
        }
        return;
    }
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    if (qrow < N) {
        T *orow = O + ((int64_t)b * N + qrow) * D + head * HD;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                T *dst = orow + db * 32 + acc_row(4 * u, g);
                *reinterpret_cast<uint2 *>(dst) = make_uint2(pack2<T>(o[db][4 * u] * inv, o[db][4 * u + 1] * inv),
                                                             pack2<T>(o[db][4 * u + 2] * inv, o[db][4 * u + 3] * inv));
            }
    }
}

// The fp32 and row-split calls run the prefix rows as a kernel of their own:
// grid (row groups of every (item, head), runs).
template <typename T, int HD, int QR>
__global__ __launch_bounds__(kPrefixThreads) void prefix_partial_kernel(const T *__restrict__ Q,
                                                                        const T *__restrict__ K,
                                                                        const T *__restrict__ Vt, int N, int ldv,
                                                                        int p, float scale_log2,
                                                                        float *__restrict__ part) {
    __shared__ float smem[prefix_smem_floats<HD, QR>()];
    const int gpb = (p + QR - 1) / QR;       // row groups per (item, head)
    const int bh = blockIdx.x / gpb, pq0 = (blockIdx.x - bh * gpb) * QR, nq = min(QR, p - pq0);
    prefix_run<T, HD, QR>(Q, K, Vt, N, ldv, p, scale_log2, part, bh, pq0, nq, blockIdx.y, gridDim.y, smem);
}

// Merge of the runs of one row: 256 threads, a group of HD threads per share
// of the runs (each thread one output dim), the shares added in a fixed order
// at the end; loads of different runs are independent, so a thread keeps
// several in flight.
constexpr int kMergeThreads = 256;

template <typename T, int HD>
__device__ __forceinline__ void prefix_merge_row(const float *__restrict__ part, int runs, int N, int H, int p,
                                                 int row, T *__restrict__ O) {
    constexpr int RG = kMergeThreads / HD;  // run groups
    constexpr int NW = kMergeThreads / 64;
    __shared__ float sacc[RG][HD];
    __shared__ float sl[RG];
    __shared__ float smax[NW];
    const int bh = row / p, pq = row - bh * p;
    const int b = bh / H, head = bh - b * H;
    const float *pr = part + (int64_t)row * runs * (HD + 2);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float mx = -INFINITY;
    for (int r = tid; r < runs; r += kMergeThreads) mx = fmaxf(mx, pr[(int64_t)r * (HD + 2)]);
    mx = wave_max(mx);
    if (lane == 0) smax[wave] = mx;
    __syncthreads();
    float M = smax[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, smax[w]);
    const int dd = tid % HD, rg = tid / HD;
    float L = 0.0f, acc = 0.0f;
#pragma unroll 4
    for (int r = rg; r < runs; r += RG) {
        const float *q = pr + (int64_t)r * (HD + 2);
        const float f = __builtin_amdgcn_exp2f(q[0] - M);
        L = fmaf(q[1], f, L);
        acc = fmaf(q[2 + dd], f, acc);
    }
    sacc[rg][dd] = acc;
    if (dd == 0) sl[rg] = L;
    __syncthreads();
    if (rg == 0) {
        float a = 0.0f, l = 0.0f;
#pragma unroll
        for (int g2 = 0; g2 < RG; ++g2) {
            a += sacc[g2][dd];
            l += sl[g2];
        }
        O[((int64_t)b * N + pq) * H * HD + head * HD + dd] = from_f32<T>(l > 0.0f ? a / l : 0.0f);
    }
}

template <typename T, int HD>
__global__ __launch_bounds__(kMergeThreads) void prefix_merge_kernel(const float *__restrict__ part, int runs, int N,
                                                                      int H, int p, T *__restrict__ O) {
    prefix_merge_row<T, HD>(part, runs, N, H, p, (int)blockIdx.x, O);
}

// Combines the two halves of a split query tile (TileOrder): with the running
// maxima m0, m1 (log2 units) and M = max(m0, m1), o = (o0 2^(m0-M) + o1
// 2^(m1-M)) / (l0 2^(m0-M) + l1 2^(m1-M)).  One thread per 4 output dims of
// a row.
template <typename T, int HD>
__device__ __forceinline__ void split_merge_quad(const float *__restrict__ part, int64_t idx, int64_t n, int N,
                                                 int H, int q_begin, int qs, int nslots, int bq,
                                                 T *__restrict__ O) {
    constexpr int G = HD / 4, PS = HD + 4;
    if (idx >= n) return;
    const int64_t row = idx / G;
    const int d = (int)(idx - row * G) * 4;
    const int local = (int)(row % bq);
    const int64_t rest = row / bq;
    const int slot = (int)(rest % nslots), bh = (int)(rest / nslots);
    const int q = q_begin + (qs + slot) * bq + local;
    if (q >= N) return;
    const float *p0 = part + row * 2 * PS, *p1 = p0 + PS;
    const float2 ml0 = *reinterpret_cast<const float2 *>(p0 + HD), ml1 = *reinterpret_cast<const float2 *>(p1 + HD);
    const float M = fmaxf(ml0.x, ml1.x);
    // a half in which this row sees no key (max -inf) is dropped by a select,
    // never multiplied by 0 (its partial is not read at all)
    const bool h0 = ml0.x != -INFINITY, h1 = ml1.x != -INFINITY;
    const float f0 = h0 ? __builtin_amdgcn_exp2f(ml0.x - M) : 0.0f;
    const float f1 = h1 ? __builtin_amdgcn_exp2f(ml1.x - M) : 0.0f;
    const float L = (h0 ? ml0.y * f0 : 0.0f) + (h1 ? ml1.y * f1 : 0.0f);
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f), c = a;
    if (h0) a = *reinterpret_cast<const float4 *>(p0 + d);
    if (h1) c = *reinterpret_cast<const float4 *>(p1 + d);
    const int b = bh / H, head = bh - b * H;
    T *dst = O + ((int64_t)b * N + q) * H * HD + head * HD + d;
    *reinterpret_cast<uint2 *>(dst) = make_uint2(pack2<T>(fmaf(a.x, f0, c.x * f1) * inv, fmaf(a.y, f0, c.y * f1) * inv),
                                                 pack2<T>(fmaf(a.z, f0, c.z * f1) * inv, fmaf(a.w, f0, c.w * f1) * inv));
}

// Both merges of a 16-bit call in one launch of kMergeThreads-thread
// workgroups: the first sblocks combine the split halves (one thread per 4
// output dims of a row), the rest merge one prefix row each.
template <typename T, int HD>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const float *__restrict__ part, int64_t n, int sblocks,
                                                              int N, int H, int q_begin, int qs, int nslots, int bq,
                                                              const float *__restrict__ pre_part, int runs,
                                                              T *__restrict__ O) {
    if ((int)blockIdx.x < sblocks)
        split_merge_quad<T, HD>(part, (int64_t)blockIdx.x * kMergeThreads + threadIdx.x, n, N, H, q_begin, qs,
                                nslots, bq, O);
    else
        prefix_merge_row<T, HD>(pre_part, runs, N, H, q_begin, (int)blockIdx.x - sblocks, O);
}

// the first query row the tiled kernels cover: the prefix rows go to
// prefix_attention_kernel (all of them: a model has at most a few)
inline int query_begin(int N, int p) { return p < N ? p : 0; }

// When the query tiles make fewer than kRowSplitTiles workgroups (a single
// small image: 257 tokens and 3 heads make 6), most CUs would idle while each
// tile walks every key; with full attention all rows then take the row
// kernels above instead (a workgroup per row and run of keys, then the merge).
constexpr int kRowSplitTiles = 16;
inline bool row_split(int B, int N, int H, int qb) { return (int64_t)B * H * cdiv(N - qb, BQ) < kRowSplitTiles; }

// Key tiles (of BKV) a query tile of bq rows starting at q0 walks.
inline int tile_key_tiles(int q0, int bq, int N, int causal, int p, int S) {
    int lo, hi, tmp;
    key_interval(q0, N, causal, p, S, lo, tmp);
    key_interval(q0 + bq - 1 < N - 1 ? q0 + bq - 1 : N - 1, N, causal, p, S, tmp, hi);
    if (q0 < p) hi = N;
    return (int)(cdiv(hi, BKV) - lo / BKV);
}

// Workgroups of the direct-to-LDS kernel resident at once: 256 CUs, three
// per CU at hd 64 (48 KB of LDS, 156 VGPRs) and at hd 32 (32 KB, 130 VGPRs).
// A constant, so that the scratch size a call is planned with never depends
// on the device it is asked on.
constexpr int kLdsSlots = 256 * 3;

// The TileOrder of a 16-bit attention call (bq queries per tile); returns
// false (ord.n = 0) when no tile is split.  Two cases split tiles:
//  - block-causal, grid of at most kSplitMaxWorkgroups: the late tiles
//    (above a third of the largest key count) run as two halves each;
//  - tiles of equal cost whose grid exceeds the resident slots and leaves
//    its last round less than half full (the 18432-token clip: 3168
//    workgroups on 768 slots, a last round of 96): the last k tiles of every
//    (item, head) run as halves, k the fewest that move every whole tile
//    into the full rounds, so the last round holds half tiles only.
inline bool plan_tile_order(int B, int N, int H, int causal, int p, int S, int bq, TileOrder &ord) {
    ord.n = 0;
    ord.qs = ord.nslots = 0;
    const int qb = query_begin(N, p), T = (int)cdiv(N - qb, bq);
    const int64_t tiles = (int64_t)B * H * T;
    int cnt[kMaxJobs];
    if (T < 4 || T > kMaxJobs) return false;
    int maxn = 0, minn = 1 << 30;
    for (int qt = 0; qt < T; ++qt) {
        cnt[qt] = tile_key_tiles(qb + qt * bq, bq, N, causal, p, S);
        maxn = cnt[qt] > maxn ? cnt[qt] : maxn;
        minn = cnt[qt] < minn ? cnt[qt] : minn;
    }
    int qs = T; // split: the tiles qs .. T-1
    if (causal) {
        if (tiles > kSplitMaxWorkgroups) return false;
        if (maxn < 2 * minn) return false; // tiles of alike cost (a single frame): nothing to balance
        // the run of last tiles above the threshold (block-causal counts never fall)
        while (qs > 0 && cnt[qs - 1] >= kSplitMinKeyTiles && 3 * cnt[qs - 1] > maxn) --qs;
    } else {
        const int64_t rem = tiles % kLdsSlots;
        if (tiles <= kLdsSlots || rem == 0 || 2 * rem >= kLdsSlots || minn < kSplitMinKeyTiles) return false;
        qs = T - (int)cdiv(rem, (int64_t)B * H);
    }
    if (qs <= 0 || qs == T || T + (T - qs) > kMaxJobs) return false;
    // jobs with their key-tile counts, sorted largest first (ties: later tile first)
    int njob = 0, size[kMaxJobs];
    for (int qt = T - 1; qt >= 0; --qt) {
        if (qt >= qs) {
            size[njob] = cnt[qt] / 2;
            ord.job[njob++] = (uint16_t)(qt | (1 << 14));
            size[njob] = cnt[qt] - cnt[qt] / 2;
            ord.job[njob++] = (uint16_t)(qt | (2 << 14));
        } else {
            size[njob] = cnt[qt];
            ord.job[njob++] = (uint16_t)qt;
        }
    }
    for (int i = 1; i < njob; ++i) { // insertion sort, stable
        const int sz = size[i];
        const uint16_t jb = ord.job[i];
        int k = i - 1;
        while (k >= 0 && size[k] < sz) {
            size[k + 1] = size[k];
            ord.job[k + 1] = ord.job[k];
            --k;
        }
        size[k + 1] = sz;
        ord.job[k + 1] = jb;
    }
    ord.n = njob;
    ord.qs = qs;
    ord.nslots = T - qs;
    return true;
}

// fp32 scratch layout of a 16-bit attention call: the prefix rows' partials,
// then (16-byte aligned) the split tiles' halves
inline int64_t prefix_scratch_floats(int B, int N, int H, int hd, int rows_per_bh) {
    return (int64_t)B * H * rows_per_bh * cdiv(N, kPrefixKeys) * (hd + 2);
}
inline int64_t split_scratch_floats(int B, int H, int hd, int bq, const TileOrder &ord) {
    return ord.n > 0 ? (int64_t)B * H * ord.nslots * bq * 2 * (hd + 4) : 0;
}

template <typename T, int HD, int QR = 1>
hipError_t launch_prefix(const void *Q, const void *K, const void *Vt, int B, int N, int H, int ldv, int qb,
                         float scale_log2, float *scratch, void *O, hipStream_t s) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || qb == 0) return e;
    if (!scratch) return hipErrorInvalidValue;
    const int runs = (int)cdiv(N, kPrefixKeys), rows = B * H * qb;
    const int groups = B * H * (int)cdiv(qb, QR);
    hipLaunchKernelGGL((prefix_partial_kernel<T, HD, QR>), dim3((unsigned)groups, (unsigned)runs),
                       dim3(kPrefixThreads), 0, s, reinterpret_cast<const T *>(Q), reinterpret_cast<const T *>(K),
                       reinterpret_cast<const T *>(Vt), N, ldv, qb, scale_log2, scratch);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((prefix_merge_kernel<T, HD>), dim3((unsigned)rows), dim3(kMergeThreads), 0, s, scratch, runs,
                       N, H, qb, reinterpret_cast<T *>(O));
    return hipGetLastError();
}

// 16-bit types: the direct-to-LDS kernel; fp32: the register-staged one
template <typename T, int HD>
hipError_t launch_t(const void *Q, const void *K, const void *Vt, int B, int N, int H, int ldv, int causal, int p,
                    int S, float *scratch, void *O, hipStream_t s) {
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)HD);
    // hd 32 tiles are too small to split their loads over more than 4 waves
    constexpr int NWV = HD == 64 ? kLdsWaves : 4;
    constexpr int BQL = 32 * NWV;
    const int qb = query_begin(N, p);
    const int ntq = (int)cdiv(N - qb, BQL);
    TileOrder ord;
    plan_tile_order(B, N, H, causal, p, S, BQL, ord);
    float *part = nullptr;
    if (ord.n > 0 || qb > 0) {
        if (!scratch) return hipErrorInvalidValue;
        part = scratch + cdiv(prefix_scratch_floats(B, N, H, HD, qb), 4) * 4;
    }
    // grid y: the query-tile jobs, then (prefix rows x runs of keys) prefix jobs
    const int jobs = ord.n > 0 ? ord.n : ntq, runs = (int)cdiv(N, kPrefixKeys);
    dim3 grid((unsigned)(B * H), (unsigned)(jobs + qb * runs));
    // measured at hd 64: the inline-assembly tile loads pay from about 4096
    // keys on (a 4097-token clip 0.4 % faster per encode, an 18432-token one
    // 3.5-6 %) and cost 1 % per encode at 2048 keys; at hd 32 they pay at
    // 2048 keys already
    if (N >= kDeepKeys<HD>)
        hipLaunchKernelGGL((attention_lds_kernel<T, HD, kStages<HD>, NWV, true>), grid, dim3(64 * NWV), 0, s,
                           reinterpret_cast<const T *>(Q), reinterpret_cast<const T *>(K),
                           reinterpret_cast<const T *>(Vt), N, H, ldv, causal, p, S, qb, scale_log2, ord, part, jobs,
                           scratch, reinterpret_cast<T *>(O));
    else
        hipLaunchKernelGGL((attention_lds_kernel<T, HD, kStages<HD>, NWV, false>), grid, dim3(64 * NWV), 0, s,
                           reinterpret_cast<const T *>(Q), reinterpret_cast<const T *>(K),
                           reinterpret_cast<const T *>(Vt), N, H, ldv, causal, p, S, qb, scale_log2, ord, part, jobs,
                           scratch, reinterpret_cast<T *>(O));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = ord.n > 0 ? (int64_t)B * H * ord.nslots * BQL * (HD / 4) : 0;
    const int sblocks = (int)cdiv(n, kMergeThreads), prows = B * H * qb;
    if (sblocks + prows > 0)
        hipLaunchKernelGGL((merge_kernel<T, HD>), dim3((unsigned)(sblocks + prows)), dim3(kMergeThreads), 0, s, part,
                           n, sblocks, N, H, qb, ord.qs, ord.nslots, BQL, scratch, runs, reinterpret_cast<T *>(O));
    return hipGetLastError();
}

template <>
hipError_t launch_t<float, 64>(const void *Q, const void *K, const void *Vt, int B, int N, int H, int ldv, int causal,
                               int p, int S, float *scratch, void *O, hipStream_t s) {
    const int qb = query_begin(N, p);
    const float scale_log2 = 1.4426950408889634f / 8.0f;
    if (!causal && row_split(B, N, H, qb))
        return launch_prefix<float, 64, 4>(Q, K, Vt, B, N, H, ldv, N, scale_log2, scratch, O, s);
    dim3 grid((unsigned)(B * H), (unsigned)cdiv(N - qb, BQ));
    hipLaunchKernelGGL((attention_kernel<float, 64>), grid, dim3(kThreads), 0, s, reinterpret_cast<const float *>(Q),
                       reinterpret_cast<const float *>(K), reinterpret_cast<const float *>(Vt), N, H, ldv, causal, p,
                       S, qb, scale_log2, reinterpret_cast<float *>(O));
    return launch_prefix<float, 64>(Q, K, Vt, B, N, H, ldv, qb, scale_log2, scratch, O, s);
}

template <>
hipError_t launch_t<float, 32>(const void *Q, const void *K, const void *Vt, int B, int N, int H, int ldv, int causal,
                               int p, int S, float *scratch, void *O, hipStream_t s) {
    const int qb = query_begin(N, p);
    const float scale_log2 = 1.4426950408889634f / sqrtf(32.0f);
    if (!causal && row_split(B, N, H, qb))
        return launch_prefix<float, 32, 4>(Q, K, Vt, B, N, H, ldv, N, scale_log2, scratch, O, s);
    dim3 grid((unsigned)(B * H), (unsigned)cdiv(N - qb, BQ));
    hipLaunchKernelGGL((attention_kernel<float, 32>), grid, dim3(kThreads), 0, s, reinterpret_cast<const float *>(Q),
                       reinterpret_cast<const float *>(K), reinterpret_cast<const float *>(Vt), N, H, ldv, causal, p,
                       S, qb, scale_log2, reinterpret_cast<float *>(O));
    return launch_prefix<float, 32>(Q, K, Vt, B, N, H, ldv, qb, scale_log2, scratch, O, s);
}

template <typename T>
hipError_t launch_hd(int head_dim, const void *Q, const void *K, const void *Vt, int B, int N, int H, int ldv,
                     int causal, int p, int S, float *scratch, void *O, hipStream_t s) {
    if (head_dim == 64) return launch_t<T, 64>(Q, K, Vt, B, N, H, ldv, causal, p, S, scratch, O, s);
    if (head_dim == 32) return launch_t<T, 32>(Q, K, Vt, B, N, H, ldv, causal, p, S, scratch, O, s);
    return hipErrorInvalidValue;
}

} // namespace

int64_t attention_scratch_floats(int dtype, int B, int N, int H, int head_dim, int attn_mode, int n_prefix,
                                 int tokens_per_frame) {
    if (B <= 0 || N <= 0) return 0;
    const int causal = attn_mode == 1;
    const int S = tokens_per_frame > 0 ? tokens_per_frame : 1;
    const int qb = query_begin(N, n_prefix);
    if (dtype == DT_F32)
        return prefix_scratch_floats(B, N, H, head_dim, !causal && row_split(B, N, H, qb) ? N : qb);
    TileOrder ord;
    plan_tile_order(B, N, H, causal, n_prefix, S, 32 * (head_dim == 64 ? kLdsWaves : 4), ord);
    const int64_t pre = prefix_scratch_floats(B, N, H, head_dim, qb);
    return ord.n > 0 ? cdiv(pre, 4) * 4 + split_scratch_floats(B, H, head_dim, 32 * (head_dim == 64 ? kLdsWaves : 4), ord)
                     : pre;
}

hipError_t launch_attention(int dtype, const void *Q, const void *K, const void *Vt, int B, int N, int H,
                            int head_dim, int ldv, int attn_mode, int n_prefix, int tokens_per_frame,
                            float *scratch, void *O, hipStream_t s) {
    if (B <= 0 || N <= 0) return hipSuccess;
    const int causal = attn_mode == 1;
    const int S = tokens_per_frame > 0 ? tokens_per_frame : 1;
    switch (dtype) {
    case DT_F32: return launch_hd<float>(head_dim, Q, K, Vt, B, N, H, ldv, causal, n_prefix, S, scratch, O, s);
    case DT_BF16: return launch_hd<bf16_t>(head_dim, Q, K, Vt, B, N, H, ldv, causal, n_prefix, S, scratch, O, s);
    case DT_F16: return launch_hd<f16_t>(head_dim, Q, K, Vt, B, N, H, ldv, causal, n_prefix, S, scratch, O, s);
    }
    return hipErrorInvalidValue;
}

} // namespace vitenc
