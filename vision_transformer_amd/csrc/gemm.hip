// C[M, N] = A[M, K] * W[N, K]^T + bias, with the encoder's fused epilogues.
//
// Both operands are K-contiguous (PyTorch row-major activations and weights),
// which is the layout MFMA operands want: each lane feeds 16 contiguous bytes
// of one row.  A 256-thread workgroup computes a BM x BN tile as a 2 x 2 grid
// of waves; each wave owns a (BM/2) x (BN/2) block of 32x32 MFMA tiles with
// fp32 accumulators.  K advances 128 bytes per step (64 bf16/f16 or 32 fp32
// elements); the A and W slabs of step k+2 are fetched into registers while
// step k is multiplied out of LDS (two LDS buffers, two register staging
// sets, one barrier per step).  LDS rows are 8 chunks of 16 bytes with the
// chunk index XOR-swizzled by the row, so the 32 rows a wave reads in one
// MFMA operand fetch fall on distinct banks (swz8).  The operand fragments of
// sub-step s+1 are read from LDS while the MFMAs of sub-step s run.
//
// Epilogues (jepa.cpp "Architecture", "The shared ViT graph"; "GGUF schema
// (v1)", "Encoder tensors"):
//   STORE  out = v                       (T)
//   GELU   out = GELU_erf(v)             (T)   ffn_up
//   RESID  Z  += ls * v                  (fp32 residual) attn_out, ffn_down
//   PATCH  Z[token row] = v + pos + mod  (fp32 residual) patch embedding
//   QKV    split [q; k; v] into heads, 3-D RoPE on q and k of patch tokens
//          ("Architecture", "3-D RoPE"), V written transposed per head
// where v = accumulator + bias.
#include "common.h"
#include "launch.h"

namespace vitenc {

namespace {

constexpr int kThreads = 256;

struct RowInfo {
    int out_row; // PATCH: token row in Z; QKV: item index b
    int tok;     // QKV: token index inside the item
    int pos;     // PATCH: pos-table row; QKV: packed (t,h,w) or -1 for prefix tokens
    int pad;
};

template <typename T, bool ALIGNED>
__device__ __forceinline__ Chunk load_tile_chunk(const T *__restrict__ base, int64_t ld, int row, int rows,
                                                 int k, int K) {
    constexpr int KPC = Elem<T>::kPerChunk;
    if (row >= rows) return zero_chunk();
    const T *p = base + (int64_t)row * ld + k;
    if constexpr (ALIGNED) {
        if (k < K) return load_chunk(p);
        return zero_chunk();
    } else {
        Chunk c = zero_chunk();
        if constexpr (KPC == 4) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (k + e < K) c.w[e] = __builtin_bit_cast(uint32_t, p[e]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (k + e < K) c.w[e >> 1] |= bits16(p[e]) << (16 * (e & 1));
        }
        return c;
    }
}

__device__ __forceinline__ float gelu_erf(float x) {
    return 0.5f * x * (1.0f + erff(x * 0.70710678118654752440f));
}

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup b runs on
// XCD b % 8).  Remap so that each XCD receives a contiguous run of tiles; with
// the N tiles of one M block adjacent, an XCD's L2 serves the A row panel of
// its tiles instead of every XCD fetching every panel.
__device__ __forceinline__ int xcd_tile(int b, int nb) {
    constexpr int kXcd = 8;
    const int x = b % kXcd, q = nb / kXcd, r = nb % kXcd;
    return x * q + min(x, r) + b / kXcd;
}

// FAST: 16-byte aligned rows and K a multiple of the K step, so every load is
// a full chunk; rows past M / N are clamped to the last row (they only feed
// accumulator rows / columns that are never stored).  Otherwise loads are
// element-wise with zero fill past K and past the last row.
template <typename T, int BM, int BN, int EPI, bool FAST>
__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(const T *__restrict__ A, int64_t lda,
                                                           const T *__restrict__ W, int64_t ldw, int M,
                                                           int N, int K, int tiles_n, EpiArgs ep) {
    constexpr int KPC = Elem<T>::kPerChunk;
    constexpr int BK = 8 * KPC;
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int FM = WM / 32, FN = WN / 32;
    constexpr int A_PER = BM * 8 / kThreads, B_PER = BN * 8 / kThreads;
    static_assert(FM >= 1 && FN >= 1 && A_PER >= 1 && B_PER >= 1, "tile too small");

    __shared__ Chunk sA[2][BM][8];
    __shared__ Chunk sB[2][BN][8];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int g = lane >> 5, l32 = lane & 31;
    const int tile = xcd_tile(blockIdx.x, gridDim.x);
    const int tm = tile / tiles_n, tn = tile - tm * tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;
    const int lc = tid & 7, lr = tid >> 3;

    // per-thread row pointers of the chunks this thread stages
    const T *pa[A_PER];
    const T *pb[B_PER];
#pragma unroll
    for (int i = 0; i < A_PER; ++i) pa[i] = A + (int64_t)min(m0 + lr + 32 * i, M - 1) * lda + lc * KPC;
#pragma unroll
    for (int i = 0; i < B_PER; ++i) pb[i] = W + (int64_t)min(n0 + lr + 32 * i, N - 1) * ldw + lc * KPC;

    auto gload = [&](Chunk *ra, Chunk *rb, int k0) {
        if constexpr (FAST) {
#pragma unroll
            for (int i = 0; i < A_PER; ++i) ra[i] = load_chunk(pa[i] + k0);
#pragma unroll
            for (int i = 0; i < B_PER; ++i) rb[i] = load_chunk(pb[i] + k0);
        } else {
#pragma unroll
            for (int i = 0; i < A_PER; ++i)
                ra[i] = load_tile_chunk<T, false>(A, lda, m0 + lr + 32 * i, M, k0 + lc * KPC, K);
#pragma unroll
            for (int i = 0; i < B_PER; ++i)
                rb[i] = load_tile_chunk<T, false>(W, ldw, n0 + lr + 32 * i, N, k0 + lc * KPC, K);
        }
    };
    auto sstore = [&](const Chunk *ra, const Chunk *rb, int buf) {
#pragma unroll
        for (int i = 0; i < A_PER; ++i) {
            const int r = lr + 32 * i;
            sA[buf][r][lc ^ swz8(r)] = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_PER; ++i) {
            const int r = lr + 32 * i;
            sB[buf][r][lc ^ swz8(r)] = rb[i];
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[fm][fn][i] = 0.0f;

    auto frags = [&](Chunk *a, Chunk *b, int buf, int s) {
        const int cc = 2 * s + g;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int r = wm * WM + fm * 32 + l32;
            a[fm] = sA[buf][r][cc ^ swz8(r)];
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int r = wn * WN + fn * 32 + l32;
            b[fn] = sB[buf][r][cc ^ swz8(r)];
        }
    };
    auto compute = [&](int buf) {
        Chunk a0[FM], b0[FN], a1[FM], b1[FN];
        frags(a0, b0, buf, 0);
#pragma unroll
        for (int s = 0; s < 4; s += 2) {
            frags(a1, b1, buf, s + 1);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) mfma_chunk<T>(acc[fm][fn], a0[fm], b0[fn]);
            if (s + 2 < 4) frags(a0, b0, buf, s + 2);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) mfma_chunk<T>(acc[fm][fn], a1[fm], b1[fn]);
        }
    };

    // Two LDS buffers and two register staging sets: the slab of step k+2 is
    // fetched while step k is multiplied, so each load has two compute phases
    // to land before it is written to LDS.
    const int nk = (int)cdiv(K, BK);
    Chunk ra0[A_PER], rb0[B_PER], ra1[A_PER], rb1[B_PER];
    gload(ra0, rb0, 0);
    if (nk > 1) gload(ra1, rb1, BK);
    sstore(ra0, rb0, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
        if (kt + 2 < nk) gload(ra0, rb0, (kt + 2) * BK);
        compute(0);
        if (kt + 1 < nk) sstore(ra1, rb1, 1);
        __syncthreads();
        if (kt + 1 >= nk) break;
        if (kt + 3 < nk) gload(ra1, rb1, (kt + 3) * BK);
        compute(1);
        if (kt + 2 < nk) sstore(ra0, rb0, 0);
        __syncthreads();
    }

    // ---------------------------------------------------------------- epilogue
    RowInfo *ri = reinterpret_cast<RowInfo *>(&sA[0][0][0]);
    if constexpr (EPI == EPI_PATCH || EPI == EPI_QKV) {
        if (tid < BM) {
            const int row = m0 + tid;
            RowInfo info{0, 0, -1, 0};
            if (row < M) {
                if constexpr (EPI == EPI_PATCH) {
                    const int b = row / ep.Np, n = row - b * ep.Np;
                    info.out_row = b * ep.Ntok + ep.prefix + n;
                    info.pos = ep.prefix + n;
                } else {
                    const int b = row / ep.Ntok, tok = row - b * ep.Ntok;
                    info.out_row = b;
                    info.tok = tok;
                    info.pos = (ep.rope && tok >= ep.prefix) ? ep.tok_pos[tok - ep.prefix] : -1;
                }
            }
            ri[tid] = info;
        }
        __syncthreads();
    }

#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
        const int col = n0 + wn * WN + fn * 32 + l32;
        const bool col_ok = col < N;
        const float bias = (col_ok && ep.bias) ? ep.bias[col] : 0.0f;
        float lsv = 1.0f;
        if constexpr (EPI == EPI_RESID) {
            if (col_ok && ep.ls) lsv = ep.ls[col];
        }
        // QKV column geometry
        int which = 0, head = 0, dd = 0, axis = 0, jrot = 0, tab_base = 0;
        bool rot = false;
        if constexpr (EPI == EPI_QKV) {
            which = col / ep.D;
            const int within = col - which * ep.D;
            head = within / ep.head_dim;
            dd = within - head * ep.head_dim;
            rot = ep.rope && which < 2 && dd < 3 * ep.d_rot;
            if (rot) {
                axis = dd / ep.d_rot;
                jrot = dd - axis * ep.d_rot;
                tab_base = (axis == 0 ? 0 : axis == 1 ? ep.gt : ep.gt + ep.gh) * ep.d_rot;
            }
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = wm * WM + fm * 32 + acc_row(i, g);
                const int row = m0 + r;
                float v = acc[fm][fn][i] + bias;
                if constexpr (EPI == EPI_QKV) {
                    const float partner = __shfl_xor(v, 1, 64);
                    if (row < M && col_ok) {
                        const RowInfo info = ri[r];
                        if (rot && info.pos >= 0) {
                            const int p = (info.pos >> (10 * axis)) & 1023;
                            const float2 cs =
                                reinterpret_cast<const float2 *>(ep.rope_tab)[tab_base + p * ep.d_rot + jrot];
                            v = v * cs.x + partner * cs.y;
                        }
                        const int H = ep.D / ep.head_dim;
                        const int64_t bh = (int64_t)info.out_row * H + head;
                        if (which < 2) {
                            T *dst = reinterpret_cast<T *>(which == 0 ? ep.Q : ep.K);
                            dst[(bh * ep.Ntok + info.tok) * ep.head_dim + dd] = from_f32<T>(v);
                        } else {
                            T *dst = reinterpret_cast<T *>(ep.Vt);
                            dst[(bh * ep.head_dim + dd) * ep.ldv + info.tok] = from_f32<T>(v);
                        }
                    }
                } else {
                    if (row < M && col_ok) {
                        if constexpr (EPI == EPI_STORE) {
                            reinterpret_cast<T *>(ep.out)[(int64_t)row * ep.ldo + col] = from_f32<T>(v);
                        } else if constexpr (EPI == EPI_GELU) {
                            reinterpret_cast<T *>(ep.out)[(int64_t)row * ep.ldo + col] = from_f32<T>(gelu_erf(v));
                        } else if constexpr (EPI == EPI_RESID) {
                            float *z = ep.Z + (int64_t)row * ep.ldz + col;
                            *z = *z + lsv * v;
                        } else if constexpr (EPI == EPI_PATCH) {
                            const RowInfo info = ri[r];
                            float x = v;
                            if (ep.pos) x += ep.pos[(int64_t)info.pos * ep.ldz + col];
                            if (ep.mod) x += ep.mod[col];
                            ep.Z[(int64_t)info.out_row * ep.ldz + col] = x;
                        }
                    }
                }
            }
        }
    }
}

template <typename T, int EPI, bool FAST>
hipError_t launch_t(const void *A, int64_t lda, const void *W, int64_t ldw, int M, int N, int K,
                    const EpiArgs &ep, hipStream_t s) {
    constexpr int BM = 128, BN = 128;
    const int tiles_n = (int)cdiv(N, BN), tiles_m = (int)cdiv(M, BM);
    hipLaunchKernelGGL((gemm_kernel<T, BM, BN, EPI, FAST>), dim3((unsigned)(tiles_m * tiles_n)), dim3(kThreads), 0,
                       s, reinterpret_cast<const T *>(A), lda, reinterpret_cast<const T *>(W), ldw, M, N, K, tiles_n,
                       ep);
    return hipGetLastError();
}

template <typename T, int EPI>
hipError_t launch_align(const void *A, int64_t lda, const void *W, int64_t ldw, int M, int N, int K,
                        const EpiArgs &ep, hipStream_t s) {
    constexpr int KPC = Elem<T>::kPerChunk;
    const bool fast = (K % (8 * KPC) == 0) && (lda % KPC == 0) && (ldw % KPC == 0) &&
                      ((uintptr_t)A % 16 == 0) && ((uintptr_t)W % 16 == 0);
    if (fast) return launch_t<T, EPI, true>(A, lda, W, ldw, M, N, K, ep, s);
    return launch_t<T, EPI, false>(A, lda, W, ldw, M, N, K, ep, s);
}

template <typename T>
hipError_t launch_epi(int epi, const void *A, int64_t lda, const void *W, int64_t ldw, int M, int N, int K,
                      const EpiArgs &ep, hipStream_t s) {
    switch (epi) {
    case EPI_STORE: return launch_align<T, EPI_STORE>(A, lda, W, ldw, M, N, K, ep, s);
    case EPI_GELU: return launch_align<T, EPI_GELU>(A, lda, W, ldw, M, N, K, ep, s);
    case EPI_RESID: return launch_align<T, EPI_RESID>(A, lda, W, ldw, M, N, K, ep, s);
    case EPI_PATCH: return launch_align<T, EPI_PATCH>(A, lda, W, ldw, M, N, K, ep, s);
    case EPI_QKV: return launch_align<T, EPI_QKV>(A, lda, W, ldw, M, N, K, ep, s);
    }
    return hipErrorInvalidValue;
}

} // namespace

hipError_t launch_gemm(int dtype, int epi, const void *A, int64_t lda, const void *W, int64_t ldw, int M, int N,
                       int K, const EpiArgs &ep, hipStream_t s) {
    if (M <= 0 || N <= 0 || K <= 0) return hipSuccess;
    switch (dtype) {
    case DT_F32: return launch_epi<float>(epi, A, lda, W, ldw, M, N, K, ep, s);
    case DT_BF16: return launch_epi<bf16_t>(epi, A, lda, W, ldw, M, N, K, ep, s);
    case DT_F16: return launch_epi<f16_t>(epi, A, lda, W, ldw, M, N, K, ep, s);
    }
    return hipErrorInvalidValue;
}

} // namespace vitenc
