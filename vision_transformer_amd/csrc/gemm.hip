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
#include <algorithm>
#include <climits>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace vitenc {

namespace {

constexpr int kThreads = 256;

struct RowInfo {
    int out_row;    // PATCH: token row in Z; QKV: item index b
    int tok;        // QKV: token index inside the item
    int pos;        // PATCH: pos-table row; QKV: 1 if the row is rotated (a patch token), else 0
    int base[3];    // QKV: first table entry of this row's position on axis t, h, w
    int64_t qk_off; // QKV: element offset of (b, head 0, tok, dim 0) in Q / K [B, H, N, hd]
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

// 8 consecutive outputs from fp32: one 16-byte store for 16-bit types, two for fp32
template <typename T> __device__ __forceinline__ void store_vec8(T *dst, const float (&v)[8]) {
    if constexpr (sizeof(T) == 4) {
        reinterpret_cast<float4 *>(dst)[0] = make_float4(v[0], v[1], v[2], v[3]);
        reinterpret_cast<float4 *>(dst)[1] = make_float4(v[4], v[5], v[6], v[7]);
    } else {
        Chunk c;
#pragma unroll
        for (int e = 0; e < 4; ++e) c.w[e] = pack2<T>(v[2 * e], v[2 * e + 1]);
        store_chunk(dst, c);
    }
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

// Row path of the epilogue: after staging, lane l of a wave owns the 8
// consecutive columns (l % CPR) * 8 .. + 7 of the wave's WN columns and, in
// each MI-row block, the rows p * RPP + l / CPR for p < NPASS.
template <int MI, int WN> struct RowPath {
    static constexpr int CPR = WN / 8;                  // 8-column groups per row
    static constexpr int RPP = 64 / CPR;                // rows per pass
    static constexpr int NPASS = (MI + RPP - 1) / RPP;  // passes per MI-row block
};

// What the epilogue of a lane reads besides the accumulators, requested at
// kernel start so that its latency hides under the main loop: the bias and
// layer scale of the lane's 8 columns; for the residual epilogue the fp32
// residual values the lane will update (NZ rows of 8 columns, when they fit
// in registers; wider tiles request each row block's values one block
// ahead instead); for QKV the packed (t, h, w) of tile row m0 + tid and this
// thread's share (NTAB pairs) of the RoPE cos / sin table.
template <int NZ, int NTAB> struct EpiPre {
    float bias8[8], ls8[8]; // 0 past N (ls8 is used only when there is a layer scale)
    float4 z[NZ > 0 ? NZ : 1][2];
    int pk;
    float2 tab[NTAB > 0 ? NTAB : 1];
    float vbias; // QKV: bias of the lane's column of the transposed V path
};

// the fast (vector) residual access of one lane-row: the 8 columns exist
// and the rows are 16-byte aligned
__device__ __forceinline__ bool z_vec(const EpiArgs &ep, int row, int M, bool col_full) {
    return row < M && col_full && (ep.ldz % 4) == 0;
}

// All loads here are range-checked buffer loads with no branch around them
// (see buf_rsrc): their results are consumed only in the epilogue.
template <int EPI, int NZ, int NTAB, int BM, int FM, int NT, int MI, int WN>
__device__ __forceinline__ EpiPre<NZ, NTAB> epi_prefetch(int m0, int n0, int woff_m, int woff_n, int M, int N,
                                                         const EpiArgs &ep) {
    using RP = RowPath<MI, WN>;
    EpiPre<NZ, NTAB> pre;
    const int tid = threadIdx.x, lane = tid & 63;
    const int col0 = n0 + woff_n + (lane % RP::CPR) * 8;
    const __amdgpu_buffer_rsrc_t rb = buf_rsrc(ep.bias, (uint32_t)N * 4u);
#pragma unroll
    for (int j = 0; j < 8; ++j) pre.bias8[j] = buf_f32(rb, (uint32_t)(col0 + j) * 4u);
    if constexpr (EPI == EPI_RESID) {
        const __amdgpu_buffer_rsrc_t rl = buf_rsrc(ep.ls, (uint32_t)N * 4u);
#pragma unroll
        for (int j = 0; j < 8; ++j) pre.ls8[j] = buf_f32(rl, (uint32_t)(col0 + j) * 4u);
        if constexpr (NZ > 0) {
            // rows of this wave's part of the tile, from its first row on
            const int64_t r0 = m0 + woff_m;
            const int64_t bytes = r0 < M && ep.splits == 1 ? (int64_t)(M - r0) * ep.ldz * 4 : 0;
            const __amdgpu_buffer_rsrc_t rz =
                buf_rsrc(ep.Z + r0 * ep.ldz, (uint32_t)(bytes < 0xFFFFFFF0ll ? bytes : 0xFFFFFFF0ll));
#pragma unroll
            for (int i = 0; i < NZ; ++i) {
                const int fm = i / RP::NPASS, p = i % RP::NPASS;
                const int r = fm * MI + p * RP::RPP + lane / RP::CPR;
                const uint32_t off = (uint32_t)(((int64_t)r * ep.ldz + col0) * 4);
                pre.z[i][0] = buf_f32x4(rz, off);
                pre.z[i][1] = buf_f32x4(rz, off + 16u);
            }
        }
    }
    if constexpr (EPI == EPI_QKV) {
        // the transposed V path: lane -> column woff_n + lane % WN
        pre.vbias = buf_f32(rb, (uint32_t)(n0 + woff_n + lane % WN) * 4u);
        // packed position of row m0 + tid (read only for rows that have one)
        const int row = m0 + tid;
        const int b = row / ep.Ntok, tok = row - b * ep.Ntok;
        const bool has = tid < BM && row < M && ep.rope && tok >= ep.prefix;
        const __amdgpu_buffer_rsrc_t rp = buf_rsrc(ep.rope ? ep.tok_pos : nullptr, 0xFFFFFFF0u);
        pre.pk = buf_i32(rp, has ? (uint32_t)(((int64_t)b * ep.tok_pos_stride + tok - ep.prefix) * 4) : 0u);
        if constexpr (NTAB > 0) {
            const bool fits = ep.rope && ep.rope_tab_pairs <= NTAB * NT;
            const __amdgpu_buffer_rsrc_t rt = buf_rsrc(ep.rope_tab, fits ? (uint32_t)ep.rope_tab_pairs * 8u : 0u);
#pragma unroll
            for (int i = 0; i < NTAB; ++i) pre.tab[i] = buf_f32x2(rt, (uint32_t)(tid + i * NT) * 8u);
        }
    }
    return pre;
}

// GELU of the epilogue
template <int EPI> __device__ __forceinline__ float epi_act(float v) {
    if constexpr (EPI == EPI_GELU) return gelu_erf(v);
    else return v;
}

// The residual rows the RESID epilogue updates when they were not prefetched
// at kernel start (NZ == 0): ZD row blocks of the wave's tile in flight, each
// lane holding its 8 columns of NPASS rows per block.  request(f) asks for
// row block f into slot f % ZD with branch-free range-checked loads (see
// buf_rsrc) from the wave's first row.
template <int EPI, int NZ, int FM, int MI, int WN> struct ZRows {
    using RP = RowPath<MI, WN>;
    static constexpr bool kOn = EPI == EPI_RESID && NZ == 0;
    static constexpr int NZB = kOn ? RP::NPASS : 1;
    static constexpr int ZD = FM < 2 ? FM : 2; // blocks in flight
    float4 q[ZD][NZB][2];
    __device__ __forceinline__ void request(int f, int m0, int woff_m, int n0, int woff_n, int M, const EpiArgs &ep,
                                            bool to_part) {
        if constexpr (kOn) {
            const int lane = threadIdx.x & 63;
            const int col0 = n0 + woff_n + (lane % RP::CPR) * 8;
            const int64_t zr0 = m0 + woff_m;
            const int64_t zbytes = !to_part && zr0 < M ? (int64_t)(M - zr0) * ep.ldz * 4 : 0;
            const __amdgpu_buffer_rsrc_t rzb =
                buf_rsrc(ep.Z + zr0 * ep.ldz, (uint32_t)(zbytes < 0xFFFFFFF0ll ? zbytes : 0xFFFFFFF0ll));
#pragma unroll
            for (int p = 0; p < RP::NPASS; ++p) {
                const int r = f * MI + p * RP::RPP + lane / RP::CPR;
                const uint32_t off = (uint32_t)(((int64_t)r * ep.ldz + col0) * 4);
                q[f % ZD][p][0] = buf_f32x4(rzb, off);
                q[f % ZD][p][1] = buf_f32x4(rzb, off + 16u);
            }
        }
    }
};

// Epilogue of one workgroup tile: v = accumulator + bias, then the EPI
// operation.  Each wave stages one MI-row block of its accumulators at a time
// through a private LDS area (MI x (WN + 4) fp32) and reads it back so that
// every lane owns 8 consecutive columns of one row: loads and stores of the
// outputs are then 16-byte, row-contiguous vectors instead of per-element
// accesses.  The V part of the QKV projection is read back transposed (8
// consecutive rows of one column) because V is stored transposed per head.
// Everything the epilogue reads from global memory besides the accumulators
// was requested at kernel start (epi_prefetch), except for the residual rows
// of tiles too wide to hold them in registers: those are requested one row
// block ahead.
// ri: LDS scratch for BM row descriptors, stage: this wave's staging area.
// Every thread of the workgroup must call this (it contains a barrier).
template <typename T, int BM, int FM, int FN, int EPI, int NT, int MI, int WN, bool SWAP, int NZ, int NTAB,
          typename AccT>
__device__ __forceinline__ void gemm_epilogue(AccT (&acc)[FM][FN], const EpiPre<NZ, NTAB> &pre, RowInfo *ri,
                                              float *stage, float2 *lds_tab, int lds_tab_cap, int m0, int n0,
                                              int woff_m, int woff_n, int M, int N, const EpiArgs &ep,
                                              float *part, ZRows<EPI, NZ, FM, MI, WN> &zr, bool z_requested) {
    using RP = RowPath<MI, WN>;
    constexpr int NV = MI == 32 ? 16 : 4; // accumulator values per lane per block
    constexpr int LD = WN + 4;            // staging row stride (floats), 16-byte aligned
    constexpr int CPR = RP::CPR, RPP = RP::RPP, NPASS = RP::NPASS;
    const int tid = threadIdx.x, lane = tid & 63;
    const int lcol = lane & (MI - 1);
    auto vrow = [&](int i) { return MI == 32 ? acc_row(i, lane >> 5) : 4 * (lane >> 4) + i; };

    if constexpr (EPI == EPI_QKV && MI == 32 && !SWAP) {
        // A tile of V columns only: the accumulators already hold, per lane,
        // one feature and runs of 4 consecutive tokens (slots 4q..4q+3 are rows
        // 8q + 4(l/32) + 0..3), which is V^T's layout: store them directly as
        // 8-byte runs, with no staging.  Needs token runs that never cross an
        // item (N % 4 == 0); the condition is uniform over the workgroup.
        if (n0 >= 2 * ep.D && (ep.Ntok & 3) == 0) {
            const int H = ep.D / ep.head_dim, g = lane >> 5;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int col = n0 + woff_n + fn * MI + lcol;
                if (col >= N) continue;
                const float bias = ep.bias ? ep.bias[col] : 0.0f;
                const int within = col - 2 * ep.D;
                const int head = within / ep.head_dim, dd = within - head * ep.head_dim;
                T *vcol = reinterpret_cast<T *>(ep.Vt) + (int64_t)head * ep.head_dim * ep.ldv + (int64_t)dd * ep.ldv;
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int row0 = m0 + woff_m + fm * MI + 8 * q + 4 * g;
                        if (row0 >= M) continue;
                        const int b = row0 / ep.Ntok, tok = row0 - b * ep.Ntok;
                        T *dst = vcol + (int64_t)b * H * ep.head_dim * ep.ldv + tok;
                        const float v0 = acc[fm][fn][4 * q] + bias, v1 = acc[fm][fn][4 * q + 1] + bias;
                        const float v2 = acc[fm][fn][4 * q + 2] + bias, v3 = acc[fm][fn][4 * q + 3] + bias;
                        if constexpr (sizeof(T) == 4) {
                            *reinterpret_cast<float4 *>(dst) = make_float4(v0, v1, v2, v3);
                        } else {
                            *reinterpret_cast<uint2 *>(dst) = make_uint2(pack2<T>(v0, v1), pack2<T>(v2, v3));
                        }
                    }
            }
            return;
        }
    }

    if constexpr (EPI == EPI_PATCH || EPI == EPI_QKV) {
        for (int t = tid; t < BM; t += NT) {
            const int row = m0 + t;
            RowInfo info{0, 0, 0, {0, 0, 0}, 0};
            if (row < M) {
                if constexpr (EPI == EPI_PATCH) {
                    if (ep.row_map) {
                        info.out_row = ep.row_map[row];
                        info.pos = 0;
                    } else {
                        const int b = row / ep.Np, n = row - b * ep.Np;
                        info.out_row = b * ep.Ntok + ep.prefix + n;
                        info.pos = ep.prefix + n;
                    }
                } else {
                    const int b = row / ep.Ntok, tok = row - b * ep.Ntok;
                    info.out_row = b;
                    info.tok = tok;
                    info.pos = 0;
                    info.qk_off = ((int64_t)b * (ep.D / ep.head_dim) * ep.Ntok + tok) * ep.head_dim;
                    if (ep.rope && tok >= ep.prefix) {
                        const int pk = pre.pk; // t < BM <= NT: this thread's own prefetched row
                        info.pos = 1;
                        info.base[0] = (pk & 1023) * ep.d_rot;
                        info.base[1] = (ep.gt + ((pk >> 10) & 1023)) * ep.d_rot;
                        info.base[2] = (ep.gt + ep.gh + ((pk >> 20) & 1023)) * ep.d_rot;
                    }
                }
            }
            ri[t] = info;
        }
    }
    // The RoPE table goes to LDS when it fits, followed by two identity pairs
    // (cos 1, sin 0) that the unrotated dims read, so that the rotation needs
    // no per-element branch.  Otherwise it is read from global memory.
    const float2 *tab = reinterpret_cast<const float2 *>(ep.rope_tab);
    const int id_pair = ep.rope_tab_pairs;
    const bool tab_lds = EPI == EPI_QKV && ep.rope && ep.rope_tab_pairs + 2 <= lds_tab_cap;
    if constexpr (EPI == EPI_QKV) {
        if (tab_lds) {
            if (NTAB > 0 && ep.rope_tab_pairs <= NTAB * NT) {
#pragma unroll
                for (int i = 0; i < (NTAB > 0 ? NTAB : 1); ++i)
                    if (tid + i * NT < ep.rope_tab_pairs) lds_tab[tid + i * NT] = pre.tab[i];
            } else {
                for (int t = tid; t < ep.rope_tab_pairs; t += NT) lds_tab[t] = tab[t];
            }
            if (tid < 2) lds_tab[id_pair + tid] = make_float2(1.0f, 0.0f);
        }
    }
    __syncthreads();

    // Row path: lane -> (row, 8-column group).  A lane's 8 columns are the
    // same for every row it handles, so everything that depends only on the
    // column (bias, layer scale, QKV head geometry, RoPE axis and table
    // column) is set up once here.
    const int c0 = (lane % CPR) * 8;
    const int col0 = n0 + woff_n + c0;
    const bool col_any = col0 < N;
    const bool col_full = col0 + 8 <= N;
    int which = 0, head = 0, dd0 = 0;
    int axis8[8], jr8[8];
    // LDS-table RoPE: a lane's 8 dims meet at most two axis segments (every
    // segment is at least 10 dims wide): selectors s_lo / s_hi of the row's
    // table base (0..2 = t, h, w; 3 = the identity pairs), dims j < jsplit use
    // s_lo, and off8[j] is the entry within the segment (0 for the identity).
    // Segments and 8-column groups start at even dims, so every aligned pair
    // (2u, 2u + 1) of a lane's dims reads two adjacent table entries with one
    // 16-byte LDS read.
    int s_lo = 3, s_hi = 3, jsplit = 8, off8[8];
    int64_t qk_col = 0;
    if constexpr (EPI == EPI_QKV) {
        which = col0 / ep.D;
        const int within = col0 - which * ep.D;
        head = within / ep.head_dim;
        dd0 = within - head * ep.head_dim;
        qk_col = (int64_t)head * ep.Ntok * ep.head_dim + dd0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int dd = dd0 + j;
            const int ax = dd >= 3 * ep.d_rot ? 3 : dd >= 2 * ep.d_rot ? 2 : dd >= ep.d_rot ? 1 : 0;
            axis8[j] = ax; // 3: not rotated
            jr8[j] = dd - (ax < 3 ? ax : 0) * ep.d_rot;
            off8[j] = ax < 3 ? jr8[j] : 0;
        }
        s_lo = axis8[0];
        s_hi = axis8[7];
        jsplit = 8;
#pragma unroll
        for (int j = 7; j >= 1; --j)
            if (axis8[j] != axis8[0]) jsplit = j;
    }
    const bool qk_cols = EPI == EPI_QKV && which < 2;

    // residual rows (when not prefetched at kernel start): the values of row
    // blocks fm and fm + 1 are requested before block fm is processed, so one
    // round trip to memory serves two blocks (the first ZD blocks may have been
    // requested by the caller already, under its last K step)
    constexpr int ZD = ZRows<EPI, NZ, FM, MI, WN>::ZD;
    auto &zq = zr.q;
    if (!z_requested) {
#pragma unroll
        for (int f = 0; f < ZD; ++f) zr.request(f, m0, woff_m, n0, woff_n, M, ep, part != nullptr);
    }

    auto row_path = [&](int rt, int zi, int p, int zslot, const float (&x)[8]) {
        const int row = m0 + rt;
        if (row >= M || !col_any) return;
        if (part) {
            // split-K: the raw partial sum of this workgroup's K range, fp32 [M, N]
            float *dst = part + (int64_t)row * N + col0;
            if (col_full) {
                reinterpret_cast<float4 *>(dst)[0] = make_float4(x[0], x[1], x[2], x[3]);
                reinterpret_cast<float4 *>(dst)[1] = make_float4(x[4], x[5], x[6], x[7]);
            } else {
                for (int j = 0; j < 8; ++j)
                    if (col0 + j < N) dst[j] = x[j];
            }
            return;
        }
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = x[j] + pre.bias8[j];
        if constexpr (EPI == EPI_STORE || EPI == EPI_GELU) {
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = epi_act<EPI>(v[j]);
            T *dst = reinterpret_cast<T *>(ep.out) + (int64_t)row * ep.ldo + col0;
            if (col_full && (ep.ldo % 8) == 0) {
                store_vec8<T>(dst, v);
            } else {
                for (int j = 0; j < 8; ++j)
                    if (col0 + j < N) dst[j] = from_f32<T>(v[j]);
            }
        } else if constexpr (EPI == EPI_RESID) {
            float *z = ep.Z + (int64_t)row * ep.ldz + col0;
            if (z_vec(ep, row, M, col_full)) {
                float4 z0, z1;
                if constexpr (NZ > 0) {
                    z0 = pre.z[zi][0];
                    z1 = pre.z[zi][1];
                } else {
                    z0 = zq[zslot][p][0];
                    z1 = zq[zslot][p][1];
                }
                if (ep.ls) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) v[j] *= pre.ls8[j];
                }
                z0.x += v[0]; z0.y += v[1]; z0.z += v[2]; z0.w += v[3];
                z1.x += v[4]; z1.y += v[5]; z1.z += v[6]; z1.w += v[7];
                reinterpret_cast<float4 *>(z)[0] = z0;
                reinterpret_cast<float4 *>(z)[1] = z1;
            } else {
                for (int j = 0; j < 8; ++j)
                    if (col0 + j < N) z[j] += (ep.ls ? pre.ls8[j] : 1.0f) * v[j];
            }
        } else if constexpr (EPI == EPI_PATCH) {
            const RowInfo info = ri[rt];
            float *z = ep.Z + (int64_t)info.out_row * ep.ldz + col0;
            for (int j = 0; j < 8; ++j) {
                if (col0 + j >= N) break;
                float y = v[j];
                if (ep.pos) y += ep.pos[(int64_t)info.pos * ep.ldz + col0 + j];
                if (ep.mod) y += ep.mod[col0 + j];
                z[j] = y;
            }
        } else if constexpr (EPI == EPI_QKV) {
            if (!qk_cols) return; // V columns go through the transposed path
            const RowInfo info = ri[rt];
            if (ep.rope && info.pos) {
                float y[8];
                if (tab_lds) {
                    auto sel = [&](int sx) {
                        return sx == 0 ? info.base[0] : sx == 1 ? info.base[1] : sx == 2 ? info.base[2] : id_pair;
                    };
                    const int b_lo = sel(s_lo), b_hi = sel(s_hi);
                    const float4 *tab4 = reinterpret_cast<const float4 *>(lds_tab);
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        // entries (2u, 2u + 1): (cos, signed sin) of dim 2u, then of dim 2u + 1
                        const float4 cs = tab4[((2 * u < jsplit ? b_lo : b_hi) + off8[2 * u]) >> 1];
                        y[2 * u] = v[2 * u] * cs.x + v[2 * u + 1] * cs.y;
                        y[2 * u + 1] = v[2 * u + 1] * cs.z + v[2 * u] * cs.w;
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        y[j] = v[j];
                        if (axis8[j] < 3) {
                            const int base = axis8[j] == 0 ? info.base[0] : axis8[j] == 1 ? info.base[1] : info.base[2];
                            const float2 cs = tab[base + jr8[j]];
                            y[j] = v[j] * cs.x + v[j ^ 1] * cs.y;
                        }
                    }
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] = y[j];
            }
            T *dst = reinterpret_cast<T *>(which == 0 ? ep.Q : ep.K) + info.qk_off + qk_col;
            store_vec8<T>(dst, v);
        }
    };

#pragma clang loop unroll(full)
    for (int fm = 0; fm < FM; ++fm) {
        // stage block row fm of this wave's accumulators
        if constexpr (SWAP) {
            // the block holds D^T (weight fragment as MFMA operand A): lane l has
            // row l % 32 and, per slot group q, 4 consecutive columns 8q + 4(l/32)
            static_assert(MI == 32, "swapped staging assumes 32x32 blocks");
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<float4 *>(&stage[lcol * LD + fn * MI + 8 * q + 4 * (lane >> 5)]) =
                        make_float4(acc[fm][fn][4 * q], acc[fm][fn][4 * q + 1], acc[fm][fn][4 * q + 2],
                                    acc[fm][fn][4 * q + 3]);
        } else {
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int i = 0; i < NV; ++i) stage[vrow(i) * LD + fn * MI + lcol] = acc[fm][fn][i];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // row path: lane -> (row, 8-column group)
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
            const int r = p * RPP + lane / CPR;
            if (r < MI && lane < RPP * CPR) {
                const float4 x0 = *reinterpret_cast<const float4 *>(&stage[r * LD + c0]);
                const float4 x1 = *reinterpret_cast<const float4 *>(&stage[r * LD + c0 + 4]);
                const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
                row_path(woff_m + fm * MI + r, fm * NPASS + p, p, fm % ZD, x);
            }
        }
        // the slot of block fm is free: request block fm + ZD into it
        if (fm + ZD < FM) zr.request(fm + ZD, m0, woff_m, n0, woff_n, M, ep, part != nullptr);
        if constexpr (EPI == EPI_QKV) {
            // V columns: lane -> (column, 8 consecutive rows), stored along tokens
            static_assert(64 % WN == 0, "one V column per lane");
            const int cbase = n0 + woff_n;
            if (cbase + WN > 2 * ep.D) {
                const int H = ep.D / ep.head_dim;
                for (int cc = lane; cc < WN * (MI / 8); cc += 64) {
                    const int c = cc % WN, rg = cc / WN;
                    const int col = cbase + c;
                    if (col < 2 * ep.D || col >= N) continue;
                    const float bias = pre.vbias;
                    const int within = col - 2 * ep.D;
                    const int head = within / ep.head_dim, dd = within - head * ep.head_dim;
                    float v[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = stage[(rg * 8 + e) * LD + c] + bias;
                    const int rt0 = woff_m + fm * MI + rg * 8;
                    const RowInfo i0 = ri[rt0];
                    const bool vec = (m0 + rt0 + 7 < M) && (i0.tok % 8 == 0) && (i0.tok + 8 <= ep.Ntok);
                    if (vec) {
                        T *dst = reinterpret_cast<T *>(ep.Vt) +
                                 (((int64_t)i0.out_row * H + head) * ep.head_dim + dd) * ep.ldv + i0.tok;
                        store_vec8<T>(dst, v);
                    } else {
                        for (int e = 0; e < 8; ++e) {
                            if (m0 + rt0 + e >= M) break;
                            const RowInfo ie = ri[rt0 + e];
                            T *dst = reinterpret_cast<T *>(ep.Vt) +
                                     (((int64_t)ie.out_row * H + head) * ep.head_dim + dd) * ep.ldv + ie.tok;
                            *dst = from_f32<T>(v[e]);
                        }
                    }
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
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

    // A rows [0, BM) and W rows [BM, BM + BN) of each buffer
    __shared__ Chunk smem[2][BM + BN][8];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6); // wave-uniform, lives in an SGPR
    const int wm = wave >> 1, wn = wave & 1;
    const int g = lane >> 5, l32 = lane & 31;
    const int ntile = gridDim.x / ep.splits;
    const int split = blockIdx.x / ntile;
    const int tile = xcd_tile(blockIdx.x - split * ntile, ntile);
    const int tm = tile / tiles_n, tn = tile - tm * tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;
    const int lc = tid & 7, lr = tid >> 3;
    using RP = RowPath<32, WN>;
    constexpr int kNZ = 0;
    // the 128 x 128 tiles of this kernel use nearly every register already:
    // their QKV epilogue copies the RoPE table from global memory instead
    constexpr int kNTab = (EPI == EPI_QKV && BM < 128) ? 4 : 0;
    const auto pre = epi_prefetch<EPI, kNZ, kNTab, BM, FM, kThreads, 32, WN>(m0, n0, wm * WM, wn * WN, M, N, ep);

    // per-thread row pointers of the chunks this thread stages
    const T *pa[A_PER];
    const T *pb[B_PER];
#pragma unroll
    for (int i = 0; i < A_PER; ++i) pa[i] = A + (int64_t)min(m0 + lr + 32 * i, M - 1) * lda + lc * KPC;
#pragma unroll
    for (int i = 0; i < B_PER; ++i) pb[i] = W + (int64_t)min(n0 + lr + 32 * i, N - 1) * ldw + lc * KPC;

    const int kw = ep.kwrap ? ep.kwrap : K; // W columns
    auto gload = [&](Chunk *ra, Chunk *rb, int k0) {
        const int kb = k0 >= kw ? k0 - kw : k0; // W column of A column k0
        if constexpr (FAST) {
#pragma unroll
            for (int i = 0; i < A_PER; ++i) ra[i] = load_chunk(pa[i] + k0);
#pragma unroll
            for (int i = 0; i < B_PER; ++i) rb[i] = load_chunk(pb[i] + kb);
        } else {
#pragma unroll
            for (int i = 0; i < A_PER; ++i)
                ra[i] = load_tile_chunk<T, false>(A, lda, m0 + lr + 32 * i, M, k0 + lc * KPC, K);
#pragma unroll
            for (int i = 0; i < B_PER; ++i)
                rb[i] = load_tile_chunk<T, false>(W, ldw, n0 + lr + 32 * i, N, kb + lc * KPC, kw);
        }
    };
    auto sstore = [&](const Chunk *ra, const Chunk *rb, int buf) {
#pragma unroll
        for (int i = 0; i < A_PER; ++i) {
            const int r = lr + 32 * i;
            smem[buf][r][lc ^ swz8(r)] = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_PER; ++i) {
            const int r = lr + 32 * i;
            smem[buf][BM + r][lc ^ swz8(BM + r)] = rb[i];
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
            a[fm] = smem[buf][r][cc ^ swz8(r)];
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int r = BM + wn * WN + fn * 32 + l32;
            b[fn] = smem[buf][r][cc ^ swz8(r)];
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
    // this workgroup's K steps: [kb0, kb0 + nk) of cdiv(K, BK)
    const int nk_all = (int)cdiv(K, BK);
    const int kb0 = (int)((int64_t)split * nk_all / ep.splits);
    const int nk = (int)((int64_t)(split + 1) * nk_all / ep.splits) - kb0;
    const int kbase = kb0 * BK;
    Chunk ra0[A_PER], rb0[B_PER], ra1[A_PER], rb1[B_PER];
    gload(ra0, rb0, kbase);
    if (nk > 1) gload(ra1, rb1, kbase + BK);
    sstore(ra0, rb0, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
        if (kt + 2 < nk) gload(ra0, rb0, kbase + (kt + 2) * BK);
        compute(0);
        if (kt + 1 < nk) sstore(ra1, rb1, 1);
        __syncthreads();
        if (kt + 1 >= nk) break;
        if (kt + 3 < nk) gload(ra1, rb1, kbase + (kt + 3) * BK);
        compute(1);
        if (kt + 2 < nk) sstore(ra0, rb0, 0);
        __syncthreads();
    }

    char *sbase = reinterpret_cast<char *>(&smem[0][0][0]);
    constexpr int kRiBytes = (BM * (int)sizeof(RowInfo) + 255) / 256 * 256;
    constexpr int kStageBytes = 4 * 32 * (WN + 4) * 4;
    static_assert(kRiBytes + kStageBytes <= (int)sizeof(smem), "epilogue staging exceeds LDS");
    RowInfo *ri = reinterpret_cast<RowInfo *>(sbase);
    float *stage = reinterpret_cast<float *>(sbase + kRiBytes) + wave * 32 * (WN + 4);
    float2 *ltab = reinterpret_cast<float2 *>(sbase + kRiBytes + kStageBytes);
    constexpr int kTabCap = ((int)sizeof(smem) - kRiBytes - kStageBytes) / 8;
    ZRows<EPI, kNZ, FM, 32, WN> zr;
    gemm_epilogue<T, BM, FM, FN, EPI, kThreads, 32, WN, false>(
        acc, pre, ri, stage, ltab, kTabCap, m0, n0, wm * WM, wn * WN, M, N, ep,
        ep.splits > 1 ? ep.sk_part + (int64_t)split * M * N : nullptr, zr, false);
}



// Wide-tile variant for shapes with enough tiles to fill the chip: a BM x BN
// tile per workgroup of WGM x WGN waves, each wave owning a (BM/WGM) x
// (BN/WGN) block of 32x32 MFMA tiles, so one 16-byte operand fragment read
// from LDS feeds several MFMAs.  Slabs of BK = 8*NCH bytes per row go from
// global memory straight into LDS with buffer loads (lane l of a load
// instruction writes bytes [16 l, 16 l + 16) of a 1 KB LDS run; rows past M
// or N lie outside the buffer resource and read as zero), so no staging
// registers are needed; the LDS swizzle is applied on the global side by
// choosing which chunk each lane fetches.  A ring of STAGES LDS stages keeps
// STAGES - 1 slabs in flight while one is multiplied.  Requires the FAST
// conditions (K a multiple of the slab width, 16-byte aligned rows).
// The direct-to-LDS kernel computes each 32x32 block transposed (weight
// fragment as MFMA operand A), so that every lane holds runs of 4 consecutive
// output columns and stages them into LDS with 16-byte writes.

//
// WQ (8-bit weights, bf16 activations): W holds one E4M3 byte per weight and
// every 32 weights of a row share a power-of-two scale (EpiArgs::wscale).  A
// weight row of the slab is then NCH/2 chunks; each lane reads the 16 codes
// of its row for k in [32t + 16g, 32t + 16g + 16) (t: the 32-weight block of
// the slab, g = lane / 32) and expands 8 of them per MFMA k-step into bf16
// with the scaled conversion, which multiplies by the block's 2^e exactly.
// The activation chunk of a step is picked to hold the same k indices (chunk
// 4t + 2g + h at step 2t + h).  The scale bytes of a slab (2 per weight row,
// contiguous over the rows in the [K/64][N][2] layout) come along with it:
// wave 0 issues one more direct-to-LDS load per slab.
// One 16-byte-per-lane buffer load straight into LDS at dst (wave-uniform;
// lane l's 16 bytes land at dst + 16 l), issued from inline assembly.  The
// direct-to-LDS kernel issues all its slab loads this way: with the builtin,
// the compiler cannot always tell the ring stages apart and then waits for
// every refill (vmcnt(0)) before the next stage's fragment reads, which
// serialises the ring (whether it does depends on how its alias analysis of
// the surrounding code comes out); the kernel orders these loads itself
// (vm_wait + barrier).  M0 carries the LDS address; nothing else in that
// kernel keeps a value in M0.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, const void *dst, uint32_t voff, uint32_t soff) {
    const uint32_t lds = (uint32_t)(uintptr_t)(const lds_void_t *)dst;
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds), "v"(voff), "s"(rs),
                 "s"(soff)
                 : "memory");
}

// Longest prefix row (K) the tile kernel takes beside its grid (EpiArgs::pre_a)
constexpr int kPreMaxK = 4096;
// acc + a.lo * b.lo + a.hi * b.hi for dwords holding two 16-bit values
// (one packed dot product, fp32 accumulation)
template <typename T> __device__ __forceinline__ float dot2_acc(uint32_t a, uint32_t b, float acc);
template <> __device__ __forceinline__ float dot2_acc<bf16_t>(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), acc,
                                           false);
}
template <> __device__ __forceinline__ float dot2_acc<f16_t>(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), acc, false);
}

template <typename T, int BM, int BN, int WGM, int WGN, int NCH, int STAGES, int MI, int EPI, bool WQ, bool PRE>
__device__ __forceinline__ void gemm_lds_body(const T *__restrict__ A, int64_t lda, const void *__restrict__ W,
                                              int64_t ldw, int M, int N, int K, int tiles_n, int a_bytes,
                                              int b_bytes, int s_bytes, const EpiArgs &ep) {
    constexpr int KPC = Elem<T>::kPerChunk;
    constexpr int BK = NCH * KPC;
    constexpr int NW = WGM * WGN, NT = 64 * NW;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int FM = WM / MI, FN = WN / MI;
    using AccT = typename std::conditional<MI == 32, f32x16, f32x4>::type;
    constexpr int NV = MI == 32 ? 16 : 4;
    constexpr int RPI = 64 / NCH;                       // slab rows per load instruction
    constexpr int WCH = WQ ? NCH / 2 : NCH;             // chunks per weight row of a slab
    constexpr int RPW = 64 / WCH;                       // weight rows per load instruction
    constexpr int AI = BM / (RPI * NW), BI = BN / (RPW * NW); // load instructions per wave and slab
    constexpr int SC_CH = WQ ? 64 : 0;                  // scale bytes of a slab: one 1 KB load
    constexpr int STAGE_CH = BM * NCH + BN * WCH + SC_CH; // chunks per LDS stage
    static_assert(NCH == 4 || NCH == 8 || NCH == 16, "slab of 64, 128 or 256 bytes per row");
    static_assert(WM % MI == 0 && WN % MI == 0 && AI * RPI * NW == BM && BI * RPW * NW == BN, "tile");
    static_assert(MI == 32 || MI == 16, "MFMA tile");
    static_assert(!WQ || (std::is_same<T, bf16_t>::value && MI == 32 && NCH == 8 && 2 * BN <= 1024),
                  "8-bit weights: bf16 activations, 32x32 MFMAs, 64-k slabs");

    // PRE: the prefix row of A, K values, after the ring
    constexpr int kPreOff = STAGES * STAGE_CH, kPreChunks = PRE ? kPreMaxK / KPC : 0;
    static_assert(!PRE || ((EPI == EPI_RESID || EPI == EPI_GELU) && !WQ && MI == 32), "prefix row: RESID / GELU");
    __shared__ Chunk lds[STAGES * STAGE_CH + kPreChunks];
    auto lA = [&](int stage, int r, int c) -> Chunk & { return lds[stage * STAGE_CH + r * NCH + c]; };
    auto lW = [&](int stage, int r, int c) -> Chunk & { return lds[stage * STAGE_CH + BM * NCH + r * WCH + c]; };
    auto lS = [&](int stage) { return reinterpret_cast<const uint16_t *>(&lds[stage * STAGE_CH + BM * NCH + BN * WCH]); };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6); // wave-uniform, lives in an SGPR
    const int wm = wave / WGN, wn = wave % WGN;
    const int g = lane >> 5, l32 = lane & 31;
    const int ntile = gridDim.x / ep.splits;
    const int split = blockIdx.x / ntile;
    const int tile = xcd_tile(blockIdx.x - split * ntile, ntile);
    const int tm = tile / tiles_n, tn = tile - tm * tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;
    using RP = RowPath<MI, WN>;
    // (the residual rows are requested at the start of the epilogue: requested
    // here they would be returned, in order, ahead of the first slabs)
    constexpr int kNZ = 0;
    constexpr int kNTab = EPI == EPI_QKV ? 4 : 0;
    const auto pre = epi_prefetch<EPI, kNZ, kNTab, BM, FM, NT, MI, WN>(m0, n0, wm * WM, wn * WN, M, N, ep);

    // Buffer loads: one resource per operand, a per-lane byte offset and a
    // scalar offset for the slab and the instruction's row block.  Lane l of
    // load instruction j fetches row RPI*j + l/NCH of the wave's share of the
    // slab.  The swizzle repeats every 16 rows and each wave's share starts
    // on a multiple of 16, so the swizzled chunk of rows RPI*j + r depends on
    // j only through j mod 16/RPI: one lane offset for 4-chunk rows, two for
    // 8-chunk rows, four for 16-chunk rows.
    constexpr uint32_t ES = sizeof(T);
    constexpr uint32_t WES = WQ ? 1 : sizeof(T); // bytes per weight
    constexpr int JA = 16 / RPI, JB = 16 / RPW;  // distinct lane offsets per operand
    static_assert((BM / NW) % 16 == 0 && (BN / NW) % 16 == 0, "wave shares of whole 16-row blocks");
    const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc((void *)A, 0, a_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc((void *)W, 0, b_bytes, 0x00020000);
    const int lrow = lane / NCH, lch = lane % NCH;
    const int64_t arow = (int64_t)(m0 + wave * AI * RPI + lrow) * lda;
    uint32_t va[JA];
#pragma unroll
    for (int j = 0; j < JA; ++j) va[j] = (uint32_t)((arow + (lch ^ swz<NCH>(j * RPI + lrow)) * KPC) * ES);
    const int wrow = lane / WCH, wch = lane % WCH;
    const int64_t brow = (int64_t)(n0 + wave * BI * RPW + wrow) * ldw * WES;
    uint32_t vb[JB];
#pragma unroll
    for (int j = 0; j < JB; ++j) vb[j] = (uint32_t)(brow + (wch ^ swz<WCH>(j * RPW + wrow)) * 16);
    const int kw = ep.kwrap ? ep.kwrap : K; // W columns
    const __amdgpu_buffer_rsrc_t rss =
        __builtin_amdgcn_make_buffer_rsrc((void *)(WQ ? ep.wscale : nullptr), 0, WQ ? s_bytes : 0, 0x00020000);
    auto load = [&](__amdgpu_buffer_rsrc_t rs, const void *dst, uint32_t voff, uint32_t soff) {
        dma16(rs, dst, voff, soff);
    };
    auto issue = [&](int stage, int k0) {
#pragma unroll
        for (int j = 0; j < AI; ++j) {
            const int row = (wave * AI + j) * RPI;
            const uint32_t soff = (uint32_t)((k0 + (int64_t)j * RPI * lda) * ES);
            load(rsa, &lA(stage, row, 0), va[j % JA], soff);
        }
        const int kb = k0 >= kw ? k0 - kw : k0; // W column of A column k0
#pragma unroll
        for (int j = 0; j < BI; ++j) {
            const int row = (wave * BI + j) * RPW;
            const uint32_t soff = (uint32_t)((kb + (int64_t)j * RPW * ldw) * WES);
            load(rsb, &lW(stage, row, 0), vb[j % JB], soff);
        }
        if constexpr (WQ) {
            // scale bytes of rows n0 .. n0 + BN for this slab: [k0/64][n][2]
            if (wave == 0)
                load(rss, lS(stage), (uint32_t)(lane * 16 + 2 * n0), (uint32_t)((int64_t)(k0 / 64) * 2 * N));
        }
    };

    AccT acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int i = 0; i < NV; ++i) acc[fm][fn][i] = 0.0f;

    // one MFMA k-step: 32x32x16 consumes chunk 2s + (l/32); 16x16x32 consumes
    // chunk 4s + (l/16) of each operand row
    constexpr int KSUB = MI == 32 ? NCH / 2 : NCH / 4;
    const int lr = lane & (MI - 1);
    const int lq = MI == 32 ? (lane >> 5) : (lane >> 4);
    Chunk wraw[WQ ? FN : 1]; // WQ: the 16 codes of the current 32-weight block
    uint32_t wsc[WQ ? FN : 1]; // WQ: the two scale bytes of the slab
    auto frags = [&](Chunk *a, Chunk *b, int stage, int s) {
        if constexpr (WQ) {
            const int t = s >> 1, h = s & 1;
            const int cc = 4 * t + 2 * lq + h;
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int r = wm * WM + fm * MI + lr;
                a[fm] = lA(stage, r, cc ^ swz<NCH>(r));
            }
            // only the reads here: the codes are expanded by expand() after
            // the current step's MFMAs are issued, so that the wave does not
            // wait on these reads before issuing them
            (void)b;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int r = wn * WN + fn * MI + lr;
                if (s == 0) wsc[fn] = lS(stage)[r];
                if (h == 0) wraw[fn] = lW(stage, r, (2 * t + lq) ^ swz<WCH>(r));
            }
        } else {
            const int cc = (MI == 32 ? 2 : 4) * s + lq;
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int r = wm * WM + fm * MI + lr;
                a[fm] = lA(stage, r, cc ^ swz<NCH>(r));
            }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int r = wn * WN + fn * MI + lr;
                b[fn] = lW(stage, r, cc ^ swz<NCH>(r));
            }
        }
    };
    // WQ: the bf16 weight fragment of step s from the codes read by frags()
    auto expand = [&](Chunk *b, int s) {
        if constexpr (WQ) {
            const int t = s >> 1, h = s & 1;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                // E8M0 byte -> fp32 2^(byte - 127); the conversion uses its exponent
                const float sc = __builtin_bit_cast(float, ((wsc[fn] >> (8 * t)) & 0xFFu) << 23);
                const uint32_t lo = wraw[fn].w[2 * h], hi = wraw[fn].w[2 * h + 1];
                b[fn].w[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, sc, false));
                b[fn].w[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, sc, true));
                b[fn].w[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, sc, false));
                b[fn].w[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, sc, true));
            }
        }
    };
    auto mfmas = [&](const Chunk *a, const Chunk *b) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                if constexpr (MI == 32) mfma_chunk<T>(acc[fm][fn], b[fn], a[fm]); // D^T
                else mfma16_chunk<T>(acc[fm][fn], a[fm], b[fn]);
            }
    };
    // keep the next sub-step's fragment reads ahead of this sub-step's MFMAs
    auto order_reads_first = [&]() {
        __builtin_amdgcn_sched_group_barrier(0x100, FM + FN, 0); // DS reads
        __builtin_amdgcn_sched_group_barrier(0x008, FM * FN, 0); // MFMAs
        if constexpr (WQ) __builtin_amdgcn_sched_group_barrier(0x002, 4 * FN + 2, 0); // expansion (VALU)
    };
    // Wait until this wave's loads of one slab have landed while `later`
    // slabs issued after it may still be in flight, then barrier: every
    // wave's part of the slab is visible and every wave has finished reading
    // what it read before.  (STAGES - 1 is at most 7, so `later` is at most 6
    // wherever a later slab exists.)
    constexpr int PER = AI + BI; // load instructions per wave and slab (wave 0: + 1 with WQ)
    static_assert(STAGES >= 2 && STAGES <= 8 && (STAGES - 1) * (PER + 1) <= 63, "vmcnt range");
    auto wait_n = [&](auto per_c, int later) {
        constexpr int P = decltype(per_c)::value;
        switch (later) {
        case 0: vm_wait<0>(); break;
        case 1: vm_wait<P>(); break;
        case 2: vm_wait<(STAGES > 2 ? 2 * P : 0)>(); break;
        case 3: vm_wait<(STAGES > 3 ? 3 * P : 0)>(); break;
        case 4: vm_wait<(STAGES > 4 ? 4 * P : 0)>(); break;
        case 5: vm_wait<(STAGES > 5 ? 5 * P : 0)>(); break;
        default: vm_wait<(STAGES > 6 ? 6 * P : 0)>(); break;
        }
    };
    auto wait_slab = [&](int later) {
        if (WQ && wave == 0) wait_n(std::integral_constant<int, PER + 1>{}, later);
        else wait_n(std::integral_constant<int, PER>{}, later);
        __syncthreads();
    };

    // Software pipeline over the whole K loop: the fragments of sub-step s+1
    // are read while the MFMAs of sub-step s run.  At the last sub-step of
    // slab kt the hand-off comes before that sub-step's MFMAs: wait for slab
    // kt+1, barrier (after which slab kt's stage is free), issue slab
    // kt+STAGES into it, and read the first fragments of slab kt+1; those
    // reads then overlap the last MFMAs of slab kt.
    // this workgroup's slabs: [kb0, kb0 + nk) of K / BK
    const int nk_all = K / BK;
    const int kb0 = (int)((int64_t)split * nk_all / ep.splits);
    const int nk = (int)((int64_t)(split + 1) * nk_all / ep.splits) - kb0;
    const int kbase = kb0 * BK;
    // PRE: this workgroup's share of the prefix row's N columns is cpw
    // columns from n0 + tm * cpw (the tiles of one column block split its BN
    // columns; the launcher checks that they divide evenly), cpw / NW per
    // wave; lane l takes column l / NCH of its wave's share and, in every
    // slab, chunk l % NCH of that column's weights and of the prefix row.
    // The row itself is fetched into LDS before the first slab, so the first
    // slab wait covers it.
    float pre_acc = 0.0f;
    int pre_r = 0;
    bool pre_live = false;
    if constexpr (PRE) {
        const int tiles_m = (M + BM - 1) / BM, cpw = BN / tiles_m, cpwv = cpw / NW;
        const int j = lane / NCH;
        pre_live = j < cpwv;
        pre_r = tm * cpw + wave * cpwv + (pre_live ? j : 0);
        const __amdgpu_buffer_rsrc_t rsp =
            __builtin_amdgcn_make_buffer_rsrc((void *)ep.pre_a, 0, K * (int)sizeof(T), 0x00020000);
        for (int b = wave; b * 64 < K / KPC; b += NW)
            dma16(rsp, &lds[kPreOff + b * 64], (uint32_t)lane * 16u, (uint32_t)b * 1024u);
    }
    // (read at the top of a slab's K step, added at its end, so that the LDS
    // round trip hides under the step's MFMAs)
    Chunk pre_w, pre_a;
    auto pre_read = [&](int stg, int kt) {
        if constexpr (PRE) {
            const int c = lane % NCH;
            pre_w = lW(stg, pre_r, c ^ swz<NCH>(pre_r));
            pre_a = lds[kPreOff + (kbase / KPC) + kt * NCH + c];
        }
    };
    auto pre_add = [&]() {
        if constexpr (PRE) {
#pragma unroll
            for (int e = 0; e < 4; ++e) pre_acc = dot2_acc<T>(pre_a.w[e], pre_w.w[e], pre_acc);
        }
    };
#pragma unroll
    for (int s = 0; s < STAGES; ++s)
        if (s < nk) issue(s, kbase + s * BK);
    wait_slab(min(STAGES, nk) - 1);
    Chunk a0[FM], b0[FN], a1[FM], b1[FN];
    frags(a0, b0, 0, 0);
    expand(b0, 0);
    int stage = 0;
    // RESID: the first residual row blocks are requested at the start of the
    // last K step, after its slab has landed (no slab load is issued after
    // them), so that their round trip hides under that step's MFMAs.  Not in
    // the configurations whose registers are full already: 256-row tiles
    // (the values would spill) and the 128 x 128 two-stage tiles that need
    // 128 registers or fewer for two workgroups per CU.
    ZRows<EPI, kNZ, FM, MI, WN> zr;
    constexpr bool kZEarly =
        ZRows<EPI, kNZ, FM, MI, WN>::kOn && BM <= 128 && !(BM == 128 && NW == 8 && STAGES == 2);
    for (int kt = 0; kt < nk; ++kt) {
        int nstage = stage + 1;
        if (nstage == STAGES) nstage = 0;
        pre_read(stage, kt);
        if (kZEarly && kt == nk - 1) {
#pragma unroll
            for (int f = 0; f < ZRows<EPI, kNZ, FM, MI, WN>::ZD; ++f)
                zr.request(f, m0, wm * WM, n0, wn * WN, M, ep, ep.splits > 1);
        }
#pragma unroll
        for (int s = 0; s < KSUB; ++s) {
            Chunk *ca = (s & 1) ? a1 : a0, *cb = (s & 1) ? b1 : b0;
            Chunk *na = (s & 1) ? a0 : a1, *nb = (s & 1) ? b0 : b1;
            if (s + 1 < KSUB) {
                frags(na, nb, stage, s + 1);
                mfmas(ca, cb);
                expand(nb, s + 1);
                order_reads_first();
            } else {
                if (kt + 1 < nk) {
                    // slabs issued so far: 0 .. min(kt + STAGES - 1, nk - 1)
                    wait_slab(min(kt + STAGES - 1, nk - 1) - (kt + 1));
                    if (kt + STAGES < nk) issue(stage, kbase + (kt + STAGES) * BK);
                    frags(na, nb, nstage, 0);
                }
                mfmas(ca, cb);
                if (kt + 1 < nk) {
                    expand(nb, 0);
                    order_reads_first();
                }
            }
        }
        pre_add();
        stage = nstage;
        if (KSUB & 1) {
            // odd sub-step count: the next slab's first fragments sit in the
            // other register set; swap the roles of the two sets
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) { Chunk t = a0[fm]; a0[fm] = a1[fm]; a1[fm] = t; }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) { Chunk t = b0[fn]; b0[fn] = b1[fn]; b1[fn] = t; }
        }
    }
    if constexpr (PRE) {
        // sum over the NCH lanes of each column, then the epilogue of the row
#pragma unroll
        for (int o = NCH / 2; o >= 1; o >>= 1) pre_acc += __shfl_xor(pre_acc, o, 64);
        const int col = n0 + pre_r;
        if (pre_live && lane % NCH == 0 && col < N) {
            const float v = pre_acc + (ep.bias ? ep.bias[col] : 0.0f);
            if constexpr (EPI == EPI_RESID) ep.pre_z[col] += ep.ls ? ep.ls[col] * v : v;
            else reinterpret_cast<T *>(ep.pre_out)[col] = from_f32<T>(gelu_erf(v));
        }
    }
    __syncthreads();
    char *sbase = reinterpret_cast<char *>(&lds[0]);
    constexpr int kRiBytes = (BM * (int)sizeof(RowInfo) + 255) / 256 * 256;
    constexpr int kStageBytes = NW * MI * (WN + 4) * 4;
    static_assert(kRiBytes + kStageBytes <= (int)sizeof(lds), "epilogue staging exceeds LDS");
    RowInfo *ri = reinterpret_cast<RowInfo *>(sbase);
    float *estage = reinterpret_cast<float *>(sbase + kRiBytes) + wave * MI * (WN + 4);
    float2 *ltab = reinterpret_cast<float2 *>(sbase + kRiBytes + kStageBytes);
    constexpr int kTabCap = ((int)sizeof(lds) - kRiBytes - kStageBytes) / 8;
    gemm_epilogue<T, BM, FM, FN, EPI, NT, MI, WN, MI == 32>(acc, pre, ri, estage, ltab, kTabCap, m0, n0, wm * WM,
                                                            wn * WN, M, N, ep,
                                                            ep.splits > 1 ? ep.sk_part + (int64_t)split * M * N : nullptr,
                                                            zr, kZEarly && nk > 0);
}

template <typename T, int BM, int BN, int WGM, int WGN, int NCH, int STAGES, int MI, int EPI, bool WQ>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void gemm_lds_kernel(const T *__restrict__ A, int64_t lda,
                                                                     const void *__restrict__ W, int64_t ldw, int M,
                                                                     int N, int K, int tiles_n, int a_bytes,
                                                                     int b_bytes, int s_bytes, EpiArgs ep) {
    gemm_lds_body<T, BM, BN, WGM, WGN, NCH, STAGES, MI, EPI, WQ, false>(A, lda, W, ldw, M, N, K, tiles_n, a_bytes,
                                                                        b_bytes, s_bytes, ep);
}
// the same with one prefix row beside the tile grid (EpiArgs::pre_a)
template <typename T, int BM, int BN, int WGM, int WGN, int NCH, int STAGES, int MI, int EPI>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void gemm_lds_pre_kernel(const T *__restrict__ A, int64_t lda,
                                                                         const void *__restrict__ W, int64_t ldw,
                                                                         int M, int N, int K, int tiles_n,
                                                                         int a_bytes, int b_bytes, EpiArgs ep) {
    gemm_lds_body<T, BM, BN, WGM, WGN, NCH, STAGES, MI, EPI, false, true>(A, lda, W, ldw, M, N, K, tiles_n, a_bytes,
                                                                          b_bytes, 0, ep);
}

// Split-K where the output tiles fill at most half of the per_cu workgroup
// slots of the 256 CUs (the tiles of small inputs walk K serially, bound by the
// latency of each step): enough splits to fill them, each split keeping at
// least min_steps K steps, at most 16.  The partials cost 8 bytes per output
// and split of HBM traffic, so short-K GEMMs with many outputs do not split.
// Only the STORE, GELU and RESID epilogues split (the reduction kernel below
// applies them); N must be a multiple of 4.
inline int splits_for(int epi, int64_t tiles, int nk, int per_cu, int min_steps, int M, int N, int K) {
    if (!(epi == EPI_STORE || epi == EPI_GELU || epi == EPI_RESID) || N % 4 != 0) return 1;
    const int64_t target = 256 * (int64_t)per_cu;
    // measured: 400 tiles of 64 x 64 (target 768) run slower split, and so do
    // GEMMs with fewer than four splits' worth of K steps (the reduction's
    // launch costs more than the split saves)
    if (2 * tiles > target || nk < 4 * min_steps) return 1;
    int S = (int)std::min<int64_t>({cdiv(target, tiles), (int64_t)nk / min_steps, 16});
    if (S > 1 && K < 2048 && (int64_t)M * N * 4 * S > (int64_t(8) << 20)) S = 1;
    return std::max(S, 1);
}
// ... and as far as the caller's scratch allows
inline int splits_with(int epi, int64_t tiles, int nk, int per_cu, int min_steps, int M, int N, int K,
                       const EpiArgs &ep) {
    if (!ep.sk_part) return 1;
    int S = splits_for(epi, tiles, nk, per_cu, min_steps, M, N, K);
    while (S > 1 && (int64_t)S * M * N > ep.sk_part_floats) --S;
    return S;
}
// workgroups per CU and minimum K steps per split of each kernel configuration
constexpr int kRegPerCU = 2, kRegMinSteps = 2, kLdsMinSteps = 8;
constexpr int lds_per_cu(int BM, int NCH, int STAGES) {
    return NCH == 16 ? 1 : BM == 64 ? 3 : (BM == 128 && STAGES == 2) ? 2 : 1;
}

// Second half of a split GEMM: v = (partial_0 + ... + partial_{S-1}) + bias,
// added in split order (the result does not depend on the order in which
// the splits finished), then the epilogue: STORE out = v, GELU out =
// GELU_erf(v), RESID Z += ls * v.  Four consecutive columns per thread.
template <typename T, int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ part, int S, int M, int N,
                                                            EpiArgs ep) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; // float4 index
    const int64_t MN = (int64_t)M * N;
    if (q * 4 >= MN) return;
    const int64_t e = q * 4;
    const int row = (int)(e / N), col = (int)(e - (int64_t)row * N);
    float4 v = reinterpret_cast<const float4 *>(part)[q];
    for (int sp = 1; sp < S; ++sp) {
        const float4 p = reinterpret_cast<const float4 *>(part + sp * MN)[q];
        v.x += p.x; v.y += p.y; v.z += p.z; v.w += p.w;
    }
    float r[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] += ep.bias ? ep.bias[col + j] : 0.0f;
    if constexpr (EPI == EPI_RESID) {
        float4 *z = reinterpret_cast<float4 *>(ep.Z + (int64_t)row * ep.ldz + col);
        float4 zz = *z;
        const float l0 = ep.ls ? ep.ls[col] : 1.0f, l1 = ep.ls ? ep.ls[col + 1] : 1.0f;
        const float l2 = ep.ls ? ep.ls[col + 2] : 1.0f, l3 = ep.ls ? ep.ls[col + 3] : 1.0f;
        zz.x += l0 * r[0]; zz.y += l1 * r[1]; zz.z += l2 * r[2]; zz.w += l3 * r[3];
        *z = zz;
    } else {
        if constexpr (EPI == EPI_GELU) {
#pragma unroll
            for (int j = 0; j < 4; ++j) r[j] = gelu_erf(r[j]);
        }
        T *o = reinterpret_cast<T *>(ep.out) + (int64_t)row * ep.ldo + col;
        if constexpr (sizeof(T) == 4) {
            *reinterpret_cast<float4 *>(o) = make_float4(r[0], r[1], r[2], r[3]);
        } else {
            *reinterpret_cast<uint2 *>(o) = make_uint2(pack2<T>(r[0], r[1]), pack2<T>(r[2], r[3]));
        }
    }
}

template <typename T, int EPI>
hipError_t launch_reduce(int S, int M, int N, const EpiArgs &ep, hipStream_t s) {
    if constexpr (EPI == EPI_STORE || EPI == EPI_GELU || EPI == EPI_RESID) {
        const int64_t n4 = (int64_t)M * N / 4;
        hipLaunchKernelGGL((splitk_reduce_kernel<T, EPI>), dim3((unsigned)cdiv(n4, 256)), dim3(256), 0, s, ep.sk_part,
                           S, M, N, ep);
        return hipGetLastError();
    } else {
        return hipErrorInvalidValue;
    }
}

// register-staged kernel, BM x BM tiles
template <typename T, int EPI, int BM, bool FAST>
hipError_t launch_t(const void *A, int64_t lda, const void *W, int64_t ldw, int M, int N, int K,
                    const EpiArgs &ep, hipStream_t s) {
    constexpr int BN = BM;
    const int tiles_n = (int)cdiv(N, BN), tiles_m = (int)cdiv(M, BM);
    EpiArgs e = ep;
    e.splits = splits_with(EPI, (int64_t)tiles_m * tiles_n, (int)cdiv(K, 8 * Elem<T>::kPerChunk), kRegPerCU,
                           kRegMinSteps, M, N, K, ep);
    hipLaunchKernelGGL((gemm_kernel<T, BM, BN, EPI, FAST>), dim3((unsigned)(tiles_m * tiles_n * e.splits)),
                       dim3(kThreads), 0, s, reinterpret_cast<const T *>(A), lda, reinterpret_cast<const T *>(W),
                       ldw, M, N, K, tiles_n, e);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess || e.splits == 1) return err;
    return launch_reduce<T, EPI>(e.splits, M, N, e, s);
}

template <typename T, int EPI, int BM, int BN, int WGM, int WGN, int NCH, int STAGES, int MI, bool WQ = false,
          bool PRE = false>
hipError_t launch_lds(const void *A, int64_t lda, const void *W, int64_t ldw, int M, int N, int K, const EpiArgs &ep,
                      hipStream_t s) {
    const int tiles_n = (int)cdiv(N, BN), tiles_m = (int)cdiv(M, BM);
    const int64_t wbytes = WQ ? 1 : (int64_t)sizeof(T);
    EpiArgs e = ep;
    e.splits = splits_with(EPI, (int64_t)tiles_m * tiles_n, K / (NCH * Elem<T>::kPerChunk), lds_per_cu(BM, NCH, STAGES),
                           kLdsMinSteps, M, N, K, ep);
    if constexpr (PRE) {
        // the tiles of a column block split its BN columns evenly, each wave's
        // share fits its lanes, and the K range is whole
        constexpr int NW = WGM * WGN;
        const int cpw = tiles_m > 0 && BN % tiles_m == 0 ? BN / tiles_m : 0;
        if (e.splits != 1 || K > kPreMaxK || cpw == 0 || cpw % NW != 0 || (cpw / NW) * NCH > 64 ||
            (uintptr_t)ep.pre_a % 16 != 0 || (EPI == EPI_RESID ? !ep.pre_z : !ep.pre_out))
            return hipErrorNotSupported;
    }
    if constexpr (PRE)
        hipLaunchKernelGGL((gemm_lds_pre_kernel<T, BM, BN, WGM, WGN, NCH, STAGES, MI, EPI>),
                           dim3((unsigned)(tiles_m * tiles_n)), dim3(64 * WGM * WGN), 0, s,
                           reinterpret_cast<const T *>(A), lda, W, ldw, M, N, K, tiles_n,
                           (int)((int64_t)M * lda * sizeof(T)), (int)((int64_t)N * ldw * wbytes), e);
    else
        hipLaunchKernelGGL((gemm_lds_kernel<T, BM, BN, WGM, WGN, NCH, STAGES, MI, EPI, WQ>),
                           dim3((unsigned)(tiles_m * tiles_n * e.splits)), dim3(64 * WGM * WGN), 0, s,
                           reinterpret_cast<const T *>(A), lda, W, ldw, M, N, K, tiles_n,
                           (int)((int64_t)M * lda * sizeof(T)), (int)((int64_t)N * ldw * wbytes),
                           WQ ? (int)((int64_t)(K / 64) * N * 2) : 0, e);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess || e.splits == 1) return err;
    return launch_reduce<T, EPI>(e.splits, M, N, e, s);
}

// Tile configuration (measured on the ViT-L shapes: M = 4096, N = 1024 ..
// 4096): 256 x 256 tiles (8 waves) when they give at least one full wave of
// workgroups over the 256 CUs, else 128 x 128 tiles (8 waves of 64 x 32, up
// to two workgroups per CU), both with direct-to-LDS slabs.  fp32 and shapes that break the
// FAST conditions use the register-staged kernel.
enum TileCfg { TILE_REG = 0, TILE_256x256 = 1, TILE_128x128 = 2, TILE_128x128_DEEP = 3, TILE_64x64 = 4 };

constexpr int kDeepStages = 3; // LDS ring of the one-tile-per-CU 128 x 128 configuration

// With at most one 128 x 128 tile per CU (the N = D projections of one clip)
// occupancy cannot hide the first touch of the weights in HBM: those tiles
// keep more slabs in flight instead, and (when K is a multiple of 128) run as
// 4 waves of 64 x 64 blocks over 128-deep slabs in a two-stage ring, which
// reads a third fewer fragment bytes from LDS per MFMA than 8 waves of 64 x 32
// and takes half as many barriers.
// 256 x 256 tiles are skipped when they would need a nearly empty second
// round.  When 128 x 128 tiles would leave more than half of the CUs idle (the
// width-384 projections of the predictor), 64 x 64 tiles of 4 waves spread
// the work instead.
inline int pick_tile(int M, int N, bool fast, bool fp32) {
    constexpr int kCUs = 256;
    if (!fast || fp32) return TILE_REG;
    {
        const int64_t t256 = cdiv(M, 256) * cdiv(N, 256);
        // a second round of 256x256 tiles that is mostly empty (M = 4097: one
        // CLS row past 4096) costs more than the smaller tiles
        if (t256 >= kCUs && !(t256 % kCUs != 0 && t256 % kCUs < kCUs / 4)) return TILE_256x256;
        if (t256 >= kCUs && cdiv(M, 128) * cdiv(N, 128) > kCUs) return TILE_128x128;
    }
    if (cdiv(M, 128) * cdiv(N, 128) < kCUs / 2) return TILE_64x64;
    if (cdiv(M, 128) * cdiv(N, 128) <= kCUs) return TILE_128x128_DEEP;
    return TILE_128x128;
}

inline bool reg_small_tiles(int M, int N) { return cdiv(M, 128) * cdiv(N, 128) < 128; }

template <typename T, int EPI>
hipError_t launch_align(const void *A, int64_t lda, const void *W, int64_t ldw, int M, int N, int K,
                        const EpiArgs &ep, hipStream_t s) {
    constexpr int KPC = Elem<T>::kPerChunk;
    const bool fast = (K % (8 * KPC) == 0) && (lda % KPC == 0) && (ldw % KPC == 0) &&
                      ((uintptr_t)A % 16 == 0) && ((uintptr_t)W % 16 == 0);
    // buffer offsets are 32-bit: the wide kernel needs both operands (plus a
    // tile of overhang) below 2 GiB
    const bool small = ((int64_t)M + 256) * lda * (int64_t)sizeof(T) < INT32_MAX &&
                       ((int64_t)N + 256) * ldw * (int64_t)sizeof(T) < INT32_MAX;
    if (ep.pre_a) {
        if constexpr (!std::is_same<T, float>::value && (EPI == EPI_RESID || EPI == EPI_GELU)) {
            if (fast && small && !ep.wscale && !ep.kwrap) {
                switch (pick_tile(M, N, true, false)) {
                case TILE_256x256:
                    return launch_lds<T, EPI, 256, 256, 2, 4, 8, 2, 32, false, true>(A, lda, W, ldw, M, N, K, ep, s);
                case TILE_128x128_DEEP:
                    if (K % 128 == 0)
                        return launch_lds<T, EPI, 128, 128, 2, 2, 16, 2, 32, false, true>(A, lda, W, ldw, M, N, K,
                                                                                          ep, s);
                    break;
                default: break;
                }
            }
        }
        return hipErrorNotSupported;
    }
    if constexpr (std::is_same<T, bf16_t>::value) {
        if (ep.wscale) {
            // 8-bit weights: the direct-to-LDS kernel only (conditions checked by the caller)
            const bool wfast = fast && small && K % 64 == 0 && N % 8 == 0 && ep.kwrap == 0 && ldw % 16 == 0;
            if (!wfast) return hipErrorInvalidValue;
            switch (pick_tile(M, N, true, false)) {
            case TILE_256x256: return launch_lds<T, EPI, 256, 256, 2, 4, 8, 2, 32, true>(A, lda, W, ldw, M, N, K, ep, s);
            case TILE_128x128: return launch_lds<T, EPI, 128, 128, 2, 4, 8, 2, 32, true>(A, lda, W, ldw, M, N, K, ep, s);
            case TILE_128x128_DEEP:
                return launch_lds<T, EPI, 128, 128, 2, 4, 8, kDeepStages, 32, true>(A, lda, W, ldw, M, N, K,
                                                                                          ep, s);
            case TILE_64x64: return launch_lds<T, EPI, 64, 64, 2, 2, 8, 3, 32, true>(A, lda, W, ldw, M, N, K, ep, s);
            default: return hipErrorInvalidValue;
            }
        }
    } else {
        if (ep.wscale) return hipErrorInvalidValue;
    }
    if constexpr (!std::is_same<T, float>::value) {
        switch (pick_tile(M, N, fast && small, false)) {
        case TILE_256x256: return launch_lds<T, EPI, 256, 256, 2, 4, 8, 2, 32>(A, lda, W, ldw, M, N, K, ep, s);
        case TILE_128x128: return launch_lds<T, EPI, 128, 128, 2, 4, 8, 2, 32>(A, lda, W, ldw, M, N, K, ep, s);
        case TILE_128x128_DEEP:
            if (K % 128 == 0) return launch_lds<T, EPI, 128, 128, 2, 2, 16, 2, 32>(A, lda, W, ldw, M, N, K, ep, s);
            return launch_lds<T, EPI, 128, 128, 2, 4, 8, kDeepStages, 32>(A, lda, W, ldw, M, N, K, ep, s);
        case TILE_64x64: return launch_lds<T, EPI, 64, 64, 2, 2, 8, 3, 32>(A, lda, W, ldw, M, N, K, ep, s);
        default: break;
        }
    }
    // register-staged kernel: 64 x 64 tiles when 128 x 128 ones would leave
    // more than half of the CUs idle
    if (reg_small_tiles(M, N)) {
        if (fast) return launch_t<T, EPI, 64, true>(A, lda, W, ldw, M, N, K, ep, s);
        return launch_t<T, EPI, 64, false>(A, lda, W, ldw, M, N, K, ep, s);
    }
    if (fast) return launch_t<T, EPI, 128, true>(A, lda, W, ldw, M, N, K, ep, s);
    return launch_t<T, EPI, 128, false>(A, lda, W, ldw, M, N, K, ep, s);
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

int64_t gemm_splitk_floats(int dtype, int epi, int M, int N, int K, bool wq) {
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    int bm, nk, per_cu, min_steps;
    if (dtype != DT_F32 && (K % 64 == 0 || wq)) {
        nk = K / 64;
        switch (pick_tile(M, N, true, false)) {
        case TILE_256x256: bm = 256; per_cu = lds_per_cu(256, 8, 2); break;
        case TILE_128x128: bm = 128; per_cu = lds_per_cu(128, 8, 2); break;
        case TILE_128x128_DEEP:
            bm = 128;
            if (K % 128 == 0 && !wq) {
                per_cu = lds_per_cu(128, 16, 2);
                nk = K / 128;
            } else {
                per_cu = lds_per_cu(128, 8, kDeepStages);
            }
            break;
        default: bm = 64; per_cu = lds_per_cu(64, 8, 3); break;
        }
        min_steps = kLdsMinSteps;
    } else {
        bm = reg_small_tiles(M, N) ? 64 : 128;
        nk = (int)cdiv(K, dtype == DT_F32 ? 32 : 64);
        per_cu = kRegPerCU;
        min_steps = kRegMinSteps;
    }
    const int64_t tiles = cdiv(M, bm) * cdiv(N, bm);
    const int S = splits_for(epi, tiles, nk, per_cu, min_steps, M, N, K);
    return S > 1 ? (int64_t)S * M * N : 0;
}

namespace {
// launch_gemm_rows: one wave per output column.  Its lanes read the
// column's weight row in 16-byte chunks, 8 chunks per lane in flight at once
// (1 KB of contiguous weights per load instruction; K = 4096 is one round),
// with the same chunks of each A row; the wave sum goes to the epilogue.
// Chunks past K read as zero (buffer range check), so there is no tail.
constexpr int kRowsWaves = 4, kRowsUnroll = 8;
__device__ __forceinline__ Chunk buf_chunk(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(Chunk, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
template <typename T, int EPI>
__global__ __launch_bounds__(64 * kRowsWaves) void gemm_rows_kernel(const T *__restrict__ A, int64_t lda,
                                                                     const T *__restrict__ W, int64_t ldw, int R,
                                                                     int N, int K, EpiArgs ep) {
    constexpr int KPC = Elem<T>::kPerChunk;
    const int lane = threadIdx.x & 63;
    const int n = blockIdx.x * kRowsWaves + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    if (n >= N) return;
    const uint32_t rowb = (uint32_t)(K / KPC) * 16u;
    const __amdgpu_buffer_rsrc_t rw = buf_rsrc(W + (int64_t)n * ldw, rowb);
    float acc[kGemmRowsMax];
#pragma unroll
    for (int r = 0; r < kGemmRowsMax; ++r) acc[r] = 0.0f;
    for (int c0 = 0; c0 < K / KPC; c0 += 64 * kRowsUnroll) {
        Chunk wc[kRowsUnroll];
#pragma unroll
        for (int u = 0; u < kRowsUnroll; ++u) wc[u] = buf_chunk(rw, (uint32_t)(c0 + lane + 64 * u) * 16u);
#pragma unroll
        for (int r = 0; r < kGemmRowsMax; ++r) {
            if (r >= R) break;
            const __amdgpu_buffer_rsrc_t ra = buf_rsrc(A + r * lda, rowb);
            Chunk ac[kRowsUnroll];
#pragma unroll
            for (int u = 0; u < kRowsUnroll; ++u) ac[u] = buf_chunk(ra, (uint32_t)(c0 + lane + 64 * u) * 16u);
#pragma unroll
            for (int u = 0; u < kRowsUnroll; ++u) {
                const T *we = reinterpret_cast<const T *>(&wc[u]), *ae = reinterpret_cast<const T *>(&ac[u]);
#pragma unroll
                for (int e = 0; e < KPC; ++e) acc[r] = fmaf(to_f32(ae[e]), to_f32(we[e]), acc[r]);
            }
        }
    }
    const float bias = ep.bias ? ep.bias[n] : 0.0f;
    const float ls = EPI == EPI_RESID && ep.ls ? ep.ls[n] : 1.0f;
    for (int r = 0; r < R; ++r) {
        const float v0 = wave_sum(acc[r]) + bias;
        if (lane != 0) continue;
        if constexpr (EPI == EPI_STORE || EPI == EPI_GELU) {
            const float v = EPI == EPI_GELU ? gelu_erf(v0) : v0;
            reinterpret_cast<T *>(ep.out)[(int64_t)r * ep.ldo + n] = from_f32<T>(v);
        } else if constexpr (EPI == EPI_RESID) {
            ep.Z[(int64_t)r * ep.ldz + n] += ep.ls ? v0 * ls : v0;
        }
    }
}

template <typename T>
hipError_t launch_rows_t(int epi, const void *A, int64_t lda, const void *W, int64_t ldw, int R, int N, int K,
                         const EpiArgs &ep, hipStream_t s) {
    const dim3 grid((unsigned)cdiv(N, kRowsWaves)), block(64 * kRowsWaves);
    const T *a = reinterpret_cast<const T *>(A), *w = reinterpret_cast<const T *>(W);
    switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL((gemm_rows_kernel<T, EPI_STORE>), grid, block, 0, s, a, lda, w, ldw, R, N, K, ep); break;
    case EPI_GELU: hipLaunchKernelGGL((gemm_rows_kernel<T, EPI_GELU>), grid, block, 0, s, a, lda, w, ldw, R, N, K, ep); break;
    case EPI_RESID: hipLaunchKernelGGL((gemm_rows_kernel<T, EPI_RESID>), grid, block, 0, s, a, lda, w, ldw, R, N, K, ep); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
} // namespace

hipError_t launch_gemm_rows(int dtype, int epi, const void *A, int64_t lda, const void *W, int64_t ldw, int R,
                            int N, int K, const EpiArgs &ep, hipStream_t s) {
    if (R <= 0 || N <= 0) return hipSuccess;
    if (R > kGemmRowsMax || K % 8 != 0 || lda % 8 != 0 || ldw % 8 != 0 || ep.wscale || ep.kwrap ||
        (uintptr_t)A % 16 != 0 || (uintptr_t)W % 16 != 0)
        return hipErrorInvalidValue;
    switch (dtype) {
    case DT_BF16: return launch_rows_t<bf16_t>(epi, A, lda, W, ldw, R, N, K, ep, s);
    case DT_F16: return launch_rows_t<f16_t>(epi, A, lda, W, ldw, R, N, K, ep, s);
    }
    return hipErrorInvalidValue;
}

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
