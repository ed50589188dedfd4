// Device-side building blocks shared by the gfx950 kernels: element types,
// 16-byte vector loads, conversions and the MFMA tiles the kernels use.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vitenc {

typedef __bf16 bf16_t;
typedef _Float16 f16_t;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// 16 bytes of operand data; reinterpreted as 8 x 16-bit or 4 x fp32.
struct alignas(16) Chunk {
    uint32_t w[4];
};

template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr int kPerChunk = 4;     // elements per 16-byte chunk
    static constexpr int kMfmaPerChunk = 4; // 32x32x2 f32 MFMAs consuming one chunk per lane
};
template <> struct Elem<bf16_t> {
    static constexpr int kPerChunk = 8;
    static constexpr int kMfmaPerChunk = 1; // one 32x32x16 bf16 MFMA
};
template <> struct Elem<f16_t> {
    static constexpr int kPerChunk = 8;
    static constexpr int kMfmaPerChunk = 1; // one 32x32x16 f16 MFMA
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return (float)x; }
__device__ __forceinline__ float to_f32(f16_t x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// fp32 -> bf16, round to nearest even (the hardware conversion on gfx950)
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return (bf16_t)x; }
template <> __device__ __forceinline__ f16_t from_f32<f16_t>(float x) { return (f16_t)x; }

// 16-bit payload of an element (for packing two halves into one dword)
__device__ __forceinline__ uint32_t bits16(bf16_t x) { return __builtin_bit_cast(uint16_t, x); }
__device__ __forceinline__ uint32_t bits16(f16_t x) { return __builtin_bit_cast(uint16_t, x); }

// two fp32 values -> one dword of two 16-bit values (a in the low half), with
// one packed hardware conversion (round to nearest even)
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
template <typename T> __device__ __forceinline__ uint32_t pack2(float a, float b);
template <> __device__ __forceinline__ uint32_t pack2<bf16_t>(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
}
template <> __device__ __forceinline__ uint32_t pack2<f16_t>(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), f16x2_t));
}

__device__ __forceinline__ Chunk load_chunk(const void *p) {
    return *reinterpret_cast<const Chunk *>(p);
}
__device__ __forceinline__ void store_chunk(void *p, const Chunk &c) {
    *reinterpret_cast<Chunk *>(p) = c;
}
__device__ __forceinline__ Chunk zero_chunk() {
    Chunk c;
    c.w[0] = c.w[1] = c.w[2] = c.w[3] = 0u;
    return c;
}

// ----------------------------------------------------------------------------
// 32x32 MFMA tiles.  Operand layout (one 64-lane wave): lane l supplies row
// (l % 32) of A / column (l % 32) of B, and the k-slice owned by lane group
// g = l / 32.  The accumulator holds, in lane l, column (l % 32) and rows
//   8*(i/4) + 4*g + (i%4),  i = 0..15.
// mfma_chunk() consumes one 16-byte chunk per lane: for 16-bit types that is
// one 32x32x16 MFMA (the chunk is the lane group's 8 k values); for fp32 it
// is four 32x32x2 MFMAs, MFMA j taking element j of every lane's chunk.  In
// both cases the k values a lane group contributes are the same for A and B,
// so any assignment of actual k indices to chunks is a valid contraction as
// long as the A and B lanes of one group read the same k indices.
// ----------------------------------------------------------------------------
template <typename T> __device__ __forceinline__ void mfma_chunk(f32x16 &acc, const Chunk &a, const Chunk &b);

template <> __device__ __forceinline__ void mfma_chunk<bf16_t>(f32x16 &acc, const Chunk &a, const Chunk &b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                  acc, 0, 0, 0);
}
template <> __device__ __forceinline__ void mfma_chunk<f16_t>(f32x16 &acc, const Chunk &a, const Chunk &b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                 acc, 0, 0, 0);
}
template <> __device__ __forceinline__ void mfma_chunk<float>(f32x16 &acc, const Chunk &a, const Chunk &b) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__builtin_bit_cast(float, a.w[j]),
                                                   __builtin_bit_cast(float, b.w[j]), acc, 0, 0, 0);
}

// XOR swizzle of the 16-byte chunk index of an LDS row of 8 chunks (128 B).
// Operand fetches read one chunk per lane from 32 consecutive rows; the LDS
// serves a 128-bit read per group of lanes covering 128 or 256 bytes of
// banks, i.e. 8 or 16 consecutive rows.  With this swizzle any 8 consecutive
// rows use 8 distinct chunk slots, and any 16 consecutive rows use 16
// distinct (row parity, slot) pairs, so both groupings are conflict-free.
__device__ __forceinline__ int swz8(int row) { return (row & 7) ^ ((row >> 3) & 1); }
// the same property for rows of 4 chunks (64 B) and of 16 chunks (256 B)
__device__ __forceinline__ int swz4(int row) { return ((row >> 1) & 3) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int swz16(int row) { return row & 15; }
template <int NCH> __device__ __forceinline__ int swz(int row) {
    static_assert(NCH == 4 || NCH == 8 || NCH == 16, "row of 4, 8 or 16 chunks");
    if constexpr (NCH == 4) return swz4(row);
    else if constexpr (NCH == 8) return swz8(row);
    else return swz16(row);
}

// LDS destination of the direct global -> LDS buffer loads
typedef __attribute__((address_space(3))) void lds_void_t;

// Wait until at most N of this wave's vector memory operations are still in
// flight (the direct-to-LDS loads retire in issue order).
template <int N> __device__ __forceinline__ void vm_wait() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// 16x16x32 MFMA tiles (16-bit types): lane l supplies row (l % 16) of A /
// column (l % 16) of B and the 8 k values of lane group q = l / 16 (one
// 16-byte chunk); the accumulator holds, in lane l, column (l % 16) and rows
// 4*q + i, i = 0..3.
template <typename T> __device__ __forceinline__ void mfma16_chunk(f32x4 &acc, const Chunk &a, const Chunk &b);
template <> __device__ __forceinline__ void mfma16_chunk<bf16_t>(f32x4 &acc, const Chunk &a, const Chunk &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                  acc, 0, 0, 0);
}
template <> __device__ __forceinline__ void mfma16_chunk<f16_t>(f32x4 &acc, const Chunk &a, const Chunk &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), acc,
                                                 0, 0, 0);
}

// accumulator row owned by lane group g for accumulator slot i
__device__ __forceinline__ int acc_row(int i, int g) { return 8 * (i >> 2) + 4 * g + (i & 3); }

// ----------------------------------------------------------------------------
// wave-level reductions (64 lanes)
// ----------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// GELU(x) = x/2 (1 + erf(x / sqrt 2)), with erf from the rational
// approximation 7.1.26 of Abramowitz & Stegun (Handbook of Mathematical
// Functions): erf(z) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) e^{-z^2},
// t = 1 / (1 + p z), z >= 0, |error| <= 1.5e-7, and erf(-z) = -erf(z).
__device__ __forceinline__ float gelu_erf(float x) {
    const float z = fabsf(x) * 0.70710678118654752440f;
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.0f));
    float poly = fmaf(1.061405429f, t, -1.453152027f);
    poly = fmaf(poly, t, 1.421413741f);
    poly = fmaf(poly, t, -0.284496736f);
    poly = fmaf(poly, t, 0.254829592f);
    poly *= t;
    const float e = __builtin_amdgcn_exp2f(-z * z * 1.4426950408889634f);
    const float erf_abs = fmaf(-poly, e, 1.0f);
    const float erf = x < 0.0f ? -erf_abs : erf_abs;
    return 0.5f * x * (1.0f + erf);
}

__host__ __device__ __forceinline__ int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
__host__ __device__ __forceinline__ int64_t cdiv(int64_t x, int64_t m) { return (x + m - 1) / m; }

} // namespace vitenc
