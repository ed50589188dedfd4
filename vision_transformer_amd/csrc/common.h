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

// Range-checked loads through a buffer resource: bytes at or past `bytes`
// from the base (and everything, when the base is NULL) read as zero, with no
// branch.  Used for loads issued early and consumed much later: a load under a
// branch whose result lands in different registers on the two paths makes the
// compiler wait for it where the paths join.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, base ? bytes : 0u, 0x00020000);
}
__device__ __forceinline__ float buf_f32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ int buf_i32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return (int)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
// (the loaded vector is reinterpreted whole: taking the bits of one element
// expression of a vector with __builtin_bit_cast reads element 0 with this
// compiler)
__device__ __forceinline__ float2 buf_f32x2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const f32x2_t f = __builtin_bit_cast(f32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    return make_float2(f.x, f.y);
}
__device__ __forceinline__ float4 buf_f32x4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const f32x4 f = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    return make_float4(f.x, f.y, f.z, f.w);
}

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
// Butterfly reductions: at every step each lane combines its value with one
// partner whose own partner it is, so all 64 lanes end with the same result
// (the two operands of each step are the same pair).  Within a row of 16
// lanes the partners come from DPP (quad xor 1 and xor 2, then the 8- and
// 16-lane mirrors), across rows of a half from a swizzle (xor 16), and across
// the two halves from one permute (xor 32).  `id` fills inactive sources.
template <int CTRL> __device__ __forceinline__ float dpp_f32(float v, float id) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, id), __builtin_bit_cast(int, v),
                                                                 CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float swizzle_xor16(float v) {
    // bit mode: and_mask 0x1F, or_mask 0, xor_mask 0x10 (within 32 lanes)
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppRowMirror = 0x140, kDppHalfMirror = 0x141;
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f32<kDppXor1>(v, 0.0f);
    v += dpp_f32<kDppXor2>(v, 0.0f);
    v += dpp_f32<kDppHalfMirror>(v, 0.0f);
    v += dpp_f32<kDppRowMirror>(v, 0.0f);
    v += swizzle_xor16(v);
    return v + __shfl_xor(v, 32, 64);
}
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_f32<kDppXor1>(v, -INFINITY));
    v = fmaxf(v, dpp_f32<kDppXor2>(v, -INFINITY));
    v = fmaxf(v, dpp_f32<kDppHalfMirror>(v, -INFINITY));
    v = fmaxf(v, dpp_f32<kDppRowMirror>(v, -INFINITY));
    v = fmaxf(v, swizzle_xor16(v));
    return fmaxf(v, __shfl_xor(v, 32, 64));
}

// GELU(x) = x Phi(x), Phi(x) = (1 + erf(x / sqrt 2)) / 2, with erfc from the
// rational approximation 7.1.26 of Abramowitz & Stegun (Handbook of
// Mathematical Functions): erfc(z) = (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5)
// e^{-z^2}, t = 1 / (1 + p z), z >= 0, |error| <= 1.5e-7.  With z = |x| / sqrt 2
// and u = erfc(z) / 2 (the factor 1/2 folded into the coefficients),
// Phi(x) = 1 - u for x >= 0 and u for x < 0, so GELU(x) = max(x, 0) - |x| u
// in both cases: one FMA instead of a compare, a select and a subtraction.
__device__ __forceinline__ float gelu_erf(float x) {
    const float ax = fabsf(x);
    const float t = __builtin_amdgcn_rcpf(fmaf(ax, 0.3275911f * 0.70710678118654752440f, 1.0f));
    float h = fmaf(0.5f * 1.061405429f, t, 0.5f * -1.453152027f);
    h = fmaf(h, t, 0.5f * 1.421413741f);
    h = fmaf(h, t, 0.5f * -0.284496736f);
    h = fmaf(h, t, 0.5f * 0.254829592f);
    // e^{-x^2 / 2} = 2^{-x^2 log2(e) / 2}
    const float e = __builtin_amdgcn_exp2f((x * -0.72134752044448170368f) * x);
    const float u = (t * h) * e;
    return fmaf(-ax, u, fmaxf(x, 0.0f));
}

__host__ __device__ __forceinline__ int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
__host__ __device__ __forceinline__ int64_t cdiv(int64_t x, int64_t m) { return (x + m - 1) / m; }

} // namespace vitenc
