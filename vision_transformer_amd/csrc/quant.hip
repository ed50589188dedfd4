// Quantisation of a weight matrix to the 8-bit block format the GEMMs read
// (the quantised matrices of jepa.cpp "GGUF schema (v1)", "Quantization
// rules": every 32 consecutive weights of a row share one scale).
//
// Format: a block's scale is 2^e with e the smallest integer such that the
// block's largest magnitude amax <= 448 * 2^e (clamped to [-117, 117]; an
// all-zero block takes -117), stored as the byte e + 127; each weight becomes
// the E4M3 code (sign, 4 exponent bits of bias 7, 3 mantissa bits, subnormals
// m/8 * 2^-6, largest magnitude 448) nearest to w / 2^e, ties to the even
// mantissa, with the sign bit of w.  Everything is integer arithmetic on the
// fp32 bit patterns, so the result is exact for every finite input.
//
// Layout: codes [rows, cols] row-major; scale bytes [cols/64][rows][2] (the
// two blocks of a 64-column slab of a row side by side, the rows of a slab
// contiguous, which is the order the GEMM stages them in).
#include "common.h"
#include "launch.h"

namespace vitenc {

namespace {

constexpr int kEMin = -117, kEMax = 117;

// e for a block whose largest magnitude has fp32 bit pattern abits (sign clear)
__device__ __forceinline__ int block_exponent(uint32_t abits) {
    const int ef = (int)(abits >> 23);
    if (ef == 0) return kEMin; // zero or below 2^-126: far under 448 * 2^-117
    // amax = f * 2^E with f = 1.m / 2 in [0.5, 1), E = ef - 126; 448 = 0.875 * 2^9
    const int e = ef - 126 - 9 + ((abits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    return min(max(e, kEMin), kEMax);
}

// E4M3 code of |x| / 2^e (x given by its fp32 bits), sign bit from x
__device__ __forceinline__ uint32_t e4m3_code(uint32_t xbits, int e) {
    const uint32_t sign = (xbits >> 31) << 7;
    const int ef = (int)((xbits >> 23) & 0xFF);
    uint32_t M = xbits & 0x7FFFFFu;
    int ex; // |x| = M * 2^ex
    if (ef == 0) {
        ex = -149;
    } else {
        M |= 0x800000u;
        ex = ef - 150;
    }
    if (M == 0) return sign;
    // a = |x| / 2^e = M * 2^(ex - e); its binade k = floor(log2 a)
    const int msb = 31 - __builtin_clz(M);
    const int k = msb + ex - e;
    const int kk = k < -6 ? -6 : k;      // subnormals share binade -6
    // units of the E4M3 spacing 2^(kk - 3): a / 2^(kk - 3) = M * 2^(ex - e - kk + 3)
    const int sh = ex - e - kk + 3;
    uint32_t units;
    if (sh >= 0) {
        units = M << sh; // M has at most 4 significant bits here (sh <= 3): exact
    } else if (-sh > 25) {
        units = 0;       // a < spacing / 4
    } else {
        const int r = -sh;
        const uint32_t q = M >> r, rem = M & ((1u << r) - 1u), half = 1u << (r - 1);
        units = q + ((rem > half || (rem == half && (q & 1u))) ? 1u : 0u); // ties to even
    }
    // units is in [8, 16] in a normal binade and in [0, 8] below 2^-6
    int kb = kk;
    if (units == 16) { // rounded up into the next binade
        units = 8;
        kb += 1;
    }
    uint32_t mag;
    if (units < 8) {
        mag = units; // subnormal (or zero): exponent field 0
    } else {
        const int efield = kb + 7;
        if (efield > 15 || (efield == 15 && units == 15)) mag = 0x7E; // above 448: saturate
        else mag = ((uint32_t)efield << 3) | (units - 8);
    }
    return sign | mag;
}

// One thread per 32-weight block.
__global__ __launch_bounds__(256) void mxfp8_quantize_kernel(const float *__restrict__ w, int rows, int cols,
                                                              uint8_t *__restrict__ codes,
                                                              uint8_t *__restrict__ scales) {
    const int nb = cols / 32;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)rows * nb) return;
    const int row = (int)(idx / nb), blk = (int)(idx - (int64_t)row * nb);
    const float4 *src = reinterpret_cast<const float4 *>(w + (int64_t)row * cols + 32 * blk);
    uint32_t xb[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 v = src[i];
        xb[4 * i] = __builtin_bit_cast(uint32_t, v.x);
        xb[4 * i + 1] = __builtin_bit_cast(uint32_t, v.y);
        xb[4 * i + 2] = __builtin_bit_cast(uint32_t, v.z);
        xb[4 * i + 3] = __builtin_bit_cast(uint32_t, v.w);
    }
    uint32_t amax = 0; // magnitudes compare as integers
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = max(amax, xb[i] & 0x7FFFFFFFu);
    const int e = block_exponent(amax);
    uint32_t out[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        out[i] = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) out[i] |= e4m3_code(xb[4 * i + j], e) << (8 * j);
    }
    uint4 *dst = reinterpret_cast<uint4 *>(codes + (int64_t)row * cols + 32 * blk);
    dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
    dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
    scales[(int64_t)(blk >> 1) * rows * 2 + 2 * row + (blk & 1)] = (uint8_t)(e + 127);
}

} // namespace

hipError_t launch_mxfp8_quantize(const float *w, int rows, int cols, uint8_t *codes, uint8_t *scales,
                                 hipStream_t s) {
    const int64_t n = (int64_t)rows * (cols / 32);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(mxfp8_quantize_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, w, rows, cols, codes,
                       scales);
    return hipGetLastError();
}

} // namespace vitenc
