// vitenc_op_attention_noalloc (include/vitenc.h): the attention step for
// callers that cannot allocate device memory.  vitenc_op_attention keeps the
// partial results of rows or query tiles split over their keys in a scratch
// buffer the caller passes; this entry point keeps them in `scratch`, a
// fixed device array of this library instead, so the caller passes inputs
// and outputs only and the call allocates nothing.  The kernels are the same.
//
// Each device holds its own copy of the array (it lives as long as the
// process).  Host code must not pass the array's name to a kernel: on the
// host it is a stand-in symbol, not a device address.  The device address is
// looked up once per device, with that device current, on the first call
// there, and kept in g_scratch_ptr.
#include "vitenc.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

static __device__ __align__(256) float scratch[VITENC_NOALLOC_SCRATCH_FLOATS];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float *g_scratch_ptr[kMaxDevices] = {};

// the current device's address of `scratch` (NULL and a refusal message on
// failure)
float *device_scratch(vitenc_status &st) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        st = vitenc::device_status(e, "hipGetDevice");
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        st = vitenc::fail(VITENC_EUNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            st = vitenc::device_status(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
            return nullptr;
        }
        g_scratch_ptr[dev] = static_cast<float *>(p);
    }
    st = VITENC_OK;
    return g_scratch_ptr[dev];
}

} // namespace

extern "C" {

vitenc_status vitenc_op_attention_noalloc(int32_t dtype, const void *Q, const void *K, const void *Vt, int32_t B,
                                          int32_t N, int32_t n_head, int32_t head_dim, int32_t attn_mode,
                                          int32_t n_prefix, int32_t tokens_per_frame, void *O, void *stream) {
    vitenc::clear_error();
    if (dtype != VITENC_F32 && dtype != VITENC_BF16 && dtype != VITENC_F16)
        return vitenc::fail(VITENC_EINVAL, "unknown dtype %d", dtype);
    if (!Q || !K || !Vt || !O) return vitenc::fail(VITENC_ENULL, "a required pointer is NULL");
    if (B <= 0 || N <= 0 || n_head <= 0) return vitenc::fail(VITENC_ESHAPE, "bad sizes");
    if (head_dim != 64 && head_dim != 32) return vitenc::fail(VITENC_EUNSUPPORTED, "head_dim %d", head_dim);
    if (n_prefix < 0 || n_prefix >= N) return vitenc::fail(VITENC_ESHAPE, "n_prefix %d outside [0, N)", n_prefix);
    if (attn_mode != VITENC_ATTN_FULL && attn_mode != VITENC_ATTN_BLOCK_CAUSAL)
        return vitenc::fail(VITENC_EINVAL, "unknown attn_mode %d", attn_mode);
    if (attn_mode == VITENC_ATTN_BLOCK_CAUSAL && tokens_per_frame <= 0)
        return vitenc::fail(VITENC_ESHAPE, "block-causal geometry");
    const int64_t need =
        vitenc::attention_scratch_floats(dtype, B, N, n_head, head_dim, attn_mode, n_prefix, tokens_per_frame);
    if (need > VITENC_NOALLOC_SCRATCH_FLOATS)
        return vitenc::fail(VITENC_EUNSUPPORTED,
                            "this call needs %lld floats of scratch; the fixed array holds %lld (use "
                            "vitenc_op_attention with a caller scratch)",
                            (long long)need, (long long)VITENC_NOALLOC_SCRATCH_FLOATS);
    float *ptr = nullptr;
    if (need > 0) {
        vitenc_status st;
        ptr = device_scratch(st);
        if (!ptr) return st;
    }
    return vitenc::device_status(vitenc::launch_attention(dtype, Q, K, Vt, B, N, n_head, head_dim, (N + 63) / 64 * 64,
                                                          attn_mode, n_prefix, tokens_per_frame, ptr, O,
                                                          reinterpret_cast<hipStream_t>(stream)),
                                 "attention");
}

} // extern "C"
