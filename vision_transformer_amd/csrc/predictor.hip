// Memory-bound steps of the masked-latent predictor that follows the encoder
// (SkyVision.cpp README, V-JEPA 2 backend notes, "masked-latent predictor";
// jepa.cpp "GGUF schema (v1)", "Predictor (jepa.pred.*)"): putting context and
// target tokens in position order, gathering encoder rows, and filling the
// target rows with a mask token.  The blocks themselves run on the encoder's
// kernels.
//
// Ids are validated on the host (strictly increasing per list, disjoint, in
// [0, n_grid)); the kernels clamp what they read so that ids breaking that
// contract give wrong values, never an out-of-bounds access.
#include "common.h"
#include "launch.h"

namespace vitenc {

namespace {

// number of entries of the sorted list v[0..n) below x
__device__ __forceinline__ int count_below(const int *__restrict__ v, int n, int x) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (v[mid] < x) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

// One thread per id of either list.  The position-order rank of context id j
// of an item is j plus the number of target ids below it (and symmetrically),
// which is a merge of the two sorted lists; every rank lies in [0, nc + nt)
// whatever the ids hold.
__global__ __launch_bounds__(256) void pred_order_kernel(const int *__restrict__ ctx, int nc,
                                                         const int *__restrict__ tgt, int nt, int B, int gh,
                                                         int gw, int n_grid, int *__restrict__ row_ctx,
                                                         int *__restrict__ row_tgt, int *__restrict__ tok_pos) {
    const int per = nc + nt;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)B * per) return;
    const int b = (int)(idx / per), j = (int)(idx - (int64_t)b * per);
    const bool is_ctx = j < nc;
    const int jj = is_ctx ? j : j - nc;
    const int *own = is_ctx ? ctx + (int64_t)b * nc : tgt + (int64_t)b * nt;
    const int *other = is_ctx ? tgt + (int64_t)b * nt : ctx + (int64_t)b * nc;
    const int id = own[jj];
    const int rank = jj + count_below(other, is_ctx ? nt : nc, id);
    const int row = b * per + rank;
    if (is_ctx) row_ctx[(int64_t)b * nc + jj] = row;
    else row_tgt[(int64_t)b * nt + jj] = row;
    const int p = min(max(id, 0), n_grid - 1);
    const int t = p / (gh * gw), h = (p / gw) % gh, w = p % gw;
    tok_pos[row] = t | (h << 10) | (w << 20);
}

// out[r, :] = src row of r, converted to T.  The source row is rows[r] when
// rows is set, else item r / per_item's row ids[r] (clamped to the item).
// SPLIT: the rounded value goes to columns [0, D) and what rounding left
// over to [lo_off, lo_off + D) of the out row (lo_off = D: a row of 2D
// columns; the levels of a concatenated row use the offset of its second half).  One workgroup per row, four columns per
// thread and step (VEC: 16-byte source loads, set when lds, D and src allow).
template <typename T, bool SPLIT, bool VEC>
__global__ __launch_bounds__(256) void gather_rows_kernel(const float *__restrict__ src, int64_t lds,
                                                          const int *__restrict__ rows, const int *__restrict__ ids,
                                                          int per_item, int src_rows, int D, T *__restrict__ out,
                                                          int64_t ldo, int64_t lo_off) {
    const int r = blockIdx.x;
    int64_t srow;
    if (rows) {
        srow = rows[r];
    } else {
        const int item = r / per_item;
        srow = (int64_t)item * src_rows + min(max(ids[r], 0), src_rows - 1);
    }
    const float *s = src + srow * lds;
    T *o = out + (int64_t)r * ldo;
    for (int c = 4 * threadIdx.x; c < D; c += 4 * blockDim.x) {
        float v[4];
        if constexpr (VEC) {
            const float4 q = *reinterpret_cast<const float4 *>(s + c);
            v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
        } else {
            for (int i = 0; i < 4; ++i) v[i] = c + i < D ? s[c + i] : 0.0f;
        }
        for (int i = 0; i < 4 && c + i < D; ++i) {
            const T h = from_f32<T>(v[i]);
            o[c + i] = h;
            if constexpr (SPLIT) o[lo_off + c + i] = from_f32<T>(v[i] - to_f32(h));
        }
    }
}

// Z row rows[r] = vec (+ add), one workgroup per row
__global__ __launch_bounds__(256) void fill_rows_kernel(const float *__restrict__ vec, const float *__restrict__ add,
                                                        const int *__restrict__ rows, int D, float *__restrict__ Z) {
    float *z = Z + (int64_t)rows[blockIdx.x] * D;
    for (int c = threadIdx.x; c < D; c += blockDim.x) z[c] = add ? vec[c] + add[c] : vec[c];
}

__global__ __launch_bounds__(256) void zero_kernel(float *__restrict__ x, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        x[i] = 0.0f;
}

template <typename T, bool SPLIT>
hipError_t launch_gather_t2(const float *src, int64_t lds, const int *rows, const int *ids, int per_item,
                            int src_rows, int R, int D, T *out, int64_t ldo, int64_t lo_off, hipStream_t s) {
    const bool vec = D % 4 == 0 && lds % 4 == 0 && reinterpret_cast<uintptr_t>(src) % 16 == 0;
    const unsigned threads = (unsigned)std::min<int64_t>(256, std::max<int64_t>(64, cdiv(D, 4) / 64 * 64));
    if (vec)
        hipLaunchKernelGGL((gather_rows_kernel<T, SPLIT, true>), dim3((unsigned)R), dim3(threads), 0, s, src, lds,
                           rows, ids, per_item, src_rows, D, out, ldo, lo_off);
    else
        hipLaunchKernelGGL((gather_rows_kernel<T, SPLIT, false>), dim3((unsigned)R), dim3(threads), 0, s, src, lds,
                           rows, ids, per_item, src_rows, D, out, ldo, lo_off);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_gather_t(const float *src, int64_t lds, const int *rows, const int *ids, int per_item,
                           int src_rows, int R, int D, bool split, T *out, int64_t ldo, int64_t lo_off,
                           hipStream_t s) {
    if (split) return launch_gather_t2<T, true>(src, lds, rows, ids, per_item, src_rows, R, D, out, ldo, lo_off, s);
    return launch_gather_t2<T, false>(src, lds, rows, ids, per_item, src_rows, R, D, out, ldo, lo_off, s);
}

} // namespace

hipError_t launch_pred_order(const int *ctx_ids, int nc, const int *tgt_ids, int nt, int B, int gt, int gh, int gw,
                             int *row_ctx, int *row_tgt, int *tok_pos, hipStream_t s) {
    const int64_t n = (int64_t)B * (nc + nt);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(pred_order_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, ctx_ids, nc, tgt_ids, nt, B,
                       gh, gw, gt * gh * gw, row_ctx, row_tgt, tok_pos);
    return hipGetLastError();
}

hipError_t launch_gather_rows(int out_dtype, const float *src, int64_t lds, const int *rows, const int *ids,
                              int per_item, int src_rows, int R, int D, bool split, void *out, int64_t ldo,
                              hipStream_t s, int64_t lo_off) {
    if (R == 0) return hipSuccess;
    if (lo_off < 0) lo_off = D;
    switch (out_dtype) {
    case DT_F32:
        if (split) return hipErrorInvalidValue;
        return launch_gather_t<float>(src, lds, rows, ids, per_item, src_rows, R, D, false,
                                      reinterpret_cast<float *>(out), ldo, lo_off, s);
    case DT_BF16:
        return launch_gather_t<bf16_t>(src, lds, rows, ids, per_item, src_rows, R, D, split,
                                       reinterpret_cast<bf16_t *>(out), ldo, lo_off, s);
    case DT_F16:
        return launch_gather_t<f16_t>(src, lds, rows, ids, per_item, src_rows, R, D, split,
                                      reinterpret_cast<f16_t *>(out), ldo, lo_off, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_fill_rows(const float *vec, const float *add, const int *rows, int R, int D, float *Z,
                            hipStream_t s) {
    if (R == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_rows_kernel, dim3((unsigned)R), dim3(256), 0, s, vec, add, rows, D, Z);
    return hipGetLastError();
}

hipError_t launch_zero(float *x, int64_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>(cdiv(n, 256), 4096);
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, n);
    return hipGetLastError();
}

} // namespace vitenc
