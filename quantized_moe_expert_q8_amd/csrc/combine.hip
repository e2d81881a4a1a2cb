// Weighted masked combine (lucebox PR #826, the routed combine commit: route
// weighting and route sum in one launch, rounding the products and the sums
// separately as the unfused ops do; the review of moe_combine_masked_kernel: a
// route masked to -1 is skipped before anything is read for it).
#include "moeq8_device.hpp"
#include "moeq8_host.hpp"

namespace moeq8 {

// Every load is issued before any is used: the slots' ids and weights
// (scalar loads), every slot's y value and the add term, so the combine
// waits for one round trip to memory.  A masked slot's y element (in bounds:
// y has a row for every route) is loaded but never used: the sum skips the
// slot by selection, so whatever that row holds (NaN, stale values) never
// reaches the output.
// add (nullable): the shared expert's output [ncols][n], added once after
// the routed sum; it may be out itself (each element is read, then written,
// by the same thread).
template <int KMAX>
__global__ void k_combine(const float* __restrict__ y, const int32_t* __restrict__ ids,
                          const float* __restrict__ w, int topk, int64_t n, const float* add,
                          float* out) {
    const int j = blockIdx.y;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    int id[KMAX];
    float wt[KMAX], yv[KMAX];
#pragma unroll
    for (int s = 0; s < KMAX; ++s) {
        const int r = j * topk + min(s, topk - 1);      // in range for every s
        const int idr = ids[r];                          // loaded for every s, then masked
        id[s] = s < topk ? idr : -1;
        wt[s] = w[r];
        yv[s] = y[(int64_t)r * n + i];
    }
    const float addv = add ? add[(int64_t)j * n + i] : 0.0f;
    float acc = 0.0f;  // +0 then the valid products in slot order
#pragma unroll
    for (int s = 0; s < KMAX; ++s) {
        const float sum = acc + wt[s] * yv[s];
        acc = id[s] >= 0 ? sum : acc;
    }
    if (add) acc = acc + addv;
    out[(int64_t)j * n + i] = acc;
}

}  // namespace moeq8

namespace {
int combine_call(const float* y, const int32_t* ids, const float* weights, int64_t ncols,
                 int32_t topk, int64_t n, const float* add, float* out, void* stream) {
    using namespace moeq8;
    if (!y || !ids || !weights || !out) return MOEQ8_EINVAL;
    if (ncols < 1 || ncols > MOEQ8_MAX_WIDE_COLS || topk < 1 || topk > MOEQ8_MAX_TOPK || n < 0)
        return MOEQ8_EINVAL;
    if (((uintptr_t)y | (uintptr_t)ids | (uintptr_t)weights | (uintptr_t)out | (uintptr_t)add) & 3u)
        return MOEQ8_EALIGN;
    if (n == 0) return MOEQ8_OK;
    const int64_t bx = (n + 255) / 256;
    if (bx > 0x7fffffff) return MOEQ8_EUNSUPPORTED;
    const dim3 grid((uint32_t)bx, (uint32_t)ncols);
    if (topk <= 8)
        hipLaunchKernelGGL(k_combine<8>, grid, dim3(256), 0, (hipStream_t)stream, y, ids, weights, topk, n,
                           add, out);
    else
        hipLaunchKernelGGL(k_combine<MOEQ8_MAX_TOPK>, grid, dim3(256), 0, (hipStream_t)stream, y, ids,
                           weights, topk, n, add, out);
    return check_launch();
}
}  // namespace

extern "C" int moe_combine(const float* y, const int32_t* ids, const float* weights, int64_t ncols,
                           int32_t topk, int64_t n, float* out, void* stream) {
    return combine_call(y, ids, weights, ncols, topk, n, nullptr, out, stream);
}

extern "C" int moe_combine_shared(const float* y, const int32_t* ids, const float* weights,
                                  int64_t ncols, int32_t topk, int64_t n, const float* shared_y,
                                  float* out, void* stream) {
    if (!shared_y) return MOEQ8_EINVAL;
    return combine_call(y, ids, weights, ncols, topk, n, shared_y, out, stream);
}
