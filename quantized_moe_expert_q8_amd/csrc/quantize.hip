// q8_1 activation and Q8_0 weight quantisation (one thread per 32-value block).
//
// Block rule: fp32 d = amax / 127 (IEEE division), q = roundf(x / d) on the
// fp32 quotient (halves away from zero), d stored as fp16 (nearest even);
// q8_1 adds s = fp16(d * sum(q)) with the fp32 d.  An all-zero block is all
// zero bytes.  The pages (lucebox PR #826: the fused DS4.1 decode kernels and
// routed-combine commits) use q8_1 rows as the input every MMVQ reads and
// quantise an activation once for all its consumers.
#include "moeq8_device.hpp"
#include "moeq8_host.hpp"

namespace moeq8 {

template <bool Q81>
__global__ void k_quantize_rows(const float* __restrict__ x, int64_t n_rows, int64_t nb,
                                int64_t row_stride, uint8_t* __restrict__ out) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= n_rows * nb) return;
    const int64_t r = gid / nb;
    const int64_t b = gid - r * nb;
    const float* src = x + r * row_stride + b * QK;
    float v[QK];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < QK; ++i) {
        v[i] = src[i];
        amax = fmaxf(amax, fabsf(v[i]));
    }
    const float d = amax / 127.0f;
    uint32_t packed[QK / 4];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < QK / 4; ++i) packed[i] = 0u;
    if (d != 0.0f) {
#pragma unroll
        for (int i = 0; i < QK; ++i) {
            const int q = (int)roundf(v[i] / d);
            sum += q;
            packed[i / 4] |= ((uint32_t)q & 0xffu) << (8 * (i % 4));
        }
    }
    const uint32_t dbits = float_to_half_bits(d);
    if constexpr (Q81) {
        uint32_t* dst = reinterpret_cast<uint32_t*>(out + gid * Q81_BYTES);
        // s = fp16 of the fp32 product (two roundings, as defined)
        const uint32_t sbits = float_to_half_bits(materialize_f32(d * (float)sum));
        dst[0] = dbits | (sbits << 16);
#pragma unroll
        for (int i = 0; i < QK / 4; ++i) dst[1 + i] = packed[i];
    } else {
        uint16_t* dst = reinterpret_cast<uint16_t*>(out + gid * Q80_BYTES);
        dst[0] = (uint16_t)dbits;
#pragma unroll
        for (int i = 0; i < QK / 4; ++i) {
            dst[1 + 2 * i] = (uint16_t)(packed[i] & 0xffffu);
            dst[2 + 2 * i] = (uint16_t)(packed[i] >> 16);
        }
    }
}

namespace {
template <bool Q81>
int launch_quantize(const float* x, int64_t n_rows, int64_t k, int64_t stride, void* out,
                    void* stream) {
    if (!x || !out || n_rows < 0 || k <= 0 || (k % QK) != 0 || stride < k) return MOEQ8_EINVAL;
    if (((uintptr_t)x & 3u) || ((uintptr_t)out & (Q81 ? 3u : 1u))) return MOEQ8_EALIGN;
    const int64_t total = n_rows * (k / QK);
    if (total == 0) return MOEQ8_OK;
    const int64_t blocks = (total + 255) / 256;
    if (blocks > 0x7fffffff) return MOEQ8_EUNSUPPORTED;
    hipLaunchKernelGGL(k_quantize_rows<Q81>, dim3((uint32_t)blocks), dim3(256), 0,
                       (hipStream_t)stream, x, n_rows, k / QK, stride, (uint8_t*)out);
    return check_launch();
}
}  // namespace
}  // namespace moeq8

extern "C" int q8_1_quantize_rows(const float* x, int64_t n_rows, int64_t k, int64_t x_row_stride,
                                  void* xq, void* stream) {
    return moeq8::launch_quantize<true>(x, n_rows, k, x_row_stride, xq, stream);
}

extern "C" int q8_0_quantize_rows(const float* w, int64_t n_rows, int64_t k, int64_t w_row_stride,
                                  void* wq, void* stream) {
    return moeq8::launch_quantize<false>(w, n_rows, k, w_row_stride, wq, stream);
}
