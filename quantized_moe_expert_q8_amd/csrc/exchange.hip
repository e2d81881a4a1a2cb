// The 8-bit block exchange codec of the prefill partials (lucebox PR #826,
// the 8-bit prefill exchange commit): a partial is sent as blocks of 32 int8
// values with one f32 scale (1.125 bytes a value against 2 for bf16), the
// blocks of every rank are gathered, and every rank sums the ranks'
// dequantized values in rank order, so all ranks get the same result.  The
// gather itself crosses devices and is not here; these are the two HBM-bound
// kernels on either side of it.
//
// Block: {f32 d; int8 qs[32]} (36 bytes).  d = amax / 127 in fp32 (kept in
// fp32, not rounded to fp16), q = roundf(x / d) on the fp32 quotient; an
// all-zero block is all-zero bytes.  Decode: each rank's value is the fp32
// product d * q, and the values are added in fp32 in ascending rank order
// from +0 (no fused multiply-add: the product is rounded on its own).
//
// Both kernels give a block to 8 consecutive lanes, 4 values each, so a wave
// covers 8 blocks: 1 KB of fp32 read or written with 16-byte accesses and
// 288 contiguous bytes of blocks.
#include "moeq8_device.hpp"
#include "moeq8_host.hpp"

namespace moeq8 {
namespace {

constexpr int XB_BYTES = 36;
constexpr int LANES_PER_BLOCK = 8;
constexpr int EXCH_THREADS = 256;

template <bool VEC>
__global__ __launch_bounds__(EXCH_THREADS) void k_q8x_encode(const float* __restrict__ x, int64_t nblocks,
                                                            int64_t nbr, int64_t x_stride,
                                                            uint8_t* __restrict__ out) {
    const int64_t t = (int64_t)blockIdx.x * EXCH_THREADS + threadIdx.x;
    const int64_t b = t / LANES_PER_BLOCK;
    const int j = (int)(t % LANES_PER_BLOCK);
    const bool live = b < nblocks;
    float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (live) {
        const int64_t row = b / nbr, cb = b - row * nbr;
        const float* p = x + row * x_stride + cb * QK + 4 * j;
        if constexpr (VEC) {
            const float4 f = *reinterpret_cast<const float4*>(p);
            v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = p[i];
        }
    }
    // amax over the block's 8 lanes (max does not depend on the order)
    float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    amax = fmaxf(amax, __shfl_xor(amax, 4));
    if (!live) return;
    const float d = amax / 127.0f;
    uint32_t packed = 0u;
    if (d != 0.0f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = (int)roundf(v[i] / d);
            packed |= ((uint32_t)q & 0xffu) << (8 * i);
        }
    }
    uint32_t* o = reinterpret_cast<uint32_t*>(out + b * XB_BYTES);
    o[1 + j] = packed;
    if (j == 0) o[0] = __float_as_uint(d);
}

template <bool VEC>
__global__ __launch_bounds__(EXCH_THREADS) void k_q8x_decode_sum(const uint8_t* __restrict__ in, int nranks,
                                                                int64_t rank_stride, int64_t nblocks,
                                                                int64_t nbr, float* __restrict__ out,
                                                                int64_t out_stride) {
    const int64_t t = (int64_t)blockIdx.x * EXCH_THREADS + threadIdx.x;
    const int64_t b = t / LANES_PER_BLOCK;
    const int j = (int)(t % LANES_PER_BLOCK);
    if (b >= nblocks) return;
    const uint8_t* p = in + b * XB_BYTES;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
    for (int r = 0; r < nranks; ++r) {
        const uint32_t* blk = reinterpret_cast<const uint32_t*>(p + (int64_t)r * rank_stride);
        const float d = __uint_as_float(blk[0]);
        const uint32_t q4 = blk[1 + j];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float q = (float)(int8_t)(q4 >> (8 * i));
            acc[i] = acc[i] + materialize_f32(d * q);
        }
    }
    const int64_t row = b / nbr, cb = b - row * nbr;
    float* o = out + row * out_stride + cb * QK + 4 * j;
    if constexpr (VEC) {
        *reinterpret_cast<float4*>(o) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = acc[i];
    }
}

int64_t grid_for(int64_t nblocks) {
    return (nblocks * LANES_PER_BLOCK + EXCH_THREADS - 1) / EXCH_THREADS;
}

}  // namespace
}  // namespace moeq8

using namespace moeq8;

extern "C" int q8_block_encode(const float* x, int64_t rows, int64_t n, int64_t x_stride, void* blocks,
                               void* stream) {
    if (rows < 0 || n <= 0 || n % QK != 0 || x_stride < n) return MOEQ8_EINVAL;
    if (rows > 0 && (!x || !blocks)) return MOEQ8_EINVAL;
    if (((uintptr_t)x & 3u) || ((uintptr_t)blocks & 3u)) return MOEQ8_EALIGN;
    if (rows == 0) return MOEQ8_OK;
    const int64_t nbr = n / QK, nblocks = rows * nbr;
    const int64_t grid = grid_for(nblocks);
    if (grid > 0x7fffffff) return MOEQ8_EUNSUPPORTED;
    const bool vec = ((uintptr_t)x & 15u) == 0 && x_stride % 4 == 0;
    if (vec)
        hipLaunchKernelGGL(k_q8x_encode<true>, dim3((uint32_t)grid), dim3(EXCH_THREADS), 0, (hipStream_t)stream,
                           x, nblocks, nbr, x_stride, (uint8_t*)blocks);
    else
        hipLaunchKernelGGL(k_q8x_encode<false>, dim3((uint32_t)grid), dim3(EXCH_THREADS), 0, (hipStream_t)stream,
                           x, nblocks, nbr, x_stride, (uint8_t*)blocks);
    return check_launch();
}

extern "C" int q8_block_decode_sum(const void* gathered, int32_t nranks, int64_t rank_stride_bytes, int64_t rows,
                                   int64_t n, float* out, int64_t out_stride, void* stream) {
    if (rows < 0 || n <= 0 || n % QK != 0 || out_stride < n) return MOEQ8_EINVAL;
    if (nranks < 1 || nranks > MOEQ8_MAX_EXCHANGE_RANKS) return MOEQ8_EINVAL;
    const int64_t nbr = n / QK, nblocks = rows * nbr;
    if (nranks > 1 && rank_stride_bytes < nblocks * XB_BYTES) return MOEQ8_EINVAL;
    if (rows > 0 && (!gathered || !out)) return MOEQ8_EINVAL;
    if (((uintptr_t)gathered & 3u) || (rank_stride_bytes & 3) || ((uintptr_t)out & 3u)) return MOEQ8_EALIGN;
    if (rows == 0) return MOEQ8_OK;
    const int64_t grid = grid_for(nblocks);
    if (grid > 0x7fffffff) return MOEQ8_EUNSUPPORTED;
    const bool vec = ((uintptr_t)out & 15u) == 0 && out_stride % 4 == 0;
    if (vec)
        hipLaunchKernelGGL(k_q8x_decode_sum<true>, dim3((uint32_t)grid), dim3(EXCH_THREADS), 0,
                           (hipStream_t)stream, (const uint8_t*)gathered, (int)nranks, rank_stride_bytes,
                           nblocks, nbr, out, out_stride);
    else
        hipLaunchKernelGGL(k_q8x_decode_sum<false>, dim3((uint32_t)grid), dim3(EXCH_THREADS), 0,
                           (hipStream_t)stream, (const uint8_t*)gathered, (int)nranks, rank_stride_bytes,
                           nblocks, nbr, out, out_stride);
    return check_launch();
}
