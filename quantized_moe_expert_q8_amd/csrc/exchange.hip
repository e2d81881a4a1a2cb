// The 8-bit block exchange codec of the prefill partials (lucebox PR #826,
// the 8-bit prefill exchange commit): a partial is sent as blocks of 32 int8
// values with one f32 scale (1.125 bytes a value against 2 for bf16), all
// ranks' blocks are gathered, and the decode adds the per-rank fp32 products
// in ascending rank order from +0, which gives identical bits on every rank.
// The gather itself crosses devices and is not here; these are the two HBM-bound
// kernels on either side of it.
//
// Block: {f32 d; int8 qs[32]} (36 bytes).  d = amax / 127 in fp32 (kept in
// fp32, not rounded to fp16), q = roundf(x / d) on the fp32 quotient; an
// all-zero block is all-zero bytes.  Decode: each rank's value is the fp32
// product d * q, and the values are added in fp32 in ascending rank order
// from +0 (no fused multiply-add: the product is rounded on its own).
//
// Both kernels give a block to LPB consecutive lanes (32 / LPB values each),
// so a wave covers 64 / LPB blocks: contiguous fp32 read or written with
// 16-byte accesses and contiguous blocks.
#include "moeq8_device.hpp"
#include "moeq8_host.hpp"

namespace moeq8 {
namespace {

constexpr int XB_BYTES = 36;
constexpr int EXCH_THREADS = 256;
// Lanes per block, measured on an [8192 x 4096] partial: the encoder is
// fastest with 2 (16 values, four 16-byte loads a lane: 6.7 TB/s against 5.2
// with 8); the decoder with 8 for two ranks (6.9 TB/s) and with 4 for more
// (8 ranks: 5.2 TB/s against 4.0 with 8 lanes, whose lanes then wait on many
// 4-byte loads).
constexpr int ENC_LPB = 2;
constexpr int dec_lpb(int nranks) { return nranks <= 2 ? 8 : 4; }

typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2a4 __attribute__((ext_vector_type(2), aligned(4)));

// Code of x for the scale d: roundf of the fp32 quotient x / d, as the block
// rule defines it.  The quotient comes from the reciprocal (v_rcp_f32, within
// an ulp or so) and one multiply; its rounding to an integer can only differ
// from that of the correctly rounded quotient when it lies within a few ulps
// of a half-integer, and lanes there take the IEEE division.  |x / d| <= 127
// here (d = amax / 127), where an ulp is at most 2^-17; the margin is 2^-12.
__device__ __forceinline__ int block_code(float x, float d, float rd) {
    const float t = x * rd;
    const float a = fabsf(t);
    const bool near = !(fabsf((a - floorf(a)) - 0.5f) >= 0x1p-12f) || !(a < 256.0f);
    int q = (int)roundf(t);
    if (__builtin_expect(__ballot(near) != 0, 0)) {
        if (near) q = (int)roundf(x / d);
    }
    return q;
}

template <int LPB, bool VEC>
__global__ __launch_bounds__(EXCH_THREADS) void k_q8x_encode(const float* __restrict__ x, int64_t nblocks,
                                                            int64_t nbr, int64_t x_stride,
                                                            uint8_t* __restrict__ out) {
    constexpr int V = QK / LPB;                        // values per lane: 4, 8 or 16
    const int64_t t = (int64_t)blockIdx.x * EXCH_THREADS + threadIdx.x;
    const int64_t b = t / LPB;
    const int j = (int)(t % LPB);
    const bool live = b < nblocks;
    float v[V];
#pragma unroll
    for (int i = 0; i < V; ++i) v[i] = 0.0f;
    if (live) {
        const int64_t row = b / nbr, cb = b - row * nbr;
        const float* p = x + row * x_stride + cb * QK + V * j;
        if constexpr (VEC) {
#pragma unroll
            for (int i = 0; i < V / 4; ++i) {
                const float4 f = reinterpret_cast<const float4*>(p)[i];
                v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i) v[i] = p[i];
        }
    }
    // amax over the block's lanes (max does not depend on the order)
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < V; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
    for (int m = 1; m < LPB; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
    const float d = amax / 127.0f;
    const float rd = __builtin_amdgcn_rcpf(d);
    uint32_t packed[V / 4];
#pragma unroll
    for (int i = 0; i < V / 4; ++i) packed[i] = 0u;
    if (d != 0.0f) {
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const int q = block_code(v[i], d, rd);
            packed[i / 4] |= ((uint32_t)q & 0xffu) << (8 * (i % 4));
        }
    }
    if (!live) return;
    uint8_t* o = out + b * XB_BYTES;
    if constexpr (V == 4) {
        reinterpret_cast<uint32_t*>(o + 4)[j] = packed[0];
    } else if constexpr (V == 8) {
        reinterpret_cast<u32x2a4*>(o + 4)[j] = u32x2a4{packed[0], packed[1]};
    } else {
        reinterpret_cast<u32x4a4*>(o + 4)[j] = u32x4a4{packed[0], packed[1], packed[2], packed[3]};
    }
    if (j == 0) *reinterpret_cast<uint32_t*>(o) = __float_as_uint(d);
}

template <int LPB, bool VEC>
__global__ __launch_bounds__(EXCH_THREADS) void k_q8x_decode_sum(const uint8_t* __restrict__ in, int nranks,
                                                                int64_t rank_stride, int64_t nblocks,
                                                                int64_t nbr, float* __restrict__ out,
                                                                int64_t out_stride) {
    constexpr int V = QK / LPB;
    const int64_t t = (int64_t)blockIdx.x * EXCH_THREADS + threadIdx.x;
    const int64_t b = t / LPB;
    const int j = (int)(t % LPB);
    if (b >= nblocks) return;
    const uint8_t* p = in + b * XB_BYTES;
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.0f;
#pragma unroll 4
    for (int r = 0; r < nranks; ++r) {
        const uint8_t* blk = p + (int64_t)r * rank_stride;
        const float d = __uint_as_float(*reinterpret_cast<const uint32_t*>(blk));
        uint32_t q4[V / 4];
        if constexpr (V == 4) {
            q4[0] = reinterpret_cast<const uint32_t*>(blk + 4)[j];
        } else if constexpr (V == 8) {
            const u32x2a4 w = reinterpret_cast<const u32x2a4*>(blk + 4)[j];
            q4[0] = w.x; q4[1] = w.y;
        } else {
            const u32x4a4 w = reinterpret_cast<const u32x4a4*>(blk + 4)[j];
            q4[0] = w.x; q4[1] = w.y; q4[2] = w.z; q4[3] = w.w;
        }
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const float q = (float)(int8_t)(q4[i / 4] >> (8 * (i % 4)));
            acc[i] = acc[i] + materialize_f32(d * q);
        }
    }
    const int64_t row = b / nbr, cb = b - row * nbr;
    float* o = out + row * out_stride + cb * QK + V * j;
    if constexpr (VEC) {
#pragma unroll
        for (int i = 0; i < V / 4; ++i)
            reinterpret_cast<float4*>(o)[i] = make_float4(acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]);
    } else {
#pragma unroll
        for (int i = 0; i < V; ++i) o[i] = acc[i];
    }
}

int64_t grid_for(int64_t nblocks, int lpb) {
    return (nblocks * lpb + EXCH_THREADS - 1) / EXCH_THREADS;
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
    const int64_t grid = grid_for(nblocks, ENC_LPB);
    if (grid > 0x7fffffff) return MOEQ8_EUNSUPPORTED;
    const bool vec = ((uintptr_t)x & 15u) == 0 && x_stride % 4 == 0;
    if (vec)
        hipLaunchKernelGGL((k_q8x_encode<ENC_LPB, true>), dim3((uint32_t)grid), dim3(EXCH_THREADS), 0, (hipStream_t)stream,
                           x, nblocks, nbr, x_stride, (uint8_t*)blocks);
    else
        hipLaunchKernelGGL((k_q8x_encode<ENC_LPB, false>), dim3((uint32_t)grid), dim3(EXCH_THREADS), 0, (hipStream_t)stream,
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
    const int lpb = dec_lpb(nranks);
    const int64_t grid = grid_for(nblocks, lpb);
    if (grid > 0x7fffffff) return MOEQ8_EUNSUPPORTED;
    const bool vec = ((uintptr_t)out & 15u) == 0 && out_stride % 4 == 0;
    const hipStream_t hs = (hipStream_t)stream;
    const uint8_t* in = (const uint8_t*)gathered;
    const dim3 g((uint32_t)grid), blk(EXCH_THREADS);
    if (lpb == 8) {
        if (vec) hipLaunchKernelGGL((k_q8x_decode_sum<8, true>), g, blk, 0, hs, in, (int)nranks, rank_stride_bytes, nblocks, nbr, out, out_stride);
        else hipLaunchKernelGGL((k_q8x_decode_sum<8, false>), g, blk, 0, hs, in, (int)nranks, rank_stride_bytes, nblocks, nbr, out, out_stride);
    } else {
        if (vec) hipLaunchKernelGGL((k_q8x_decode_sum<4, true>), g, blk, 0, hs, in, (int)nranks, rank_stride_bytes, nblocks, nbr, out, out_stride);
        else hipLaunchKernelGGL((k_q8x_decode_sum<4, false>), g, blk, 0, hs, in, (int)nranks, rank_stride_bytes, nblocks, nbr, out, out_stride);
    }
    return check_launch();
}
