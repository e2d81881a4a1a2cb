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
    quantize_block<Q81>(x + r * row_stride + b * QK, out + gid * (Q81 ? Q81_BYTES : Q80_BYTES));
}

__global__ void k_quantize_rows_q4(const float* __restrict__ x, int64_t n_rows, int64_t nb,
                                   int64_t row_stride, uint8_t* __restrict__ out) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= n_rows * nb) return;
    const int64_t r = gid / nb;
    const int64_t b = gid - r * nb;
    quantize_block_q4(x + r * row_stride + b * QK, out + gid * Q4_BYTES);
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

// 4-bit weight blocks (Q4: fp16 d = amax / 7, 32 codes of 4 bits), for
// bandwidth-only expert weights.
extern "C" int q4_quantize_rows(const float* w, int64_t n_rows, int64_t k, int64_t w_row_stride,
                                void* wq, void* stream) {
    using namespace moeq8;
    if (!w || !wq || n_rows < 0 || k <= 0 || (k % QK) != 0 || w_row_stride < k) return MOEQ8_EINVAL;
    if (((uintptr_t)w & 3u) || ((uintptr_t)wq & 1u)) return MOEQ8_EALIGN;
    const int64_t total = n_rows * (k / QK);
    if (total == 0) return MOEQ8_OK;
    const int64_t blocks = (total + 255) / 256;
    if (blocks > 0x7fffffff) return MOEQ8_EUNSUPPORTED;
    hipLaunchKernelGGL(k_quantize_rows_q4, dim3((uint32_t)blocks), dim3(256), 0, (hipStream_t)stream, w,
                       n_rows, k / QK, w_row_stride, (uint8_t*)wq);
    return check_launch();
}

// Repack Q8_0 rows into the 64-chunk packed layout (P64, moeq8_device.hpp):
// one thread per destination dword.
namespace {
__global__ void k_pack64(const uint32_t* __restrict__ src, int64_t n_rows, int64_t segs,
                         int64_t src_stride_dw, uint32_t* __restrict__ dst, int64_t dst_stride_dw) {
    using namespace moeq8;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per_row = segs * P64_SEGMENT_DWORDS;
    if (t >= n_rows * per_row) return;
    const int64_t row = t / per_row;
    const int64_t rem = t - row * per_row;
    const int64_t seg = rem / P64_SEGMENT_DWORDS;
    const int p = (int)(rem - seg * P64_SEGMENT_DWORDS);
    dst[row * dst_stride_dw + seg * P64_SEGMENT_DWORDS + p] =
        src[row * src_stride_dw + seg * P64_SEGMENT_DWORDS + p64_source_dword(p)];
}
}  // namespace

extern "C" int q8_0_pack64_rows(const void* src, int64_t n_rows, int64_t k, int64_t src_row_stride_bytes,
                                void* dst, int64_t dst_row_stride_bytes, void* stream) {
    using namespace moeq8;
    if (!src || !dst || n_rows < 0 || k <= 0 || k % (P64_CHUNKS * 2 * QK) != 0) return MOEQ8_EINVAL;
    const int64_t row_bytes = k / QK * Q80_BYTES;
    if (src_row_stride_bytes < row_bytes || dst_row_stride_bytes < row_bytes) return MOEQ8_EINVAL;
    if (((uintptr_t)src | (uintptr_t)dst | (uint64_t)src_row_stride_bytes | (uint64_t)dst_row_stride_bytes) & 3u)
        return MOEQ8_EALIGN;
    const uint8_t* s8 = (const uint8_t*)src;
    const uint8_t* d8 = (const uint8_t*)dst;
    const int64_t span_s = n_rows == 0 ? 0 : (n_rows - 1) * src_row_stride_bytes + row_bytes;
    const int64_t span_d = n_rows == 0 ? 0 : (n_rows - 1) * dst_row_stride_bytes + row_bytes;
    if (s8 < d8 + span_d && d8 < s8 + span_s) return MOEQ8_EINVAL;     // no overlap (not in place)
    const int64_t total = n_rows * (row_bytes / 4);
    if (total == 0) return MOEQ8_OK;
    const int64_t blocks = (total + 255) / 256;
    if (blocks > 0x7fffffff) return MOEQ8_EUNSUPPORTED;
    hipLaunchKernelGGL(k_pack64, dim3((uint32_t)blocks), dim3(256), 0, (hipStream_t)stream,
                       (const uint32_t*)src, n_rows, k / (P64_CHUNKS * 2 * QK), src_row_stride_bytes / 4,
                       (uint32_t*)dst, dst_row_stride_bytes / 4);
    return check_launch();
}

// Repack 4-bit rows into their 64-chunk packed layout (moeq8_device.hpp):
// one thread per destination dword.
namespace {
__global__ void k_pack64_q4(const uint32_t* __restrict__ src, int64_t n_rows, int64_t segs,
                            int64_t src_stride_dw, uint32_t* __restrict__ dst, int64_t dst_stride_dw) {
    using namespace moeq8;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per_row = segs * P64Q4_SEGMENT_DWORDS;
    if (t >= n_rows * per_row) return;
    const int64_t row = t / per_row;
    const int64_t rem = t - row * per_row;
    const int64_t seg = rem / P64Q4_SEGMENT_DWORDS;
    const int p = (int)(rem - seg * P64Q4_SEGMENT_DWORDS);
    dst[row * dst_stride_dw + seg * P64Q4_SEGMENT_DWORDS + p] =
        src[row * src_stride_dw + seg * P64Q4_SEGMENT_DWORDS + p64q4_source_dword(p)];
}
}  // namespace

extern "C" int q4_pack64_rows(const void* src, int64_t n_rows, int64_t k, int64_t src_row_stride_bytes,
                              void* dst, int64_t dst_row_stride_bytes, void* stream) {
    using namespace moeq8;
    if (!src || !dst || n_rows < 0 || k <= 0 || k % (P64_CHUNKS * 2 * QK) != 0) return MOEQ8_EINVAL;
    const int64_t row_bytes = k / QK * Q4_BYTES;
    if (src_row_stride_bytes < row_bytes || dst_row_stride_bytes < row_bytes) return MOEQ8_EINVAL;
    if (((uintptr_t)src | (uintptr_t)dst | (uint64_t)src_row_stride_bytes | (uint64_t)dst_row_stride_bytes) & 3u)
        return MOEQ8_EALIGN;
    const uint8_t* s8 = (const uint8_t*)src;
    const uint8_t* d8 = (const uint8_t*)dst;
    const int64_t span_s = n_rows == 0 ? 0 : (n_rows - 1) * src_row_stride_bytes + row_bytes;
    const int64_t span_d = n_rows == 0 ? 0 : (n_rows - 1) * dst_row_stride_bytes + row_bytes;
    if (s8 < d8 + span_d && d8 < s8 + span_s) return MOEQ8_EINVAL;     // no overlap (not in place)
    const int64_t total = n_rows * (row_bytes / 4);
    if (total == 0) return MOEQ8_OK;
    const int64_t blocks = (total + 255) / 256;
    if (blocks > 0x7fffffff) return MOEQ8_EUNSUPPORTED;
    hipLaunchKernelGGL(k_pack64_q4, dim3((uint32_t)blocks), dim3(256), 0, (hipStream_t)stream,
                       (const uint32_t*)src, n_rows, k / (P64_CHUNKS * 2 * QK), src_row_stride_bytes / 4,
                       (uint32_t*)dst, dst_row_stride_bytes / 4);
    return check_launch();
}

// Repack Q8_0 rows into the grouped GEMM's layout (q8_0_pack_gemm_rows in
// moeq8.h): each 272-byte group of 8 blocks becomes 16 bytes of scales, then
// the 8 blocks' quants 8-byte aligned, with the 8-byte halves of each 16-byte
// quant piece swapped in rows i % 16 >= 8.  One thread per destination dword;
// the four bytes of a dword come from one region and one 8-byte half.
namespace {
constexpr int G8_GROUP_BYTES = 8 * 34;                // 272
constexpr int G8_GROUP_DWORDS = G8_GROUP_BYTES / 4;   // 68
__global__ void k_pack_gemm(const uint8_t* __restrict__ src, int64_t n_rows, int64_t groups,
                            int64_t src_stride, uint32_t* __restrict__ dst, int64_t dst_stride_dw) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per_row = groups * G8_GROUP_DWORDS;
    if (t >= n_rows * per_row) return;
    const int64_t row = t / per_row;
    const int64_t rem = t - row * per_row;
    const int64_t grp = rem / G8_GROUP_DWORDS;
    const int o = (int)(rem - grp * G8_GROUP_DWORDS) * 4;      // byte of the group
    const uint8_t* g = src + row * src_stride + grp * G8_GROUP_BYTES;
    int from;                                                   // source byte of byte o
    if (o < 16) {
        from = 34 * (o >> 1);                                   // scale of block o / 2 (o even)
    } else {
        const int qo = o - 16;
        const int b = (qo & 31) ^ ((row & 15) >= 8 ? 8 : 0);
        from = 34 * (qo >> 5) + 2 + b;
    }
    uint32_t v;
    if (o < 16)   // two scales: bytes 0-1 of block o/2 and of block o/2 + 1
        v = (uint32_t)g[from] | ((uint32_t)g[from + 1] << 8) | ((uint32_t)g[from + 34] << 16) |
            ((uint32_t)g[from + 35] << 24);
    else
        v = (uint32_t)g[from] | ((uint32_t)g[from + 1] << 8) | ((uint32_t)g[from + 2] << 16) |
            ((uint32_t)g[from + 3] << 24);
    dst[row * dst_stride_dw + rem] = v;
}
}  // namespace

extern "C" int q8_0_pack_gemm_rows(const void* src, int64_t n_rows, int64_t k, int64_t src_row_stride_bytes,
                                   void* dst, int64_t dst_row_stride_bytes, void* stream) {
    using namespace moeq8;
    if (!src || !dst || n_rows < 0 || k <= 0 || k % (8 * QK) != 0) return MOEQ8_EINVAL;
    const int64_t row_bytes = k / QK * Q80_BYTES;
    if (src_row_stride_bytes < row_bytes || dst_row_stride_bytes < row_bytes) return MOEQ8_EINVAL;
    if (((uintptr_t)src | (uintptr_t)dst | (uint64_t)src_row_stride_bytes | (uint64_t)dst_row_stride_bytes) & 3u)
        return MOEQ8_EALIGN;
    const uint8_t* s8 = (const uint8_t*)src;
    const uint8_t* d8 = (const uint8_t*)dst;
    const int64_t span_s = n_rows == 0 ? 0 : (n_rows - 1) * src_row_stride_bytes + row_bytes;
    const int64_t span_d = n_rows == 0 ? 0 : (n_rows - 1) * dst_row_stride_bytes + row_bytes;
    if (s8 < d8 + span_d && d8 < s8 + span_s) return MOEQ8_EINVAL;     // no overlap (not in place)
    const int64_t total = n_rows * (row_bytes / 4);
    if (total == 0) return MOEQ8_OK;
    const int64_t blocks = (total + 255) / 256;
    if (blocks > 0x7fffffff) return MOEQ8_EUNSUPPORTED;
    hipLaunchKernelGGL(k_pack_gemm, dim3((uint32_t)blocks), dim3(256), 0, (hipStream_t)stream, s8, n_rows,
                       k / (8 * QK), src_row_stride_bytes, (uint32_t*)dst, dst_row_stride_bytes / 4);
    return check_launch();
}

// Repack Q8_0 rows into the round-major four-row packed layout
// (moeq8_device.hpp): round r (16 chunks, 1088 bytes) of every row goes to
// the matrix dst + r * n_rows * 1088 of contiguous 1088-byte rows, in which
// rows 4q .. 4q + 3 form one 4352-byte unit permuted as a 64-chunk segment.
// One thread per dword.
namespace {
__global__ void k_pack64_rounds(const uint32_t* __restrict__ src, int64_t n_rows, int64_t rounds,
                                int64_t src_stride_dw, uint32_t* __restrict__ dst) {
    using namespace moeq8;
    constexpr int ROW_DW = P64_SEGMENT_DWORDS / 4;                     // 272
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per_round = n_rows * ROW_DW;
    if (t >= rounds * per_round) return;
    const int64_t r = t / per_round;
    const int64_t rem = t - r * per_round;                             // dword within round r's matrix
    const int64_t q = rem / P64_SEGMENT_DWORDS;
    const int p = (int)(rem - q * P64_SEGMENT_DWORDS);
    const int sp = p64_source_dword(p);                                // unit dword it takes
    dst[t] = src[(4 * q + sp / ROW_DW) * src_stride_dw + r * ROW_DW + sp % ROW_DW];
}
}  // namespace

extern "C" int q8_0_pack64_rounds(const void* src, int64_t n_rows, int64_t k, int64_t src_row_stride_bytes,
                                  void* dst, void* stream) {
    using namespace moeq8;
    constexpr int64_t ROUND_VALUES = LANES_PER_ROW * 2 * QK;          // 1024
    if (!src || !dst || n_rows < 0 || n_rows % 4 != 0 || k <= 0 || k % ROUND_VALUES != 0) return MOEQ8_EINVAL;
    const int64_t row_bytes = k / QK * Q80_BYTES;
    if (src_row_stride_bytes < row_bytes) return MOEQ8_EINVAL;
    if (((uintptr_t)src | (uintptr_t)dst | (uint64_t)src_row_stride_bytes) & 3u) return MOEQ8_EALIGN;
    const uint8_t* s8 = (const uint8_t*)src;
    const uint8_t* d8 = (const uint8_t*)dst;
    const int64_t span_s = n_rows == 0 ? 0 : (n_rows - 1) * src_row_stride_bytes + row_bytes;
    const int64_t span_d = n_rows * row_bytes;
    if (s8 < d8 + span_d && d8 < s8 + span_s) return MOEQ8_EINVAL;     // no overlap (not in place)
    const int64_t total = n_rows * (row_bytes / 4);
    if (total == 0) return MOEQ8_OK;
    const int64_t blocks = (total + 255) / 256;
    if (blocks > 0x7fffffff) return MOEQ8_EUNSUPPORTED;
    hipLaunchKernelGGL(k_pack64_rounds, dim3((uint32_t)blocks), dim3(256), 0, (hipStream_t)stream,
                       (const uint32_t*)src, n_rows, k / ROUND_VALUES, src_row_stride_bytes / 4, (uint32_t*)dst);
    return check_launch();
}
