// Device fill of synthetic Q8_0 blocks from the SplitMix64 counter-based
// generator defined in moeq8_synth.h (bench-sized weight sets).
#include "moeq8_host.hpp"
#include "../../include/moeq8_synth.h"

namespace {

constexpr uint64_t GAMMA = 0x9E3779B97F4A7C15ull;

__host__ __device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ull;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__host__ __device__ __forceinline__ uint64_t key_of(uint32_t seed, uint32_t layer, uint32_t expert,
                                                    uint32_t matrix) {
    const uint64_t s = ((uint64_t)(seed & 0xFFFFu) << 48) | ((uint64_t)(layer & 0xFFFFu) << 32) |
                       ((uint64_t)(expert & 0xFFFFu) << 16) | (uint64_t)(matrix & 0xFFFFu);
    return mix64(s + GAMMA);
}

__global__ void k_synth_fill(uint8_t* dst, int64_t n_mats, int64_t blocks_per_mat,
                             int64_t mats_per_layer, uint32_t seed, uint32_t layer0,
                             uint32_t expert0, uint32_t matrix) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= n_mats * blocks_per_mat) return;
    const int64_t mat = gid / blocks_per_mat;
    const uint64_t b = (uint64_t)(gid - mat * blocks_per_mat);
    const uint64_t key = key_of(seed, layer0 + (uint32_t)(mat / mats_per_layer),
                                expert0 + (uint32_t)(mat % mats_per_layer), matrix);
    int8_t q[32];
    for (int t = 0; t < 16; ++t) {
        const uint64_t o = mix64(key + (b * 17 + (uint64_t)t + 1) * GAMMA);
        for (int h = 0; h < 2; ++h) {
            const uint32_t v = (uint32_t)((o >> (32 * h)) & 0xFF) + (uint32_t)((o >> (32 * h + 8)) & 0xFF) +
                               (uint32_t)((o >> (32 * h + 16)) & 0xFF) + (uint32_t)((o >> (32 * h + 24)) & 0xFF);
            int qi = (int)((v * 43u) >> 7) - 171;
            qi = qi < -127 ? -127 : (qi > 127 ? 127 : qi);
            q[2 * t + h] = (int8_t)qi;
        }
    }
    const uint64_t o = mix64(key + (b * 17 + 16 + 1) * GAMMA);
    const int pos = (int)((o >> 10) & 31);
    q[pos] = ((o >> 15) & 1) ? (int8_t)-127 : (int8_t)127;
    uint16_t* d16 = reinterpret_cast<uint16_t*>(dst + gid * 34);
    d16[0] = (uint16_t)(0x0C00u | (uint32_t)(o & 0x3FF));
    for (int i = 0; i < 16; ++i)
        d16[1 + i] = (uint16_t)((uint8_t)q[2 * i] | ((uint16_t)(uint8_t)q[2 * i + 1] << 8));
}

}  // namespace

extern "C" uint64_t moeq8_synth_stream_key(uint32_t seed, uint32_t layer, uint32_t expert,
                                            uint32_t matrix) {
    return key_of(seed, layer, expert, matrix);
}

extern "C" int moeq8_synth_q8_0_fill(void* dst, int64_t n_mats, int64_t blocks_per_mat,
                                     int64_t mats_per_layer, uint32_t seed, uint32_t layer0,
                                     uint32_t expert0, uint32_t matrix, void* stream) {
    if (!dst || n_mats < 0 || blocks_per_mat < 0 || mats_per_layer < 1) return MOEQ8_EINVAL;
    if ((uintptr_t)dst & 1u) return MOEQ8_EALIGN;
    const int64_t total = n_mats * blocks_per_mat;
    if (total == 0) return MOEQ8_OK;
    const int64_t blocks = (total + 255) / 256;
    if (blocks > 0x7fffffff) return MOEQ8_EUNSUPPORTED;
    hipLaunchKernelGGL(k_synth_fill, dim3((uint32_t)blocks), dim3(256), 0, (hipStream_t)stream,
                       (uint8_t*)dst, n_mats, blocks_per_mat, mats_per_layer, seed, layer0, expert0,
                       matrix);
    return moeq8::check_launch();
}

namespace {

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

// WG_BYTES bytes a workgroup of 256 threads, every load issued before the
// first use, nontemporal 16-byte loads.
template <int WG_BYTES>
__global__ __launch_bounds__(256) void k_stream_read(const u32x4v* __restrict__ p, int64_t n16,
                                                     uint32_t* sink) {
    constexpr int PER = WG_BYTES / 16 / 256;
    const int64_t base = (int64_t)blockIdx.x * (WG_BYTES / 16);
    u32x4v v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int64_t idx = base + i * 256 + threadIdx.x;
        v[i] = idx < n16 ? __builtin_nontemporal_load(p + idx) : u32x4v{0u, 0u, 0u, 0u};
    }
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

extern "C" int moeq8_stream_read_shape(const void* buf, int64_t bytes, int64_t wg_bytes, uint32_t* sink,
                                       void* stream) {
    if (!buf || !sink || bytes < 0) return MOEQ8_EINVAL;
    if (wg_bytes != 8192 && wg_bytes != 16384 && wg_bytes != 32768 && wg_bytes != 65536) return MOEQ8_EINVAL;
    if ((((uintptr_t)buf) & 15u) || (bytes & 15) || (((uintptr_t)sink) & 3u)) return MOEQ8_EALIGN;
    if (bytes == 0) return MOEQ8_OK;
    const int64_t blocks = (bytes + wg_bytes - 1) / wg_bytes;
    if (blocks > 0x7fffffff) return MOEQ8_EUNSUPPORTED;
    const dim3 grid((uint32_t)blocks), block(256);
    const hipStream_t s = (hipStream_t)stream;
    const u32x4v* p = (const u32x4v*)buf;
    switch (wg_bytes) {
        case 8192: hipLaunchKernelGGL(k_stream_read<8192>, grid, block, 0, s, p, bytes / 16, sink); break;
        case 16384: hipLaunchKernelGGL(k_stream_read<16384>, grid, block, 0, s, p, bytes / 16, sink); break;
        case 32768: hipLaunchKernelGGL(k_stream_read<32768>, grid, block, 0, s, p, bytes / 16, sink); break;
        default: hipLaunchKernelGGL(k_stream_read<65536>, grid, block, 0, s, p, bytes / 16, sink); break;
    }
    return moeq8::check_launch();
}

extern "C" int moeq8_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
    return moeq8_stream_read_shape(buf, bytes, 65536, sink, stream);
}
