// Router top-k select and weights over the same logits, owner mask and the
// layer's expert grouping, in one launch (lucebox PR #826, the fused DS4.1
// decode kernels commit: "the router's select and weights over the same logits"
// and "one expert grouping per MoE layer for gate, up and down"; the routed
// combine commit: the owner route mask).
//
// One workgroup; wave j selects column j's top-k by repeated wave-wide argmax
// under the order (key descending, expert index ascending), which is a strict
// total order, so the selection is exact and deterministic.  Then the whole
// workgroup sorts the <= ncols*topk routes by (local expert, route index) and
// writes the grouping the grouped MMVQ launches read.
#include "moeq8_device.hpp"
#include "moeq8_host.hpp"

namespace moeq8 {

constexpr int ROUTE_MAX_COLS = 8;
constexpr int ROUTE_MAX_TOPK = MOEQ8_MAX_TOPK;
constexpr int ROUTE_MAX_EXPERT = MOEQ8_MAX_EXPERTS;
constexpr int ROUTE_PER_LANE = ROUTE_MAX_EXPERT / 64;

__device__ __forceinline__ bool key_before(float ka, int ea, float kb, int eb) {
    return ka > kb || (ka == kb && ea < eb);
}

__global__ __launch_bounds__(64 * ROUTE_MAX_COLS) void k_route_topk(
    const float* __restrict__ logits, const float* __restrict__ bias,
    const int32_t* __restrict__ owner, int ncols, int n_expert, int n_local, int topk,
    int32_t* __restrict__ ids, float* __restrict__ weights, int32_t* __restrict__ grouping) {
    __shared__ int32_t s_id[ROUTE_MAX_COLS * ROUTE_MAX_TOPK];
    __shared__ int32_t s_head[ROUTE_MAX_COLS * ROUTE_MAX_TOPK];
    __shared__ int32_t s_sel_e[ROUTE_MAX_COLS * ROUTE_MAX_TOPK];
    __shared__ float s_sel_score[ROUTE_MAX_COLS * ROUTE_MAX_TOPK];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;

    if (wave < ncols) {
        const int j = wave;
        float key[ROUTE_PER_LANE];
        float score[ROUTE_PER_LANE];
        bool taken[ROUTE_PER_LANE];
#pragma unroll
        for (int i = 0; i < ROUTE_PER_LANE; ++i) {
            const int e = lane + 64 * i;
            taken[i] = true;
            key[i] = 0.0f;
            score[i] = 0.0f;
            if (e < n_expert) {
                const double z = (double)logits[(int64_t)j * n_expert + e];
                // sigmoid in fp64, rounded once to fp32
                score[i] = (float)(1.0 / (1.0 + exp(-z)));
                key[i] = bias ? score[i] + bias[e] : score[i];
                taken[i] = false;
            }
        }
        for (int s = 0; s < topk; ++s) {
            float bk = -INFINITY, bs = 0.0f;
            int be = 0x7fffffff;
#pragma unroll
            for (int i = 0; i < ROUTE_PER_LANE; ++i) {
                const int e = lane + 64 * i;
                if (!taken[i] && key_before(key[i], e, bk, be)) {
                    bk = key[i];
                    be = e;
                    bs = score[i];
                }
            }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) {
                const float ok = __shfl_xor(bk, off, 64);
                const int oe = __shfl_xor(be, off, 64);
                const float os = __shfl_xor(bs, off, 64);
                if (key_before(ok, oe, bk, be)) {
                    bk = ok;
                    be = oe;
                    bs = os;
                }
            }
#pragma unroll
            for (int i = 0; i < ROUTE_PER_LANE; ++i)
                if (lane + 64 * i == be) taken[i] = true;
            if (lane == 0) {
                s_sel_e[j * topk + s] = be;
                s_sel_score[j * topk + s] = bs;
            }
        }
        if (lane == 0) {
            float sum = 0.0f;
            for (int s = 0; s < topk; ++s) sum = sum + s_sel_score[j * topk + s];
            for (int s = 0; s < topk; ++s) {
                const int e = s_sel_e[j * topk + s];
                int id = owner ? owner[e] : e;
                if (id < 0 || id >= n_local) id = -1;
                ids[j * topk + s] = id;
                weights[j * topk + s] = s_sel_score[j * topk + s] / sum;
                s_id[j * topk + s] = id;
            }
        }
    }
    __syncthreads();

    // grouping: one thread per route sorts the valid routes by (id, route)
    const int R = ncols * topk;  // <= blockDim.x
    int32_t* g_expert = grouping + 4;
    int32_t* g_offset = grouping + 4 + R;
    int32_t* g_route = grouping + 4 + 2 * R + 1;
    const int r = threadIdx.x;
    const bool in = r < R;
    const int id = in ? s_id[r] : -1;
    const bool valid = id >= 0;
    bool head = valid;
    int pos = 0;
    if (valid) {
        for (int q = 0; q < R; ++q) {
            const int iq = s_id[q];
            if (iq < 0) continue;
            if (iq < id || (iq == id && q < r)) ++pos;
            if (iq == id && q < r) head = false;
        }
    }
    if (in) s_head[r] = head ? 1 : 0;
    const int n_valid = __syncthreads_count(valid);
    const int n_heads = __syncthreads_count(head);
    if (head) {
        int act = 0;
        for (int q = 0; q < R; ++q) act += (s_head[q] && s_id[q] < id) ? 1 : 0;
        g_expert[act] = id;
        g_offset[act] = pos;
    }
    if (valid) g_route[pos] = r;
    if (in) {
        if (r >= n_valid) g_route[r] = -1;
        if (r >= n_heads) g_expert[r] = -1;
        if (r > n_heads) g_offset[r] = n_valid;
    }
    if (r == 0) {
        grouping[0] = n_heads;
        grouping[1] = n_valid;
        grouping[2] = ncols;
        grouping[3] = topk;
        g_offset[n_heads] = n_valid;
        g_offset[R] = n_valid;
    }
}

}  // namespace moeq8

using namespace moeq8;

extern "C" size_t moe_grouping_bytes(int64_t ncols, int32_t topk) {
    if (ncols < 1 || ncols > ROUTE_MAX_COLS || topk < 1 || topk > ROUTE_MAX_TOPK) return 0;
    const size_t R = (size_t)ncols * (size_t)topk;
    const size_t bytes = 4 * (4 + 3 * R + 1);
    return (bytes + 255) & ~(size_t)255;
}

extern "C" int moe_route_topk(const float* logits, const float* bias, const int32_t* owner_slot,
                              int64_t ncols, int64_t n_expert, int64_t n_local_expert, int32_t topk,
                              int32_t* ids, float* weights, void* grouping, void* stream) {
    if (!logits || !ids || !weights || !grouping) return MOEQ8_EINVAL;
    if (ncols < 1 || ncols > ROUTE_MAX_COLS || topk < 1 || topk > ROUTE_MAX_TOPK) return MOEQ8_EINVAL;
    if (n_expert < 1 || topk > n_expert || n_local_expert < 1) return MOEQ8_EINVAL;
    if (!owner_slot && n_local_expert != n_expert) return MOEQ8_EINVAL;
    if (n_expert > ROUTE_MAX_EXPERT) return MOEQ8_EUNSUPPORTED;
    if (((uintptr_t)logits | (uintptr_t)bias | (uintptr_t)owner_slot | (uintptr_t)ids |
         (uintptr_t)weights | (uintptr_t)grouping) & 3u)
        return MOEQ8_EALIGN;
    hipLaunchKernelGGL(k_route_topk, dim3(1), dim3(64 * (unsigned)ncols), 0, (hipStream_t)stream,
                       logits, bias, owner_slot, (int)ncols, (int)n_expert, (int)n_local_expert,
                       (int)topk, ids, weights, (int32_t*)grouping);
    return check_launch();
}
