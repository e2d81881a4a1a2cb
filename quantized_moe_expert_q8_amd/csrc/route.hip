// Router top-k select and weights over the same logits, owner mask and the
// layer's expert grouping, in one launch (lucebox PR #826, the fused DS4.1
// decode kernels commit: the router's select and weights over the same logits,
// one expert grouping per MoE layer for gate, up and down; the routed combine
// commit: the owner route mask).
//
// One workgroup; wave j selects column j's top-k.  Lane l of the wave holds
// experts [l*PER, (l+1)*PER) (contiguous, so among equal keys the lowest lane
// holds the lowest index).  Keys are compared as order-preserving u32 images
// of the fp32 key (the same order as the fp32 comparison for non-NaN keys, -0
// canonicalised to +0).  Each lane sorts its entries once (stable, key
// descending); each of the topk rounds takes the wave maximum of the lanes'
// first entries (DPP within rows of 16, then the four rows) and the lowest
// lane holding it (ballot), whose list then shifts by one: exact (key
// descending, expert ascending) selection.  Rounds run in slot order, so the weight sum is
// accumulated there in slot order; lane s keeps slot s.  Then the routes are
// sorted by (local expert, route index) for the grouping: with ballots in one
// wave when there are at most 64 routes, else from the ids in LDS.
#include "moeq8_device.hpp"
#include "moeq8_host.hpp"

namespace moeq8 {

constexpr int ROUTE_MAX_COLS = 8;
constexpr int ROUTE_MAX_TOPK = MOEQ8_MAX_TOPK;
constexpr int ROUTE_MAX_EXPERT = MOEQ8_MAX_EXPERTS;
constexpr int ROUTE_MAX_R = ROUTE_MAX_COLS * ROUTE_MAX_TOPK;   // 128

__device__ __forceinline__ uint32_t ordered_key(float f) {
    const uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The router's score of a logit: the sigmoid evaluated in fp64 and rounded
// once to fp32 (one expression for the router and for moe_router_scores).
__device__ __forceinline__ float router_score(float logit) {
    return (float)(1.0 / (1.0 + exp(-(double)logit)));
}

template <int CTRL>
__device__ __forceinline__ uint32_t max_dpp(uint32_t v) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
    return v > o ? v : o;
}

// maximum over the 64 lanes, returned to every lane
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max_dpp<0xB1>(v);    // quad_perm [1,0,3,2]
    v = max_dpp<0x4E>(v);    // quad_perm [2,3,0,1]
    v = max_dpp<0x141>(v);   // row_half_mirror
    v = max_dpp<0x140>(v);   // row_mirror: every lane holds its row's maximum
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    const uint32_t a = r0 > r1 ? r0 : r1;
    const uint32_t b = r2 > r3 ? r2 : r3;
    return a > b ? a : b;
}

template <int PER, bool GROUP = true>
__device__ __forceinline__ void route_body(
    const float* __restrict__ logits, const float* __restrict__ bias,
    const int32_t* __restrict__ owner, int ncols, int n_expert, int n_local, int topk,
    int32_t* __restrict__ ids, float* __restrict__ weights, int32_t* __restrict__ grouping) {
    __shared__ __attribute__((aligned(16))) int32_t s_id[ROUTE_MAX_R];
    __shared__ __attribute__((aligned(16))) int32_t s_headid[ROUTE_MAX_R];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int j = tid >> 6;
    const int e0 = lane * PER;
    const int R = ncols * topk;
    const int Rpad = (R + 7) & ~7;

    if (tid < ROUTE_MAX_R) {
        s_id[tid] = -1;
        s_headid[tid] = -1;
    }
    __syncthreads();

    float sum = 0.0f;
    float slot_score = 0.0f;
    int slot_id = -1;
    if (j < ncols) {
        float lg[PER], bs[PER], score[PER];
        int own[PER];
        uint32_t key[PER];
        uint32_t valid = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = e0 + i;
            const bool ok = e < n_expert;
            valid |= ok ? (1u << i) : 0u;
            lg[i] = ok ? logits[(int64_t)j * n_expert + e] : 0.0f;
            bs[i] = (ok && bias) ? bias[e] : 0.0f;
            own[i] = ok ? (owner ? owner[e] : e) : -1;
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            // sigmoid in fp64, rounded once to fp32; key = score + bias in fp32.
            // An expert past n_expert gets key 0, below every real key (the
            // ordered image of a finite float is positive).
            score[i] = router_score(lg[i]);
            key[i] = ((valid >> i) & 1u) ? ordered_key(bias ? score[i] + bs[i] : score[i]) : 0u;
        }
        // Sort the lane's entries once by key, descending: odd-even
        // transposition swapping only on a strictly larger key, which keeps
        // equal keys in expert order.  The lane's candidate is then always
        // entry 0, and the lane that wins a round shifts its list by one.
#pragma unroll
        for (int pass = 0; pass < PER; ++pass) {
#pragma unroll
            for (int i = pass & 1; i + 1 < PER; i += 2) {
                const bool sw = key[i + 1] > key[i];
                const uint32_t k0 = key[i], k1 = key[i + 1];
                const float s0 = score[i], s1 = score[i + 1];
                const int o0 = own[i], o1 = own[i + 1];
                key[i] = sw ? k1 : k0;
                key[i + 1] = sw ? k0 : k1;
                score[i] = sw ? s1 : s0;
                score[i + 1] = sw ? s0 : s1;
                own[i] = sw ? o1 : o0;
                own[i + 1] = sw ? o0 : o1;
            }
        }
        // topk <= n_expert (checked on the host), so every round has a
        // positive maximum and a winner
        for (int s = 0; s < topk; ++s) {
            const uint32_t wmax = wave_max_u32(key[0]);
            const uint64_t mask = __ballot(key[0] == wmax);
            const int w = (int)__builtin_ctzll(mask);          // lowest lane: lowest expert
            const float win = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(score[0]), w));
            const int win_own = __builtin_amdgcn_readlane(own[0], w);
            const bool shift = lane == w;
#pragma unroll
            for (int i = 0; i + 1 < PER; ++i) {
                key[i] = shift ? key[i + 1] : key[i];
                score[i] = shift ? score[i + 1] : score[i];
                own[i] = shift ? own[i + 1] : own[i];
            }
            key[PER - 1] = shift ? 0u : key[PER - 1];
            sum = sum + win;                                    // slot order
            if (lane == s) {
                slot_score = win;
                slot_id = (win_own < 0 || win_own >= n_local) ? -1 : win_own;
            }
        }
        if (lane < topk) s_id[j * topk + lane] = slot_id;
    }
    // only LDS traffic is outstanding at the barriers (every global store is
    // issued at the end, so no barrier waits for one)
    __syncthreads();

    if (j < ncols && lane < topk) {
        const int rr = j * topk + lane;
        ids[rr] = slot_id;
        weights[rr] = slot_score / sum;
    }
    if constexpr (!GROUP) return;
    int32_t* g_expert = grouping + 4;
    int32_t* g_offset = grouping + 4 + R;
    int32_t* g_route = grouping + 4 + 2 * R + 1;
    int4* g_table = reinterpret_cast<int4*>(grouping + grouping_table_word(R));

    if (R <= 64) {
        // one wave: lane r holds route r.  An 11-bit radix pass of ballots over
        // the local ids (< 1024) gives each lane the masks of valid routes with
        // a smaller id (lt) and with the same id (eq).
        if (j != 0) return;
        const int r = lane;
        const int id = r < R ? s_id[r] : -1;
        const bool valid = id >= 0;
        const uint64_t vmask = __ballot(valid);
        uint64_t lt = 0, eq = vmask;
#pragma unroll
        for (int b = 10; b >= 0; --b) {
            const uint64_t ones = __ballot(valid && ((id >> b) & 1));
            const bool mine = valid && ((id >> b) & 1);
            if (mine) lt |= eq & ~ones;
            eq &= mine ? ones : ~ones;
        }
        const uint64_t below = (r == 0) ? 0ull : (~0ull >> (64 - r));
        const int before = __popcll(eq & below);
        const bool head = valid && before == 0;
        const uint64_t hmask = __ballot(head);
        const int n_valid = __popcll(vmask);
        const int n_heads = __popcll(hmask);
        const int pos = __popcll(lt) + before;
        if (head) {
            const int act = __popcll(lt & hmask);
            g_expert[act] = id;
            g_offset[act] = pos;
            g_table[act] = make_int4(id, pos, pos + __popcll(eq), 0);
        }
        if (valid) g_route[pos] = r;
        if (r < R) {
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
        return;
    }

    // R in (64, 128]: thread r < R places route r from the ids in LDS
    const int r = tid;
    const bool in = r < R;
    const int id = in ? s_id[r] : -1;
    const bool valid = id >= 0;
    int pos = 0, before = 0, n_valid = 0, same = 0;
    const int4* v4 = reinterpret_cast<const int4*>(s_id);
#pragma unroll
    for (int q4 = 0; q4 < ROUTE_MAX_R / 4; ++q4) {
        if (q4 * 4 < Rpad) {
            const int4 v = v4[q4];
            const int vq[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int q = q4 * 4 + t;
                const int iq = vq[t];
                n_valid += iq >= 0 ? 1 : 0;
                pos += (iq >= 0 && (iq < id || (iq == id && q < r))) ? 1 : 0;
                before += (iq == id && q < r) ? 1 : 0;
                same += (iq == id) ? 1 : 0;
            }
        }
    }
    const bool head = valid && before == 0;
    if (head) s_headid[r] = id;
    __syncthreads();
    int act = 0, n_heads = 0;
    const int4* h4 = reinterpret_cast<const int4*>(s_headid);
#pragma unroll
    for (int q4 = 0; q4 < ROUTE_MAX_R / 4; ++q4) {
        if (q4 * 4 < Rpad) {
            const int4 v = h4[q4];
            n_heads += (v.x >= 0) + (v.y >= 0) + (v.z >= 0) + (v.w >= 0);
            act += (v.x >= 0 && v.x < id) + (v.y >= 0 && v.y < id) + (v.z >= 0 && v.z < id) +
                   (v.w >= 0 && v.w < id);
        }
    }
    if (head) {
        g_expert[act] = id;
        g_offset[act] = pos;
        g_table[act] = make_int4(id, pos, pos + same, 0);
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

template <int PER>
__global__ __launch_bounds__(64 * ROUTE_MAX_COLS) void k_route_topk(
    const float* __restrict__ logits, const float* __restrict__ bias,
    const int32_t* __restrict__ owner, int ncols, int n_expert, int n_local, int topk,
    int32_t* __restrict__ ids, float* __restrict__ weights, int32_t* __restrict__ grouping) {
    route_body<PER>(logits, bias, owner, ncols, n_expert, n_local, topk, ids, weights, grouping);
}

// Selection and weights only, for any number of columns: workgroup b takes
// columns [8b, 8b + 8), each column exactly as in k_route_topk (columns are
// independent until the grouping, which moe_group_routes builds).
template <int PER>
__global__ __launch_bounds__(64 * ROUTE_MAX_COLS) void k_route_topk_wide(
    const float* __restrict__ logits, const float* __restrict__ bias,
    const int32_t* __restrict__ owner, int64_t ncols, int n_expert, int n_local, int topk,
    int32_t* __restrict__ ids, float* __restrict__ weights) {
    const int64_t c0 = (int64_t)blockIdx.x * ROUTE_MAX_COLS;
    const int nc = (int)min((int64_t)ROUTE_MAX_COLS, ncols - c0);
    route_body<PER, false>(logits + c0 * n_expert, bias, owner, nc, n_expert, n_local, topk,
                           ids + c0 * topk, weights + c0 * topk, nullptr);
}

// The expert grouping of any number of routes (the same layout as the one
// moe_route_topk writes), from the route ids, in one workgroup of 1024
// threads, as a counting sort that needs no ordering from atomics:
//   1. wave w counts the local experts of its contiguous share of the routes
//      (LDS atomic adds: the counts do not depend on their order);
//   2. per expert, the waves' counts become a prefix over waves, and one
//      block scan over experts gives each expert's first position and each
//      active expert's group index;
//   3. wave w places its share in ascending route order, 64 routes at a time:
//      a route's rank among the earlier lanes holding the same expert comes
//      from ballots over the expert's bits.
// So routes come out by (expert, route index) ascending, as a stable sort by
// expert gives; ids outside [0, n_local) are masked.
constexpr int WIDE_THREADS = 1024;
constexpr int WIDE_WAVES = WIDE_THREADS / 64;
constexpr int WIDE_MAX_R = 16384;                      // 1024 columns x top-16

// exclusive prefix sum over the 1024 threads; *total gets the sum
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    uint32_t incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t t = (uint32_t)__builtin_amdgcn_ds_bpermute((lane - d) << 2, (int)incl);
        if (lane >= d) incl += t;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    uint32_t before = 0, all = 0;
    for (int i = 0; i < WIDE_WAVES; ++i) {
        const uint32_t x = wsum[i];
        before += i < w ? x : 0u;
        all += x;
    }
    *total = all;
    return before + incl - v;
}

__global__ __launch_bounds__(WIDE_THREADS) void k_group_routes(
    const int32_t* __restrict__ ids, int64_t ncols, int topk, int n_local,
    int32_t* __restrict__ grouping) {
    // per-wave counts, two 16-bit counters per word (a wave holds at most
    // 1024 routes, so a counter never carries into its neighbour)
    __shared__ uint32_t cnt[WIDE_WAVES][MOEQ8_MAX_EXPERTS / 2];
    __shared__ int32_t first[MOEQ8_MAX_EXPERTS];
    __shared__ uint32_t wsum[WIDE_WAVES];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int R = (int)ncols * topk;
    const int share = ((R + WIDE_WAVES - 1) / WIDE_WAVES + 63) / 64 * 64;   // routes per wave
    const int rb = w * share, re = min(R, rb + share);
    auto key_of = [&](int r) -> int {                  // local expert, or n_local when masked
        if (r >= re) return MOEQ8_MAX_EXPERTS;
        const int id = ids[r];
        return (id >= 0 && id < n_local) ? id : MOEQ8_MAX_EXPERTS;
    };

    for (int i = tid; i < WIDE_WAVES * (MOEQ8_MAX_EXPERTS / 2); i += WIDE_THREADS) (&cnt[0][0])[i] = 0u;
    __syncthreads();
    for (int r = rb + lane; r < re; r += 64) {
        const int e = key_of(r);
        if (e < MOEQ8_MAX_EXPERTS) atomicAdd(&cnt[w][e >> 1], 1u << (16 * (e & 1)));
    }
    __syncthreads();

    // thread e: expert e's count per wave -> prefix over waves, total
    const int e = tid;
    uint32_t tot = 0;
    if (e < n_local) {
        for (int v = 0; v < WIDE_WAVES; ++v) {
            const uint32_t word = cnt[v][e >> 1];
            const uint32_t c = (word >> (16 * (e & 1))) & 0xffffu;
            tot += c;
        }
    }
    __syncthreads();                                   // every thread has read its counts
    if (e < n_local) {
        uint32_t run = 0;
        for (int v = 0; v < WIDE_WAVES; ++v) {
            const uint32_t c = (cnt[v][e >> 1] >> (16 * (e & 1))) & 0xffffu;
            // only this thread changes expert e's half of the word; xor
            // replaces it without touching the neighbour's half
            atomicXor(&cnt[v][e >> 1], ((c ^ run) & 0xffffu) << (16 * (e & 1)));
            run += c;
        }
    }
    // one scan of (active << 16 | count): positions and group indices
    uint32_t all = 0;
    const uint32_t packed = (tot > 0 ? (1u << 16) : 0u) | tot;   // tot <= 16384 < 2^16
    const uint32_t ex = block_excl_scan(packed, wsum, &all);
    const int pos0 = (int)(ex & 0xffffu), grp = (int)(ex >> 16);
    const int n_valid = (int)(all & 0xffffu), n_heads = (int)(all >> 16);
    if (e < MOEQ8_MAX_EXPERTS) first[e] = pos0;
    int32_t* g_expert = grouping + 4;
    int32_t* g_offset = grouping + 4 + R;
    int32_t* g_route = grouping + 4 + 2 * R + 1;
    int4* g_table = reinterpret_cast<int4*>(grouping + grouping_table_word(R));
    if (tot > 0) {
        g_expert[grp] = e;
        g_offset[grp] = pos0;
        g_table[grp] = make_int4(e, pos0, pos0 + (int)tot, 0);
    }
    for (int q = n_heads + tid; q < R; q += WIDE_THREADS) g_expert[q] = -1;
    for (int q = n_heads + tid; q <= R; q += WIDE_THREADS) g_offset[q] = n_valid;
    for (int q = n_valid + tid; q < R; q += WIDE_THREADS) g_route[q] = -1;
    if (tid == 0) {
        grouping[0] = n_heads;
        grouping[1] = n_valid;
        grouping[2] = (int32_t)ncols;
        grouping[3] = topk;
    }
    __syncthreads();                                   // first[] and the wave prefixes are in place

    // placement, 64 routes of the wave's share at a time, in route order
    const uint64_t below = (1ull << lane) - 1ull;
    for (int r0 = rb; r0 < re; r0 += 64) {
        const int r = r0 + lane;
        const int k = key_of(r);                        // < 2^11
        uint64_t same = ~0ull;
#pragma unroll
        for (int b = 0; b < 11; ++b) {
            const uint64_t ones = __ballot((k >> b) & 1);
            same &= ((k >> b) & 1) ? ones : ~ones;
        }
        if (k < MOEQ8_MAX_EXPERTS) {
            const uint32_t word = cnt[w][k >> 1];
            const int before_w = (int)((word >> (16 * (k & 1))) & 0xffffu);
            g_route[first[k] + before_w + __popcll(same & below)] = r;
        }
        // the wave's reads of cnt come before its updates (in-order LDS):
        // the highest lane of each expert adds the expert's routes here
        if (k < MOEQ8_MAX_EXPERTS && (same >> lane) == 1ull)
            atomicAdd(&cnt[w][k >> 1], (uint32_t)__popcll(same) << (16 * (k & 1)));
    }
}

// The layer prologue: block 0 routes; the other blocks quantise the FFN input
// to q8_1 (both read only the layer's inputs, so one launch runs them side by
// side).  Bytes and routing are those of q8_1_quantize_rows and moe_route_topk.
template <int PER>
__global__ __launch_bounds__(64 * ROUTE_MAX_COLS) void k_route_quantize(
    const float* __restrict__ logits, const float* __restrict__ bias,
    const int32_t* __restrict__ owner, int ncols, int n_expert, int n_local, int topk,
    int32_t* __restrict__ ids, float* __restrict__ weights, int32_t* __restrict__ grouping,
    const float* __restrict__ x, int64_t x_stride, int64_t nb, uint8_t* __restrict__ xq) {
    if (blockIdx.x == 0) {
        route_body<PER>(logits, bias, owner, ncols, n_expert, n_local, topk, ids, weights, grouping);
        return;
    }
    const int64_t gid = (int64_t)(blockIdx.x - 1) * blockDim.x + threadIdx.x;
    if (gid >= (int64_t)ncols * nb) return;
    const int64_t r = gid / nb;
    const int64_t b = gid - r * nb;
    quantize_block<true>(x + r * x_stride + b * QK, xq + gid * Q81_BYTES);
}

__global__ void k_router_scores(const float* __restrict__ logits, int64_t n, float* __restrict__ scores) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) scores[i] = router_score(logits[i]);
}

}  // namespace moeq8

using namespace moeq8;

namespace {
size_t grouping_bytes_of(int64_t ncols, int32_t topk) {
    const size_t R = (size_t)ncols * (size_t)topk;
    // header, expert[R], offset[R+1], route[R], eight words of padding (so
    // that readers may load eight words from any route entry), the table
    const size_t bytes = 4 * ((size_t)grouping_table_word((int64_t)R) + 4 * R);
    return (bytes + 255) & ~(size_t)255;
}
}  // namespace

extern "C" size_t moe_grouping_bytes(int64_t ncols, int32_t topk) {
    if (ncols < 1 || ncols > ROUTE_MAX_COLS || topk < 1 || topk > ROUTE_MAX_TOPK) return 0;
    return grouping_bytes_of(ncols, topk);
}

extern "C" size_t moe_grouping_bytes_wide(int64_t ncols, int32_t topk) {
    if (ncols < 1 || ncols > MOEQ8_MAX_WIDE_COLS || topk < 1 || topk > ROUTE_MAX_TOPK) return 0;
    return grouping_bytes_of(ncols, topk);
}

namespace {
int validate_route(const float* logits, const float* bias, const int32_t* owner_slot, int64_t ncols,
                   int64_t n_expert, int64_t n_local_expert, int32_t topk, const int32_t* ids,
                   const float* weights, const void* grouping) {
    if (!logits || !ids || !weights || !grouping) return MOEQ8_EINVAL;
    if (ncols < 1 || ncols > ROUTE_MAX_COLS || topk < 1 || topk > ROUTE_MAX_TOPK) return MOEQ8_EINVAL;
    if (n_expert < 1 || topk > n_expert || n_local_expert < 1) return MOEQ8_EINVAL;
    if (!owner_slot && n_local_expert != n_expert) return MOEQ8_EINVAL;
    if (n_expert > ROUTE_MAX_EXPERT || n_local_expert > ROUTE_MAX_EXPERT) return MOEQ8_EUNSUPPORTED;
    if (((uintptr_t)logits | (uintptr_t)bias | (uintptr_t)owner_slot | (uintptr_t)ids |
         (uintptr_t)weights | (uintptr_t)grouping) & 3u)
        return MOEQ8_EALIGN;
    return MOEQ8_OK;
}
}  // namespace

extern "C" int moe_route_topk(const float* logits, const float* bias, const int32_t* owner_slot,
                              int64_t ncols, int64_t n_expert, int64_t n_local_expert, int32_t topk,
                              int32_t* ids, float* weights, void* grouping, void* stream) {
    const int st = validate_route(logits, bias, owner_slot, ncols, n_expert, n_local_expert, topk,
                                  ids, weights, grouping);
    if (st) return st;
    // the grouping needs R = ncols * topk <= 128 threads: at least two waves
    const dim3 block(64 * (unsigned)std::max<int64_t>(ncols, 2));
    const int per = (int)((n_expert + 63) / 64);
    const hipStream_t hs = (hipStream_t)stream;
#define MOEQ8_ROUTE_LAUNCH(P)                                                                    \
    hipLaunchKernelGGL(k_route_topk<P>, dim3(1), block, 0, hs, logits, bias, owner_slot,         \
                       (int)ncols, (int)n_expert, (int)n_local_expert, (int)topk, ids, weights, \
                       (int32_t*)grouping)
    if (per <= 1) MOEQ8_ROUTE_LAUNCH(1);
    else if (per <= 2) MOEQ8_ROUTE_LAUNCH(2);
    else if (per <= 4) MOEQ8_ROUTE_LAUNCH(4);
    else if (per <= 8) MOEQ8_ROUTE_LAUNCH(8);
    else MOEQ8_ROUTE_LAUNCH(16);
#undef MOEQ8_ROUTE_LAUNCH
    return check_launch();
}

extern "C" int moe_route_topk_quantize(const float* x, int64_t x_row_stride, int64_t k, void* xq,
                                       const float* logits, const float* bias,
                                       const int32_t* owner_slot, int64_t ncols, int64_t n_expert,
                                       int64_t n_local_expert, int32_t topk, int32_t* ids,
                                       float* weights, void* grouping, void* stream) {
    int st = validate_route(logits, bias, owner_slot, ncols, n_expert, n_local_expert, topk, ids,
                            weights, grouping);
    if (st) return st;
    if (!x || !xq || k <= 0 || (k % QK) != 0 || x_row_stride < k) return MOEQ8_EINVAL;
    if (((uintptr_t)x & 3u) || ((uintptr_t)xq & 3u)) return MOEQ8_EALIGN;
    const int64_t nb = k / QK;
    const unsigned threads = 64 * (unsigned)std::max<int64_t>(ncols, 2);
    const int64_t qblocks = (ncols * nb + threads - 1) / threads;
    if (qblocks + 1 > 0x7fffffff) return MOEQ8_EUNSUPPORTED;
    const dim3 grid((uint32_t)(qblocks + 1)), block(threads);
    const int per = (int)((n_expert + 63) / 64);
    const hipStream_t hs = (hipStream_t)stream;
#define MOEQ8_PRO_LAUNCH(P)                                                                          \
    hipLaunchKernelGGL(k_route_quantize<P>, grid, block, 0, hs, logits, bias, owner_slot, (int)ncols, \
                       (int)n_expert, (int)n_local_expert, (int)topk, ids, weights,                   \
                       (int32_t*)grouping, x, x_row_stride, nb, (uint8_t*)xq)
    if (per <= 1) MOEQ8_PRO_LAUNCH(1);
    else if (per <= 2) MOEQ8_PRO_LAUNCH(2);
    else if (per <= 4) MOEQ8_PRO_LAUNCH(4);
    else if (per <= 8) MOEQ8_PRO_LAUNCH(8);
    else MOEQ8_PRO_LAUNCH(16);
#undef MOEQ8_PRO_LAUNCH
    return check_launch();
}

extern "C" int moe_route_topk_wide(const float* logits, const float* bias, const int32_t* owner_slot,
                                   int64_t ncols, int64_t n_expert, int64_t n_local_expert,
                                   int32_t topk, int32_t* ids, float* weights, void* stream) {
    if (!logits || !ids || !weights) return MOEQ8_EINVAL;
    if (ncols < 1 || ncols > MOEQ8_MAX_WIDE_COLS || topk < 1 || topk > ROUTE_MAX_TOPK) return MOEQ8_EINVAL;
    if (n_expert < 1 || topk > n_expert || n_local_expert < 1) return MOEQ8_EINVAL;
    if (!owner_slot && n_local_expert != n_expert) return MOEQ8_EINVAL;
    if (n_expert > ROUTE_MAX_EXPERT || n_local_expert > ROUTE_MAX_EXPERT) return MOEQ8_EUNSUPPORTED;
    if (((uintptr_t)logits | (uintptr_t)bias | (uintptr_t)owner_slot | (uintptr_t)ids |
         (uintptr_t)weights) & 3u)
        return MOEQ8_EALIGN;
    const dim3 grid((uint32_t)((ncols + ROUTE_MAX_COLS - 1) / ROUTE_MAX_COLS)), block(64 * ROUTE_MAX_COLS);
    const int per = (int)((n_expert + 63) / 64);
    const hipStream_t hs = (hipStream_t)stream;
#define MOEQ8_WIDE_LAUNCH(P)                                                                      \
    hipLaunchKernelGGL(k_route_topk_wide<P>, grid, block, 0, hs, logits, bias, owner_slot, ncols, \
                       (int)n_expert, (int)n_local_expert, (int)topk, ids, weights)
    if (per <= 1) MOEQ8_WIDE_LAUNCH(1);
    else if (per <= 2) MOEQ8_WIDE_LAUNCH(2);
    else if (per <= 4) MOEQ8_WIDE_LAUNCH(4);
    else if (per <= 8) MOEQ8_WIDE_LAUNCH(8);
    else MOEQ8_WIDE_LAUNCH(16);
#undef MOEQ8_WIDE_LAUNCH
    return check_launch();
}

extern "C" int moe_group_routes(const int32_t* ids, int64_t ncols, int32_t topk,
                                int64_t n_local_expert, void* grouping, void* stream) {
    if (!ids || !grouping) return MOEQ8_EINVAL;
    if (ncols < 1 || ncols > MOEQ8_MAX_WIDE_COLS || topk < 1 || topk > ROUTE_MAX_TOPK) return MOEQ8_EINVAL;
    if (n_local_expert < 1) return MOEQ8_EINVAL;
    if (n_local_expert > ROUTE_MAX_EXPERT) return MOEQ8_EUNSUPPORTED;
    if (((uintptr_t)ids | (uintptr_t)grouping) & 3u) return MOEQ8_EALIGN;
    hipLaunchKernelGGL(k_group_routes, dim3(1), dim3(WIDE_THREADS), 0, (hipStream_t)stream, ids, ncols,
                       (int)topk, (int)n_local_expert, (int32_t*)grouping);
    return check_launch();
}

extern "C" int moe_router_scores(const float* logits, int64_t n, float* scores, void* stream) {
    if (!logits || !scores || n < 0) return MOEQ8_EINVAL;
    if (((uintptr_t)logits | (uintptr_t)scores) & 3u) return MOEQ8_EALIGN;
    if (n == 0) return MOEQ8_OK;
    const int64_t blocks = (n + 255) / 256;
    if (blocks > 0x7fffffff) return MOEQ8_EUNSUPPORTED;
    hipLaunchKernelGGL(k_router_scores, dim3((uint32_t)blocks), dim3(256), 0, (hipStream_t)stream, logits, n,
                       scores);
    return check_launch();
}
