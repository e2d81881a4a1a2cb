// Grouped per-expert Q8_0 x q8_1 products on the int8 matrix cores, for wide
// batches (many columns, so many routes per expert): the prefill-sized
// counterpart of the grouped MMVQ.  The pages run their large expert batches
// on a matrix-core GEMM (the WMMA routed-expert GEMM in the PR description's
// Results, and MMQ routing for wide Q4_K products in the fused-kernels commit);
// here the GEMM keeps the Q8_0 / q8_1 formats and the expert grouping of the
// decode path.
//
// One Q8_0 block is 32 values along K, exactly the K of
// v_mfma_i32_16x16x32_i8, so each block's 16x16 integer tile is scaled on its
// own: acc += float(sumi) * (d_w * d_x), one fused multiply-add per output and
// block, blocks in ascending order.  d_w * d_x is exact in fp32 (two fp16
// values) and sumi is exact as an fp32 integer (|sumi| <= 32 * 127 * 127), so
// each block adds its exact term with one rounding.  This order differs from
// the MMVQ's 16-lane tree, so the two paths agree to rounding, not bit for bit.
//
// Operands: A (16 routes x 32) is the q8_1 activation block of 16 routes, B
// (32 x 16 weight rows) a Q8_0 block of 16 rows.  Lane l supplies route l%16
// (A) and weight row l%16 (B), bytes 8*(l/16) .. +8 of the block, and receives
// D for weight row l%16 and routes 4*(l/16) + i, i = 0..3.  So a lane needs
// one weight scale per block (its own row) and four activation scales.
//
// Work item = (group, tile of rows).  The item stages the q8_1 rows of up to
// RT of its group's routes in LDS (quants as [block][route][32 B], scales as
// fp32 [block][route]) and every wave streams its own weight rows straight
// from HBM into registers, several block pairs ahead of use, so the weight
// loads never wait on LDS traffic.  Groups with more than RT routes take them
// in passes (re-streaming the rows).
//   gate/up: a wave owns 16 rows of the gate and the same 16 rows of the up
//            matrix; both share every activation fragment; SwiGLU-DS4 epilogue.
//   down:    a wave owns 32 consecutive rows (two 16-row fragments).
#include "moeq8_device.hpp"
#include "moeq8_host.hpp"

#include <atomic>

namespace moeq8 {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int GEMM_WAVES = 4;
constexpr int GEMM_THREADS = 64 * GEMM_WAVES;
constexpr int TILE_ROUTES = 16;          // routes per matrix-core tile
constexpr int PF = 4;                    // block pairs of weights in flight per wave
constexpr size_t GEMM_LDS_TARGET = 80 * 1024;   // two workgroups per CU
constexpr size_t GEMM_LDS_MAX = 160 * 1024;

struct GemmParams {
    const uint8_t* w0;          // gate (gate/up) or down, expert 0
    const uint8_t* w1;          // up (gate/up) or null
    int64_t expert_stride;      // bytes
    int64_t row_stride;         // bytes
    int64_t n;                  // rows per expert matrix
    int64_t n_local;
    int32_t nb;                 // blocks per row (k / 32)
    int32_t tiles;              // row tiles per group
    int32_t ncols;
    int32_t topk;
    uint64_t act_route_mul;     // activation row of route r = (r * act_route_mul) >> 32
    const uint8_t* act;         // q8_1 rows
    int64_t act_row_bytes;      // nb * 36
    const int32_t* grouping;
    float* out;                 // [ncols * topk][n]
};

// Weight bytes of one block pair of one 16-row fragment, as lane (c, q) loads
// them: dwords at +8q .. +8q+12 of the pair's 68 bytes (block 0's quants start
// at byte 2, so they straddle dwords) and the two dwords at +36+8q (block 1's
// quants, dword aligned).
struct WPair {
    uint32_t a0, a1, a2, b0, b1;
};

__device__ __forceinline__ void load_pair(WPair& w, const uint8_t* p) {
    const u32x2 lo = *reinterpret_cast<const u32x2*>(p);
    w.a0 = lo.x;
    w.a1 = lo.y;
    w.a2 = *reinterpret_cast<const uint32_t*>(p + 8);
    const u32x2 hi = *reinterpret_cast<const u32x2*>(p + 36);
    w.b0 = hi.x;
    w.b1 = hi.y;
}

template <bool PAIR, int NT>
__global__ __launch_bounds__(GEMM_THREADS) void k_grouped_gemm(const GemmParams p) {
    constexpr int RT = NT * TILE_ROUTES;
    constexpr int WAVE_ROWS = PAIR ? 16 : 32;
    constexpr int WG_ROWS = WAVE_ROWS * GEMM_WAVES;
    extern __shared__ __align__(16) uint8_t lds[];

    const int nb = p.nb;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int l = tid & 63;
    const int c = l & 15;                 // B: weight row of the fragment; D: weight row
    const int q = l >> 4;                 // 8-byte slice of the block; D: routes 4q .. 4q+3

    uint8_t* aq = lds;                                          // [nb][RT][32]
    float* dxt = reinterpret_cast<float*>(lds + (size_t)nb * RT * 32);   // [nb][RT]
    int32_t* rid = reinterpret_cast<int32_t*>(lds + (size_t)nb * RT * 36);   // [RT]

    // work item: group a, row tile t
    const uint32_t tiles = (uint32_t)p.tiles;
    const uint32_t a = blockIdx.x / tiles;
    const uint32_t t = blockIdx.x - a * tiles;
    const int Rk = p.ncols * p.topk;
    const int4w hdr = grouping_words4(p.grouping, 0);
    const int4w grp = grouping_words4(p.grouping, grouping_table_word(Rk) + 4 * (int64_t)a);
    const int e = grp[0];
    const bool bad = ((int)a >= hdr[0]) | (hdr[2] != p.ncols) | (hdr[3] != p.topk) | (e < 0) |
                     (e >= p.n_local) | (grp[1] < 0) | (grp[2] < grp[1]) | (grp[2] > Rk);
    if (bad) return;
    const int begin = grp[1], end = grp[2];
    const int32_t* route = p.grouping + 4 + 2 * (int64_t)Rk + 1;

    const int64_t r0 = (int64_t)t * WG_ROWS + (int64_t)wave * WAVE_ROWS;
    const bool wave_rows = r0 < p.n;      // n is a multiple of 32, so a wave is all in or all out
    const uint8_t* wbase0 = p.w0 + (int64_t)e * p.expert_stride + (r0 + c) * p.row_stride + 8 * q;
    const uint8_t* wbase1 = PAIR ? p.w1 + (int64_t)e * p.expert_stride + (r0 + c) * p.row_stride + 8 * q
                                 : wbase0 + 16 * p.row_stride;
    const int npairs = nb >> 1;

    for (int p0 = begin; p0 < end; p0 += RT) {
        const int nr = min(end - p0, RT);
        __syncthreads();                   // the previous pass has finished reading LDS

        // the first block pairs of this wave's rows go out before the staging
        WPair ring[PF][2];
        if (wave_rows) {
#pragma unroll
            for (int s = 0; s < PF; ++s) {
                const int64_t off = (int64_t)min(s, npairs - 1) * (2 * Q80_BYTES);
                load_pair(ring[s][0], wbase0 + off);
                load_pair(ring[s][1], wbase1 + off);
            }
        }

        // stage the pass's routes: ids, then (route, block) items with the
        // route index fastest so that neighbouring lanes write neighbouring
        // 32-byte LDS slots; routes past nr stage zeros
        for (int i = tid; i < RT; i += GEMM_THREADS) {
            int r = -1;
            if (i < nr) {
                r = route[p0 + i];
                if (r < 0 || r >= Rk) r = -1;
            }
            rid[i] = r;
        }
        for (int idx = tid; idx < RT * nb; idx += GEMM_THREADS) {
            const int rho = idx % RT;
            const int b = idx / RT;
            int r = -1;
            if (rho < nr) {
                r = route[p0 + rho];
                if (r >= Rk) r = -1;
            }
            uint32_t v[9];
            if (r >= 0) {
                const int64_t arow = (int64_t)(((uint64_t)r * p.act_route_mul) >> 32);
                const uint8_t* src = p.act + arow * p.act_row_bytes + (int64_t)b * Q81_BYTES;
                const u32x4 x0 = *reinterpret_cast<const u32x4*>(src);
                const u32x4 x1 = *reinterpret_cast<const u32x4*>(src + 16);
                v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
                v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
                v[8] = *reinterpret_cast<const uint32_t*>(src + 32);
            } else {
#pragma unroll
                for (int i = 0; i < 9; ++i) v[i] = 0u;
            }
            uint4* dq = reinterpret_cast<uint4*>(aq + ((size_t)b * RT + rho) * 32);
            dq[0] = make_uint4(v[1], v[2], v[3], v[4]);
            dq[1] = make_uint4(v[5], v[6], v[7], v[8]);
            dxt[(size_t)b * RT + rho] = half_bits_to_float(v[0]);
        }
        __syncthreads();
        if (!wave_rows) continue;

        float acc[NT][2][4];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[tt][f][i] = 0.0f;

        for (int j0 = 0; j0 < npairs; j0 += PF) {
#pragma unroll
            for (int s = 0; s < PF; ++s) {
                const int j = j0 + s;
                if (j >= npairs) break;
                const WPair cur0 = ring[s][0], cur1 = ring[s][1];
                {
                    const int64_t off = (int64_t)min(j + PF, npairs - 1) * (2 * Q80_BYTES);
                    load_pair(ring[s][0], wbase0 + off);
                    load_pair(ring[s][1], wbase1 + off);
                }
                // B fragments of blocks 2j and 2j+1, and the rows' scales:
                // d of block 2j is the low half of lane (c, q=0)'s first
                // dword, d of block 2j+1 the high half of lane (c, q=3)'s third
                const WPair* cw[2] = {&cur0, &cur1};
                long wb[2][2];
                float dw[2][2];
#pragma unroll
                for (int f = 0; f < 2; ++f) {
                    const uint32_t lo = __builtin_amdgcn_alignbit(cw[f]->a1, cw[f]->a0, 16);
                    const uint32_t hi = __builtin_amdgcn_alignbit(cw[f]->a2, cw[f]->a1, 16);
                    wb[f][0] = (long)((uint64_t)lo | ((uint64_t)hi << 32));
                    wb[f][1] = (long)((uint64_t)cw[f]->b0 | ((uint64_t)cw[f]->b1 << 32));
                    const int d0 = __builtin_amdgcn_ds_bpermute(c << 2, (int)cw[f]->a0);
                    const int d1 = __builtin_amdgcn_ds_bpermute((48 + c) << 2, (int)cw[f]->a2);
                    dw[f][0] = half_bits_to_float((uint32_t)d0);
                    dw[f][1] = half_bits_to_float((uint32_t)d1 >> 16);
                }
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    if (tt * TILE_ROUTES >= nr) break;
#pragma unroll
                    for (int hb = 0; hb < 2; ++hb) {
                        const int b = 2 * j + hb;
                        const long xa = *reinterpret_cast<const long*>(
                            aq + ((size_t)b * RT + tt * TILE_ROUTES + c) * 32 + 8 * q);
                        const float4 dx = *reinterpret_cast<const float4*>(
                            dxt + (size_t)b * RT + tt * TILE_ROUTES + 4 * q);
                        const float dxv[4] = {dx.x, dx.y, dx.z, dx.w};
#pragma unroll
                        for (int f = 0; f < 2; ++f) {
                            const i32x4 z = {0, 0, 0, 0};
                            const i32x4 d = __builtin_amdgcn_mfma_i32_16x16x32_i8(xa, wb[f][hb], z, 0, 0, 0);
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                acc[tt][f][i] = fmaf((float)d[i], dw[f][hb] * dxv[i], acc[tt][f][i]);
                        }
                    }
                }
            }
        }

        // epilogue: lane (c, q) holds rows r0 + c (+16 for the second down
        // fragment) of routes 4q + i of each tile
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rho = tt * TILE_ROUTES + 4 * q + i;
                if (rho >= nr) continue;
                const int r = rid[rho];
                if (r < 0) continue;
                float* o = p.out + (int64_t)r * p.n + r0 + c;
                if constexpr (PAIR) {
                    o[0] = swiglu_ds4_f32(acc[tt][0][i], acc[tt][1][i]);
                } else {
                    o[0] = acc[tt][0][i];
                    o[16] = acc[tt][1][i];
                }
            }
        }
    }
}

size_t gemm_lds_bytes(int nt, int64_t nb) {
    const int64_t rt = (int64_t)nt * TILE_ROUTES;
    return (size_t)(nb * rt * 36 + rt * 4);
}

// Route tiles per pass: the most (up to 4) whose staging fits the LDS of two
// workgroups per CU, else one tile if it fits the CU at all.
int pick_nt(int64_t nb) {
    for (int nt = 4; nt >= 1; nt >>= 1)
        if (gemm_lds_bytes(nt, nb) <= GEMM_LDS_TARGET) return nt;
    return gemm_lds_bytes(1, nb) <= GEMM_LDS_MAX ? 1 : 0;
}

template <bool PAIR, int NT>
int launch_gemm(const GemmParams& p, int64_t grid, hipStream_t stream) {
    const size_t lds = gemm_lds_bytes(NT, p.nb);
    // dynamic LDS beyond 64 KB must be allowed per kernel first (once per
    // size reached; a second thread repeating the call is harmless)
    static std::atomic<size_t> lds_allowed{64 * 1024};
    if (lds > lds_allowed.load()) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(&k_grouped_gemm<PAIR, NT>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
            return MOEQ8_EHIP;
        lds_allowed.store(lds);
    }
    hipLaunchKernelGGL((k_grouped_gemm<PAIR, NT>), dim3((uint32_t)grid), dim3(GEMM_THREADS), lds, stream, p);
    return check_launch();
}

template <bool PAIR>
int launch_nt(int nt, const GemmParams& p, int64_t grid, hipStream_t stream) {
    switch (nt) {
        case 4: return launch_gemm<PAIR, 4>(p, grid, stream);
        case 2: return launch_gemm<PAIR, 2>(p, grid, stream);
        default: return launch_gemm<PAIR, 1>(p, grid, stream);
    }
}

int validate_weights(const void* w, int64_t row_stride, int64_t n, int64_t k) {
    if (!w) return MOEQ8_EINVAL;
    if (((uintptr_t)w & 3u) != 0 || (row_stride & 3) != 0) return MOEQ8_EALIGN;
    if (row_stride < (k / QK) * Q80_BYTES) return MOEQ8_EINVAL;
    (void)n;
    return MOEQ8_OK;
}

}  // namespace
}  // namespace moeq8

using namespace moeq8;

extern "C" int moe_grouped_gemm(int32_t stage, const void* w_a, const void* w_b,
                                int64_t expert_stride_bytes, int64_t w_row_stride_bytes,
                                int64_t n_local_expert, int64_t n, int64_t k, const void* act_q,
                                const void* grouping, int64_t ncols, int32_t topk, float* out,
                                void* stream) {
    if (stage != MOEQ8_GATE_UP_SWIGLU && stage != MOEQ8_DOWN) return MOEQ8_EINVAL;
    const bool pair = stage == MOEQ8_GATE_UP_SWIGLU;
    if (n < 0 || k <= 0 || k % 64 != 0 || n % 32 != 0) return MOEQ8_EINVAL;
    int st = validate_weights(w_a, w_row_stride_bytes, n, k);
    if (st) return st;
    if (pair) {
        st = validate_weights(w_b, w_row_stride_bytes, n, k);
        if (st) return st;
    }
    if (!act_q || !grouping || !out) return MOEQ8_EINVAL;
    if (ncols < 1 || ncols > MOEQ8_MAX_WIDE_COLS || topk < 1 || topk > MOEQ8_MAX_TOPK) return MOEQ8_EINVAL;
    if (n_local_expert < 1) return MOEQ8_EINVAL;
    if (expert_stride_bytes < 0 || (expert_stride_bytes & 3)) return MOEQ8_EALIGN;
    if (n_local_expert > 1 && expert_stride_bytes < n * w_row_stride_bytes) return MOEQ8_EINVAL;
    if (((uintptr_t)act_q & 3u) || ((uintptr_t)grouping & 3u) || ((uintptr_t)out & 3u))
        return MOEQ8_EALIGN;
    const int64_t nb = k / QK;
    const int nt = pick_nt(nb);
    if (nt == 0) return MOEQ8_EUNSUPPORTED;
    if (n == 0) return MOEQ8_OK;
    const int wg_rows = (pair ? 16 : 32) * GEMM_WAVES;
    const int64_t tiles = (n + wg_rows - 1) / wg_rows;
    const int64_t max_active = std::min<int64_t>(ncols * topk, n_local_expert);
    const int64_t grid = max_active * tiles;
    if (grid > 0x7fffffff || tiles > 0x7fffffff) return MOEQ8_EUNSUPPORTED;

    GemmParams p = {};
    p.w0 = (const uint8_t*)w_a;
    p.w1 = (const uint8_t*)w_b;
    p.expert_stride = expert_stride_bytes;
    p.row_stride = w_row_stride_bytes;
    p.n = n;
    p.n_local = n_local_expert;
    p.nb = (int32_t)nb;
    p.tiles = (int32_t)tiles;
    p.ncols = (int32_t)ncols;
    p.topk = topk;
    const uint64_t route_div = pair ? (uint64_t)topk : 1u;
    p.act_route_mul = ((1ull << 32) + route_div - 1) / route_div;
    p.act = (const uint8_t*)act_q;
    p.act_row_bytes = nb * Q81_BYTES;
    p.grouping = (const int32_t*)grouping;
    p.out = out;
    const hipStream_t hs = (hipStream_t)stream;
    return pair ? launch_nt<true>(nt, p, grid, hs) : launch_nt<false>(nt, p, grid, hs);
}
