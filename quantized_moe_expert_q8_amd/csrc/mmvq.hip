// Q8_0 x q8_1 matrix-vector products (MMVQ) for gfx950: the single product, the
// gate/up pair with the SwiGLU-DS4 epilogue, and the grouped per-expert launch.
//
// One kernel body serves all three (lucebox PR #826, the commit on MMVQ fusion
// following mul_mat's kernel choice: a fused path must run the arithmetic the
// unfused path runs).  The reduction order is fixed in moeq8_device.hpp; this
// file only decides which physical lanes compute which logical chunks.
//
// Physical layout.  A wave is 4 lane groups of 16 lanes.  Physical lane l of a
// group always holds logical lane l.  G lane groups cooperate on one row: group
// g handles absolute round r0 + g (G = 2 or 4, one round each), or G = 1 and
// the group walks all rounds of the slice in order.  A wave therefore covers
// 4/G rows per row set and U row sets, with all weight loads of the U row sets
// issued before the first dot product (the prefetching loop of the grouped MoE
// MMVQ commit: loads of several iterations first, then the dot products in the
// same order into the same accumulators).  Weights are streamed once; the q8_1
// activation chunk of a round is loaded once per column and reused by every
// row and both matrices of the pair (one load of each activation fragment).
#include "moeq8_device.hpp"
#include "moeq8_host.hpp"

namespace moeq8 {

#ifndef MOEQ8_WAVES_PER_WG
#define MOEQ8_WAVES_PER_WG 4
#endif
#ifndef MOEQ8_U_ROWSETS
#define MOEQ8_U_ROWSETS 2
#endif
constexpr int WAVES_PER_WG = MOEQ8_WAVES_PER_WG;
constexpr int MAX_COLS = 8;

struct MmvqParams {
    const uint8_t* w0;          // matrix 0 (single, gate, or grouped w_a) of expert 0 / the matrix
    const uint8_t* w1;          // matrix 1 (up) or null
    int64_t w_row_stride;       // bytes
    int64_t expert_stride;      // bytes (grouped)
    int64_t n_local;            // grouped: valid expert range
    int64_t n;                  // rows
    int32_t nchunks;            // chunks in the slice (k / 64)
    int32_t chunk0;             // absolute index of the slice's first chunk (k_block_offset / 2)
    int32_t r0;                 // first absolute round touched (chunk0 / 16)
    int32_t nsteps;             // G == 1: rounds to walk
    const uint8_t* act;         // q8_1 activation rows
    int64_t act_row_bytes;      // (k / 32) * 36
    int32_t ncols;              // dense: columns
    int32_t topk;               // grouped
    int32_t act_route_div;      // grouped: activation row of route r is r / act_route_div
    int32_t rows_per_wg;
    int32_t wg_per_expert;      // grouped
    const int32_t* grouping;    // grouped
    float* out0;                // dense: y (single) or h (pair); grouped: out rows per route
    float* out_g;               // dense pair: optional raw gate products
    float* out_u;               // dense pair: optional raw up products
};

__device__ __forceinline__ int dpp_row_mirror_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, 0x140, 0xf, 0xf, false);
}

// Pairwise tree over the 16 logical lanes of a group using DPP lane moves:
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.  The
// pairs combined at each level are the same values as an xor 1, 2, 4, 8
// butterfly (quads, then the two quads of each half, then the two halves), and
// a + b == b + a, so every lane ends with the same tree sum.
__device__ __forceinline__ float tree16(float v) {
    int iv = __float_as_int(v);
    v = v + __int_as_float(__builtin_amdgcn_update_dpp(0, iv, 0xB1, 0xf, 0xf, false));
    iv = __float_as_int(v);
    v = v + __int_as_float(__builtin_amdgcn_update_dpp(0, iv, 0x4E, 0xf, 0xf, false));
    iv = __float_as_int(v);
    v = v + __int_as_float(__builtin_amdgcn_update_dpp(0, iv, 0x141, 0xf, 0xf, false));
    iv = __float_as_int(v);
    v = v + __int_as_float(dpp_row_mirror_i(iv));
    return v;
}

// Chain the G per-round values of one logical lane in round order (group 0
// holds the earliest round), result valid in group 0.
template <int G>
__device__ __forceinline__ float chain_groups(float v, int lane) {
    if constexpr (G == 1) {
        return v;
    } else {
        float t = v;
#pragma unroll
        for (int g = 1; g < G; ++g) t = t + __shfl(v, (lane + 16 * g) & 63, 64);
        return t;
    }
}

template <int G, int NMAT, int U, bool GROUPED>
__global__ __launch_bounds__(64 * WAVES_PER_WG) void k_mmvq(const MmvqParams p) {
    constexpr int RPW = 4 / G;                         // rows per row set
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int grp = lane >> 4;                         // lane group 0..3
    const int l = lane & 15;                           // logical lane
    const int gsub = grp % G;                          // round slot within the row
    const int rslot = grp / G;                         // row slot within the row set

    const uint8_t* w0 = p.w0;
    const uint8_t* w1 = p.w1;
    int64_t row_block = blockIdx.x;
    int ncols = p.ncols;
    int route_begin = 0;
    if constexpr (GROUPED) {
        const int a = (int)(blockIdx.x / (uint32_t)p.wg_per_expert);
        row_block = blockIdx.x - (int64_t)a * p.wg_per_expert;
        const int n_active = p.grouping[0];
        if (a >= n_active) return;
        // a grouping written for another column count or top-k is not used
        if (p.grouping[2] != p.ncols || p.grouping[3] != p.topk) return;
        const int R = p.grouping[2] * p.grouping[3];
        const int e = p.grouping[4 + a];
        if (e < 0 || e >= p.n_local) return;
        route_begin = p.grouping[4 + R + a];
        ncols = p.grouping[4 + R + a + 1] - route_begin;
        if (route_begin < 0 || ncols < 0 || route_begin + ncols > R) return;
        w0 += (int64_t)e * p.expert_stride;
        if (NMAT == 2) w1 += (int64_t)e * p.expert_stride;
    }
    const int64_t row_base = row_block * p.rows_per_wg + (int64_t)wave * (U * RPW) + rslot;

    for (int c0 = 0; c0 < ncols; c0 += MAX_COLS) {
        const int nc = min(ncols - c0, MAX_COLS);
        float acc[MAX_COLS][U][NMAT];
#pragma unroll
        for (int c = 0; c < MAX_COLS; ++c)
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int m = 0; m < NMAT; ++m) acc[c][u][m] = 0.0f;

        const uint8_t* act_row[MAX_COLS];
#pragma unroll
        for (int c = 0; c < MAX_COLS; ++c) {
            int r = c0 + c;
            if constexpr (GROUPED) {
                const int R = p.grouping[2] * p.grouping[3];
                r = (c < nc) ? p.grouping[4 + 2 * R + 1 + route_begin + c0 + c] : 0;
                r = (r >= 0 && r < R) ? r / p.act_route_div : 0;
            }
            act_row[c] = p.act + (int64_t)r * p.act_row_bytes;
        }

        for (int s = 0; s < p.nsteps; ++s) {
            const int round = p.r0 + (G == 1 ? s : gsub);
            const int cabs = round * LANES_PER_ROW + l;            // absolute chunk
            const int crel = cabs - p.chunk0;                      // chunk within the slice
            const bool cvalid = (crel >= 0) && (crel < p.nchunks);

            WChunk wc[U][NMAT];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t row = row_base + (int64_t)u * RPW;
                const bool ok = cvalid && row < p.n;
#pragma unroll
                for (int m = 0; m < NMAT; ++m) {
                    if (ok) {
                        const uint8_t* base = (m == 0 ? w0 : w1) + row * p.w_row_stride +
                                              (int64_t)crel * W_CHUNK_BYTES;
                        load_w_chunk(wc[u][m], base);
                    } else {
                        zero_w_chunk(wc[u][m]);
                    }
                }
            }
#pragma unroll
            for (int c = 0; c < MAX_COLS; ++c) {
                if (c < nc) {
                    XChunk xc;
                    if (cvalid) load_x_chunk(xc, act_row[c] + (int64_t)crel * X_CHUNK_BYTES);
                    else zero_x_chunk(xc);
#pragma unroll
                    for (int u = 0; u < U; ++u)
#pragma unroll
                        for (int m = 0; m < NMAT; ++m) acc[c][u][m] += chunk_dot(wc[u][m], xc);
                }
            }
        }

        // reduce: chain the groups of a row in round order, then the 16-lane tree
#pragma unroll
        for (int c = 0; c < MAX_COLS; ++c) {
            if (c < nc) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    float v[NMAT];
#pragma unroll
                    for (int m = 0; m < NMAT; ++m) v[m] = tree16(chain_groups<G>(acc[c][u][m], lane));
                    const int64_t row = row_base + (int64_t)u * RPW;
                    // one writer lane per (column, row set) among the 16
                    const bool writer = (gsub == 0) && (l == ((c * U + u) & 15)) && row < p.n;
                    if (writer) {
                        int64_t orow;
                        if constexpr (GROUPED) {
                            const int R = p.grouping[2] * p.grouping[3];
                            orow = p.grouping[4 + 2 * R + 1 + route_begin + c0 + c];
                            if (orow < 0 || orow >= R) continue;
                        } else {
                            orow = c0 + c;
                        }
                        float* o = p.out0 + orow * p.n + row;
                        if constexpr (NMAT == 2) {
                            *o = swiglu_ds4_f32(v[0], v[1]);
                            if constexpr (!GROUPED) {
                                if (p.out_g) p.out_g[orow * p.n + row] = v[0];
                                if (p.out_u) p.out_u[orow * p.n + row] = v[1];
                            }
                        } else {
                            *o = v[0];
                        }
                    }
                }
            }
        }
    }
}

__global__ void k_swiglu_ds4(const float* g, const float* u, int64_t count, float* h) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) h[i] = swiglu_ds4_f32(g[i], u[i]);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

namespace {

constexpr int U_ROWSETS = MOEQ8_U_ROWSETS;

struct Shape {
    int G;
    int nsteps;
    int r0;
};

Shape pick_shape(int64_t chunk0, int64_t nchunks) {
    const int64_t r0 = chunk0 / LANES_PER_ROW;
    const int64_t r1 = (chunk0 + nchunks - 1) / LANES_PER_ROW;
    const int64_t rounds = r1 - r0 + 1;
    Shape s;
    s.r0 = (int)r0;
    if (rounds == 1) { s.G = 1; s.nsteps = 1; }
    else if (rounds == 2) { s.G = 2; s.nsteps = 1; }
    else if (rounds <= 4) { s.G = 4; s.nsteps = 1; }
    else { s.G = 1; s.nsteps = (int)rounds; }
    return s;
}

template <int NMAT, bool GROUPED>
int launch_mmvq(MmvqParams& p, const Shape& s, int64_t n_items_outer, hipStream_t stream) {
    const int rpw = 4 / s.G;
    p.rows_per_wg = WAVES_PER_WG * U_ROWSETS * rpw;
    p.r0 = s.r0;
    p.nsteps = s.nsteps;
    const int64_t wg_rows = (p.n + p.rows_per_wg - 1) / p.rows_per_wg;
    p.wg_per_expert = (int32_t)wg_rows;
    const int64_t grid = GROUPED ? wg_rows * n_items_outer : wg_rows;
    if (grid <= 0) return MOEQ8_OK;
    if (grid > 0x7fffffff) return MOEQ8_EUNSUPPORTED;
    const dim3 block(64 * WAVES_PER_WG);
    switch (s.G) {
        case 1: hipLaunchKernelGGL((k_mmvq<1, NMAT, U_ROWSETS, GROUPED>), dim3((uint32_t)grid), block, 0, stream, p); break;
        case 2: hipLaunchKernelGGL((k_mmvq<2, NMAT, U_ROWSETS, GROUPED>), dim3((uint32_t)grid), block, 0, stream, p); break;
        default: hipLaunchKernelGGL((k_mmvq<4, NMAT, U_ROWSETS, GROUPED>), dim3((uint32_t)grid), block, 0, stream, p); break;
    }
    return check_launch();
}

int validate_matrix(const void* w, int64_t w_row_stride_bytes, int64_t n, int64_t k,
                    int64_t k_block_offset) {
    if (!w || n < 0 || k <= 0) return MOEQ8_EINVAL;
    if (k % 64 != 0) return MOEQ8_EINVAL;
    if (k_block_offset < 0) return MOEQ8_EINVAL;
    if (k_block_offset % 2 != 0) return MOEQ8_EALIGN;
    if (((uintptr_t)w & 3u) != 0 || (w_row_stride_bytes & 3) != 0) return MOEQ8_EALIGN;
    if (n > 1 && w_row_stride_bytes < (k / QK) * Q80_BYTES) return MOEQ8_EINVAL;
    if (k / 64 > (int64_t)1 << 24 || k_block_offset > ((int64_t)1 << 26)) return MOEQ8_EUNSUPPORTED;
    return MOEQ8_OK;
}

}  // namespace
}  // namespace moeq8

using namespace moeq8;

extern "C" int mmvq_q8_0(const void* w, int64_t w_row_stride_bytes, int64_t n, int64_t k,
                         int64_t k_block_offset, const void* xq, int64_t ncols, float* y,
                         void* stream) {
    int st = validate_matrix(w, w_row_stride_bytes, n, k, k_block_offset);
    if (st) return st;
    if (!xq || !y || ncols < 1 || ncols > MAX_COLS) return MOEQ8_EINVAL;
    if (((uintptr_t)xq & 3u) || ((uintptr_t)y & 3u)) return MOEQ8_EALIGN;
    if (n == 0) return MOEQ8_OK;
    MmvqParams p = {};
    p.w0 = (const uint8_t*)w;
    p.w_row_stride = w_row_stride_bytes;
    p.n = n;
    p.nchunks = (int32_t)(k / 64);
    p.chunk0 = (int32_t)(k_block_offset / 2);
    p.act = (const uint8_t*)xq;
    p.act_row_bytes = (k / QK) * Q81_BYTES;
    p.ncols = (int32_t)ncols;
    p.out0 = y;
    return launch_mmvq<1, false>(p, pick_shape(p.chunk0, p.nchunks), 1, (hipStream_t)stream);
}

extern "C" int mmvq_q8_0_glu_pair(const void* w_gate, const void* w_up, int64_t w_row_stride_bytes,
                                  int64_t n, int64_t k, int64_t k_block_offset, const void* xq,
                                  int64_t ncols, float* h_out, float* g_out, float* u_out,
                                  void* stream) {
    int st = validate_matrix(w_gate, w_row_stride_bytes, n, k, k_block_offset);
    if (st) return st;
    st = validate_matrix(w_up, w_row_stride_bytes, n, k, k_block_offset);
    if (st) return st;
    if (!xq || !h_out || ncols < 1 || ncols > MAX_COLS) return MOEQ8_EINVAL;
    if (((uintptr_t)xq & 3u) || ((uintptr_t)h_out & 3u) || ((uintptr_t)g_out & 3u) ||
        ((uintptr_t)u_out & 3u))
        return MOEQ8_EALIGN;
    if (n == 0) return MOEQ8_OK;
    MmvqParams p = {};
    p.w0 = (const uint8_t*)w_gate;
    p.w1 = (const uint8_t*)w_up;
    p.w_row_stride = w_row_stride_bytes;
    p.n = n;
    p.nchunks = (int32_t)(k / 64);
    p.chunk0 = (int32_t)(k_block_offset / 2);
    p.act = (const uint8_t*)xq;
    p.act_row_bytes = (k / QK) * Q81_BYTES;
    p.ncols = (int32_t)ncols;
    p.out0 = h_out;
    p.out_g = g_out;
    p.out_u = u_out;
    return launch_mmvq<2, false>(p, pick_shape(p.chunk0, p.nchunks), 1, (hipStream_t)stream);
}

extern "C" int swiglu_ds4(const float* g, const float* u, int64_t count, float* h, void* stream) {
    if (count < 0 || (count > 0 && (!g || !u || !h))) return MOEQ8_EINVAL;
    if (count == 0) return MOEQ8_OK;
    const int64_t blocks = (count + 255) / 256;
    if (blocks > 0x7fffffff) return MOEQ8_EUNSUPPORTED;
    hipLaunchKernelGGL(k_swiglu_ds4, dim3((uint32_t)blocks), dim3(256), 0, (hipStream_t)stream, g,
                       u, count, h);
    return check_launch();
}

extern "C" int moe_grouped_mmvq(int32_t stage, const void* w_a, const void* w_b,
                                int64_t expert_stride_bytes, int64_t w_row_stride_bytes,
                                int64_t n_local_expert, int64_t n, int64_t k, const void* act_q,
                                const void* grouping, int64_t ncols, int32_t topk, float* out,
                                void* stream) {
    if (stage != MOEQ8_GATE_UP_SWIGLU && stage != MOEQ8_DOWN) return MOEQ8_EINVAL;
    int st = validate_matrix(w_a, w_row_stride_bytes, n, k, 0);
    if (st) return st;
    if (stage == MOEQ8_GATE_UP_SWIGLU) {
        st = validate_matrix(w_b, w_row_stride_bytes, n, k, 0);
        if (st) return st;
    }
    if (!act_q || !grouping || !out) return MOEQ8_EINVAL;
    if (ncols < 1 || ncols > MAX_COLS || topk < 1 || topk > MOEQ8_MAX_TOPK) return MOEQ8_EINVAL;
    if (n_local_expert < 1 || expert_stride_bytes < 0 || (expert_stride_bytes & 3)) {
        return n_local_expert < 1 ? MOEQ8_EINVAL : MOEQ8_EALIGN;
    }
    if (n_local_expert > 1 && expert_stride_bytes < n * w_row_stride_bytes) return MOEQ8_EINVAL;
    if (((uintptr_t)act_q & 3u) || ((uintptr_t)grouping & 3u) || ((uintptr_t)out & 3u))
        return MOEQ8_EALIGN;
    if (n == 0) return MOEQ8_OK;
    MmvqParams p = {};
    p.w0 = (const uint8_t*)w_a;
    p.w1 = (const uint8_t*)w_b;
    p.w_row_stride = w_row_stride_bytes;
    p.expert_stride = expert_stride_bytes;
    p.n_local = n_local_expert;
    p.n = n;
    p.nchunks = (int32_t)(k / 64);
    p.chunk0 = 0;
    p.act = (const uint8_t*)act_q;
    p.act_row_bytes = (k / QK) * Q81_BYTES;
    p.topk = topk;
    p.ncols = (int32_t)ncols;
    p.act_route_div = (stage == MOEQ8_GATE_UP_SWIGLU) ? topk : 1;
    p.grouping = (const int32_t*)grouping;
    p.out0 = out;
    // at most min(ncols * topk, n_local) experts are active; blocks of groups
    // past the device-side count exit at once
    const int64_t max_active = std::min<int64_t>(ncols * topk, n_local_expert);
    const Shape s = pick_shape(0, p.nchunks);
    if (stage == MOEQ8_GATE_UP_SWIGLU) return launch_mmvq<2, true>(p, s, max_active, (hipStream_t)stream);
    return launch_mmvq<1, true>(p, s, max_active, (hipStream_t)stream);
}
