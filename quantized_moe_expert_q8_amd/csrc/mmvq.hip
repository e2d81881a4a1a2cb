// Q8_0 x q8_1 matrix-vector products (MMVQ) for gfx950: the single product, the
// gate/up pair with the SwiGLU-DS4 epilogue, and the grouped per-expert launch
// (optionally with a dense product over all columns, the shared expert's
// share, as extra work items of the same launch, and optionally quantising
// fp32 activation rows to q8_1 inside the launch).
//
// One kernel body serves all of them (lucebox PR #826, the commit on MMVQ
// fusion following mul_mat's kernel choice: a fused path must run the
// arithmetic the unfused path runs).  The reduction order is fixed in
// moeq8_device.hpp; this file only decides which physical lanes compute which
// logical chunks, and the in-launch quantisation calls the same block
// quantiser as q8_1_quantize_rows, so fused and unfused launches agree bit for
// bit.
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

#include <mutex>
#include <type_traits>

namespace moeq8 {

#ifndef MOEQ8_WAVES_PER_WG
#define MOEQ8_WAVES_PER_WG 4
#endif
#ifndef MOEQ8_U_ROWSETS
#define MOEQ8_U_ROWSETS 2
#endif
#ifndef MOEQ8_U_F32
#define MOEQ8_U_F32 MOEQ8_U_ROWSETS
#endif
#ifndef MOEQ8_U_SINGLE
#define MOEQ8_U_SINGLE MOEQ8_U_ROWSETS
#endif
constexpr int WAVES_PER_WG = MOEQ8_WAVES_PER_WG;
constexpr int U_ROWSETS = MOEQ8_U_ROWSETS;          // row sets per wave: gate/up pair
constexpr int U_SINGLE = MOEQ8_U_SINGLE;            // one matrix, q8_1 activations
constexpr int U_F32 = MOEQ8_U_F32;                  // one matrix, fp32 activations
constexpr int MAX_COLS = 8;

// One matrix (or gate/up pair) and the column range of its rows that is read.
struct MatDesc {
    const uint8_t* w0;          // matrix 0 (single, gate, down)
    const uint8_t* w1;          // matrix 1 (up) or null
    int64_t row_stride;         // bytes
    int64_t n;                  // rows
    int32_t nchunks;            // chunks in the slice (k / 64)
    int32_t chunk0;             // absolute index of the slice's first chunk (k_block_offset / 2)
    int32_t r0;                 // first absolute round touched (chunk0 / 16)
    int32_t wg;                 // row blocks
};

struct MmvqParams {
    MatDesc m;                  // the matrix, or expert 0 of the routed experts
    int64_t expert_stride;      // grouped: bytes between experts
    int64_t n_local;            // grouped: valid expert range
    int32_t nsteps;             // G == 1: rounds to walk (same for m and s)
    int32_t ncols;
    int32_t topk;
    int32_t pad0;
    uint64_t act_route_mul;     // grouped: activation row of route r is (r * act_route_mul) >> 32
                                // = r / d for d = 1 (down) or topk (gate/up)
    int32_t rows_per_wg;
    int32_t max_active;         // grouped: bound on the device-side active count
    const uint8_t* act;         // q8_1 activation rows
    int64_t act_row_bytes;      // (k / 32) * 36
    const float* act_f32;       // fp32 activation rows, quantised in the launch
    int64_t act_f32_stride;     // elements
    const int32_t* grouping;    // grouped
    float* out0;                // dense: y (single) or h (pair); grouped: rows per route
    float* out_g;               // dense pair: optional raw gate products
    float* out_u;               // dense pair: optional raw up products
    // dense extra items after the routed ones (grouped launches only)
    MatDesc s;
    const uint8_t* s_act_q;     // q8_1 rows [ncols][k/32] of the dense part (q8_1 mode)
    const float* s_act_f32;     // fp32 rows [ncols][k] of the dense part (fp32 mode)
    int64_t s_act_f32_stride;
    float* s_out;               // [ncols][s.n]
};

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

// P64: the weights are in a 64-chunk packed layout (moeq8_device.hpp).  With
// four lane groups a row (G = 4) the launch reads one 64-chunk segment a row
// (K = 4096 at a segment boundary) and lane L holds chunk L of it.  With one
// lane group a row (G = 1, the down launch with fp32 activations, K = 1024
// contiguous rows of 1088 bytes) a row set is a quad of rows, 4352 contiguous
// bytes packed as one segment whose chunk L (chunk L % 16 of row L / 16) is
// again lane L's.  The packed weights are loaded nontemporally (each row is
// read once) unless REREAD: a launch whose items make several passes of
// MAX_COLS columns over the same rows takes ordinary loads, whose lines stay
// in L2 for the next pass.
//
// MC: the columns of one pass (accumulators are kept for MC columns).  A
// launch whose groups hold at most MC routes each runs one pass; decode
// launches take the smallest of 1, 2, 4, 8 that covers their columns, so
// fewer registers are held and more waves fit on a SIMD.
template <int G, int NMAT, int U, bool GROUPED, bool ACT_F32, bool STX, bool Q4, bool P64 = false,
          bool REREAD = false, int MC = MAX_COLS>
__device__ __forceinline__ void mmvq_item(const MmvqParams& p, int64_t item, uint8_t* lds_act) {
    static_assert(MC == MAX_COLS || (P64 && !REREAD), "narrow passes serve the packed decode stages");
    static_assert(!REREAD || P64, "REREAD selects the packed weights' load kind");
    static_assert(!P64 || (!STX && ((G == 4 && !ACT_F32) || (G == 1 && NMAT == 1 && ACT_F32))),
                  "the packed layouts serve the four-group gate/up rows and the one-group down quads");
    // weight chunk: two Q8_0 blocks (68 B) or two 4-bit blocks (36 B); the
    // chunk's value has the same form either way, so the reduction order and
    // every launch shape are shared
    using WC = std::conditional_t<Q4, W4Chunk, WChunk>;
    constexpr int64_t WCB = Q4 ? W4_CHUNK_BYTES : W_CHUNK_BYTES;
    constexpr int RPW = 4 / G;                         // rows per row set
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int grp = lane >> 4;                         // lane group 0..3
    const int l = lane & 15;                           // logical lane
    const int gsub = grp % G;                          // round slot within the row
    const int rslot = grp / G;                         // row slot within the row set

    // ---- decode the work item (uniform over the workgroup) ---------------
    // (fields are copied, never addressed: taking the address of the kernel
    // argument would move it to scratch memory)
    const uint8_t* w0 = p.m.w0;
    const uint8_t* w1 = p.m.w1;
    int64_t row_stride = p.m.row_stride;
    int64_t n_rows = p.m.n;
    int32_t nchunks = p.m.nchunks;
    int32_t chunk0 = p.m.chunk0;
    int32_t r0 = p.m.r0;
    const int32_t m_wg = p.m.wg;
    const int32_t s_wg = p.s.wg;
    const int64_t expert_stride = p.expert_stride;
    const int64_t n_local = p.n_local;
    const int32_t p_ncols = p.ncols;
    const int32_t p_topk = p.topk;
    const int32_t rows_per_wg = p.rows_per_wg;
    const int32_t* grouping = p.grouping;
    const uint8_t* act_q = p.act;
    const uint8_t* s_act_q = p.s_act_q;
    float* out0 = p.out0;
    float* s_out = p.s_out;
    const int64_t act_row_bytes = p.act_row_bytes;
    const uint64_t act_route_mul = p.act_route_mul;
    const int32_t nsteps = p.nsteps;
    // The arguments the decode and the first loads need arrive in one batch
    // of scalar loads at entry; left alone, the compiler fetches each after
    // the branch that first uses it, one round trip at a time.
    asm volatile("" ::"s"(w0), "s"(w1), "s"(row_stride), "s"(n_rows), "s"(nchunks), "s"(chunk0),
                 "s"(r0), "s"(m_wg), "s"(s_wg), "s"(expert_stride), "s"(n_local), "s"(p_ncols),
                 "s"(p_topk), "s"(rows_per_wg), "s"(grouping), "s"(act_q), "s"(s_act_q), "s"(out0),
                 "s"(s_out), "s"(act_row_bytes), "s"(act_route_mul), "s"(nsteps));
    int64_t row_block = item;
    int ncols = p_ncols;
    int route_begin = 0;
    int R = 0;
    bool routed = false;
    if constexpr (GROUPED) {
        // the dense part's items come first: its blocks carry every column, so
        // dispatching them early keeps them out of the launch's tail
        const uint32_t n_dense = (uint32_t)s_wg;       // grids stay below 2^31 items
        const uint32_t it = (uint32_t)item;
        if (it >= n_dense) {
            const uint32_t wgm = (uint32_t)m_wg;
            const uint32_t a = (it - n_dense) / wgm;
            row_block = (int64_t)(it - n_dense - a * wgm);
            // The header and the group's table entry {expert, first route,
            // end} in two scalar reads issued together, before any check: the
            // grid holds at most min(ncols*topk, n_local) groups, so a < R and
            // both reads are inside the grouping whatever it holds.
            const int Rk = p_ncols * p_topk;
            const int4w hdr = grouping_words4(grouping, 0);
            const int4w grp = grouping_words4(grouping, grouping_table_word(Rk) + 4 * (int64_t)a);
            const int e = grp[0];
            // one combined check (no short-circuit): a past the active count, a
            // grouping written for another column count or top-k, an expert or
            // route range out of bounds
            const bool bad = ((int)a >= hdr[0]) | (hdr[2] != p_ncols) | (hdr[3] != p_topk) |
                             (e < 0) | (e >= n_local) | (grp[1] < 0) | (grp[2] < grp[1]) |
                             (grp[2] > Rk);
            if (bad) return;
            R = Rk;
            route_begin = grp[1];
            ncols = grp[2] - grp[1];
            w0 += (int64_t)e * expert_stride;
            if (NMAT == 2) w1 += (int64_t)e * expert_stride;
            routed = true;
        } else {
            row_block = item;
            w0 = p.s.w0;
            w1 = p.s.w1;
            row_stride = p.s.row_stride;
            n_rows = p.s.n;
            nchunks = p.s.nchunks;
            chunk0 = p.s.chunk0;
            r0 = p.s.r0;
        }
    }
    const int64_t row_base = row_block * rows_per_wg + (int64_t)wave * (U * RPW) + rslot;

    for (int c0 = 0; c0 < ncols; c0 += MC) {
        const int nc = min(ncols - c0, MC);
        float acc[MC][U][NMAT];
#pragma unroll
        for (int c = 0; c < MC; ++c)
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int m = 0; m < NMAT; ++m) acc[c][u][m] = 0.0f;

        // A lane whose chunk or row lies outside the matrix contributes +0.
        // With q8_1 activations it skips the loads and uses zero chunks.  With
        // fp32 activations every load is issued (such a lane reads chunk 0 of
        // row 0 and adds +0 in place of its product): a cleared register with
        // a load in flight would make the activation quantisation wait for the
        // weight loads as well.
        constexpr bool UNCOND = ACT_F32;
        WC wc[U][NMAT];
        int crel = 0;                                      // chunk within the slice (clamped)
        bool cvalid = false;
        bool ok[U];
        auto load_weights = [&](int s) {
            const int round = r0 + (G == 1 ? s : gsub);
            const int cr = round * LANES_PER_ROW + l - chunk0;
            cvalid = (cr >= 0) && (cr < nchunks);
            crel = cvalid ? cr : 0;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t row = row_base + (int64_t)u * RPW;
                ok[u] = cvalid && row < n_rows;
                const int64_t off = ok[u] ? row * row_stride + (int64_t)crel * WCB : 0;
#pragma unroll
                for (int m = 0; m < NMAT; ++m) {
                    if constexpr (P64 && G == 1) {
                        // the quad of this row set (n % 4 == 0: a quad is inside
                        // the matrix or wholly past it, and then reads the first
                        // quad and adds +0, as every unconditional load does)
                        const int64_t quad = ok[u] ? row - rslot : 0;
                        load_w_chunk_p64<!REREAD>(wc[u][m], w0 + quad * row_stride, lane);
                    } else if constexpr (P64) {
                        if (ok[u]) load_w_chunk_p64<!REREAD>(wc[u][m], (m == 0 ? w0 : w1) + row * row_stride, crel);
                        else zero_w_chunk(wc[u][m]);
                    } else if (UNCOND || ok[u]) {
                        load_w_chunk(wc[u][m], (m == 0 ? w0 : w1) + off);
                    } else {
                        zero_w_chunk(wc[u][m]);
                    }
                }
            }
        };

        // With q8_1 activations the weight loads go out first: the route read
        // below is a scalar load, which does not wait for them.
        if constexpr (!ACT_F32) load_weights(0);

        // output row and activation row of each column of this pass
        int orow[MC];
        int arow[MC];
        int8w w8 = {};
        if constexpr (GROUPED) {
            // the route entries of this pass as one eight-word read (words
            // past the pass's nc columns are read but not used)
            if (routed) w8 = grouping_words8(grouping, 4 + 2 * R + 1 + route_begin + c0);
#pragma unroll
            for (int c = 0; c < MC; ++c) {
                const int r = (c >= nc || w8[c] < 0 || w8[c] >= R) ? -1 : w8[c];
                orow[c] = routed ? r : c0 + c;
                arow[c] = routed ? (r < 0 ? 0 : (int)(((uint64_t)r * act_route_mul) >> 32)) : c0 + c;
            }
        } else {
#pragma unroll
            for (int c = 0; c < MC; ++c) {
                orow[c] = c0 + c;
                arow[c] = c0 + c;
            }
        }

        const uint8_t* act_base = (GROUPED && !routed) ? s_act_q : act_q;
        if constexpr (STX && !ACT_F32) {
            // Copy this pass's q8_1 activation chunks into LDS once for the
            // workgroup (column c at c * act_row_bytes), with 16-byte
            // coalesced loads straight into LDS, the waves taking turns by
            // 1 KB.  Read per lane from global memory instead, every wave
            // would fetch the same bytes, 72 scattered bytes per lane.  The
            // host stages only rows of a multiple of 16 bytes, so no piece
            // straddles two columns.
            __syncthreads();                               // a previous pass may still read LDS
            const int total = nc * (int)act_row_bytes;
            for (int k = wave; k * 1024 < total; k += WAVES_PER_WG) {
                const int pos = k * 1024 + lane * 16;
                int c = 0;
#pragma unroll
                for (int q = 1; q < MC; ++q) c += (pos >= q * (int)act_row_bytes) ? 1 : 0;
                int ar = c0 + c;
                if (routed) {
                    const int r = w8[c];                   // c < nc wherever pos < total
                    ar = (r < 0 || r >= R) ? 0 : (int)(((uint64_t)r * act_route_mul) >> 32);
                }
                if (pos < total)
                    __builtin_amdgcn_global_load_lds(
                        (const void*)(act_base + (int64_t)ar * act_row_bytes + (pos - c * (int)act_row_bytes)),
                        (void*)(lds_act + k * 1024), 16, 0, 0);
            }
            // this wave's copies (and the weight loads issued before them)
            // have landed; after the barrier so have everyone's
            __builtin_amdgcn_s_waitcnt(0x0F70);            // vmcnt(0)
            __syncthreads();
            act_base = lds_act;
        }
        if constexpr (ACT_F32) {
            // Quantise this item's activation rows into LDS with the block rule
            // of q8_1_quantize_rows.  Two neighbouring lanes share a block, 16
            // values each, so fewer registers are held across the weight
            // loads.  The first pass's values are loaded before the weights:
            // quantising waits for them alone (loads complete in issue order)
            // while the weight loads are still in flight.
            __syncthreads();                               // a previous pass may still read LDS
            const int nb = nchunks * 2;
            const int units = nc * nb * 2;                 // half blocks
            const float* src = routed ? p.act_f32 : p.s_act_f32;
            const int64_t stride = routed ? p.act_f32_stride : p.s_act_f32_stride;
            float v[QK / 2];
            auto load_half = [&](int u) {
                if (u < units) {
                    const int blk = u >> 1;
                    const int c = blk / nb;
                    const int b = blk - c * nb;
                    int ar = c0 + c;
                    if (routed) {
                        const int r = w8[c];               // c < nc here
                        ar = (r < 0 || r >= R) ? 0 : (int)(((uint64_t)r * act_route_mul) >> 32);
                    }
                    const float* sp = src + (int64_t)ar * stride + (int64_t)b * QK + (u & 1) * (QK / 2);
#pragma unroll
                    for (int i = 0; i < QK / 2; ++i) v[i] = sp[i];
                } else {
#pragma unroll
                    for (int i = 0; i < QK / 2; ++i) v[i] = 0.0f;
                }
            };
            constexpr int THREADS = 64 * WAVES_PER_WG;     // the launch's block size
            const int passes = (units + THREADS - 1) / THREADS;
            load_half(threadIdx.x);
            load_weights(0);
            for (int ps = 0; ps < passes; ++ps) {          // uniform: every lane takes part
                const int u = ps * THREADS + (int)threadIdx.x;
                if (ps > 0) load_half(u);
                const int blk = u >> 1;
                const int c = blk / nb;
                quantize_half_q81(v, u & 1, u < units,
                                  lds_act + (int64_t)c * act_row_bytes + (int64_t)(blk - c * nb) * Q81_BYTES);
            }
            __syncthreads();
            act_base = lds_act;
        }

        for (int s = 0; s < nsteps; ++s) {
            if (s > 0) load_weights(s);
#pragma unroll
            for (int c = 0; c < MC; ++c) {
                if (c < nc) {
                    XChunk xc;
                    if constexpr (ACT_F32 || STX) {
                        // staged in LDS (a lane outside the matrix reads
                        // chunk 0 of the column and adds +0 below)
                        load_x_chunk_lds(xc, act_base + (int64_t)c * act_row_bytes +
                                                 (int64_t)crel * X_CHUNK_BYTES);
                    } else if (cvalid) {
                        load_x_chunk(xc, act_base + (int64_t)arow[c] * act_row_bytes +
                                             (int64_t)crel * X_CHUNK_BYTES);
                    } else {
                        zero_x_chunk(xc);
                    }
                    [[maybe_unused]] XBias xb{0, 0};
                    if constexpr (Q4) xb = q4_x_bias(xc);      // once per column, for every row set
#pragma unroll
                    for (int u = 0; u < U; ++u)
#pragma unroll
                        for (int m = 0; m < NMAT; ++m) {
                            float d;
                            if constexpr (Q4) d = chunk_dot(wc[u][m], xc, xb);
                            else d = chunk_dot(wc[u][m], xc);
                            acc[c][u][m] += ((UNCOND || STX) && !ok[u]) ? 0.0f : d;
                        }
                }
            }
        }

        // reduce: chain the groups of a row in round order, then the 16-lane tree
        float* out = (GROUPED && !routed) ? s_out : out0;
        if constexpr (MC * U <= 16) {
            // Every lane of the 16 ends the tree with every (column, row set)
            // value, and each such pair has a lane of its own (lane c*U + u):
            // each lane keeps its pair's values and finishes it alone, so the
            // epilogue (SwiGLU, the store) runs once per lane instead of once
            // per pair.
            float sel[NMAT];
#pragma unroll
            for (int m = 0; m < NMAT; ++m) sel[m] = 0.0f;
            int sel_orow = -1;
            int sel_u = 0;
#pragma unroll
            for (int c = 0; c < MC; ++c) {
                if (c < nc) {
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const bool mine = l == c * U + u;
#pragma unroll
                        for (int m = 0; m < NMAT; ++m) {
                            const float v = tree16(chain_groups<G>(acc[c][u][m], lane));
                            sel[m] = mine ? v : sel[m];
                        }
                        sel_orow = mine ? orow[c] : sel_orow;
                        sel_u = mine ? u : sel_u;
                    }
                }
            }
            const int64_t row = row_base + (int64_t)sel_u * RPW;
            if (gsub == 0 && sel_orow >= 0 && row < n_rows) {
                const int64_t at = (int64_t)sel_orow * n_rows + row;
                if constexpr (NMAT == 2) {
                    out[at] = swiglu_ds4_f32(sel[0], sel[1]);
                    if constexpr (!GROUPED) {
                        if (p.out_g) p.out_g[at] = sel[0];
                        if (p.out_u) p.out_u[at] = sel[1];
                    }
                } else {
                    out[at] = sel[0];
                }
            }
            continue;
        }
#pragma unroll
        for (int c = 0; c < MC; ++c) {
            if (c < nc) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    float v[NMAT];
#pragma unroll
                    for (int m = 0; m < NMAT; ++m) v[m] = tree16(chain_groups<G>(acc[c][u][m], lane));
                    const int64_t row = row_base + (int64_t)u * RPW;
                    // one writer lane per (column, row set) among the 16
                    const bool writer = (gsub == 0) && (l == ((c * U + u) & 15)) && row < n_rows;
                    if (writer && orow[c] >= 0) {
                        float* o = out + (int64_t)orow[c] * n_rows + row;
                        if constexpr (NMAT == 2) {
                            *o = swiglu_ds4_f32(v[0], v[1]);
                            if constexpr (!GROUPED) {
                                if (p.out_g) p.out_g[(int64_t)orow[c] * n_rows + row] = v[0];
                                if (p.out_u) p.out_u[(int64_t)orow[c] * n_rows + row] = v[1];
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

// One work item = one row block: of one active expert (grouped), of the dense
// extra matrix (grouped launches with a shared part), or of the one matrix.
template <int G, int NMAT, int U, bool GROUPED, bool ACT_F32, bool STX, bool Q4, bool P64 = false,
          bool REREAD = false, int MC = MAX_COLS>
__global__ __launch_bounds__(64 * WAVES_PER_WG) void k_mmvq(const MmvqParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_act[];
    mmvq_item<G, NMAT, U, GROUPED, ACT_F32, STX, Q4, P64, REREAD, MC>(p, blockIdx.x, lds_act);
}

__global__ void k_swiglu_ds4(const float* g, const float* u, int64_t count, float* h) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) h[i] = swiglu_ds4_f32(g[i], u[i]);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

namespace {

struct Shape {
    int G;
    int nsteps;
};

Shape pick_shape(int64_t chunk0, int64_t nchunks) {
    const int64_t r0 = chunk0 / LANES_PER_ROW;
    const int64_t r1 = (chunk0 + nchunks - 1) / LANES_PER_ROW;
    const int64_t rounds = r1 - r0 + 1;
    if (rounds == 1) return {1, 1};
    if (rounds == 2) return {2, 1};
    if (rounds <= 4) return {4, 1};
    return {1, (int)rounds};
}

MatDesc make_desc(const void* w0, const void* w1, int64_t row_stride, int64_t n, int64_t k,
                  int64_t k_block_offset, int rows_per_wg) {
    MatDesc d = {};
    d.w0 = (const uint8_t*)w0;
    d.w1 = (const uint8_t*)w1;
    d.row_stride = row_stride;
    d.n = n;
    d.nchunks = (int32_t)(k / 64);
    d.chunk0 = (int32_t)(k_block_offset / 2);
    d.r0 = d.chunk0 / LANES_PER_ROW;
    d.wg = (int32_t)((n + rows_per_wg - 1) / rows_per_wg);
    return d;
}

#ifndef MOEQ8_U_Q4_SCALE
#define MOEQ8_U_Q4_SCALE 1
#endif
constexpr int u_for(int nmat, bool act_f32, bool q4 = false) {
    return (nmat == 2 ? U_ROWSETS : act_f32 ? U_F32 : U_SINGLE) * (q4 ? MOEQ8_U_Q4_SCALE : 1);
}

int rows_per_wg_for(const Shape& s, int u) { return WAVES_PER_WG * u * (4 / s.G); }

// row sets a wave of the packed gate/up takes for passes of 1-2 columns
constexpr int P64_SMALL_U = 1;

template <int NMAT, bool GROUPED, bool ACT_F32, bool STX, bool Q4, int U = u_for(NMAT, ACT_F32, Q4)>
int launch_shape(MmvqParams& p, const Shape& s, int64_t grid, size_t lds_bytes, hipStream_t stream) {
    const dim3 block(64 * WAVES_PER_WG);
    switch (s.G) {
        case 1: hipLaunchKernelGGL((k_mmvq<1, NMAT, U, GROUPED, ACT_F32, STX, Q4>), dim3((uint32_t)grid), block, lds_bytes, stream, p); break;
        case 2: hipLaunchKernelGGL((k_mmvq<2, NMAT, U, GROUPED, ACT_F32, STX, Q4>), dim3((uint32_t)grid), block, lds_bytes, stream, p); break;
        default: hipLaunchKernelGGL((k_mmvq<4, NMAT, U, GROUPED, ACT_F32, STX, Q4>), dim3((uint32_t)grid), block, lds_bytes, stream, p); break;
    }
    return check_launch();
}

// the grouped gate/up pair on 64-chunk packed weights (four lane groups a
// row), and the grouped down with fp32 activations on quad-packed weights (one
// lane group a row)
template <bool Q4>
int launch_p64(bool down, MmvqParams& p, const Shape& s, int64_t grid, size_t lds, hipStream_t stream) {
    p.nsteps = s.nsteps;
    if (grid <= 0) return MOEQ8_OK;
    if (grid > 0x7fffffff) return MOEQ8_EUNSUPPORTED;
    // a grouping wider than one pass can give an expert several passes
    const bool reread = p.ncols > MAX_COLS;
    const dim3 block(64 * WAVES_PER_WG);
    const dim3 g((uint32_t)grid);
    // a decode grouping's groups hold at most ncols routes (top-k picks
    // distinct experts per column), so one pass of the next power of two
    // covers them
    const int mc = p.ncols <= 1 ? 1 : p.ncols <= 2 ? 2 : p.ncols <= 4 ? 4 : 8;
    if (down) {
        constexpr int U = u_for(1, true, Q4);
        if (reread) hipLaunchKernelGGL((k_mmvq<1, 1, U, true, true, false, Q4, true, true>), g, block, lds, stream, p);
        else if (mc == 1) hipLaunchKernelGGL((k_mmvq<1, 1, U, true, true, false, Q4, true, false, 1>), g, block, lds, stream, p);
        else if (mc == 2) hipLaunchKernelGGL((k_mmvq<1, 1, U, true, true, false, Q4, true, false, 2>), g, block, lds, stream, p);
        else if (mc == 4) hipLaunchKernelGGL((k_mmvq<1, 1, U, true, true, false, Q4, true, false, 4>), g, block, lds, stream, p);
        else hipLaunchKernelGGL((k_mmvq<1, 1, U, true, true, false, Q4, true>), g, block, lds, stream, p);
    } else {
        constexpr int U = u_for(2, false, Q4);
        constexpr int US = P64_SMALL_U;                 // passes of 1-2 columns (the host sized the grid so)
        if (reread) hipLaunchKernelGGL((k_mmvq<4, 2, U, true, false, false, Q4, true, true>), g, block, 0, stream, p);
        else if (mc == 1) hipLaunchKernelGGL((k_mmvq<4, 2, US, true, false, false, Q4, true, false, 1>), g, block, 0, stream, p);
        else if (mc == 2) hipLaunchKernelGGL((k_mmvq<4, 2, US, true, false, false, Q4, true, false, 2>), g, block, 0, stream, p);
        else if (mc == 4) hipLaunchKernelGGL((k_mmvq<4, 2, U, true, false, false, Q4, true, false, 4>), g, block, 0, stream, p);
        else hipLaunchKernelGGL((k_mmvq<4, 2, U, true, false, false, Q4, true>), g, block, 0, stream, p);
    }
    return check_launch();
}

// LDS for q8_1 activations staged per workgroup (ncols rows of the slice),
// or 0 when staging does not pay or does not fit.  Staging pays when one work
// item carries many columns (measured on a 1024-row pair at K = 4096 with 8
// columns: 9.4 -> 8.1 us; with 1 column it costs 6%), so it is used for the
// dense launches from 4 columns on.  A grouped launch's routed items carry
// about ncols*topk / active-expert columns (1-2 at 8 columns, top-8), where
// staging measured slower, so grouped launches never stage.  Rows must be a
// whole number of 16-byte pieces and all rows must fit in 64 KB.
size_t staged_act_bytes(bool grouped, int64_t ncols, int64_t act_row_bytes) {
    const int64_t bytes = ncols * act_row_bytes;
    const bool stage = !grouped && ncols >= 4 && act_row_bytes % 16 == 0 && bytes <= 64 * 1024;
    return stage ? (size_t)bytes : 0;
}

template <int NMAT, bool GROUPED, bool ACT_F32, bool Q4>
int launch_mmvq(MmvqParams& p, const Shape& s, int64_t grid, size_t lds_bytes, hipStream_t stream) {
    p.nsteps = s.nsteps;
    if (grid <= 0) return MOEQ8_OK;
    if (grid > 0x7fffffff) return MOEQ8_EUNSUPPORTED;
    if constexpr (ACT_F32) {
        return launch_shape<NMAT, GROUPED, true, false, Q4>(p, s, grid, lds_bytes, stream);
    } else if constexpr (!GROUPED) {
        // a dense launch has one pass of p.ncols <= MAX_COLS columns
        const size_t staged = staged_act_bytes(false, p.ncols, p.act_row_bytes);
        if (staged) return launch_shape<NMAT, false, false, true, Q4>(p, s, grid, staged, stream);
        return launch_shape<NMAT, false, false, false, Q4>(p, s, grid, 0, stream);
    } else {
        return launch_shape<NMAT, true, false, false, Q4>(p, s, grid, 0, stream);
    }
}

int validate_matrix(const void* w, int64_t w_row_stride_bytes, int64_t n, int64_t k,
                    int64_t k_block_offset, int64_t block_bytes = Q80_BYTES) {
    if (!w || n < 0 || k <= 0) return MOEQ8_EINVAL;
    if (k % 64 != 0) return MOEQ8_EINVAL;
    if (k_block_offset < 0) return MOEQ8_EINVAL;
    if (k_block_offset % 2 != 0) return MOEQ8_EALIGN;
    if (((uintptr_t)w & 3u) != 0 || (w_row_stride_bytes & 3) != 0) return MOEQ8_EALIGN;
    if (n > 1 && w_row_stride_bytes < (k / QK) * block_bytes) return MOEQ8_EINVAL;
    if (k / 64 > ((int64_t)1 << 24) || k_block_offset > ((int64_t)1 << 26)) return MOEQ8_EUNSUPPORTED;
    if (n > ((int64_t)1 << 31)) return MOEQ8_EUNSUPPORTED;
    return MOEQ8_OK;
}

int dense_call(int nmat, const void* w0, const void* w1, int64_t stride, int64_t n, int64_t k,
               int64_t kb, const void* xq, int64_t ncols, float* out, float* g, float* u,
               void* stream, bool q4 = false) {
    MmvqParams p = {};
    const Shape s = pick_shape(kb / 2, k / 64);
    p.rows_per_wg = rows_per_wg_for(s, u_for(nmat, false, q4));
    p.m = make_desc(w0, w1, stride, n, k, kb, p.rows_per_wg);
    p.act = (const uint8_t*)xq;
    p.act_row_bytes = (k / QK) * Q81_BYTES;
    p.ncols = (int32_t)ncols;
    p.out0 = out;
    p.out_g = g;
    p.out_u = u;
    const hipStream_t hs = (hipStream_t)stream;
    if (q4) {
        if (nmat == 2) return launch_mmvq<2, false, false, true>(p, s, p.m.wg, 0, hs);
        return launch_mmvq<1, false, false, true>(p, s, p.m.wg, 0, hs);
    }
    if (nmat == 2) return launch_mmvq<2, false, false, false>(p, s, p.m.wg, 0, hs);
    return launch_mmvq<1, false, false, false>(p, s, p.m.wg, 0, hs);
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
    return dense_call(1, w, nullptr, w_row_stride_bytes, n, k, k_block_offset, xq, ncols, y, nullptr,
                      nullptr, stream);
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
    return dense_call(2, w_gate, w_up, w_row_stride_bytes, n, k, k_block_offset, xq, ncols, h_out,
                      g_out, u_out, stream);
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

namespace moeq8 {
namespace {
// A grouped launch's parameters, grid and LDS, after the host checks.
struct GroupedLaunch {
    MmvqParams p;
    Shape s;
    int64_t grid;
    size_t lds;
    bool pair, f32, p64, p64d;
};

int prepare_grouped(GroupedLaunch& L, bool q4, int32_t stage, const void* w_a, const void* w_b,
                    int64_t expert_stride_bytes, int64_t w_row_stride_bytes,
                    int64_t n_local_expert, int64_t n, int64_t k, const void* act,
                    int64_t act_row_stride, const void* grouping, int64_t ncols,
                    int32_t topk, float* out, const void* s_a, const void* s_b,
                    int64_t s_row_stride_bytes, int64_t s_n, int64_t s_k,
                    int64_t s_k_block_offset, const void* s_act,
                    int64_t s_act_row_stride, float* s_out) {
    const int64_t bb = q4 ? Q4_BYTES : Q80_BYTES;
    if (stage != MOEQ8_GATE_UP_SWIGLU && stage != MOEQ8_DOWN && stage != MOEQ8_DOWN_F32_ACT &&
        stage != MOEQ8_GATE_UP_SWIGLU_P64 && stage != MOEQ8_DOWN_F32_ACT_P64)
        return MOEQ8_EINVAL;
    const bool p64 = stage == MOEQ8_GATE_UP_SWIGLU_P64;
    const bool p64d = stage == MOEQ8_DOWN_F32_ACT_P64;
    const bool pair = stage == MOEQ8_GATE_UP_SWIGLU || p64;
    const bool f32 = stage == MOEQ8_DOWN_F32_ACT || p64d;
    int st = validate_matrix(w_a, w_row_stride_bytes, n, k, 0, bb);
    if (st) return st;
    if (pair) {
        st = validate_matrix(w_b, w_row_stride_bytes, n, k, 0, bb);
        if (st) return st;
    }
    if (!act || !grouping || !out) return MOEQ8_EINVAL;
    // wide groupings (moe_group_routes) too: an item takes its routes in
    // passes of MAX_COLS columns
    if (ncols < 1 || ncols > MOEQ8_MAX_WIDE_COLS || topk < 1 || topk > MOEQ8_MAX_TOPK) return MOEQ8_EINVAL;
    if (n_local_expert < 1) return MOEQ8_EINVAL;
    if (expert_stride_bytes < 0 || (expert_stride_bytes & 3)) return MOEQ8_EALIGN;
    if (n_local_expert > 1 && expert_stride_bytes < n * w_row_stride_bytes) return MOEQ8_EINVAL;
    if (((uintptr_t)act & 3u) || ((uintptr_t)grouping & 3u) || ((uintptr_t)out & 3u))
        return MOEQ8_EALIGN;
    if (f32 && act_row_stride < k) return MOEQ8_EINVAL;
    const bool has_s = s_a != nullptr;
    if (has_s) {
        // the shared part runs in the same kernel instance: same k and slice shape
        if (s_k != k) return MOEQ8_EUNSUPPORTED;
        st = validate_matrix(s_a, s_row_stride_bytes, s_n, k, s_k_block_offset, bb);
        if (st) return st;
        if (pair) {
            st = validate_matrix(s_b, s_row_stride_bytes, s_n, k, s_k_block_offset, bb);
            if (st) return st;
        }
        if (!s_out) return MOEQ8_EINVAL;
        if ((uintptr_t)s_out & 3u) return MOEQ8_EALIGN;
        if (f32 && (!s_act || s_act_row_stride < k)) return MOEQ8_EINVAL;
        if ((uintptr_t)s_act & 3u) return MOEQ8_EALIGN;
        const Shape a = pick_shape(0, k / 64), b = pick_shape(s_k_block_offset / 2, k / 64);
        if (a.G != b.G || a.nsteps != b.nsteps) return MOEQ8_EUNSUPPORTED;
    }
    if (p64) {
        // one 64-chunk segment a row, 16-byte aligned segments
        if (k != P64_CHUNKS * 2 * QK) return MOEQ8_EUNSUPPORTED;
        if (((uintptr_t)w_a | (uintptr_t)w_b | (uint64_t)w_row_stride_bytes | (uint64_t)expert_stride_bytes) & 15u)
            return MOEQ8_EALIGN;
        if (has_s) {
            if (s_k_block_offset % (P64_CHUNKS * 2) != 0) return MOEQ8_EALIGN;
            if (((uintptr_t)s_a | (uintptr_t)s_b | (uint64_t)s_row_stride_bytes) & 15u) return MOEQ8_EALIGN;
        }
    }
    if (p64d) {
        // contiguous rows of one 16-chunk round (a quad is one 64-chunk
        // packed segment: 4352 bytes in Q8_0, 2304 in 4-bit), 16-byte aligned
        const int64_t ROUND_BYTES = (q4 ? P64Q4_SEGMENT_BYTES : P64_SEGMENT_BYTES) / 4;   // 1088 / 576
        if (k != LANES_PER_ROW * 2 * QK || n % 4 != 0 || (has_s && s_n % 4 != 0)) return MOEQ8_EUNSUPPORTED;
        if (w_row_stride_bytes != ROUND_BYTES || (has_s && (s_row_stride_bytes != ROUND_BYTES || s_k_block_offset != 0)))
            return MOEQ8_EUNSUPPORTED;
        if (((uintptr_t)w_a | (uint64_t)expert_stride_bytes | (uintptr_t)s_a) & 15u) return MOEQ8_EALIGN;
    }
    L.grid = 0;                                    // nothing to launch unless set below
    if (n == 0 && (!has_s || s_n == 0)) return MOEQ8_OK;

    MmvqParams p = {};
    const Shape s = pick_shape(0, k / 64);
    // the packed gate/up takes one row set a wave for passes of 1-2 columns
    // (twice the workgroups, each finishing sooner: 13.08 -> 12.85 us at one
    // column, 23.29 -> 22.61 at two); the down keeps two at every width (one
    // measured 7.72 -> 8.30 us at one column)
    p.rows_per_wg = rows_per_wg_for(s, (p64 && ncols <= 2) ? P64_SMALL_U : u_for(pair ? 2 : 1, f32, q4));
    p.m = make_desc(w_a, w_b, w_row_stride_bytes, n, k, 0, p.rows_per_wg);
    p.expert_stride = expert_stride_bytes;
    p.n_local = n_local_expert;
    p.ncols = (int32_t)ncols;
    p.topk = topk;
    // route r's activation row is r / d, d = topk for gate/up (a column per
    // route group) or 1 for down (a row per route); r < ncols*topk <= 2^14
    // and d <= 16, where (r * ceil(2^32 / d)) >> 32 is exactly r / d (the
    // multiplier's excess adds under 2^14/2^32 to r/d, whose fractional part
    // is at most 15/16)
    const uint64_t route_div = pair ? (uint64_t)topk : 1u;
    p.act_route_mul = ((1ull << 32) + route_div - 1) / route_div;
    p.act = (const uint8_t*)act;
    p.act_row_bytes = (k / QK) * Q81_BYTES;
    if (f32) {
        p.act_f32 = (const float*)act;
        p.act_f32_stride = act_row_stride;
    }
    p.grouping = (const int32_t*)grouping;
    p.out0 = out;
    // at most min(ncols * topk, n_local) experts are active; blocks of groups
    // past the device-side count exit at once
    const int64_t max_active = std::min<int64_t>(ncols * topk, n_local_expert);
    p.max_active = (int32_t)max_active;
    int64_t grid = max_active * p.m.wg;
    if (has_s) {
        p.s = make_desc(s_a, s_b, s_row_stride_bytes, s_n, k, s_k_block_offset, p.rows_per_wg);
        if (f32) {
            p.s_act_f32 = (const float*)s_act;
            p.s_act_f32_stride = s_act_row_stride;
        } else {
            // q8_1 rows of the dense part: s_act, or act rows 0..ncols-1
            p.s_act_q = s_act ? (const uint8_t*)s_act : (const uint8_t*)act;
        }
        p.s_out = s_out;
        grid += p.s.wg;
    }
    const size_t lds = f32 ? (size_t)MAX_COLS * (size_t)p.act_row_bytes : 0;
    if (lds > 64 * 1024) return MOEQ8_EUNSUPPORTED;
    p.nsteps = s.nsteps;
    L.p = p;
    L.s = s;
    L.grid = grid;
    L.lds = lds;
    L.pair = pair;
    L.f32 = f32;
    L.p64 = p64;
    L.p64d = p64d;
    return MOEQ8_OK;
}

int grouped_impl(bool q4, int32_t stage, const void* w_a, const void* w_b,
                 int64_t expert_stride_bytes, int64_t w_row_stride_bytes,
                 int64_t n_local_expert, int64_t n, int64_t k, const void* act,
                 int64_t act_row_stride, const void* grouping, int64_t ncols,
                 int32_t topk, float* out, const void* s_a, const void* s_b,
                 int64_t s_row_stride_bytes, int64_t s_n, int64_t s_k,
                 int64_t s_k_block_offset, const void* s_act,
                 int64_t s_act_row_stride, float* s_out, void* stream) {
    GroupedLaunch L;
    const int st = prepare_grouped(L, q4, stage, w_a, w_b, expert_stride_bytes, w_row_stride_bytes,
                                   n_local_expert, n, k, act, act_row_stride, grouping, ncols, topk, out,
                                   s_a, s_b, s_row_stride_bytes, s_n, s_k, s_k_block_offset, s_act,
                                   s_act_row_stride, s_out);
    if (st != MOEQ8_OK) return st;
    if (n == 0 && (!s_a || s_n == 0)) return MOEQ8_OK;
    MmvqParams& p = L.p;
    const Shape& s = L.s;
    const int64_t grid = L.grid;
    const size_t lds = L.lds;
    const hipStream_t hs = (hipStream_t)stream;
    if (q4) {
        if (L.p64 || L.p64d) return launch_p64<true>(L.p64d, p, s, grid, lds, hs);
        if (L.pair) return launch_mmvq<2, true, false, true>(p, s, grid, 0, hs);
        if (L.f32) return launch_mmvq<1, true, true, true>(p, s, grid, lds, hs);
        return launch_mmvq<1, true, false, true>(p, s, grid, 0, hs);
    }
    if (L.p64 || L.p64d) return launch_p64<false>(L.p64d, p, s, grid, lds, hs);
    if (L.pair) return launch_mmvq<2, true, false, false>(p, s, grid, 0, hs);
    if (L.f32) return launch_mmvq<1, true, true, false>(p, s, grid, lds, hs);
    return launch_mmvq<1, true, false, false>(p, s, grid, 0, hs);
}

// The routed FFN product after routing: the packed gate/up stage (h written
// to the caller's buffer), then the packed down stage reading h, two launches
// on the caller's stream.
int ffn_impl(const void* w_gate, const void* w_up, const void* w_down, int64_t gate_up_expert_stride_bytes,
             int64_t down_expert_stride_bytes, int64_t n_local_expert, int64_t hidden, int64_t inter,
             const void* xq, const void* grouping, int64_t ncols, int32_t topk, float* h, float* y,
             const void* s_gate, const void* s_up, int64_t s_row_stride_bytes, int64_t s_rows,
             const void* s_down, float* hs, float* ys, void* stream) {
    if (ncols < 1 || ncols > MAX_COLS || hidden <= 0 || inter <= 0) return MOEQ8_EINVAL;
    if (!w_down || !h || !y) return MOEQ8_EINVAL;
    const bool has_s = s_gate != nullptr;
    if (has_s && (!s_up || !s_down || !hs || !ys || s_rows < 1)) return MOEQ8_EINVAL;
    constexpr int64_t ROUND_BYTES = P64_SEGMENT_BYTES / 4;           // 1088
    // both stages are checked before either is launched
    GroupedLaunch G, D;
    int st = prepare_grouped(G, false, MOEQ8_GATE_UP_SWIGLU_P64, w_gate, w_up, gate_up_expert_stride_bytes,
                             (hidden / QK) * Q80_BYTES, n_local_expert, inter, hidden, xq, 0, grouping, ncols,
                             topk, h, s_gate, s_up, s_row_stride_bytes, has_s ? s_rows : 0, hidden, 0, nullptr, 0,
                             has_s ? hs : nullptr);
    if (st != MOEQ8_OK) return st;
    st = prepare_grouped(D, false, MOEQ8_DOWN_F32_ACT_P64, w_down, nullptr, down_expert_stride_bytes, ROUND_BYTES,
                         n_local_expert, hidden, inter, h, inter, grouping, ncols, topk, y, has_s ? s_down : nullptr,
                         nullptr, ROUND_BYTES, has_s ? hidden : 0, has_s ? s_rows : 0, 0, has_s ? hs : nullptr,
                         has_s ? s_rows : 0, has_s ? ys : nullptr);
    if (st != MOEQ8_OK) return st;
    const hipStream_t hs_ = (hipStream_t)stream;
    st = launch_p64<false>(false, G.p, G.s, G.grid, G.lds, hs_);
    if (st != MOEQ8_OK) return st;
    return launch_p64<false>(true, D.p, D.s, D.grid, D.lds, hs_);
}
}  // namespace
}  // namespace moeq8

extern "C" int moe_grouped_ffn_p64(const void* w_gate, const void* w_up, const void* w_down,
                                   int64_t gate_up_expert_stride_bytes, int64_t down_expert_stride_bytes,
                                   int64_t n_local_expert, int64_t hidden, int64_t inter, const void* xq,
                                   const void* grouping, int64_t ncols, int32_t topk, float* h, float* y,
                                   const void* s_gate, const void* s_up, int64_t s_row_stride_bytes,
                                   int64_t s_rows, const void* s_down, float* hs, float* ys, void* stream) {
    return ffn_impl(w_gate, w_up, w_down, gate_up_expert_stride_bytes, down_expert_stride_bytes, n_local_expert,
                    hidden, inter, xq, grouping, ncols, topk, h, y, s_gate, s_up, s_row_stride_bytes, s_rows,
                    s_down, hs, ys, stream);
}

// ---- the routed FFN product with its workspace in library-held memory ----
// h (and the shared share's hs) live in `scratch`, a device array of this
// file that every GPU the library runs on holds until the process ends.  Host
// code reaches it only through the per-device address hipGetSymbolAddress
// returns (the array's name is a host-side stand-in, not a device address).
namespace moeq8 {
namespace {
constexpr size_t FFN_SCRATCH_H_BYTES = (size_t)MAX_COLS * MOEQ8_MAX_TOPK * 1024 * 4;   // routes x inter 1024
constexpr size_t FFN_SCRATCH_HS_BYTES = (size_t)MAX_COLS * 1024 * 4;                  // columns x share rows
static_assert(FFN_SCRATCH_H_BYTES + FFN_SCRATCH_HS_BYTES == MOEQ8_FFN_SCRATCH_BYTES, "scratch size in the header");
}  // namespace
}  // namespace moeq8

static __device__ __align__(256) uint8_t scratch[MOEQ8_FFN_SCRATCH_BYTES];

namespace {
constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[SCRATCH_MAX_DEVICES] = {};

// The current device's address of `scratch`, looked up once per device with
// that device current (the caller's), or an error status.
int scratch_for_current_device(uint8_t** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return MOEQ8_EHIP;
    }
    if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return MOEQ8_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return MOEQ8_EHIP;
        }
        g_scratch_ptr[dev] = ptr;
    }
    *out = (uint8_t*)g_scratch_ptr[dev];
    return MOEQ8_OK;
}
}  // namespace

extern "C" int moe_grouped_ffn_p64_noalloc(const void* w_gate, const void* w_up, const void* w_down,
                                           int64_t gate_up_expert_stride_bytes, int64_t down_expert_stride_bytes,
                                           int64_t n_local_expert, int64_t hidden, int64_t inter, const void* xq,
                                           const void* grouping, int64_t ncols, int32_t topk, float* y,
                                           const void* s_gate, const void* s_up, int64_t s_row_stride_bytes,
                                           int64_t s_rows, const void* s_down, float* ys, void* stream) {
    // sizes beyond what the library holds are refused before anything else
    if (ncols < 1 || ncols > MAX_COLS || topk < 1 || topk > MOEQ8_MAX_TOPK || inter <= 0) return MOEQ8_EINVAL;
    if ((size_t)(ncols * topk) * (size_t)inter * 4 > FFN_SCRATCH_H_BYTES) return MOEQ8_EUNSUPPORTED;
    if (s_gate && (s_rows < 1 || (size_t)ncols * (size_t)s_rows * 4 > FFN_SCRATCH_HS_BYTES)) return MOEQ8_EUNSUPPORTED;
    uint8_t* base = nullptr;
    const int st = scratch_for_current_device(&base);
    if (st != MOEQ8_OK) return st;
    float* h = (float*)base;
    float* hs = s_gate ? (float*)(base + FFN_SCRATCH_H_BYTES) : nullptr;
    return ffn_impl(w_gate, w_up, w_down, gate_up_expert_stride_bytes, down_expert_stride_bytes, n_local_expert,
                    hidden, inter, xq, grouping, ncols, topk, h, y, s_gate, s_up, s_row_stride_bytes, s_rows,
                    s_down, hs, ys, stream);
}

extern "C" int moe_grouped_mmvq_ex(int32_t stage, const void* w_a, const void* w_b,
                                   int64_t expert_stride_bytes, int64_t w_row_stride_bytes,
                                   int64_t n_local_expert, int64_t n, int64_t k, const void* act,
                                   int64_t act_row_stride, const void* grouping, int64_t ncols,
                                   int32_t topk, float* out, const void* s_a, const void* s_b,
                                   int64_t s_row_stride_bytes, int64_t s_n, int64_t s_k,
                                   int64_t s_k_block_offset, const void* s_act,
                                   int64_t s_act_row_stride, float* s_out, void* stream) {
    return grouped_impl(false, stage, w_a, w_b, expert_stride_bytes, w_row_stride_bytes, n_local_expert, n,
                        k, act, act_row_stride, grouping, ncols, topk, out, s_a, s_b, s_row_stride_bytes,
                        s_n, s_k, s_k_block_offset, s_act, s_act_row_stride, s_out, stream);
}


extern "C" int moe_grouped_mmvq(int32_t stage, const void* w_a, const void* w_b,
                                int64_t expert_stride_bytes, int64_t w_row_stride_bytes,
                                int64_t n_local_expert, int64_t n, int64_t k, const void* act_q,
                                const void* grouping, int64_t ncols, int32_t topk, float* out,
                                void* stream) {
    if (stage != MOEQ8_GATE_UP_SWIGLU && stage != MOEQ8_DOWN) return MOEQ8_EINVAL;
    return moe_grouped_mmvq_ex(stage, w_a, w_b, expert_stride_bytes, w_row_stride_bytes,
                               n_local_expert, n, k, act_q, 0, grouping, ncols, topk, out, nullptr,
                               nullptr, 0, 0, 0, 0, nullptr, 0, nullptr, stream);
}

// ---- 4-bit weights (Q4 blocks of 18 bytes; the same kernels and reduction
// order, a 36-byte chunk per lane) ------------------------------------------

extern "C" int mmvq_q4(const void* w, int64_t w_row_stride_bytes, int64_t n, int64_t k,
                       int64_t k_block_offset, const void* xq, int64_t ncols, float* y, void* stream) {
    int st = validate_matrix(w, w_row_stride_bytes, n, k, k_block_offset, Q4_BYTES);
    if (st) return st;
    if (!xq || !y || ncols < 1 || ncols > MAX_COLS) return MOEQ8_EINVAL;
    if (((uintptr_t)xq & 3u) || ((uintptr_t)y & 3u)) return MOEQ8_EALIGN;
    if (n == 0) return MOEQ8_OK;
    return dense_call(1, w, nullptr, w_row_stride_bytes, n, k, k_block_offset, xq, ncols, y, nullptr,
                      nullptr, stream, true);
}

extern "C" int mmvq_q4_glu_pair(const void* w_gate, const void* w_up, int64_t w_row_stride_bytes,
                                int64_t n, int64_t k, int64_t k_block_offset, const void* xq,
                                int64_t ncols, float* h_out, float* g_out, float* u_out, void* stream) {
    int st = validate_matrix(w_gate, w_row_stride_bytes, n, k, k_block_offset, Q4_BYTES);
    if (st) return st;
    st = validate_matrix(w_up, w_row_stride_bytes, n, k, k_block_offset, Q4_BYTES);
    if (st) return st;
    if (!xq || !h_out || ncols < 1 || ncols > MAX_COLS) return MOEQ8_EINVAL;
    if (((uintptr_t)xq & 3u) || ((uintptr_t)h_out & 3u) || ((uintptr_t)g_out & 3u) ||
        ((uintptr_t)u_out & 3u))
        return MOEQ8_EALIGN;
    if (n == 0) return MOEQ8_OK;
    return dense_call(2, w_gate, w_up, w_row_stride_bytes, n, k, k_block_offset, xq, ncols, h_out,
                      g_out, u_out, stream, true);
}

extern "C" int moe_grouped_mmvq_q4(int32_t stage, const void* w_a, const void* w_b,
                                   int64_t expert_stride_bytes, int64_t w_row_stride_bytes,
                                   int64_t n_local_expert, int64_t n, int64_t k, const void* act,
                                   int64_t act_row_stride, const void* grouping, int64_t ncols,
                                   int32_t topk, float* out, void* stream) {
    return grouped_impl(true, stage, w_a, w_b, expert_stride_bytes, w_row_stride_bytes, n_local_expert, n,
                        k, act, act_row_stride, grouping, ncols, topk, out, nullptr, nullptr, 0, 0, 0, 0,
                        nullptr, 0, nullptr, stream);
}
