// Grouped per-expert Q8_0 x q8_1 products on the int8 matrix cores, for wide
// batches (many columns, so many routes per expert): the prefill-sized
// counterpart of the grouped MMVQ.  The pages run their large expert batches
// on a matrix-core GEMM (the WMMA routed-expert GEMM in the PR description's
// Results, and MMQ routing for wide Q4_K products in the fused-kernels commit);
// here the GEMM keeps the Q8_0 / q8_1 formats and the expert grouping of the
// decode path.
//
// Arithmetic.  One Q8_0 block is 32 values along K, exactly the K of
// v_mfma_i32_16x16x32_i8, so each block's 16x16 integer tile is scaled on its
// own: acc = fma(float(sumi), d_w * d_x, acc), blocks in ascending order from
// +0.  d_w * d_x is exact in fp32 (two fp16 values) and sumi is exact as an
// fp32 integer (|sumi| <= 32 * 127 * 127), so each block adds its exact term
// with one rounding.  This order differs from the MMVQ's 16-lane tree, so the
// two paths agree to rounding, not bit for bit.
//
// Operands: A (16 routes x 32) holds a q8_1 block of 16 routes, B (32 x 16
// weight rows) a Q8_0 block of 16 rows.  Lane (c, q) = (l % 16, l / 16)
// supplies route c (A) and weight row c (B), bytes 8q .. 8q+7 of the block,
// and receives D for weight row c and routes 4q + i, i = 0..3.
//
// Loads.  A lane fetches whole 68-byte weight pairs (two blocks of one row)
// and whole 72-byte activation pairs with 16-byte loads, four consecutive
// pairs of 16 rows per step: measured on this GPU, that pattern streams at
// 5.3 TB/s where loading each lane's 8-byte MFMA slices straight from HBM
// reached 3.9 TB/s.  Each wave then rearranges its own step into MFMA
// fragments through a private LDS area (no workgroup barrier anywhere), while
// the next step's loads are in flight.
//
// Work.  A work unit is (group, row tile, chunk of up to 16 * NT of the
// group's routes); a wave runs its chunk as NT 16-route tiles against each
// weight load (the rearranged weights stay in LDS while the tiles'
// activations pass through one LDS area of the wave in turn), so weight rows
// are read once per chunk.  The routing is very uneven at wide batches (one
// expert may get hundreds of routes), so a heavily routed expert is spread
// over several chunks instead of one unit looping over its routes.  Units are
// numbered with the chunk fastest, and unit u runs on XCD u / ceil(units / 8)
// (workgroups are dispatched to the 8 XCDs round-robin), so the chunks that
// read the same weight rows run on one XCD close together in time.
//   gate/up: a wave owns 16 rows of the gate and the same 16 rows of the up
//            matrix; both share every activation fragment; SwiGLU-DS4 epilogue.
//   down:    a wave owns 32 consecutive rows (two 16-row fragments).
#include "moeq8_device.hpp"
#include "moeq8_host.hpp"

#include <atomic>
#include <type_traits>

namespace moeq8 {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// fp16 bits h as element 0 of a 4-vector, the rest +0.
__device__ __forceinline__ f16x4 half4_lo(uint32_t h) {
    const uint64_t v = h;
    return __builtin_bit_cast(f16x4, v);
}

// The fp16 bits h of block K0 + kk's activation scale at K term (K0 + kk) % 4
// of a 4-vector, the other terms +0.
template <int K0>
__device__ __forceinline__ f16x4 dx_term(uint32_t h, int kk) {
    const int term = (K0 + kk) % 4;
    const uint32_t v = (term & 1) ? h << 16 : h;
    const uint64_t w = (term & 2) ? (uint64_t)v << 32 : (uint64_t)v;
    return __builtin_bit_cast(f16x4, w);
}


#ifndef MOEQ8_GEMM_WAVES
#define MOEQ8_GEMM_WAVES 2
#endif
constexpr int GEMM_WAVES = MOEQ8_GEMM_WAVES;
constexpr int GEMM_THREADS = 64 * GEMM_WAVES;
constexpr int TILE = 16;                 // routes per matrix-core tile = MFMA M
// Tiles per wave (each step's weights serve all of them): 4 for gate/up, 2
// for down.  Measured on 256 experts at 32..1024 columns: gate/up with 4
// tiles 6-8% faster than with 2 (two waves per SIMD instead of three, but the
// rows are read once per 64 routes instead of 32); down no faster with 4.
constexpr int nt_for(bool pair) { return pair ? 4 : 2; }
constexpr int chunk_for(bool pair) { return TILE * nt_for(pair); }   // routes per work unit
constexpr int SP = 4;                    // block pairs per step (one per lane quarter)
constexpr int SB = 2 * SP;               // blocks per step
constexpr int XCDS = 8;

// Wave-private LDS (bytes).  Fragment areas are [block k][quarter][lane row c]
// of 8 bytes, rotated by 32 bytes per block pair so that the writes of one
// instruction spread over more banks; a fragment read (fixed k) covers one
// rotated 512-byte row and is conflict-free.
constexpr int L_AQ = 0;                          // A quants, SB x 512
constexpr int L_WQ = L_AQ + SB * 512;            // W quants, 2 fragments x SB x 512
constexpr int L_DX = L_WQ + 2 * SB * 512;        // fp32 [SB][16] activation scales
constexpr int L_DW = L_DX + SB * 16 * 4;         // fp32 [2][16][SB] weight scales
constexpr int L_WAVE = L_DW + 2 * 16 * SB * 4;   // 13824

__device__ __forceinline__ int frag_off(int k, int qq, int c) {
    return k * 512 + ((qq * 128 + c * 8 + (k >> 1) * 32) & 511);
}

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
    int32_t ticket_slot;        // the staged form's work counters (below)
};

struct W68 { uint32_t v[17]; };          // one weight pair as loaded
struct A72 { uint32_t v[18]; };          // one activation pair as loaded

__device__ __forceinline__ void load68(W68& w, const uint8_t* p) {
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u32x4 t = q[i];
        w.v[4 * i] = t.x; w.v[4 * i + 1] = t.y; w.v[4 * i + 2] = t.z; w.v[4 * i + 3] = t.w;
    }
    w.v[16] = *reinterpret_cast<const uint32_t*>(p + 64);
}

__device__ __forceinline__ void load72(A72& a, const uint8_t* p) {
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u32x4 t = q[i];
        a.v[4 * i] = t.x; a.v[4 * i + 1] = t.y; a.v[4 * i + 2] = t.z; a.v[4 * i + 3] = t.w;
    }
    const u32x2 t = *reinterpret_cast<const u32x2*>(p + 64);
    a.v[16] = t.x;
    a.v[17] = t.y;
}

// inclusive prefix sum over the wave
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t t = (uint32_t)__builtin_amdgcn_ds_bpermute((lane - d) << 2, (int)v);
        if (lane >= d) v += t;
    }
    return v;
}

// Work units are (group, row tile, chunk of up to CHUNK of the group's
// routes), numbered chunk-fastest; the units are dealt to the 8 XCDs in
// contiguous ranges (workgroups are dispatched to the XCDs round-robin), so
// the chunks that read the same weight rows run on one XCD close together in
// time.  Every lane of a workgroup computes the same values (wave-uniform
// loads and scans only).

// The grouping's number of active groups and of units; false for a grouping
// that does not match the launch.
template <int CHUNK>
__device__ __forceinline__ bool grouping_units(const GemmParams& p, int l, int& n_active, uint32_t& total) {
    const int Rk = p.ncols * p.topk;
    const int4w hdr = grouping_words4(p.grouping, 0);
    if ((hdr[2] != p.ncols) | (hdr[3] != p.topk) | (hdr[0] < 0) | (hdr[0] > Rk) | (hdr[1] < 0) |
        (hdr[1] > Rk))
        return false;
    n_active = hdr[0];
    const uint32_t tiles = (uint32_t)p.tiles;
    const int4* table = reinterpret_cast<const int4*>(p.grouping + grouping_table_word(Rk));
    total = 0;
    for (int b0 = 0; b0 < n_active; b0 += 64) {
        uint32_t un = 0;
        const int a = b0 + l;
        if (a < n_active) {
            const int4 g = table[a];
            const bool ok = (g.x >= 0) & (g.x < p.n_local) & (g.y >= 0) & (g.z >= g.y) & (g.z <= Rk);
            un = ok ? (uint32_t)((g.z - g.y + CHUNK - 1) / CHUNK) * tiles : 0u;
        }
        const uint32_t s = wave_incl_scan(un, l);
        total += (uint32_t)__builtin_amdgcn_readlane((int)s, 63);
    }
    return true;
}

// Unit u (< the total): its local expert e, first route entry rbegin, route
// count nr (1..CHUNK) and row tile t; false if its group is empty.
template <int CHUNK>
__device__ __forceinline__ bool unit_at(const GemmParams& p, int l, int n_active, uint32_t u, int& e, int& rbegin,
                                        int& nr, uint32_t& t) {
    const int Rk = p.ncols * p.topk;
    const uint32_t tiles = (uint32_t)p.tiles;
    const int4* table = reinterpret_cast<const int4*>(p.grouping + grouping_table_word(Rk));
    int gbegin = 0, gend = 0;
    uint32_t ubase = 0;
    e = 0;
    uint32_t carry = 0;
    bool found = false;
    // 256 groups at a time: their records are read before any is scanned
    for (int b0 = 0; b0 < n_active && !found; b0 += 256) {
        int4 gq[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int a = b0 + 64 * k + l;
            gq[k] = a < n_active ? table[a] : make_int4(0, 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (found || b0 + 64 * k >= n_active) break;
            const int4 g = gq[k];
            const bool ok = (b0 + 64 * k + l < n_active) & (g.x >= 0) & (g.x < p.n_local) & (g.y >= 0) &
                            (g.z >= g.y) & (g.z <= Rk);
            const uint32_t un = ok ? (uint32_t)((g.z - g.y + CHUNK - 1) / CHUNK) * tiles : 0u;
            const uint32_t incl = wave_incl_scan(un, l) + carry;
            const bool hit = (un > 0) & (incl - un <= u) & (u < incl);
            const uint64_t m = __ballot(hit);
            if (m) {
                const int src = __builtin_ctzll(m);
                e = __builtin_amdgcn_readlane(g.x, src);
                gbegin = __builtin_amdgcn_readlane(g.y, src);
                gend = __builtin_amdgcn_readlane(g.z, src);
                ubase = (uint32_t)__builtin_amdgcn_readlane((int)(incl - un), src);
                found = true;
            } else {
                carry = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
            }
        }
    }
    if (gend <= gbegin) return false;
    const uint32_t nchunk = (uint32_t)(gend - gbegin + CHUNK - 1) / CHUNK;
    const uint32_t rem = u - ubase;
    t = rem / nchunk;                                  // row tile
    rbegin = gbegin + (int)(rem - t * nchunk) * CHUNK;
    nr = min(gend - rbegin, CHUNK);                    // routes of this unit, 1..CHUNK
    return true;
}

// The units of XCD x: [first, end) of the total, contiguous.
__device__ __forceinline__ void xcd_range(uint32_t total, uint32_t x, uint32_t& first, uint32_t& end) {
    const uint32_t per = total / XCDS, extra = total % XCDS;
    first = x * per + min(x, extra);
    end = first + per + (x < extra ? 1u : 0u);
}

// The one unit of this workgroup in a grid of one workgroup per unit (the
// grid covers an upper bound of the units; the excess returns false).
template <int CHUNK>
__device__ __forceinline__ bool find_unit(const GemmParams& p, int l, int& e, int& rbegin, int& nr, uint32_t& t) {
    {
        // units <= (active groups + valid routes / CHUNK) * tiles: slots past
        // that bound leave before the scan
        const int4w hdr = grouping_words4(p.grouping, 0);
        const uint32_t bound = ((uint32_t)max(hdr[0], 0) + (uint32_t)max(hdr[1], 0) / CHUNK) * (uint32_t)p.tiles;
        if (blockIdx.x / XCDS >= (bound + XCDS - 1) / XCDS) return false;
    }
    int n_active;
    uint32_t total;
    if (!grouping_units<CHUNK>(p, l, n_active, total)) return false;
    uint32_t first, end;
    xcd_range(total, blockIdx.x % XCDS, first, end);
    const uint32_t u = first + blockIdx.x / XCDS;
    if (u >= end) return false;
    return unit_at<CHUNK>(p, l, n_active, u, e, rbegin, nr, t);
}

template <bool PAIR>
__global__ __launch_bounds__(GEMM_THREADS) __attribute__((amdgpu_waves_per_eu(nt_for(PAIR) <= 2 ? 3 : 2))) void k_grouped_gemm(
    const GemmParams p) {
    constexpr int NT = nt_for(PAIR);
    constexpr int CHUNK = chunk_for(PAIR);
    constexpr int WAVE_ROWS = PAIR ? 16 : 32;
    constexpr int WG_ROWS = WAVE_ROWS * GEMM_WAVES;
    __shared__ __align__(16) uint8_t lds_all[GEMM_WAVES * L_WAVE];

    const int wave = threadIdx.x >> 6;
    const int l = threadIdx.x & 63;
    const int c = l & 15;
    const int q = l >> 4;
    uint8_t* lds = lds_all + wave * L_WAVE;

    // ---- work unit of this workgroup ------------------------------------
    const int Rk = p.ncols * p.topk;
    int e, rbegin, nr;
    uint32_t t;
    if (!find_unit<CHUNK>(p, l, e, rbegin, nr, t)) return;

    const int64_t r0 = (int64_t)t * WG_ROWS + (int64_t)wave * WAVE_ROWS;
    if (r0 >= p.n) return;                             // n % 32 == 0: whole waves in or out

    // ---- operands ---------------------------------------------------------
    const int32_t* route = p.grouping + 4 + 2 * (int64_t)Rk + 1;
    // lane (c, q) loads route slot 16t + c of each tile t (clamped to the
    // unit's last route: its results are computed but not stored) and weight
    // row c of each fragment
    const uint8_t* abase[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
        const int myroute = route[rbegin + min(TILE * tt + c, nr - 1)];
        const int rr = (myroute >= 0 && myroute < Rk) ? myroute : 0;
        const int64_t arow = (int64_t)(((uint64_t)(uint32_t)rr * p.act_route_mul) >> 32);
        abase[tt] = p.act + arow * p.act_row_bytes + (int64_t)q * (2 * Q81_BYTES);
    }
    const int ntiles = (nr + TILE - 1) / TILE;         // tiles holding routes, 1..NT
    const int64_t ew = (int64_t)e * p.expert_stride + (r0 + c) * p.row_stride + (int64_t)q * (2 * Q80_BYTES);
    const uint8_t* wbase0 = p.w0 + ew;
    const uint8_t* wbase1 = PAIR ? p.w1 + ew : wbase0 + 16 * p.row_stride;
    const int npairs = p.nb >> 1;
    const int nsteps = (npairs + SP - 1) / SP;

    // Weights of a step are double-buffered; the activations of each tile
    // are single-buffered: tile t's loads for step s + 1 go out as soon as its
    // step-s values are in LDS, which is after step s + 1's weight loads and
    // before step s + 2's, so every wait is for the oldest loads in flight.
    auto pair_of = [&](int s) {
        // pair SP*s + q of each row (clamped to the last pair: re-read, unused),
        // as an offset from the lane's own pair q
        return min(SP * min(s, nsteps - 1) + q, npairs - 1) - q;
    };
    auto load_w = [&](W68 (&w)[2], int s) {
        const int64_t wo = (int64_t)pair_of(s) * (2 * Q80_BYTES);
        load68(w[0], wbase0 + wo);
        load68(w[1], wbase1 + wo);
    };
    A72 areg[NT];
    auto load_a = [&](int tt, int s) {
        load72(areg[tt], abase[tt] + (int64_t)pair_of(s) * (2 * Q81_BYTES));
    };

    float acc[NT][2][4];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[tt][f][i] = 0.0f;

    // Rearrange a step into fragment order in LDS, then run its blocks.
    auto run_step = [&](const W68 (&wst)[2], int s) {
        // this lane's two blocks are k = 2q and 2q + 1 of the step
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            const W68& w = wst[f];
            uint32_t q0[8];                                // block 2q's quants, dword aligned
#pragma unroll
            for (int i = 0; i < 8; ++i) q0[i] = __builtin_amdgcn_alignbit(w.v[i + 1], w.v[i], 16);
            uint8_t* wq = lds + L_WQ + f * (SB * 512);
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                *reinterpret_cast<uint2*>(wq + frag_off(2 * q, qq, c)) = make_uint2(q0[2 * qq], q0[2 * qq + 1]);
                *reinterpret_cast<uint2*>(wq + frag_off(2 * q + 1, qq, c)) =
                    make_uint2(w.v[9 + 2 * qq], w.v[10 + 2 * qq]);
            }
            *reinterpret_cast<float2*>(lds + L_DW + ((f * 16 + c) * SB + 2 * q) * 4) =
                make_float2(half_bits_to_float(w.v[0]), half_bits_to_float(w.v[8] >> 16));
        }
        // the row scales of this lane's weight row for all blocks of the step
        float dw[2][SB];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            const float4 lo = *reinterpret_cast<const float4*>(lds + L_DW + ((f * 16 + c) * SB) * 4);
            const float4 hi = *reinterpret_cast<const float4*>(lds + L_DW + ((f * 16 + c) * SB + 4) * 4);
            dw[f][0] = lo.x; dw[f][1] = lo.y; dw[f][2] = lo.z; dw[f][3] = lo.w;
            dw[f][4] = hi.x; dw[f][5] = hi.y; dw[f][6] = hi.z; dw[f][7] = hi.w;
        }
        const int kvalid = min(SB, p.nb - SB * s);         // blocks of this step inside the row
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            if (tt >= ntiles) break;
            {
                const A72& a = areg[tt];
                uint8_t* aq = lds + L_AQ;
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                    *reinterpret_cast<uint2*>(aq + frag_off(2 * q, qq, c)) = make_uint2(a.v[1 + 2 * qq], a.v[2 + 2 * qq]);
                    *reinterpret_cast<uint2*>(aq + frag_off(2 * q + 1, qq, c)) =
                        make_uint2(a.v[10 + 2 * qq], a.v[11 + 2 * qq]);
                }
                float* dx = reinterpret_cast<float*>(lds + L_DX);
                dx[(2 * q) * 16 + c] = half_bits_to_float(a.v[0]);
                dx[(2 * q + 1) * 16 + c] = half_bits_to_float(a.v[9]);
            }
            load_a(tt, s + 1);
#pragma unroll
            for (int k = 0; k < SB; ++k) {
                if (k >= kvalid) break;
                const long xa = *reinterpret_cast<const long*>(lds + L_AQ + frag_off(k, q, c));
                const float4 dx4 = *reinterpret_cast<const float4*>(lds + L_DX + (k * 16 + 4 * q) * 4);
                const float dxv[4] = {dx4.x, dx4.y, dx4.z, dx4.w};
#pragma unroll
                for (int f = 0; f < 2; ++f) {
                    const long wb = *reinterpret_cast<const long*>(lds + L_WQ + f * (SB * 512) + frag_off(k, q, c));
                    const i32x4 z = {0, 0, 0, 0};
                    const i32x4 d = __builtin_amdgcn_mfma_i32_16x16x32_i8(xa, wb, z, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[tt][f][i] = fmaf((float)d[i], dw[f][k] * dxv[i], acc[tt][f][i]);
                }
            }
        }
    };

    W68 wa[2], wb[2];
    load_w(wa, 0);
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
        if (tt < ntiles) load_a(tt, 0);
    for (int s = 0; s < nsteps; s += 2) {
        load_w(wb, s + 1);
        run_step(wa, s);
        if (s + 1 >= nsteps) break;
        load_w(wa, s + 2);
        run_step(wb, s + 1);
    }

    // ---- epilogue: lane (c, q) holds row r0 + c (+16 for the second down
    // fragment) of route slots 16t + 4q + i ---------------------------------
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int slotr = TILE * tt + 4 * q + i;
            if (slotr >= nr) continue;
            const int r = route[rbegin + slotr];
            if (r < 0 || r >= Rk) continue;
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

// Staged form (k % 256 == 0, whole row tiles, 16-byte aligned operands): a
// workgroup of eight waves stages each K step of 8 blocks (256 values) of its
// unit's 64 weight rows (gate/up: 32 rows of each matrix) and of up to 64
// routes' activations in LDS with direct 16-byte global-to-LDS loads (no
// registers on the way), and every wave reads its matrix-core fragments from
// there: a staged weight row serves every route tile and a staged activation
// row every row group, so each byte is fetched once per workgroup (the
// register-fed form above fetches each activation once per wave).  Only whole
// 16-route tiles that hold routes are staged and run.
//   gate/up: wave w runs rows 16 (w & 1) + [0, 16) of both matrices against
//            route tile w >> 1;  down: rows 16 (w & 3) + [0, 16) against route
//            tiles 2 (w >> 2) and 2 (w >> 2) + 1.
// The grid is two workgroups a CU; the workgroups of an XCD take that XCD's
// units from a work counter in the order they ask (below), and the steps of a
// workgroup's units form one pipeline: the next step's loads, the next unit's
// first step included, are in flight while a step is computed, and the next
// unit's lookup and route entries are read while the last step's data
// arrives, so a unit costs its steps and not a fresh fill.  Units of at most
// four steps a row tile (the down at k = 1024) take two row tiles of their
// routes (TPU = 2): the second follows with no lookup.  On the GEMM layout
// the lookup reads an LDS copy of the group table (below).
//   LDS per step: weights 64 rows x 272 bytes (a row's 8 blocks, as stored),
//   activations 64 routes x 288 bytes; per wave, fp32 activation scales of
//   its route slots.  A wave issues up to six loads a step (the stage's 17
//   weight and 18 activation wave-loads over the eight waves; the step's
//   wait covers all of them).  A weight row's quants sit 2
//   bytes into each 34-byte block, so a fragment of an even block is cut from
//   three aligned dwords.
// Arithmetic and order are those of the form above: acc = fma(float(sumi),
// d_w * d_x, acc), blocks ascending from +0, so both forms give the same bits.
// Timing copies put the form's time in its loads and its instruction issue
// together (on the GEMM layout at 1024 columns: loads alone about 85% of the
// whole, the arithmetic alone about 25%, the per-block scaling two or three
// VALU operations for every output, row and block).
constexpr int S_THREADS = 512;
constexpr int S_WG_PER_CU = 2;                   // the LDS below holds two
constexpr int S_CHUNK = 64;                      // routes per unit
constexpr int S_STEP_BLOCKS = 8;                 // blocks per K step
constexpr int S_WROW = S_STEP_BLOCKS * Q80_BYTES;   // 272
constexpr int S_AROW = S_STEP_BLOCKS * Q81_BYTES;   // 288
constexpr int S_W = 64 * S_WROW;                 // 17408: 64 weight rows
constexpr int S_A = S_CHUNK * S_AROW;            // 18432: 64 routes
constexpr int S_STAGE = S_W + S_A;               // 35840
constexpr int S_DX = 2 * S_STAGE;                // per wave: fp32 [8 blocks][32 slots]
constexpr int S_DX_WAVE = S_STEP_BLOCKS * 32 * 4;    // 1024
constexpr int S_ZERO = S_DX + 8 * S_DX_WAVE;     // 256 zero bytes (the GEMM layout's scale operands)
constexpr int S_ROUTES = S_ZERO + 256;           // the next unit's 64 route entries (the GEMM layout's gate/up)
constexpr int S_LDS = S_ROUTES + 256;            // 80384
constexpr int S_W_LOADS = S_W / 1024;            // 17 wave-loads of 1 KB
constexpr int S_A_LOADS = S_A / 1024;            // 18
constexpr int S_SLOTS = (S_A_LOADS + 7) / 8;     // 3 wave-loads of each kind per wave
static_assert(S_WG_PER_CU * S_LDS <= 160 * 1024, "LDS of a CU");

// Work counters of the staged form: the workgroups of one XCD take that XCD's
// units in the order they ask for them (one counter a call slot and XCD, 128
// bytes apart), so the chunks of one row tile, consecutive units, start
// together and the later ones find the rows in L2 whatever each unit's
// length.  The draw that takes a counter's last value (units + workgroups -
// 1: every workgroup ends with one draw past the units) sets it back to zero,
// so a slot is zero between calls.  The host hands the slots out in turn: up
// to S_TICKET_SLOTS calls may be in flight on one device at once.
constexpr int S_TICKET_SLOTS = 256;
__device__ uint32_t g_tickets[S_TICKET_SLOTS * XCDS * 32];

// Workgroup barrier over LDS only: waits for this wave's LDS operations, not
// for its global loads, so a step's loads stay in flight across it (the
// barrier of __syncthreads also waits for every outstanding global load).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One wave-wide direct load of 16 bytes a lane from global memory into LDS:
// lane i writes LDS bytes [lds + 16 i, lds + 16 i + 16).  `lds` is the
// wave-uniform LDS byte address (the low 32 bits of a shared pointer).  The
// load has no register results; its completion is tracked by vmcnt alone,
// which the caller waits for before any wave reads the bytes (issued this
// way the compiler adds no wait of its own before unrelated LDS reads).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // m0 is set here and used by nothing else
__device__ __forceinline__ void load_lds16(const void* src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0) alone

// One wave-wide direct load of 4 bytes a lane into LDS (lane i writes bytes
// [lds + 4 i, lds + 4 i + 4)); as load_lds16.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_lds4(const void* src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :: "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t lds_u32(const uint8_t* b, int off) {
    return *reinterpret_cast<const uint32_t*>(b + off);
}

// Eight quant bytes of block k of a staged weight row (row base `wr`, byte q8
// = 8q of the block): 2-byte aligned for even k, 4-byte aligned for odd k.
template <int K>
__device__ __forceinline__ long w_frag(const uint8_t* wr, int q8) {
    constexpr int off = K * Q80_BYTES + 2;
    if constexpr (off % 4 == 0) {
        const uint32_t lo = lds_u32(wr, off + q8), hi = lds_u32(wr, off + q8 + 4);
        return (long)(((uint64_t)hi << 32) | lo);
    } else {
        const uint32_t d0 = lds_u32(wr, off - 2 + q8), d1 = lds_u32(wr, off + 2 + q8), d2 = lds_u32(wr, off + 6 + q8);
        const uint32_t lo = __builtin_amdgcn_alignbit(d1, d0, 16), hi = __builtin_amdgcn_alignbit(d2, d1, 16);
        return (long)(((uint64_t)hi << 32) | lo);
    }
}

template <int K>
__device__ __forceinline__ long a_frag(const uint8_t* ar, int q8) {
    constexpr int off = K * Q81_BYTES + 4;             // always 4-byte aligned
    const uint32_t lo = lds_u32(ar, off + q8), hi = lds_u32(ar, off + q8 + 4);
    return (long)(((uint64_t)hi << 32) | lo);
}

// The activation rows of a stage (288 bytes, 72 dwords apart) put slots c,
// c + 4, c + 8, c + 12 of a 16-route tile on the same LDS banks.  On the
// GEMM's weight layout, and in the down (two route tiles a wave) on either,
// the pieces of slots with bit 2 set are stored rotated by one 16-byte place,
// so a tile's fragment reads meet two rows a bank group instead of four
// (measured at 512 / 1024 columns: gate/up on the layout 458 -> 450 and
// 602 -> 586 us, its down 317 -> 286 and 460 -> 391; the plain rows' down at
// k = 1024 staged 294 / 407 us against 336 / 497 register-fed; the plain
// rows' gate/up, whose weight reads are split and conflict on their own,
// measured slower with it: 196 -> 219 us at 32 columns).  Byte o of slot s's
// row sits at o + 16 a_rot(s), except in the row's last piece (o >= 272),
// which wraps to the row's start.
template <bool ROT>
__device__ __forceinline__ int a_rot(int slot) { return ROT ? (slot >> 2) & 1 : 0; }

// Where this lane's pieces of a step come from and go to, the same for every
// unit and step: weight piece j of the wave is row wrow, 16-byte part wpart
// of the stage's weight rows (gate/up: rows 0..31 gate, 32..63 up);
// activation piece j is route slot aslot (-1: past the stage), part apart.
struct StageGeometry {
    int w_off[S_SLOTS];                                // wrow' * row_stride + 16 wpart (wrow' = row in its matrix)
    uint32_t w_up;                                     // bit j: piece j is of the second matrix
    int a_slot[S_SLOTS];
    int a_part[S_SLOTS];                               // 16 apart
};

template <bool PAIR, bool ROT>
__device__ __forceinline__ void stage_geometry(const GemmParams& p, int wave, int l, StageGeometry& G) {
    G.w_up = 0;
#pragma unroll
    for (int j = 0; j < S_SLOTS; ++j) {
        const int i = 8 * j + wave;                    // wave-load index
        const int piece = min(i, S_W_LOADS - 1) * 64 + l;
        const int wrow = piece / 17, part = piece - wrow * 17;
        const int m = PAIR ? wrow / 32 : 0;
        const int r = PAIR ? wrow % 32 : wrow;
        G.w_off[j] = r * (int)p.row_stride + part * 16;
        G.w_up |= (uint32_t)m << j;
        const int apiece = min(i, S_A_LOADS - 1) * 64 + l;
        const int slot = apiece / 18;
        G.a_slot[j] = i < S_A_LOADS ? slot : -1;
        // LDS position pp of the slot's row holds piece pp - a_rot(slot) (mod 18)
        G.a_part[j] = (apiece - slot * 18 + 18 - a_rot<ROT>(slot)) % 18 * 16;
    }
}

// The activation sources of a unit: byte offsets into the activations of
// this lane's pieces (a piece past the unit's staged route slots reads the
// unit's first activation piece, one cached line for all such lanes).
// (in two parts: the route entries, read at indices inside the unit; the
// offsets from them)
__device__ __forceinline__ void stage_routes(const GemmParams& p, const StageGeometry& G, int rbegin, int nr,
                                             int& r_first, int (&rts)[S_SLOTS]) {
    const int Rk = p.ncols * p.topk;
    const int32_t* route = p.grouping + 4 + 2 * (int64_t)Rk + 1;
    r_first = route[rbegin];
#pragma unroll
    for (int j = 0; j < S_SLOTS; ++j) rts[j] = route[rbegin + min(max(G.a_slot[j], 0), nr - 1)];
}

__device__ __forceinline__ void stage_offsets(const GemmParams& p, const StageGeometry& G, int nr, int r_first,
                                              const int (&rts)[S_SLOTS], int (&a_off)[S_SLOTS]) {
    const int Rk = p.ncols * p.topk;
    const int nslot = (nr + 15) & ~15;                 // staged route slots: whole tiles
    auto row_off = [&](int rt) {
        const int rr = (rt >= 0 && rt < Rk) ? rt : 0;
        return (int)(((uint64_t)(uint32_t)rr * p.act_route_mul) >> 32) * (int)p.act_row_bytes;
    };
    const int first = row_off(r_first);
#pragma unroll
    for (int j = 0; j < S_SLOTS; ++j) {
        const int slot = G.a_slot[j];
        a_off[j] = (slot >= 0 && slot < nslot) ? row_off(rts[j]) + G.a_part[j] : first;
    }
}

__device__ __forceinline__ void stage_act(const GemmParams& p, const StageGeometry& G, int rbegin, int nr,
                                          int (&a_off)[S_SLOTS]) {
    int r_first, rts[S_SLOTS];
    stage_routes(p, G, rbegin, nr, r_first, rts);
    stage_offsets(p, G, nr, r_first, rts, a_off);
}

// The GEMM layout's kernels keep a copy of the grouping's group table in the
// LDS the plain layout uses for its fp32 activation scales: entry a is
// {expert, or -1 for an invalid entry; first route; end; units of groups
// 0..a}, so a unit is looked up in LDS instead of by a scan over the table
// in memory (a round trip a unit change).
constexpr int S_TABLE_GROUPS = 8 * S_DX_WAVE / 16;   // 512

// Wave-wide: the table of the n_active <= S_TABLE_GROUPS groups.
__device__ void build_unit_table(const GemmParams& p, int l, int n_active, int4* tab) {
    const int Rk = p.ncols * p.topk;
    const int4* gt = reinterpret_cast<const int4*>(p.grouping + grouping_table_word(Rk));
    const uint32_t tiles = (uint32_t)p.tiles;
    uint32_t carry = 0;
    for (int b0 = 0; b0 < n_active; b0 += 64) {
        const int a = b0 + l;
        const int4 g = a < n_active ? gt[a] : make_int4(-1, 0, 0, 0);
        const bool ok = (a < n_active) & (g.x >= 0) & (g.x < p.n_local) & (g.y >= 0) & (g.z >= g.y) & (g.z <= Rk);
        const uint32_t un = ok ? (uint32_t)((g.z - g.y + S_CHUNK - 1) / S_CHUNK) * tiles : 0u;
        const uint32_t incl = wave_incl_scan(un, l) + carry;
        if (a < n_active) tab[a] = make_int4(ok ? g.x : -1, g.y, g.z, (int)incl);
        carry = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    }
}

// Unit u (below the total) from the LDS table, as unit_at.
__device__ __forceinline__ bool unit_at_lds(const int4* tab, uint32_t tiles, int n_active, int l, uint32_t u,
                                            int& e, int& rbegin, int& nr, uint32_t& t) {
    int gbegin = 0, gend = 0;
    uint32_t ubase = 0;
    bool found = false;
    for (int b0 = 0; b0 < n_active && !found; b0 += 64) {
        const int a = b0 + l;
        const int4 g = a < n_active ? tab[a] : make_int4(-1, 0, 0, 0);
        const uint32_t un = g.x >= 0 ? (uint32_t)((g.z - g.y + S_CHUNK - 1) / S_CHUNK) * tiles : 0u;
        const uint32_t incl = (uint32_t)g.w;
        const uint64_t m = __ballot((un > 0) & (incl - un <= u) & (u < incl));
        if (m) {
            const int src = __builtin_ctzll(m);
            e = __builtin_amdgcn_readlane(g.x, src);
            gbegin = __builtin_amdgcn_readlane(g.y, src);
            gend = __builtin_amdgcn_readlane(g.z, src);
            ubase = (uint32_t)__builtin_amdgcn_readlane((int)(incl - un), src);
            found = true;
        }
    }
    if (!found || gend <= gbegin) return false;
    const uint32_t nchunk = (uint32_t)(gend - gbegin + S_CHUNK - 1) / S_CHUNK;
    const uint32_t rem = u - ubase;
    t = rem / nchunk;
    rbegin = gbegin + (int)(rem - t * nchunk) * S_CHUNK;
    nr = min(gend - rbegin, S_CHUNK);
    return true;
}

// G8: the weights (gate/up, or down) are in the layout of q8_0_pack_gemm_rows (per 8-block
// group, 16 bytes of scales, then 8-byte aligned quants with the 8-byte halves
// of each 16-byte piece swapped in rows 8-15 of every 16): a lane's operand
// piece is one aligned 8-byte read, and the 16 rows of a wave's read fall
// into different LDS banks.  The same bytes reach the same lanes, so the
// results are those of the plain layout.
// TPU: row tiles a unit (p.tiles counts units of TPU tiles).
template <bool PAIR, bool G8 = false, int TPU = 1>
__global__ __launch_bounds__(S_THREADS) __attribute__((amdgpu_waves_per_eu(4, 4))) void k_grouped_gemm_staged(
    const GemmParams p) {
    __shared__ __align__(16) uint8_t lds[S_LDS];
    constexpr int NM = PAIR ? 2 : 1;                   // weight fragments a wave reads a block
    constexpr int NR = PAIR ? 1 : 2;                   // route tiles a wave runs
    constexpr int TILE_ROWS = PAIR ? 32 : 64;
    const int wave = threadIdx.x >> 6;
    const int l = threadIdx.x & 63;
    const int c = l & 15;
    const int q8 = (l >> 4) * 8;
    const int rh = PAIR ? (wave & 1) * 16 : (wave & 3) * 16;   // this wave's rows (of each matrix)
    const int tile0 = PAIR ? (wave >> 1) : (wave >> 2) * 2;    // and first route tile
    const int Rk = p.ncols * p.topk;
    const int32_t* route = p.grouping + 4 + 2 * (int64_t)Rk + 1;

    int n_active;
    uint32_t total;
    if (!grouping_units<S_CHUNK>(p, l, n_active, total)) return;   // every workgroup alike: no draw
    if (G8 && PAIR && threadIdx.x < 64) reinterpret_cast<uint32_t*>(lds + S_ZERO)[threadIdx.x] = 0u;
    const uint32_t x = blockIdx.x % XCDS;
    uint32_t first, end;
    xcd_range(total, x, first, end);
    const uint32_t cnt = end - first;                  // units of this XCD
    const uint32_t nwg = gridDim.x / XCDS;             // its workgroups (the grid is a multiple of 8)
    uint32_t* const ctr = g_tickets + ((uint32_t)p.ticket_slot * XCDS + x) * 32;
    __shared__ uint32_t s_tick;                        // thread 0's last draw, for every wave
    auto draw = [&]() -> uint32_t {
        const uint32_t v = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (v == cnt + nwg - 1) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return v;
    };
    // a unit that cannot be looked up (a grouping changed under the call) is
    // skipped with the rest of the workgroup's draws, so the counter still
    // returns to zero
    auto drain = [&]() {
        if (threadIdx.x == 0)
            while (draw() < cnt) {
            }
    };
    // the GEMM layout's units are looked up in an LDS copy of the group table
    int4* const tab = reinterpret_cast<int4*>(lds + S_DX);
    const bool use_tab = G8 && n_active <= S_TABLE_GROUPS;
    if (use_tab && wave == 0) build_unit_table(p, l, n_active, tab);
    auto lookup = [&](uint32_t uu, int& ee, int& rb, int& rn, uint32_t& tt) -> bool {
        return use_tab ? unit_at_lds(tab, (uint32_t)p.tiles, n_active, l, uu, ee, rb, rn, tt)
                       : unit_at<S_CHUNK>(p, l, n_active, uu, ee, rb, rn, tt);
    };
    if (threadIdx.x == 0) s_tick = draw();
    __syncthreads();
    uint32_t u = first + s_tick;
    if (u >= end) return;
    // the current unit: expert, route entries, row tile (wave-uniform)
    int e, rbegin, nr;
    uint32_t t;
    if (!lookup(u, e, rbegin, nr, t)) {                // before any load
        drain();
        return;
    }
    t *= (uint32_t)TPU;                                // the unit's first row tile
    int ti = 0;                                        // row tile of the unit

    StageGeometry G;
    constexpr bool ROT = G8 || !PAIR;
    stage_geometry<PAIR, ROT>(p, wave, l, G);
    int a_off[S_SLOTS];
    stage_act(p, G, rbegin, nr, a_off);

    const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
    // step s of the unit of expert ee, row tile tt, activation offsets ao, into buffer b
    auto load_step = [&](int ee, uint32_t tt, const int (&ao)[S_SLOTS], int s, int b) {
        const int64_t wb = (int64_t)ee * p.expert_stride + (int64_t)tt * TILE_ROWS * p.row_stride + (int64_t)s * S_WROW;
        const uint8_t* w0 = p.w0 + wb;
        const uint8_t* w1 = PAIR ? p.w1 + wb : w0;
        const uint8_t* act = p.act + (int64_t)s * S_AROW;
        const uint32_t base = lds0 + b * S_STAGE;
#pragma unroll
        for (int j = 0; j < S_SLOTS; ++j) {
            const int i = 8 * j + wave;                // wave-uniform: a wave skips the pieces past the stage
            if (i < S_W_LOADS) load_lds16(((G.w_up >> j) & 1u ? w1 : w0) + G.w_off[j], base + i * 1024);
            if (i < S_A_LOADS) load_lds16(act + ao[j], base + S_W + i * 1024);
        }
    };
    float* dxt = reinterpret_cast<float*>(lds + S_DX + wave * S_DX_WAVE);   // [8 blocks][32 slots]
    const int nsteps = p.nb / S_STEP_BLOCKS;

    load_step(e, t, a_off, 0, 0);
    int g = 0;                                         // steps of this workgroup so far
    for (;;) {
        // this lane's output rows (route slots 16 tile + 4q + i), read while
        // the unit's first step loads
        int out_route[NR][4];
#pragma unroll
        for (int rt = 0; rt < NR; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int slotr = (tile0 + rt) * 16 + q8 / 2 + i;
                const int r = route[rbegin + min(slotr, nr - 1)];   // an entry of the unit either way
                out_route[rt][i] = (slotr < nr && r >= 0 && r < Rk) ? r : -1;
            }
        const int nslot = (nr + 15) & ~15;
        bool live[NR];
#pragma unroll
        for (int rt = 0; rt < NR; ++rt) live[rt] = (tile0 + rt) * 16 < nslot;
        float acc[NR][NM][4];
#pragma unroll
        for (int rt = 0; rt < NR; ++rt)
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[rt][m][i] = 0.0f;

        // one step from LDS buffer b
        auto compute = [&](int b) {
            const uint8_t* W = lds + b * S_STAGE;
            const uint8_t* A = W + S_W;
            // this wave's activation scales, fp32 (read back by this wave only;
            // the plain layout's forms)
#pragma unroll
            for (int h = 0; h < (G8 ? 0 : 2 * NR); ++h) {
                const int ent = h * 64 + l;
                const int k = ent / (16 * NR), sl = ent % (16 * NR);
                dxt[k * 32 + sl] = half_bits_to_float(*reinterpret_cast<const uint16_t*>(
                    A + (tile0 * 16 + sl) * S_AROW + 16 * a_rot<ROT>(sl) + k * Q81_BYTES));
            }
            // two blocks at a time: fragments of both, then the matrix-core
            // products of both, then the scaled sums in block order (block K
            // enters every accumulator before block K + 1)
            auto run_step = [&](auto nlive) {
                constexpr int NL = decltype(nlive)::value;   // live route tiles of this wave
                auto two_blocks = [&](auto kc) {
                    constexpr int K0 = 2 * decltype(kc)::value;
                    long wb[2][NM], xa[2][NL];
                    float dwv[2][NM];
                    float4 dx4[2][NL];
                    i32x4 d[2][NL][NM];
                    // G8: the scale products d_x * d_w of each block's 16 x 16 tile
                    // come from the matrix cores, an fp16 product with one
                    // nonzero K term (exact in fp32: the same values as the fp32
                    // multiply).  Gate/up: the weight operand is four of the
                    // row's scales as stored (blocks 4 (K / 4) .. + 3 at K terms
                    // 0..3) and the activation operand holds block K's d_x at
                    // term K % 4, zeros elsewhere, lane groups 1..3 reading it
                    // from a zero area, so neither needs masking.  The down (two
                    // route tiles a wave, no registers to spare) masks both
                    // operands to lane group 0's first term.
                    f16x4 dws[NM];
                    uint32_t dxh[2][NL], dwh[2][NM];
                    const uint32_t kmask = (l >> 4) == 0 ? 0xFFFFu : 0u;
                    f32x4 sc[2][NL][NM];
#pragma unroll
                    for (int m = 0; m < NM; ++m) {
                        const uint8_t* wr = W + (m * 32 + rh + c) * S_WROW;
                        if constexpr (G8) {
                            // operand piece q of block K at 16 + 32K + 8 (q ^ (row / 8 % 2));
                            // the scales of blocks K0, K0 + 1 in one dword
                            const int qx = q8 ^ (c & 8);
                            wb[0][m] = *reinterpret_cast<const long*>(wr + 16 + 32 * K0 + qx);
                            wb[1][m] = *reinterpret_cast<const long*>(wr + 16 + 32 * (K0 + 1) + qx);
                            if constexpr (PAIR) {
                                dws[m] = *reinterpret_cast<const f16x4*>(wr + 8 * (K0 / 4));
                            } else {
                                const uint32_t sw = *reinterpret_cast<const uint32_t*>(wr + 2 * K0);
                                dwh[0][m] = sw & kmask;
                                dwh[1][m] = (sw >> 16) & kmask;
                            }
                        } else {
                            wb[0][m] = w_frag<K0>(wr, q8);
                            wb[1][m] = w_frag<K0 + 1>(wr, q8);
                            dwv[0][m] = half_bits_to_float(*reinterpret_cast<const uint16_t*>(wr + K0 * Q80_BYTES));
                            dwv[1][m] = half_bits_to_float(*reinterpret_cast<const uint16_t*>(wr + (K0 + 1) * Q80_BYTES));
                        }
                    }
#pragma unroll
                    for (int rt = 0; rt < NL; ++rt) {
                        // the fragment of block 7 at q8 >= 16 lies in the row's
                        // last piece (rotated to the row's start when a_rot)
                        const uint8_t* ar = A + ((tile0 + rt) * 16 + c) * S_AROW;
                        const uint8_t* ar0 = ar + 16 * a_rot<ROT>(c);
                        const uint8_t* ar7 = q8 < 16 ? ar0 : a_rot<ROT>(c) ? ar - 272 : ar;
                        xa[0][rt] = a_frag<K0>(K0 == 7 ? ar7 : ar0, q8);
                        xa[1][rt] = a_frag<K0 + 1>(K0 + 1 == 7 ? ar7 : ar0, q8);
                        if constexpr (G8) {
                            if constexpr (PAIR) {
                                const uint8_t* dxa = (l >> 4) == 0 ? ar0 : lds + S_ZERO;
                                dxh[0][rt] = *reinterpret_cast<const uint16_t*>(dxa + K0 * Q81_BYTES);
                                dxh[1][rt] = *reinterpret_cast<const uint16_t*>(dxa + (K0 + 1) * Q81_BYTES);
                            } else {
                                dxh[0][rt] = *reinterpret_cast<const uint16_t*>(ar0 + K0 * Q81_BYTES) & kmask;
                                dxh[1][rt] = *reinterpret_cast<const uint16_t*>(ar0 + (K0 + 1) * Q81_BYTES) & kmask;
                            }
                        } else {
                            dx4[0][rt] = *reinterpret_cast<const float4*>(dxt + K0 * 32 + rt * 16 + q8 / 2);
                            dx4[1][rt] = *reinterpret_cast<const float4*>(dxt + (K0 + 1) * 32 + rt * 16 + q8 / 2);
                        }
                    }
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                        for (int rt = 0; rt < NL; ++rt)
#pragma unroll
                            for (int m = 0; m < NM; ++m) {
                                const i32x4 z = {0, 0, 0, 0};
                                d[kk][rt][m] = __builtin_amdgcn_mfma_i32_16x16x32_i8(xa[kk][rt], wb[kk][m], z, 0, 0, 0);
                                if constexpr (G8) {
                                    const f32x4 zf = {0.0f, 0.0f, 0.0f, 0.0f};
                                    sc[kk][rt][m] = __builtin_amdgcn_mfma_f32_16x16x16f16(
                                        PAIR ? dx_term<K0>(dxh[kk][rt], kk) : half4_lo(dxh[kk][rt]),
                                        PAIR ? dws[m] : half4_lo(dwh[kk][m]), zf, 0, 0, 0);
                                }
                            }
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                        for (int rt = 0; rt < NL; ++rt) {
                            if constexpr (G8) {
#pragma unroll
                                for (int m = 0; m < NM; ++m)
#pragma unroll
                                    for (int i = 0; i < 4; ++i)
                                        acc[rt][m][i] = fmaf((float)d[kk][rt][m][i], sc[kk][rt][m][i], acc[rt][m][i]);
                            } else {
                                const float dxv[4] = {dx4[kk][rt].x, dx4[kk][rt].y, dx4[kk][rt].z, dx4[kk][rt].w};
#pragma unroll
                                for (int m = 0; m < NM; ++m)
#pragma unroll
                                    for (int i = 0; i < 4; ++i)
                                        acc[rt][m][i] = fmaf((float)d[kk][rt][m][i], dwv[kk][m] * dxv[i], acc[rt][m][i]);
                            }
                        }
                };
                two_blocks(std::integral_constant<int, 0>{});
                two_blocks(std::integral_constant<int, 1>{});
                two_blocks(std::integral_constant<int, 2>{});
                two_blocks(std::integral_constant<int, 3>{});
            };
            if (NR == 2 && live[NR - 1]) run_step(std::integral_constant<int, NR>{});
            else run_step(std::integral_constant<int, 1>{});
        };

        // step s is in LDS once every wave has waited for its own loads and
        // passed the barrier; every wave is then also done with the step
        // before, whose buffer takes the next step's loads
        // the next unit's ticket: drawn two steps before the last (its
        // result is in after the next step's wait), published by the barrier
        // of the step after; a unit of one or two steps draws at its last
        // step and waits for it
        // the next unit is drawn only in its last row tile; before that the
        // next row tile of the same routes follows, with no lookup
        const bool last_tile = ti + 1 == TPU;
        uint32_t t_pend = 0;
        // the gate/up on the GEMM layout looks the next unit up in LDS a step
        // before the last, and wave 0 fetches its 64 route entries into LDS
        // then (the last step's wait covers the load, its barrier publishes
        // the entries)
        constexpr bool EARLY = G8 && PAIR;
        bool x_done = false, x_has = false, x_more = false;
        uint32_t x_un = 0, x_nt = 0;
        int x_ne = 0, x_nrb = 0, x_nnr = 0;
        for (int s = 0; s + 1 < nsteps; ++s, ++g) {
            wait_vm0();
            if (last_tile && nsteps >= 3 && s == nsteps - 2 && threadIdx.x == 0) s_tick = t_pend;
            lds_barrier();
            load_step(e, t, a_off, s + 1, (g & 1) ^ 1);
            if (last_tile && nsteps >= 3 && s == nsteps - 3 && threadIdx.x == 0) t_pend = draw();
            if (EARLY && use_tab && last_tile && nsteps >= 3 && s == nsteps - 2) {
                x_un = first + s_tick;
                x_more = x_un < end;
                x_has = x_more && unit_at_lds(tab, (uint32_t)p.tiles, n_active, l, x_un, x_ne, x_nrb, x_nnr, x_nt);
                if (x_has && wave == 0) load_lds4(route + x_nrb + min(l, x_nnr - 1), lds0 + S_ROUTES);
                x_done = true;
            }
            if (live[0]) compute(g & 1);
        }
        if (last_tile && nsteps < 3) {
            if (threadIdx.x == 0) s_tick = draw();
            lds_barrier();
        }
        // the last step: the next unit's lookup and activation sources are
        // read while this step's data arrives, and its first step loads while
        // this one is computed
        uint32_t un = 0;
        int ne = e, nrb = rbegin, nnr = nr;
        uint32_t nt = t + 1;
        bool more = true, has_next = true;
        if (last_tile && EARLY && x_done) {
            un = x_un;
            more = x_more;
            has_next = x_has;
            ne = x_ne;
            nrb = x_nrb;
            nnr = x_nnr;
            nt = x_nt * (uint32_t)TPU;
        } else if (last_tile) {
            un = first + s_tick;
            more = un < end;
            has_next = more && lookup(un, ne, nrb, nnr, nt);
            nt *= (uint32_t)TPU;
            if (has_next) stage_act(p, G, nrb, nnr, a_off);   // this unit's are no longer needed
        }
        wait_vm0();
        lds_barrier();
        if (EARLY && x_done && has_next) {
            // the activation sources of the next unit from its route entries in LDS
            const int32_t* rr = reinterpret_cast<const int32_t*>(lds + S_ROUTES);
            int rts[S_SLOTS];
#pragma unroll
            for (int j = 0; j < S_SLOTS; ++j) rts[j] = rr[min(max(G.a_slot[j], 0), nnr - 1)];
            stage_offsets(p, G, nnr, rr[0], rts, a_off);
        }
        if (has_next) load_step(ne, nt, a_off, 0, (g & 1) ^ 1);
        if (live[0]) compute(g & 1);
        ++g;

        // lane (c, q) holds row rh + c (of each matrix) of route slots 16 tile + 4q + i
        const int64_t r0 = (int64_t)t * TILE_ROWS;
#pragma unroll
        for (int rt = 0; rt < NR; ++rt) {
            if (!live[rt]) break;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = out_route[rt][i];
                if (r < 0) continue;
                float* o = p.out + (int64_t)r * p.n + r0 + rh + c;
                if constexpr (PAIR) o[0] = swiglu_ds4_f32(acc[rt][0][i], acc[rt][1][i]);
                else o[0] = acc[rt][0][i];
            }
        }
        if (!has_next) {                               // no load is in flight
            if (more) drain();
            break;
        }
        if (last_tile) {
            u = un;
            ti = 0;
        } else {
            ++ti;
        }
        e = ne;
        rbegin = nrb;
        nr = nnr;
        t = nt;
    }
}

// CUs of the current device (cached per device; 0 if HIP cannot tell).
int compute_units() {
    constexpr int MAX_DEVICES = 64;
    static std::atomic<int> cached[MAX_DEVICES] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (dev >= 0 && dev < MAX_DEVICES) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (dev >= 0 && dev < MAX_DEVICES && cus > 0) cached[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

int validate_weights(const void* w, int64_t row_stride, int64_t k) {
    if (!w) return MOEQ8_EINVAL;
    if (((uintptr_t)w & 3u) != 0 || (row_stride & 3) != 0) return MOEQ8_EALIGN;
    if (row_stride < (k / QK) * Q80_BYTES) return MOEQ8_EINVAL;
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
    if (stage != MOEQ8_GATE_UP_SWIGLU && stage != MOEQ8_DOWN && stage != MOEQ8_GATE_UP_SWIGLU_G8 &&
        stage != MOEQ8_DOWN_G8)
        return MOEQ8_EINVAL;
    const bool g8 = stage == MOEQ8_GATE_UP_SWIGLU_G8 || stage == MOEQ8_DOWN_G8;
    const bool pair = stage == MOEQ8_GATE_UP_SWIGLU || stage == MOEQ8_GATE_UP_SWIGLU_G8;
    if (n < 0 || k <= 0 || k % 64 != 0 || n % 32 != 0) return MOEQ8_EINVAL;
    int st = validate_weights(w_a, w_row_stride_bytes, k);
    if (st) return st;
    if (pair) {
        st = validate_weights(w_b, w_row_stride_bytes, k);
        if (st) return st;
    }
    if (!act_q || !grouping || !out) return MOEQ8_EINVAL;
    if (ncols < 1 || ncols > MOEQ8_MAX_WIDE_COLS || topk < 1 || topk > MOEQ8_MAX_TOPK) return MOEQ8_EINVAL;
    if (n_local_expert < 1) return MOEQ8_EINVAL;
    if (expert_stride_bytes < 0 || (expert_stride_bytes & 3)) return MOEQ8_EALIGN;
    if (n_local_expert > 1 && expert_stride_bytes < n * w_row_stride_bytes) return MOEQ8_EINVAL;
    if (((uintptr_t)act_q & 3u) || ((uintptr_t)grouping & 3u) || ((uintptr_t)out & 3u))
        return MOEQ8_EALIGN;
    if (k / 64 > ((int64_t)1 << 24)) return MOEQ8_EUNSUPPORTED;
    if (n == 0) return MOEQ8_OK;
    const int64_t R = ncols * topk;
    const hipStream_t hs = (hipStream_t)stream;
    GemmParams p = {};
    p.w0 = (const uint8_t*)w_a;
    p.w1 = (const uint8_t*)w_b;
    p.expert_stride = expert_stride_bytes;
    p.row_stride = w_row_stride_bytes;
    p.n = n;
    p.n_local = n_local_expert;
    p.nb = (int32_t)(k / QK);
    p.ncols = (int32_t)ncols;
    p.topk = topk;
    const uint64_t route_div = pair ? (uint64_t)topk : 1u;
    p.act_route_mul = ((1ull << 32) + route_div - 1) / route_div;
    p.act = (const uint8_t*)act_q;
    p.act_row_bytes = (k / QK) * Q81_BYTES;
    p.grouping = (const int32_t*)grouping;
    p.out = out;
    static std::atomic<uint32_t> next_slot{0};
    p.ticket_slot = (int32_t)(next_slot.fetch_add(1, std::memory_order_relaxed) % S_TICKET_SLOTS);
    // the staged form: whole 8-block steps, whole row tiles, 16-byte aligned
    // rows and steps (every staged piece is one aligned 16-byte load), piece
    // offsets within 32 bits (a tile's rows, the activation rows); the down
    // from 4 steps a unit on (k >= 1024; at k = 1024 on the 256-expert layer
    // 119 / 192 / 294 / 407 us at 32 / 128 / 512 / 1024 columns against 117 /
    // 193 / 336 / 497 for the register-fed form, which takes shorter k)
    const int srows = pair ? 32 : 64;
    const int64_t act_rows = pair ? ncols : R;
    const bool staged = (pair || g8 || k >= 4 * S_STEP_BLOCKS * QK) && k % (S_STEP_BLOCKS * QK) == 0 &&
                        n % srows == 0 &&
                        64 * w_row_stride_bytes < ((int64_t)1 << 31) &&
                        act_rows * p.act_row_bytes < ((int64_t)1 << 31) &&
                        (((uintptr_t)w_a | (uintptr_t)w_b | (uintptr_t)act_q | (uint64_t)w_row_stride_bytes |
                          (uint64_t)expert_stride_bytes | (uint64_t)p.act_row_bytes) & 15u) == 0;
    if (staged) {
        const int64_t tiles = n / srows;
        // a unit of at most 4 steps a tile (the down at k = 1024) takes two
        // row tiles of its routes when the tiles pair up: half the unit
        // changes, whose lookup waits on two dependent reads (the down 285 ->
        // 261 and 386 -> 350 us at 512 / 1024 columns on 256 experts); longer
        // units keep one, as two made the last units of a launch too long
        // (the plain rows' gate/up 484 -> 531 us at 512 columns)
        const int tpu = !pair && tiles % 2 == 0 && k <= 4 * S_STEP_BLOCKS * QK ? 2 : 1;
        // an upper bound of the units; the grid is at most two workgroups a
        // CU, a multiple of the XCDs, each taking its units in turn
        const int64_t units = (std::min<int64_t>(R, n_local_expert) + R / S_CHUNK) * (tiles / tpu);
        if (units > 0xffffffffLL) return MOEQ8_EUNSUPPORTED;
        const int cus = compute_units();
        if (cus < 1) return MOEQ8_EHIP;
        const int64_t cap = (int64_t)S_WG_PER_CU * cus;
        const int64_t grid = (std::min<int64_t>(units, cap) + XCDS - 1) / XCDS * XCDS;
        p.tiles = (int32_t)(tiles / tpu);
        const dim3 sg((uint32_t)grid), sb(S_THREADS);
        if (g8 && pair)
            hipLaunchKernelGGL((k_grouped_gemm_staged<true, true>), sg, sb, 0, hs, p);
        else if (g8 && tpu == 2)
            hipLaunchKernelGGL((k_grouped_gemm_staged<false, true, 2>), sg, sb, 0, hs, p);
        else if (g8)
            hipLaunchKernelGGL((k_grouped_gemm_staged<false, true>), sg, sb, 0, hs, p);
        else if (pair)
            hipLaunchKernelGGL(k_grouped_gemm_staged<true>, sg, sb, 0, hs, p);
        else if (tpu == 2)
            hipLaunchKernelGGL((k_grouped_gemm_staged<false, false, 2>), sg, sb, 0, hs, p);
        else
            hipLaunchKernelGGL(k_grouped_gemm_staged<false>, sg, sb, 0, hs, p);
        return check_launch();
    }
    if (g8) return MOEQ8_EUNSUPPORTED;                 // the GEMM layout is read by the staged form only
    const int wg_rows = (pair ? 16 : 32) * GEMM_WAVES;
    const int64_t tiles = (n + wg_rows - 1) / wg_rows;
    // units <= (groups + valid routes / 16) * tiles for any grouping of these
    // routes; one workgroup per unit, rounded up to whole rounds of the XCDs
    const int64_t units = (std::min<int64_t>(R, n_local_expert) + R / chunk_for(pair)) * tiles;
    const int64_t grid = (units + XCDS - 1) / XCDS * XCDS;
    if (grid > 0x7fffffff || units > 0xffffffffLL) return MOEQ8_EUNSUPPORTED;
    p.tiles = (int32_t)tiles;
    if (pair)
        hipLaunchKernelGGL(k_grouped_gemm<true>, dim3((uint32_t)grid), dim3(GEMM_THREADS), 0, hs, p);
    else
        hipLaunchKernelGGL(k_grouped_gemm<false>, dim3((uint32_t)grid), dim3(GEMM_THREADS), 0, hs, p);
    return check_launch();
}
