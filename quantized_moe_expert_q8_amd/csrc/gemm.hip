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

#include <type_traits>

namespace moeq8 {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

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

// The work unit of this workgroup: units are (group, row tile, chunk of up
// to CHUNK of the group's routes), numbered chunk-fastest; unit u runs on XCD
// u / ceil(units / 8) (workgroups are dispatched to the 8 XCDs round-robin),
// so the chunks that read the same weight rows run on one XCD close together
// in time.  Returns false when this workgroup has no unit.  Every lane of the
// workgroup gets the same answer (wave-uniform values only).
template <int CHUNK>
__device__ __forceinline__ bool find_unit(const GemmParams& p, int l, int& e, int& rbegin, int& nr, uint32_t& t) {
    const int Rk = p.ncols * p.topk;
    const int4w hdr = grouping_words4(p.grouping, 0);
    if ((hdr[2] != p.ncols) | (hdr[3] != p.topk) | (hdr[0] < 0) | (hdr[0] > Rk) | (hdr[1] < 0) |
        (hdr[1] > Rk))
        return false;
    const int n_active = hdr[0];
    const uint32_t tiles = (uint32_t)p.tiles;
    const uint32_t xcd = blockIdx.x % XCDS;
    const uint32_t slot = blockIdx.x / XCDS;
    // chunks <= n_active + n_valid / CHUNK, so slots past this bound have nothing
    const uint32_t bound = ((uint32_t)n_active + (uint32_t)hdr[1] / CHUNK) * tiles;
    if (slot >= (bound + XCDS - 1) / XCDS) return false;

    const int4* table = reinterpret_cast<const int4*>(p.grouping + grouping_table_word(Rk));
    auto units_of = [&](int a, int4& g) -> uint32_t {
        if (a >= n_active) return 0u;
        g = table[a];
        const bool ok = (g.x >= 0) & (g.x < p.n_local) & (g.y >= 0) & (g.z >= g.y) & (g.z <= Rk);
        return ok ? (uint32_t)((g.z - g.y + CHUNK - 1) / CHUNK) * tiles : 0u;
    };
    uint32_t total = 0;
    for (int b0 = 0; b0 < n_active; b0 += 64) {
        int4 g;
        const uint32_t s = wave_incl_scan(units_of(b0 + l, g), l);
        total += (uint32_t)__builtin_amdgcn_readlane((int)s, 63);
    }
    const uint32_t per = total / XCDS, extra = total % XCDS;
    if (slot >= per + (xcd < extra ? 1u : 0u)) return false;
    const uint32_t u = xcd * per + min(xcd, extra) + slot;
    int gbegin = 0, gend = 0;
    uint32_t ubase = 0;
    e = 0;
    {
        uint32_t carry = 0;
        for (int b0 = 0; b0 < n_active; b0 += 64) {
            int4 g = make_int4(0, 0, 0, 0);
            const uint32_t un = units_of(b0 + l, g);
            const uint32_t incl = wave_incl_scan(un, l) + carry;
            const bool hit = (un > 0) & (incl - un <= u) & (u < incl);
            const uint64_t m = __ballot(hit);
            if (m) {
                const int src = __builtin_ctzll(m);
                e = __builtin_amdgcn_readlane(g.x, src);
                gbegin = __builtin_amdgcn_readlane(g.y, src);
                gend = __builtin_amdgcn_readlane(g.z, src);
                ubase = (uint32_t)__builtin_amdgcn_readlane((int)(incl - un), src);
                break;
            }
            carry = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
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

// Staged gate/up pair (k % 256 == 0, n % 32 == 0, 16-byte aligned operands):
// a workgroup of eight waves stages each K step of 8 blocks (256 values) of
// 32 rows of the gate and of the up matrix and of its routes' activations in
// LDS with direct 16-byte global-to-LDS loads (no registers on the way), the
// next step in flight while one is computed, and every wave reads its
// matrix-core fragments from there: a staged weight row serves all four
// route tiles and a staged activation row both row groups, so each byte is
// fetched once per workgroup (the register-fed form above fetches each
// activation once per wave).  Only whole 16-route tiles that hold routes are
// staged and run.  Wave w runs rows 16 (w & 1) + [0, 16) of both matrices
// against route tile w >> 1.
//   LDS per step: weights 64 rows x 272 bytes (a row's 8 blocks, as stored),
//   activations 64 routes x 288 bytes; per wave, fp32 activation scales of
//   its route slots.  Every wave issues the same six loads a step (pieces it
//   has no use for go to a scratch area of LDS), so the wait for a step is a
//   fixed count of loads still in flight.  A weight row's quants sit 2 bytes
//   into each 34-byte block, so a fragment of an even block is cut from three
//   aligned dwords.
// Arithmetic and order are those of the form above: acc = fma(float(sumi),
// d_w * d_x, acc), blocks ascending from +0, so both forms give the same bits.
// The form is bound by that per-block scaling (three VALU operations per
// output, row and block) and its LDS reads more than by the loads; with the
// down product's short K (a few steps) the pipeline fill outweighs the shared
// staging, so the down product stays on the register-fed form.
constexpr int S_THREADS = 512;
constexpr int S_CHUNK = 64;                      // routes per unit
constexpr int S_STEP_BLOCKS = 8;                 // blocks per K step
constexpr int S_WROW = S_STEP_BLOCKS * Q80_BYTES;   // 272
constexpr int S_AROW = S_STEP_BLOCKS * Q81_BYTES;   // 288
constexpr int S_W = 64 * S_WROW;                 // 17408: 32 gate rows, then 32 up rows
constexpr int S_A = S_CHUNK * S_AROW;            // 18432: 64 routes
constexpr int S_STAGE = S_W + S_A;               // 35840
constexpr int S_STAGES = 2;                      // steps staged at once
constexpr int S_DX = S_STAGES * S_STAGE;         // per wave: fp32 [8 blocks][16 slots]
constexpr int S_DX_WAVE = S_STEP_BLOCKS * 16 * 4;    // 512
constexpr int S_JUNK = S_DX + 8 * S_DX_WAVE;     // 1 KB target of the loads no wave needs
constexpr int S_LDS = S_JUNK + 1024;             // 76800: two workgroups a CU
constexpr int S_W_LOADS = S_W / 1024;            // 17 wave-loads of 1 KB
constexpr int S_A_LOADS = S_A / 1024;            // 18
constexpr int S_SLOTS = (S_A_LOADS + 7) / 8;     // 3 wave-loads of each kind per wave
constexpr int S_LOADS = 2 * S_SLOTS;             // loads every wave issues a step

// s_waitcnt with vmcnt(n) alone (n < 64; expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

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

__global__ __launch_bounds__(S_THREADS) void k_grouped_gemm_pair_staged(const GemmParams p) {
    __shared__ __align__(16) uint8_t lds[S_LDS];
    const int wave = threadIdx.x >> 6;
    const int l = threadIdx.x & 63;
    const int c = l & 15;
    const int q8 = (l >> 4) * 8;

    const int Rk = p.ncols * p.topk;
    int e, rbegin, nr;
    uint32_t t;
    if (!find_unit<S_CHUNK>(p, l, e, rbegin, nr, t)) return;
    const int64_t r0 = (int64_t)t * 32;                // first row of the unit in each matrix
    const int32_t* route = p.grouping + 4 + 2 * (int64_t)Rk + 1;
    const int nslot = (nr + 15) & ~15;                 // staged route slots: whole tiles
    const int rh = (wave & 1) * 16;                    // this wave's rows (of each matrix)
    const int slot0 = (wave >> 1) * 16;                // and route slots
    const bool live = slot0 < nslot;                   // the tile holds routes

    // per-lane sources of this wave's loads (the same for every K step).  A
    // wave-load past the stage goes to the scratch area; a lane whose piece
    // is past the staged route slots reads the unit's first activation piece
    // (one cached line for all such lanes) into an unused slot.
    const uint8_t* wsrc[S_SLOTS];
    const uint8_t* asrc[S_SLOTS];
    const uint8_t* a_first;
    {
        const int rt = route[rbegin];
        const int rr = (rt >= 0 && rt < Rk) ? rt : 0;
        a_first = p.act + (int64_t)(((uint64_t)(uint32_t)rr * p.act_route_mul) >> 32) * p.act_row_bytes;
    }
#pragma unroll
    for (int j = 0; j < S_SLOTS; ++j) {
        const int i = 8 * j + wave;                    // wave-load index
        const int piece = min(i, S_W_LOADS - 1) * 64 + l;
        const int wrow = piece / 17, part = piece - wrow * 17;
        wsrc[j] = (wrow < 32 ? p.w0 : p.w1) + (int64_t)e * p.expert_stride + (r0 + wrow % 32) * p.row_stride +
                  part * 16;
        const int apiece = min(i, S_A_LOADS - 1) * 64 + l;
        const int slot = apiece / 18, apart = apiece - slot * 18;
        if (i < S_A_LOADS && slot < nslot) {
            const int rt = route[rbegin + min(slot, nr - 1)];
            const int rr = (rt >= 0 && rt < Rk) ? rt : 0;
            const int64_t arow = (int64_t)(((uint64_t)(uint32_t)rr * p.act_route_mul) >> 32);
            asrc[j] = p.act + arow * p.act_row_bytes + apart * 16;
        } else {
            asrc[j] = a_first;
        }
    }
    const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
    auto load_step = [&](int s, int b) {
        const uint32_t base = lds0 + b * S_STAGE;
#pragma unroll
        for (int j = 0; j < S_SLOTS; ++j) {
            const int i = 8 * j + wave;
            load_lds16(wsrc[j] + (int64_t)s * S_WROW, i < S_W_LOADS ? base + i * 1024 : lds0 + S_JUNK);
            load_lds16(asrc[j] + (int64_t)s * S_AROW, i < S_A_LOADS ? base + S_W + i * 1024 : lds0 + S_JUNK);
        }
    };

    float acc[2][4];                                   // [gate, up][route slot slot0 + 4q + i]
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[m][i] = 0.0f;

    float* dxt = reinterpret_cast<float*>(lds + S_DX + wave * S_DX_WAVE);   // [8 blocks][16 slots]
    const int nsteps = p.nb / S_STEP_BLOCKS;
#pragma unroll
    for (int st = 0; st < S_STAGES - 1; ++st)
        if (st < nsteps) load_step(st, st);
    for (int s = 0; s < nsteps; ++s) {
        const int b = s % S_STAGES;
        // step s is in LDS once this wave's loads of the steps after it are
        // all that is left in flight (loads complete in order) and every
        // wave has passed this barrier; every wave is then also done with
        // step s - 1, whose buffer takes step s + S_STAGES - 1
        static_assert(S_STAGES >= 2 && S_STAGES <= 4, "the waits below cover up to two steps ahead");
        const int ahead = min(S_STAGES - 2, nsteps - 1 - s);
        if (ahead >= 2) wait_vm<2 * S_LOADS>();
        else if (ahead == 1) wait_vm<S_LOADS>();
        else wait_vm<0>();
        lds_barrier();
        if (s + S_STAGES - 1 < nsteps) load_step(s + S_STAGES - 1, (s + S_STAGES - 1) % S_STAGES);
        if (!live) continue;
        const uint8_t* W = lds + b * S_STAGE;
        const uint8_t* A = W + S_W;
        // this wave's activation scales, fp32 (read back by this wave only)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int ent = h * 64 + l;
            const int k = ent >> 4, sl = ent & 15;
            dxt[k * 16 + sl] = half_bits_to_float(
                *reinterpret_cast<const uint16_t*>(A + (slot0 + sl) * S_AROW + k * Q81_BYTES));
        }
        const uint8_t* wg = W + (rh + c) * S_WROW;
        const uint8_t* wu = W + (32 + rh + c) * S_WROW;
        const uint8_t* ar = A + (slot0 + c) * S_AROW;
        // two blocks at a time: fragments of both, then the matrix-core
        // products of both, then the scaled sums in block order (block K
        // enters every accumulator before block K + 1)
        auto two_blocks = [&](auto kc) {
            constexpr int K0 = 2 * decltype(kc)::value;
            long wb[2][2], xa[2];
            float dwv[2][2];
            float4 dx4[2];
            i32x4 d[2][2];
            wb[0][0] = w_frag<K0>(wg, q8);
            wb[0][1] = w_frag<K0>(wu, q8);
            wb[1][0] = w_frag<K0 + 1>(wg, q8);
            wb[1][1] = w_frag<K0 + 1>(wu, q8);
            dwv[0][0] = half_bits_to_float(*reinterpret_cast<const uint16_t*>(wg + K0 * Q80_BYTES));
            dwv[0][1] = half_bits_to_float(*reinterpret_cast<const uint16_t*>(wu + K0 * Q80_BYTES));
            dwv[1][0] = half_bits_to_float(*reinterpret_cast<const uint16_t*>(wg + (K0 + 1) * Q80_BYTES));
            dwv[1][1] = half_bits_to_float(*reinterpret_cast<const uint16_t*>(wu + (K0 + 1) * Q80_BYTES));
            xa[0] = a_frag<K0>(ar, q8);
            xa[1] = a_frag<K0 + 1>(ar, q8);
            dx4[0] = *reinterpret_cast<const float4*>(dxt + K0 * 16 + q8 / 2);
            dx4[1] = *reinterpret_cast<const float4*>(dxt + (K0 + 1) * 16 + q8 / 2);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const i32x4 z = {0, 0, 0, 0};
                    d[kk][m] = __builtin_amdgcn_mfma_i32_16x16x32_i8(xa[kk], wb[kk][m], z, 0, 0, 0);
                }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const float dxv[4] = {dx4[kk].x, dx4[kk].y, dx4[kk].z, dx4[kk].w};
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[m][i] = fmaf((float)d[kk][m][i], dwv[kk][m] * dxv[i], acc[m][i]);
            }
        };
        two_blocks(std::integral_constant<int, 0>{});
        two_blocks(std::integral_constant<int, 1>{});
        two_blocks(std::integral_constant<int, 2>{});
        two_blocks(std::integral_constant<int, 3>{});
    }

    // lane (c, q) holds row rh + c of both matrices for route slots slot0 + 4q + i
    if (!live) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int slotr = slot0 + q8 / 2 + i;
        if (slotr >= nr) continue;
        const int r = route[rbegin + slotr];
        if (r < 0 || r >= Rk) continue;
        p.out[(int64_t)r * p.n + r0 + rh + c] = swiglu_ds4_f32(acc[0][i], acc[1][i]);
    }
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
    if (stage != MOEQ8_GATE_UP_SWIGLU && stage != MOEQ8_DOWN) return MOEQ8_EINVAL;
    const bool pair = stage == MOEQ8_GATE_UP_SWIGLU;
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
    // the staged gate/up pair: whole 8-block steps, 16-byte aligned rows and
    // steps (every staged piece is one aligned 16-byte load); n % 32 == 0 holds
    const bool staged = pair && k % (S_STEP_BLOCKS * QK) == 0 &&
                        (((uintptr_t)w_a | (uintptr_t)w_b | (uintptr_t)act_q | (uint64_t)w_row_stride_bytes |
                          (uint64_t)expert_stride_bytes | (uint64_t)p.act_row_bytes) & 15u) == 0;
    if (staged) {
        const int64_t tiles = n / 32;
        const int64_t units = (std::min<int64_t>(R, n_local_expert) + R / S_CHUNK) * tiles;
        const int64_t grid = (units + XCDS - 1) / XCDS * XCDS;
        if (grid > 0x7fffffff || units > 0xffffffffLL) return MOEQ8_EUNSUPPORTED;
        p.tiles = (int32_t)tiles;
        hipLaunchKernelGGL(k_grouped_gemm_pair_staged, dim3((uint32_t)grid), dim3(S_THREADS), 0, hs, p);
        return check_launch();
    }
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
