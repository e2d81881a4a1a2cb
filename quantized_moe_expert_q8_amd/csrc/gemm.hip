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
    const int4w hdr = grouping_words4(p.grouping, 0);
    if ((hdr[2] != p.ncols) | (hdr[3] != p.topk) | (hdr[0] < 0) | (hdr[0] > Rk) | (hdr[1] < 0) |
        (hdr[1] > Rk))
        return;
    const int n_active = hdr[0];
    const uint32_t tiles = (uint32_t)p.tiles;
    const uint32_t xcd = blockIdx.x % XCDS;
    const uint32_t slot = blockIdx.x / XCDS;
    // chunks <= n_active + n_valid / CHUNK, so slots past this bound have nothing
    const uint32_t bound = ((uint32_t)n_active + (uint32_t)hdr[1] / CHUNK) * tiles;
    if (slot >= (bound + XCDS - 1) / XCDS) return;

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
    if (slot >= per + (xcd < extra ? 1u : 0u)) return;
    const uint32_t u = xcd * per + min(xcd, extra) + slot;
    int e = 0, gbegin = 0, gend = 0;
    uint32_t ubase = 0;
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
    if (gend <= gbegin) return;
    const uint32_t nchunk = (uint32_t)(gend - gbegin + CHUNK - 1) / CHUNK;
    const uint32_t rem = u - ubase;
    const uint32_t t = rem / nchunk;                   // row tile
    const int rbegin = gbegin + (int)(rem - t * nchunk) * CHUNK;
    const int nr = min(gend - rbegin, CHUNK);          // routes of this unit, 1..CHUNK

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
    const int wg_rows = (pair ? 16 : 32) * GEMM_WAVES;
    const int64_t tiles = (n + wg_rows - 1) / wg_rows;
    // units <= (groups + valid routes / 16) * tiles for any grouping of these
    // routes; one workgroup per unit, rounded up to whole rounds of the XCDs
    const int64_t R = ncols * topk;
    const int64_t units = (std::min<int64_t>(R, n_local_expert) + R / chunk_for(pair)) * tiles;
    const int64_t grid = (units + XCDS - 1) / XCDS * XCDS;
    if (grid > 0x7fffffff || units > 0xffffffffLL) return MOEQ8_EUNSUPPORTED;

    GemmParams p = {};
    p.w0 = (const uint8_t*)w_a;
    p.w1 = (const uint8_t*)w_b;
    p.expert_stride = expert_stride_bytes;
    p.row_stride = w_row_stride_bytes;
    p.n = n;
    p.n_local = n_local_expert;
    p.nb = (int32_t)(k / QK);
    p.tiles = (int32_t)tiles;
    p.ncols = (int32_t)ncols;
    p.topk = topk;
    const uint64_t route_div = pair ? (uint64_t)topk : 1u;
    p.act_route_mul = ((1ull << 32) + route_div - 1) / route_div;
    p.act = (const uint8_t*)act_q;
    p.act_row_bytes = (k / QK) * Q81_BYTES;
    p.grouping = (const int32_t*)grouping;
    p.out = out;
    const hipStream_t hs = (hipStream_t)stream;
    if (pair)
        hipLaunchKernelGGL(k_grouped_gemm<true>, dim3((uint32_t)grid), dim3(GEMM_THREADS), 0, hs, p);
    else
        hipLaunchKernelGGL(k_grouped_gemm<false>, dim3((uint32_t)grid), dim3(GEMM_THREADS), 0, hs, p);
    return check_launch();
}
