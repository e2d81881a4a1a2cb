// Device-side building blocks shared by every libmoeq8 kernel (gfx950, wave64).
//
// Block formats: Q8_0 = {fp16 d; int8 qs[32]} (34 B), q8_1 = {fp16 d; fp16 s;
// int8 qs[32]} (36 B), rows of K/32 consecutive blocks.
//
// Reduction order of every Q8_0 x q8_1 product (single, gate/up pair, grouped):
//   * A row is cut into 2-block chunks (68 weight bytes, 72 activation bytes).
//     Absolute chunk c (counted from the first block of the FULL row, so a
//     column-range slice starting at block k_block_offset has its first chunk at
//     c = k_block_offset / 2) belongs to logical lane c % 16, round c / 16.
//   * Chunk value: p(b) = (fp32(d_w) * fp32(d_x)) * float(sumi_b) for its two
//     blocks b, then p(b0) + p(b1).  fp32(d_w) * fp32(d_x) is exact.
//   * Logical lane l accumulates its chunks' values in ascending round order,
//     starting from +0.
//   * The 16 lane sums are added as a pairwise tree (xor 1, 2, 4, 8).
// The order never depends on the number of columns, on whether one or two
// matrices are read, on which rows are launched, or on grouping, so the pair
// equals the separate products, the grouped launch equals per-route products,
// results are batch invariant, and a slice equals the zero-padded full row
// (a zero chunk adds +0, which leaves a lane sum unchanged): the properties the
// RDNA4 Q8_0 gate/up pair and whole-row-lane slice commits of lucebox PR #826
// state for their kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moeq8 {

constexpr int QK = 32;
constexpr int Q80_BYTES = 34;
constexpr int Q81_BYTES = 36;
constexpr int LANES_PER_ROW = 16;       // logical lanes of one row
constexpr int BLOCKS_PER_CHUNK = 2;     // blocks per lane per round
constexpr int W_CHUNK_BYTES = BLOCKS_PER_CHUNK * Q80_BYTES;  // 68
constexpr int X_CHUNK_BYTES = BLOCKS_PER_CHUNK * Q81_BYTES;  // 72
constexpr int W_CHUNK_DWORDS = W_CHUNK_BYTES / 4;            // 17
constexpr int X_CHUNK_DWORDS = X_CHUNK_BYTES / 4;            // 18
constexpr float SWIGLU_LIMIT = 7.0f;

// Word index of the per-group table of an expert grouping with R routes: it
// follows the header, expert[R], offset[R+1], route[R] and eight words of
// padding, rounded up to a 16-byte boundary.  Entry a (4 words) is
// {expert[a], offset[a], offset[a+1], 0}.
__host__ __device__ constexpr int64_t grouping_table_word(int64_t R) {
    return (4 + 3 * R + 1 + 8 + 3) & ~(int64_t)3;
}

// Grouping words are written by an earlier launch and only read in this one,
// so they may be read through the constant address space: wave-uniform
// indices then become scalar loads, which do not queue behind the vector loads
// of weights already in flight.  Eight or four consecutive words from word i
// (4-byte alignment; the buffer is padded so that eight words from any route
// entry stay inside it).
typedef int32_t int8w __attribute__((ext_vector_type(8), aligned(4)));
typedef int32_t int4w __attribute__((ext_vector_type(4), aligned(4)));
__device__ __forceinline__ int8w grouping_words8(const int32_t* g, int64_t i) {
    return *(const __attribute__((address_space(4))) int8w*)(g + i);
}
__device__ __forceinline__ int4w grouping_words4(const int32_t* g, int64_t i) {
    return *(const __attribute__((address_space(4))) int4w*)(g + i);
}

// 16-byte vectors that only promise 4-byte alignment: the 34-byte blocks put
// chunks on 4-byte boundaries, and gfx950 global loads accept that.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2), aligned(4)));

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(bits16 & 0xffffu));
}

// Pins an fp32 value in a register so that instruction selection cannot fold
// the operation that produced it into its consumer.  Needed where an fp32
// rounding is part of the definition: without it hipcc turns
// fp16(a * b) into one v_fma_mixlo_f16, rounding once instead of twice.
__device__ __forceinline__ float materialize_f32(float x) {
    asm volatile("" : "+v"(x));
    return x;
}

__device__ __forceinline__ uint32_t float_to_half_bits(float f) {
    // round to nearest even (the default rounding mode), subnormals kept
    return (uint32_t)__builtin_bit_cast(unsigned short, (_Float16)f);
}

struct WChunk { uint32_t v[W_CHUNK_DWORDS]; };
struct XChunk { uint32_t v[X_CHUNK_DWORDS]; };

#ifndef MOEQ8_NT_WEIGHTS
#define MOEQ8_NT_WEIGHTS 0
#endif

// Raw 68 bytes of a weight chunk (4-byte aligned address).
__device__ __forceinline__ void load_w_chunk(WChunk& w, const uint8_t* p) {
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#if MOEQ8_NT_WEIGHTS
        u32x4 t = __builtin_nontemporal_load(q + i);
#else
        u32x4 t = q[i];
#endif
        w.v[4 * i + 0] = t.x;
        w.v[4 * i + 1] = t.y;
        w.v[4 * i + 2] = t.z;
        w.v[4 * i + 3] = t.w;
    }
#if MOEQ8_NT_WEIGHTS
    w.v[16] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p + 64));
#else
    w.v[16] = *reinterpret_cast<const uint32_t*>(p + 64);
#endif
}

// Raw 72 bytes of an activation chunk (8-byte aligned address).
__device__ __forceinline__ void load_x_chunk(XChunk& x, const uint8_t* p) {
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        u32x4 t = q[i];
        x.v[4 * i + 0] = t.x;
        x.v[4 * i + 1] = t.y;
        x.v[4 * i + 2] = t.z;
        x.v[4 * i + 3] = t.w;
    }
    u32x2 t = *reinterpret_cast<const u32x2*>(p + 64);
    x.v[16] = t.x;
    x.v[17] = t.y;
}

// Activation chunk from LDS (72 bytes at an 8-byte aligned offset).
__device__ __forceinline__ void load_x_chunk_lds(XChunk& x, const uint8_t* p) {
    const uint2* q = reinterpret_cast<const uint2*>(p);
#pragma unroll
    for (int i = 0; i < 9; ++i) {
        const uint2 t = q[i];
        x.v[2 * i] = t.x;
        x.v[2 * i + 1] = t.y;
    }
}

// The 64-chunk packed layout (P64) of Q8_0 rows whose length is a multiple
// of 4096 values: each 4352-byte segment of 64 chunks (two blocks each) is
// stored with dword d < 16 of chunk c at dword 256 * (d / 4) + 4 * c + d % 4
// and dword 16 of chunk c at dword 1024 + c.  Lane c of a wave that reads the
// segment's chunk c then fetches its 68 bytes as four 16-byte loads at
// 1024-byte steps and one 4-byte load, each load of the wave reading one
// contiguous span (every cache line consumed by one instruction), and holds
// the same 17 dwords as with the plain layout.
typedef uint32_t u32x4a16 __attribute__((ext_vector_type(4), aligned(16)));
constexpr int P64_CHUNKS = 64;
constexpr int P64_SEGMENT_BYTES = P64_CHUNKS * W_CHUNK_BYTES;      // 4352
constexpr int P64_SEGMENT_DWORDS = P64_SEGMENT_BYTES / 4;          // 1088

// Chunk c of a packed segment (16-byte aligned).  NT: nontemporal loads, for
// weights read once; otherwise ordinary loads.
template <bool NT = true>
__device__ __forceinline__ void load_w_chunk_p64(WChunk& w, const uint8_t* seg, int c) {
    const u32x4a16* q = reinterpret_cast<const u32x4a16*>(seg) + c;
    const uint32_t* tail = reinterpret_cast<const uint32_t*>(seg + 4096) + c;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        u32x4a16 t;
        if constexpr (NT) t = __builtin_nontemporal_load(q + 64 * i);
        else t = q[64 * i];
        w.v[4 * i + 0] = t.x;
        w.v[4 * i + 1] = t.y;
        w.v[4 * i + 2] = t.z;
        w.v[4 * i + 3] = t.w;
    }
    if constexpr (NT) w.v[16] = __builtin_nontemporal_load(tail);
    else w.v[16] = *tail;
}

// Source dword (index 17 c + d of the plain segment) of packed dword p.
__host__ __device__ constexpr int p64_source_dword(int p) {
    return p < 1024 ? 17 * ((p & 255) >> 2) + 4 * (p >> 8) + (p & 3) : 17 * (p - 1024) + 16;
}

__device__ __forceinline__ void zero_w_chunk(WChunk& w) {
#pragma unroll
    for (int i = 0; i < W_CHUNK_DWORDS; ++i) w.v[i] = 0u;
}

__device__ __forceinline__ void zero_x_chunk(XChunk& x) {
#pragma unroll
    for (int i = 0; i < X_CHUNK_DWORDS; ++i) x.v[i] = 0u;
}

// Value of one chunk: two blocks, each (d_w * d_x) * sumi, then their sum.
// Weight block 0 occupies bytes 0..33 (d in the low half of dword 0, quants at
// byte 2, so each quant dword is funnel-shifted out of two loaded dwords);
// weight block 1 occupies bytes 34..67 (d in the high half of dword 8, quants in
// dwords 9..16).  Activation block 0: dword 0 = d | s << 16, quants dwords 1..8;
// block 1: dword 9, quants dwords 10..17.
__device__ __forceinline__ float chunk_dot(const WChunk& w, const XChunk& x) {
    int s0 = 0, s1 = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t q0 = (w.v[j] >> 16) | (w.v[j + 1] << 16);
        s0 = __builtin_amdgcn_sdot4((int)q0, (int)x.v[1 + j], s0, false);
        s1 = __builtin_amdgcn_sdot4((int)w.v[9 + j], (int)x.v[10 + j], s1, false);
    }
    const float dw0 = half_bits_to_float(w.v[0]);
    const float dw1 = half_bits_to_float(w.v[8] >> 16);
    const float dx0 = half_bits_to_float(x.v[0]);
    const float dx1 = half_bits_to_float(x.v[9]);
    const float p0 = (dw0 * dx0) * (float)s0;
    const float p1 = (dw1 * dx1) * (float)s1;
    return p0 + p1;
}

// Reciprocal of a block scale for q8_code: NaN for a scale below the normal
// range, which sends every value of the block to the IEEE division.
__device__ __forceinline__ float q8_code_rcp(float d) {
    return d >= 0x1p-126f ? __builtin_amdgcn_rcpf(d) : __builtin_nanf("");
}

// Code of x in a block of scale d (|x| <= 127 d): roundf of the correctly
// rounded fp32 quotient x / d, as the block rule defines it, without a
// division for almost every value.  t = x * rcp(d) is within 3.1e-5 of the
// correctly rounded quotient (v_rcp_f32 within an ulp, one rounded multiply,
// |x / d| <= 127), so where t lies more than 2^-12 from every half-integer
// both round to the same integer and rint(t) is it; the other values (and a
// NaN t from q8_code_rcp) take the IEEE division.  The division is the rule;
// this only decides when it can be skipped.
__device__ __forceinline__ int q8_code(float x, float d, float rd) {
    const float t = x * rd;
    const float r = __builtin_rintf(t);
    const bool near = !(fabsf(t - r) < 0.5f - 0x1p-12f);
    int q = (int)r;
    if (__builtin_expect(__ballot(near) != 0, 0)) {
        if (near) q = (int)roundf(x / d);
    }
    return q;
}

// Quantise one 32-value block (the block rule of both formats): fp32
// d = amax / 127 (IEEE division), q = roundf(x / d) on the fp32 quotient
// (halves away from zero), d stored as fp16 (nearest even); q8_1 adds
// s = fp16(d * sum(q)) with the fp32 product rounded first.  An all-zero block
// gives all-zero bytes.  dst: 36 bytes (q8_1, 4-byte aligned) or 34 bytes
// (Q8_0, 2-byte aligned), global or LDS.
template <bool Q81>
__device__ __forceinline__ void quantize_block(const float* __restrict__ src, uint8_t* dst) {
    float v[QK];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < QK; ++i) {
        v[i] = src[i];
        amax = fmaxf(amax, fabsf(v[i]));
    }
    const float d = amax / 127.0f;
    const float rd = q8_code_rcp(d);
    uint32_t packed[QK / 4];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < QK / 4; ++i) packed[i] = 0u;
    if (d != 0.0f) {
#pragma unroll
        for (int i = 0; i < QK; ++i) {
            const int q = q8_code(v[i], d, rd);
            sum += q;
            packed[i / 4] |= ((uint32_t)q & 0xffu) << (8 * (i % 4));
        }
    }
    const uint32_t dbits = float_to_half_bits(d);
    if constexpr (Q81) {
        uint32_t* o = reinterpret_cast<uint32_t*>(dst);
        // s = fp16 of the fp32 product (two roundings, as defined)
        const uint32_t sbits = float_to_half_bits(materialize_f32(d * (float)sum));
        o[0] = dbits | (sbits << 16);
#pragma unroll
        for (int i = 0; i < QK / 4; ++i) o[1 + i] = packed[i];
    } else {
        uint16_t* o = reinterpret_cast<uint16_t*>(dst);
        o[0] = (uint16_t)dbits;
#pragma unroll
        for (int i = 0; i < QK / 4; ++i) {
            o[1 + 2 * i] = (uint16_t)(packed[i] & 0xffffu);
            o[2 + 2 * i] = (uint16_t)(packed[i] >> 16);
        }
    }
}

// ---- 4-bit weight blocks -------------------------------------------------
// Q4 block = {fp16 d; uint8 qs[16]} (18 B): value i < 16 in the low nibble of
// qs[i], value i + 16 in the high nibble, w = d * (code - 8).  A chunk is two
// blocks (36 B, dword aligned in any row of an even number of blocks): block
// 0's d in the low half of dword 0 and its codes at bytes 2..17 (so each code
// dword is funnel-shifted out of two loaded dwords), block 1's d in the high
// half of dword 4 and its codes in dwords 5..8.
constexpr int Q4_BYTES = 18;
constexpr int W4_CHUNK_BYTES = BLOCKS_PER_CHUNK * Q4_BYTES;   // 36
constexpr int W4_CHUNK_DWORDS = W4_CHUNK_BYTES / 4;           // 9

struct W4Chunk { uint32_t v[W4_CHUNK_DWORDS]; };

__device__ __forceinline__ void load_w_chunk(W4Chunk& w, const uint8_t* p) {
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#if MOEQ8_NT_WEIGHTS
        u32x4 t = __builtin_nontemporal_load(q + i);
#else
        u32x4 t = q[i];
#endif
        w.v[4 * i + 0] = t.x;
        w.v[4 * i + 1] = t.y;
        w.v[4 * i + 2] = t.z;
        w.v[4 * i + 3] = t.w;
    }
    w.v[8] = *reinterpret_cast<const uint32_t*>(p + 32);
}

__device__ __forceinline__ void zero_w_chunk(W4Chunk& w) {
#pragma unroll
    for (int i = 0; i < W4_CHUNK_DWORDS; ++i) w.v[i] = 0u;
}

// The 64-chunk packed layout of 4-bit rows (the P64 rule for 9-dword chunks):
// each 2304-byte segment of 64 chunks stores dword d < 8 of chunk c at dword
// 256 * (d / 4) + 4 * c + d % 4 and dword 8 at dword 512 + c, so lane c
// fetches its 36 bytes as two 16-byte loads 1024 bytes apart and one 4-byte
// load, each load of the wave one contiguous span, and holds the same 9
// dwords as with the plain layout.
constexpr int P64Q4_SEGMENT_BYTES = P64_CHUNKS * W4_CHUNK_BYTES;    // 2304
constexpr int P64Q4_SEGMENT_DWORDS = P64Q4_SEGMENT_BYTES / 4;       // 576

template <bool NT = true>
__device__ __forceinline__ void load_w_chunk_p64(W4Chunk& w, const uint8_t* seg, int c) {
    const u32x4a16* q = reinterpret_cast<const u32x4a16*>(seg) + c;
    const uint32_t* tail = reinterpret_cast<const uint32_t*>(seg + 2048) + c;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        u32x4a16 t;
        if constexpr (NT) t = __builtin_nontemporal_load(q + 64 * i);
        else t = q[64 * i];
        w.v[4 * i + 0] = t.x;
        w.v[4 * i + 1] = t.y;
        w.v[4 * i + 2] = t.z;
        w.v[4 * i + 3] = t.w;
    }
    if constexpr (NT) w.v[8] = __builtin_nontemporal_load(tail);
    else w.v[8] = *tail;
}

// Source dword (index 9 c + d of the plain segment) of packed dword p.
__host__ __device__ constexpr int p64q4_source_dword(int p) {
    return p < 512 ? 9 * ((p & 255) >> 2) + 4 * (p >> 8) + (p & 3) : 9 * (p - 512) + 8;
}

// -8 times the quant sum of each block of a q8_1 chunk (v_dot4 against -8 in
// every byte): the term that turns a dot product of raw 4-bit codes (0..15,
// valid signed bytes) into one of code - 8.  Computed once per activation
// chunk and shared by every weight chunk it meets.
struct XBias { int b0, b1; };

__device__ __forceinline__ XBias q4_x_bias(const XChunk& x) {
    constexpr int M8 = (int)0xF8F8F8F8u;                            // four int8 -8
    int b0 = 0, b1 = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        b0 = __builtin_amdgcn_sdot4(M8, (int)x.v[1 + i], b0, false);
        b1 = __builtin_amdgcn_sdot4(M8, (int)x.v[10 + i], b1, false);
    }
    return {b0, b1};
}

// Value of a 4-bit chunk against a q8_1 chunk, in the same form as the Q8_0
// chunk: (d_w * d_x) * sumi per block, then the sum of the two blocks.  sumi
// is the exact integer sum of (code - 8) * q, taken as sum(code * q) started
// from the block's -8 * sum(q) (xb, from q4_x_bias of the same chunk): the same
// integer as summing (code - 8) * q term by term.
__device__ __forceinline__ float chunk_dot(const W4Chunk& w, const XChunk& x, const XBias& xb) {
    int s0 = xb.b0, s1 = xb.b1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t c0 = (w.v[i] >> 16) | (w.v[i + 1] << 16);   // block 0, bytes 4i .. 4i+3
        s0 = __builtin_amdgcn_sdot4((int)(c0 & 0x0f0f0f0fu), (int)x.v[1 + i], s0, false);
        s0 = __builtin_amdgcn_sdot4((int)((c0 >> 4) & 0x0f0f0f0fu), (int)x.v[5 + i], s0, false);
        const uint32_t c1 = w.v[5 + i];                             // block 1
        s1 = __builtin_amdgcn_sdot4((int)(c1 & 0x0f0f0f0fu), (int)x.v[10 + i], s1, false);
        s1 = __builtin_amdgcn_sdot4((int)((c1 >> 4) & 0x0f0f0f0fu), (int)x.v[14 + i], s1, false);
    }
    const float dw0 = half_bits_to_float(w.v[0]);
    const float dw1 = half_bits_to_float(w.v[4] >> 16);
    const float dx0 = half_bits_to_float(x.v[0]);
    const float dx1 = half_bits_to_float(x.v[9]);
    const float p0 = (dw0 * dx0) * (float)s0;
    const float p1 = (dw1 * dx1) * (float)s1;
    return p0 + p1;
}

// The 4-bit block rule: fp32 d = amax / 7 (IEEE division), code =
// clamp(roundf(x / d), -8, 7) + 8 on the fp32 quotient, d stored fp16 (nearest
// even); an all-zero block has d = 0 and every code 8.  dst: 18 bytes, 2-byte
// aligned.
__device__ __forceinline__ void quantize_block_q4(const float* __restrict__ src, uint8_t* dst) {
    float v[QK];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < QK; ++i) {
        v[i] = src[i];
        amax = fmaxf(amax, fabsf(v[i]));
    }
    const float d = amax / 7.0f;
    uint32_t code[QK];
#pragma unroll
    for (int i = 0; i < QK; ++i) {
        int q = 0;
        if (d != 0.0f) q = min(7, max(-8, (int)roundf(v[i] / d)));
        code[i] = (uint32_t)(q + 8);
    }
    uint16_t* o = reinterpret_cast<uint16_t*>(dst);
    o[0] = (uint16_t)float_to_half_bits(d);
#pragma unroll
    for (int i = 0; i < QK / 4; ++i)                   // bytes 2i, 2i+1 of qs
        o[1 + i] = (uint16_t)(code[2 * i] | (code[16 + 2 * i] << 4) |
                              ((code[2 * i + 1] | (code[16 + 2 * i + 1] << 4)) << 8));
}

// The q8_1 block rule on half a block: this lane holds 16 of the block's 32
// values, the neighbouring lane (lane ^ 1) the other 16.  The block's amax and
// its integer quant sum are combined across the pair (max and integer sums do
// not depend on order), so both lanes see the same d and s.  Every lane of the
// wave must call this; lanes with active == false write nothing.
__device__ __forceinline__ void quantize_half_q81(const float (&v)[QK / 2], int half, bool active,
                                                  uint8_t* block) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < QK / 2; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0xB1,
                                                                   0xf, 0xf, false)));
    const float d = amax / 127.0f;
    const float rd = q8_code_rcp(d);
    uint32_t packed[QK / 8] = {0u, 0u, 0u, 0u};
    int sum = 0;
    if (d != 0.0f) {
#pragma unroll
        for (int i = 0; i < QK / 2; ++i) {
            const int q = q8_code(v[i], d, rd);
            sum += q;
            packed[i / 4] |= ((uint32_t)q & 0xffu) << (8 * (i % 4));
        }
    }
    sum += __builtin_amdgcn_update_dpp(0, sum, 0xB1, 0xf, 0xf, false);
    if (active) {
        uint32_t* o = reinterpret_cast<uint32_t*>(block);
        if (half == 0) {
            // s = fp16 of the fp32 product (two roundings, as defined)
            const uint32_t sbits = float_to_half_bits(materialize_f32(d * (float)sum));
            o[0] = float_to_half_bits(d) | (sbits << 16);
        }
#pragma unroll
        for (int j = 0; j < QK / 8; ++j) o[1 + 4 * half + j] = packed[j];
    }
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
    v = v + __int_as_float(__builtin_amdgcn_update_dpp(0, iv, 0x140, 0xf, 0xf, false));
    return v;
}

// SwiGLU-DS4 in fp32: silu(min(g, 7)) * clamp(u, -7, 7).
__device__ __forceinline__ float swiglu_ds4_f32(float g, float u) {
    const float gc = fminf(g, SWIGLU_LIMIT);
    const float uc = fminf(fmaxf(u, -SWIGLU_LIMIT), SWIGLU_LIMIT);
    const float silu = gc / (1.0f + expf(-gc));
    return silu * uc;
}

}  // namespace moeq8
