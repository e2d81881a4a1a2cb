/* libmoeq8 benchmark helpers (not part of the FFN path).
 *
 * 1. Synthetic inputs: fills device memory with Q8_0 weight blocks
 * drawn from a counter-based generator, for benchmark-sized weight sets (tens of
 * GB) that would take minutes to draw and quantise on the host.  Not part of the
 * FFN path; the same generator is implemented independently on the host so any
 * filled block can be reproduced there.
 *
 * Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014).  Output i of the stream with key s is
 * mix(s + (i + 1) * 0x9E3779B97F4A7C15) with
 *   mix(z): z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
 *           z *= 0x94D049BB133111EB; z ^= z >> 31    (all modulo 2^64).
 * Block b of a stream uses outputs 17b .. 17b + 16:
 *   outputs 17b + t, t < 16: element 2t + h takes bytes 4h .. 4h + 3 of the
 *     output (little-endian); v = their sum; q = clamp(((v * 43) >> 7) - 171,
 *     -127, 127);
 *   output 17b + 16 = o: d = fp16 bits 0x0C00 | (o & 0x3FF); element
 *     (o >> 10) & 31 becomes -127 if bit 15 of o is set, else +127.
 * Stream key of (seed, layer, expert, matrix):
 *   mix(((seed & 0xFFFF) << 48 | (layer & 0xFFFF) << 32 | (expert & 0xFFFF) << 16
 *        | (matrix & 0xFFFF)) + 0x9E3779B97F4A7C15).
 */
#ifndef MOEQ8_SYNTH_H
#define MOEQ8_SYNTH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Stream key of (seed, layer, expert, matrix) as defined above (host function). */
uint64_t moeq8_synth_stream_key(uint32_t seed, uint32_t layer, uint32_t expert, uint32_t matrix);

/* Fill `n_mats` consecutive matrices of `blocks_per_mat` Q8_0 blocks each (34 B
 * per block, contiguous, dst 2-byte aligned, device memory owned by the caller).
 * Matrix i holds blocks 0 .. blocks_per_mat-1 of the stream with key
 * moeq8_synth_stream_key(seed, layer0 + i / mats_per_layer,
 *                        expert0 + i % mats_per_layer, matrix).
 * Enqueued on `stream` (hipStream_t); returns 0 or a negative moeq8 status. */
int moeq8_synth_q8_0_fill(void* dst, int64_t n_mats, int64_t blocks_per_mat,
                          int64_t mats_per_layer, uint32_t seed, uint32_t layer0,
                          uint32_t expert0, uint32_t matrix, void* stream);

/* 2. Streaming-read ceiling: reads `bytes` of device memory at `buf` once
 * (`bytes` a multiple of 16, `buf` 16-byte aligned), each workgroup 64 KB with
 * coalesced 16-byte nontemporal loads (the fastest plain read measured on
 * MI355X: 6.46 TB/s for a 214 MB launch against 5.87 TB/s without the
 * nontemporal hint), and folds the words into an xor that is written to
 * `sink` (one uint32, device memory) only if it equals 0x9E3779B9, so the
 * loads cannot be dropped.  Measures what a plain read of the same buffers
 * achieves, the ceiling a bandwidth-bound kernel is compared with.  Enqueued
 * on `stream`; returns 0 or a negative moeq8 status. */
int moeq8_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

/* The same read with `wg_bytes` (8192, 16384, 32768 or 65536) bytes a
 * workgroup; moeq8_stream_read is wg_bytes = 65536.  Which shape reads a given
 * byte count fastest depends on the count (ramp and tail against the number of
 * workgroups), so a ceiling is taken as the best of the shapes.  Other
 * wg_bytes values are MOEQ8_EINVAL. */
int moeq8_stream_read_shape(const void* buf, int64_t bytes, int64_t wg_bytes, uint32_t* sink,
                            void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOEQ8_SYNTH_H */
