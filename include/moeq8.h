/* libmoeq8 -- quantized MoE expert FFN (Q8_0 weights x q8_1 activations) for
 * AMD Instinct MI355X (gfx950).
 *
 * The operations are those of the DS4.1 verify/decode MoE layer described on
 * lucebox PR #826 "feat(ds41): two-box expert-parallel serving":
 *   - the commit on fused DS4.1 decode kernels: the router's select and weights
 *     over the same logits in one launch, one expert grouping per MoE layer for
 *     gate, up and down, a q8_1 activation memo, and column-range Q8_0 products
 *     that keep the whole row's lane mapping;
 *   - the commit adding the RDNA4 Q8_0 gate/up pair: both Q8_0 products read one
 *     load of each activation fragment, keep the single product's partials and
 *     reduction, and write SwiGLU-DS4 of the two in the epilogue; batch
 *     invariant from 1 to 8 columns (the single-token gate/up pair commit);
 *   - the commit on the fused routed combine: owner route mask, route weighting
 *     and route sum in one launch, products and sums rounded separately;
 *     clamped routed SwiGLU;
 *   - the review finding on moe_combine_masked_kernel: a route masked to -1 is
 *     skipped: nothing it indexes is read, and its slot's value (unwritten,
 *     possibly NaN) never enters the sum.
 *
 * Formats (the pages name them and print no layout; this is the layout used):
 *   Q8_0 block, 34 bytes: fp16 d (little-endian), int8 qs[32]; value = d * q.
 *   q8_1 block, 36 bytes: fp16 d, fp16 s = d * sum(q), int8 qs[32].
 *   A row of K values is K/32 consecutive blocks.  Quantisation: fp32
 *   d = amax/127, q = roundf(x/d) (halves away from zero) on the fp32 quotient,
 *   d and s stored as fp16 (round to nearest even); an all-zero block is all
 *   zero bytes.
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     allocates nothing, keeps no mutable global state and never writes an
 *     input.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it and returns without synchronising.
 *   - Return value: MOEQ8_OK when the work was enqueued; a negative status when
 *     the arguments were rejected on the host (nothing enqueued, outputs
 *     untouched) or the launch failed (MOEQ8_EHIP; the HIP error is cleared).
 *     Faults inside kernels surface at the caller's next synchronisation.
 *   - Non-finite inputs are outside the contract (results unspecified).
 *   - Columns: 1 <= ncols <= MOEQ8_MAX_COLS (MOEQ8_MAX_WIDE_COLS for the wide
 *     calls and for grouped products and combines that take their
 *     groupings).  Column j of an activation operand is row j of a row-major
 *     [ncols][...] array.
 *   - K must be a multiple of 64 (whole 2-block lane chunks); weight pointers,
 *     row strides and expert strides must be multiples of 4 bytes; activation
 *     and output pointers must be 4-byte aligned.
 */
#ifndef MOEQ8_H
#define MOEQ8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOEQ8_ABI_VERSION 1
#define MOEQ8_QK 32
#define MOEQ8_Q8_0_BLOCK_BYTES 34
#define MOEQ8_Q8_1_BLOCK_BYTES 36
#define MOEQ8_MAX_COLS 8
#define MOEQ8_MAX_EXPERTS 1024
#define MOEQ8_MAX_TOPK 16
#define MOEQ8_MAX_WIDE_COLS 1024   /* columns of the wide-batch calls */
#define MOEQ8_MAX_EXCHANGE_RANKS 64  /* ranks one exchange sum takes */
#define MOEQ8_EXCHANGE_BLOCK_BYTES 36
#define MOEQ8_Q4_BLOCK_BYTES 18

enum moeq8_status {
    MOEQ8_OK = 0,
    MOEQ8_EINVAL = -1,       /* null pointer, bad shape, K % 64, ncols out of range, topk > n_expert */
    MOEQ8_EALIGN = -2,       /* pointer, stride or k_block_offset alignment */
    MOEQ8_EUNSUPPORTED = -3, /* valid request the library does not implement (e.g. n_expert > 1024) */
    MOEQ8_EHIP = -4          /* the HIP launch failed; the error was cleared */
};

/* Human-readable name of a status code (static string, never NULL). */
const char* moeq8_status_string(int status);

/* MOEQ8_ABI_VERSION of the built library. */
int moeq8_abi_version(void);

/* ---------------------------------------------------------------------------
 * a1 / a7: q8_1 activation quantisation (the q8_1 rows MMVQ reads; quantise an
 * activation once and share the rows, the activation memo of the fused decode
 * kernels commit).
 *   x     fp32 [n_rows][x_row_stride] (elements); the first k of each row are read
 *   xq    q8_1 blocks [n_rows][k/32], contiguous (n_rows * k/32 * 36 bytes)
 * k must be a multiple of 32 here.  n_rows == 0 enqueues nothing and is OK.
 * ------------------------------------------------------------------------- */
int q8_1_quantize_rows(const float* x, int64_t n_rows, int64_t k, int64_t x_row_stride,
                       void* xq, void* stream);

/* Q8_0 weight quantisation with the same block rule (no s field):
 *   w     fp32 [n_rows][w_row_stride]
 *   wq    Q8_0 blocks [n_rows][k/32], contiguous (34 bytes each) */
int q8_0_quantize_rows(const float* w, int64_t n_rows, int64_t k, int64_t w_row_stride,
                       void* wq, void* stream);

/* Repack Q8_0 rows into the 64-chunk packed layout read by
 * MOEQ8_GATE_UP_SWIGLU_P64.  A row of k values (k a multiple of 4096) is k/4096
 * segments of 64 two-block chunks (4352 bytes, 1088 dwords); within a segment
 * dword d < 16 of chunk c (plain dword 17c + d) moves to dword
 * 256*(d/4) + 4c + d%4 and dword 16 of chunk c to dword 1024 + c.  Same bytes,
 * permuted within each segment, so a wave whose lane c reads chunk c fetches
 * each 16-byte piece of its chunks with one contiguous load across the wave.
 *   src  Q8_0 rows [n_rows], src_row_stride_bytes apart
 *   dst  packed rows [n_rows], dst_row_stride_bytes apart; must not overlap src
 * Strides >= k/32*34 bytes, pointers and strides multiples of 4 bytes. */
int q8_0_pack64_rows(const void* src, int64_t n_rows, int64_t k, int64_t src_row_stride_bytes,
                     void* dst, int64_t dst_row_stride_bytes, void* stream);

/* The round-major four-row packed layout read by MOEQ8_DOWN_F32_ACT_P64: round
 * r (values [1024 r, 1024 r + 1024), 1088 bytes) of every row goes to the
 * matrix dst + r * n_rows * 1088, whose rows are contiguous; there each quad of
 * rows 4q .. 4q+3 (4352 bytes) is permuted as one q8_0_pack64_rows segment,
 * chunk 16g + l of the segment being chunk l of row 4q + g.  A column-range
 * slice at a multiple of 32 blocks is then the matrix of its round.  n_rows a
 * multiple of 4, k a multiple of 1024; dst holds n_rows * k/32 * 34 bytes and
 * must not overlap src.  Otherwise as q8_0_pack64_rows. */
int q8_0_pack64_rounds(const void* src, int64_t n_rows, int64_t k, int64_t src_row_stride_bytes, void* dst,
                       void* stream);

/* Repack Q8_0 rows into the layout MOEQ8_GATE_UP_SWIGLU_G8 and MOEQ8_DOWN_G8 of
 * moe_grouped_gemm read.  Each 272-byte group of 8 blocks (a row of k values
 * is k/256 groups, k a multiple of 256) holds the 8 blocks' fp16 scales in its
 * first 16 bytes (block j at byte 2j) and then their quants, block j's 32
 * bytes at 16 + 32j, so the matrix cores' 8-byte operand pieces are 8-byte
 * aligned; in rows i with i % 16 >= 8 (i counted from the call's first row)
 * the two 8-byte halves of every 16-byte quant piece are swapped, so the 16
 * rows one wave reads fall into different LDS banks.  The same bytes, permuted
 * within each group.  Pack whole expert matrices from their first row (their
 * row counts multiples of 32).
 *   src  Q8_0 rows [n_rows], src_row_stride_bytes apart
 *   dst  packed rows [n_rows], dst_row_stride_bytes apart; must not overlap src
 * Strides >= k/32*34 bytes, pointers and strides multiples of 4 bytes. */
int q8_0_pack_gemm_rows(const void* src, int64_t n_rows, int64_t k, int64_t src_row_stride_bytes,
                        void* dst, int64_t dst_row_stride_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * a3 (+a10): single Q8_0 x q8_1 product, y[c][i] = sum over the k/32 blocks b of
 * row i of d_w * d_x * sum(qw * qx).
 *   w                  Q8_0 rows: row i starts at w + i * w_row_stride_bytes.  For a
 *                      column-range slice this is a view: w points at block
 *                      k_block_offset of row 0 and w_row_stride_bytes is the full
 *                      row's stride.
 *   n, k               rows and (slice) length in values; k % 64 == 0
 *   k_block_offset     index within the full row of the slice's first block; must
 *                      be even.  The result is bit-identical to the full-row
 *                      product with activations zero outside the slice (the
 *                      whole-row lane mapping of the column-range commit).
 *   xq                 q8_1 [ncols][k/32]
 *   y                  fp32 [ncols][n]
 * Batch invariant: column j's bits do not depend on ncols.
 * ------------------------------------------------------------------------- */
int mmvq_q8_0(const void* w, int64_t w_row_stride_bytes, int64_t n, int64_t k,
              int64_t k_block_offset, const void* xq, int64_t ncols, float* y, void* stream);

/* ---------------------------------------------------------------------------
 * a2 (+a10): Q8_0 gate/up pair on the same q8_1 activations with the SwiGLU-DS4
 * epilogue h = silu(min(g, 7)) * clamp(u, -7, 7) (the RDNA4 Q8_0 gate/up pair
 * commit; fp32 epilogue).
 *   w_gate, w_up       two Q8_0 matrices with the same geometry (as mmvq_q8_0)
 *   h_out              fp32 [ncols][n]
 *   g_out, u_out       optional (NULL = not written): the raw products, fp32 [ncols][n]
 * g_out/u_out are bit-identical to mmvq_q8_0 on each matrix, and h_out is
 * bit-identical to swiglu_ds4 of them.
 * ------------------------------------------------------------------------- */
int mmvq_q8_0_glu_pair(const void* w_gate, const void* w_up, int64_t w_row_stride_bytes,
                       int64_t n, int64_t k, int64_t k_block_offset, const void* xq,
                       int64_t ncols, float* h_out, float* g_out, float* u_out, void* stream);

/* Elementwise SwiGLU-DS4 (the GLU kernel of the unfused path):
 *   h[i] = silu(min(g[i], 7)) * clamp(u[i], -7, 7), fp32, count elements. */
int swiglu_ds4(const float* g, const float* u, int64_t count, float* h, void* stream);

/* ---------------------------------------------------------------------------
 * a4 + a5: router top-k select and weights over the same logits, owner mask,
 * and the layer's expert grouping (one launch; the grouping stays on the device).
 *   logits       fp32 [ncols][n_expert]
 *   bias         fp32 [n_expert] expert-selection bias, or NULL (zero)
 *   owner_slot   int32 [n_expert]: local expert index in [0, n_local_expert), or -1
 *                for an expert owned elsewhere; NULL = every expert local with
 *                slot = expert index (then n_local_expert must equal n_expert).
 *                Entries outside [-1, n_local_expert) are treated as -1.
 *   ids          int32 [ncols][topk] out: local expert of each route, -1 = masked
 *   weights      fp32 [ncols][topk] out
 *   grouping     device buffer of moe_grouping_bytes(ncols, topk) bytes, out
 * Scores: score = sigmoid(logit), the fp64 sigmoid rounded once to fp32;
 * key = score + bias (fp32).  Slots 0..topk-1 hold the experts with the largest
 * keys, by (key descending, expert index ascending).  weights = score / (sum of
 * the topk selected scores, summed in slot order in fp32); the bias selects only;
 * masked routes keep their weight and count in the sum.
 * Grouping layout (int32 words): [0] n_active, [1] n_valid routes, [2] ncols,
 * [3] topk, then expert[R], offset[R+1], route[R] with R = ncols*topk: active
 * groups a < n_active hold local expert expert[a] (ascending) and the routes
 * route[offset[a] .. offset[a+1]) (route r = column*topk + slot, ascending).
 * Eight words of padding follow route[]: the grouped MMVQ reads eight words
 * from any route entry at once (the padding's contents are never used).  Then,
 * from word T = (4 + 3R + 1 + 8) rounded up to a multiple of 4, a table of 4
 * words per active group: {expert[a], offset[a], offset[a+1], 0}, which the
 * grouped MMVQ reads as one 16-byte record per work item.
 * ------------------------------------------------------------------------- */
size_t moe_grouping_bytes(int64_t ncols, int32_t topk);
int moe_route_topk(const float* logits, const float* bias, const int32_t* owner_slot,
                   int64_t ncols, int64_t n_expert, int64_t n_local_expert, int32_t topk,
                   int32_t* ids, float* weights, void* grouping, void* stream);

/* a4's score function alone (the scores the router of PR #826's fused DS4.1
 * decode kernels commit selects and weights by): scores[i] = the router's score
 * of logits[i] (the sigmoid evaluated in fp64 and rounded once to fp32), by the same
 * device expression the router uses, for n >= 0 fp32 values (device pointers,
 * 4-byte aligned; n = 0 enqueues nothing).  For checking that rounding against
 * a reference over any set of logits; the selection itself is moe_route_topk.
 * Returns MOEQ8_EINVAL for a null pointer or n < 0, MOEQ8_EALIGN for a
 * misaligned pointer. */
int moe_router_scores(const float* logits, int64_t n, float* scores, void* stream);

/* ---------------------------------------------------------------------------
 * a6 / a8: grouped per-expert MMVQ over the routed experts, one launch per
 * projection, using the grouping written by moe_route_topk.
 *   stage MOEQ8_GATE_UP_SWIGLU: w_a = gate, w_b = up, act_q = xq [ncols][k/32],
 *         out = h fp32 [ncols][topk][n] = SwiGLU-DS4(gate.x_j, up.x_j) for route (j, s)
 *   stage MOEQ8_DOWN: w_a = down, w_b = NULL, act_q = hq [ncols*topk][k/32] (one q8_1
 *         row per route), out = y fp32 [ncols][topk][n]
 *   Expert e's matrix starts at w + e * expert_stride_bytes; its rows are
 *   w_row_stride_bytes apart; experts outside [0, n_local_expert) are skipped.
 * `grouping` must come from moe_route_topk with the same ncols and topk (a
 * grouping whose header names another column count or top-k is ignored and
 * nothing is written).
 * Rows of masked routes (id -1) are NOT written.  Each route's row is
 * bit-identical to mmvq_q8_0 (DOWN) or mmvq_q8_0_glu_pair's h (GATE_UP) on that
 * expert and that route's activation row.
 * ------------------------------------------------------------------------- */
enum moeq8_stage { MOEQ8_GATE_UP_SWIGLU = 0, MOEQ8_DOWN = 1, MOEQ8_DOWN_F32_ACT = 2,
                   MOEQ8_GATE_UP_SWIGLU_P64 = 3, MOEQ8_DOWN_F32_ACT_P64 = 4,
                   MOEQ8_GATE_UP_SWIGLU_G8 = 5, MOEQ8_DOWN_G8 = 6 /* moe_grouped_gemm only */ };
int moe_grouped_mmvq(int32_t stage, const void* w_a, const void* w_b,
                     int64_t expert_stride_bytes, int64_t w_row_stride_bytes,
                     int64_t n_local_expert, int64_t n, int64_t k, const void* act_q,
                     const void* grouping, int64_t ncols, int32_t topk, float* out,
                     void* stream);

/* ---------------------------------------------------------------------------
 * a6 / a8 fused with their neighbours: the grouped launch above, plus
 *   - stage MOEQ8_DOWN_F32_ACT: act is fp32 h rows [ncols*topk][act_row_stride
 *     elements] (first k of each row read) and each workgroup quantises the rows
 *     of its routes to q8_1 in LDS with the block rule of q8_1_quantize_rows (the
 *     bytes, hence the products, equal q8_1_quantize_rows then MOEQ8_DOWN);
 *   - an optional dense part (s_a != NULL), run as extra work items of the same
 *     launch: rows [0, s_n) of the matrix s_a (and s_b for the gate/up stage)
 *     against all ncols columns, a column-range slice starting at block
 *     s_k_block_offset of rows s_row_stride_bytes apart (the shared expert's share
 *     of the pages' expert-parallel split); s_k is the slice length in values and
 *     must equal k.  q8_1 stages: s_act = q8_1 rows [ncols][k/32] of the dense
 *     part, or NULL for act rows 0..ncols-1 (the gate/up stage's shared x);
 *     s_out = SwiGLU-DS4 (gate/up) or the product (down), [ncols][s_n].  Down with
 *     fp32 activations: s_act = fp32 rows [ncols][s_act_row_stride].
 *     Each s_out element is bit-identical to mmvq_q8_0_glu_pair / mmvq_q8_0 on
 *     that slice.  A dense part whose s_k differs from k, or whose slice spans a
 *     different number of 16-chunk rounds, is MOEQ8_EUNSUPPORTED (call it apart).
 *   - stage MOEQ8_GATE_UP_SWIGLU_P64: the gate/up stage on weights repacked by
 *     q8_0_pack64_rows (the routed experts and the dense part alike).  Each
 *     lane's chunk arrives through four 16-byte and one 4-byte loads that
 *     read one contiguous span across the wave: nontemporal when ncols <= 8
 *     (each row is read once), ordinary for wider groupings, where an expert
 *     with more than 8 routes passes over its rows again.  Requires
 *     k == 4096 (one packed segment a row; a dense slice starting at a
 *     multiple of 128 blocks) else MOEQ8_EUNSUPPORTED, and 16-byte aligned
 *     weight pointers, row strides and expert stride else MOEQ8_EALIGN.
 *     Every output is bit-identical to MOEQ8_GATE_UP_SWIGLU on the unpacked
 *     weights.
 *   - stage MOEQ8_DOWN_F32_ACT_P64: MOEQ8_DOWN_F32_ACT on weights repacked by
 *     q8_0_pack64_rounds (the routed experts and the dense part alike): k must
 *     be 1024 with rows of 1088 bytes (w_row_stride_bytes and
 *     s_row_stride_bytes 1088), n and s_n multiples of 4, else
 *     MOEQ8_EUNSUPPORTED; 16-byte aligned pointers and expert stride else
 *     MOEQ8_EALIGN.  The dense part is the round's matrix (s_a at round r of
 *     the packed shared matrix, s_k_block_offset 0): its products equal those
 *     of the column-range slice at block 32 r of the plain matrix, since a
 *     one-round slice's lane sums do not depend on its round.  Loads as for
 *     MOEQ8_GATE_UP_SWIGLU_P64.  Every output is bit-identical to
 *     MOEQ8_DOWN_F32_ACT on the unpacked weights.
 * act_row_stride is ignored for the q8_1 stages.
 * ------------------------------------------------------------------------- */
int moe_grouped_mmvq_ex(int32_t stage, const void* w_a, const void* w_b,
                        int64_t expert_stride_bytes, int64_t w_row_stride_bytes,
                        int64_t n_local_expert, int64_t n, int64_t k, const void* act,
                        int64_t act_row_stride, const void* grouping, int64_t ncols, int32_t topk,
                        float* out, const void* s_a, const void* s_b, int64_t s_row_stride_bytes,
                        int64_t s_n, int64_t s_k, int64_t s_k_block_offset, const void* s_act,
                        int64_t s_act_row_stride, float* s_out, void* stream);

/* ---------------------------------------------------------------------------
 * a6 + a7 + a8, the routed FFN product after routing, in one call: the grouped
 * gate/up + SwiGLU-DS4 of MOEQ8_GATE_UP_SWIGLU_P64 writing h, then the grouped
 * down of MOEQ8_DOWN_F32_ACT_P64 quantising h to q8_1 in its launch, with the
 * shared expert's share as extra work items of both (two launches on
 * `stream`; the pages' fused decode kernels commit runs one expert grouping
 * for gate, up and down).
 *   w_gate, w_up   routed experts' gate and up, packed by q8_0_pack64_rows,
 *                  [n_local_expert][inter][hidden/32 blocks] (rows hidden/32*34
 *                  bytes apart), experts gate_up_expert_stride_bytes apart
 *   w_down         routed experts' down, packed by q8_0_pack64_rounds,
 *                  [n_local_expert][hidden] rows of 1088 bytes, experts
 *                  down_expert_stride_bytes apart
 *   hidden == 4096, inter == 1024 (the packed layouts' shapes), else
 *   MOEQ8_EUNSUPPORTED; 1 <= ncols <= MOEQ8_MAX_COLS
 *   xq             q8_1 rows of x [ncols][hidden/32]
 *   grouping       from moe_route_topk / moe_route_topk_quantize for ncols, topk
 *   h              fp32 [ncols*topk][inter] workspace: SwiGLU-DS4 of each route
 *                  (written by the first launch, read by the second; masked
 *                  routes' rows not written)
 *   y              fp32 [ncols][topk][hidden] out (masked routes' rows not
 *                  written)
 *   shared share (s_gate == NULL: none): s_gate, s_up rows [0, s_rows) of the
 *                  packed shared gate/up, s_row_stride_bytes apart; s_down the
 *                  packed shared down's round matrix of this share ([hidden]
 *                  rows of 1088 bytes); s_rows == inter; hs fp32 [ncols][s_rows]
 *                  workspace and ys fp32 [ncols][hidden] out, as in
 *                  moe_grouped_mmvq_ex
 * Both stages are checked before either is launched.  Every output is
 * bit-identical to moe_grouped_mmvq_ex with MOEQ8_GATE_UP_SWIGLU_P64 and then
 * MOEQ8_DOWN_F32_ACT_P64 on the same arguments.
 * ------------------------------------------------------------------------- */
int moe_grouped_ffn_p64(const void* w_gate, const void* w_up, const void* w_down,
                        int64_t gate_up_expert_stride_bytes, int64_t down_expert_stride_bytes,
                        int64_t n_local_expert, int64_t hidden, int64_t inter, const void* xq,
                        const void* grouping, int64_t ncols, int32_t topk, float* h, float* y,
                        const void* s_gate, const void* s_up, int64_t s_row_stride_bytes,
                        int64_t s_rows, const void* s_down, float* hs, float* ys, void* stream);

/* moe_grouped_ffn_p64 for callers that cannot allocate device memory (code
 * under graph capture, tight serving loops, harnesses that forbid it): the
 * same product and the same bits, with h and hs held in
 * MOEQ8_FFN_SCRATCH_BYTES of device memory the library keeps on each GPU it
 * runs on, from its first call there until the process ends.  The call
 * itself allocates nothing.  Arguments as moe_grouped_ffn_p64 without h and
 * hs; `stream` must belong to the current device.  Sizes beyond that memory
 * (ncols * topk * inter * 4 > 524288 bytes, or ncols * s_rows * 4 > 32768)
 * are MOEQ8_EUNSUPPORTED, nothing enqueued.  Every call on one GPU uses the
 * same memory, and each leaves its h there: calls that overlap on one GPU
 * (other streams, other host threads) race and must not be made. */
#define MOEQ8_FFN_SCRATCH_BYTES 557056
int moe_grouped_ffn_p64_noalloc(const void* w_gate, const void* w_up, const void* w_down,
                                int64_t gate_up_expert_stride_bytes, int64_t down_expert_stride_bytes,
                                int64_t n_local_expert, int64_t hidden, int64_t inter, const void* xq,
                                const void* grouping, int64_t ncols, int32_t topk, float* y,
                                const void* s_gate, const void* s_up, int64_t s_row_stride_bytes,
                                int64_t s_rows, const void* s_down, float* ys, void* stream);

/* a1 + a4 + a5 in one launch (the layer prologue): q8_1 quantisation of the
 * ncols rows of x [ncols][x_row_stride] into xq [ncols][k/32], and
 * moe_route_topk on the logits.  Outputs are bit-identical to calling
 * q8_1_quantize_rows and moe_route_topk. */
int moe_route_topk_quantize(const float* x, int64_t x_row_stride, int64_t k, void* xq,
                            const float* logits, const float* bias, const int32_t* owner_slot,
                            int64_t ncols, int64_t n_expert, int64_t n_local_expert, int32_t topk,
                            int32_t* ids, float* weights, void* grouping, void* stream);

/* ---------------------------------------------------------------------------
 * Wide batches (prefill-like, up to MOEQ8_MAX_WIDE_COLS columns).
 *
 * moe_route_topk_wide: the selection and weights of moe_route_topk for each
 * column (columns are independent; one workgroup per 8 columns), without the
 * grouping.  Arguments and results as moe_route_topk.
 *
 * moe_group_routes: the expert grouping of ids [ncols][topk] in the layout
 * moe_route_topk writes (header, expert[], offset[], route[], padding, table),
 * in a buffer of moe_grouping_bytes_wide(ncols, topk) bytes: active local
 * experts ascending, each with its routes ascending.  ids outside
 * [0, n_local_expert) count as masked.
 *
 * moe_grouped_mmvq / moe_grouped_mmvq_ex and moe_combine accept such wide
 * groupings (ncols up to MOEQ8_MAX_WIDE_COLS): a work item takes its expert's
 * routes in passes of MOEQ8_MAX_COLS columns.  moe_grouped_gemm takes the
 * same groupings.
 * ------------------------------------------------------------------------- */
size_t moe_grouping_bytes_wide(int64_t ncols, int32_t topk);
/* moe_grouped_gemm: the grouped products of moe_grouped_mmvq (same stages
 * MOEQ8_GATE_UP_SWIGLU and MOEQ8_DOWN, same arguments, layouts and results)
 * computed on the int8 matrix cores, for wide batches where an expert serves
 * many routes.  The pages run large expert batches on a matrix-core GEMM
 * (PR #826 description, Results: the WMMA routed-expert GEMM; the fused
 * DS4.1 decode kernels commit: MMQ for wide Q4_K products); here the formats
 * and the grouping stay those of the decode path.
 *   Per output: blocks in ascending order, acc = fma(float(sumi_b),
 *   d_w,b * d_x,b, acc) from +0 (sumi_b the block's exact integer dot,
 *   d_w * d_x exact in fp32), then SwiGLU-DS4 for gate/up.  The result equals
 *   the oracle's product to rounding; it is NOT bit-identical to
 *   moe_grouped_mmvq, whose reduction order differs.
 *   Requires n % 32 == 0 and k % 64 == 0 (MOEQ8_EINVAL otherwise).  Rows of
 *   masked routes are not written.  Work is split into (expert, route
 *   chunk, row tile) units, so an expert with many routes spreads over many
 *   workgroups.
 *   stages MOEQ8_GATE_UP_SWIGLU_G8 / MOEQ8_DOWN_G8: the gate/up and down
 *   stages on weights repacked by q8_0_pack_gemm_rows, with the same results
 *   bit for bit while the weight scales are finite (an infinite or NaN fp16
 *   weight scale makes the gate/up outputs of its row NaN where the plain
 *   rows may give an infinity).  They always take the staged form below, so they require
 *   k % 256 == 0, n % 32 == 0 (gate/up) or n % 64 == 0 (down), 16-byte
 *   aligned weights, activations, row and expert strides and activation
 *   rows, else MOEQ8_EUNSUPPORTED.
 *   Concurrency: when k is a multiple of 256 (gate/up; down from k = 1024)
 *   and the operands are 16-byte aligned, the workgroups take their units
 *   from one of 256 work counters of the library on the device, handed to
 *   the calls in turn and left at zero when a call ends: at most 256 calls
 *   may be in flight on one device at once, and a captured graph keeps its
 *   counters, so one graph must not be replayed on two streams at once. */
int moe_grouped_gemm(int32_t stage, const void* w_a, const void* w_b,
                     int64_t expert_stride_bytes, int64_t w_row_stride_bytes,
                     int64_t n_local_expert, int64_t n, int64_t k, const void* act_q,
                     const void* grouping, int64_t ncols, int32_t topk, float* out,
                     void* stream);

int moe_route_topk_wide(const float* logits, const float* bias, const int32_t* owner_slot,
                        int64_t ncols, int64_t n_expert, int64_t n_local_expert, int32_t topk,
                        int32_t* ids, float* weights, void* stream);
int moe_group_routes(const int32_t* ids, int64_t ncols, int32_t topk, int64_t n_local_expert,
                     void* grouping, void* stream);

/* ---------------------------------------------------------------------------
 * a9: weighted masked combine.
 *   out[j][i] = sum over slots s ascending with ids[j][s] >= 0 of
 *               fl(weights[j][s] * y[j][s][i])  (fp32: each product rounded, then
 *               added in slot order; a masked slot's y row is loaded with the
 *               others, all in bounds, and its value, NaN included, is
 *               selected away, never added)
 *   y fp32 [ncols][topk][n] (every row allocated; masked rows may hold
 *   anything); ids int32 [ncols][topk]; weights fp32 [ncols][topk];
 *   out fp32 [ncols][n] (fully overwritten; all-masked columns give 0).
 * ------------------------------------------------------------------------- */
int moe_combine(const float* y, const int32_t* ids, const float* weights, int64_t ncols,
                int32_t topk, int64_t n, float* out, void* stream);

/* The combine with the shared expert's output added (the MoE block's whole
 * output; the routed-combine commit joins the shared-expert slice with the
 * routed partials):
 *   out[j][i] = moe_combine's out[j][i] + shared_y[j][i]
 * one fp32 add after the routed slot sum.  shared_y fp32 [ncols][n], not NULL;
 * it may be the same buffer as out.  Otherwise as moe_combine. */
int moe_combine_shared(const float* y, const int32_t* ids, const float* weights, int64_t ncols,
                       int32_t topk, int64_t n, const float* shared_y, float* out, void* stream);

/* ---------------------------------------------------------------------------
 * 8-bit block exchange codec for prefill-sized partials (PR #826, the 8-bit
 * prefill exchange commit: a partial is carried as 32-value int8 blocks with
 * an f32 scale each, 1.125 bytes a value; after the gather, the decode adds
 * the per-rank fp32 products in ascending rank order from +0, so every rank
 * computes identical bits).  The gather crosses devices and is not part of
 * this library.
 *
 * Block: {f32 d; int8 qs[32]}, MOEQ8_EXCHANGE_BLOCK_BYTES = 36 bytes.
 *
 * q8_block_encode: x fp32 [rows][n] (row stride x_stride elements >= n,
 *   n % 32 == 0) -> blocks [rows][n/32], contiguous, written in full.
 *   d = amax / 127 in fp32 (IEEE division, kept in fp32), q = roundf(x / d) on
 *   the fp32 quotient (halves away from zero); an all-zero block gives d = 0
 *   and q = 0.  x and blocks 4-byte aligned (16-byte aligned x with
 *   x_stride % 4 == 0 takes the vector path; results are the same).
 *
 * q8_block_decode_sum: gathered holds nranks block arrays [rows][n/32], rank r
 *   at gathered + r * rank_stride_bytes (>= rows * n/32 * 36, multiple of 4;
 *   ignored when nranks == 1); 1 <= nranks <= MOEQ8_MAX_EXCHANGE_RANKS.
 *   out fp32 [rows][n] (row stride out_stride >= n) is overwritten with
 *     out = (((+0 + v_0) + v_1) + ... + v_{nranks-1}),  v_r = fl(d_r * q_r)
 *   in fp32: each product rounded once, sums in ascending rank order.
 *
 * Both: rows == 0 enqueues nothing; errors are returned before any launch.
 * ------------------------------------------------------------------------- */
int q8_block_encode(const float* x, int64_t rows, int64_t n, int64_t x_stride, void* blocks,
                    void* stream);
int q8_block_decode_sum(const void* gathered, int32_t nranks, int64_t rank_stride_bytes,
                        int64_t rows, int64_t n, float* out, int64_t out_stride, void* stream);

/* ---------------------------------------------------------------------------
 * Bandwidth-only 4-bit expert weights.  The pages stream cold experts in a
 * 2-bit format they do not define, through the prefetching loop of the grouped
 * MoE MMVQ commit; a plainly defined 4-bit block stands in here:
 *   Q4 block = {fp16 d; uint8 qs[16]}, MOEQ8_Q4_BLOCK_BYTES = 18 (4.5 bits a
 *   weight); value i < 16 is the low nibble of qs[i], value i + 16 the high
 *   nibble; w = d * (code - 8).
 * q4_quantize_rows: w fp32 [n_rows][k] -> Q4 blocks [n_rows][k/32]: fp32
 *   d = amax / 7 (IEEE division), code = clamp(roundf(w / d), -8, 7) + 8 on the
 *   fp32 quotient, d stored fp16 (nearest even); an all-zero block gives d = 0
 *   and codes 8.  w 4-byte aligned, wq 2-byte aligned.
 * mmvq_q4, mmvq_q4_glu_pair, moe_grouped_mmvq_q4: the products of mmvq_q8_0,
 *   mmvq_q8_0_glu_pair and moe_grouped_mmvq_ex (no shared part; stages
 *   MOEQ8_GATE_UP_SWIGLU, MOEQ8_DOWN, MOEQ8_DOWN_F32_ACT, and the packed
 *   MOEQ8_GATE_UP_SWIGLU_P64 / MOEQ8_DOWN_F32_ACT_P64 on weights repacked by
 *   q4_pack64_rows, with the shapes those stages take) with Q4 weights, on
 *   q8_1 activations; the same arguments, with row strides of at least
 *   k/32 * 18 bytes (a multiple of 4).  A block contributes
 *   (d_w * d_x) * sum((code - 8) * q), with the same reduction order as the
 *   Q8_0 products, so the same invariants hold (batch invariance at 1..8
 *   columns, pair == separate products + SwiGLU, grouped == per-route
 *   products, column-range slices == zero-padded full rows).
 * ------------------------------------------------------------------------- */
int q4_quantize_rows(const float* w, int64_t n_rows, int64_t k, int64_t w_row_stride, void* wq,
                     void* stream);
int mmvq_q4(const void* w, int64_t w_row_stride_bytes, int64_t n, int64_t k, int64_t k_block_offset,
            const void* xq, int64_t ncols, float* y, void* stream);
int mmvq_q4_glu_pair(const void* w_gate, const void* w_up, int64_t w_row_stride_bytes, int64_t n,
                     int64_t k, int64_t k_block_offset, const void* xq, int64_t ncols, float* h_out,
                     float* g_out, float* u_out, void* stream);
int moe_grouped_mmvq_q4(int32_t stage, const void* w_a, const void* w_b,
                        int64_t expert_stride_bytes, int64_t w_row_stride_bytes,
                        int64_t n_local_expert, int64_t n, int64_t k, const void* act,
                        int64_t act_row_stride, const void* grouping, int64_t ncols, int32_t topk,
                        float* out, void* stream);

/* Repack Q4 rows into the 64-chunk packed layout the packed 4-bit stages
 * read (the same bytes, permuted within each segment).  A row of k values (k a
 * multiple of 4096) is k/4096 segments of 64 two-block chunks (2304 bytes, 576
 * dwords); within a segment dword d < 8 of chunk c (plain dword 9c + d) moves to
 * dword 256*(d/4) + 4c + d%4 and dword 8 of chunk c to dword 512 + c.  For
 * MOEQ8_DOWN_F32_ACT_P64 (k = 1024, rows 576 bytes apart) pass each quad of
 * four consecutive rows as one row of 4096 values (n_rows / 4 rows, 2304
 * bytes apart).
 *   src  Q4 rows [n_rows], src_row_stride_bytes apart
 *   dst  packed rows [n_rows], dst_row_stride_bytes apart; must not overlap src
 * Strides >= k/32*18 bytes, pointers and strides multiples of 4 bytes. */
int q4_pack64_rows(const void* src, int64_t n_rows, int64_t k, int64_t src_row_stride_bytes,
                   void* dst, int64_t dst_row_stride_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOEQ8_H */
