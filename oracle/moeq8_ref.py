"""Plain CPU oracle for the quantized MoE expert FFN (Q8_0 weights, q8_1 activations).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or run
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and imports nothing from it.

Sources (the pages):
  * lucebox PR #826 "feat(ds41): two-box expert-parallel serving" -- the
    commit on fused DS4.1 decode kernels (one router launch for select and
    weights, one expert grouping per layer, q8_1 activation memo, whole-row-lane
    column-range Q8_0 products), the commit on the fused routed combine (owner
    mask + weighting + route sum, products and sums rounded separately, clamped
    routed SwiGLU), the commit adding the RDNA4 Q8_0 gate/up pair with the
    SwiGLU-DS4 epilogue, and the review finding on masked (-1) route ids in
    moe_combine_masked_kernel.
  * llama.cpp compare page, convert_hf_to_gguf.py Sarvam-MoE hunk: expert bias
    normalised to zero mean at load time.

The pages name the formats and operations but print no byte layout, scale rule,
clamp constant or routing rule.  Readings taken here:
  R1  Q8_0 block = {fp16 d; int8 qs[32]} (34 B); q8_1 block = {fp16 d; fp16 s;
      int8 qs[32]} (36 B), little-endian, array of structures.  A row of K
      values is K/32 consecutive blocks.
  R2  d = amax/127 in fp32 (IEEE division); the fp32 d quantises, the stored d
      is fp16 (round to nearest even).  q = round-half-away-from-zero of the
      fp32 quotient x/d; an all-zero block has d = 0 and q = 0.
  R3  q8_1 s = fp16(d * sum(q)) with the fp32 d and an fp32 multiply.
  R4  SwiGLU-DS4: h = silu(min(g, 7)) * clamp(u, -7, 7).
  R5  router: score = sigmoid(logit) rounded to fp32; key = score + bias (fp32
      add); top-k by (key descending, expert index ascending); weights =
      score / sum of the k selected scores (bias used for selection only).
  R6  owner mask: a route whose expert is not local is masked to id -1 but
      still counts in the normalising sum; masked slots are never read.
  R7  combine: out[j] = sum over slots s ascending with id >= 0 of w[j,s]*y[j,s].
  R8  the activations handed to a quantiser are fp32 tensors, so the SwiGLU
      output is rounded to fp32 before it is quantised for the down projection.
  R15 the MoE block's output is the routed experts' weighted sum plus the
      shared expert's output: one add after the routed sum.
  R17 8-bit exchange block (the prefill partials' wire format of PR #826's
      8-bit prefill exchange commit: 32 int8 values and one f32 scale) =
      {f32 d; int8 qs[32]} (36 B, 1.125 B a value), little-endian, array of
      structures; d and the codes follow R2's rule, but d is kept as the fp32
      quotient (the scale is f32 on the wire, so no fp16 rounding).
  R18 the exchange sum: each rank's value is the fp32 product d * q (one
      rounding); the ranks' values are added in fp32 in ascending rank order
      from +0, which makes the result the same on every rank.
  R19 a bandwidth-only low-bit weight format (the pages' cold experts use a
      2-bit format they do not define): Q4 block = {fp16 d; uint8 qs[16]}
      (18 B, 4.5 bits a weight); value i < 16 is the low nibble of qs[i],
      value i + 16 its high nibble; w = d * (code - 8).  Quantiser: fp32
      d = amax / 7 (IEEE division), code = clamp(roundf(x / d), -8, 7) + 8 on
      the fp32 quotient, d stored fp16 (nearest even); an all-zero block has
      d = 0 and every code 8.  Products with q8_1 activations are the exact
      sums over blocks of d_w * d_x * sum((code - 8) * q).
  (R9-R14 concern the launch layouts and the synthetic workloads, not what
  this module computes.)

Floating point here is fp64 unless a step is defined by fp32 rounding (the
quantisers, the router keys and the exchange codec's f32 scale and rank-order
sum), where it is done in fp32 exactly as defined.
"""

from __future__ import annotations

import numpy as np

QK = 32  # values per block
Q8_0_DTYPE = np.dtype([("d", "<f2"), ("qs", "i1", (QK,))])  # 34 bytes
Q8_1_DTYPE = np.dtype([("d", "<f2"), ("s", "<f2"), ("qs", "i1", (QK,))])  # 36 bytes
Q8X_DTYPE = np.dtype([("d", "<f4"), ("qs", "i1", (QK,))])  # 36 bytes: exchange block (R17)
Q4_DTYPE = np.dtype([("d", "<f2"), ("qs", "u1", (QK // 2,))])  # 18 bytes: 4-bit weights (R19)
assert Q8_0_DTYPE.itemsize == 34 and Q8_1_DTYPE.itemsize == 36 and Q8X_DTYPE.itemsize == 36
assert Q4_DTYPE.itemsize == 18

SWIGLU_LIMIT = 7.0


# ---------------------------------------------------------------------------
# a1 / a7 and weight preparation: block quantisation (readings R1-R3)
# ---------------------------------------------------------------------------

def _round_half_away(v32: np.ndarray) -> np.ndarray:
    """C roundf() on fp32 values: nearest integer, halves away from zero.

    Done in fp64, where |v| + 0.5 is exact for every fp32 |v| < 2**29, so no
    double rounding can turn 0.49999997f into 1.
    """
    v = v32.astype(np.float64)
    return np.sign(v) * np.floor(np.abs(v) + 0.5)


def _quantize_blocks(x: np.ndarray):
    """Shared block rule of Q8_0 and q8_1 (R2).

    x: float32 [..., nb, 32].  Returns (d fp32 [..., nb], q int32 [..., nb, 32]).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)                     # exact in fp32
    d = (amax / np.float32(127.0)).astype(np.float32)     # IEEE fp32 division
    safe_d = np.where(d == 0, np.float32(1.0), d).astype(np.float32)
    quot = (x / safe_d[..., None]).astype(np.float32)     # fp32 quotient x/d
    q = _round_half_away(quot).astype(np.int32)
    q = np.where(d[..., None] == 0, 0, q)
    return d, q


def quantize_q8_0(w: np.ndarray) -> np.ndarray:
    """Weights fp32 [rows, K] -> Q8_0 blocks [rows, K/32] (R1, R2)."""
    w = np.asarray(w, dtype=np.float32)
    rows, k = w.shape
    assert k % QK == 0
    d, q = _quantize_blocks(w.reshape(rows, k // QK, QK))
    out = np.zeros((rows, k // QK), dtype=Q8_0_DTYPE)
    out["d"] = d.astype(np.float16)
    out["qs"] = q.astype(np.int8)
    return out


def quantize_q8_1(x: np.ndarray) -> np.ndarray:
    """Activations fp32 [rows, K] -> q8_1 blocks [rows, K/32] (R1-R3).

    The q8_1 activation quantiser of the fused DS4.1 decode kernels commit and
    the "q8_1 rows its MMVQ reads" of the routed-combine commit.
    """
    x = np.asarray(x, dtype=np.float32)
    rows, k = x.shape
    assert k % QK == 0
    d, q = _quantize_blocks(x.reshape(rows, k // QK, QK))
    sumq = q.sum(axis=-1).astype(np.float32)              # exact integer, fits fp32
    s = (d * sumq).astype(np.float32)                     # fp32 multiply (R3)
    out = np.zeros((rows, k // QK), dtype=Q8_1_DTYPE)
    out["d"] = d.astype(np.float16)
    out["s"] = s.astype(np.float16)
    out["qs"] = q.astype(np.int8)
    return out


def dequantize(blocks: np.ndarray) -> np.ndarray:
    """Q8_0 or q8_1 blocks [rows, nb] -> fp64 values [rows, nb*32] (d16 * q)."""
    d = blocks["d"].astype(np.float64)
    q = blocks["qs"].astype(np.float64)
    return (d[..., None] * q).reshape(blocks.shape[0], -1)


# ---------------------------------------------------------------------------
# a2 / a3 / a6 / a8: Q8_0 x q8_1 products (MMVQ)
# ---------------------------------------------------------------------------

def block_dots(w: np.ndarray, xq: np.ndarray) -> np.ndarray:
    """Integer block dots sumi[c, n, b] = sum_i qw[n,b,i] * qx[c,b,i] (exact)."""
    qw = w["qs"].astype(np.int64)                         # [N, nb, 32]
    qx = xq["qs"].astype(np.int64)                        # [C, nb, 32]
    return np.einsum("nbi,cbi->cnb", qw, qx)


def mmvq(w: np.ndarray, xq: np.ndarray) -> np.ndarray:
    """y[c, n] = sum_b d_w[n,b] * d_x[c,b] * sumi[c,n,b], accumulated in fp64.

    Each term is exact in fp64 (fp16*fp16*int with |sumi| <= 516128), so this is
    the true product up to fp64 addition rounding.
    w: Q8_0 [N, nb]; xq: q8_1 [C, nb].  Returns fp64 [C, N].
    """
    assert w.shape[1] == xq.shape[1]
    sumi = block_dots(w, xq).astype(np.float64)
    dw = w["d"].astype(np.float64)                        # [N, nb]
    dx = xq["d"].astype(np.float64)                       # [C, nb]
    return np.einsum("nb,cb,cnb->cn", dw, dx, sumi)


def mmvq_bruteforce(w: np.ndarray, xq: np.ndarray) -> np.ndarray:
    """The same product by definition: dequantise both operands, fp64 matmul."""
    return dequantize(xq) @ dequantize(w).T


def swiglu_ds4(g, u):
    """SwiGLU-DS4 (R4), fp64: silu(min(g, 7)) * clamp(u, -7, 7).

    The clamped routed SwiGLU of the routed-combine commit and the epilogue of
    the RDNA4 Q8_0 gate/up pair commit.
    """
    g = np.minimum(np.asarray(g, dtype=np.float64), SWIGLU_LIMIT)
    u = np.clip(np.asarray(u, dtype=np.float64), -SWIGLU_LIMIT, SWIGLU_LIMIT)
    return g / (1.0 + np.exp(-g)) * u


def glu_pair(w_gate, w_up, xq):
    """Gate/up pair on the same q8_1 activations with the SwiGLU-DS4 epilogue.

    Returns (h, g, u), all fp64 [C, N].
    """
    g = mmvq(w_gate, xq)
    u = mmvq(w_up, xq)
    return swiglu_ds4(g, u), g, u


def mmvq_column_range(w_full: np.ndarray, xq_slice: np.ndarray, k_block_offset: int):
    """Column-range product: blocks [k_block_offset, k_block_offset + nb') of each
    row of ``w_full`` against activations covering just that range.

    Defined as the full-row product with the activations zero-padded outside
    the range (the whole-row-lane slice commit states the two are equal).
    """
    n, nb = w_full.shape
    c, nbs = xq_slice.shape
    padded = np.zeros((c, nb), dtype=Q8_1_DTYPE)
    padded[:, k_block_offset:k_block_offset + nbs] = xq_slice
    return mmvq(w_full, padded)


# ---------------------------------------------------------------------------
# a4 / a5: router select + weights over the same logits, owner mask, grouping
# ---------------------------------------------------------------------------

def sigmoid_f32(logits: np.ndarray) -> np.ndarray:
    """Score = sigmoid(logit) evaluated in fp64 and rounded once to fp32 (R5)."""
    z = np.asarray(logits, dtype=np.float32).astype(np.float64)
    return (1.0 / (1.0 + np.exp(-z))).astype(np.float32)


def route_topk(logits, bias, owner_slot, topk: int):
    """Top-k select and weights over the same logits (R5).

    logits fp32 [C, E]; bias fp32 [E] or None; owner_slot int [E] (local expert
    index or -1) or None for "every expert local, identity".
    Returns (ids int32 [C, topk] with -1 for masked routes, weights fp64
    [C, topk], selected global experts int32 [C, topk]).
    """
    logits = np.asarray(logits, dtype=np.float32)
    c, e = logits.shape
    assert 1 <= topk <= e
    score = sigmoid_f32(logits)
    if bias is None:
        key = score
    else:
        key = (score + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)
    sel = np.zeros((c, topk), dtype=np.int32)
    for j in range(c):
        # plain full sort by (key descending, index ascending)
        order = sorted(range(e), key=lambda i: (-float(key[j, i]), i))
        sel[j] = order[:topk]
    chosen = np.take_along_axis(score, sel, axis=1).astype(np.float64)
    weights = chosen / chosen.sum(axis=1, keepdims=True)
    if owner_slot is None:
        ids = sel.copy()
    else:
        owner = np.asarray(owner_slot, dtype=np.int32)
        ids = owner[sel].astype(np.int32)
    return ids, weights, sel


def group_routes(ids: np.ndarray):
    """One expert grouping per layer: distinct local experts in ascending order,
    each with its routes r = j*topk + s in ascending order.  Masked routes
    (id < 0) belong to no group.  Returns list of (expert, [routes])."""
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    groups = []
    for ex in sorted(set(int(v) for v in flat if v >= 0)):
        groups.append((ex, [r for r in range(flat.size) if flat[r] == ex]))
    return groups


# ---------------------------------------------------------------------------
# a9: weighted masked combine
# ---------------------------------------------------------------------------

def moe_combine(y, ids, weights, shared=None):
    """out[j, n] = sum over slots s (ascending) with ids[j,s] >= 0 of
    weights[j,s] * y[j,s,n], in fp64 (R6, R7).  Masked slots are never read, as the
    review of moe_combine_masked_kernel requires.

    shared [C, n] (optional): the shared expert's output for the same columns,
    added once after the routed sum (R15; the routed-combine commit queues the
    shared-expert slice into the same join as the routed partials)."""
    y = np.asarray(y, dtype=np.float64)
    c, k, n = y.shape
    out = np.zeros((c, n), dtype=np.float64)
    for j in range(c):
        for s in range(k):
            if ids[j, s] >= 0:
                out[j] += float(weights[j, s]) * y[j, s]
    if shared is not None:
        out = out + np.asarray(shared, dtype=np.float64)
    return out


# ---------------------------------------------------------------------------
# 4-bit weight blocks (reading R19)
# ---------------------------------------------------------------------------

def quantize_q4(w: np.ndarray) -> np.ndarray:
    """Weights fp32 [rows, K] -> Q4 blocks [rows, K/32] (R19)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, k = w.shape
    assert k % QK == 0
    x = w.reshape(rows, k // QK, QK)
    amax = np.max(np.abs(x), axis=-1)
    d = (amax / np.float32(7.0)).astype(np.float32)
    safe_d = np.where(d == 0, np.float32(1.0), d).astype(np.float32)
    quot = (x / safe_d[..., None]).astype(np.float32)
    q = np.clip(_round_half_away(quot), -8, 7).astype(np.int32)
    q = np.where(d[..., None] == 0, 0, q)
    code = (q + 8).astype(np.uint8)                       # 0..15
    out = np.zeros((rows, k // QK), dtype=Q4_DTYPE)
    out["d"] = d.astype(np.float16)
    out["qs"] = code[..., :QK // 2] | (code[..., QK // 2:] << 4)
    return out


def q4_values(blocks: np.ndarray) -> np.ndarray:
    """Q4 blocks [..., nb] -> signed codes (code - 8) int32 [..., nb, 32]."""
    qs = blocks["qs"].astype(np.int32)
    return np.concatenate([qs & 0xF, qs >> 4], axis=-1) - 8


def dequantize_q4(blocks: np.ndarray) -> np.ndarray:
    """Q4 blocks [rows, nb] -> fp64 weights [rows, nb*32]."""
    d = blocks["d"].astype(np.float64)
    return (d[..., None] * q4_values(blocks)).reshape(blocks.shape[0], -1)


def mmvq_q4(w: np.ndarray, xq: np.ndarray) -> np.ndarray:
    """y[c, n] = sum_b d_w[n,b] * d_x[c,b] * sum_i (code - 8) * q_x, in fp64
    (every term exact).  w: Q4 [N, nb]; xq: q8_1 [C, nb].  Returns fp64 [C, N]."""
    assert w.shape[1] == xq.shape[1]
    wv = q4_values(w).astype(np.int64)                    # [N, nb, 32]
    xv = xq["qs"].astype(np.int64)                        # [C, nb, 32]
    sumi = np.einsum("nbk,cbk->cnb", wv, xv).astype(np.float64)
    dw = w["d"].astype(np.float64)
    dx = xq["d"].astype(np.float64)
    return np.einsum("nb,cb,cnb->cn", dw, dx, sumi)


def glu_pair_q4(w_gate, w_up, xq):
    """Gate/up pair of Q4 matrices with the SwiGLU-DS4 epilogue: (h, g, u) fp64."""
    g = mmvq_q4(w_gate, xq)
    u = mmvq_q4(w_up, xq)
    return swiglu_ds4(g, u), g, u


# ---------------------------------------------------------------------------
# 8-bit block exchange codec (readings R17, R18)
# ---------------------------------------------------------------------------

def q8x_encode(x: np.ndarray) -> np.ndarray:
    """Prefill partials fp32 [rows, n] -> exchange blocks [rows, n/32] (R17):
    the block rule of R2 with the scale kept in fp32.  The 8-bit prefill
    exchange commit of PR #826 sends partials in this form."""
    x = np.asarray(x, dtype=np.float32)
    rows, n = x.shape
    assert n % QK == 0
    d, q = _quantize_blocks(x.reshape(rows, n // QK, QK))
    out = np.zeros((rows, n // QK), dtype=Q8X_DTYPE)
    out["d"] = d
    out["qs"] = q.astype(np.int8)
    return out


def q8x_dequantize(blocks: np.ndarray) -> np.ndarray:
    """Exchange blocks [rows, nb] -> fp32 values [rows, nb*32]: the fp32
    product d * q, rounded once (R18)."""
    d = blocks["d"].astype(np.float32)
    q = blocks["qs"].astype(np.float32)                   # exact
    return (d[..., None] * q).astype(np.float32).reshape(blocks.shape[0], -1)


def q8x_decode_sum(parts) -> np.ndarray:
    """The exchange's sum (R18): every rank's dequantized values added in fp32
    in ascending rank order from +0.  parts: the ranks' block arrays in rank
    order, each [rows, nb].  Returns fp32 [rows, nb*32]."""
    parts = list(parts)
    acc = np.zeros((parts[0].shape[0], parts[0].shape[1] * QK), dtype=np.float32)
    for blocks in parts:
        acc = (acc + q8x_dequantize(blocks)).astype(np.float32)
    return acc


# ---------------------------------------------------------------------------
# Whole paths
# ---------------------------------------------------------------------------

def expert_ffn(w_gate, w_up, w_down, xq_col):
    """One expert (or the shared expert) on one q8_1 column: gate/up pair with
    SwiGLU-DS4, h rounded to fp32 and quantised to q8_1 (R8), down product.
    Returns dict of fp64 g, u, h, the q8_1 hq and fp64 y (all for one column)."""
    h, g, u = glu_pair(w_gate, w_up, xq_col)
    hq = quantize_q8_1(h.astype(np.float32))
    y = mmvq(w_down, hq)
    return {"g": g[0], "u": u[0], "h": h[0], "hq": hq[0], "y": y[0]}


def moe_layer(x, logits, bias, owner_slot, experts, topk: int):
    """Routed MoE layer, unfused: quantise x once, route, then for every column
    j and slot s (the unfused per-route reference) run the expert FFN, then the
    weighted masked combine.

    experts(e) -> (w_gate, w_up, w_down) Q8_0 arrays of local expert e.
    Returns dict with xq, ids, weights, per-route y [C, topk, N_out] (zeros for
    masked routes) and out [C, N_out] fp64.
    """
    x = np.asarray(x, dtype=np.float32)
    c = x.shape[0]
    xq = quantize_q8_1(x)
    ids, weights, sel = route_topk(logits, bias, owner_slot, topk)
    y = None
    for j in range(c):
        for s in range(topk):
            e = int(ids[j, s])
            if e < 0:
                continue
            wg, wu, wd = experts(e)
            r = expert_ffn(wg, wu, wd, xq[j:j + 1])
            if y is None:
                y = np.zeros((c, topk, r["y"].shape[0]), dtype=np.float64)
            y[j, s] = r["y"]
    if y is None:
        n_out = experts(0)[2].shape[0]
        y = np.zeros((c, topk, n_out), dtype=np.float64)
    out = moe_combine(y, ids, weights)
    return {"xq": xq, "ids": ids, "weights": weights, "sel": sel, "y": y, "out": out}
