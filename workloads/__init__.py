"""Seeded synthetic inputs for the quantized MoE expert FFN workloads.

This module only draws inputs: fp32 activations, router logits and biases,
fp32 weights to be quantised by whichever side consumes them, and ready-made
Q8_0 weight blocks from a counter-based integer generator.  It holds none of
the method's arithmetic (no quantiser, no product, no routing) and imports
neither the library nor the oracle, so both can be fed from it.

Workloads (the pages' DS4.1 verify/decode step: 43 MoE layers, 256 routed
experts of hidden 4096 / intermediate 1024, a Q8_0 shared expert, q=4 drafts
so 5 verify columns, two-way expert split with half the shared expert per
GPU):

  pair_n512_k256          one gate/up pair, N=512, K=256, 1 column, seed 0
  shared_ffn_h4096_i2048  shared expert FFN 4096 -> 2048 -> 4096, 1..8 columns, seed 2
  routed_e256_c1          routed layer, 256 experts, top-8, 1 column, seed 3
  verify_e256_c5          routed layer, 5 columns (4 drafts + 1), seed 4
  ep_share_l43_e128_c8    one GPU's share of a two-way split: 43 layers x 128
                          local experts, routing over 256 with the other 128
                          masked, 8 columns, half of the shared expert, seed 5
  wide_e256               the routed layer at 32, 128, 512 and 1024 columns
                          (prefill-like batches), seed 6
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

QK = 32
Q8_0_BLOCK_BYTES = 34
Q8_0_DTYPE = np.dtype([("d", "<f2"), ("qs", "i1", (QK,))])

WEIGHT_SIGMA = 0.02
BIAS_SIGMA = 0.1

CONFIGS = {
    "pair_n512_k256": dict(kind="pair", n=512, k=256, cols=(1,), seed=0),
    "shared_ffn_h4096_i2048": dict(kind="shared", hidden=4096, inter=2048,
                                   cols=(1, 2, 4, 5, 8), seed=2),
    "routed_e256_c1": dict(kind="routed", experts=256, local_experts=256, layers=1,
                           hidden=4096, inter=1024, cols=(1,), topk=8, seed=3),
    "verify_e256_c5": dict(kind="routed", experts=256, local_experts=256, layers=1,
                           hidden=4096, inter=1024, cols=(5,), topk=8, seed=4),
    "ep_share_l43_e128_c8": dict(kind="routed", experts=256, local_experts=128, layers=43,
                                 hidden=4096, inter=1024, cols=(8,), topk=8, seed=5,
                                 shared_inter=2048, shared_share=2),
    # wide batches (prefill-like, many columns) on the same 256-expert layer:
    # the grouped products at 32..1024 columns, every expert typically active
    "wide_e256": dict(kind="wide", experts=256, local_experts=256, layers=1, hidden=4096,
                      inter=1024, cols=(32, 128, 512, 1024), topk=8, seed=6),
}


def expert_seed(seed: int, layer: int, expert: int) -> int:
    """Per-expert sub-seed seed*10^6 + layer*10^3 + expert."""
    return seed * 1_000_000 + layer * 1_000 + expert


def normal_f32(seed: int, shape, sigma: float = 1.0) -> np.ndarray:
    """N(0, sigma^2) fp32 values from numpy's default_rng(seed)."""
    rng = np.random.default_rng(seed)
    return rng.normal(0.0, sigma, size=shape).astype(np.float32)


def activations(seed: int, cols: int, hidden: int, layer: int = 0) -> np.ndarray:
    """FFN input x fp32 [cols, hidden] ~ N(0, 1)."""
    return normal_f32(seed * 7919 + 101 + layer * 131 + cols, (cols, hidden), 1.0)


def router_logits(seed: int, cols: int, n_expert: int, layer: int = 0) -> np.ndarray:
    """Router logits fp32 [cols, n_expert] ~ N(0, 1)."""
    return normal_f32(seed * 7919 + 202 + layer * 131 + cols, (cols, n_expert), 1.0)


def router_bias(seed: int, n_expert: int, layer: int = 0) -> np.ndarray:
    """Expert-selection bias fp32 [n_expert]: N(0, 0.1^2) drawn in fp64, made
    zero-mean in fp64 and rounded once to fp32 (the converter's load-time
    zero-mean bias normalisation applied while synthesising the input)."""
    rng = np.random.default_rng(seed * 7919 + 303 + layer * 131)
    b = rng.normal(0.0, BIAS_SIGMA, size=n_expert)
    return (b - b.mean()).astype(np.float32)


def expert_weights_f32(seed: int, layer: int, expert: int, hidden: int, inter: int):
    """fp32 weights of one expert ~ N(0, 0.02^2): gate [inter, hidden],
    up [inter, hidden], down [hidden, inter]."""
    rng = np.random.default_rng(expert_seed(seed, layer, expert))
    wg = rng.normal(0.0, WEIGHT_SIGMA, size=(inter, hidden)).astype(np.float32)
    wu = rng.normal(0.0, WEIGHT_SIGMA, size=(inter, hidden)).astype(np.float32)
    wd = rng.normal(0.0, WEIGHT_SIGMA, size=(hidden, inter)).astype(np.float32)
    return wg, wu, wd


def owner_slots(n_expert: int, local_experts: int, first_local: int = 0) -> np.ndarray:
    """Owner map int32 [n_expert]: experts [first_local, first_local+local) are
    local with slot e - first_local, every other expert is -1 (foreign)."""
    own = np.full(n_expert, -1, dtype=np.int32)
    own[first_local:first_local + local_experts] = np.arange(local_experts, dtype=np.int32)
    return own


# ---------------------------------------------------------------------------
# Counter-based Q8_0 block generator (integer only; the device fill in the
# library implements the same published generator independently).
#
# SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
# generators", OOPSLA 2014): the i-th output of a stream seeded with s is
# mix(s + (i+1)*GAMMA) with
#   mix(z): z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
#           z *= 0x94D049BB133111EB; z ^= z >> 31.
# All arithmetic is modulo 2^64.
#
# Block b of the stream with key s uses outputs i = 17*b .. 17*b + 16:
#   outputs 0..15: element 2t+h (h = 0, 1) takes bytes 4h..4h+3 of output t;
#                  v = sum of the four bytes (0..1020);
#                  q = clamp(((v * 43) >> 7) - 171, -127, 127)  (sd about 50)
#   output 16:     d bits = 0x0C00 | (o & 0x3FF)  (fp16 in [2^-12, 2^-11),
#                  the scale range Q8_0 gives N(0, 0.02^2) weights);
#                  element p = (o >> 10) & 31 is set to +127, or to -127 when
#                  bit 15 of o is set (every real Q8_0 block has a +-127).
# The stream key of (seed, layer, expert, matrix) is
#   mix(((seed & 0xFFFF) << 48 | (layer & 0xFFFF) << 32 |
#        (expert & 0xFFFF) << 16 | (matrix & 0xFFFF)) + GAMMA).
# ---------------------------------------------------------------------------

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
WORDS_PER_BLOCK = 17

MATRIX_GATE, MATRIX_UP, MATRIX_DOWN = 0, 1, 2
MATRIX_SHARED_GATE, MATRIX_SHARED_UP, MATRIX_SHARED_DOWN = 3, 4, 5


def _mix(z: np.ndarray) -> np.ndarray:
    z = z ^ (z >> np.uint64(30))
    z = z * _M1
    z = z ^ (z >> np.uint64(27))
    z = z * _M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, layer: int, expert: int, matrix: int) -> int:
    s = ((seed & 0xFFFF) << 48) | ((layer & 0xFFFF) << 32) | ((expert & 0xFFFF) << 16) | (matrix & 0xFFFF)
    with np.errstate(over="ignore"):
        return int(_mix(np.array([s], dtype=np.uint64) + GAMMA)[0])


_HERE = os.path.dirname(os.path.abspath(__file__))
_C_SRC = os.path.join(_HERE, "synth_q8_0.c")
_C_LIB = os.path.join(_HERE, "_synth_q8_0.so")
_C = None


def build_c(force: bool = False) -> str:
    """Compile the C version of the block generator (gcc, host only)."""
    if force or not os.path.exists(_C_LIB) or os.path.getmtime(_C_LIB) < os.path.getmtime(_C_SRC):
        tmp = _C_LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-shared", "-fPIC", _C_SRC, "-o", tmp], check=True)
        os.replace(tmp, _C_LIB)
    return _C_LIB


def _c_lib():
    global _C
    if _C is None:
        try:
            so = ctypes.CDLL(build_c())
            so.synth_q8_0_blocks.restype = None
            so.synth_q8_0_blocks.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64,
                                             ctypes.c_void_p]
            _C = so
        except (OSError, subprocess.CalledProcessError):
            _C = False
    return _C


def synth_q8_0_blocks(key: int, first_block: int, n_blocks: int, use_c: bool = True) -> np.ndarray:
    """Blocks [first_block, first_block + n_blocks) of the stream ``key`` as a
    Q8_0 structured array (34-byte records)."""
    c = _c_lib() if use_c else False
    if c:
        out = np.empty(n_blocks, dtype=Q8_0_DTYPE)
        c.synth_q8_0_blocks(key, first_block, n_blocks, out.ctypes.data)
        return out
    b = np.arange(first_block, first_block + n_blocks, dtype=np.uint64)
    i = b[:, None] * np.uint64(WORDS_PER_BLOCK) + np.arange(WORDS_PER_BLOCK, dtype=np.uint64)[None, :]
    with np.errstate(over="ignore"):
        o = _mix(np.uint64(key) + (i + np.uint64(1)) * GAMMA)          # [n, 17]
    words = o[:, :16]
    # byte sums of each 32-bit half of every output (bytes 0..3 and 4..7, little-endian)
    lo8 = np.uint64(0x00FF00FF00FF00FF)
    lo16 = np.uint64(0x0000FFFF0000FFFF)
    t = (words & lo8) + ((words >> np.uint64(8)) & lo8)
    u = (t & lo16) + ((t >> np.uint64(16)) & lo16)
    v = np.stack([u & np.uint64(0xFFFFFFFF), u >> np.uint64(32)], axis=-1).reshape(n_blocks, 32)
    q = np.clip(((v.astype(np.int64) * 43) >> 7) - 171, -127, 127)
    last = o[:, 16]
    p = ((last >> np.uint64(10)) & np.uint64(31)).astype(np.int64)
    neg = ((last >> np.uint64(15)) & np.uint64(1)).astype(bool)
    q[np.arange(n_blocks), p] = np.where(neg, -127, 127)
    dbits = (np.uint64(0x0C00) | (last & np.uint64(0x3FF))).astype(np.uint16)
    out = np.zeros(n_blocks, dtype=Q8_0_DTYPE)
    out["d"] = dbits.view(np.float16)
    out["qs"] = q.astype(np.int8)
    return out


def synth_q8_0_matrix(seed: int, layer: int, expert: int, matrix: int, rows: int, k: int,
                      row0: int = 0, nrows: int | None = None) -> np.ndarray:
    """Rows [row0, row0 + nrows) of a synthetic Q8_0 matrix [rows, k/32]."""
    nb = k // QK
    nrows = rows - row0 if nrows is None else nrows
    blocks = synth_q8_0_blocks(stream_key(seed, layer, expert, matrix), row0 * nb, nrows * nb)
    return blocks.reshape(nrows, nb)
