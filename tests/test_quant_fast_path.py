"""Host check of the quantisers' division-skipping rule (q8_code in
csrc/moeq8_device.hpp), emulated in numpy fp32.

The block rule rounds the correctly rounded fp32 quotient x / d half away from
zero.  The kernels first form t = x * rcp(d) with the hardware reciprocal
(within an ulp of 1/d) and keep rint(t) unless t lies within 2^-12 of a
half-integer, where they divide.  This test emulates t for each reciprocal an
ulp-accurate rcp can return (the correctly rounded 1/d and its two fp32
neighbours) on random and adversarial blocks and checks that every kept code
equals the rule's code.  No GPU and no oracle code is involved: the rule is
restated here from its definition.
"""

import json
import os

import numpy as np

MARGIN = np.float32(0.5) - np.float32(2.0 ** -12)


def rule_codes(x32, d32):
    """roundf(fl32(x / d)) computed exactly: the fp32 quotient, then halves
    away from zero in fp64 (where a - floor(a) is exact)."""
    q = (x32 / d32).astype(np.float32).astype(np.float64)
    a = np.abs(q)
    f = np.floor(a)
    r = f + (a - f >= 0.5)
    return (np.sign(q) * r).astype(np.int64)


def fast_codes(x32, rd32):
    """(kept, code): the code rint(t) and whether the kernel keeps it."""
    t = (x32 * rd32).astype(np.float32)
    r = np.rint(t)
    with np.errstate(invalid="ignore"):
        kept = np.abs((t - r).astype(np.float32)) < MARGIN
    return kept, np.nan_to_num(r).astype(np.int64)


def blocks_scale(x32):
    amax = np.abs(x32).max(axis=1, keepdims=True).astype(np.float32)
    return (amax / np.float32(127.0)).astype(np.float32)


def check(x32):
    d = blocks_scale(x32)
    live = (d[:, 0] >= np.float32(2.0 ** -126))
    x32, d = x32[live], d[live]
    exact = rule_codes(x32, d)
    rcp = (np.float32(1.0) / d).astype(np.float32)
    n_kept_total = 0
    for rd in (rcp, np.nextafter(rcp, np.float32(np.inf)), np.nextafter(rcp, np.float32(0))):
        kept, code = fast_codes(x32, rd.astype(np.float32))
        assert np.array_equal(code[kept], exact[kept])
        n_kept_total += int(kept.sum())
    return n_kept_total / (3 * x32.size)


def test_fast_path_random_blocks():
    rng = np.random.default_rng(11)
    x = rng.normal(0.0, 1.0, size=(60000, 32)).astype(np.float32)
    frac = check(x)
    assert frac > 0.999          # the division is the exception


def test_fast_path_scaled_and_wide_range_blocks():
    rng = np.random.default_rng(12)
    x = rng.normal(0.0, 1.0, size=(20000, 32))
    x *= np.exp2(rng.integers(-100, 100, size=(20000, 1)))
    check(x.astype(np.float32))


def test_fast_path_half_integer_quotients():
    """Blocks built so that many quotients are exact or near half-integers."""
    rng = np.random.default_rng(13)
    n = 20000
    d = np.float32(1.0) * np.exp2(rng.integers(-20, 20, size=(n, 1))).astype(np.float32)
    k = rng.integers(-126, 127, size=(n, 32)) + 0.5
    x = (k * d).astype(np.float32)
    x[:, 0] = np.float32(127.0) * d[:, 0]                   # the amax element fixes d
    x = np.nextafter(x, rng.choice([-np.inf, 0, np.inf], size=x.shape).astype(np.float32)).astype(np.float32)
    check(x)


def test_fast_path_rule_discriminating_blocks():
    """The golden blocks where x / d and x * (1/d) give different codes."""
    path = os.path.join(os.path.dirname(__file__), "golden", "q8_rule_discriminating_blocks.json")
    with open(path) as f:
        data = json.load(f)
    x = np.array([[float.fromhex(v) for v in b] for b in data["blocks_hex"]], dtype=np.float32)
    d = blocks_scale(x)
    exact = rule_codes(x, d)
    rcp = (np.float32(1.0) / d).astype(np.float32)
    # x * (1/d) rounded half away: the other rule, which differs somewhere here
    p = (x * rcp).astype(np.float32).astype(np.float64)
    other = (np.sign(p) * np.floor(np.abs(p) + 0.5)).astype(np.int64)
    assert np.any(other != exact)
    for rd in (rcp, np.nextafter(rcp, np.float32(np.inf)), np.nextafter(rcp, np.float32(0))):
        kept, code = fast_codes(x, rd.astype(np.float32))
        assert np.array_equal(code[kept], exact[kept])
        assert not np.any(kept & (other != exact))    # those values take the division
