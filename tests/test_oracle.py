"""Pins of the CPU oracle against things other than itself (CPU only).

* q8_1 / Q8_0 bytes: hand-worked blocks (tests/golden/q8_blocks_worked.json)
  and an exact-rational re-derivation of the block rule (Python Fractions with
  explicit round-to-nearest-even to fp32/fp16) on random and adversarial blocks.
* products: fp64 dequantise-then-matmul brute force, the unit-scale closed form
  (every d = 1 makes the product the integer dot itself), exact rationals.
* SwiGLU-DS4: closed forms.
* router: brute-force properties of the selection, special cases with known
  answers (equal logits; planted tie), weights ratio.
* combine / grouping / layer: one-hot, all-masked, NaN in masked slots never
  read, permutation equivariance.
* mutation checks: plausible mistakes planted in copies of oracle functions
  (on the CPU) must each fail one of the pins above.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import moeq8_ref as ref
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# exact-rational IEEE helpers (independent of numpy's float arithmetic)
# ---------------------------------------------------------------------------

def _round_binary(x: Fraction, p: int, emin: int) -> Fraction:
    """Round x to the nearest value with p significant bits and minimum
    exponent emin (subnormals below), ties to even."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - p + 1)
    m = a / ulp
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def rn32(x):
    return _round_binary(Fraction(x), 24, -126)


def rn16(x):
    return _round_binary(Fraction(x), 11, -14)


def exact_block(xs):
    """Block rule in exact rationals: returns (d16, s16, q list)."""
    fx = [Fraction(float(v)) for v in np.asarray(xs, dtype=np.float32)]
    amax = max(abs(v) for v in fx)
    d = rn32(amax / 127)
    if d == 0:
        return Fraction(0), Fraction(0), [0] * 32
    q = []
    for v in fx:
        quot = rn32(v / d)
        m = abs(quot) + Fraction(1, 2)
        n = m.numerator // m.denominator
        q.append(n if quot >= 0 else -n)
    s = rn16(rn32(d * sum(q)))
    return rn16(d), s, q


def _check_block_exact(blocks_q81, xs):
    d16, s16, q = exact_block(xs)
    assert Fraction(float(blocks_q81["d"])) == d16
    assert Fraction(float(blocks_q81["s"])) == s16
    assert [int(v) for v in blocks_q81["qs"]] == q


# ---------------------------------------------------------------------------
# quantiser pins
# ---------------------------------------------------------------------------

def _golden_cases():
    with open(os.path.join(GOLDEN, "q8_blocks_worked.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_worked_blocks(case):
    x = np.array(case["x"], dtype=np.float32)[None]
    assert oracle.quantize_q8_1(x).tobytes().hex() == case["q8_1_hex"].replace(" ", "")
    assert oracle.quantize_q8_0(x).tobytes().hex() == case["q8_0_hex"].replace(" ", "")


def _discriminating_blocks():
    with open(os.path.join(GOLDEN, "q8_rule_discriminating_blocks.json")) as f:
        blocks = json.load(f)["blocks_hex"]
    return np.array([[float.fromhex(h) for h in b] for b in blocks], dtype=np.float32)


def test_quantize_matches_exact_rational_rule():
    rng = np.random.default_rng(11)
    xs = [rng.normal(0, 1, 32).astype(np.float32) for _ in range(40)]
    # adversarial blocks: exact halves of d, denormal-range values, one huge element
    xs.append(np.array([127.0] + [k + 0.5 for k in range(-15, 16)], dtype=np.float32))
    xs.append(np.array([1e-30] * 31 + [-3e-30], dtype=np.float32))
    xs.append(np.array([6.1e-5 * (k - 16) for k in range(32)], dtype=np.float32))
    xs.append(np.array([1e4] + [0.001 * k for k in range(31)], dtype=np.float32))
    xs.extend(list(_discriminating_blocks()))
    x = np.stack(xs)
    b = oracle.quantize_q8_1(x)
    for i in range(x.shape[0]):
        _check_block_exact(b[i, 0], x[i])


def test_quantize_invariants():
    x = workloads.normal_f32(5, (500, 128), 1.0)
    b = oracle.quantize_q8_1(x).reshape(-1)
    xb = x.reshape(-1, 32).astype(np.float64)
    q = b["qs"].astype(np.int64)
    d16 = b["d"].astype(np.float64)
    assert np.all(np.abs(q).max(axis=1) == 127)           # the amax element maps to +-127
    assert np.all(np.abs(q) <= 127)
    d32 = np.abs(xb).max(axis=1) / 127.0
    err = np.abs(xb - d16[:, None] * q)
    assert np.all(err <= d32[:, None] * (0.5 + 127 * 2.0 ** -11) * (1 + 1e-6))
    # s is fp16 of d * sum(q)
    s_ref = d32 * q.sum(axis=1)
    assert np.allclose(b["s"].astype(np.float64), s_ref, rtol=2.0 ** -10, atol=1e-7)
    # Q8_0 uses the same d and q
    w = oracle.quantize_q8_0(x).reshape(-1)
    assert np.array_equal(w["d"], b["d"]) and np.array_equal(w["qs"], b["qs"])


# ---------------------------------------------------------------------------
# product pins
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,k,c", [(3, 64, 1), (17, 256, 3), (64, 512, 8), (5, 4096, 2)])
def test_mmvq_matches_dequantized_fp64(n, k, c):
    w = oracle.quantize_q8_0(workloads.normal_f32(n * 7 + k, (n, k), 0.02))
    xq = oracle.quantize_q8_1(workloads.normal_f32(n * 13 + c, (c, k), 1.0))
    y = oracle.mmvq(w, xq)
    yb = oracle.mmvq_bruteforce(w, xq)
    assert y.shape == (c, n)
    scale = np.abs(oracle.dequantize(xq)) @ np.abs(oracle.dequantize(w)).T
    assert np.all(np.abs(y - yb) <= 1e-13 * scale + 1e-300)


def test_mmvq_exact_rational_small():
    w = oracle.quantize_q8_0(workloads.normal_f32(1, (4, 96), 0.02))
    xq = oracle.quantize_q8_1(workloads.normal_f32(2, (2, 96), 1.0))
    y = oracle.mmvq(w, xq)
    for c in range(2):
        for n in range(4):
            acc = Fraction(0)
            for b in range(3):
                dw = Fraction(float(w["d"][n, b]))
                dx = Fraction(float(xq["d"][c, b]))
                acc += dw * dx * sum(int(a) * int(bq) for a, bq in zip(w["qs"][n, b], xq["qs"][c, b]))
            assert abs(Fraction(y[c, n]) - acc) <= abs(acc) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)


def test_mmvq_unit_scale_closed_form():
    # every d = 1: the product is the plain integer dot; all q = 127 at K = 256
    # gives 256 * 127 * 127 = 4,129,024
    n, k = 3, 256
    w = np.zeros((n, k // 32), dtype=oracle.Q8_0_DTYPE)
    w["d"] = 1.0
    w["qs"] = 127
    xq = np.zeros((2, k // 32), dtype=oracle.Q8_1_DTYPE)
    xq["d"] = 1.0
    xq["qs"] = 127
    xq["qs"][1] = -127
    y = oracle.mmvq(w, xq)
    assert np.all(y[0] == 4129024.0) and np.all(y[1] == -4129024.0)
    # random int8 codes, d = 1: equals the int64 dot of the code vectors (N != C
    # so a transposed operand shows)
    rng = np.random.default_rng(3)
    w["qs"] = rng.integers(-127, 128, size=w["qs"].shape)
    xq["qs"] = rng.integers(-127, 128, size=xq["qs"].shape)
    qw = w["qs"].reshape(n, -1).astype(np.int64)
    qx = xq["qs"].reshape(2, -1).astype(np.int64)
    assert np.array_equal(oracle.mmvq(w, xq), (qx @ qw.T).astype(np.float64))


def test_column_range_equals_sliced_rows():
    n, k = 8, 1024
    w = oracle.quantize_q8_0(workloads.normal_f32(21, (n, k), 0.02))
    x = workloads.normal_f32(22, (3, k), 1.0)
    for off, nbs in [(0, 16), (16, 16), (4, 8), (30, 2)]:
        xs = oracle.quantize_q8_1(x[:, off * 32:(off + nbs) * 32])
        y_range = oracle.mmvq_column_range(w, xs, off)
        y_slice = oracle.mmvq(w[:, off:off + nbs], xs)
        np.testing.assert_allclose(y_range, y_slice, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(y_range, oracle.mmvq_bruteforce(w[:, off:off + nbs], xs),
                                   rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------------------
# SwiGLU-DS4 closed forms
# ---------------------------------------------------------------------------

def test_swiglu_closed_forms():
    silu7 = 7.0 / (1.0 + math.exp(-7.0))
    assert abs(silu7 - 6.993622642) < 1e-9
    h = oracle.swiglu_ds4([7.0, 100.0, -7.0, 0.0, 1.0, 2.0, -20.0],
                          [1.0, 1.0, 1.0, 5.0, 100.0, -100.0, 1.0])
    assert abs(h[0] - silu7) < 1e-15
    assert abs(h[1] - silu7) < 1e-15                      # gate clamped from above at 7
    assert abs(h[2] - (-7.0 / (1.0 + math.exp(7.0)))) < 1e-15
    assert abs(h[2] - (-0.006377358)) < 1e-9
    assert h[3] == 0.0
    assert abs(h[4] - 7.0 / (1.0 + math.exp(-1.0))) < 1e-14  # up clamped to +7
    assert abs(h[5] + 2.0 * 7.0 / (1.0 + math.exp(-2.0))) < 1e-14
    assert abs(h[6] - (-20.0 / (1.0 + math.exp(20.0)))) < 1e-20  # gate not clamped from below


# ---------------------------------------------------------------------------
# router pins
# ---------------------------------------------------------------------------

def test_sigmoid_f32_values():
    s = oracle.sigmoid_f32(np.array([0.0, 100.0, -100.0, math.log(3.0)], dtype=np.float32))
    assert s[0] == np.float32(0.5) and s[1] == np.float32(1.0)
    assert 0 < s[2] < 1e-40
    assert abs(float(s[3]) - 0.75) <= 2 ** -24
    x = workloads.normal_f32(9, (4096,), 3.0)
    sp, sn = oracle.sigmoid_f32(x), oracle.sigmoid_f32(-x)
    assert np.all(np.abs(sp.astype(np.float64) + sn - 1.0) <= 2 ** -24)


def test_route_equal_logits():
    ids, w, sel = oracle.route_topk(np.zeros((2, 256), np.float32), np.zeros(256, np.float32), None, 8)
    assert np.array_equal(ids, np.tile(np.arange(8, dtype=np.int32), (2, 1)))
    assert np.all(w == 0.125)


def test_route_planted_tie_lower_index_wins():
    logits = np.full((1, 16), -5.0, np.float32)
    top = [3, 9, 1, 12, 7, 0, 14]
    for r, e in enumerate(top):
        logits[0, e] = 4.0 - 0.5 * r
    logits[0, 11] = -1.0
    logits[0, 5] = -1.0                                  # exact tie for the 8th place
    ids, w, _ = oracle.route_topk(logits, None, None, 8)
    assert list(ids[0]) == top + [5]


def _check_selection(logits, bias, ids_sel, topk):
    score = (1.0 / (1.0 + np.exp(-logits.astype(np.float64)))).astype(np.float32)
    key = score + (bias if bias is not None else np.float32(0))
    for j in range(logits.shape[0]):
        s = list(ids_sel[j])
        assert len(set(s)) == topk
        rest = [e for e in range(logits.shape[1]) if e not in s]
        for e in s:
            for r in rest:
                assert key[j, e] > key[j, r] or (key[j, e] == key[j, r] and e < r)
        for a, b in zip(s, s[1:]):
            assert key[j, a] > key[j, b] or (key[j, a] == key[j, b] and a < b)


def test_route_brute_force_properties():
    c, e = 6, 256
    logits = workloads.router_logits(3, c, e)
    bias = workloads.router_bias(3, e)
    ids, w, sel = oracle.route_topk(logits, bias, None, 8)
    _check_selection(logits, bias, sel, 8)
    assert np.array_equal(ids, sel)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    score = oracle.sigmoid_f32(logits).astype(np.float64)
    chosen = np.take_along_axis(score, sel, axis=1)
    np.testing.assert_allclose(w * chosen[:, :1], chosen * w[:, :1], rtol=1e-15)  # w proportional to score


def test_route_bias_selects_only():
    logits = np.zeros((1, 12), np.float32)
    logits[0, :8] = 1.0                                  # experts 0..7 win without bias
    bias = np.zeros(12, np.float32)
    bias[10] = 1.0                                       # expert 10 is pulled in by the bias
    ids, w, _ = oracle.route_topk(logits, bias, None, 8)
    assert ids[0, 0] == 10 and 7 not in ids[0]
    s1, s0 = 1 / (1 + math.exp(-1)), 0.5
    tot = 7 * s1 + s0
    np.testing.assert_allclose(w[0, 0], float(np.float32(s0)) / (7 * float(np.float32(s1)) + float(np.float32(s0))), rtol=1e-15)
    assert abs(w[0, 1] - s1 / tot) < 1e-7


def test_route_owner_mask():
    c, e = 4, 256
    logits = workloads.router_logits(5, c, e)
    bias = workloads.router_bias(5, e)
    own = workloads.owner_slots(e, 128)
    ids, w, sel = oracle.route_topk(logits, bias, own, 8)
    ids_all, w_all, _ = oracle.route_topk(logits, bias, None, 8)
    assert np.array_equal(w, w_all)                     # normalised over all 8 routes
    assert np.array_equal(ids, np.where(sel < 128, sel, -1))
    own2 = workloads.owner_slots(e, 128, first_local=128)
    ids2, _, _ = oracle.route_topk(logits, bias, own2, 8)
    assert np.array_equal(ids2, np.where(sel >= 128, sel - 128, -1))


# ---------------------------------------------------------------------------
# grouping / combine / layer
# ---------------------------------------------------------------------------

def test_group_routes_brute_force():
    ids = np.array([[5, 2, -1, 7], [2, 9, 5, -1], [7, 7, 0, 2]], dtype=np.int32)
    groups = oracle.group_routes(ids)
    assert groups == [(0, [10]), (2, [1, 4, 11]), (5, [0, 6]), (7, [3, 8, 9]), (9, [5])]


def test_combine_pins():
    rng = np.random.default_rng(4)
    y = rng.normal(size=(3, 4, 16))
    ids = np.array([[0, 1, 2, 3], [-1, -1, -1, -1], [4, -1, 5, 6]], dtype=np.int32)
    w = np.array([[0, 0, 1, 0], [0.25] * 4, [0.5, 0.2, 0.3, 0.0]])
    y[2, 1] = np.nan                                      # a masked slot's content is never read
    out = oracle.moe_combine(y, ids, w)
    assert np.array_equal(out[0], y[0, 2])                # one-hot weight -> that route's y
    assert np.all(out[1] == 0.0)                          # all masked -> zero
    np.testing.assert_allclose(out[2], 0.5 * y[2, 0] + 0.3 * y[2, 2], rtol=1e-15)
    # the shared expert's output is added once after the routed sum (R15):
    # all masked -> exactly the shared output; one-hot on small integers ->
    # the exact sum; a zero shared output leaves the routed sum unchanged
    shared = rng.integers(-8, 8, size=(3, 16)).astype(np.float64)
    yi = np.round(y * 4)
    yi[2, 1] = np.nan
    out_s = oracle.moe_combine(yi, ids, w, shared=shared)
    assert np.array_equal(out_s[1], shared[1])
    assert np.array_equal(out_s[0], yi[0, 2] + shared[0])
    assert np.array_equal(oracle.moe_combine(y, ids, w, shared=np.zeros((3, 16))), out)


def _tiny_experts(seed, n_exp, hidden, inter):
    cache = {}

    def get(e):
        if e not in cache:
            wg, wu, wd = workloads.expert_weights_f32(seed, 0, e, hidden, inter)
            cache[e] = (oracle.quantize_q8_0(wg), oracle.quantize_q8_0(wu), oracle.quantize_q8_0(wd))
        return cache[e]
    return get


def test_moe_layer_composition_and_permutation():
    hidden, inter, n_exp, c = 128, 64, 16, 3
    experts = _tiny_experts(7, n_exp, hidden, inter)
    x = workloads.activations(7, c, hidden)
    logits = workloads.router_logits(7, c, n_exp)
    bias = workloads.router_bias(7, n_exp)
    r = oracle.moe_layer(x, logits, bias, None, experts, 4)
    # composition by fp64 brute force: dequantised matrices, the same q8_1 rule
    xq = oracle.quantize_q8_1(x)
    xd = oracle.dequantize(xq)
    for j in range(c):
        acc = np.zeros(hidden)
        for s in range(4):
            wg, wu, wd = experts(int(r["ids"][j, s]))
            g = oracle.dequantize(wg) @ xd[j]
            u = oracle.dequantize(wu) @ xd[j]
            h = oracle.swiglu_ds4(g, u).astype(np.float32)[None]
            y = oracle.dequantize(wd) @ oracle.dequantize(oracle.quantize_q8_1(h))[0]
            acc += r["weights"][j, s] * y
        np.testing.assert_allclose(r["out"][j], acc, rtol=1e-9, atol=1e-12)
    perm = [2, 0, 1]
    r2 = oracle.moe_layer(x[perm], logits[perm], bias, None, experts, 4)
    np.testing.assert_array_equal(r2["out"], r["out"][perm])


# ---------------------------------------------------------------------------
# mutation checks: each planted mistake fails a pin above
# ---------------------------------------------------------------------------

def _half_even_q81(x):
    x = np.asarray(x, np.float32).reshape(-1, 32)
    amax = np.abs(x).max(1)
    d = (amax / np.float32(127)).astype(np.float32)
    q = np.round(x / d[:, None]).astype(np.int32)       # mistake: ties to even
    out = np.zeros((x.shape[0], 1), dtype=oracle.Q8_1_DTYPE)
    out["d"][:, 0] = d.astype(np.float16)
    out["s"][:, 0] = (d * q.sum(1).astype(np.float32)).astype(np.float16)
    out["qs"][:, 0] = q
    return out


def _reciprocal_q81(x):
    x = np.asarray(x, np.float32).reshape(-1, 32)
    amax = np.abs(x).max(1)
    d = (amax / np.float32(127)).astype(np.float32)
    inv = (np.float32(1) / d).astype(np.float32)
    v = (x * inv[:, None]).astype(np.float32)           # mistake: x * (1/d)
    q = (np.sign(v) * np.floor(np.abs(v.astype(np.float64)) + 0.5)).astype(np.int32)
    out = np.zeros((x.shape[0], 1), dtype=oracle.Q8_1_DTYPE)
    out["d"][:, 0] = d.astype(np.float16)
    out["s"][:, 0] = (d * q.sum(1).astype(np.float32)).astype(np.float16)
    out["qs"][:, 0] = q
    return out


def test_mutation_half_even_caught_by_worked_block():
    case = [c for c in _golden_cases() if c["name"] == "halves_round_away"][0]
    x = np.array(case["x"], np.float32)[None]
    assert _half_even_q81(x).tobytes().hex() != case["q8_1_hex"].replace(" ", "")


def test_mutation_reciprocal_caught_by_exact_rule():
    caught = 0
    for xs in _discriminating_blocks():
        try:
            _check_block_exact(_reciprocal_q81(xs[None])[0, 0], xs)
        except AssertionError:
            caught += 1
    assert caught == 3


def test_mutation_product_mistakes_caught():
    n, k, c = 5, 256, 2
    w = oracle.quantize_q8_0(workloads.normal_f32(31, (n, k), 0.02))
    xq = oracle.quantize_q8_1(workloads.normal_f32(32, (c, k), 1.0))
    yb = oracle.mmvq_bruteforce(w, xq)
    sumi = oracle.block_dots(w, xq).astype(np.float64)
    dw, dx = w["d"].astype(np.float64), xq["d"].astype(np.float64)
    dropped = np.einsum("nb,cb,cnb->cn", dw[:, :-1], dx[:, :-1], sumi[:, :, :-1])
    wrong_scale = np.einsum("nb,cb,cnb->cn", dw, dx[:, ::-1], sumi)
    for bad in (dropped, wrong_scale, -yb):
        assert not np.allclose(bad, yb, rtol=1e-6, atol=1e-9)


def test_mutation_router_mistakes_caught():
    logits = np.zeros((1, 12), np.float32)
    logits[0, :8] = 1.0
    bias = np.zeros(12, np.float32)
    bias[10] = 1.0
    key_minus = oracle.sigmoid_f32(logits) - bias        # mistake: bias subtracted
    sel_minus = sorted(range(12), key=lambda i: (-float(key_minus[0, i]), i))[:8]
    assert sel_minus[0] != 10
    # mistake: weights taken from the biased keys
    ids, w, _ = oracle.route_topk(logits, bias, None, 8)
    key = oracle.sigmoid_f32(logits) + bias
    wk = key[0, ids[0]] / key[0, ids[0]].sum()
    assert abs(wk[0] - w[0, 0]) > 1e-3


def test_mutation_swiglu_symmetric_clamp_caught():
    g = np.array([-20.0])
    bad = np.clip(g, -7, 7) / (1 + np.exp(-np.clip(g, -7, 7)))   # mistake: gate clamped both ways
    assert abs(bad[0] - oracle.swiglu_ds4(g, [1.0])[0]) > 1e-3


# ---------------------------------------------------------------------------
# input generator: the C and numpy versions of the counter-based block
# generator agree (the oracle's inputs never depend on which one ran)
# ---------------------------------------------------------------------------

def test_synthetic_generator_c_matches_numpy():
    for key_args, first, n in [((5, 1, 2, 0), 0, 4096), ((0, 0, 0, 0), 5, 1000),
                               ((65535, 42, 127, 5), 123456, 777)]:
        key = workloads.stream_key(*key_args)
        a = workloads.synth_q8_0_blocks(key, first, n)
        b = workloads.synth_q8_0_blocks(key, first, n, use_c=False)
        assert a.tobytes() == b.tobytes()
        q = b["qs"].astype(np.int64)
        assert np.all(np.abs(q).max(axis=1) == 127)
        d = b["d"].view(np.uint16)
        assert np.all((d >= 0x0C00) & (d < 0x1000))


# ---------------------------------------------------------------------------
# 8-bit block exchange codec pins (R17, R18)
# ---------------------------------------------------------------------------

def exact_block_q8x(xs):
    """R17 in exact rationals: (d as the fp32 quotient amax/127, codes)."""
    fx = [Fraction(float(v)) for v in np.asarray(xs, dtype=np.float32)]
    amax = max(abs(v) for v in fx)
    d = rn32(amax / 127)
    if d == 0:
        return Fraction(0), [0] * 32
    q = []
    for v in fx:
        quot = rn32(v / d)
        m = abs(quot) + Fraction(1, 2)
        n = m.numerator // m.denominator
        q.append(n if quot >= 0 else -n)
    return d, q


def test_q8x_block_is_1_125_bytes_per_value():
    # 32 int8 values and one f32 scale: 1.125 bytes a value, as the pages state
    assert oracle.Q8X_DTYPE.itemsize == 36
    assert oracle.Q8X_DTYPE.itemsize / 32 == 1.125
    b = oracle.q8x_encode(np.zeros((3, 64), np.float32))
    assert b.shape == (3, 2) and b.tobytes() == bytes(3 * 2 * 36)   # all-zero blocks: all-zero bytes


def test_q8x_power_of_two_scale_closed_form():
    # amax = 127 * 2^-2: d = 2^-2 exactly, and values on the grid are their own codes
    q = np.array([127, -127] + list(range(-15, 15)), np.int32)
    x = (q.astype(np.float32) * np.float32(0.25))[None]
    b = oracle.q8x_encode(x)
    assert float(b["d"][0, 0]) == 0.25
    assert list(b["qs"][0, 0]) == list(q)
    assert np.array_equal(oracle.q8x_dequantize(b), x)
    raw = b.tobytes()
    assert raw[:4] == np.float32(0.25).tobytes() and raw[4] == 127 and raw[5] == 256 - 127


def test_q8x_codes_match_exact_rational_rule():
    rng = np.random.default_rng(12)
    xs = [rng.normal(0, 1, 32).astype(np.float32) for _ in range(40)]
    xs.append(np.array([127.0] + [k + 0.5 for k in range(-15, 16)], dtype=np.float32))   # exact halves
    xs.append(np.array([1.0] + [0.3 * (k - 15) / 15 for k in range(31)], np.float32))       # d = 1/127
    xs.append(np.array([1e-30] * 31 + [-3e-30], dtype=np.float32))
    xs.extend(list(_discriminating_blocks()))
    x = np.stack(xs)
    b = oracle.q8x_encode(x)
    for i in range(x.shape[0]):
        d, q = exact_block_q8x(x[i])
        assert Fraction(float(b["d"][i, 0])) == d
        assert [int(v) for v in b["qs"][i, 0]] == q


def test_q8x_round_trip_within_half_a_code():
    x = workloads.normal_f32(21, (64, 4096), 3.0)
    b = oracle.q8x_encode(x)
    back = oracle.q8x_dequantize(b).astype(np.float64)
    d = np.repeat(b["d"].astype(np.float64), 32, axis=1)
    # |x/d - q| <= 1/2 up to the fp32 quotient's and product's roundings
    assert np.all(np.abs(x - back) <= 0.5 * d * (1 + 2.0 ** -20) + np.abs(x) * 2.0 ** -22)


def _blocks_from(dq_rows):
    """Exchange blocks from explicit (d, codes) per row: one block per row."""
    out = np.zeros((len(dq_rows), 1), dtype=oracle.Q8X_DTYPE)
    for i, (d, q) in enumerate(dq_rows):
        out["d"][i, 0] = np.float32(d)
        out["qs"][i, 0] = np.asarray(q, np.int8)
    return out


def test_q8x_decode_sum_in_rank_order():
    # rank 0 holds 127 * 2^20 (fp32 spacing 8 there), ranks 1 and 2 hold 3:
    # ((127*2^20 + 3) + 3) = 127*2^20 in fp32, while the exact sum 127*2^20 + 6
    # rounds to 127*2^20 + 8; so the rank order is visible in the result
    big = _blocks_from([(2.0 ** 20, [127] + [0] * 31)])
    three = _blocks_from([(1.0, [3] + [0] * 31)])
    s = oracle.q8x_decode_sum([big, three, three])
    assert s[0, 0] == np.float32(127 * 2 ** 20)
    assert oracle.q8x_decode_sum([three, three, big])[0, 0] == np.float32(127 * 2 ** 20 + 8)
    assert np.all(s[0, 1:] == 0)


def test_q8x_decode_sum_single_rank_and_fp64_bound():
    rng = np.random.default_rng(9)
    parts = [oracle.q8x_encode(workloads.normal_f32(100 + r, (8, 256), 1.0 + r)) for r in range(5)]
    assert np.array_equal(oracle.q8x_decode_sum(parts[:1]), oracle.q8x_dequantize(parts[0]))
    vals = np.stack([oracle.q8x_dequantize(p).astype(np.float64) for p in parts])
    s = oracle.q8x_decode_sum(parts).astype(np.float64)
    exact = vals.sum(axis=0)
    # fp32 left-to-right sum of 5 terms: |error| <= 4 * 2^-24 * sum |terms| (first order)
    assert np.all(np.abs(s - exact) <= 4 * 2.0 ** -24 * np.abs(vals).sum(axis=0) * (1 + 1e-6))
    # a product d*q that is not exact in fp32 is rounded once
    b = _blocks_from([(np.float32(1) / np.float32(3), [127] + [0] * 31)])
    assert oracle.q8x_dequantize(b)[0, 0] == np.float32(np.float32(1 / 3) * np.float32(127))
    _ = rng


def test_mutation_q8x_mistakes_caught():
    # an fp16-rounded scale fails the exact rule on a block whose d is not an fp16 value
    xs = np.array([1.0] + [0.3 * (k - 15) / 15 for k in range(31)], np.float32)
    d_exact, _ = exact_block_q8x(xs)
    assert Fraction(float(np.float16(float(d_exact)))) != d_exact
    # summing in reverse rank order fails the planted-order pin
    big = _blocks_from([(2.0 ** 20, [127] + [0] * 31)])
    three = _blocks_from([(1.0, [3] + [0] * 31)])
    rev = np.zeros((1, 32), np.float32)
    for blocks in reversed([big, three, three]):
        rev = (rev + oracle.q8x_dequantize(blocks)).astype(np.float32)
    assert rev[0, 0] != oracle.q8x_decode_sum([big, three, three])[0, 0]
    # ties to even on the exact-halves block changes codes
    xh = np.array([127.0] + [k + 0.5 for k in range(-15, 16)], dtype=np.float32)
    _, q = exact_block_q8x(xh)
    assert list(np.round(xh / np.float32(1.0)).astype(int)) != q


# ---------------------------------------------------------------------------
# 4-bit weight blocks (R19)
# ---------------------------------------------------------------------------

def exact_block_q4(xs):
    """R19 in exact rationals: (fp16 d, codes 0..15)."""
    fx = [Fraction(float(v)) for v in np.asarray(xs, dtype=np.float32)]
    amax = max(abs(v) for v in fx)
    d = rn32(amax / 7)
    if d == 0:
        return Fraction(0), [8] * 32
    codes = []
    for v in fx:
        quot = rn32(v / d)
        m = abs(quot) + Fraction(1, 2)
        n = m.numerator // m.denominator
        n = n if quot >= 0 else -n
        codes.append(min(7, max(-8, n)) + 8)
    return rn16(d), codes


def test_q4_block_layout_closed_form():
    # amax = 7 * 2^-3: d = 2^-3; values on the grid are their codes; nibble order
    q = np.array([7, -7, 0, 1, -1] + [k % 15 - 7 for k in range(27)], np.int32)
    x = (q.astype(np.float32) * np.float32(0.125))[None]
    b = oracle.quantize_q4(x)
    assert oracle.Q4_DTYPE.itemsize == 18 and b.shape == (1, 1)
    assert float(b["d"][0, 0]) == 0.125
    codes = q + 8
    raw = b.tobytes()
    assert raw[:2] == np.float16(0.125).tobytes()
    for i in range(16):
        assert raw[2 + i] == (codes[i] | (codes[16 + i] << 4))
    assert np.array_equal(oracle.q4_values(b)[0, 0], q)
    assert np.array_equal(oracle.dequantize_q4(b)[0], x[0].astype(np.float64))
    z = oracle.quantize_q4(np.zeros((1, 32), np.float32))
    assert z.tobytes() == bytes(2) + bytes([0x88] * 16)


def test_q4_quantize_matches_exact_rational_rule():
    rng = np.random.default_rng(13)
    xs = [rng.normal(0, 0.02, 32).astype(np.float32) for _ in range(40)]
    xs.append(np.array([7.0] + [k + 0.5 for k in range(-8, 7)] + [0.25 * k for k in range(16)], np.float32))
    xs.append(np.array([1.0] + [0.9 * (k - 15) / 15 for k in range(31)], np.float32))
    for x in xs:
        b = oracle.quantize_q4(x[None])[0, 0]
        d16, codes = exact_block_q4(x)
        assert Fraction(float(b["d"])) == d16
        got = [int(v) for v in np.concatenate([b["qs"] & 0xF, b["qs"] >> 4])]
        assert got == codes


def test_q4_products_match_dequantized_fp64():
    rng = np.random.default_rng(14)
    w = oracle.quantize_q4(rng.normal(0, 0.02, (24, 256)).astype(np.float32))
    xq = oracle.quantize_q8_1(rng.normal(0, 1, (3, 256)).astype(np.float32))
    y = oracle.mmvq_q4(w, xq)
    brute = oracle.dequantize(xq) @ oracle.dequantize_q4(w).T
    np.testing.assert_allclose(y, brute, rtol=1e-12, atol=1e-12)


def test_q4_unit_scale_closed_form():
    # all scales 1: the product is the integer dot of (code - 8) with the quants
    rng = np.random.default_rng(15)
    w = np.zeros((5, 4), oracle.Q4_DTYPE)
    w["d"] = 1.0
    w["qs"] = rng.integers(0, 256, size=(5, 4, 16))
    xq = np.zeros((2, 4), oracle.Q8_1_DTYPE)
    xq["d"] = 1.0
    xq["qs"] = rng.integers(-127, 128, size=(2, 4, 32))
    y = oracle.mmvq_q4(w, xq)
    for c in range(2):
        for n in range(5):
            tot = 0
            for b in range(4):
                for i in range(16):
                    byte = int(w["qs"][n, b, i])
                    tot += ((byte & 15) - 8) * int(xq["qs"][c, b, i]) + ((byte >> 4) - 8) * int(xq["qs"][c, b, 16 + i])
            assert y[c, n] == tot


def test_mutation_q4_mistakes_caught():
    # swapping the nibble halves, or dropping the -8 offset, breaks the closed forms
    q = np.array([7, -7, 0, 1, -1] + [k % 15 - 7 for k in range(27)], np.int32)
    x = (q.astype(np.float32) * np.float32(0.125))[None]
    b = oracle.quantize_q4(x)
    qs = b["qs"][0, 0].astype(np.int32)
    swapped = np.concatenate([qs >> 4, qs & 0xF]) - 8
    assert not np.array_equal(swapped, q)
    no_offset = np.concatenate([qs & 0xF, qs >> 4])
    assert not np.array_equal(no_offset, q)


def _unit_q4(codes_rows):
    """Q4 rows of unit scale from signed values in [-8, 7] (value i < 16 in the
    low nibble of byte i, value i + 16 in the high one)."""
    v = np.asarray(codes_rows, np.int32)
    rows, k = v.shape
    c = (v + 8).reshape(rows, k // 32, 32).astype(np.uint8)
    w = np.zeros((rows, k // 32), oracle.Q4_DTYPE)
    w["d"] = 1.0
    w["qs"] = c[..., :16] | (c[..., 16:] << 4)
    return w


def test_q4_glu_pair_closed_form():
    # Unit scales make the two products integer dots that can be read off:
    # gate row 0 picks x value 0, up row 0 picks twice x value 1, and the
    # SwiGLU-DS4 closed form of (g, u) follows (gate clamped above at 7 only,
    # up clamped to +-7).  The RDNA4 Q8_0 gate/up pair commit of PR #826
    # defines the pair as the two separate products followed by the GLU.
    k = 64
    gate = np.zeros((4, k), np.int32)
    up = np.zeros((4, k), np.int32)
    gate[0, 0], up[0, 1] = 1, 2            # g = x0,       u = 2 x1
    gate[1, 2], up[1, 3] = 3, 7            # g = 3 x2,     u = 7 x3
    gate[2, 4], up[2, 5] = -5, 1           # g = -5 x4,    u = x5
    gate[3, 40], up[3, 33] = 7, -6         # second block
    xq = np.zeros((1, k // 32), oracle.Q8_1_DTYPE)
    xq["d"] = 1.0
    q = np.zeros(k, np.int32)
    q[[0, 1, 2, 3, 4, 5, 33, 40]] = [1, 2, 3, 2, 1, 9, 1, 2]
    xq["qs"][0] = q.reshape(k // 32, 32)
    h, g, u = oracle.glu_pair_q4(_unit_q4(gate), _unit_q4(up), xq)
    assert list(g[0]) == [1.0, 9.0, -5.0, 14.0]
    assert list(u[0]) == [4.0, 14.0, 9.0, -6.0]

    def silu(z):
        return z / (1.0 + math.exp(-z))
    want = [silu(1.0) * 4.0, silu(7.0) * 7.0, silu(-5.0) * 7.0, silu(7.0) * -6.0]
    for a, b in zip(h[0], want):
        assert abs(a - b) <= 1e-15 * max(1.0, abs(b))


def test_q4_glu_pair_matches_dequantized_products():
    # the pair equals dequantise-then-fp64 products of each matrix followed by
    # SwiGLU-DS4, gate through the first operand and up through the second
    rng = np.random.default_rng(16)
    wg = oracle.quantize_q4(rng.normal(0, 0.02, (20, 512)).astype(np.float32))
    wu = oracle.quantize_q4(rng.normal(0, 0.02, (20, 512)).astype(np.float32))
    xq = oracle.quantize_q8_1(rng.normal(0, 1, (3, 512)).astype(np.float32) * 40)
    h, g, u = oracle.glu_pair_q4(wg, wu, xq)
    xd = oracle.dequantize(xq)
    gb = xd @ oracle.dequantize_q4(wg).T
    ub = xd @ oracle.dequantize_q4(wu).T
    np.testing.assert_allclose(g, gb, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(u, ub, rtol=1e-12, atol=1e-12)
    assert np.abs(gb).max() > 7 and np.abs(ub).max() > 7      # both clamps are exercised
    gc = np.minimum(gb, 7.0)
    hb = gc / (1.0 + np.exp(-gc)) * np.clip(ub, -7.0, 7.0)
    np.testing.assert_allclose(h, hb, rtol=1e-12, atol=1e-12)


def test_mutation_q4_glu_pair_caught():
    # planted mistakes in copies of the pair: gate and up swapped, the Q8_0
    # product called on 4-bit blocks, the offset -8 dropped
    rng = np.random.default_rng(17)
    wg = oracle.quantize_q4(rng.normal(0, 0.02, (8, 256)).astype(np.float32))
    wu = oracle.quantize_q4(rng.normal(0, 0.02, (8, 256)).astype(np.float32))
    xq = oracle.quantize_q8_1(rng.normal(0, 1, (2, 256)).astype(np.float32) * 40)
    h = oracle.glu_pair_q4(wg, wu, xq)[0]
    swapped = oracle.swiglu_ds4(oracle.mmvq_q4(wu, xq), oracle.mmvq_q4(wg, xq))
    assert not np.allclose(swapped, h, rtol=1e-6, atol=1e-9)
    with pytest.raises(Exception):
        oracle.mmvq(wg, xq)                                 # 16 code bytes are not 32 quants
    def no_offset(w):
        qs = w["qs"].astype(np.int64)
        v = np.concatenate([qs & 0xF, qs >> 4], axis=-1)
        return np.einsum("nb,cb,cnbk,->cn", w["d"].astype(np.float64), xq["d"].astype(np.float64),
                         v[None] * xq["qs"].astype(np.int64)[:, None], 1.0)
    bad = oracle.swiglu_ds4(no_offset(wg), no_offset(wu))
    assert not np.allclose(bad, h, rtol=1e-6, atol=1e-9)


def test_glu_pair_and_expert_ffn_match_dequantized_products():
    # the Q8_0 pair and the one-column expert FFN by dequantise-then-fp64
    # brute force: g through the first matrix, u through the second, SwiGLU-DS4
    # written out, h rounded to fp32 before its q8_1 (R8), then the down
    rng = np.random.default_rng(18)
    wg = oracle.quantize_q8_0(rng.normal(0, 0.02, (16, 256)).astype(np.float32))
    wu = oracle.quantize_q8_0(rng.normal(0, 0.02, (16, 256)).astype(np.float32))
    wd = oracle.quantize_q8_0(rng.normal(0, 0.02, (256, 32)).astype(np.float32))
    xq = oracle.quantize_q8_1(rng.normal(0, 1, (2, 256)).astype(np.float32) * 40)
    h, g, u = oracle.glu_pair(wg, wu, xq)
    xd = oracle.dequantize(xq)
    gb, ub = xd @ oracle.dequantize(wg).T, xd @ oracle.dequantize(wu).T
    np.testing.assert_allclose(g, gb, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(u, ub, rtol=1e-12, atol=1e-12)
    assert np.abs(gb).max() > 7 and np.abs(ub).max() > 7
    gc = np.minimum(gb, 7.0)
    hb = gc / (1.0 + np.exp(-gc)) * np.clip(ub, -7.0, 7.0)
    np.testing.assert_allclose(h, hb, rtol=1e-12, atol=1e-12)
    swapped = oracle.swiglu_ds4(ub, gb)                    # planted: gate and up swapped
    assert not np.allclose(swapped, h, rtol=1e-6, atol=1e-9)
    # expert_ffn at an intermediate size of one block (32 values)
    wg2 = oracle.quantize_q8_0(rng.normal(0, 0.02, (32, 256)).astype(np.float32))
    wu2 = oracle.quantize_q8_0(rng.normal(0, 0.02, (32, 256)).astype(np.float32))
    r = oracle.expert_ffn(wg2, wu2, wd, xq[1:2])
    g2 = oracle.dequantize(wg2) @ xd[1]
    u2 = oracle.dequantize(wu2) @ xd[1]
    g2c = np.minimum(g2, 7.0)
    h2 = (g2c / (1.0 + np.exp(-g2c)) * np.clip(u2, -7.0, 7.0)).astype(np.float32)
    hq2 = oracle.quantize_q8_1(h2[None])
    assert r["hq"].tobytes() == hq2[0].tobytes()
    np.testing.assert_allclose(r["y"], oracle.dequantize(wd) @ oracle.dequantize(hq2)[0],
                               rtol=1e-12, atol=1e-12)


def test_every_oracle_function_is_pinned_here():
    # every public function of the oracle module is exercised by a pin in this
    # file (a function no CPU test calls would be trusted unchecked)
    import inspect
    with open(__file__) as f:
        src = f.read()
    names = [n for n, fn in inspect.getmembers(ref, inspect.isfunction)
             if fn.__module__ == ref.__name__ and not n.startswith("_")]
    missing = [n for n in names if f"oracle.{n}(" not in src and f"ref.{n}(" not in src]
    assert not missing, missing
