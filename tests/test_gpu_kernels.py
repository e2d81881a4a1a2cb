"""GPU parity of each libmoeq8 call against the CPU oracle, plus the GPU-internal
bit-for-bit invariants (pair == separate + SwiGLU, batch invariance, column-range
slice == zero-padded full row, row slice == rows of the full product, grouped ==
per-route products, graph replay == eager, repeat determinism).

Inputs come from the seeded generators only; the oracle never consumes GPU data.
Bars: bytes/ids/integer dots bit-exact; products <= 1e-5*max(1,|ref|); SwiGLU,
weights and combine <= 1e-4*max(1,|ref|).
"""

import json
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import workloads  # noqa: E402
import quantized_moe_expert_q8_amd as moeq8  # noqa: E402
from _gpu import DEV, assert_close, bits_equal, host, q80_from_dev, q81_from_dev, say, to_dev  # noqa: E402

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
PROD_TOL = 1e-5
EPI_TOL = 1e-4


def synth_matrix(seed, n, k, matrix=0, expert=0, layer=0):
    """Same generator bytes for both sides: (numpy Q8_0 array, device tensor)."""
    w = workloads.synth_q8_0_matrix(seed, layer, expert, matrix, n, k)
    return w, to_dev(w)


def quantized_pair(x32):
    """Quantise x on both sides; assert identical bytes; return (oracle, device)."""
    xo = oracle.quantize_q8_1(x32)
    xd = moeq8.q8_1_quantize_rows(to_dev(x32))
    torch.cuda.synchronize()
    assert host(xd).tobytes() == xo.tobytes()
    return xo, xd


# ---------------------------------------------------------------------------
# a1 / a7: quantisers
# ---------------------------------------------------------------------------

def test_quantize_golden_blocks():
    say("quantize golden")
    with open(os.path.join(GOLDEN, "q8_blocks_worked.json")) as f:
        cases = json.load(f)["cases"]
    x = np.stack([np.array(c["x"], np.float32) for c in cases])
    q1 = host(moeq8.q8_1_quantize_rows(to_dev(x)))
    q0 = host(moeq8.q8_0_quantize_rows(to_dev(x)))
    for i, c in enumerate(cases):
        assert q1[i].tobytes().hex() == c["q8_1_hex"].replace(" ", ""), c["name"]
        assert q0[i].tobytes().hex() == c["q8_0_hex"].replace(" ", ""), c["name"]


@pytest.mark.parametrize("rows,k", [(1, 32), (3, 256), (37, 4096), (64, 1024), (5, 2048)])
def test_quantize_bit_exact(rows, k):
    say(f"quantize rows={rows} k={k}")
    x = workloads.normal_f32(rows * 31 + k, (rows, k), 1.0)
    if rows > 2:
        x[0, :64 if k >= 64 else k] = 0.0                  # all-zero blocks
        x[1, :] *= np.float32(1e-30)                       # values near the fp32 subnormal range
        x[2, :32] = np.arange(-16, 16, dtype=np.float32) + np.float32(0.5)  # exact halves
    xd = to_dev(x)
    assert host(moeq8.q8_1_quantize_rows(xd)).tobytes() == oracle.quantize_q8_1(x).tobytes()
    assert host(moeq8.q8_0_quantize_rows(xd)).tobytes() == oracle.quantize_q8_0(x).tobytes()


def test_quantize_strided_rows_and_discriminating_blocks():
    with open(os.path.join(GOLDEN, "q8_rule_discriminating_blocks.json")) as f:
        blocks = json.load(f)["blocks_hex"]
    b = np.array([[float.fromhex(h) for h in r] for r in blocks], np.float32)
    wide = np.zeros((3, 96), np.float32)
    wide[:, :32] = b
    wide[:, 32:] = 7.0                                   # beyond k: must not be read
    xd = to_dev(wide)[:, :64]
    got = host(moeq8.q8_1_quantize_rows(xd))
    ref = oracle.quantize_q8_1(wide[:, :64])
    assert got.tobytes() == ref.tobytes()


# ---------------------------------------------------------------------------
# a3: single product
# ---------------------------------------------------------------------------

def test_integer_block_dots_unit_scale():
    """All d = 1: y is the integer dot itself, exactly (|y| < 2^24)."""
    say("unit-scale integer dots")
    rng = np.random.default_rng(5)
    n, k, c = 70, 1024, 3
    w = np.zeros((n, k // 32), dtype=oracle.Q8_0_DTYPE)
    w["d"] = 1.0
    w["qs"] = rng.integers(-127, 128, size=w["qs"].shape)
    xq = np.zeros((c, k // 32), dtype=oracle.Q8_1_DTYPE)
    xq["d"] = 1.0
    xq["qs"] = rng.integers(-127, 128, size=xq["qs"].shape)
    xq["qs"][2] = 127
    w["qs"][0] = 127
    y = host(moeq8.mmvq_q8_0(to_dev(w), to_dev(xq), n, k))
    exact = xq["qs"].reshape(c, -1).astype(np.int64) @ w["qs"].reshape(n, -1).astype(np.int64).T
    assert np.array_equal(y.astype(np.int64), exact)
    assert y[2, 0] == 127 * 127 * 1024


@pytest.mark.parametrize("n,k,c", [(1, 64, 1), (5, 256, 3), (63, 1024, 8), (65, 2048, 2),
                                   (300, 4096, 5), (33, 3072, 4), (17, 8192, 1), (129, 1024, 7)])
def test_mmvq_vs_oracle(n, k, c):
    say(f"mmvq n={n} k={k} c={c}")
    w, wd = synth_matrix(n + k, n, k)
    xo, xd = quantized_pair(workloads.normal_f32(c * 17 + k, (c, k)))
    y = host(moeq8.mmvq_q8_0(wd, xd, n, k))
    assert_close(y, oracle.mmvq(w, xo), PROD_TOL, "mmvq")


# ---------------------------------------------------------------------------
# a2: gate/up pair + SwiGLU-DS4, and the pages' invariants
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,k,c", [(512, 256, 1), (100, 4096, 8), (2048, 4096, 5), (64, 1024, 3)])
def test_pair_vs_oracle_and_separate(n, k, c):
    say(f"pair n={n} k={k} c={c}")
    wg, wgd = synth_matrix(1, n, k, matrix=0)
    wu, wud = synth_matrix(1, n, k, matrix=1)
    x = workloads.normal_f32(c + 3 * k, (c, k))
    x[0] *= 40.0                                          # drive g, u past the clamp at 7
    xo, xd = quantized_pair(x)
    g = torch.empty((c, n), dtype=torch.float32, device=DEV)
    u = torch.empty_like(g)
    h = moeq8.mmvq_q8_0_glu_pair(wgd, wud, xd, n, k, g_out=g, u_out=u)
    h_ref, g_ref, u_ref = oracle.glu_pair(wg, wu, xo)
    assert_close(host(g), g_ref, PROD_TOL, "gate")
    assert_close(host(u), u_ref, PROD_TOL, "up")
    assert_close(host(h), h_ref, EPI_TOL, "swiglu")
    assert (np.abs(g_ref) > 7).any() and (np.abs(u_ref) > 7).any()
    # fused pair == the products kept apart + the GLU kernel, bit for bit
    g_sep = moeq8.mmvq_q8_0(wgd, xd, n, k)
    u_sep = moeq8.mmvq_q8_0(wud, xd, n, k)
    assert bits_equal(g, g_sep) and bits_equal(u, u_sep)
    assert bits_equal(h, moeq8.swiglu_ds4(g_sep, u_sep))
    h2 = moeq8.mmvq_q8_0_glu_pair(wgd, wud, xd, n, k)    # without the optional outputs
    assert bits_equal(h, h2)


def test_swiglu_kernel_vs_oracle():
    g = workloads.normal_f32(91, (4096,), 6.0)
    u = workloads.normal_f32(92, (4096,), 6.0)
    g[:4] = [7.0, 100.0, -100.0, 0.0]
    h = host(moeq8.swiglu_ds4(to_dev(g), to_dev(u)))
    assert_close(h, oracle.swiglu_ds4(g, u), EPI_TOL, "swiglu_ds4")


@pytest.mark.parametrize("k", [256, 1024, 4096])
def test_batch_invariance(k):
    say(f"batch invariance k={k}")
    n = 96
    wg, wgd = synth_matrix(7, n, k, matrix=0)
    wu, wud = synth_matrix(7, n, k, matrix=1)
    _, xd = quantized_pair(workloads.normal_f32(8 + k, (8, k)))
    h8 = moeq8.mmvq_q8_0_glu_pair(wgd, wud, xd, n, k)
    y8 = moeq8.mmvq_q8_0(wgd, xd, n, k)
    for c in range(1, 9):
        hc = moeq8.mmvq_q8_0_glu_pair(wgd, wud, xd[:c].contiguous(), n, k)
        yc = moeq8.mmvq_q8_0(wgd, xd[:c].contiguous(), n, k)
        assert bits_equal(hc, h8[:c]) and bits_equal(yc, y8[:c]), c
        # a single column alone gives the same bits as inside a batch
        h1 = moeq8.mmvq_q8_0_glu_pair(wgd, wud, xd[c - 1:c].contiguous(), n, k)
        assert bits_equal(h1, h8[c - 1:c])


@pytest.mark.parametrize("k,kb_off,kslice", [(4096, 0, 2048), (4096, 64, 2048), (2048, 0, 1024),
                                             (2048, 32, 1024), (1024, 16, 512), (4096, 2, 1024),
                                             (4096, 38, 2048), (1024, 0, 1024)])
def test_column_range_slice_equals_zero_padded_full(k, kb_off, kslice):
    say(f"column range k={k} off={kb_off} k'={kslice}")
    n = 80
    nb = k // 32
    w, wd = synth_matrix(11, n, k, matrix=2)
    x = workloads.normal_f32(kb_off + kslice, (3, k))
    x_pad = np.zeros_like(x)
    lo, hi = kb_off * 32, kb_off * 32 + kslice
    x_pad[:, lo:hi] = x[:, lo:hi]
    _, xs = quantized_pair(np.ascontiguousarray(x[:, lo:hi]))
    _, xpad = quantized_pair(x_pad)
    row_bytes = nb * 34
    y_slice = moeq8.mmvq_q8_0(wd, xs, n, kslice, k_block_offset=kb_off, w_offset_bytes=kb_off * 34,
                              w_row_stride_bytes=row_bytes)
    y_full = moeq8.mmvq_q8_0(wd, xpad, n, k)
    assert bits_equal(y_slice, y_full)
    # the pair keeps the same lanes
    wu, wud = synth_matrix(11, n, k, matrix=3)
    h_slice = moeq8.mmvq_q8_0_glu_pair(wd, wud, xs, n, kslice, k_block_offset=kb_off,
                                       w_offset_bytes=kb_off * 34, w_row_stride_bytes=row_bytes)
    h_full = moeq8.mmvq_q8_0_glu_pair(wd, wud, xpad, n, k)
    assert bits_equal(h_slice, h_full)
    # and the slice matches the oracle's column-range product
    xo = oracle.quantize_q8_1(np.ascontiguousarray(x[:, lo:hi]))
    assert_close(host(y_slice), oracle.mmvq_column_range(w, xo, kb_off), PROD_TOL, "slice")


def test_row_slice_equals_rows_of_full():
    n, k = 2048, 4096
    w, wd = synth_matrix(12, n, k, matrix=0)
    wu, wud = synth_matrix(12, n, k, matrix=1)
    _, xd = quantized_pair(workloads.normal_f32(13, (8, k)))
    h_full = moeq8.mmvq_q8_0_glu_pair(wd, wud, xd, n, k)
    row_bytes = (k // 32) * 34
    for r0, nr in [(0, 1024), (1024, 1024), (5, 77)]:
        h_rows = moeq8.mmvq_q8_0_glu_pair(wd, wud, xd, nr, k, w_offset_bytes=r0 * row_bytes,
                                          w_row_stride_bytes=row_bytes)
        assert bits_equal(h_rows, h_full[:, r0:r0 + nr].contiguous())


def test_repeat_determinism():
    n, k = 1024, 4096
    _, wd = synth_matrix(14, n, k)
    _, wud = synth_matrix(14, n, k, matrix=1)
    _, xd = quantized_pair(workloads.normal_f32(15, (5, k)))
    a = moeq8.mmvq_q8_0_glu_pair(wd, wud, xd, n, k)
    for _ in range(3):
        assert bits_equal(a, moeq8.mmvq_q8_0_glu_pair(wd, wud, xd, n, k))


# ---------------------------------------------------------------------------
# a4 / a5: router + grouping
# ---------------------------------------------------------------------------

def _grouping_words(gt):
    return host(gt).view(np.int32)


def _defined_grouping_words(gt):
    """The words a grouping defines: header, expert[R], offset[R+1], route[R]
    and the table entries of the active groups (padding and unused entries
    hold whatever the buffer held before)."""
    words = _grouping_words(gt)
    R = int(words[2]) * int(words[3])
    t0 = (4 + 3 * R + 1 + 8 + 3) // 4 * 4
    return (list(words[:4 + 3 * R + 1]), list(words[t0:t0 + 4 * int(words[0])]))


def _check_grouping(words, ids_ref):
    R = ids_ref.size
    n_active, n_valid, ncols, topk = words[:4]
    groups = oracle.group_routes(ids_ref)
    assert n_active == len(groups) and ncols * topk == R
    assert n_valid == int((ids_ref >= 0).sum())
    expert = words[4:4 + R]
    offset = words[4 + R:4 + 2 * R + 1]
    route = words[4 + 2 * R + 1:4 + 3 * R + 1]
    # per-group table {expert, first route, end, 0} at a 16-byte boundary
    # after route[] and eight words of padding
    t0 = (4 + 3 * R + 1 + 8 + 3) // 4 * 4
    table = words[t0:t0 + 4 * R].reshape(R, 4)
    for a, (e, routes) in enumerate(groups):
        assert expert[a] == e
        assert list(route[offset[a]:offset[a + 1]]) == routes
        assert list(table[a]) == [e, offset[a], offset[a + 1], 0]


@pytest.mark.parametrize("c,n_exp,topk,local", [(1, 256, 8, 256), (5, 256, 8, 256), (8, 256, 8, 128),
                                                (8, 64, 6, 64), (3, 1024, 16, 512), (2, 8, 8, 8),
                                                (8, 256, 16, 256), (5, 64, 16, 20), (7, 100, 10, 100)])
def test_route_topk_vs_oracle(c, n_exp, topk, local):
    say(f"route c={c} E={n_exp} k={topk} local={local}")
    logits = workloads.router_logits(c + n_exp, c, n_exp)
    bias = workloads.router_bias(c + n_exp, n_exp)
    own = None if local == n_exp else workloads.owner_slots(n_exp, local)
    ids_ref, w_ref, _ = oracle.route_topk(logits, bias, own, topk)
    ids, w, grouping = moeq8.moe_route_topk(to_dev(logits), topk, bias=to_dev(bias),
                                            owner_slot=None if own is None else to_dev(own),
                                            n_local_expert=local)
    assert np.array_equal(host(ids), ids_ref)
    assert_close(host(w), w_ref, EPI_TOL, "route weights")
    assert np.abs(host(w).astype(np.float64) - w_ref).max() < 1e-6
    _check_grouping(_grouping_words(grouping), ids_ref)


def test_route_ties_and_no_bias():
    logits = np.zeros((2, 256), np.float32)
    ids, w, _ = moeq8.moe_route_topk(to_dev(logits), 8)
    assert np.array_equal(host(ids), np.tile(np.arange(8, dtype=np.int32), (2, 1)))
    assert np.all(host(w) == np.float32(0.125))
    lg = np.full((1, 16), -5.0, np.float32)
    top = [3, 9, 1, 12, 7, 0, 14]
    for r, e in enumerate(top):
        lg[0, e] = 4.0 - 0.5 * r
    lg[0, 11] = lg[0, 5] = -1.0
    ids, _, _ = moeq8.moe_route_topk(to_dev(lg), 8)
    assert list(host(ids)[0]) == top + [5]


def test_route_all_masked():
    logits = workloads.router_logits(3, 4, 256)
    own = np.full(256, -1, np.int32)
    own[200] = 0                                           # one local expert that is never picked
    logits[:, 200] = -50.0
    ids, w, grouping = moeq8.moe_route_topk(to_dev(logits), 8, owner_slot=to_dev(own), n_local_expert=1)
    assert np.all(host(ids) == -1)
    words = _grouping_words(grouping)
    assert words[0] == 0 and words[1] == 0


# ---------------------------------------------------------------------------
# a6 / a8 / a9: grouped products and the combine
# ---------------------------------------------------------------------------

def _tiny_layer(seed, n_local, hidden, inter):
    wg = np.stack([workloads.synth_q8_0_matrix(seed, 0, e, 0, inter, hidden) for e in range(n_local)])
    wu = np.stack([workloads.synth_q8_0_matrix(seed, 0, e, 1, inter, hidden) for e in range(n_local)])
    wdn = np.stack([workloads.synth_q8_0_matrix(seed, 0, e, 2, hidden, inter) for e in range(n_local)])
    dev = [to_dev(a.reshape(-1)).reshape(-1) for a in (wg, wu, wdn)]
    return (wg, wu, wdn), dev


@pytest.mark.parametrize("c,n_exp,local,hidden,inter", [(1, 32, 32, 1024, 256), (5, 16, 16, 2048, 512),
                                                        (8, 64, 32, 1024, 1024), (8, 4, 4, 256, 128)])
def test_grouped_gate_up_down_combine(c, n_exp, local, hidden, inter):
    say(f"grouped c={c} E={n_exp} local={local} hidden={hidden} inter={inter}")
    topk = min(8, n_exp)
    (wg, wu, wdn), (wgd, wud, wdd) = _tiny_layer(c + local, local, hidden, inter)
    x = workloads.activations(c, c, hidden)
    logits = workloads.router_logits(c, c, n_exp)
    bias = workloads.router_bias(c, n_exp)
    own = workloads.owner_slots(n_exp, local)
    xo, xd = quantized_pair(x)
    ids, w, grouping = moeq8.moe_route_topk(to_dev(logits), topk, bias=to_dev(bias),
                                            owner_slot=to_dev(own), n_local_expert=local)
    ids_ref, w_ref, _ = oracle.route_topk(logits, bias, own, topk)
    assert np.array_equal(host(ids), ids_ref)

    # gate/up: each route's h against the oracle and against the pair on that expert
    h = torch.full((c, topk, inter), float("nan"), device=DEV)
    moeq8.moe_grouped_mmvq(moeq8.GATE_UP_SWIGLU, wgd, wud, xd, grouping, n=inter, k=hidden,
                           n_local_expert=local, ncols=c, topk=topk, out=h)
    hh = host(h)
    row_b = (hidden // 32) * 34
    for j in range(c):
        for s in range(topk):
            e = ids_ref[j, s]
            if e < 0:
                assert np.isnan(hh[j, s]).all()              # masked rows untouched
                continue
            h_ref, _, _ = oracle.glu_pair(wg[e], wu[e], xo[j:j + 1])
            assert_close(hh[j, s], h_ref[0], EPI_TOL, f"grouped h ({j},{s})")
            hp = moeq8.mmvq_q8_0_glu_pair(wgd, wud, xd[j:j + 1].contiguous(), inter, hidden,
                                          w_offset_bytes=int(e) * inter * row_b, w_row_stride_bytes=row_b)
            assert bits_equal(h[j, s:s + 1].contiguous(), hp)

    # a7 on the oracle's h: the GPU quantiser gives the oracle's bytes
    h_ref32 = np.zeros((c * topk, inter), np.float32)
    for j in range(c):
        for s in range(topk):
            if ids_ref[j, s] >= 0:
                h_ref32[j * topk + s] = oracle.glu_pair(wg[ids_ref[j, s]], wu[ids_ref[j, s]],
                                                        xo[j:j + 1])[0][0].astype(np.float32)
    hq_dev = moeq8.q8_1_quantize_rows(to_dev(h_ref32))
    hq_ref_all = oracle.quantize_q8_1(h_ref32)
    assert host(hq_dev).tobytes() == hq_ref_all.tobytes()

    # down on the oracle's hq
    y = torch.full((c, topk, hidden), float("nan"), device=DEV)
    moeq8.moe_grouped_mmvq(moeq8.DOWN, wdd, None, hq_dev, grouping, n=hidden, k=inter,
                           n_local_expert=local, ncols=c, topk=topk, out=y)
    yy = host(y)
    y_ref = np.zeros((c, topk, hidden))
    row_d = (inter // 32) * 34
    for j in range(c):
        for s in range(topk):
            e = ids_ref[j, s]
            if e < 0:
                assert np.isnan(yy[j, s]).all()
                continue
            y_ref[j, s] = oracle.mmvq(wdn[e], hq_ref_all[j * topk + s:j * topk + s + 1])[0]
            assert_close(yy[j, s], y_ref[j, s], PROD_TOL, f"grouped y ({j},{s})")
            ys = moeq8.mmvq_q8_0(wdd, hq_dev[j * topk + s:j * topk + s + 1].contiguous(), hidden, inter,
                                 w_offset_bytes=int(e) * hidden * row_d, w_row_stride_bytes=row_d)
            assert bits_equal(y[j, s:s + 1].contiguous(), ys)

    # combine on the oracle's y and weights (masked slots hold NaN, which must not reach the output)
    y32 = np.where(ids_ref[..., None] >= 0, y_ref, np.nan).astype(np.float32)
    w32 = w_ref.astype(np.float32)
    out = host(moeq8.moe_combine(to_dev(y32), ids, to_dev(w32)))
    assert_close(out, oracle.moe_combine(y32.astype(np.float64), ids_ref, w32.astype(np.float64)),
                 EPI_TOL, "combine")
    assert np.isfinite(out).all()


def test_combine_one_hot_and_all_masked():
    rng = np.random.default_rng(2)
    y = rng.normal(size=(3, 8, 4096)).astype(np.float32)
    ids = np.array([[0, 1, 2, 3, 4, 5, 6, 7], [-1] * 8, [1, -1, 2, -1, 3, -1, 4, -1]], np.int32)
    w = np.zeros((3, 8), np.float32)
    w[0, 5] = 1.0
    w[2] = 0.125
    y[2, 1] = np.nan
    out = host(moeq8.moe_combine(to_dev(y), to_dev(ids), to_dev(w)))
    assert np.array_equal(out[0], y[0, 5])
    assert np.all(out[1] == 0.0)
    ref = np.float32(0.125) * y[2, 0]
    for s in (2, 4, 6):
        ref = ref + np.float32(0.125) * y[2, s]
    assert np.array_equal(out[2], ref)                     # fp32: products rounded, sums in slot order


def test_combine_shared_adds_after_the_routed_sum():
    """moe_combine_shared = the routed combine, then one fp32 add of the shared
    expert's output (R15): bit for bit against the plain combine plus the
    shared output on the host, in place (shared is out) too; all masked gives
    the shared output itself; within tolerance of the oracle."""
    rng = np.random.default_rng(3)
    c, topk, n = 5, 8, 4096
    y = rng.normal(size=(c, topk, n)).astype(np.float32)
    ids = rng.integers(-1, 20, size=(c, topk)).astype(np.int32)
    ids[1] = -1
    w = rng.random((c, topk)).astype(np.float32)
    shared = rng.normal(size=(c, n)).astype(np.float32)
    y[ids < 0] = np.nan
    yd, idd, wd, sd = to_dev(y), to_dev(ids), to_dev(w), to_dev(shared)
    plain = host(moeq8.moe_combine(yd, idd, wd))
    got = host(moeq8.moe_combine(yd, idd, wd, shared=sd))
    assert np.array_equal(got.view(np.int32), (plain + shared).view(np.int32))
    assert np.array_equal(got[1].view(np.int32), shared[1].view(np.int32))
    inplace = sd.clone()
    moeq8.moe_combine(yd, idd, wd, out=inplace, shared=inplace)
    assert np.array_equal(host(inplace).view(np.int32), got.view(np.int32))
    ref = oracle.moe_combine(np.nan_to_num(y.astype(np.float64)), ids, w.astype(np.float64),
                             shared=shared.astype(np.float64))
    assert_close(got, ref, EPI_TOL, "combine + shared")


def test_graph_replay_matches_eager():
    """One routed layer captured in a HIP graph and replayed several times, with
    eager work and synchronisation between replays, equals the eager run."""
    say("graph replay")
    c, n_exp, hidden, inter, topk = 5, 32, 1024, 256, 8
    (_, _, _), (wgd, wud, wdd) = _tiny_layer(21, n_exp, hidden, inter)
    xd = to_dev(workloads.activations(21, c, hidden))
    lg = to_dev(workloads.router_logits(21, c, n_exp))
    bias = to_dev(workloads.router_bias(21, n_exp))
    xq = torch.empty((c, hidden // 32 * 36), dtype=torch.uint8, device=DEV)
    ids = torch.empty((c, topk), dtype=torch.int32, device=DEV)
    w = torch.empty((c, topk), dtype=torch.float32, device=DEV)
    grouping = torch.empty(moeq8.moe_grouping_bytes(c, topk), dtype=torch.uint8, device=DEV)
    h = torch.empty((c, topk, inter), dtype=torch.float32, device=DEV)
    hq = torch.empty((c * topk, inter // 32 * 36), dtype=torch.uint8, device=DEV)
    y = torch.empty((c, topk, hidden), dtype=torch.float32, device=DEV)
    out = torch.empty((c, hidden), dtype=torch.float32, device=DEV)

    def layer():
        moeq8.q8_1_quantize_rows(xd, out=xq)
        moeq8.moe_route_topk(lg, topk, bias=bias, ids=ids, weights=w, grouping=grouping)
        moeq8.moe_grouped_mmvq(moeq8.GATE_UP_SWIGLU, wgd, wud, xq, grouping, n=inter, k=hidden,
                               n_local_expert=n_exp, ncols=c, topk=topk, out=h)
        moeq8.q8_1_quantize_rows(h.view(c * topk, inter), out=hq)
        moeq8.moe_grouped_mmvq(moeq8.DOWN, wdd, None, hq, grouping, n=hidden, k=inter,
                               n_local_expert=n_exp, ncols=c, topk=topk, out=y)
        moeq8.moe_combine(y, ids, w, out=out)

    layer()
    torch.cuda.synchronize()
    ref = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer()
    for i in range(4):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert bits_equal(out, ref), i
        layer()                                            # eager work between replays
        torch.cuda.synchronize()
        assert bits_equal(out, ref)


def test_synth_fill_matches_host_generator():
    n_mats, bpm = 3, 4096
    dst = torch.empty(n_mats * bpm * 34, dtype=torch.uint8, device=DEV)
    moeq8.synth_q8_0_fill(dst, n_mats, bpm, 2, seed=5, layer0=7, expert0=3, matrix=2)
    got = host(dst)
    for i in range(n_mats):
        ref = workloads.synth_q8_0_blocks(workloads.stream_key(5, 7 + i // 2, 3 + i % 2, 2), 0, bpm)
        assert got[i * bpm * 34:(i + 1) * bpm * 34].tobytes() == ref.tobytes()


# ---------------------------------------------------------------------------
# fused launches == the separate calls, bit for bit
# ---------------------------------------------------------------------------

def test_route_topk_quantize_equals_separate():
    c, n_exp, hidden, topk = 8, 256, 4096, 8
    x = to_dev(workloads.activations(31, c, hidden))
    lg = to_dev(workloads.router_logits(31, c, n_exp))
    b = to_dev(workloads.router_bias(31, n_exp))
    own = to_dev(workloads.owner_slots(n_exp, 128))
    xq, ids, w, g = moeq8.moe_route_topk_quantize(x, lg, topk, bias=b, owner_slot=own, n_local_expert=128)
    ids2, w2, g2 = moeq8.moe_route_topk(lg, topk, bias=b, owner_slot=own, n_local_expert=128)
    assert torch.equal(xq, moeq8.q8_1_quantize_rows(x))
    assert torch.equal(ids, ids2) and bits_equal(w, w2)
    assert _defined_grouping_words(g) == _defined_grouping_words(g2)


@pytest.mark.parametrize("c,n_exp,hidden,inter,share_rows,half", [(8, 32, 1024, 256, 512, 0),
                                                                  (8, 32, 1024, 256, 512, 1),
                                                                  (5, 16, 2048, 1024, 1024, 1),
                                                                  (1, 8, 4096, 1024, 1024, 0)])
def test_fused_layer_equals_unfused(c, n_exp, hidden, inter, share_rows, half):
    """The four-launch layer (prologue, gate/up + shared rows, down with
    in-launch q8_1 of h and hs + shared slice, combine) against the nine
    separate calls, every output bit for bit."""
    from quantized_moe_expert_q8_amd import moe_layer as ml
    say(f"fused layer c={c} E={n_exp} H={hidden} I={inter} share={share_rows} half={half}")
    topk = 8 if n_exp >= 8 else n_exp
    _, (wgd, wud, wdd) = _tiny_layer(c + n_exp, n_exp, hidden, inter)
    inter_full = 2 * share_rows
    rb_h, rb_f = hidden // 32 * 34, inter_full // 32 * 34
    sg = to_dev(workloads.synth_q8_0_matrix(3, 0, 0, 3, inter_full, hidden)).reshape(inter_full, rb_h)
    su = to_dev(workloads.synth_q8_0_matrix(3, 0, 0, 4, inter_full, hidden)).reshape(inter_full, rb_h)
    sd = to_dev(workloads.synth_q8_0_matrix(3, 0, 0, 5, hidden, inter_full)).reshape(hidden, rb_f)
    shared = ml.SharedExpertShare(sg, su, sd, hidden, inter_full, half * share_rows, share_rows)
    experts = ml.RoutedExperts(wgd, wud, wdd, n_exp, hidden, inter)
    x = to_dev(workloads.activations(c, c, hidden))
    lg = to_dev(workloads.router_logits(c, c, n_exp))
    b = to_dev(workloads.router_bias(c, n_exp))
    own = to_dev(workloads.owner_slots(n_exp, n_exp // 2))
    wa = ml.Workspace(c, hidden, inter, topk, share_rows, DEV)
    wb = ml.Workspace(c, hidden, inter, topk, share_rows, DEV)
    ml.forward(x, lg, b, own, n_exp // 2, experts, shared, wa, fused=False)
    ml.forward(x, lg, b, own, n_exp // 2, experts, shared, wb, fused=True)
    torch.cuda.synchronize()
    # with the shared expert's output added inside the combine: both forms
    # agree, and the total is the routed sum plus ys in one fp32 add
    wc = ml.Workspace(c, hidden, inter, topk, share_rows, DEV)
    wd = ml.Workspace(c, hidden, inter, topk, share_rows, DEV)
    ml.forward(x, lg, b, own, n_exp // 2, experts, shared, wc, fused=False, add_shared=True)
    ml.forward(x, lg, b, own, n_exp // 2, experts, shared, wd, fused=True, add_shared=True)
    torch.cuda.synchronize()
    assert bits_equal(wc.out, wd.out)
    total = host(wb.out) + host(wb.ys)
    assert np.array_equal(host(wd.out).view(np.int32), total.view(np.int32))
    assert torch.equal(wa.xq, wb.xq) and torch.equal(wa.ids, wb.ids)
    assert _defined_grouping_words(wa.grouping) == _defined_grouping_words(wb.grouping)
    assert bits_equal(wa.weights, wb.weights)
    assert bits_equal(wa.hs, wb.hs) and bits_equal(wa.ys, wb.ys)
    valid = (host(wa.ids) >= 0)
    ha, hb = host(wa.h), host(wb.h)
    ya, yb = host(wa.y), host(wb.y)
    for j in range(c):
        for s in range(topk):
            if valid[j, s]:
                assert np.array_equal(ha[j, s].view(np.int32), hb[j, s].view(np.int32))
                assert np.array_equal(ya[j, s].view(np.int32), yb[j, s].view(np.int32))
    assert bits_equal(wa.out, wb.out)


@pytest.mark.parametrize("c,n_exp,hidden,inter", [(8, 32, 1024, 1024), (3, 16, 2048, 512)])
def test_down_f32_act_equals_quantize_then_down(c, n_exp, hidden, inter):
    """MOEQ8_DOWN_F32_ACT (q8_1 of h inside the launch, shared slice as extra
    items) against q8_1_quantize_rows + MOEQ8_DOWN, bit for bit."""
    topk = 8
    _, (_, _, wdd) = _tiny_layer(5 + c, n_exp, hidden, inter)
    lg = to_dev(workloads.router_logits(c + 1, c, n_exp))
    ids, w, grouping = moeq8.moe_route_topk(lg, topk)
    h = to_dev(workloads.normal_f32(77, (c * topk, inter), 2.0))
    hs = to_dev(workloads.normal_f32(78, (c, inter), 2.0))
    inter_full = 2 * inter
    sd = to_dev(workloads.synth_q8_0_matrix(3, 0, 0, 5, hidden, inter_full)).reshape(hidden, -1)
    rbf = inter_full // 32 * 34
    for half in (0, 1):
        kb = half * inter // 32
        y1 = torch.full((c, topk, hidden), float("nan"), device=DEV)
        ys1 = torch.empty((c, hidden), device=DEV)
        moeq8.moe_grouped_mmvq_ex(moeq8.DOWN_F32_ACT, wdd, None, h, grouping, n=hidden, k=inter,
                                  n_local_expert=n_exp, ncols=c, topk=topk, out=y1,
                                  shared={"a": sd, "row_stride": rbf, "n": hidden, "k": inter,
                                          "k_block_offset": kb, "offset_bytes": kb * 34,
                                          "out": ys1, "act": hs})
        hq, hsq = moeq8.q8_1_quantize_rows(h), moeq8.q8_1_quantize_rows(hs)
        y2 = torch.full((c, topk, hidden), float("nan"), device=DEV)
        moeq8.moe_grouped_mmvq(moeq8.DOWN, wdd, None, hq, grouping, n=hidden, k=inter,
                               n_local_expert=n_exp, ncols=c, topk=topk, out=y2)
        ys2 = moeq8.mmvq_q8_0(sd, hsq, hidden, inter, k_block_offset=kb, w_offset_bytes=kb * 34,
                              w_row_stride_bytes=rbf)
        assert np.array_equal(host(y1).view(np.int32), host(y2).view(np.int32))
        assert bits_equal(ys1, ys2)


def test_fused_layer_all_routes_masked():
    """A layer whose routes are all masked writes a zero combine on the fused
    path, as on the separate calls."""
    from quantized_moe_expert_q8_amd import moe_layer as ml
    c, n_exp, hidden, inter, topk = 4, 16, 1024, 256, 8
    _, (wgd, wud, wdd) = _tiny_layer(44, n_exp, hidden, inter)
    experts = ml.RoutedExperts(wgd, wud, wdd, n_exp, hidden, inter)
    x = to_dev(workloads.activations(44, c, hidden))
    lg = workloads.router_logits(44, c, n_exp)
    own = np.full(n_exp, -1, np.int32)
    own[15] = 0
    lg[:, 15] = -60.0                                     # never selected: every route masked
    ws = ml.Workspace(c, hidden, inter, topk, 0, DEV)
    ws.out.fill_(float("nan"))
    out, _ = ml.forward(x, to_dev(lg), None, to_dev(own), 1, experts, None, ws)
    torch.cuda.synchronize()
    assert np.all(host(ws.ids) == -1)
    assert np.all(host(out) == 0.0)


# ---------------------------------------------------------------------------
# the 64-chunk packed layout of the gate/up weights
# ---------------------------------------------------------------------------

def _p64_reference(raw: np.ndarray, rows: int, k: int) -> np.ndarray:
    """The packed layout restated on the host: within each 4352-byte segment of
    a row, dword 17c + d moves to 256*(d//4) + 4c + d%4 (d < 16) and dword
    17c + 16 to 1024 + c."""
    w = np.ascontiguousarray(raw).reshape(-1).view(np.uint32).reshape(rows, k // 4096, 1088)
    out = np.empty_like(w)
    c = np.arange(64)
    for d in range(16):
        out[:, :, 256 * (d // 4) + 4 * c + d % 4] = w[:, :, 17 * c + d]
    out[:, :, 1024 + c] = w[:, :, 17 * c + 16]
    return out.reshape(-1).view(np.uint8)


@pytest.mark.parametrize("rows,k", [(1, 4096), (3, 8192), (64, 4096)])
def test_pack64_layout(rows, k):
    raw = np.random.default_rng(rows + k).integers(0, 256, size=rows * (k // 32) * 34, dtype=np.uint8)
    got = host(moeq8.q8_0_pack64_rows(to_dev(raw), rows, k))
    assert np.array_equal(got, _p64_reference(raw, rows, k))
    # and every byte is kept: the packing only permutes within a segment
    assert np.array_equal(np.sort(got.reshape(rows, -1), axis=1), np.sort(raw.reshape(rows, -1), axis=1))


def _rounds_reference(raw: np.ndarray, rows: int, k: int, stride: int) -> np.ndarray:
    """The round-major four-row packed layout restated on the host: round r of
    every row goes to matrix r of contiguous 1088-byte rows, where the 4352
    bytes of rows 4q..4q+3 are permuted as one 64-chunk segment (packed dword
    256*(d//4) + 4c + d%4 takes unit dword 17c + d, packed dword 1024 + c takes
    17c + 16; unit dword 272g + i is dword i of row 4q + g's round)."""
    src = np.ascontiguousarray(raw).reshape(-1).view(np.uint32).reshape(rows, stride // 4)
    c = np.arange(64)
    perm = np.empty(1088, np.int64)
    for d in range(16):
        perm[256 * (d // 4) + 4 * c + d % 4] = 17 * c + d
    perm[1024 + c] = 17 * c + 16
    out = []
    for r in range(k // 1024):
        rnd = src[:, r * 272:(r + 1) * 272]                   # [rows][272]
        units = rnd.reshape(rows // 4, 1088)
        out.append(units[:, perm].reshape(-1))
    return np.concatenate(out).view(np.uint8)


@pytest.mark.parametrize("rows,k,extra", [(4, 1024, 0), (8, 2048, 0), (12, 1024, 1088)])
def test_pack64_rounds_layout(rows, k, extra):
    stride = k // 32 * 34 + extra
    raw = np.random.default_rng(rows + k + extra).integers(0, 256, size=rows * stride, dtype=np.uint8)
    got = host(moeq8.q8_0_pack64_rounds(to_dev(raw), rows, k, src_row_stride_bytes=stride))
    assert np.array_equal(got, _rounds_reference(raw, rows, k, stride))


def _synth_dev(seed, n_mats, rows, k, matrix, layer=0):
    t = torch.empty(n_mats * rows * (k // 32) * 34, dtype=torch.uint8, device=DEV)
    moeq8.synth_q8_0_fill(t, n_mats, rows * k // 32, n_mats, seed, layer, 0, matrix)
    return t


def _route_any(lg, topk, c, n_exp, local, bias=None):
    """ids, weights and the grouping of c columns: one launch up to 8 columns,
    the wide router and the grouping launch beyond."""
    own = to_dev(workloads.owner_slots(n_exp, local))
    if c <= 8:
        return moeq8.moe_route_topk(lg, topk, bias=bias, owner_slot=own, n_local_expert=local)
    ids, w = moeq8.moe_route_topk_wide(lg, topk, bias=bias, owner_slot=own, n_local_expert=local)
    return ids, w, moeq8.moe_group_routes(ids, local)


@pytest.mark.parametrize("c,n_exp,local,inter,share_rows,half", [(1, 32, 32, 256, 0, 0),
                                                                 (5, 64, 32, 512, 256, 1),
                                                                 (8, 32, 16, 1024, 512, 0),
                                                                 (3, 16, 16, 72, 40, 1),
                                                                 (24, 16, 8, 256, 256, 1)])
def test_grouped_gate_up_p64_equals_plain(c, n_exp, local, inter, share_rows, half):
    """GATE_UP_SWIGLU_P64 on packed copies against GATE_UP_SWIGLU on the plain
    weights, every written h and hs row bit for bit (owner mask, ragged row
    counts, the shared rows at either half; 24 columns: a wide grouping, whose
    launch takes the packed kernel's ordinary-load form and several passes)."""
    say(f"p64 gate/up c={c} E={n_exp} local={local} inter={inter} share={share_rows} half={half}")
    H, topk, seed = 4096, 8, 60 + c
    wg, wu = _synth_dev(seed, local, inter, H, 0), _synth_dev(seed, local, inter, H, 1)
    pg = moeq8.q8_0_pack64_rows(wg, local * inter, H)
    pu = moeq8.q8_0_pack64_rows(wu, local * inter, H)
    x = to_dev(workloads.activations(seed, c, H))
    xq = moeq8.q8_1_quantize_rows(x)
    lg = to_dev(workloads.router_logits(seed, c, n_exp))
    ids, w, grouping = _route_any(lg, topk, c, n_exp, local, bias=to_dev(workloads.router_bias(seed, n_exp)))
    rb = H // 32 * 34
    outs = []
    for stage, a, b in ((moeq8.GATE_UP_SWIGLU, wg, wu), (moeq8.GATE_UP_SWIGLU_P64, pg, pu)):
        h = torch.full((c, topk, inter), float("nan"), device=DEV)
        sh = None
        hs = None
        if share_rows:
            full = 2 * share_rows
            sgp, sup = _synth_dev(seed, 1, full, H, 3), _synth_dev(seed, 1, full, H, 4)
            if stage == moeq8.GATE_UP_SWIGLU_P64:
                sgp, sup = moeq8.q8_0_pack64_rows(sgp, full, H), moeq8.q8_0_pack64_rows(sup, full, H)
            hs = torch.full((c, share_rows), float("nan"), device=DEV)
            sh = {"a": sgp, "b": sup, "row_stride": rb, "n": share_rows, "k": H, "k_block_offset": 0,
                  "offset_bytes": half * share_rows * rb, "out": hs}
        moeq8.moe_grouped_mmvq_ex(stage, a, b, xq, grouping, n=inter, k=H, n_local_expert=local, ncols=c,
                                  topk=topk, out=h, shared=sh)
        outs.append((h, hs))
    torch.cuda.synchronize()
    valid = host(ids) >= 0
    h0, h1 = host(outs[0][0]), host(outs[1][0])
    for j in range(c):
        for s in range(topk):
            if valid[j, s]:
                assert np.array_equal(h0[j, s].view(np.int32), h1[j, s].view(np.int32)), (j, s)
            else:
                assert np.isnan(h1[j, s]).all()          # masked rows untouched
    if share_rows:
        assert bits_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("c,n_exp,local,hidden,half", [(1, 32, 32, 1024, 0), (5, 64, 32, 4096, 1),
                                                      (8, 32, 16, 516, 0), (3, 16, 16, 256, 1),
                                                      (24, 16, 8, 256, 0)])
def test_grouped_down_p64_equals_plain(c, n_exp, local, hidden, half):
    """DOWN_F32_ACT_P64 on round-major packed copies (routed experts, and the
    shared matrix's round for its column-range share) against DOWN_F32_ACT on
    the plain weights with the column-range slice, every written y and ys row
    bit for bit (owner mask, a row count that is not a multiple of the
    workgroup's rows; 24 columns: a wide grouping, the ordinary-load form)."""
    say(f"p64 down c={c} E={n_exp} local={local} hidden={hidden} half={half}")
    topk, seed, inter = 8, 70 + c, 1024
    wd = _synth_dev(seed, local, hidden, inter, 2)
    pd = moeq8.q8_0_pack64_rounds(wd, local * hidden, inter)
    lg = to_dev(workloads.router_logits(seed, c, n_exp))
    ids, w, grouping = _route_any(lg, topk, c, n_exp, local)
    h = to_dev(workloads.normal_f32(seed + 1, (c * topk, inter), 2.0))
    hs = to_dev(workloads.normal_f32(seed + 2, (c, inter), 2.0))
    full = 2 * inter
    rbf = full // 32 * 34
    sd = _synth_dev(seed, 1, hidden, full, 5)
    psd = moeq8.q8_0_pack64_rounds(sd, hidden, full)
    kb = half * inter // 32
    rb = moeq8.ops.ROUND_BYTES
    outs = []
    for stage, a, sh in ((moeq8.DOWN_F32_ACT, wd, {"a": sd, "row_stride": rbf, "k_block_offset": kb,
                                                   "offset_bytes": kb * 34}),
                         (moeq8.DOWN_F32_ACT_P64, pd, {"a": psd, "row_stride": rb, "k_block_offset": 0,
                                                       "offset_bytes": half * hidden * rb})):
        y = torch.full((c, topk, hidden), float("nan"), device=DEV)
        ys = torch.full((c, hidden), float("nan"), device=DEV)
        moeq8.moe_grouped_mmvq_ex(stage, a, None, h, grouping, n=hidden, k=inter, n_local_expert=local,
                                  ncols=c, topk=topk, out=y,
                                  shared=dict(sh, n=hidden, k=inter, out=ys, act=hs))
        outs.append((y, ys))
    torch.cuda.synchronize()
    valid = host(ids) >= 0
    y0, y1 = host(outs[0][0]), host(outs[1][0])
    for j in range(c):
        for s in range(topk):
            if valid[j, s]:
                assert np.array_equal(y0[j, s].view(np.int32), y1[j, s].view(np.int32)), (j, s)
            else:
                assert np.isnan(y1[j, s]).all()
    assert bits_equal(outs[0][1], outs[1][1])


def test_p64_rejects_what_it_cannot_read():
    """Host checks of the packed stage: K other than 4096, a weight pointer or
    a shared slice off the 16-byte / segment grid."""
    c, topk, local, inter = 2, 4, 8, 64
    lg = to_dev(workloads.router_logits(9, c, local))
    ids, w, grouping = moeq8.moe_route_topk(lg, topk)
    h = torch.zeros((c, topk, inter), device=DEV)
    for H, off, status in ((2048, 0, -3), (4096, 4, -2)):
        wt = torch.zeros(local * inter * (H // 32) * 34 + 64, dtype=torch.uint8, device=DEV)
        xq = torch.zeros((c, H // 32 * 36), dtype=torch.uint8, device=DEV)
        a = wt[off:]
        with pytest.raises(moeq8.MoeQ8Error) as ei:
            moeq8.moe_grouped_mmvq_ex(moeq8.GATE_UP_SWIGLU_P64, a, a, xq, grouping, n=inter, k=H,
                                      n_local_expert=local, ncols=c, topk=topk, out=h)
        assert ei.value.status == status
    # the quad-packed down: k read by more than one lane group a row, n not a multiple of 4
    for n, K, status in ((64, 2048, -3), (62, 1024, -3)):
        wt = torch.zeros(local * n * (K // 32) * 34, dtype=torch.uint8, device=DEV)
        hh = torch.zeros((c * topk, K), device=DEV)
        y = torch.zeros((c, topk, n), device=DEV)
        with pytest.raises(moeq8.MoeQ8Error) as ei:
            moeq8.moe_grouped_mmvq_ex(moeq8.DOWN_F32_ACT_P64, wt, None, hh, grouping, n=n, k=K,
                                      n_local_expert=local, ncols=c, topk=topk, out=y)
        assert ei.value.status == status


@pytest.mark.parametrize("c,n_exp", [(1, 16), (5, 32), (8, 32)])
def test_fused_layer_packed_equals_unfused(c, n_exp):
    """The four-launch layer with packed gate/up (routed and shared) against the
    nine separate calls on the plain weights: every output bit for bit."""
    from quantized_moe_expert_q8_amd import moe_layer as ml
    say(f"packed fused layer c={c} E={n_exp}")
    H, I, topk, share_rows = 4096, 1024, 8, 1024     # the packed down reads whole 1024-value rounds
    seed = 80 + c
    wg, wu, wd = _synth_dev(seed, n_exp, I, H, 0), _synth_dev(seed, n_exp, I, H, 1), _synth_dev(seed, n_exp, H, I, 2)
    full = 2 * share_rows
    rb_h, rb_f = H // 32 * 34, full // 32 * 34
    sg = _synth_dev(seed, 1, full, H, 3).view(full, rb_h)
    su = _synth_dev(seed, 1, full, H, 4).view(full, rb_h)
    sd = _synth_dev(seed, 1, H, full, 5).view(H, rb_f)
    experts = ml.RoutedExperts(wg, wu, wd, n_exp, H, I)
    shared = ml.SharedExpertShare(sg, su, sd, H, full, share_rows, share_rows)
    pe, ps = ml.pack_experts(experts, shared)
    x = to_dev(workloads.activations(seed, c, H))
    lg = to_dev(workloads.router_logits(seed, c, n_exp))
    b = to_dev(workloads.router_bias(seed, n_exp))
    own = to_dev(workloads.owner_slots(n_exp, n_exp // 2))
    for add in (False, True):
        wa = ml.Workspace(c, H, I, topk, share_rows, DEV)
        wb = ml.Workspace(c, H, I, topk, share_rows, DEV)
        ml.forward(x, lg, b, own, n_exp // 2, experts, shared, wa, fused=False, add_shared=add)
        ml.forward(x, lg, b, own, n_exp // 2, pe, ps, wb, fused=True, add_shared=add)
        torch.cuda.synchronize()
        assert bits_equal(wa.out, wb.out) and bits_equal(wa.ys, wb.ys) and bits_equal(wa.hs, wb.hs)
        valid = host(wa.ids) >= 0
        ha, hb = host(wa.h), host(wb.h)
        for j in range(c):
            for s in range(topk):
                if valid[j, s]:
                    assert np.array_equal(ha[j, s].view(np.int32), hb[j, s].view(np.int32))
    with pytest.raises(ValueError):
        ml.forward(x, lg, b, own, n_exp // 2, pe, ps, wb, fused=False)
    with pytest.raises(ValueError):                  # the wide GEMM reads the plain layout only
        ml.forward_wide(x, lg, b, own, n_exp // 2, pe, ml.WideWorkspace(c, H, I, topk, DEV), products="gemm")


@pytest.mark.parametrize("c", [3, 40, 1024])
def test_wide_mmvq_packed_equals_plain(c):
    """forward_wide's MMVQ passes on packed experts (the packed stages, h
    quantised inside the down launch) against the plain MMVQ passes: every
    output bit for bit, at wide groupings of several passes of 8 columns up
    to the widest (1024 columns: about 64 passes an expert, the packed
    kernels' ordinary-load form)."""
    from quantized_moe_expert_q8_amd import moe_layer as ml
    say(f"wide mmvq packed c={c}")
    H, I, topk, n_exp, seed = 4096, 1024, 8, 16, 90 + c
    wg, wu, wd = _synth_dev(seed, n_exp, I, H, 0), _synth_dev(seed, n_exp, I, H, 1), _synth_dev(seed, n_exp, H, I, 2)
    experts = ml.RoutedExperts(wg, wu, wd, n_exp, H, I)
    pe, _ = ml.pack_experts(experts)
    x = to_dev(workloads.activations(seed, c, H))
    lg = to_dev(workloads.router_logits(seed, c, n_exp))
    b = to_dev(workloads.router_bias(seed, n_exp))
    wa, wb = ml.WideWorkspace(c, H, I, topk, DEV), ml.WideWorkspace(c, H, I, topk, DEV)
    ml.forward_wide(x, lg, b, None, n_exp, experts, wa, products="mmvq")
    ml.forward_wide(x, lg, b, None, n_exp, pe, wb)                # auto: the MMVQ passes
    torch.cuda.synchronize()
    assert torch.equal(wa.ids, wb.ids)
    assert bits_equal(wa.h, wb.h) and bits_equal(wa.y, wb.y) and bits_equal(wa.out, wb.out)


# ---------------------------------------------------------------------------
# benchmark helper: the streaming-read ceiling reads every word once
# ---------------------------------------------------------------------------

@pytest.mark.gpu
@pytest.mark.parametrize("where", ["first", "last"])
def test_stream_read_reads_every_word(where):
    """A buffer of zeros with one marker word: the xor of the 16-byte piece
    holding it equals the marker, so the sink is written only if that piece
    was read (the size is not a whole number of 64 KB workgroups)."""
    say(f"stream read marker {where}")
    n = 70001 * 16
    buf = torch.zeros(n, dtype=torch.uint8, device=DEV)
    at = 0 if where == "first" else n - 4
    buf[at:at + 4] = torch.tensor([0xB9, 0x79, 0x37, 0x9E], dtype=torch.uint8, device=DEV)
    sink = torch.zeros(4, dtype=torch.uint8, device=DEV)
    moeq8.stream_read(buf, n, sink)
    torch.cuda.synchronize()
    assert int(host(sink.view(torch.int32))[0]) == 0x9E3779B9 - (1 << 32)
    clean = torch.zeros(4, dtype=torch.uint8, device=DEV)
    # the same buffer without the marker's piece: nothing is written
    moeq8.stream_read(buf, n - 16, clean, offset_bytes=16 if where == "first" else 0)
    torch.cuda.synchronize()
    assert int(host(clean.view(torch.int32))[0]) == 0
    # every read shape, the same way
    for wg in moeq8.STREAM_READ_SHAPES:
        sink.zero_()
        clean.zero_()
        moeq8.stream_read_shape(buf, n, wg, sink)
        moeq8.stream_read_shape(buf, n - 16, wg, clean, offset_bytes=16 if where == "first" else 0)
        torch.cuda.synchronize()
        assert int(host(sink.view(torch.int32))[0]) == 0x9E3779B9 - (1 << 32), wg
        assert int(host(clean.view(torch.int32))[0]) == 0, wg


# ---------------------------------------------------------------------------
# wide batches: selection for many columns, the grouping of many routes, and
# the grouped products taking an expert's routes in passes of 8 columns
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("c,n_exp,topk,local", [(1, 256, 8, 256), (9, 256, 8, 128), (64, 256, 8, 128),
                                                (300, 256, 8, 256), (33, 64, 16, 20)])
def test_route_topk_wide_vs_oracle(c, n_exp, topk, local):
    say(f"route wide c={c} E={n_exp} k={topk} local={local}")
    logits = workloads.router_logits(c + 3 * n_exp, c, n_exp)
    bias = workloads.router_bias(c + 3 * n_exp, n_exp)
    own = None if local == n_exp else workloads.owner_slots(n_exp, local)
    ids_ref, w_ref, _ = oracle.route_topk(logits, bias, own, topk)
    ids, w = moeq8.moe_route_topk_wide(to_dev(logits), topk, bias=to_dev(bias),
                                       owner_slot=None if own is None else to_dev(own), n_local_expert=local)
    assert np.array_equal(host(ids), ids_ref)
    assert np.abs(host(w).astype(np.float64) - w_ref).max() < 1e-6
    if c <= 8:
        ids8, w8, g8 = moeq8.moe_route_topk(to_dev(logits), topk, bias=to_dev(bias),
                                            owner_slot=None if own is None else to_dev(own),
                                            n_local_expert=local)
        assert torch.equal(ids, ids8) and bits_equal(w, w8)
        assert _defined_grouping_words(moeq8.moe_group_routes(ids, local)) == _defined_grouping_words(g8)


@pytest.mark.parametrize("c,topk,n_local", [(3, 8, 16), (64, 8, 128), (257, 8, 256), (1024, 8, 1024),
                                            (511, 16, 37)])
def test_group_routes_vs_oracle(c, topk, n_local):
    """The wide grouping against the oracle's grouping (experts ascending,
    routes ascending within each), with masked routes and ids past n_local."""
    say(f"group routes c={c} topk={topk} local={n_local}")
    rng = np.random.default_rng(c + topk)
    ids = np.stack([rng.choice(n_local + 8, size=topk, replace=False) for _ in range(c)]).astype(np.int32)
    ids[rng.random((c, topk)) < 0.2] = -1
    g = moeq8.moe_group_routes(to_dev(ids), n_local)
    # ids at or past n_local count as masked
    _check_grouping(_grouping_words(g), np.where(ids < n_local, ids, -1).astype(np.int32))


def test_router_scores_dense_sweep():
    """Every key the router sorts is score + bias with score = the fp64
    sigmoid rounded once to fp32 (the router's own device expression).  Over a
    dense sweep (2^24 logits evenly spaced over [-24, 24], 2^21 consecutive fp32
    values upward from 0.5 and from -3, and special values) the GPU's scores
    equal the oracle's bit for bit; the two fp64 exp implementations could only
    part where an fp64 sigmoid lies within an ulp or two of an fp32 rounding
    boundary."""
    say("router scores: dense sweep")
    even = np.linspace(-24.0, 24.0, 1 << 24).astype(np.float32)
    runs = [(np.arange(1 << 21, dtype=np.int64) + np.int64(np.float32(v).view(np.int32))).astype(np.int32)
            .view(np.float32) for v in (0.5, -3.0)]
    special = np.array([0.0, -0.0, 1e-30, -1e-30, 1e-45, 16.635532, 88.0, -88.0, 100.0, -100.0, -103.97,
                        1e30, -1e30], np.float32)
    lg = np.concatenate([even] + runs + [special])
    got = host(moeq8.moe_router_scores(to_dev(lg)))
    ref = oracle.sigmoid_f32(lg)
    bad = np.flatnonzero(got.view(np.int32) != ref.view(np.int32))
    assert bad.size == 0, (bad[:8], lg[bad[:8]], got[bad[:8]], ref[bad[:8]])


@pytest.mark.parametrize("c,n_exp,hidden,inter", [(40, 32, 1024, 256), (130, 64, 512, 256)])
def test_wide_grouped_products_vs_oracle(c, n_exp, hidden, inter):
    """Grouped gate/up and down over a wide grouping (items take their routes
    in passes of 8 columns) against the oracle, route by route; the down
    product and the combine read the oracle's h and y."""
    say(f"wide grouped c={c} E={n_exp} H={hidden} I={inter}")
    topk = 8
    (wg, wu, wd), (wgd, wud, wdd) = _tiny_layer(c + n_exp, n_exp, hidden, inter)
    x = workloads.activations(c, c, hidden)
    logits = workloads.router_logits(c + 5, c, n_exp)
    ids_ref, w_ref, _ = oracle.route_topk(logits, None, None, topk)
    ids, w = moeq8.moe_route_topk_wide(to_dev(logits), topk)
    assert np.array_equal(host(ids), ids_ref)
    g = moeq8.moe_group_routes(ids, n_exp)
    xo, xd = quantized_pair(x)
    h = torch.full((c, topk, inter), float("nan"), device=DEV)
    moeq8.moe_grouped_mmvq(moeq8.GATE_UP_SWIGLU, wgd, wud, xd, g, n=inter, k=hidden, n_local_expert=n_exp,
                           ncols=c, topk=topk, out=h)
    hh = host(h).reshape(c * topk, inter)
    h_ref = np.zeros((c * topk, inter))
    for e, routes in oracle.group_routes(ids_ref):
        cols = [r // topk for r in routes]
        h_ref[routes] = oracle.glu_pair(wg[e], wu[e], xo[cols])[0]
    assert_close(hh, h_ref, EPI_TOL, "wide h")
    h32 = h_ref.astype(np.float32)
    hq_ref = oracle.quantize_q8_1(h32)
    hq = moeq8.q8_1_quantize_rows(to_dev(h32))
    assert host(hq).tobytes() == hq_ref.tobytes()
    y = host(moeq8.moe_grouped_mmvq(moeq8.DOWN, wdd, None, hq, g, n=hidden, k=inter, n_local_expert=n_exp,
                                    ncols=c, topk=topk)).reshape(c * topk, hidden)
    y_ref = np.zeros((c * topk, hidden))
    for e, routes in oracle.group_routes(ids_ref):
        y_ref[routes] = oracle.mmvq(wd[e], hq_ref[routes])
    assert_close(y, y_ref, PROD_TOL, "wide y")
    y32 = y_ref.astype(np.float32).reshape(c, topk, hidden)
    w32 = w_ref.astype(np.float32)
    out = host(moeq8.moe_combine(to_dev(y32), ids, to_dev(w32)))
    assert_close(out, oracle.moe_combine(y32.astype(np.float64), ids_ref, w32.astype(np.float64)),
                 EPI_TOL, "wide combine")


# ---------------------------------------------------------------------------
# wide batches on the int8 matrix cores (moe_grouped_gemm)
# ---------------------------------------------------------------------------

def _gemm_case(c, n_exp, local, topk, hidden, inter, seed):
    (wg, wu, wd), (wgd, wud, wdd) = _tiny_layer(seed, local, hidden, inter)
    x = workloads.activations(seed, c, hidden)
    logits = workloads.router_logits(seed + 1, c, n_exp)
    own = None if local == n_exp else workloads.owner_slots(n_exp, local)
    ids_ref, w_ref, _ = oracle.route_topk(logits, None, own, topk)
    ids, _ = moeq8.moe_route_topk_wide(to_dev(logits), topk, owner_slot=None if own is None else to_dev(own),
                                       n_local_expert=local)
    assert np.array_equal(host(ids), ids_ref)
    g = moeq8.moe_group_routes(ids, local)
    return (wg, wu, wd), (wgd, wud, wdd), x, ids_ref, ids, g


@pytest.mark.parametrize("c,n_exp,local,topk,hidden,inter", [
    (40, 32, 32, 8, 1024, 256),      # gate/up K = 1024
    (40, 8, 8, 4, 4096, 256),        # K = 4096, ~20 routes per expert: two 16-route chunks
    (300, 4, 4, 4, 256, 64),         # every column routes to all 4 experts: 19 chunks each
    (48, 256, 256, 8, 256, 64),      # ~150 active experts: the unit search spans several waves of groups
    (130, 64, 40, 8, 320, 128),      # owner mask (masked routes); down n = 320: a half-empty row tile
    (3, 16, 16, 8, 128, 64),         # K = 128 and 64: fewer block pairs than a step holds
    (1, 4, 4, 4, 64, 64),
    (24, 8, 8, 8, 256, 2048),        # down K = 2048: the down staged in LDS too
    (33, 16, 16, 8, 512, 1024),      # down K = 1024, 8 row tiles: units of two tiles
    (20, 8, 8, 8, 320, 1024),        # down K = 1024, 5 row tiles: units of one
])
def test_grouped_gemm_vs_oracle(c, n_exp, local, topk, hidden, inter):
    """moe_grouped_gemm gate/up (h) and down (y) against the oracle route by
    route; the down stage reads the oracle's h (quantised on both sides, bytes
    equal); rows of masked routes stay untouched."""
    say(f"grouped gemm c={c} E={n_exp} local={local} k={topk} H={hidden} I={inter}")
    (wg, wu, wd), (wgd, wud, wdd), x, ids_ref, ids, g = _gemm_case(c, n_exp, local, topk, hidden, inter,
                                                                   c + hidden + inter)
    xo, xd = quantized_pair(x)
    h = torch.full((c, topk, inter), float("nan"), device=DEV)
    moeq8.moe_grouped_gemm(moeq8.GATE_UP_SWIGLU, wgd, wud, xd, g, n=inter, k=hidden, n_local_expert=local,
                           ncols=c, topk=topk, out=h)
    hh = host(h).reshape(c * topk, inter)
    masked = ids_ref.reshape(-1) < 0
    assert np.isnan(hh[masked]).all()
    h_ref = np.zeros((c * topk, inter))
    for e, routes in oracle.group_routes(ids_ref):
        h_ref[routes] = oracle.glu_pair(wg[e], wu[e], xo[[r // topk for r in routes]])[0]
    assert_close(hh[~masked], h_ref[~masked], EPI_TOL, "gemm h")

    h32 = h_ref.astype(np.float32)
    hq_ref = oracle.quantize_q8_1(h32)
    hq = moeq8.q8_1_quantize_rows(to_dev(h32))
    assert host(hq).tobytes() == hq_ref.tobytes()
    y = torch.full((c, topk, hidden), float("nan"), device=DEV)
    moeq8.moe_grouped_gemm(moeq8.DOWN, wdd, None, hq, g, n=hidden, k=inter, n_local_expert=local,
                           ncols=c, topk=topk, out=y)
    yy = host(y).reshape(c * topk, hidden)
    assert np.isnan(yy[masked]).all()
    y_ref = np.zeros((c * topk, hidden))
    for e, routes in oracle.group_routes(ids_ref):
        y_ref[routes] = oracle.mmvq(wd[e], hq_ref[routes])
    assert_close(yy[~masked], y_ref[~masked], PROD_TOL, "gemm y")


def test_grouped_gemm_integer_dots_unit_scale():
    """With every block scale 1.0 (fp16 0x3C00) each output is the exact
    integer sum of the block dots, which fp32 holds exactly here: the matrix
    core path must give it bit for bit (a wrong fragment layout, block order or
    scale pairing changes it)."""
    c, topk, n_exp, hidden, inter = 24, 4, 4, 256, 64
    rng = np.random.default_rng(7)
    nb = hidden // 32

    def q8_0(rows):
        w = np.zeros((n_exp, rows, nb), workloads.Q8_0_DTYPE)
        w["d"] = np.float16(1.0)
        w["qs"] = rng.integers(-127, 128, size=(n_exp, rows, nb, 32))
        return w

    wg, wu = q8_0(inter), q8_0(inter)
    xq = np.zeros((c, nb), np.dtype([("d", "<f2"), ("s", "<f2"), ("qs", "i1", (32,))]))
    xq["d"] = np.float16(1.0)
    xq["qs"] = rng.integers(-127, 128, size=(c, nb, 32))
    ids_np = np.stack([rng.choice(n_exp, size=topk, replace=False) for _ in range(c)]).astype(np.int32)
    g = moeq8.moe_group_routes(to_dev(ids_np), n_exp)
    h = moeq8.moe_grouped_gemm(moeq8.DOWN, to_dev(wg.reshape(-1)).reshape(-1), None,
                               to_dev(np.repeat(xq, topk, axis=0).reshape(-1)).reshape(-1), g, n=inter,
                               k=hidden, n_local_expert=n_exp, ncols=c, topk=topk)
    hh = host(h).reshape(c * topk, inter)
    qs_w = wg["qs"].astype(np.int64)                  # [E, rows, nb, 32]
    qs_x = np.repeat(xq, topk, axis=0)["qs"].astype(np.int64)   # [R, nb, 32]
    for r in range(c * topk):
        e = ids_np.reshape(-1)[r]
        exact = np.einsum("nbk,bk->n", qs_w[e], qs_x[r])
        assert np.array_equal(hh[r], exact.astype(np.float32)), r


def _off_alignment(t: torch.Tensor, shift: int = 4) -> torch.Tensor:
    """A copy of t's bytes that starts `shift` bytes past a 16-byte boundary."""
    raw = t.reshape(-1).view(torch.uint8)
    buf = torch.zeros(raw.numel() + 32, dtype=torch.uint8, device=DEV)
    view = buf[16 + shift:16 + shift + raw.numel()]
    view.copy_(raw)
    assert view.data_ptr() % 16 == shift
    return view


@pytest.mark.parametrize("c,n_exp,local,topk,hidden,inter", [
    (200, 16, 16, 8, 1024, 512),     # ~100 routes an expert: a full and a ragged 64-route unit
    (130, 64, 40, 8, 2048, 256),     # owner mask (masked routes); down: one K step, nothing to prefetch
    (64, 4, 4, 4, 4096, 256),        # 16 K steps; every column routes to all 4 experts
    (1, 8, 8, 8, 256, 256),          # one column, one K step
    (256, 64, 64, 8, 1024, 512),     # ~1024 units: workgroups take several units in turn
    (64, 8, 8, 8, 256, 2048),        # down K = 2048 (8 steps): the down staged too
    (256, 64, 64, 8, 1024, 2048),    # ~1024 down units of 8 steps each
])
def test_staged_gemm_equals_register_gemm(c, n_exp, local, topk, hidden, inter):
    """With k % 256 == 0, whole row tiles and 16-byte aligned operands the
    grouped GEMM stages its operands in LDS (persistent workgroups, the steps
    of their units in one pipeline; the down from k = 2048 on); the same call
    on weights copied 4 bytes off that alignment runs the register-fed form.  Both take the same integer
    dots, scale products and accumulation order, so every output (and every
    untouched row of a masked route) has the same bits."""
    say(f"staged vs register gemm c={c} E={n_exp} local={local} k={topk} H={hidden} I={inter}")
    (wg, wu, wd), (wgd, wud, wdd), x, ids_ref, ids, g = _gemm_case(c, n_exp, local, topk, hidden, inter,
                                                                   3 * c + hidden)
    xo, xd = quantized_pair(x)
    live = torch.from_numpy(ids_ref.reshape(-1) >= 0).to(DEV)
    outs = []
    for a, b in ((wgd, wud), (_off_alignment(wgd), _off_alignment(wud))):
        h = torch.full((c, topk, inter), float("nan"), device=DEV)
        moeq8.moe_grouped_gemm(moeq8.GATE_UP_SWIGLU, a, b, xd, g, n=inter, k=hidden, n_local_expert=local,
                               ncols=c, topk=topk, out=h)
        outs.append(h)
    assert bits_equal(outs[0], outs[1])
    assert not torch.isnan(outs[0].reshape(c * topk, -1)[live]).any()
    assert torch.isnan(outs[0].reshape(c * topk, -1)[~live]).all()
    hq = moeq8.q8_1_quantize_rows(torch.nan_to_num(outs[0]).reshape(c * topk, inter))
    outs = []
    for a in (wdd, _off_alignment(wdd)):
        y = torch.full((c, topk, hidden), float("nan"), device=DEV)
        moeq8.moe_grouped_gemm(moeq8.DOWN, a, None, hq, g, n=hidden, k=inter, n_local_expert=local,
                               ncols=c, topk=topk, out=y)
        outs.append(y)
    assert bits_equal(outs[0], outs[1])
    assert not torch.isnan(outs[0].reshape(c * topk, -1)[live]).any()
    assert torch.isnan(outs[0].reshape(c * topk, -1)[~live]).all()


def test_staged_gemm_work_counters_return_to_zero():
    """The staged GEMM's workgroups take their units from the library's work
    counters (256 call slots, handed out in turn); a call leaves its counters
    at zero.  300 calls in a row (every slot reused) with units of one, two
    and four K steps (the next unit drawn at the last step, or two steps
    before it) and downs of 8 steps and of 4 (units of two row tiles), on the
    plain rows and the GEMM layout in turn: every call gives the bits of the
    register-fed form (a counter left off zero would skip units, leaving NaN
    rows)."""
    say("staged gemm work counters, 300 calls")
    c, n_exp, local, topk, inter = 40, 8, 8, 8, 64
    cases = []
    for hidden in (256, 512, 1024):
        (_, _, _), (wgd, wud, _), x, ids_ref, ids, g = _gemm_case(c, n_exp, local, topk, hidden, inter, 7 + hidden)
        xd = moeq8.q8_1_quantize_rows(to_dev(x))
        ref = torch.full((c, topk, inter), float("nan"), device=DEV)
        moeq8.moe_grouped_gemm(moeq8.GATE_UP_SWIGLU, _off_alignment(wgd), _off_alignment(wud), xd, g, n=inter,
                               k=hidden, n_local_expert=local, ncols=c, topk=topk, out=ref)
        cases.append((hidden, wgd, wud, xd, g, ref))
    downs = []
    for kd in (2048, 1024):                            # 8 steps a unit; 4, two row tiles a unit
        (_, _, _), (_, _, wdd), _, _, _, gd = _gemm_case(c, n_exp, local, topk, 256, kd, 11 + kd)
        hq = moeq8.q8_1_quantize_rows(to_dev(workloads.normal_f32(12 + kd, (c * topk, kd), 1.0)))
        yref = torch.full((c, topk, 256), float("nan"), device=DEV)
        moeq8.moe_grouped_gemm(moeq8.DOWN, _off_alignment(wdd), None, hq, gd, n=256, k=kd, n_local_expert=local,
                               ncols=c, topk=topk, out=yref)
        downs.append((kd, wdd, moeq8.q8_0_pack_gemm_rows(wdd, local * 256, kd), gd, hq, yref))
    # the GEMM layout's kernels draw from the same counters
    packed = {hidden: (moeq8.q8_0_pack_gemm_rows(wgd, local * inter, hidden),
                       moeq8.q8_0_pack_gemm_rows(wud, local * inter, hidden)) for hidden, wgd, wud, _, _, _ in cases}
    h = torch.empty((c, topk, inter), device=DEV)
    y = torch.empty((c, topk, 256), device=DEV)
    for i in range(300):
        g8 = (i // 4) % 2 == 1
        if i % 4 == 3:
            kd, wdd, pdd, gd, hq, yref = downs[(i // 8) % 2]
            y.fill_(float("nan"))
            moeq8.moe_grouped_gemm(moeq8.DOWN_G8 if g8 else moeq8.DOWN, pdd if g8 else wdd, None, hq, gd, n=256,
                                   k=kd, n_local_expert=local, ncols=c, topk=topk, out=y)
            assert bits_equal(y, yref), (i, kd)
        else:
            hidden, wgd, wud, xd, g, ref = cases[i % 4]
            a, b = packed[hidden] if g8 else (wgd, wud)
            h.fill_(float("nan"))
            moeq8.moe_grouped_gemm(moeq8.GATE_UP_SWIGLU_G8 if g8 else moeq8.GATE_UP_SWIGLU, a, b, xd, g, n=inter,
                                   k=hidden, n_local_expert=local, ncols=c, topk=topk, out=h)
            assert bits_equal(h, ref), (i, hidden, g8)


def _gemm_layout_reference(raw: np.ndarray, rows: int, k: int) -> np.ndarray:
    """The grouped GEMM's weight layout restated on the host: per 272-byte
    group of 8 blocks, the 8 scales (block j's two bytes at 2j), then block j's
    32 quants at 16 + 32j, the two 8-byte halves of each 16-byte piece swapped
    in rows i with i % 16 >= 8."""
    g = k // 256
    b = np.ascontiguousarray(raw).reshape(rows, g, 8, 34)
    out = np.empty((rows, g, 272), np.uint8)
    out[:, :, :16] = b[:, :, :, :2].reshape(rows, g, 16)
    q = b[:, :, :, 2:].reshape(rows, g, 8, 4, 8).copy()          # [row, group, block, 8-byte piece, byte]
    swap = (np.arange(rows) % 16) >= 8
    q[swap] = q[swap][:, :, :, [1, 0, 3, 2], :]
    out[:, :, 16:] = q.reshape(rows, g, 256)
    return out.reshape(-1)


@pytest.mark.parametrize("rows,k", [(1, 256), (40, 512), (64, 4096)])
def test_gemm_layout_bytes(rows, k):
    say(f"gemm layout rows={rows} k={k}")
    raw = np.random.default_rng(rows + k).integers(0, 256, size=rows * (k // 32) * 34, dtype=np.uint8)
    got = host(moeq8.q8_0_pack_gemm_rows(to_dev(raw), rows, k))
    assert np.array_equal(got, _gemm_layout_reference(raw, rows, k))


@pytest.mark.parametrize("c,n_exp,local,topk,hidden,inter", [
    (200, 16, 16, 8, 1024, 512),     # ~100 routes an expert: a full and a ragged 64-route unit
    (130, 64, 40, 8, 2048, 256),     # owner mask (masked routes)
    (64, 4, 4, 4, 4096, 256),        # 16 K steps; every column routes to all 4 experts
    (1, 8, 8, 8, 256, 256),          # one column, one K step
    (40, 8, 8, 8, 512, 64),          # two K steps
    (96, 256, 256, 8, 1024, 1024),   # ~240 active experts; the down at k = 1024 (4 steps a unit)
    (20, 16, 16, 8, 2048, 2048),     # k = 2048 both ways: 8 steps a unit
    (48, 512, 512, 8, 1024, 256),    # 384 routes over 512 local experts
    (128, 1024, 1024, 8, 256, 256),  # more active experts than the LDS unit table holds (global lookup)
])
def test_gemm_layout_equals_plain(c, n_exp, local, topk, hidden, inter):
    """GATE_UP_SWIGLU_G8 and DOWN_G8 on weights repacked by q8_0_pack_gemm_rows
    against GATE_UP_SWIGLU and DOWN on the plain rows: every output bit for
    bit, rows of masked routes untouched."""
    say(f"gemm layout vs plain c={c} E={n_exp} local={local} k={topk} H={hidden} I={inter}")
    (_, _, _), (wgd, wud, wdd), x, ids_ref, ids, g = _gemm_case(c, n_exp, local, topk, hidden, inter, 5 * c + hidden)
    xd = moeq8.q8_1_quantize_rows(to_dev(x))
    pg = moeq8.q8_0_pack_gemm_rows(wgd, local * inter, hidden)
    pu = moeq8.q8_0_pack_gemm_rows(wud, local * inter, hidden)
    outs = []
    for stage, a, b in ((moeq8.GATE_UP_SWIGLU, wgd, wud), (moeq8.GATE_UP_SWIGLU_G8, pg, pu)):
        h = torch.full((c, topk, inter), float("nan"), device=DEV)
        moeq8.moe_grouped_gemm(stage, a, b, xd, g, n=inter, k=hidden, n_local_expert=local, ncols=c,
                               topk=topk, out=h)
        outs.append(h)
    assert bits_equal(outs[0], outs[1])
    live = torch.from_numpy(ids_ref.reshape(-1) >= 0).to(DEV)
    assert not torch.isnan(outs[1].reshape(c * topk, -1)[live]).any()
    if inter % 256:
        return                                       # the down's layout takes whole 8-block groups
    # the down: DOWN_G8 (always staged) against DOWN on the plain rows
    hq = moeq8.q8_1_quantize_rows(torch.nan_to_num(outs[0]).reshape(c * topk, inter))
    pd = moeq8.q8_0_pack_gemm_rows(wdd, local * hidden, inter)
    ys = []
    for stage, a in ((moeq8.DOWN, wdd), (moeq8.DOWN_G8, pd)):
        y = torch.full((c, topk, hidden), float("nan"), device=DEV)
        moeq8.moe_grouped_gemm(stage, a, None, hq, g, n=hidden, k=inter, n_local_expert=local, ncols=c,
                               topk=topk, out=y)
        ys.append(y)
    assert bits_equal(ys[0], ys[1])
    assert not torch.isnan(ys[1].reshape(c * topk, -1)[live]).any()


@pytest.mark.parametrize("c", [40, 512])
def test_wide_layer_gemm_layout_equals_plain(c):
    """forward_wide on the matrix cores with gate/up in the GEMM layout
    (pack_gemm_experts) against the plain layout: every output bit for bit."""
    from quantized_moe_expert_q8_amd import moe_layer as ml
    say(f"wide gemm layout layer c={c}")
    H, I, topk, n_exp, seed = 4096, 1024, 8, 16, 120 + c
    wg, wu, wd = _synth_dev(seed, n_exp, I, H, 0), _synth_dev(seed, n_exp, I, H, 1), _synth_dev(seed, n_exp, H, I, 2)
    experts = ml.RoutedExperts(wg, wu, wd, n_exp, H, I)
    ge = ml.pack_gemm_experts(experts)
    x = to_dev(workloads.activations(seed, c, H))
    lg = to_dev(workloads.router_logits(seed, c, n_exp))
    b = to_dev(workloads.router_bias(seed, n_exp))
    wa, wb = ml.WideWorkspace(c, H, I, topk, DEV), ml.WideWorkspace(c, H, I, topk, DEV)
    ml.forward_wide(x, lg, b, None, n_exp, experts, wa, products="gemm")
    ml.forward_wide(x, lg, b, None, n_exp, ge, wb, products="gemm")
    torch.cuda.synchronize()
    assert bits_equal(wa.h, wb.h) and bits_equal(wa.y, wb.y) and bits_equal(wa.out, wb.out)


# ---------------------------------------------------------------------------
# 8-bit block exchange codec: bytes and sums bit for bit against the oracle
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("rows,n,stride", [(1, 32, 32), (7, 96, 96), (33, 4096, 4096), (5, 64, 67),
                                           (1024, 4096, 4096)])
def test_q8_block_encode_bytes(rows, n, stride):
    """Encode against the oracle, byte for byte: contiguous and strided rows (a
    stride that is not a multiple of 4 takes the scalar path), zero blocks,
    a block of exact halves and a block whose scale is not an fp16 value."""
    say(f"q8x encode rows={rows} n={n} stride={stride}")
    x = workloads.normal_f32(rows * 7 + n, (rows, stride), 2.0)
    x[0, :32] = 0.0
    if n >= 64:
        x[0, 32:64] = np.array([127.0] + [k + 0.5 for k in range(-15, 16)], np.float32)
    if rows > 1:
        x[1, :32] = np.array([1.0] + [0.3 * (k - 15) / 15 for k in range(31)], np.float32)
    xd = to_dev(x)
    blocks = moeq8.q8_block_encode(xd[:, :n])
    ref = oracle.q8x_encode(np.ascontiguousarray(x[:, :n]))
    assert host(blocks).tobytes() == ref.tobytes()


@pytest.mark.parametrize("nranks,rows,n", [(1, 3, 64), (2, 1024, 4096), (3, 17, 160), (8, 64, 1024)])
def test_q8_block_decode_sum_bits(nranks, rows, n):
    """The rank-order sum of the oracle-encoded blocks of every rank, bit for
    bit (fp32 products and sums in the defined order), including the planted
    case where only ascending rank order gives the result."""
    say(f"q8x decode_sum nranks={nranks} rows={rows} n={n}")
    parts = [oracle.q8x_encode(workloads.normal_f32(50 + r, (rows, n), 1.0 + 3 * r)) for r in range(nranks)]
    if nranks == 3:
        parts[0]["d"][0, 0] = np.float32(2.0 ** 20)
        parts[0]["qs"][0, 0, 0] = 127
        for r in (1, 2):
            parts[r]["d"][0, 0] = np.float32(1.0)
            parts[r]["qs"][0, 0, 0] = 3
    gathered = np.stack([p.reshape(-1).view(np.uint8) for p in parts])
    out = moeq8.q8_block_decode_sum(to_dev(gathered), rows, n)
    ref = oracle.q8x_decode_sum(parts)
    got = host(out)
    assert got.tobytes() == ref.tobytes()
    if nranks == 3:
        assert got[0, 0] == np.float32(127 * 2 ** 20)


def test_q8_block_round_trip_on_gpu():
    """encode -> decode of one rank gives the oracle's dequantized values."""
    x = workloads.normal_f32(3, (64, 512), 1.0)
    blocks = moeq8.q8_block_encode(to_dev(x))
    back = host(moeq8.q8_block_decode_sum(blocks.view(1, -1), 64, 512))
    assert back.tobytes() == oracle.q8x_dequantize(oracle.q8x_encode(x)).tobytes()


# ---------------------------------------------------------------------------
# 4-bit weights (Q4): quantiser bytes, products against the oracle, and the
# invariants the shared reduction order gives
# ---------------------------------------------------------------------------

def _q4_both(w32):
    """Quantise on both sides; assert identical bytes; return (oracle, device)."""
    wo = oracle.quantize_q4(w32)
    wd = moeq8.q4_quantize_rows(to_dev(w32))
    assert host(wd).tobytes() == wo.tobytes()
    return wo, wd


@pytest.mark.parametrize("n,k", [(5, 32), (64, 4096), (300, 1024)])
def test_q4_quantize_bytes(n, k):
    w = workloads.normal_f32(n + k, (n, k), 0.02)
    w[0, :32] = 0.0
    if k >= 64:
        w[0, 32:64] = np.array([7.0] + [0.5 * (i - 15) for i in range(31)], np.float32)
    _q4_both(w)


@pytest.mark.parametrize("n,k,c", [(64, 256, 1), (256, 1024, 3), (512, 4096, 8), (96, 2048, 5)])
def test_q4_mmvq_and_pair_vs_oracle(n, k, c):
    say(f"q4 mmvq n={n} k={k} c={c}")
    wg, wgd = _q4_both(workloads.normal_f32(n * 3 + k, (n, k), 0.02))
    wu, wud = _q4_both(workloads.normal_f32(n * 5 + k, (n, k), 0.02))
    xo, xd = quantized_pair(workloads.activations(c + k, c, k))
    y = host(moeq8.mmvq_q4(wgd, xd, n, k))
    assert_close(y, oracle.mmvq_q4(wg, xo), PROD_TOL, "q4 product")
    g = torch.empty((c, n), device=DEV)
    u = torch.empty((c, n), device=DEV)
    h = moeq8.mmvq_q4_glu_pair(wgd, wud, xd, n, k, g_out=g, u_out=u)
    h_ref, _, _ = oracle.glu_pair_q4(wg, wu, xo)
    assert_close(host(h), h_ref, EPI_TOL, "q4 pair")
    # the pair's raw products are the separate products, and h is their SwiGLU
    assert bits_equal(g, moeq8.mmvq_q4(wgd, xd, n, k))
    assert bits_equal(u, moeq8.mmvq_q4(wud, xd, n, k))
    assert bits_equal(h, moeq8.swiglu_ds4(g, u))


def test_q4_batch_invariance_and_slices():
    n, k = 128, 4096
    w, wd = _q4_both(workloads.normal_f32(3, (n, k), 0.02))
    xo, xd = quantized_pair(workloads.activations(9, 8, k))
    full = moeq8.mmvq_q4(wd, xd, n, k)
    for c in (1, 2, 5):
        assert bits_equal(moeq8.mmvq_q4(wd, xd[:c].contiguous(), n, k), full[:c].contiguous())
    # a column-range slice (blocks 32..64 of each row) equals the full product on
    # activations that are zero outside the slice
    kb, ks = 32, 1024
    xs = workloads.activations(10, 2, k)
    xz = np.zeros_like(xs)
    xz[:, kb * 32:kb * 32 + ks] = xs[:, kb * 32:kb * 32 + ks]
    _, xzd = quantized_pair(xz)
    _, xsd = quantized_pair(np.ascontiguousarray(xs[:, kb * 32:kb * 32 + ks]))
    sl = moeq8.mmvq_q4(wd, xsd, n, ks, k_block_offset=kb, w_offset_bytes=kb * 18,
                       w_row_stride_bytes=(k // 32) * 18)
    assert bits_equal(sl, moeq8.mmvq_q4(wd, xzd, n, k))


@pytest.mark.parametrize("c,n_exp,hidden,inter", [(1, 16, 1024, 256), (8, 32, 2048, 512), (40, 16, 1024, 256)])
def test_q4_grouped_vs_oracle_and_dense(c, n_exp, hidden, inter):
    """Grouped gate/up and down (q8_1 and fp32 h) with Q4 experts: against the
    oracle per route, and bit-equal to the dense product on each route."""
    say(f"q4 grouped c={c} E={n_exp} H={hidden} I={inter}")
    topk = 8
    gate = [workloads.normal_f32(100 + e, (inter, hidden), 0.02) for e in range(n_exp)]
    up = [workloads.normal_f32(300 + e, (inter, hidden), 0.02) for e in range(n_exp)]
    down = [workloads.normal_f32(500 + e, (hidden, inter), 0.02) for e in range(n_exp)]
    wg, wgd = _q4_both(np.concatenate(gate))
    wu, wud = _q4_both(np.concatenate(up))
    wdn, wdd = _q4_both(np.concatenate(down))
    wg = wg.reshape(n_exp, inter, -1)
    wu = wu.reshape(n_exp, inter, -1)
    wdn = wdn.reshape(n_exp, hidden, -1)
    x = workloads.activations(c + 1, c, hidden)
    logits = workloads.router_logits(c + 2, c, n_exp)
    ids_ref, _, _ = oracle.route_topk(logits, None, None, topk)
    ids, _ = moeq8.moe_route_topk_wide(to_dev(logits), topk)
    g = moeq8.moe_group_routes(ids, n_exp)
    xo, xd = quantized_pair(x)
    h = moeq8.moe_grouped_mmvq_q4(moeq8.GATE_UP_SWIGLU, wgd.view(-1), wud.view(-1), xd, g, n=inter,
                                  k=hidden, n_local_expert=n_exp, ncols=c, topk=topk)
    hh = host(h).reshape(c * topk, inter)
    h_ref = np.zeros((c * topk, inter))
    for e, routes in oracle.group_routes(ids_ref):
        h_ref[routes] = oracle.glu_pair_q4(wg[e], wu[e], xo[[r // topk for r in routes]])[0]
    assert_close(hh, h_ref, EPI_TOL, "q4 grouped h")
    rb = (hidden // 32) * 18
    for j in range(0, c, max(1, c // 4)):
        e = int(ids_ref[j, 0])
        hp = moeq8.mmvq_q4_glu_pair(wgd.view(-1), wud.view(-1), xd[j:j + 1].contiguous(), inter, hidden,
                                    w_offset_bytes=e * inter * rb, w_row_stride_bytes=rb)
        assert bits_equal(h[j, 0:1].contiguous(), hp)
    # down on the oracle's h: q8_1 rows and, in one launch, fp32 rows
    h32 = h_ref.astype(np.float32)
    hq_ref, hq = quantized_pair(h32)
    y = host(moeq8.moe_grouped_mmvq_q4(moeq8.DOWN, wdd.view(-1), None, hq, g, n=hidden, k=inter,
                                       n_local_expert=n_exp, ncols=c, topk=topk)).reshape(c * topk, hidden)
    y_ref = np.zeros((c * topk, hidden))
    for e, routes in oracle.group_routes(ids_ref):
        y_ref[routes] = oracle.mmvq_q4(wdn[e], hq_ref[routes])
    assert_close(y, y_ref, PROD_TOL, "q4 grouped y")
    yf = host(moeq8.moe_grouped_mmvq_q4(moeq8.DOWN_F32_ACT, wdd.view(-1), None, to_dev(h32), g, n=hidden,
                                        k=inter, n_local_expert=n_exp, ncols=c, topk=topk)).reshape(c * topk, hidden)
    assert yf.tobytes() == y.tobytes()


def test_q4_layer_equals_its_calls():
    """moe_layer.forward with 4-bit experts (four launches) gives the bits of
    the separate calls: route, grouped gate/up, q8_1 of h, grouped down,
    combine."""
    from quantized_moe_expert_q8_amd import moe_layer as ml
    c, n_exp, hidden, inter, topk = 5, 16, 1024, 256, 8
    wg = moeq8.q4_quantize_rows(to_dev(workloads.normal_f32(1, (n_exp * inter, hidden), 0.02))).view(-1)
    wu = moeq8.q4_quantize_rows(to_dev(workloads.normal_f32(2, (n_exp * inter, hidden), 0.02))).view(-1)
    wd = moeq8.q4_quantize_rows(to_dev(workloads.normal_f32(3, (n_exp * hidden, inter), 0.02))).view(-1)
    experts = ml.RoutedExperts(wg, wu, wd, n_exp, hidden, inter, fmt="q4")
    x = to_dev(workloads.activations(4, c, hidden))
    lg = to_dev(workloads.router_logits(5, c, n_exp))
    ws = ml.Workspace(c, hidden, inter, topk, 0, DEV)
    out, _ = ml.forward(x, lg, None, None, n_exp, experts, None, ws)
    out = out.clone()
    ids, w, g = moeq8.moe_route_topk(lg, topk)
    xq = moeq8.q8_1_quantize_rows(x)
    h = moeq8.moe_grouped_mmvq_q4(moeq8.GATE_UP_SWIGLU, wg, wu, xq, g, n=inter, k=hidden, n_local_expert=n_exp,
                                  ncols=c, topk=topk)
    hq = moeq8.q8_1_quantize_rows(h.view(c * topk, inter))
    y = moeq8.moe_grouped_mmvq_q4(moeq8.DOWN, wd, None, hq, g, n=hidden, k=inter, n_local_expert=n_exp,
                                  ncols=c, topk=topk)
    assert bits_equal(out, moeq8.moe_combine(y, ids, w))


def _p64q4_reference(raw: np.ndarray, rows: int, k: int) -> np.ndarray:
    """The 4-bit packed layout restated on the host: within each 2304-byte
    segment of a row, dword 9c + d moves to 256*(d//4) + 4c + d%4 (d < 8) and
    dword 9c + 8 to 512 + c."""
    w = np.ascontiguousarray(raw).reshape(-1).view(np.uint32).reshape(rows, k // 4096, 576)
    out = np.empty_like(w)
    c = np.arange(64)
    for d in range(8):
        out[:, :, 256 * (d // 4) + 4 * c + d % 4] = w[:, :, 9 * c + d]
    out[:, :, 512 + c] = w[:, :, 9 * c + 8]
    return out.reshape(-1).view(np.uint8)


@pytest.mark.parametrize("rows,k,extra", [(1, 4096, 0), (3, 8192, 0), (64, 4096, 16)])
def test_q4_pack64_layout(rows, k, extra):
    say(f"q4 pack64 rows={rows} k={k} extra={extra}")
    row_bytes = k // 32 * 18
    stride = row_bytes + extra
    raw = np.random.default_rng(rows + k + extra).integers(0, 256, size=rows * stride, dtype=np.uint8)
    got = host(moeq8.q4_pack64_rows(to_dev(raw), rows, k, src_row_stride_bytes=stride))
    want = _p64q4_reference(raw.reshape(rows, stride)[:, :row_bytes], rows, k)
    assert np.array_equal(got, want)
    # every byte is kept: the packing only permutes within a segment
    assert np.array_equal(np.sort(got.reshape(rows, -1), axis=1),
                          np.sort(raw.reshape(rows, stride)[:, :row_bytes], axis=1))


_Q4_BANK = {}


def _q4_bank(local, H=4096, I=1024):
    """Plain and packed 4-bit gate, up and down of `local` experts (device)."""
    if local not in _Q4_BANK:
        mats = []
        for m, (rows, k) in enumerate(((local * I, H), (local * I, H), (local * H, I))):
            mats.append(moeq8.q4_quantize_rows(to_dev(workloads.normal_f32(900 + m, (rows, k), 0.02))).view(-1))
        wg, wu, wd = mats
        packed = (moeq8.q4_pack64_rows(wg, local * I, H), moeq8.q4_pack64_rows(wu, local * I, H),
                  moeq8.q4_pack64_rows(wd, local * H // 4, 4 * I))
        _Q4_BANK.clear()
        _Q4_BANK[local] = ((wg, wu, wd), packed)
    return _Q4_BANK[local]


@pytest.mark.parametrize("c", [1, 2, 5, 8, 24])
def test_q4_grouped_p64_equals_plain(c):
    """The packed 4-bit stages (gate/up on 64-chunk packed rows, down on
    quad-packed rows, h quantised in the launch) against the plain 4-bit
    stages: every written h and y row bit for bit, masked routes untouched
    (half the experts local; 24 columns: a wide grouping, which the packed
    kernels serve with their ordinary-load form in passes of 8 columns)."""
    say(f"q4 p64 grouped c={c}")
    H, I, topk, n_exp, local, seed = 4096, 1024, 8, 16, 8, 140 + c
    (wg, wu, wd), (pg, pu, pd) = _q4_bank(local)
    x = to_dev(workloads.activations(seed, c, H))
    xq = moeq8.q8_1_quantize_rows(x)
    lg = to_dev(workloads.router_logits(seed, c, n_exp))
    ids, _, grouping = _route_any(lg, topk, c, n_exp, local, bias=to_dev(workloads.router_bias(seed, n_exp)))
    h_in = to_dev(workloads.normal_f32(seed + 1, (c * topk, I), 2.0))
    hs, ys = [], []
    for (gu, dn), (a, b, d) in (((moeq8.GATE_UP_SWIGLU, moeq8.DOWN_F32_ACT), (wg, wu, wd)),
                                ((moeq8.GATE_UP_SWIGLU_P64, moeq8.DOWN_F32_ACT_P64), (pg, pu, pd))):
        h = torch.full((c, topk, I), float("nan"), device=DEV)
        y = torch.full((c, topk, H), float("nan"), device=DEV)
        moeq8.moe_grouped_mmvq_q4(gu, a, b, xq, grouping, n=I, k=H, n_local_expert=local, ncols=c, topk=topk,
                                  out=h)
        moeq8.moe_grouped_mmvq_q4(dn, d, None, h_in, grouping, n=H, k=I, n_local_expert=local, ncols=c,
                                  topk=topk, out=y)
        hs.append(host(h))
        ys.append(host(y))
    valid = host(ids) >= 0
    assert valid.any() and not valid.all()
    for j in range(c):
        for s in range(topk):
            if valid[j, s]:
                assert np.array_equal(hs[0][j, s].view(np.int32), hs[1][j, s].view(np.int32)), (j, s)
                assert np.array_equal(ys[0][j, s].view(np.int32), ys[1][j, s].view(np.int32)), (j, s)
            else:
                assert np.isnan(hs[1][j, s]).all() and np.isnan(ys[1][j, s]).all()


@pytest.mark.parametrize("c", [1, 8])
def test_q4_layer_packed_equals_plain(c):
    """moe_layer.forward with packed 4-bit experts (pack_experts) and a plain
    Q8_0 shared share gives the bits of the plain 4-bit layer."""
    from quantized_moe_expert_q8_amd import moe_layer as ml
    say(f"q4 packed layer c={c}")
    H, I, topk, n_exp, local, share_rows, seed = 4096, 1024, 8, 16, 8, 256, 150 + c
    (wg, wu, wd), _ = _q4_bank(local)
    experts = ml.RoutedExperts(wg, wu, wd, local, H, I, fmt="q4")
    full = 2 * share_rows
    sg = _synth_dev(seed, 1, full, H, 3).view(full, H // 32 * 34)
    su = _synth_dev(seed, 1, full, H, 4).view(full, H // 32 * 34)
    sd = _synth_dev(seed, 1, H, full, 5).view(H, full // 32 * 34)
    shared = ml.SharedExpertShare(sg, su, sd, H, full, share_rows, share_rows)
    pe, ps = ml.pack_experts(experts, shared)
    assert pe.packed and pe.fmt == "q4" and ps is shared
    x = to_dev(workloads.activations(seed, c, H))
    lg = to_dev(workloads.router_logits(seed, c, n_exp))
    own = to_dev(workloads.owner_slots(n_exp, local))
    wa = ml.Workspace(c, H, I, topk, share_rows, DEV)
    wb = ml.Workspace(c, H, I, topk, share_rows, DEV)
    ml.forward(x, lg, None, own, local, experts, shared, wa, add_shared=True)
    ml.forward(x, lg, None, own, local, pe, ps, wb, add_shared=True)
    torch.cuda.synchronize()
    assert bits_equal(wa.out, wb.out) and bits_equal(wa.ys, wb.ys)
    with pytest.raises(ValueError):                  # the 4-bit layer's shared share stays plain
        ml.forward(x, lg, None, own, local, pe, ml.SharedExpertShare(sg, su, sd, H, full, share_rows,
                                                                     share_rows, packed=True), wb)


def test_grouped_gemm_takes_the_decode_grouping():
    """moe_grouped_gemm on the grouping moe_route_topk writes (8 columns, owner
    mask) gives the oracle's products, like the grouped MMVQ on it."""
    c, n_exp, local, hidden, inter, topk = 8, 64, 32, 1024, 256, 8
    (wg, wu, wdn), (wgd, wud, wdd) = _tiny_layer(77, local, hidden, inter)
    x = workloads.activations(78, c, hidden)
    logits = workloads.router_logits(79, c, n_exp)
    own = workloads.owner_slots(n_exp, local)
    xo, xd = quantized_pair(x)
    ids, _, grouping = moeq8.moe_route_topk(to_dev(logits), topk, owner_slot=to_dev(own), n_local_expert=local)
    ids_ref, _, _ = oracle.route_topk(logits, None, own, topk)
    assert np.array_equal(host(ids), ids_ref)
    h = torch.full((c, topk, inter), float("nan"), device=DEV)
    moeq8.moe_grouped_gemm(moeq8.GATE_UP_SWIGLU, wgd, wud, xd, grouping, n=inter, k=hidden, n_local_expert=local,
                           ncols=c, topk=topk, out=h)
    hh = host(h).reshape(c * topk, inter)
    masked = ids_ref.reshape(-1) < 0
    assert np.isnan(hh[masked]).all()
    for e, routes in oracle.group_routes(ids_ref):
        ref = oracle.glu_pair(wg[e], wu[e], xo[[r // topk for r in routes]])[0]
        assert_close(hh[routes], ref, EPI_TOL, f"gemm on decode grouping, expert {e}")


# ---------------------------------------------------------------------------
# the routed FFN product after routing in one call (moe_grouped_ffn_p64)
# ---------------------------------------------------------------------------

def _packed_ffn_layer(seed, local, share):
    from quantized_moe_expert_q8_amd import moe_layer as ml
    H, I = 4096, 1024
    wg, wu, wd = _synth_dev(seed, local, I, H, 0), _synth_dev(seed, local, I, H, 1), _synth_dev(seed, local, H, I, 2)
    experts = ml.RoutedExperts(wg, wu, wd, local, H, I)
    shared = None
    if share:
        full = 2 * I
        rb_h, rb_f = H // 32 * 34, full // 32 * 34
        shared = ml.SharedExpertShare(_synth_dev(seed, 1, full, H, 3).view(full, rb_h),
                                      _synth_dev(seed, 1, full, H, 4).view(full, rb_h),
                                      _synth_dev(seed, 1, H, full, 5).view(H, rb_f), H, full, I, I)
    return ml.pack_experts(experts, shared)


@pytest.mark.parametrize("c,n_exp,local,share", [(1, 16, 16, True), (2, 32, 16, False), (3, 32, 32, True),
                                                 (5, 64, 32, True), (8, 128, 48, False)])
def test_grouped_ffn_equals_its_two_stages(c, n_exp, local, share):
    """moe_grouped_ffn_p64 against GATE_UP_SWIGLU_P64 then DOWN_F32_ACT_P64:
    h, y (and hs, ys) bit for bit, masked rows untouched; every column count
    class of the launch (1, 2, up to 4, up to 8 columns a pass)."""
    from quantized_moe_expert_q8_amd import moe_layer as ml
    say(f"grouped ffn c={c} E={n_exp} local={local} share={share}")
    H, I, topk, seed = 4096, 1024, 8, 110 + c
    pe, ps = _packed_ffn_layer(seed, local, share)
    x = to_dev(workloads.activations(seed, c, H))
    lg = to_dev(workloads.router_logits(seed, c, n_exp))
    b = to_dev(workloads.router_bias(seed, n_exp))
    own = to_dev(workloads.owner_slots(n_exp, local))
    ws = [ml.Workspace(c, H, I, topk, I if share else 0, DEV) for _ in range(2)]
    for w in ws:
        moeq8.moe_route_topk_quantize(x, lg, topk, bias=b, owner_slot=own, n_local_expert=local, xq=w.xq,
                                      ids=w.ids, weights=w.weights, grouping=w.grouping)
        for t in (w.h, w.y) + ((w.hs, w.ys) if share else ()):
            t.fill_(float("nan"))
    rb = H // 32 * 34
    wa, wb = ws
    gu = dn = one = None
    if share:
        rnd = ps.down_block_offset() // (ps.rows // 32)
        doff = rnd * H * moeq8.ops.ROUND_BYTES
        gu = {"a": ps.gate, "b": ps.up, "row_stride": rb, "n": ps.rows, "k": H, "k_block_offset": 0,
              "offset_bytes": ps.gate_offset(), "out": wa.hs}
        dn = {"a": ps.down, "row_stride": moeq8.ops.ROUND_BYTES, "n": H, "k": ps.rows, "k_block_offset": 0,
              "offset_bytes": doff, "out": wa.ys, "act": wa.hs}
        one = {"gate": ps.gate, "up": ps.up, "row_stride": rb, "rows": ps.rows, "offset_bytes": ps.gate_offset(),
               "down": ps.down, "down_offset_bytes": doff, "hs": wb.hs, "ys": wb.ys}
    moeq8.moe_grouped_mmvq_ex(moeq8.GATE_UP_SWIGLU_P64, pe.gate, pe.up, wa.xq, wa.grouping, n=I, k=H,
                              n_local_expert=local, ncols=c, topk=topk, out=wa.h, shared=gu)
    moeq8.moe_grouped_mmvq_ex(moeq8.DOWN_F32_ACT_P64, pe.down, None, wa.h.view(c * topk, I), wa.grouping,
                              n=H, k=I, n_local_expert=local, ncols=c, topk=topk, out=wa.y, shared=dn)
    moeq8.moe_grouped_ffn_p64(pe.gate, pe.up, pe.down, wb.xq, wb.grouping, hidden=H, inter=I,
                              n_local_expert=local, ncols=c, topk=topk, h=wb.h, y=wb.y, shared=one)
    torch.cuda.synchronize()
    valid = host(wa.ids) >= 0
    ha, hb, ya, yb = host(wa.h), host(wb.h), host(wa.y), host(wb.y)
    for j in range(c):
        for s in range(topk):
            if valid[j, s]:
                assert np.array_equal(ha[j, s].view(np.int32), hb[j, s].view(np.int32)), (j, s)
                assert np.array_equal(ya[j, s].view(np.int32), yb[j, s].view(np.int32)), (j, s)
            else:
                assert np.isnan(hb[j, s]).all() and np.isnan(yb[j, s]).all()
    if share:
        assert bits_equal(wa.hs, wb.hs) and bits_equal(wa.ys, wb.ys)


def test_grouped_ffn_rejects_before_launching():
    """A bad down stage is found before the gate/up stage is launched: h keeps
    its contents."""
    say("grouped ffn host checks")
    c, topk, local, H, I = 2, 8, 4, 4096, 1024
    lg = to_dev(workloads.router_logits(3, c, local))
    ids, w, grouping = moeq8.moe_route_topk(lg, 4)
    g = torch.zeros(local * I * (H // 32) * 34, dtype=torch.uint8, device=DEV)
    d = torch.zeros(local * H * 1088 + 16, dtype=torch.uint8, device=DEV)
    xq = torch.zeros((c, H // 32 * 36), dtype=torch.uint8, device=DEV)
    h = torch.full((c, 4, I), 7.0, device=DEV)
    y = torch.zeros((c, 4, H), device=DEV)
    with pytest.raises(moeq8.MoeQ8Error) as ei:         # down weights off the 16-byte grid
        moeq8.moe_grouped_ffn_p64(g, g, d[4:], xq, grouping, hidden=H, inter=I, n_local_expert=local, ncols=c,
                                  topk=4, h=h, y=y)
    assert ei.value.status == -2
    torch.cuda.synchronize()
    assert bool((h == 7.0).all())
