"""GPU edge cases of the products and the boundary.

* Products whose blocks have zero scales (with non-zero codes) and fp16
  subnormal scales, on the weight and on the activation side, against the
  oracle.  Scales are powers of two chosen so that every block term and every
  partial sum is exact in fp32: the GPU result must then equal the oracle's
  fp64 value exactly, whatever its summation order (a scale flushed to zero,
  a dropped block or a wrong scale index shows as a wrong value, however
  small the values are).
* Guard canaries: every output of every call is a view into a larger buffer
  whose bytes before and after it hold a pattern; no call writes outside its
  outputs.
* A call rejected on the host enqueues nothing: its outputs, real device
  buffers, keep their contents.
"""

import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import workloads  # noqa: E402
import quantized_moe_expert_q8_amd as moeq8  # noqa: E402
from _gpu import DEV, host, say, to_dev  # noqa: E402

pytestmark = pytest.mark.gpu


# (weight scales, activation scales): within a case every non-zero product of
# a weight scale and an activation scale is the same power of two
SCALE_CASES = {
    "w_sub_x_sub": ([0.0, 2.0 ** -20], [2.0 ** -18]),
    "both_smallest_sub": ([0.0, 2.0 ** -24], [0.0, 2.0 ** -24]),
    "w_one_x_sub": ([0.0, 1.0], [0.0, 2.0 ** -15]),
    "w_min_normal_x_sub": ([2.0 ** -14], [0.0, 2.0 ** -23]),
}


def _blocks(rng, rows, nb, scales, q81):
    """Blocks with scales drawn from `scales` (fp16-exact powers of two or 0)
    and codes in [-15, 15] (a zero scale keeps its non-zero codes)."""
    dt = oracle.Q8_1_DTYPE if q81 else oracle.Q8_0_DTYPE
    b = np.zeros((rows, nb), dt)
    b["qs"] = rng.integers(-15, 16, size=(rows, nb, 32))
    d = np.array(scales, np.float64)[rng.integers(0, len(scales), size=(rows, nb))]
    b["d"] = d.astype(np.float16)
    assert np.array_equal(b["d"].astype(np.float64), d)       # every scale is exact in fp16
    if q81:
        b["s"] = (b["d"].astype(np.float32) * b["qs"].astype(np.float32).sum(-1)).astype(np.float16)
    return b


def _exact(gpu, ref, what):
    gpu = np.asarray(gpu, np.float64)
    assert np.array_equal(gpu, ref), f"{what}: max |diff| {np.abs(gpu - ref).max():.3e} (must be exact)"


@pytest.mark.parametrize("case", sorted(SCALE_CASES))
def test_products_with_zero_and_subnormal_scales(case):
    say(f"edge scales {case}")
    ws, xs = SCALE_CASES[case]
    rng = np.random.default_rng(100 + sorted(SCALE_CASES).index(case))
    n, k, c = 96, 1024, 3
    nb = k // 32
    w = _blocks(rng, n, nb, ws, False)
    w2 = _blocks(rng, n, nb, ws, False)
    xq = _blocks(rng, c, nb, xs, True)
    # the case has zero-scale blocks and non-zero products on the side it says
    assert (w["d"] != 0).any() and (xq["d"] != 0).any()
    ref = oracle.mmvq(w, xq)
    ref2 = oracle.mmvq(w2, xq)
    assert np.abs(ref).max() > 0
    wd, w2d, xd = to_dev(w), to_dev(w2), to_dev(xq)
    _exact(host(moeq8.mmvq_q8_0(wd, xd, n, k)), ref, "single product")
    g = torch.empty((c, n), device=DEV)
    u = torch.empty((c, n), device=DEV)
    moeq8.mmvq_q8_0_glu_pair(wd, w2d, xd, n, k, g_out=g, u_out=u)
    _exact(host(g), ref, "pair gate")
    _exact(host(u), ref2, "pair up")
    # a column-range slice of the second half
    half = moeq8.mmvq_q8_0(wd, to_dev(xq[:, nb // 2:]), n, k // 2, k_block_offset=nb // 2,
                           w_offset_bytes=nb // 2 * 34, w_row_stride_bytes=nb * 34)
    _exact(host(half), oracle.mmvq_column_range(w, xq[:, nb // 2:], nb // 2), "column-range slice")

    # grouped down (MMVQ and the matrix-core GEMM): 4 experts, 3 columns, top-2
    n_exp, topk = 4, 2
    wexp = np.concatenate([_blocks(rng, n, nb, ws, False) for _ in range(n_exp)])
    hq = _blocks(rng, c * topk, nb, xs, True)
    lg = to_dev(workloads.router_logits(5, c, n_exp))
    ids, _, grouping = moeq8.moe_route_topk(lg, topk)
    idh = host(ids)
    for name, fn in (("grouped MMVQ", moeq8.moe_grouped_mmvq), ("grouped GEMM", moeq8.moe_grouped_gemm)):
        y = host(fn(moeq8.DOWN, to_dev(wexp), None, to_dev(hq), grouping, n=n, k=k, n_local_expert=n_exp,
                    ncols=c, topk=topk))
        for j in range(c):
            for s in range(topk):
                e = int(idh[j, s])
                r = j * topk + s
                _exact(y[j, s], oracle.mmvq(wexp[e * n:(e + 1) * n], hq[r:r + 1])[0], f"{name} ({j},{s})")


@pytest.mark.parametrize("case", sorted(SCALE_CASES))
def test_gemm_layout_with_zero_and_subnormal_scales(case):
    """The grouped GEMM on its own weight layout takes each block's scale
    product d_x * d_w from an fp16 matrix-core product: with zero and fp16
    subnormal scales on either side the down still equals the oracle exactly
    (scales as above), and the gate/up the plain layout's bits."""
    say(f"edge scales, GEMM layout {case}")
    ws, xs = SCALE_CASES[case]
    rng = np.random.default_rng(200 + sorted(SCALE_CASES).index(case))
    n, k, c, n_exp, topk = 64, 1024, 3, 4, 2
    nb = k // 32
    wexp = np.concatenate([_blocks(rng, n, nb, ws, False) for _ in range(n_exp)])
    hq = _blocks(rng, c * topk, nb, xs, True)
    lg = to_dev(workloads.router_logits(6, c, n_exp))
    ids, _, grouping = moeq8.moe_route_topk(lg, topk)
    idh = host(ids)
    wd = to_dev(wexp)
    y = host(moeq8.moe_grouped_gemm(moeq8.DOWN_G8, moeq8.q8_0_pack_gemm_rows(wd, n_exp * n, k), None, to_dev(hq),
                                    grouping, n=n, k=k, n_local_expert=n_exp, ncols=c, topk=topk))
    for j in range(c):
        for s_ in range(topk):
            e = int(idh[j, s_])
            r = j * topk + s_
            _exact(y[j, s_], oracle.mmvq(wexp[e * n:(e + 1) * n], hq[r:r + 1])[0], f"GEMM layout down ({j},{s_})")
    # gate/up: the layout's bits against the plain rows'
    wu = to_dev(np.concatenate([_blocks(rng, n, nb, ws, False) for _ in range(n_exp)]))
    xq = to_dev(_blocks(rng, c, nb, xs, True))
    outs = []
    for stage, a, b in ((moeq8.GATE_UP_SWIGLU, wd, wu),
                        (moeq8.GATE_UP_SWIGLU_G8, moeq8.q8_0_pack_gemm_rows(wd, n_exp * n, k),
                         moeq8.q8_0_pack_gemm_rows(wu, n_exp * n, k))):
        outs.append(moeq8.moe_grouped_gemm(stage, a, b, xq, grouping, n=n, k=k, n_local_expert=n_exp, ncols=c,
                                           topk=topk))
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))


# ---------------------------------------------------------------------------
# guard canaries
# ---------------------------------------------------------------------------

GUARD = 4096      # bytes of pattern on each side of an output


class Guarded:
    """An output view with GUARD bytes of pattern before and after it."""

    def __init__(self, nbytes, dtype=torch.uint8, shape=None):
        self.buf = torch.full((nbytes + 2 * GUARD,), 0xA5, dtype=torch.uint8, device=DEV)
        self.nbytes = nbytes
        v = self.buf[GUARD:GUARD + nbytes].view(dtype)
        self.view = v.view(shape) if shape is not None else v

    def check(self, what):
        b = host(self.buf)
        assert (b[:GUARD] == 0xA5).all() and (b[GUARD + self.nbytes:] == 0xA5).all(), \
            f"{what} wrote outside its output"


def test_every_output_keeps_its_guards():
    say("guard canaries")
    rng = np.random.default_rng(77)
    c, n, k, topk, n_exp = 3, 64, 1024, 2, 8
    nb = k // 32
    x = to_dev(rng.normal(0, 1, (c, k)).astype(np.float32))
    checks = []

    def G(nbytes, dtype=torch.uint8, shape=None, what=""):
        g = Guarded(nbytes, dtype, shape)
        checks.append((g, what))
        return g.view

    moeq8.q8_1_quantize_rows(x, out=G(c * nb * 36, shape=(c, nb * 36), what="q8_1_quantize_rows"))
    wq = moeq8.q8_0_quantize_rows(to_dev(rng.normal(0, 0.02, (n, k)).astype(np.float32)),
                                  out=G(n * nb * 34, shape=(n, nb * 34), what="q8_0_quantize_rows"))
    w2 = moeq8.q8_0_quantize_rows(to_dev(rng.normal(0, 0.02, (n, k)).astype(np.float32)))
    xq = moeq8.q8_1_quantize_rows(x)
    moeq8.mmvq_q8_0(wq, xq, n, k, out=G(c * n * 4, torch.float32, (c, n), "mmvq_q8_0"))
    moeq8.mmvq_q8_0_glu_pair(wq, w2, xq, n, k, out=G(c * n * 4, torch.float32, (c, n), "pair h"),
                             g_out=G(c * n * 4, torch.float32, (c, n), "pair g"),
                             u_out=G(c * n * 4, torch.float32, (c, n), "pair u"))
    gg = moeq8.mmvq_q8_0(wq, xq, n, k)
    moeq8.swiglu_ds4(gg, gg, out=G(c * n * 4, torch.float32, (c, n), "swiglu_ds4"))
    lg = to_dev(workloads.router_logits(6, c, n_exp))
    gb = moeq8.moe_grouping_bytes(c, topk)
    ids, wts, grp = moeq8.moe_route_topk(lg, topk, ids=G(c * topk * 4, torch.int32, (c, topk), "route ids"),
                                         weights=G(c * topk * 4, torch.float32, (c, topk), "route weights"),
                                         grouping=G(gb, what="route grouping"))
    moeq8.moe_route_topk_quantize(x, lg, topk, xq=G(c * nb * 36, shape=(c, nb * 36), what="prologue xq"),
                                  ids=G(c * topk * 4, torch.int32, (c, topk), "prologue ids"),
                                  weights=G(c * topk * 4, torch.float32, (c, topk), "prologue weights"),
                                  grouping=G(gb, what="prologue grouping"))
    wexp = to_dev(np.concatenate([oracle.quantize_q8_0(rng.normal(0, 0.02, (n, k)).astype(np.float32))
                                  for _ in range(n_exp)]))
    h = moeq8.moe_grouped_mmvq(moeq8.GATE_UP_SWIGLU, wexp, wexp, xq, grp, n=n, k=k, n_local_expert=n_exp,
                               ncols=c, topk=topk, out=G(c * topk * n * 4, torch.float32, (c, topk, n),
                                                         "grouped gate/up"))
    hq = moeq8.q8_1_quantize_rows(to_dev(rng.normal(0, 1, (c * topk, k)).astype(np.float32)))
    y = moeq8.moe_grouped_mmvq(moeq8.DOWN, wexp, None, hq, grp, n=n, k=k, n_local_expert=n_exp, ncols=c,
                               topk=topk, out=G(c * topk * n * 4, torch.float32, (c, topk, n), "grouped down"))
    moeq8.moe_grouped_gemm(moeq8.DOWN, wexp, None, hq, grp, n=n, k=k, n_local_expert=n_exp, ncols=c, topk=topk,
                           out=G(c * topk * n * 4, torch.float32, (c, topk, n), "grouped GEMM"))
    hf = to_dev(rng.normal(0, 1, (c * topk, k)).astype(np.float32))
    moeq8.moe_grouped_mmvq_ex(moeq8.DOWN_F32_ACT, wexp, None, hf, grp, n=n, k=k, n_local_expert=n_exp, ncols=c,
                              topk=topk, out=G(c * topk * n * 4, torch.float32, (c, topk, n), "down f32 act"),
                              shared={"a": wq, "row_stride": nb * 34, "n": n, "k": k, "k_block_offset": 0,
                                      "offset_bytes": 0,
                                      "out": G(c * n * 4, torch.float32, (c, n), "down f32 act shared"),
                                      "act": to_dev(rng.normal(0, 1, (c, k)).astype(np.float32))})
    moeq8.moe_combine(y, ids, wts, out=G(c * n * 4, torch.float32, (c, n), "combine"))
    moeq8.moe_combine(y, ids, wts, shared=gg, out=G(c * n * 4, torch.float32, (c, n), "combine shared"))
    xe = to_dev(rng.normal(0, 1, (c, k)).astype(np.float32))
    enc = moeq8.q8_block_encode(xe, out=G(c * nb * 36, shape=(c, nb * 36), what="q8_block_encode"))
    moeq8.q8_block_decode_sum(enc.view(1, -1).expand(2, -1).contiguous(), c, k,
                              out=G(c * k * 4, torch.float32, (c, k), "q8_block_decode_sum"))
    w4 = moeq8.q4_quantize_rows(to_dev(rng.normal(0, 0.02, (n, k)).astype(np.float32)),
                                out=G(n * nb * 18, shape=(n, nb * 18), what="q4_quantize_rows"))
    moeq8.mmvq_q4(w4, xq, n, k, out=G(c * n * 4, torch.float32, (c, n), "mmvq_q4"))
    moeq8.q8_0_pack64_rows(moeq8.q8_0_quantize_rows(to_dev(rng.normal(0, 0.02, (8, 4096)).astype(np.float32))),
                           8, 4096, out=G(8 * 4352, what="q8_0_pack64_rows"))
    moeq8.q8_0_pack64_rounds(wq, n, k, out=G(n * nb * 34, what="q8_0_pack64_rounds"))
    torch.cuda.synchronize()
    for g, what in checks:
        g.check(what)


def test_rejected_calls_enqueue_nothing():
    """Calls rejected on the host, given real device buffers: negative status,
    and after a synchronisation every output still holds its pattern."""
    say("rejected calls")
    L = moeq8.lib()
    c, n, k = 2, 64, 1024
    nb = k // 32
    w = torch.zeros(n * nb * 34, dtype=torch.uint8, device=DEV)
    xq = torch.zeros(c * nb * 36, dtype=torch.uint8, device=DEV)
    out = torch.full((c * n,), 3.5, device=DEV)
    ids = torch.full((c * 8,), 7, dtype=torch.int32, device=DEV)
    wts = torch.full((c * 8,), 1.5, device=DEV)
    grp = torch.full((moeq8.moe_grouping_bytes(c, 8),), 0x5A, dtype=torch.uint8, device=DEV)
    logits = torch.zeros((c, 4), device=DEV)
    p = lambda t, off=0: ctypes.c_void_p(t.data_ptr() + off)
    cases = [
        ("mmvq ncols 9", lambda: L.mmvq_q8_0(p(w), nb * 34, n, k, 0, p(xq), 9, p(out), None), -1),
        ("mmvq k % 64", lambda: L.mmvq_q8_0(p(w), nb * 34, n, 96, 0, p(xq), c, p(out), None), -1),
        ("mmvq odd block offset", lambda: L.mmvq_q8_0(p(w), nb * 34, n, 512, 3, p(xq), c, p(out), None), -2),
        ("mmvq misaligned out", lambda: L.mmvq_q8_0(p(w), nb * 34, n, k, 0, p(xq), c, p(out, 2), None), -2),
        ("pair without up", lambda: L.mmvq_q8_0_glu_pair(p(w), None, nb * 34, n, k, 0, p(xq), c, p(out), None,
                                                         None, None), -1),
        ("route topk > experts", lambda: L.moe_route_topk(p(logits), None, None, c, 4, 4, 8, p(ids), p(wts),
                                                          p(grp), None), -1),
        ("grouped bad stage", lambda: L.moe_grouped_mmvq(7, p(w), p(w), n * nb * 34, nb * 34, 1, n, k, p(xq),
                                                         p(grp), c, 8, p(out), None), -1),
        ("combine no columns", lambda: L.moe_combine(p(out), p(ids), p(wts), 0, 8, n, p(out), None), -1),
    ]
    for what, fn, status in cases:
        assert fn() == status, what
    torch.cuda.synchronize()
    assert bool((out == 3.5).all()) and bool((ids == 7).all()) and bool((wts == 1.5).all())
    assert bool((grp == 0x5A).all())


# ---------------------------------------------------------------------------
# a slice at an odd block offset, through the even-offset call it reduces to
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kb,nbs", [(1, 63), (3, 29), (33, 31), (65, 63)])
def test_odd_offset_slice_by_widening(kb, nbs):
    """The library takes slices on whole 2-block chunks (an even block offset,
    a multiple of 64 values).  A slice of nbs blocks from an odd block offset
    kb is the even-offset slice from kb - 1 with one zero activation block in
    front (a zero block adds +0 to its lane), padded at the end to a whole
    chunk: equal to the oracle's column-range product at kb within the product
    bar, and bit-equal to the full row with the activations zero outside."""
    say(f"odd offset slice kb={kb} blocks={nbs}")
    rng = np.random.default_rng(200 + kb)
    n, nb_full, c = 40, 128, 2
    w = oracle.quantize_q8_0(rng.normal(0, 0.02, (n, nb_full * 32)).astype(np.float32))
    xs = oracle.quantize_q8_1(rng.normal(0, 1, (c, nbs * 32)).astype(np.float32))
    lo = kb - 1                                       # even
    width = 1 + nbs + ((1 + nbs) % 2)                 # whole chunks
    assert lo + width <= nb_full
    xw = np.zeros((c, width), oracle.Q8_1_DTYPE)
    xw[:, 1:1 + nbs] = xs
    wd = to_dev(w)
    y = moeq8.mmvq_q8_0(wd, to_dev(xw), n, width * 32, k_block_offset=lo, w_offset_bytes=lo * 34,
                        w_row_stride_bytes=nb_full * 34)
    ref = oracle.mmvq_column_range(w, xs, kb)
    err = np.abs(host(y).astype(np.float64) - ref)
    assert np.all(err <= 1e-5 * np.maximum(1, np.abs(ref)))
    xfull = np.zeros((c, nb_full), oracle.Q8_1_DTYPE)
    xfull[:, kb:kb + nbs] = xs
    yfull = moeq8.mmvq_q8_0(wd, to_dev(xfull), n, nb_full * 32)
    assert np.array_equal(host(y).view(np.int32), host(yfull).view(np.int32))
