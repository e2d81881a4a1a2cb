"""GPU parity on the five workloads at their full sizes.

  pair_n512_k256          gate/up pair + SwiGLU, N=512, K=256, 1 column
  shared_ffn_h4096_i2048  shared expert 4096 -> 2048 -> 4096 at 1, 2, 4, 5, 8 columns
  routed_e256_c1          routed layer, 256 experts, top-8, 1 column
  verify_e256_c5          routed layer, 5 columns, one grouping
  ep_share_l43_e128_c8    43 layers x 128 local experts (of 256), 8 columns, half
                          of the shared expert; run as bench.py times it (one
                          HIP graph of all layers), sampled layers checked

Stage by stage (the oracle never consumes GPU data; where stages chain, the
GPU stage is fed the oracle's input):
  q8_1(x) bytes and router ids bit-exact; products <= 1e-5*max(1,|ref|);
  SwiGLU, weights, combine <= 1e-4*max(1,|ref|); q8_1 of the oracle's h
  bit-exact; down on the oracle's hq <= 1e-5.
Whole chain (GPU end to end vs oracle end to end): the GPU's fp32 h can round
to a neighbouring q8_1 code where the oracle's h lies near a code boundary, so
several results are correct there.  The q8_1 bytes the GPU's quantiser makes
of the GPU's h are compared with the oracle's q8_1 of its own h: every value
that differs must sit within 1e-4 of a half-integer code boundary in the
oracle's quotient x/d (or in a block whose scale lies within 1e-6 of an fp16
rounding boundary), and the allowed difference is 1e-4*max(1,|ref|) plus the
exact effect of the values that did differ.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import workloads  # noqa: E402
import quantized_moe_expert_q8_amd as moeq8  # noqa: E402
from quantized_moe_expert_q8_amd import moe_layer as ml  # noqa: E402
from _gpu import DEV, assert_close, bits_equal, host, say, to_dev  # noqa: E402

pytestmark = pytest.mark.gpu

PROD_TOL = 1e-5
EPI_TOL = 1e-4


def quantize_both_q8_0(w32):
    """Each side quantises the same fp32 weights; the bytes must agree."""
    wo = oracle.quantize_q8_0(w32)
    wd = moeq8.q8_0_quantize_rows(to_dev(w32))
    assert host(wd).tobytes() == wo.tobytes()
    return wo, wd


def quantize_both_q8_1(x32):
    xo = oracle.quantize_q8_1(x32)
    xd = moeq8.q8_1_quantize_rows(to_dev(x32))
    assert host(xd).tobytes() == xo.tobytes()
    return xo, xd


# ---------------------------------------------------------------------------
# whole-chain flip bound, from the oracle's own h only
# ---------------------------------------------------------------------------

def flip_slack(hq_gpu_bytes, h64, wd_deq, thresh=1e-4, stats=None):
    """Allowance of one route's whole chain.  hq_gpu_bytes: the q8_1 blocks
    the GPU's quantiser made of the GPU's h (one row, raw bytes); h64: the
    oracle's h.  Values of the two q8_1 rows that differ must be flips at a
    boundary: the oracle's fp32 quotient |x/d| within `thresh` of a
    half-integer, or the whole block when the oracle's fp32 scale lies within
    1e-6 (relative) of an fp16 rounding boundary.  Returns |Wd| @ |dq_gpu -
    dq_ref|, the exact effect of the differences on the route's y."""
    h32 = np.asarray(h64, np.float32).reshape(1, -1)
    ref = oracle.quantize_q8_1(h32)[0]
    gpu = np.frombuffer(hq_gpu_bytes, dtype=oracle.Q8_1_DTYPE)
    dq_ref = ref["d"].astype(np.float64)[:, None] * ref["qs"].astype(np.float64)
    dq_gpu = gpu["d"].astype(np.float64)[:, None] * gpu["qs"].astype(np.float64)
    diff = dq_gpu - dq_ref
    moved = diff != 0
    if moved.any():
        blocks = h32.reshape(-1, 32)
        amax = np.abs(blocks).max(axis=1)
        d32 = (amax / np.float32(127.0)).astype(np.float32)
        with np.errstate(divide="ignore", invalid="ignore"):
            v = np.where(d32[:, None] > 0, np.abs(blocks / d32[:, None]).astype(np.float64), 0.0)
        dist = np.abs((v - np.floor(v)) - 0.5)
        d64 = d32.astype(np.float64)
        e = np.floor(np.log2(np.maximum(d64, 1e-300)))
        ulp16 = np.where(d64 >= 2.0 ** -14, 2.0 ** (e - 10), 2.0 ** -24)
        m = d64 / ulp16
        scale_near = np.abs((m - np.floor(m)) - 0.5) * ulp16 <= 1e-6 * d64
        legit = (dist < thresh) | scale_near[:, None]
        assert np.all(legit[moved]), (f"q8_1 values differ away from a boundary: distances "
                                      f"{dist[moved & ~legit][:8]}")
        if stats is not None:
            code = (gpu["qs"] != ref["qs"]) & (gpu["d"] == ref["d"])[:, None]
            stats["flips"] = stats.get("flips", 0) + int(code.sum())
            stats["scale_flips"] = stats.get("scale_flips", 0) + int((gpu["d"] != ref["d"]).sum())
            if code.any():
                stats["max_dist"] = max(stats.get("max_dist", 0.0), float(dist[code].max()))
    return np.abs(wd_deq) @ np.abs(diff).reshape(-1)


# ---------------------------------------------------------------------------
# 1. the single gate/up pair
# ---------------------------------------------------------------------------

def test_pair_n512_k256():
    cfg = workloads.CONFIGS["pair_n512_k256"]
    say("config pair_n512_k256")
    rng = np.random.default_rng(cfg["seed"])
    x = rng.normal(0.0, 1.0, (1, cfg["k"])).astype(np.float32)
    wg32 = rng.normal(0.0, 0.02, (cfg["n"], cfg["k"])).astype(np.float32)
    wu32 = rng.normal(0.0, 0.02, (cfg["n"], cfg["k"])).astype(np.float32)
    wg, wgd = quantize_both_q8_0(wg32)
    wu, wud = quantize_both_q8_0(wu32)
    xo, xd = quantize_both_q8_1(x)
    g = torch.empty((1, cfg["n"]), dtype=torch.float32, device=DEV)
    u = torch.empty_like(g)
    h = moeq8.mmvq_q8_0_glu_pair(wgd, wud, xd, cfg["n"], cfg["k"], g_out=g, u_out=u)
    h_ref, g_ref, u_ref = oracle.glu_pair(wg, wu, xo)
    assert_close(host(g), g_ref, PROD_TOL, "gate")
    assert_close(host(u), u_ref, PROD_TOL, "up")
    assert_close(host(h), h_ref, EPI_TOL, "h")
    assert bits_equal(h, moeq8.swiglu_ds4(moeq8.mmvq_q8_0(wgd, xd, cfg["n"], cfg["k"]),
                                          moeq8.mmvq_q8_0(wud, xd, cfg["n"], cfg["k"])))
    # the dequantise-then-fp64 definition agrees with the oracle's integer path
    assert_close(host(g), oracle.mmvq_bruteforce(wg, xo), PROD_TOL, "gate vs brute force")


# ---------------------------------------------------------------------------
# 2. the shared expert FFN at 1..8 columns
# ---------------------------------------------------------------------------

def test_shared_ffn_h4096_i2048():
    cfg = workloads.CONFIGS["shared_ffn_h4096_i2048"]
    H, I, seed = cfg["hidden"], cfg["inter"], cfg["seed"]
    say("config shared_ffn_h4096_i2048: weights")
    wg32, wu32, wd32 = workloads.expert_weights_f32(seed, 0, 999, H, I)
    wg, wgd = quantize_both_q8_0(wg32)
    wu, wud = quantize_both_q8_0(wu32)
    wd, wdd = quantize_both_q8_0(wd32)
    wd_deq = oracle.dequantize(wd)
    h8 = None
    for c in cfg["cols"]:
        say(f"  cols={c}")
        x = workloads.activations(seed, 8, H)[:c]
        xo, xd = quantize_both_q8_1(np.ascontiguousarray(x))
        h = moeq8.mmvq_q8_0_glu_pair(wgd, wud, xd, I, H)
        h_ref, _, _ = oracle.glu_pair(wg, wu, xo)
        assert_close(host(h), h_ref, EPI_TOL, f"h c={c}")
        if h8 is None:
            h8 = moeq8.mmvq_q8_0_glu_pair(wgd, wud, quantize_both_q8_1(workloads.activations(seed, 8, H))[1], I, H)
        assert bits_equal(h, h8[:c])                              # batch invariance
        # quantise the oracle's h on the GPU: bit-exact
        hq_ref = oracle.quantize_q8_1(h_ref.astype(np.float32))
        hq_dev = moeq8.q8_1_quantize_rows(to_dev(h_ref.astype(np.float32)))
        assert host(hq_dev).tobytes() == hq_ref.tobytes()
        ys = moeq8.mmvq_q8_0(wdd, hq_dev, H, I)
        ys_ref = oracle.mmvq(wd, hq_ref)
        assert_close(host(ys), ys_ref, PROD_TOL, f"down c={c}")
        # whole chain on the GPU
        hq_gpu = moeq8.q8_1_quantize_rows(h)
        ys_gpu = host(moeq8.mmvq_q8_0(wdd, hq_gpu, H, I)).astype(np.float64)
        hq_gpu_b = host(hq_gpu)
        st = {}
        for j in range(c):
            bound = EPI_TOL * np.maximum(1, np.abs(ys_ref[j])) + flip_slack(hq_gpu_b[j].tobytes(), h_ref[j],
                                                                              wd_deq, stats=st)
            assert np.all(np.abs(ys_gpu[j] - ys_ref[j]) <= bound), f"chain c={c} col {j}"
        say(f"    chain: {st.get('flips', 0)} q8_1 codes and {st.get('scale_flips', 0)} scales flipped "
            f"(codes at most {st.get('max_dist', 0):.2e} from a boundary)")


# ---------------------------------------------------------------------------
# 3 / 4. routed layers, 256 experts, 1 and 5 columns
# ---------------------------------------------------------------------------

def _routed_layer_check(name):
    cfg = workloads.CONFIGS[name]
    H, I, E, topk, seed = cfg["hidden"], cfg["inter"], cfg["experts"], cfg["topk"], cfg["seed"]
    c = cfg["cols"][0]
    say(f"config {name}")
    x = workloads.activations(seed, c, H)
    logits = workloads.router_logits(seed, c, E)
    bias = workloads.router_bias(seed, E)
    ids_ref, w_ref, _ = oracle.route_topk(logits, bias, None, topk)
    used = sorted(set(int(e) for e in ids_ref.reshape(-1)))
    assert len(used) <= c * topk
    # every expert resident: synthetic blocks, then the routed experts get
    # N(0, 0.02) weights quantised on both sides
    rb_h, rb_i = H // 32 * 34, I // 32 * 34
    gate = torch.empty(E * I * rb_h, dtype=torch.uint8, device=DEV)
    up = torch.empty_like(gate)
    down = torch.empty(E * H * rb_i, dtype=torch.uint8, device=DEV)
    moeq8.synth_q8_0_fill(gate, E, I * H // 32, E, seed, 0, 0, 0)
    moeq8.synth_q8_0_fill(up, E, I * H // 32, E, seed, 0, 0, 1)
    moeq8.synth_q8_0_fill(down, E, H * I // 32, E, seed, 0, 0, 2)
    mats = {}
    for e in used:
        wg32, wu32, wd32 = workloads.expert_weights_f32(seed, 0, e, H, I)
        trip = []
        for t, w32, rows, rb in ((gate, wg32, I, rb_h), (up, wu32, I, rb_h), (down, wd32, H, rb_i)):
            wo = oracle.quantize_q8_0(w32)
            view = t[e * rows * rb:(e + 1) * rows * rb].view(rows, rb)
            moeq8.q8_0_quantize_rows(to_dev(w32), out=view)
            trip.append(wo)
        mats[e] = tuple(trip)
        assert host(gate[e * I * rb_h:(e + 1) * I * rb_h]).tobytes() == trip[0].tobytes()
        assert host(down[e * H * rb_i:(e + 1) * H * rb_i]).tobytes() == trip[2].tobytes()
    say(f"  {len(used)} routed experts quantised on both sides")

    # the whole layer as the bench launches it
    ws = ml.Workspace(c, H, I, topk, 0, DEV)
    experts = ml.RoutedExperts(gate, up, down, E, H, I)
    xd, lgd, bd = to_dev(x), to_dev(logits), to_dev(bias)
    out, _ = ml.forward(xd, lgd, bd, None, E, experts, None, ws)
    torch.cuda.synchronize()
    ref = oracle.moe_layer(x, logits, bias, None, lambda e: mats[e], topk)
    assert host(ws.xq).tobytes() == ref["xq"].tobytes()
    assert np.array_equal(host(ws.ids), ids_ref)
    assert_close(host(ws.weights), w_ref, EPI_TOL, "weights")
    # stage: h of every route vs the oracle
    hh = host(ws.h)
    hq_gpu_b = host(moeq8.q8_1_quantize_rows(ws.h.view(c * topk, I)))   # what the down launch quantises
    h_ref32 = np.zeros((c * topk, I), np.float32)
    flip = np.zeros((c, H))
    st = {}
    for j in range(c):
        for s in range(topk):
            e = int(ids_ref[j, s])
            h_ref, _, _ = oracle.glu_pair(mats[e][0], mats[e][1], ref["xq"][j:j + 1])
            assert_close(hh[j, s], h_ref[0], EPI_TOL, f"h ({j},{s})")
            h_ref32[j * topk + s] = h_ref[0].astype(np.float32)
            flip[j] += w_ref[j, s] * flip_slack(hq_gpu_b[j * topk + s].tobytes(), h_ref[0],
                                                oracle.dequantize(mats[e][2]), stats=st)
    say(f"  chain: {st.get('flips', 0)} q8_1 codes and {st.get('scale_flips', 0)} scales flipped "
        f"(codes at most {st.get('max_dist', 0):.2e} from a boundary)")
    # stage: the GPU quantiser and the grouped down on the oracle's h
    hq_dev = moeq8.q8_1_quantize_rows(to_dev(h_ref32))
    hq_ref = oracle.quantize_q8_1(h_ref32)
    assert host(hq_dev).tobytes() == hq_ref.tobytes()
    y = moeq8.moe_grouped_mmvq(moeq8.DOWN, down, None, hq_dev, ws.grouping, n=H, k=I,
                               n_local_expert=E, ncols=c, topk=topk)
    yy = host(y)
    y_ref = np.zeros((c, topk, H))
    for j in range(c):
        for s in range(topk):
            e = int(ids_ref[j, s])
            y_ref[j, s] = oracle.mmvq(mats[e][2], hq_ref[j * topk + s:j * topk + s + 1])[0]
    assert_close(yy, y_ref, PROD_TOL, "grouped down")
    # stage: combine on the oracle's y and weights
    comb = host(moeq8.moe_combine(to_dev(y_ref.astype(np.float32)), ws.ids,
                                  to_dev(w_ref.astype(np.float32))))
    assert_close(comb, oracle.moe_combine(y_ref.astype(np.float32).astype(np.float64), ids_ref,
                                          w_ref.astype(np.float32).astype(np.float64)), EPI_TOL, "combine")
    # whole chain
    got = host(out).astype(np.float64)
    bound = EPI_TOL * np.maximum(1, np.abs(ref["out"])) + flip
    assert np.all(np.abs(got - ref["out"]) <= bound), "layer output outside the flip-aware bound"
    say(f"  chain max |diff| {np.abs(got - ref['out']).max():.3e}")


def test_routed_e256_c1():
    _routed_layer_check("routed_e256_c1")


def test_verify_e256_c5():
    _routed_layer_check("verify_e256_c5")


# ---------------------------------------------------------------------------
# 5. one GPU's share: 43 layers x 128 local experts, 8 columns, as benchmarked
# ---------------------------------------------------------------------------

def test_ep_share_l43_e128_c8():
    import bench
    cfg = dict(workloads.CONFIGS["ep_share_l43_e128_c8"])
    L, n_local, E = cfg["layers"], cfg["local_experts"], cfg["experts"]
    H, I, topk, seed, c = cfg["hidden"], cfg["inter"], cfg["topk"], cfg["seed"], cfg["cols"][0]
    share = cfg["shared_inter"] // cfg["shared_share"]
    say("config ep_share_l43_e128_c8: allocating the 43-layer share")
    bank = bench.Bank(moeq8, torch, L, n_local, H, I, seed, cfg["shared_inter"])
    bank.pack_weights(moeq8, torch)         # the launch configuration the bench times
    xs, lgs, bs = bench.layer_inputs(torch, workloads, seed, L, c, H, E)
    owner_np = workloads.owner_slots(E, n_local)
    owner = to_dev(owner_np)
    sample = (0, 21, 42)
    wss = {l: ml.Workspace(c, H, I, topk, share, DEV) for l in sample}
    ws = ml.Workspace(c, H, I, topk, share, DEV)
    experts = [bank.experts(ml, l) for l in range(L)]
    shared = [bank.shared(ml, l, share) for l in range(L)]

    def step():
        for l in range(L):
            ml.forward(xs[l], lgs[l], bs[l], owner, n_local, experts[l], shared[l], wss.get(l, ws),
                       add_shared=True)

    step()
    torch.cuda.synchronize()
    eager = {l: host(wss[l].out).copy() for l in sample}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    for l in sample:
        assert np.array_equal(host(wss[l].out).view(np.int32), eager[l].view(np.int32))

    for l in sample:
        say(f"  layer {l}")
        w = wss[l]
        x = host(xs[l])
        lg = host(lgs[l])
        b = host(bs[l])
        ids_ref, w_ref, _ = oracle.route_topk(lg, b, owner_np, topk)
        assert np.array_equal(host(w.ids), ids_ref)
        assert_close(host(w.weights), w_ref, EPI_TOL, "weights")
        used = sorted(set(int(e) for e in ids_ref.reshape(-1) if e >= 0))
        mats = {e: (workloads.synth_q8_0_matrix(seed, l, e, 0, I, H),
                    workloads.synth_q8_0_matrix(seed, l, e, 1, I, H),
                    workloads.synth_q8_0_matrix(seed, l, e, 2, H, I)) for e in used}
        ref = oracle.moe_layer(x, lg, b, owner_np, lambda e: mats[e], topk)
        assert host(w.xq).tobytes() == ref["xq"].tobytes()
        hh = host(w.h)
        hq_gpu_b = host(moeq8.q8_1_quantize_rows(w.h.view(c * topk, I)))   # what the down launch quantises
        flip = np.zeros((c, H))
        h_ref32 = np.zeros((c * topk, I), np.float32)
        st = {}
        for j in range(c):
            for s in range(topk):
                e = int(ids_ref[j, s])
                if e < 0:
                    continue
                h_ref, _, _ = oracle.glu_pair(mats[e][0], mats[e][1], ref["xq"][j:j + 1])
                assert_close(hh[j, s], h_ref[0], EPI_TOL, f"layer {l} h ({j},{s})")
                h_ref32[j * topk + s] = h_ref[0].astype(np.float32)
                flip[j] += w_ref[j, s] * flip_slack(hq_gpu_b[j * topk + s].tobytes(), h_ref[0],
                                                    oracle.dequantize(mats[e][2]), stats=st)
        say(f"    chain: {st.get('flips', 0)} q8_1 codes and {st.get('scale_flips', 0)} scales flipped "
            f"(codes at most {st.get('max_dist', 0):.2e} from a boundary)")
        hq_dev = moeq8.q8_1_quantize_rows(to_dev(h_ref32))
        hq_ref = oracle.quantize_q8_1(h_ref32)
        assert host(hq_dev).tobytes() == hq_ref.tobytes()
        # (the bank is packed; the plain-layout calls below read the layer's
        # matrices drawn again from the same generator)
        plain_down = torch.empty_like(bank.down[l])
        moeq8.synth_q8_0_fill(plain_down, n_local, H * I // 32, n_local, seed, l, 0, 2)
        y = host(moeq8.moe_grouped_mmvq(moeq8.DOWN, plain_down, None, hq_dev, w.grouping, n=H,
                                        k=I, n_local_expert=n_local, ncols=c, topk=topk))
        for j in range(c):
            for s in range(topk):
                e = int(ids_ref[j, s])
                if e >= 0:
                    y_ref = oracle.mmvq(mats[e][2], hq_ref[j * topk + s:j * topk + s + 1])[0]
                    assert_close(y[j, s], y_ref, PROD_TOL, f"layer {l} y ({j},{s})")
        # out is the whole block output (routed sum + the shared expert's ys,
        # one fp32 add); ys is checked against the oracle below
        got = host(w.out).astype(np.float64) - host(w.ys).astype(np.float64)
        slack = np.abs(host(w.out).astype(np.float64)) * 2.0 ** -23     # the add's rounding
        assert np.all(np.abs(got - ref["out"]) <= EPI_TOL * np.maximum(1, np.abs(ref["out"])) + flip + slack)
        # the shared share: rows [0, 1024) of gate/up, column range [0, 1024) of down
        sg = workloads.synth_q8_0_matrix(seed, l, 0, 3, cfg["shared_inter"], H, 0, share)
        su = workloads.synth_q8_0_matrix(seed, l, 0, 4, cfg["shared_inter"], H, 0, share)
        sd = workloads.synth_q8_0_matrix(seed, l, 0, 5, H, cfg["shared_inter"])
        hs_ref, _, _ = oracle.glu_pair(sg, su, ref["xq"])
        assert_close(host(w.hs), hs_ref, EPI_TOL, f"layer {l} shared h")
        hsq_ref = oracle.quantize_q8_1(hs_ref.astype(np.float32))
        hsq_dev = moeq8.q8_1_quantize_rows(to_dev(hs_ref.astype(np.float32)))
        assert host(hsq_dev).tobytes() == hsq_ref.tobytes()
        plain_sd = torch.empty(H * (cfg["shared_inter"] // 32 * 34), dtype=torch.uint8, device=DEV)
        moeq8.synth_q8_0_fill(plain_sd, 1, H * cfg["shared_inter"] // 32, 1, seed, l, 0, 5)
        ys = moeq8.mmvq_q8_0(plain_sd, hsq_dev, H, share, k_block_offset=0,
                             w_row_stride_bytes=cfg["shared_inter"] // 32 * 34)
        assert_close(host(ys), oracle.mmvq_column_range(sd, hsq_ref, 0), PROD_TOL, f"layer {l} shared down")
        # the layer's own shared output (the packed down launch's extra items,
        # h quantised in the launch) equals the plain slice product on its hs
        ys_layer = moeq8.mmvq_q8_0(plain_sd, moeq8.q8_1_quantize_rows(w.hs), H, share, k_block_offset=0,
                                   w_row_stride_bytes=cfg["shared_inter"] // 32 * 34)
        assert bits_equal(w.ys, ys_layer)
        # column-range slices of the shared down (both halves) equal the full row
        # with zero-padded activations, and the gate/up row slice equals those
        # rows of the full product, bit for bit
        full_pad = torch.zeros((c, cfg["shared_inter"] // 32 * 36), dtype=torch.uint8, device=DEV)
        rbq = share // 32 * 36
        for half in (0, 1):
            full_pad.zero_()
            full_pad[:, half * rbq:(half + 1) * rbq] = hsq_dev
            kb = half * share // 32
            ys_half = moeq8.mmvq_q8_0(plain_sd, hsq_dev, H, share, k_block_offset=kb,
                                      w_offset_bytes=kb * 34,
                                      w_row_stride_bytes=cfg["shared_inter"] // 32 * 34)
            ys_full = moeq8.mmvq_q8_0(plain_sd, full_pad, H, cfg["shared_inter"])
            assert bits_equal(ys_half, ys_full)
        # (the bank's gate/up are packed; the dense pair reads the plain rows,
        # drawn again from the same generator)
        rb_h = H // 32 * 34
        plain = [torch.empty(cfg["shared_inter"] * rb_h, dtype=torch.uint8, device=DEV) for _ in range(2)]
        for t, m in zip(plain, (3, 4)):
            moeq8.synth_q8_0_fill(t, 1, cfg["shared_inter"] * H // 32, 1, seed, l, 0, m)
        hs_full = moeq8.mmvq_q8_0_glu_pair(plain[0], plain[1], w.xq, cfg["shared_inter"], H)
        assert bits_equal(hs_full[:, :share].contiguous(), w.hs)
    del g, bank
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# wide batches: the 256-expert layer at 512 columns on the matrix-core GEMM
# ---------------------------------------------------------------------------

def test_wide_e256_c512():
    """The wide layer (forward_wide, products on the int8 matrix cores) at 512
    columns, 256 experts resident (synthetic blocks, the same generator on both
    sides): q8_1(x) bytes, ids and the grouping exact, weights, and for three
    sampled experts every route's h (against the oracle) and y (the down GEMM
    run on q8_1 of the oracle's h, zero rows elsewhere, which must give exact
    zeros); the combine on synthetic y at full size."""
    cfg = workloads.CONFIGS["wide_e256"]
    H, I, E, topk, seed = cfg["hidden"], cfg["inter"], cfg["experts"], cfg["topk"], cfg["seed"]
    c = 512
    say(f"config wide_e256 at {c} columns")
    rb_h, rb_i = H // 32 * 34, I // 32 * 34
    gate = torch.empty(E * I * rb_h, dtype=torch.uint8, device=DEV)
    up = torch.empty_like(gate)
    down = torch.empty(E * H * rb_i, dtype=torch.uint8, device=DEV)
    moeq8.synth_q8_0_fill(gate, E, I * H // 32, E, seed, 0, 0, workloads.MATRIX_GATE)
    moeq8.synth_q8_0_fill(up, E, I * H // 32, E, seed, 0, 0, workloads.MATRIX_UP)
    moeq8.synth_q8_0_fill(down, E, H * I // 32, E, seed, 0, 0, workloads.MATRIX_DOWN)
    experts = ml.RoutedExperts(gate, up, down, E, H, I)
    x = workloads.activations(seed, c, H)
    logits = workloads.router_logits(seed, c, E)
    bias = workloads.router_bias(seed, E)
    ws = ml.WideWorkspace(c, H, I, topk, DEV)
    ml.forward_wide(to_dev(x), to_dev(logits), to_dev(bias), None, E, experts, ws, products="gemm")
    torch.cuda.synchronize()

    xq_ref = oracle.quantize_q8_1(x)
    assert host(ws.xq).tobytes() == xq_ref.tobytes()
    ids_ref, w_ref, _ = oracle.route_topk(logits, bias, None, topk)
    assert np.array_equal(host(ws.ids), ids_ref)
    assert_close(host(ws.weights), w_ref, EPI_TOL, "weights")
    groups = oracle.group_routes(ids_ref)
    words = host(ws.grouping).view(np.int32)
    R = c * topk
    assert words[0] == len(groups) and words[1] == R
    offset = words[4 + R:4 + 2 * R + 1]
    route = words[4 + 2 * R + 1:4 + 3 * R + 1]
    for a, (e, routes) in enumerate(groups):
        assert words[4 + a] == e and list(route[offset[a]:offset[a + 1]]) == routes

    by_load = sorted(groups, key=lambda g: len(g[1]))
    sample = [by_load[0], by_load[len(by_load) // 2], by_load[-1]]
    say(f"  {len(groups)} active experts; sampled loads {[len(r) for _, r in sample]}")
    hh = host(ws.h).reshape(R, I)
    h_in = np.zeros((R, I), np.float32)
    y_ref = {}
    for e, routes in sample:
        wg = workloads.synth_q8_0_matrix(seed, 0, e, workloads.MATRIX_GATE, I, H)
        wu = workloads.synth_q8_0_matrix(seed, 0, e, workloads.MATRIX_UP, I, H)
        wd = workloads.synth_q8_0_matrix(seed, 0, e, workloads.MATRIX_DOWN, H, I)
        h_ref = oracle.glu_pair(wg, wu, xq_ref[[r // topk for r in routes]])[0]
        assert_close(hh[routes], h_ref, EPI_TOL, f"h of expert {e}")
        h_in[routes] = h_ref.astype(np.float32)
        y_ref[e] = (routes, oracle.mmvq(wd, oracle.quantize_q8_1(h_ref.astype(np.float32))))
    hq_in = moeq8.q8_1_quantize_rows(to_dev(h_in))
    assert host(hq_in).tobytes() == oracle.quantize_q8_1(h_in).tobytes()
    y = host(moeq8.moe_grouped_gemm(moeq8.DOWN, down, None, hq_in, ws.grouping, n=H, k=I,
                                    n_local_expert=E, ncols=c, topk=topk)).reshape(R, H)
    sampled = np.zeros(R, bool)
    for e, (routes, yr) in y_ref.items():
        assert_close(y[routes], yr, PROD_TOL, f"y of expert {e}")
        sampled[routes] = True
    assert np.all(y[~sampled] == 0.0)

    y32 = workloads.normal_f32(seed + 100, (c, topk, H))
    comb = host(moeq8.moe_combine(to_dev(y32), ws.ids, to_dev(w_ref.astype(np.float32))))
    assert_close(comb, oracle.moe_combine(y32.astype(np.float64), ids_ref, w_ref.astype(np.float32)
                                          .astype(np.float64)), EPI_TOL, "combine")
