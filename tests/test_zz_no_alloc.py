"""moe_grouped_ffn_p64_noalloc (h and hs in the library's own device memory)
against moe_grouped_ffn_p64 with caller-owned h and hs, bit for bit, on two
calls in a row, the second with fewer columns than the first."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import workloads  # noqa: E402
import quantized_moe_expert_q8_amd as moeq8  # noqa: E402
from quantized_moe_expert_q8_amd import moe_layer as ml  # noqa: E402
from _gpu import DEV, bits_equal, host, say, to_dev  # noqa: E402

pytestmark = pytest.mark.gpu

H, I, TOPK = 4096, 1024, 8


def _synth_dev(seed, n_mats, rows, k, matrix):
    t = torch.empty(n_mats * rows * (k // 32) * 34, dtype=torch.uint8, device=DEV)
    moeq8.synth_q8_0_fill(t, n_mats, rows * k // 32, n_mats, seed, 0, 0, matrix)
    return t


def test_noalloc_ffn_equals_ffn_twice():
    local, n_exp, seed = 32, 64, 150
    wg, wu, wd = _synth_dev(seed, local, I, H, 0), _synth_dev(seed, local, I, H, 1), _synth_dev(seed, local, H, I, 2)
    full = 2 * I
    rb_h, rb_f = H // 32 * 34, full // 32 * 34
    shared = ml.SharedExpertShare(_synth_dev(seed, 1, full, H, 3).view(full, rb_h),
                                  _synth_dev(seed, 1, full, H, 4).view(full, rb_h),
                                  _synth_dev(seed, 1, H, full, 5).view(H, rb_f), H, full, I, I)
    pe, ps = ml.pack_experts(ml.RoutedExperts(wg, wu, wd, local, H, I), shared)
    own = to_dev(workloads.owner_slots(n_exp, local))
    rnd = ps.down_block_offset() // (ps.rows // 32)
    doff = rnd * H * moeq8.ops.ROUND_BYTES
    for c in (8, 3):                                   # the second call is smaller
        say(f"no-alloc ffn c={c}")
        x = to_dev(workloads.activations(seed + c, c, H))
        lg = to_dev(workloads.router_logits(seed + c, c, n_exp))
        b = to_dev(workloads.router_bias(seed + c, n_exp))
        w = ml.Workspace(c, H, I, TOPK, I, DEV)
        moeq8.moe_route_topk_quantize(x, lg, TOPK, bias=b, owner_slot=own, n_local_expert=local, xq=w.xq,
                                      ids=w.ids, weights=w.weights, grouping=w.grouping)
        sh = {"gate": ps.gate, "up": ps.up, "row_stride": rb_h, "rows": ps.rows, "offset_bytes": ps.gate_offset(),
              "down": ps.down, "down_offset_bytes": doff, "hs": w.hs, "ys": w.ys}
        moeq8.moe_grouped_ffn_p64(pe.gate, pe.up, pe.down, w.xq, w.grouping, hidden=H, inter=I,
                                  n_local_expert=local, ncols=c, topk=TOPK, h=w.h, y=w.y, shared=sh)
        y2 = torch.full((c, TOPK, H), float("nan"), device=DEV)
        ys2 = torch.full((c, H), float("nan"), device=DEV)
        sh2 = {k: v for k, v in sh.items() if k != "hs"}
        sh2["ys"] = ys2
        moeq8.moe_grouped_ffn_p64_noalloc(pe.gate, pe.up, pe.down, w.xq, w.grouping, hidden=H, inter=I,
                                          n_local_expert=local, ncols=c, topk=TOPK, y=y2, shared=sh2)
        torch.cuda.synchronize()
        valid = host(w.ids) >= 0
        assert valid.any() and not valid.all()
        ya, yb = host(w.y), host(y2)
        for j in range(c):
            for s in range(TOPK):
                if valid[j, s]:
                    assert np.array_equal(ya[j, s].view(np.int32), yb[j, s].view(np.int32)), (c, j, s)
                else:
                    assert np.isnan(yb[j, s]).all()
        assert bits_equal(w.ys, ys2)
