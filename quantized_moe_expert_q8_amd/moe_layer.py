"""One MoE layer of the verify/decode step as a fixed sequence of libmoeq8 calls.

The layer (lucebox PR #826: fused DS4.1 decode kernels, routed combine and
shared-expert commits) on ``ncols`` columns:

    xq  = q8_1(x)                                   quantise the FFN input once
    hs  = SwiGLU-DS4(Wsg.xq, Wsu.xq)                shared expert, this GPU's rows
    ys  = Wsd[:, slice] . q8_1(hs)                  its down product, a column-range slice
    ids, w, grouping = route(logits, bias, owner)   select + weights, owner mask, grouping
    h   = grouped SwiGLU-DS4(Wg[e].xq_j, Wu[e].xq_j) per route (j, s)
    y   = grouped Wd[e] . q8_1(h)
    out = sum over unmasked slots of w * y

Buffers live in a workspace allocated once, so ``forward`` allocates nothing
and can be captured in a HIP graph.  The fused form runs the layer as four
launches on one stream, the shared expert's work riding in the grouped
launches as extra work items; the unfused form issues the calls above one by
one, the shared expert on a second stream.  No arithmetic happens here.
"""

from __future__ import annotations

from dataclasses import dataclass

import torch

from . import ops

QK = ops.QK
Q80 = ops.Q8_0_BLOCK_BYTES
Q81 = ops.Q8_1_BLOCK_BYTES


@dataclass
class RoutedExperts:
    """Local experts of one layer, each [rows][k/32] blocks, experts
    ``expert_stride`` bytes apart (views into larger tensors are fine).
    fmt: "q8_0" (34-byte blocks) or "q4" (18-byte 4-bit blocks, for
    bandwidth-only expert weights).  packed: gate and up are in the 64-chunk
    packed layout (ops.q8_0_pack64_rows; hidden 4096) and down in the
    round-major four-row packed layout (ops.q8_0_pack64_rounds; inter 1024),
    read by the fused
    path's gate/up and down launches (pack_experts makes them); with 4-bit
    weights both are ops.q4_pack64_rows (down: each quad of rows as one row)."""
    gate: torch.Tensor       # uint8, n_local x inter x hidden/32 blocks
    up: torch.Tensor
    down: torch.Tensor       # uint8, n_local x hidden x inter/32 blocks
    n_local: int
    hidden: int
    inter: int
    fmt: str = "q8_0"
    packed: bool = False
    # optional copies of gate, up and down in the grouped GEMM's layout
    # (pack_gemm_experts), read by forward_wide's matrix-core products
    gemm_gate: torch.Tensor | None = None
    gemm_up: torch.Tensor | None = None
    gemm_down: torch.Tensor | None = None


@dataclass
class SharedExpertShare:
    """This GPU's share of the shared expert: rows [row0, row0 + rows) of the
    full gate/up matrices [inter_full, hidden] and the matching column range of
    the full down matrix [hidden, inter_full]."""
    gate: torch.Tensor       # uint8 [inter_full, hidden/32*34]
    up: torch.Tensor
    down: torch.Tensor       # uint8 [hidden, inter_full/32*34]
    hidden: int
    inter_full: int
    row0: int
    rows: int
    packed: bool = False     # gate/up 64-chunk packed, down round-major four-row packed

    def gate_offset(self) -> int:
        return self.row0 * (self.hidden // QK) * Q80

    def down_block_offset(self) -> int:
        return self.row0 // QK


class Workspace:
    def __init__(self, ncols: int, hidden: int, inter: int, topk: int, shared_rows: int, device,
                 side_stream=None):
        dev = torch.device(device)
        u8, f32 = torch.uint8, torch.float32
        self.ncols, self.topk = ncols, topk
        self.xq = torch.empty((ncols, hidden // QK * Q81), dtype=u8, device=dev)
        self.ids = torch.empty((ncols, topk), dtype=torch.int32, device=dev)
        self.weights = torch.empty((ncols, topk), dtype=f32, device=dev)
        self.grouping = torch.empty(ops.moe_grouping_bytes(ncols, topk), dtype=u8, device=dev)
        # h and the shared hs live in one buffer when they have the same width
        # (rows [0, ncols*topk) routed, then ncols shared rows), so one launch
        # quantises both
        R = ncols * topk
        self.joint = bool(shared_rows) and shared_rows == inter
        rows = R + (ncols if self.joint else 0)
        self.hh = torch.zeros((rows, inter), dtype=f32, device=dev)
        self.hhq = torch.zeros((rows, inter // QK * Q81), dtype=u8, device=dev)
        self.h = self.hh[:R].view(ncols, topk, inter)
        self.hq = self.hhq[:R]
        self.y = torch.zeros((ncols, topk, hidden), dtype=f32, device=dev)
        self.out = torch.empty((ncols, hidden), dtype=f32, device=dev)
        if shared_rows:
            if self.joint:
                self.hs = self.hh[R:]
                self.hsq = self.hhq[R:]
            else:
                self.hs = torch.empty((ncols, shared_rows), dtype=f32, device=dev)
                self.hsq = torch.empty((ncols, shared_rows // QK * Q81), dtype=u8, device=dev)
            self.ys = torch.empty((ncols, hidden), dtype=f32, device=dev)
            # the shared expert needs only xq, so it runs on a second stream
            # beside the routed path (a parallel branch when captured)
            self.side = side_stream if side_stream is not None else torch.cuda.Stream(device=dev)
            self.fork = torch.cuda.Event()
            self.join = torch.cuda.Event()
        else:
            self.hs = self.hsq = self.ys = None
            self.side = None


def forward(x: torch.Tensor, logits: torch.Tensor, bias: torch.Tensor | None,
            owner_slot: torch.Tensor | None, n_local_expert: int, experts: RoutedExperts,
            shared: SharedExpertShare | None, ws: Workspace, hook=None, fused: bool = True,
            add_shared: bool = False):
    """Enqueue one layer on the current stream; returns (out, ys) device tensors
    of the workspace.  out is the routed experts' weighted sum, or with
    add_shared (and a shared share) the MoE block's whole output: that sum plus
    the shared expert's ys, added inside the combine launch.

    fused=True (four launches): prologue (router + q8_1 of x), grouped gate/up
    with the shared gate/up rows as extra items, grouped down that quantises h
    and hs to q8_1 in the launch with the shared down slice as extra items,
    combine.
    fused=False: the nine separate calls, the shared expert on a second stream.
    Both give the same bits.  ``hook(name, phase)`` (unfused only) is called
    around each launch."""
    add = add_shared and shared is not None
    if experts.packed or (shared is not None and shared.packed):
        if experts.fmt == "q4":
            if shared is not None and shared.packed:
                raise ValueError("the 4-bit layer runs its Q8_0 shared share on the plain layout")
        else:
            if not fused:
                raise ValueError("packed weights run on the fused path")
            if shared is not None and shared.packed != experts.packed:
                raise ValueError("routed and shared weights must share one layout")
    if experts.fmt == "q4":
        return _forward_q4(x, logits, bias, owner_slot, n_local_expert, experts, shared, ws, add)
    if experts.fmt != "q8_0":
        raise ValueError("experts.fmt must be 'q8_0' or 'q4'")
    if fused:
        return _forward_fused(x, logits, bias, owner_slot, n_local_expert, experts, shared, ws, add)
    c, topk = ws.ncols, ws.topk
    hidden, inter = experts.hidden, experts.inter
    mark = hook or (lambda name, phase: None)

    mark("q8_1_x", "begin")
    ops.q8_1_quantize_rows(x, out=ws.xq)
    mark("q8_1_x", "end")
    main = torch.cuda.current_stream(x.device)
    if shared is not None:
        ws.fork.record(main)
        ws.side.wait_event(ws.fork)
        with torch.cuda.stream(ws.side):
            rb = (hidden // QK) * Q80
            mark("shared_pair", "begin")
            ops.mmvq_q8_0_glu_pair(shared.gate, shared.up, ws.xq, shared.rows, hidden, ncols=c,
                                   w_offset_bytes=shared.gate_offset(), w_row_stride_bytes=rb,
                                   out=ws.hs)
            mark("shared_pair", "end")
            ops.q8_1_quantize_rows(ws.hs, out=ws.hsq)
            kb = shared.down_block_offset()
            mark("shared_down", "begin")
            ops.mmvq_q8_0(shared.down, ws.hsq, hidden, shared.rows, ncols=c, k_block_offset=kb,
                          w_offset_bytes=kb * Q80,
                          w_row_stride_bytes=(shared.inter_full // QK) * Q80, out=ws.ys)
            mark("shared_down", "end")
            ws.join.record(ws.side)
    mark("route", "begin")
    ops.moe_route_topk(logits, topk, bias=bias, owner_slot=owner_slot, n_local_expert=n_local_expert,
                       ids=ws.ids, weights=ws.weights, grouping=ws.grouping)
    mark("route", "end")
    mark("grouped_gate_up", "begin")
    ops.moe_grouped_mmvq(ops.GATE_UP_SWIGLU, experts.gate, experts.up, ws.xq, ws.grouping,
                         n=inter, k=hidden, n_local_expert=experts.n_local, ncols=c, topk=topk,
                         out=ws.h)
    mark("grouped_gate_up", "end")
    mark("q8_1_h", "begin")
    ops.q8_1_quantize_rows(ws.h.view(c * topk, inter), out=ws.hq)
    mark("q8_1_h", "end")
    mark("grouped_down", "begin")
    ops.moe_grouped_mmvq(ops.DOWN, experts.down, None, ws.hq, ws.grouping, n=hidden, k=inter,
                         n_local_expert=experts.n_local, ncols=c, topk=topk, out=ws.y)
    mark("grouped_down", "end")
    if add:
        main.wait_event(ws.join)                  # the combine reads ys
    mark("combine", "begin")
    ops.moe_combine(ws.y, ws.ids, ws.weights, out=ws.out, shared=ws.ys if add else None)
    mark("combine", "end")
    if shared is not None and not add:
        main.wait_event(ws.join)
    return ws.out, ws.ys


def _rounds(chunk0: int, nchunks: int):
    r0 = chunk0 // 16
    r1 = (chunk0 + nchunks - 1) // 16
    n = r1 - r0 + 1
    return (1, 1) if n == 1 else (2, 1) if n == 2 else (4, 1) if n <= 4 else (1, n)


def _same_round_span(k_block_offset: int, k_slice: int, k: int) -> bool:
    """Whether a column-range slice can share a launch with full rows of length
    k: same length and the same lane-group layout."""
    return k_slice == k and _rounds(k_block_offset // 2, k_slice // 64) == _rounds(0, k // 64)


def _forward_fused(x, logits, bias, owner_slot, n_local_expert, experts, shared, ws, add):
    """Prologue, gate/up (+ shared rows), down with the q8_1 quantisation of h
    and hs inside the launch (+ shared slice), combine: four launches on one
    stream.  A shared slice whose length or lane layout differs from the
    routed down product's gets its own quantisation and MMVQ launches."""
    c, topk = ws.ncols, ws.topk
    hidden, inter = experts.hidden, experts.inter
    ops.moe_route_topk_quantize(x, logits, topk, bias=bias, owner_slot=owner_slot,
                                n_local_expert=n_local_expert, xq=ws.xq, ids=ws.ids,
                                weights=ws.weights, grouping=ws.grouping)
    R = c * topk
    sh_gu = sh_dn = None
    if shared is not None:
        rb = (hidden // QK) * Q80
        sh_gu = {"a": shared.gate, "b": shared.up, "row_stride": rb, "n": shared.rows,
                 "k": hidden, "k_block_offset": 0, "offset_bytes": shared.gate_offset(),
                 "out": ws.hs}
        kb = shared.down_block_offset()
        if shared.packed:
            # the round-major packed matrix of the share's round (a one-round
            # slice's products do not depend on its round)
            if shared.rows != ops.ROUND_BYTES // Q80 * QK or kb % (shared.rows // QK) != 0:
                raise ValueError("a packed shared down share must be one whole 1024-value round")
            rnd = kb // (shared.rows // QK)
            sh_dn = {"a": shared.down, "row_stride": ops.ROUND_BYTES, "n": hidden, "k": shared.rows,
                     "k_block_offset": 0, "offset_bytes": rnd * hidden * ops.ROUND_BYTES,
                     "out": ws.ys, "act": ws.hs}
        elif _same_round_span(kb, shared.rows, inter):
            sh_dn = {"a": shared.down, "row_stride": (shared.inter_full // QK) * Q80,
                     "n": hidden, "k": shared.rows, "k_block_offset": kb,
                     "offset_bytes": kb * Q80, "out": ws.ys, "act": ws.hs}
    gate_up = ops.GATE_UP_SWIGLU_P64 if experts.packed else ops.GATE_UP_SWIGLU
    ops.moe_grouped_mmvq_ex(gate_up, experts.gate, experts.up, ws.xq, ws.grouping,
                            n=inter, k=hidden, n_local_expert=experts.n_local, ncols=c, topk=topk,
                            out=ws.h, shared=sh_gu)
    down = ops.DOWN_F32_ACT_P64 if experts.packed else ops.DOWN_F32_ACT
    ops.moe_grouped_mmvq_ex(down, experts.down, None, ws.h.view(R, inter), ws.grouping,
                            n=hidden, k=inter, n_local_expert=experts.n_local, ncols=c, topk=topk,
                            out=ws.y, shared=sh_dn)
    if shared is not None and sh_dn is None:
        if shared.packed:
            raise ValueError("a packed shared down must ride in the down launch (same slice shape)")
        kb = shared.down_block_offset()
        ops.q8_1_quantize_rows(ws.hs, out=ws.hsq)
        ops.mmvq_q8_0(shared.down, ws.hsq, hidden, shared.rows, ncols=c, k_block_offset=kb,
                      w_offset_bytes=kb * Q80, w_row_stride_bytes=(shared.inter_full // QK) * Q80,
                      out=ws.ys)
    ops.moe_combine(ws.y, ws.ids, ws.weights, out=ws.out, shared=ws.ys if add else None)
    return ws.out, ws.ys


class WideWorkspace:
    """Buffers of one wide-batch layer (up to 1024 columns, no shared expert)."""

    def __init__(self, ncols: int, hidden: int, inter: int, topk: int, device):
        dev = torch.device(device)
        u8, f32 = torch.uint8, torch.float32
        R = ncols * topk
        self.ncols, self.topk = ncols, topk
        self.xq = torch.empty((ncols, hidden // QK * Q81), dtype=u8, device=dev)
        self.ids = torch.empty((ncols, topk), dtype=torch.int32, device=dev)
        self.weights = torch.empty((ncols, topk), dtype=f32, device=dev)
        self.grouping = torch.empty(ops.moe_grouping_bytes_wide(ncols, topk), dtype=u8, device=dev)
        self.h = torch.zeros((ncols, topk, inter), dtype=f32, device=dev)
        self.hq = torch.zeros((R, inter // QK * Q81), dtype=u8, device=dev)
        self.y = torch.zeros((ncols, topk, hidden), dtype=f32, device=dev)
        self.out = torch.empty((ncols, hidden), dtype=f32, device=dev)


def wide_products_for(ncols: int, topk: int, n_local_expert: int) -> str:
    """The faster grouped products for a batch: the matrix-core GEMM once the
    mean expert serves about four routes or more, else the MMVQ passes
    (measured on 256 experts, top-8: 32 columns, one route per expert, MMVQ
    282 vs GEMM 315 us a layer; 128 columns, four routes, GEMM 512 vs 636)."""
    return "gemm" if ncols * topk >= 4 * n_local_expert else "mmvq"


def forward_wide(x: torch.Tensor, logits: torch.Tensor, bias: torch.Tensor | None,
                 owner_slot: torch.Tensor | None, n_local_expert: int, experts: RoutedExperts,
                 ws: WideWorkspace, products: str = "auto"):
    """A routed layer over many columns (prefill-like): q8_1 of x, per-column
    selection, one expert grouping, grouped gate/up + SwiGLU, q8_1 of h,
    grouped down, combine; seven launches on the current stream, nothing
    allocated.  products="gemm" runs the grouped products on the int8 matrix
    cores (moe_grouped_gemm), "mmvq" runs the grouped MMVQ in passes of 8
    columns, "auto" picks by the mean routes per expert.  Packed experts
    (pack_experts) run the MMVQ passes on the packed stages, the down
    quantising h in its launch (six launches, the same bits); the GEMM reads
    the plain layout, its gate/up the GEMM layout when the experts carry it
    (pack_gemm_experts; the same bits).  Returns ws.out."""
    if products == "auto":
        products = "mmvq" if experts.packed else wide_products_for(ws.ncols, ws.topk, experts.n_local)
    if products not in ("gemm", "mmvq"):
        raise ValueError("products must be 'gemm', 'mmvq' or 'auto'")
    if experts.packed and products == "gemm":
        raise ValueError("the wide GEMM reads the plain Q8_0 layout, not packed weights")
    grouped = ops.moe_grouped_gemm if products == "gemm" else ops.moe_grouped_mmvq
    c, topk = ws.ncols, ws.topk
    hidden, inter = experts.hidden, experts.inter
    ops.q8_1_quantize_rows(x, out=ws.xq)
    ops.moe_route_topk_wide(logits, topk, bias=bias, owner_slot=owner_slot,
                            n_local_expert=n_local_expert, ids=ws.ids, weights=ws.weights)
    ops.moe_group_routes(ws.ids, experts.n_local, grouping=ws.grouping)
    if experts.packed:
        ops.moe_grouped_mmvq_ex(ops.GATE_UP_SWIGLU_P64, experts.gate, experts.up, ws.xq, ws.grouping,
                                n=inter, k=hidden, n_local_expert=experts.n_local, ncols=c, topk=topk,
                                out=ws.h)
        ops.moe_grouped_mmvq_ex(ops.DOWN_F32_ACT_P64, experts.down, None, ws.h.view(c * topk, inter),
                                ws.grouping, n=hidden, k=inter, n_local_expert=experts.n_local, ncols=c,
                                topk=topk, out=ws.y)
    else:
        if products == "gemm" and experts.gemm_gate is not None:
            ops.moe_grouped_gemm(ops.GATE_UP_SWIGLU_G8, experts.gemm_gate, experts.gemm_up, ws.xq, ws.grouping,
                                 n=inter, k=hidden, n_local_expert=experts.n_local, ncols=c, topk=topk,
                                 out=ws.h)
        else:
            grouped(ops.GATE_UP_SWIGLU, experts.gate, experts.up, ws.xq, ws.grouping, n=inter, k=hidden,
                    n_local_expert=experts.n_local, ncols=c, topk=topk, out=ws.h)
        ops.q8_1_quantize_rows(ws.h.view(c * topk, inter), out=ws.hq)
        if products == "gemm" and experts.gemm_down is not None:
            ops.moe_grouped_gemm(ops.DOWN_G8, experts.gemm_down, None, ws.hq, ws.grouping, n=hidden, k=inter,
                                 n_local_expert=experts.n_local, ncols=c, topk=topk, out=ws.y)
        else:
            grouped(ops.DOWN, experts.down, None, ws.hq, ws.grouping, n=hidden, k=inter,
                    n_local_expert=experts.n_local, ncols=c, topk=topk, out=ws.y)
    ops.moe_combine(ws.y, ws.ids, ws.weights, out=ws.out)
    return ws.out


def _forward_q4(x, logits, bias, owner_slot, n_local_expert, experts, shared, ws, add):
    """The layer with 4-bit routed experts: prologue, grouped gate/up,
    grouped down quantising h in the launch, combine (four launches), on the
    plain or (experts.packed) the 64-chunk packed stages; a shared expert
    (Q8_0, plain layout) runs as its own pair, quantisation and down calls."""
    c, topk = ws.ncols, ws.topk
    hidden, inter = experts.hidden, experts.inter
    ops.moe_route_topk_quantize(x, logits, topk, bias=bias, owner_slot=owner_slot,
                                n_local_expert=n_local_expert, xq=ws.xq, ids=ws.ids,
                                weights=ws.weights, grouping=ws.grouping)
    R = c * topk
    gate_up = ops.GATE_UP_SWIGLU_P64 if experts.packed else ops.GATE_UP_SWIGLU
    down = ops.DOWN_F32_ACT_P64 if experts.packed else ops.DOWN_F32_ACT
    ops.moe_grouped_mmvq_q4(gate_up, experts.gate, experts.up, ws.xq, ws.grouping,
                            n=inter, k=hidden, n_local_expert=experts.n_local, ncols=c, topk=topk,
                            out=ws.h)
    ops.moe_grouped_mmvq_q4(down, experts.down, None, ws.h.view(R, inter), ws.grouping,
                            n=hidden, k=inter, n_local_expert=experts.n_local, ncols=c, topk=topk,
                            out=ws.y)
    if shared is not None:
        rb = (hidden // QK) * Q80
        ops.mmvq_q8_0_glu_pair(shared.gate, shared.up, ws.xq, shared.rows, hidden, ncols=c,
                               w_offset_bytes=shared.gate_offset(), w_row_stride_bytes=rb, out=ws.hs)
        ops.q8_1_quantize_rows(ws.hs, out=ws.hsq)
        kb = shared.down_block_offset()
        ops.mmvq_q8_0(shared.down, ws.hsq, hidden, shared.rows, ncols=c, k_block_offset=kb,
                      w_offset_bytes=kb * Q80, w_row_stride_bytes=(shared.inter_full // QK) * Q80,
                      out=ws.ys)
    ops.moe_combine(ws.y, ws.ids, ws.weights, out=ws.out, shared=ws.ys if add else None)
    return ws.out, ws.ys


def pack_experts(experts: RoutedExperts, shared: SharedExpertShare | None = None):
    """Copies of the weights in the packed layouts the fused launches read
    (allocated here): gate and up in the 64-chunk layout, down in the
    round-major four-row layout (the shared share's down slice is then the
    matrix of its round).  4-bit experts take ops.q4_pack64_rows for all three
    (down: each quad of four rows packed as one row of 4096 values), and their
    layer's Q8_0 shared share stays plain.  Returns (experts, shared)."""
    if experts.fmt not in ("q8_0", "q4") or experts.packed:
        raise ValueError("pack_experts takes plain Q8_0 or 4-bit experts")
    rows = experts.n_local * experts.inter
    if experts.fmt == "q4":
        if experts.hidden != ops.P64_K or experts.inter != 1024:
            raise ValueError("the packed 4-bit stages take hidden 4096 and inter 1024")
        pe = RoutedExperts(ops.q4_pack64_rows(experts.gate, rows, experts.hidden),
                           ops.q4_pack64_rows(experts.up, rows, experts.hidden),
                           ops.q4_pack64_rows(experts.down, experts.n_local * experts.hidden // 4,
                                              4 * experts.inter),
                           experts.n_local, experts.hidden, experts.inter, fmt="q4", packed=True)
        return pe, shared
    pe = RoutedExperts(ops.q8_0_pack64_rows(experts.gate, rows, experts.hidden),
                       ops.q8_0_pack64_rows(experts.up, rows, experts.hidden),
                       ops.q8_0_pack64_rounds(experts.down, experts.n_local * experts.hidden, experts.inter),
                       experts.n_local, experts.hidden, experts.inter, packed=True)
    ps = None
    if shared is not None:
        rb = shared.hidden // QK * Q80
        rd = shared.inter_full // QK * Q80
        g = ops.q8_0_pack64_rows(shared.gate, shared.inter_full, shared.hidden).view(shared.inter_full, rb)
        u = ops.q8_0_pack64_rows(shared.up, shared.inter_full, shared.hidden).view(shared.inter_full, rb)
        d = ops.q8_0_pack64_rounds(shared.down, shared.hidden, shared.inter_full).view(shared.hidden, rd)
        ps = SharedExpertShare(g, u, d, shared.hidden, shared.inter_full, shared.row0, shared.rows,
                               packed=True)
    return pe, ps


def pack_gemm_experts(experts: RoutedExperts, down: bool = True) -> RoutedExperts:
    """The experts with copies of gate, up and (with down=True) down in the
    grouped GEMM's layout (ops.q8_0_pack_gemm_rows, allocated here) for
    forward_wide's matrix-core products; the plain matrices stay for the
    MMVQ passes."""
    if experts.fmt != "q8_0" or experts.packed:
        raise ValueError("pack_gemm_experts takes plain Q8_0 experts")
    if experts.hidden % 256 or experts.inter % 32:
        raise ValueError("the GEMM layout takes hidden % 256 == 0 and inter % 32 == 0")
    if down and (experts.inter % 256 or experts.hidden % 64):
        raise ValueError("the GEMM layout of the down takes inter % 256 == 0 and hidden % 64 == 0")
    rows = experts.n_local * experts.inter
    return RoutedExperts(experts.gate, experts.up, experts.down, experts.n_local, experts.hidden,
                         experts.inter, gemm_gate=ops.q8_0_pack_gemm_rows(experts.gate, rows, experts.hidden),
                         gemm_up=ops.q8_0_pack_gemm_rows(experts.up, rows, experts.hidden),
                         gemm_down=(ops.q8_0_pack_gemm_rows(experts.down, experts.n_local * experts.hidden,
                                                            experts.inter) if down else None))


def expert_bytes_q4(hidden: int, inter: int) -> int:
    """Bytes of one routed expert in 4-bit blocks (gate + up + down)."""
    return 3 * inter * (hidden // QK) * ops.Q4_BLOCK_BYTES


def expert_bytes(hidden: int, inter: int) -> int:
    """Q8_0 bytes of one routed expert (gate + up + down)."""
    return 3 * inter * (hidden // QK) * Q80


def shared_share_bytes(hidden: int, rows: int) -> int:
    """Q8_0 bytes one shared-expert share reads: gate/up rows and the down slice."""
    return 2 * rows * (hidden // QK) * Q80 + hidden * (rows // QK) * Q80
