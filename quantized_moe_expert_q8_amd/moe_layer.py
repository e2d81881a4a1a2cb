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
and can be captured in a HIP graph.  No arithmetic happens here.
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
    """Local experts of one layer, Q8_0, each [rows][k/32] blocks, experts
    ``expert_stride`` bytes apart (views into larger tensors are fine)."""
    gate: torch.Tensor       # uint8, n_local x inter x hidden/32 blocks
    up: torch.Tensor
    down: torch.Tensor       # uint8, n_local x hidden x inter/32 blocks
    n_local: int
    hidden: int
    inter: int


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

    def gate_offset(self) -> int:
        return self.row0 * (self.hidden // QK) * Q80

    def down_block_offset(self) -> int:
        return self.row0 // QK


class Workspace:
    def __init__(self, ncols: int, hidden: int, inter: int, topk: int, shared_rows: int, device):
        dev = torch.device(device)
        u8, f32 = torch.uint8, torch.float32
        self.ncols, self.topk = ncols, topk
        self.xq = torch.empty((ncols, hidden // QK * Q81), dtype=u8, device=dev)
        self.ids = torch.empty((ncols, topk), dtype=torch.int32, device=dev)
        self.weights = torch.empty((ncols, topk), dtype=f32, device=dev)
        self.grouping = torch.empty(ops.moe_grouping_bytes(ncols, topk), dtype=u8, device=dev)
        self.h = torch.zeros((ncols, topk, inter), dtype=f32, device=dev)
        self.hq = torch.empty((ncols * topk, inter // QK * Q81), dtype=u8, device=dev)
        self.y = torch.zeros((ncols, topk, hidden), dtype=f32, device=dev)
        self.out = torch.empty((ncols, hidden), dtype=f32, device=dev)
        if shared_rows:
            self.hs = torch.empty((ncols, shared_rows), dtype=f32, device=dev)
            self.hsq = torch.empty((ncols, shared_rows // QK * Q81), dtype=u8, device=dev)
            self.ys = torch.empty((ncols, hidden), dtype=f32, device=dev)
        else:
            self.hs = self.hsq = self.ys = None


def forward(x: torch.Tensor, logits: torch.Tensor, bias: torch.Tensor | None,
            owner_slot: torch.Tensor | None, n_local_expert: int, experts: RoutedExperts,
            shared: SharedExpertShare | None, ws: Workspace, hook=None):
    """Enqueue one layer on the current stream.  ``hook(name, phase)`` (optional)
    is called before ('begin') and after ('end') each launch, e.g. to record
    events.  Returns (out, ys) device tensors of the workspace."""
    c, topk = ws.ncols, ws.topk
    hidden, inter = experts.hidden, experts.inter
    mark = hook or (lambda name, phase: None)

    mark("q8_1_x", "begin")
    ops.q8_1_quantize_rows(x, out=ws.xq)
    mark("q8_1_x", "end")
    if shared is not None:
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
                      w_offset_bytes=kb * Q80, w_row_stride_bytes=(shared.inter_full // QK) * Q80,
                      out=ws.ys)
        mark("shared_down", "end")
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
    mark("combine", "begin")
    ops.moe_combine(ws.y, ws.ids, ws.weights, out=ws.out)
    mark("combine", "end")
    return ws.out, ws.ys


def expert_bytes(hidden: int, inter: int) -> int:
    """Q8_0 bytes of one routed expert (gate + up + down)."""
    return 3 * inter * (hidden // QK) * Q80


def shared_share_bytes(hidden: int, rows: int) -> int:
    """Q8_0 bytes one shared-expert share reads: gate/up rows and the down slice."""
    return 2 * rows * (hidden // QK) * Q80 + hidden * (rows // QK) * Q80
