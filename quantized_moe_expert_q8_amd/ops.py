"""Thin torch wrappers over the libmoeq8 C ABI (include/moeq8.h).

Each function takes device tensors, checks dtypes, devices and that every
buffer the kernel will touch lies inside its tensor, then calls the C entry
point of the same name on the current HIP stream.  All arithmetic runs in the
library's kernels; torch only provides memory and the stream.
"""

from __future__ import annotations

import ctypes

import torch

from ._lib import call, lib

QK = 32
Q8_0_BLOCK_BYTES = 34
Q8_1_BLOCK_BYTES = 36
EXCHANGE_BLOCK_BYTES = 36
Q4_BLOCK_BYTES = 18
MAX_COLS = 8
GATE_UP_SWIGLU = 0
DOWN = 1
DOWN_F32_ACT = 2
GATE_UP_SWIGLU_P64 = 3      # gate/up on weights repacked by q8_0_pack64_rows
DOWN_F32_ACT_P64 = 4        # down (fp32 h) on weights repacked by q8_0_pack64_rounds
GATE_UP_SWIGLU_G8 = 5       # moe_grouped_gemm gate/up on weights repacked by q8_0_pack_gemm_rows
DOWN_G8 = 6                 # moe_grouped_gemm down on weights repacked by q8_0_pack_gemm_rows
ROUND_BYTES = 1088          # a 1024-value round of Q8_0 blocks
P64_K = 4096                # values in one packed segment


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t, offset: int = 0):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr() + offset)


def _cuda(t: torch.Tensor, name: str, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _nbytes_from_ptr(t: torch.Tensor) -> int:
    """Bytes from t.data_ptr() to the end of t's storage."""
    st = t.untyped_storage()
    return st.data_ptr() + st.nbytes() - t.data_ptr()


def _need(t: torch.Tensor, name: str, nbytes: int, offset: int = 0):
    if offset < 0 or offset + nbytes > _nbytes_from_ptr(t):
        raise ValueError(f"{name}: {nbytes} bytes at offset {offset} exceed the tensor's storage")


def _contig_rows(t: torch.Tensor, name: str, rows: int, row_elems: int):
    if t.dim() != 2 or t.shape[0] < rows or t.shape[1] < row_elems or t.stride(1) != 1:
        raise ValueError(f"{name} must be [>= {rows}, >= {row_elems}] with unit inner stride")


# ---------------------------------------------------------------------------
# quantisers
# ---------------------------------------------------------------------------

def q8_1_quantize_rows(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """x fp32 [rows, k] -> q8_1 blocks uint8 [rows, k/32*36]."""
    _cuda(x, "x", torch.float32)
    rows, k = x.shape
    _contig_rows(x, "x", rows, k)
    if out is None:
        out = torch.empty((rows, k // QK * Q8_1_BLOCK_BYTES), dtype=torch.uint8, device=x.device)
    _cuda(out, "out", torch.uint8)
    _need(out, "out", rows * (k // QK) * Q8_1_BLOCK_BYTES)
    call("q8_1_quantize_rows", _ptr(x), rows, k, x.stride(0), _ptr(out), _stream(x))
    return out


def q8_0_quantize_rows(w: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """w fp32 [rows, k] -> Q8_0 blocks uint8 [rows, k/32*34]."""
    _cuda(w, "w", torch.float32)
    rows, k = w.shape
    _contig_rows(w, "w", rows, k)
    if out is None:
        out = torch.empty((rows, k // QK * Q8_0_BLOCK_BYTES), dtype=torch.uint8, device=w.device)
    _cuda(out, "out", torch.uint8)
    _need(out, "out", rows * (k // QK) * Q8_0_BLOCK_BYTES)
    call("q8_0_quantize_rows", _ptr(w), rows, k, w.stride(0), _ptr(out), _stream(w))
    return out


def q8_0_pack64_rows(src: torch.Tensor, rows: int, k: int, out: torch.Tensor | None = None,
                     src_row_stride_bytes: int | None = None,
                     out_row_stride_bytes: int | None = None) -> torch.Tensor:
    """Q8_0 rows (uint8, rows of k/32*34 bytes) -> the same rows in the 64-chunk
    packed layout that GATE_UP_SWIGLU_P64 reads; k a multiple of 4096."""
    row_bytes = k // QK * Q8_0_BLOCK_BYTES
    ss = row_bytes if src_row_stride_bytes is None else src_row_stride_bytes
    ds = row_bytes if out_row_stride_bytes is None else out_row_stride_bytes
    _cuda(src, "src", torch.uint8)
    _need(src, "src", _weight_extent(rows, k, ss))
    if out is None:
        out = torch.empty(rows * ds, dtype=torch.uint8, device=src.device)
    _cuda(out, "out", torch.uint8)
    _need(out, "out", _weight_extent(rows, k, ds))
    call("q8_0_pack64_rows", _ptr(src), rows, k, ss, _ptr(out), ds, _stream(src))
    return out


def q8_0_pack64_rounds(src: torch.Tensor, rows: int, k: int, out: torch.Tensor | None = None,
                       src_row_stride_bytes: int | None = None) -> torch.Tensor:
    """Q8_0 rows -> the round-major four-row packed layout DOWN_F32_ACT_P64
    reads: k/1024 matrices [rows][1088 bytes] (round r at byte r*rows*1088);
    rows a multiple of 4, k a multiple of 1024."""
    row_bytes = k // QK * Q8_0_BLOCK_BYTES
    ss = row_bytes if src_row_stride_bytes is None else src_row_stride_bytes
    _cuda(src, "src", torch.uint8)
    _need(src, "src", _weight_extent(rows, k, ss))
    if out is None:
        out = torch.empty(rows * row_bytes, dtype=torch.uint8, device=src.device)
    _cuda(out, "out", torch.uint8)
    _need(out, "out", rows * row_bytes)
    call("q8_0_pack64_rounds", _ptr(src), rows, k, ss, _ptr(out), _stream(src))
    return out


def q8_0_pack_gemm_rows(src: torch.Tensor, rows: int, k: int, out: torch.Tensor | None = None,
                        src_row_stride_bytes: int | None = None,
                        out_row_stride_bytes: int | None = None) -> torch.Tensor:
    """Q8_0 rows -> the grouped GEMM's layout that GATE_UP_SWIGLU_G8 reads (per
    8-block group: 16 bytes of scales, then the quants 8-byte aligned, the
    8-byte halves of each 16-byte piece swapped in rows i % 16 >= 8); k a
    multiple of 256; pack whole expert matrices from their first row."""
    row_bytes = k // QK * Q8_0_BLOCK_BYTES
    ss = row_bytes if src_row_stride_bytes is None else src_row_stride_bytes
    ds = row_bytes if out_row_stride_bytes is None else out_row_stride_bytes
    _cuda(src, "src", torch.uint8)
    _need(src, "src", _weight_extent(rows, k, ss))
    if out is None:
        out = torch.empty(rows * ds, dtype=torch.uint8, device=src.device)
    _cuda(out, "out", torch.uint8)
    _need(out, "out", _weight_extent(rows, k, ds))
    call("q8_0_pack_gemm_rows", _ptr(src), rows, k, ss, _ptr(out), ds, _stream(src))
    return out


def q4_pack64_rows(src: torch.Tensor, rows: int, k: int, out: torch.Tensor | None = None,
                   src_row_stride_bytes: int | None = None,
                   out_row_stride_bytes: int | None = None) -> torch.Tensor:
    """4-bit rows (uint8, rows of k/32*18 bytes) -> the same rows in the 64-chunk
    packed layout the 4-bit GATE_UP_SWIGLU_P64 reads; k a multiple of 4096.  The
    4-bit DOWN_F32_ACT_P64 (k = 1024) takes each quad of four consecutive rows
    packed as one row of 4096 values: rows/4 rows, k = 4096."""
    row_bytes = k // QK * Q4_BLOCK_BYTES
    ss = row_bytes if src_row_stride_bytes is None else src_row_stride_bytes
    ds = row_bytes if out_row_stride_bytes is None else out_row_stride_bytes
    _cuda(src, "src", torch.uint8)
    _need(src, "src", _weight_extent(rows, k, ss, Q4_BLOCK_BYTES))
    if out is None:
        out = torch.empty(rows * ds, dtype=torch.uint8, device=src.device)
    _cuda(out, "out", torch.uint8)
    _need(out, "out", _weight_extent(rows, k, ds, Q4_BLOCK_BYTES))
    call("q4_pack64_rows", _ptr(src), rows, k, ss, _ptr(out), ds, _stream(src))
    return out


# ---------------------------------------------------------------------------
# 8-bit block exchange codec
# ---------------------------------------------------------------------------

def q8_block_encode(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Partials fp32 [rows, n] -> exchange blocks uint8 [rows, n/32*36]."""
    _cuda(x, "x", torch.float32)
    rows, n = x.shape
    _contig_rows(x, "x", rows, n)
    if out is None:
        out = torch.empty((rows, n // QK * EXCHANGE_BLOCK_BYTES), dtype=torch.uint8, device=x.device)
    _cuda(out, "out", torch.uint8)
    _need(out, "out", rows * (n // QK) * EXCHANGE_BLOCK_BYTES)
    call("q8_block_encode", _ptr(x), rows, n, x.stride(0), _ptr(out), _stream(x))
    return out


def q8_block_decode_sum(gathered: torch.Tensor, rows: int, n: int,
                        out: torch.Tensor | None = None) -> torch.Tensor:
    """gathered uint8 [nranks, >= rows*n/32*36] (rank r's blocks in row r) ->
    out fp32 [rows, n]: the ranks' dequantized values summed in rank order."""
    _cuda(gathered, "gathered", torch.uint8)
    if gathered.dim() != 2 or gathered.stride(1) != 1:
        raise ValueError("gathered must be [nranks, bytes] with unit inner stride")
    nranks = gathered.shape[0]
    need = rows * (n // QK) * EXCHANGE_BLOCK_BYTES
    if gathered.shape[1] < need:
        raise ValueError(f"gathered rows must hold {need} bytes")
    _need(gathered, "gathered", (nranks - 1) * gathered.stride(0) * gathered.element_size() + need)
    if out is None:
        out = torch.empty((rows, n), dtype=torch.float32, device=gathered.device)
    _cuda(out, "out", torch.float32)
    _contig_rows(out, "out", rows, n)
    call("q8_block_decode_sum", _ptr(gathered), nranks, gathered.stride(0), rows, n, _ptr(out),
         out.stride(0), _stream(gathered))
    return out


# ---------------------------------------------------------------------------
# products
# ---------------------------------------------------------------------------

def _weight_extent(n: int, k: int, row_stride: int, block_bytes: int = Q8_0_BLOCK_BYTES) -> int:
    return 0 if n == 0 else (n - 1) * row_stride + (k // QK) * block_bytes


def _weight_args(w, n, k, w_offset_bytes, w_row_stride_bytes, name="w", block_bytes=Q8_0_BLOCK_BYTES):
    _cuda(w, name, torch.uint8)
    if w_row_stride_bytes is None:
        w_row_stride_bytes = w.stride(0) if w.dim() == 2 else (k // QK) * block_bytes
    _need(w, name, _weight_extent(n, k, w_row_stride_bytes, block_bytes), w_offset_bytes)
    return w_row_stride_bytes


def _act_rows(xq, name, rows, k):
    _cuda(xq, name, torch.uint8)
    _need(xq, name, rows * (k // QK) * Q8_1_BLOCK_BYTES)


def mmvq_q8_0(w: torch.Tensor, xq: torch.Tensor, n: int, k: int, *, ncols: int | None = None,
              k_block_offset: int = 0, w_offset_bytes: int = 0,
              w_row_stride_bytes: int | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """y fp32 [ncols, n] = W . xq.  ``w`` holds Q8_0 rows; the matrix (or the
    column-range view) starts ``w_offset_bytes`` into it."""
    ncols = xq.shape[0] if ncols is None else ncols
    stride = _weight_args(w, n, k, w_offset_bytes, w_row_stride_bytes)
    _act_rows(xq, "xq", ncols, k)
    if out is None:
        out = torch.empty((ncols, n), dtype=torch.float32, device=w.device)
    _cuda(out, "out", torch.float32)
    _need(out, "out", ncols * n * 4)
    call("mmvq_q8_0", _ptr(w, w_offset_bytes), stride, n, k, k_block_offset, _ptr(xq), ncols,
         _ptr(out), _stream(w))
    return out


def mmvq_q8_0_glu_pair(w_gate: torch.Tensor, w_up: torch.Tensor, xq: torch.Tensor, n: int, k: int,
                       *, ncols: int | None = None, k_block_offset: int = 0,
                       w_offset_bytes: int = 0, w_row_stride_bytes: int | None = None,
                       out: torch.Tensor | None = None, g_out: torch.Tensor | None = None,
                       u_out: torch.Tensor | None = None) -> torch.Tensor:
    """h fp32 [ncols, n] = SwiGLU-DS4(Wg . xq, Wu . xq); optional raw products."""
    ncols = xq.shape[0] if ncols is None else ncols
    stride = _weight_args(w_gate, n, k, w_offset_bytes, w_row_stride_bytes, "w_gate")
    stride_u = _weight_args(w_up, n, k, w_offset_bytes, w_row_stride_bytes, "w_up")
    if stride_u != stride:
        raise ValueError("w_gate and w_up must share the row stride")
    _act_rows(xq, "xq", ncols, k)
    if out is None:
        out = torch.empty((ncols, n), dtype=torch.float32, device=w_gate.device)
    for t, nm in ((out, "out"), (g_out, "g_out"), (u_out, "u_out")):
        if t is not None:
            _cuda(t, nm, torch.float32)
            _need(t, nm, ncols * n * 4)
    call("mmvq_q8_0_glu_pair", _ptr(w_gate, w_offset_bytes), _ptr(w_up, w_offset_bytes), stride, n,
         k, k_block_offset, _ptr(xq), ncols, _ptr(out), _ptr(g_out), _ptr(u_out), _stream(w_gate))
    return out


# ---------------------------------------------------------------------------
# 4-bit weights (Q4 blocks: fp16 d, 32 codes of 4 bits, 18 bytes)
# ---------------------------------------------------------------------------

def q4_quantize_rows(w: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """w fp32 [rows, k] -> Q4 blocks uint8 [rows, k/32*18]."""
    _cuda(w, "w", torch.float32)
    rows, k = w.shape
    _contig_rows(w, "w", rows, k)
    if out is None:
        out = torch.empty((rows, k // QK * Q4_BLOCK_BYTES), dtype=torch.uint8, device=w.device)
    _cuda(out, "out", torch.uint8)
    _need(out, "out", rows * (k // QK) * Q4_BLOCK_BYTES)
    call("q4_quantize_rows", _ptr(w), rows, k, w.stride(0), _ptr(out), _stream(w))
    return out


def mmvq_q4(w: torch.Tensor, xq: torch.Tensor, n: int, k: int, *, ncols: int | None = None,
            k_block_offset: int = 0, w_offset_bytes: int = 0,
            w_row_stride_bytes: int | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """y fp32 [ncols, n] = W . xq with Q4 weight rows."""
    ncols = xq.shape[0] if ncols is None else ncols
    stride = _weight_args(w, n, k, w_offset_bytes, w_row_stride_bytes, block_bytes=Q4_BLOCK_BYTES)
    _act_rows(xq, "xq", ncols, k)
    if out is None:
        out = torch.empty((ncols, n), dtype=torch.float32, device=w.device)
    _cuda(out, "out", torch.float32)
    _need(out, "out", ncols * n * 4)
    call("mmvq_q4", _ptr(w, w_offset_bytes), stride, n, k, k_block_offset, _ptr(xq), ncols,
         _ptr(out), _stream(w))
    return out


def mmvq_q4_glu_pair(w_gate: torch.Tensor, w_up: torch.Tensor, xq: torch.Tensor, n: int, k: int,
                     *, ncols: int | None = None, k_block_offset: int = 0, w_offset_bytes: int = 0,
                     w_row_stride_bytes: int | None = None, out: torch.Tensor | None = None,
                     g_out: torch.Tensor | None = None, u_out: torch.Tensor | None = None) -> torch.Tensor:
    """h fp32 [ncols, n] = SwiGLU-DS4(Wg . xq, Wu . xq) with Q4 weights."""
    ncols = xq.shape[0] if ncols is None else ncols
    stride = _weight_args(w_gate, n, k, w_offset_bytes, w_row_stride_bytes, "w_gate", Q4_BLOCK_BYTES)
    stride_u = _weight_args(w_up, n, k, w_offset_bytes, w_row_stride_bytes, "w_up", Q4_BLOCK_BYTES)
    if stride_u != stride:
        raise ValueError("w_gate and w_up must share the row stride")
    _act_rows(xq, "xq", ncols, k)
    if out is None:
        out = torch.empty((ncols, n), dtype=torch.float32, device=w_gate.device)
    for t, nm in ((out, "out"), (g_out, "g_out"), (u_out, "u_out")):
        if t is not None:
            _cuda(t, nm, torch.float32)
            _need(t, nm, ncols * n * 4)
    call("mmvq_q4_glu_pair", _ptr(w_gate, w_offset_bytes), _ptr(w_up, w_offset_bytes), stride, n,
         k, k_block_offset, _ptr(xq), ncols, _ptr(out), _ptr(g_out), _ptr(u_out), _stream(w_gate))
    return out


def moe_grouped_mmvq_q4(stage: int, w_a: torch.Tensor, w_b: torch.Tensor | None, act: torch.Tensor,
                        grouping: torch.Tensor, *, n: int, k: int, n_local_expert: int, ncols: int,
                        topk: int, out: torch.Tensor | None = None,
                        expert_stride_bytes: int | None = None) -> torch.Tensor:
    """Grouped per-expert products with Q4 expert weights [n_local][n][k/32]:
    stages GATE_UP_SWIGLU and DOWN on q8_1 rows, DOWN_F32_ACT on fp32 h rows
    [ncols*topk, k]; GATE_UP_SWIGLU_P64 and DOWN_F32_ACT_P64 the same on weights
    repacked by q4_pack64_rows.  Returns out fp32 [ncols, topk, n]."""
    row_stride = (k // QK) * Q4_BLOCK_BYTES
    if expert_stride_bytes is None:
        expert_stride_bytes = n * row_stride
    extent = (n_local_expert - 1) * expert_stride_bytes + _weight_extent(n, k, row_stride, Q4_BLOCK_BYTES)
    _cuda(w_a, "w_a", torch.uint8)
    _need(w_a, "w_a", extent)
    act_stride = 0
    if stage in (GATE_UP_SWIGLU, GATE_UP_SWIGLU_P64):
        if w_b is None:
            raise ValueError("the gate/up stage needs w_b")
        _cuda(w_b, "w_b", torch.uint8)
        _need(w_b, "w_b", extent)
        _act_rows(act, "act", ncols, k)
    elif stage == DOWN:
        _act_rows(act, "act", ncols * topk, k)
    elif stage in (DOWN_F32_ACT, DOWN_F32_ACT_P64):
        _cuda(act, "act", torch.float32)
        _contig_rows(act, "act", ncols * topk, k)
        act_stride = act.stride(0)
    else:
        raise ValueError("stage must be GATE_UP_SWIGLU, DOWN, DOWN_F32_ACT or a packed one")
    _cuda(grouping, "grouping", torch.uint8)
    _need(grouping, "grouping", moe_grouping_bytes_wide(ncols, topk))
    if out is None:
        out = torch.empty((ncols, topk, n), dtype=torch.float32, device=w_a.device)
    _cuda(out, "out", torch.float32)
    _need(out, "out", ncols * topk * n * 4)
    call("moe_grouped_mmvq_q4", stage, _ptr(w_a), _ptr(w_b), expert_stride_bytes, row_stride,
         n_local_expert, n, k, _ptr(act), act_stride, _ptr(grouping), ncols, topk, _ptr(out),
         _stream(w_a))
    return out


def swiglu_ds4(g: torch.Tensor, u: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    _cuda(g, "g", torch.float32)
    _cuda(u, "u", torch.float32)
    if g.shape != u.shape or not g.is_contiguous() or not u.is_contiguous():
        raise ValueError("g and u must be contiguous and of one shape")
    if out is None:
        out = torch.empty_like(g)
    _cuda(out, "out", torch.float32)
    _need(out, "out", g.numel() * 4)
    call("swiglu_ds4", _ptr(g), _ptr(u), g.numel(), _ptr(out), _stream(g))
    return out


# ---------------------------------------------------------------------------
# routing, grouped products, combine
# ---------------------------------------------------------------------------

def moe_grouping_bytes(ncols: int, topk: int) -> int:
    return int(lib().moe_grouping_bytes(ncols, topk))


def moe_grouping_bytes_wide(ncols: int, topk: int) -> int:
    """Grouping size for up to MOEQ8_MAX_WIDE_COLS columns (the same layout and
    size formula as moe_grouping_bytes)."""
    return int(lib().moe_grouping_bytes_wide(ncols, topk))


def moe_route_topk_wide(logits: torch.Tensor, topk: int, *, bias: torch.Tensor | None = None,
                        owner_slot: torch.Tensor | None = None, n_local_expert: int | None = None,
                        ids: torch.Tensor | None = None, weights: torch.Tensor | None = None):
    """Selection and weights for up to 1024 columns (no grouping):
    returns (ids int32 [ncols, topk], weights fp32 [ncols, topk])."""
    _cuda(logits, "logits", torch.float32)
    if logits.dim() != 2 or not logits.is_contiguous():
        raise ValueError("logits must be contiguous [ncols, n_expert]")
    ncols, n_expert = logits.shape
    if n_local_expert is None:
        n_local_expert = n_expert if owner_slot is None else int(owner_slot.max().item()) + 1
    if bias is not None:
        _cuda(bias, "bias", torch.float32)
        _need(bias, "bias", n_expert * 4)
    if owner_slot is not None:
        _cuda(owner_slot, "owner_slot", torch.int32)
        _need(owner_slot, "owner_slot", n_expert * 4)
    dev = logits.device
    if ids is None:
        ids = torch.empty((ncols, topk), dtype=torch.int32, device=dev)
    if weights is None:
        weights = torch.empty((ncols, topk), dtype=torch.float32, device=dev)
    _need(ids, "ids", ncols * topk * 4)
    _need(weights, "weights", ncols * topk * 4)
    call("moe_route_topk_wide", _ptr(logits), _ptr(bias), _ptr(owner_slot), ncols, n_expert,
         n_local_expert, topk, _ptr(ids), _ptr(weights), _stream(logits))
    return ids, weights


def moe_group_routes(ids: torch.Tensor, n_local_expert: int, grouping: torch.Tensor | None = None):
    """The expert grouping of ids [ncols, topk] (any ncols up to 1024), in the
    layout moe_route_topk writes; returns the grouping tensor."""
    _cuda(ids, "ids", torch.int32)
    if ids.dim() != 2 or not ids.is_contiguous():
        raise ValueError("ids must be contiguous [ncols, topk]")
    ncols, topk = ids.shape
    gb = moe_grouping_bytes_wide(ncols, topk)
    if gb == 0:
        raise ValueError("ncols or topk out of range")
    if grouping is None:
        grouping = torch.empty(gb, dtype=torch.uint8, device=ids.device)
    _cuda(grouping, "grouping", torch.uint8)
    _need(grouping, "grouping", gb)
    call("moe_group_routes", _ptr(ids), ncols, topk, n_local_expert, _ptr(grouping), _stream(ids))
    return grouping


def moe_route_topk(logits: torch.Tensor, topk: int, *, bias: torch.Tensor | None = None,
                   owner_slot: torch.Tensor | None = None, n_local_expert: int | None = None,
                   ids: torch.Tensor | None = None, weights: torch.Tensor | None = None,
                   grouping: torch.Tensor | None = None):
    """Returns (ids int32 [ncols, topk], weights fp32 [ncols, topk], grouping uint8)."""
    _cuda(logits, "logits", torch.float32)
    if logits.dim() != 2 or not logits.is_contiguous():
        raise ValueError("logits must be contiguous [ncols, n_expert]")
    ncols, n_expert = logits.shape
    if n_local_expert is None:
        n_local_expert = n_expert if owner_slot is None else int(owner_slot.max().item()) + 1
    if bias is not None:
        _cuda(bias, "bias", torch.float32)
        _need(bias, "bias", n_expert * 4)
    if owner_slot is not None:
        _cuda(owner_slot, "owner_slot", torch.int32)
        _need(owner_slot, "owner_slot", n_expert * 4)
    dev = logits.device
    if ids is None:
        ids = torch.empty((ncols, topk), dtype=torch.int32, device=dev)
    if weights is None:
        weights = torch.empty((ncols, topk), dtype=torch.float32, device=dev)
    gb = moe_grouping_bytes(ncols, topk)
    if gb == 0:
        raise ValueError("ncols or topk out of range")
    if grouping is None:
        grouping = torch.empty(gb, dtype=torch.uint8, device=dev)
    _need(ids, "ids", ncols * topk * 4)
    _need(weights, "weights", ncols * topk * 4)
    _need(grouping, "grouping", gb)
    call("moe_route_topk", _ptr(logits), _ptr(bias), _ptr(owner_slot), ncols, n_expert,
         n_local_expert, topk, _ptr(ids), _ptr(weights), _ptr(grouping), _stream(logits))
    return ids, weights, grouping


def _grouped_call(fn: str, stage: int, w_a, w_b, act_q, grouping, n, k, n_local_expert, ncols, topk,
                  expert_stride_bytes, w_row_stride_bytes, out):
    if w_row_stride_bytes is None:
        w_row_stride_bytes = (k // QK) * Q8_0_BLOCK_BYTES
    if expert_stride_bytes is None:
        expert_stride_bytes = n * w_row_stride_bytes
    extent = (n_local_expert - 1) * expert_stride_bytes + _weight_extent(n, k, w_row_stride_bytes)
    _cuda(w_a, "w_a", torch.uint8)
    _need(w_a, "w_a", extent)
    if stage in (GATE_UP_SWIGLU, GATE_UP_SWIGLU_G8):
        if stage == GATE_UP_SWIGLU_G8 and fn != "moe_grouped_gemm":
            raise ValueError("GATE_UP_SWIGLU_G8 is a stage of moe_grouped_gemm")
        if w_b is None:
            raise ValueError("the gate/up stage needs w_b")
        _cuda(w_b, "w_b", torch.uint8)
        _need(w_b, "w_b", extent)
        act_rows = ncols
    elif stage in (DOWN, DOWN_G8):
        if stage == DOWN_G8 and fn != "moe_grouped_gemm":
            raise ValueError("DOWN_G8 is a stage of moe_grouped_gemm")
        act_rows = ncols * topk
    else:
        raise ValueError("stage must be GATE_UP_SWIGLU, DOWN or (GEMM) GATE_UP_SWIGLU_G8, DOWN_G8")
    _act_rows(act_q, "act_q", act_rows, k)
    _cuda(grouping, "grouping", torch.uint8)
    _need(grouping, "grouping", moe_grouping_bytes_wide(ncols, topk))
    if out is None:
        out = torch.empty((ncols, topk, n), dtype=torch.float32, device=w_a.device)
    _cuda(out, "out", torch.float32)
    _need(out, "out", ncols * topk * n * 4)
    call(fn, stage, _ptr(w_a), _ptr(w_b), expert_stride_bytes, w_row_stride_bytes,
         n_local_expert, n, k, _ptr(act_q), _ptr(grouping), ncols, topk, _ptr(out), _stream(w_a))
    return out


def moe_grouped_mmvq(stage: int, w_a: torch.Tensor, w_b: torch.Tensor | None, act_q: torch.Tensor,
                     grouping: torch.Tensor, *, n: int, k: int, n_local_expert: int, ncols: int,
                     topk: int, expert_stride_bytes: int | None = None,
                     w_row_stride_bytes: int | None = None,
                     out: torch.Tensor | None = None) -> torch.Tensor:
    """Grouped per-expert MMVQ.  Experts are stored [n_local][n][k/32] blocks.
    Returns out fp32 [ncols, topk, n] (masked routes' rows untouched)."""
    return _grouped_call("moe_grouped_mmvq", stage, w_a, w_b, act_q, grouping, n, k, n_local_expert,
                         ncols, topk, expert_stride_bytes, w_row_stride_bytes, out)


def moe_grouped_gemm(stage: int, w_a: torch.Tensor, w_b: torch.Tensor | None, act_q: torch.Tensor,
                     grouping: torch.Tensor, *, n: int, k: int, n_local_expert: int, ncols: int,
                     topk: int, expert_stride_bytes: int | None = None,
                     w_row_stride_bytes: int | None = None,
                     out: torch.Tensor | None = None) -> torch.Tensor:
    """The grouped products on the int8 matrix cores (wide batches): same
    arguments and results as moe_grouped_mmvq, equal to rounding (n % 32 == 0).
    Stages GATE_UP_SWIGLU_G8 and DOWN_G8 take weights repacked by
    q8_0_pack_gemm_rows (the bits of GATE_UP_SWIGLU / DOWN on the plain rows)."""
    return _grouped_call("moe_grouped_gemm", stage, w_a, w_b, act_q, grouping, n, k, n_local_expert,
                         ncols, topk, expert_stride_bytes, w_row_stride_bytes, out)


def moe_router_scores(logits: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """The router's score of every logit (fp64 sigmoid rounded once to fp32),
    by the router's own device expression; any shape, fp32, contiguous."""
    _cuda(logits, "logits", torch.float32)
    if not logits.is_contiguous():
        raise ValueError("logits must be contiguous")
    if out is None:
        out = torch.empty_like(logits)
    _cuda(out, "out", torch.float32)
    _need(out, "out", logits.numel() * 4)
    call("moe_router_scores", _ptr(logits), logits.numel(), _ptr(out), _stream(logits))
    return out


def moe_route_topk_quantize(x: torch.Tensor, logits: torch.Tensor, topk: int, *,
                            bias: torch.Tensor | None = None,
                            owner_slot: torch.Tensor | None = None,
                            n_local_expert: int | None = None, xq: torch.Tensor | None = None,
                            ids: torch.Tensor | None = None, weights: torch.Tensor | None = None,
                            grouping: torch.Tensor | None = None):
    """One launch: xq = q8_1(x) and moe_route_topk(logits).  Returns
    (xq, ids, weights, grouping)."""
    _cuda(x, "x", torch.float32)
    _cuda(logits, "logits", torch.float32)
    ncols, k = x.shape
    _contig_rows(x, "x", ncols, k)
    if logits.dim() != 2 or not logits.is_contiguous() or logits.shape[0] != ncols:
        raise ValueError("logits must be contiguous [ncols, n_expert]")
    n_expert = logits.shape[1]
    if n_local_expert is None:
        n_local_expert = n_expert if owner_slot is None else int(owner_slot.max().item()) + 1
    dev = x.device
    if xq is None:
        xq = torch.empty((ncols, k // QK * Q8_1_BLOCK_BYTES), dtype=torch.uint8, device=dev)
    if ids is None:
        ids = torch.empty((ncols, topk), dtype=torch.int32, device=dev)
    if weights is None:
        weights = torch.empty((ncols, topk), dtype=torch.float32, device=dev)
    gb = moe_grouping_bytes(ncols, topk)
    if gb == 0:
        raise ValueError("ncols or topk out of range")
    if grouping is None:
        grouping = torch.empty(gb, dtype=torch.uint8, device=dev)
    if bias is not None:
        _cuda(bias, "bias", torch.float32)
        _need(bias, "bias", n_expert * 4)
    if owner_slot is not None:
        _cuda(owner_slot, "owner_slot", torch.int32)
        _need(owner_slot, "owner_slot", n_expert * 4)
    _need(xq, "xq", ncols * (k // QK) * Q8_1_BLOCK_BYTES)
    _need(ids, "ids", ncols * topk * 4)
    _need(weights, "weights", ncols * topk * 4)
    _need(grouping, "grouping", gb)
    call("moe_route_topk_quantize", _ptr(x), x.stride(0), k, _ptr(xq), _ptr(logits), _ptr(bias),
         _ptr(owner_slot), ncols, n_expert, n_local_expert, topk, _ptr(ids), _ptr(weights),
         _ptr(grouping), _stream(x))
    return xq, ids, weights, grouping


def moe_grouped_mmvq_ex(stage: int, w_a: torch.Tensor, w_b: torch.Tensor | None, act: torch.Tensor,
                        grouping: torch.Tensor, *, n: int, k: int, n_local_expert: int, ncols: int,
                        topk: int, out: torch.Tensor, expert_stride_bytes: int | None = None,
                        w_row_stride_bytes: int | None = None, shared: dict | None = None):
    """Grouped MMVQ with the fused extras (q8_1 of fp32 activations in the launch
    for DOWN_F32_ACT; a dense shared-expert part as extra work items).

    shared = {"a", "b" (gate/up only), "row_stride", "n", "k" (slice length, must
              equal k), "k_block_offset", "offset_bytes", "out",
              "act" (fp32 [ncols, >= k] for DOWN_F32_ACT; q8_1 rows [ncols, k/32*36]
              for DOWN; absent for the gate/up stage, which reads act)}."""
    if w_row_stride_bytes is None:
        w_row_stride_bytes = (k // QK) * Q8_0_BLOCK_BYTES
    if expert_stride_bytes is None:
        expert_stride_bytes = n * w_row_stride_bytes
    extent = (n_local_expert - 1) * expert_stride_bytes + _weight_extent(n, k, w_row_stride_bytes)
    _cuda(w_a, "w_a", torch.uint8)
    _need(w_a, "w_a", extent)
    act_row_stride = 0
    if stage in (GATE_UP_SWIGLU, GATE_UP_SWIGLU_P64):
        _cuda(w_b, "w_b", torch.uint8)
        _need(w_b, "w_b", extent)
        _act_rows(act, "act", ncols, k)
    elif stage == DOWN:
        _act_rows(act, "act", ncols * topk, k)
    elif stage in (DOWN_F32_ACT, DOWN_F32_ACT_P64):
        _cuda(act, "act", torch.float32)
        if act.dim() != 2 or act.stride(1) != 1:
            raise ValueError("fp32 act must be 2-D with unit inner stride")
        act_row_stride = act.stride(0)
        _need(act, "act", ((ncols * topk - 1) * act_row_stride + k) * 4)
    else:
        raise ValueError("bad stage")
    _cuda(grouping, "grouping", torch.uint8)
    _need(grouping, "grouping", moe_grouping_bytes_wide(ncols, topk))
    _cuda(out, "out", torch.float32)
    _need(out, "out", ncols * topk * n * 4)
    sa = sb = sact = sout = None
    s_stride = s_n = s_k = s_kb = s_off = s_act_stride = 0
    if shared is not None:
        s_stride, s_n, s_kb = shared["row_stride"], shared["n"], shared["k_block_offset"]
        s_k = shared["k"]
        s_off = shared.get("offset_bytes", 0)
        sa, sout = shared["a"], shared["out"]
        _cuda(sa, "shared a", torch.uint8)
        _need(sa, "shared a", _weight_extent(s_n, s_k, s_stride), s_off)
        if stage in (GATE_UP_SWIGLU, GATE_UP_SWIGLU_P64):
            sb = shared["b"]
            _cuda(sb, "shared b", torch.uint8)
            _need(sb, "shared b", _weight_extent(s_n, s_k, s_stride), s_off)
        _cuda(sout, "shared out", torch.float32)
        _need(sout, "shared out", ncols * s_n * 4)
        if stage in (DOWN_F32_ACT, DOWN_F32_ACT_P64):
            sact = shared["act"]
            _cuda(sact, "shared act", torch.float32)
            s_act_stride = sact.stride(0)
            _need(sact, "shared act", ((ncols - 1) * s_act_stride + s_k) * 4)
        elif stage == DOWN:
            sact = shared["act"]
            _act_rows(sact, "shared act", ncols, s_k)
    call("moe_grouped_mmvq_ex", stage, _ptr(w_a), _ptr(w_b), expert_stride_bytes,
         w_row_stride_bytes, n_local_expert, n, k, _ptr(act), act_row_stride, _ptr(grouping),
         ncols, topk, _ptr(out), _ptr(sa, s_off), _ptr(sb, s_off), s_stride, s_n, s_k, s_kb, _ptr(sact),
         s_act_stride, _ptr(sout), _stream(w_a))
    return out


def moe_grouped_ffn_p64(w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor, xq: torch.Tensor,
                        grouping: torch.Tensor, *, hidden: int, inter: int, n_local_expert: int, ncols: int,
                        topk: int, h: torch.Tensor, y: torch.Tensor, shared: dict | None = None):
    """The routed FFN product after routing: grouped gate/up + SwiGLU into the
    workspace h, then the grouped down quantising h in its launch, on packed
    experts (contiguous: gate/up experts inter rows of hidden/32 blocks, down
    experts hidden rows of 1088 bytes).

    shared = {"gate", "up" (packed rows of the shared gate/up), "row_stride",
              "rows" (== inter), "offset_bytes" (of the share's first row),
              "down" (the packed shared down), "down_offset_bytes" (of the
              share's round matrix), "hs" (fp32 [ncols, rows]), "ys" (fp32
              [ncols, hidden])}."""
    rb_h = (hidden // QK) * Q8_0_BLOCK_BYTES
    gu_stride = inter * rb_h
    dn_stride = hidden * ROUND_BYTES
    for t, name, nb in ((w_gate, "w_gate", gu_stride), (w_up, "w_up", gu_stride), (w_down, "w_down", dn_stride)):
        _cuda(t, name, torch.uint8)
        _need(t, name, n_local_expert * nb)
    _act_rows(xq, "xq", ncols, hidden)
    _cuda(grouping, "grouping", torch.uint8)
    _need(grouping, "grouping", moe_grouping_bytes(ncols, topk))
    _cuda(h, "h", torch.float32)
    _need(h, "h", ncols * topk * inter * 4)
    _cuda(y, "y", torch.float32)
    _need(y, "y", ncols * topk * hidden * 4)
    sg = su = sd = hs = ys = None
    s_stride = s_rows = s_off = d_off = 0
    if shared is not None:
        sg, su, sd = shared["gate"], shared["up"], shared["down"]
        s_stride, s_rows = shared["row_stride"], shared["rows"]
        s_off, d_off = shared.get("offset_bytes", 0), shared.get("down_offset_bytes", 0)
        hs, ys = shared["hs"], shared["ys"]
        for t, name in ((sg, "shared gate"), (su, "shared up")):
            _cuda(t, name, torch.uint8)
            _need(t, name, _weight_extent(s_rows, hidden, s_stride), s_off)
        _cuda(sd, "shared down", torch.uint8)
        _need(sd, "shared down", hidden * ROUND_BYTES, d_off)
        _cuda(hs, "hs", torch.float32)
        _need(hs, "hs", ncols * s_rows * 4)
        _cuda(ys, "ys", torch.float32)
        _need(ys, "ys", ncols * hidden * 4)
    call("moe_grouped_ffn_p64", _ptr(w_gate), _ptr(w_up), _ptr(w_down), gu_stride, dn_stride, n_local_expert,
         hidden, inter, _ptr(xq), _ptr(grouping), ncols, topk, _ptr(h), _ptr(y), _ptr(sg, s_off), _ptr(su, s_off),
         s_stride, s_rows, _ptr(sd, d_off), _ptr(hs), _ptr(ys), _stream(w_gate))
    return y


def moe_grouped_ffn_p64_noalloc(w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor,
                                xq: torch.Tensor, grouping: torch.Tensor, *, hidden: int, inter: int,
                                n_local_expert: int, ncols: int, topk: int, y: torch.Tensor,
                                shared: dict | None = None):
    """moe_grouped_ffn_p64 with h and hs in the library's own device memory:
    the same arguments without h and hs (shared: the same dict without "hs").
    Calls on one GPU must not overlap."""
    rb_h = (hidden // QK) * Q8_0_BLOCK_BYTES
    gu_stride = inter * rb_h
    dn_stride = hidden * ROUND_BYTES
    for t, name, nb in ((w_gate, "w_gate", gu_stride), (w_up, "w_up", gu_stride), (w_down, "w_down", dn_stride)):
        _cuda(t, name, torch.uint8)
        _need(t, name, n_local_expert * nb)
    _act_rows(xq, "xq", ncols, hidden)
    _cuda(grouping, "grouping", torch.uint8)
    _need(grouping, "grouping", moe_grouping_bytes(ncols, topk))
    _cuda(y, "y", torch.float32)
    _need(y, "y", ncols * topk * hidden * 4)
    sg = su = sd = ys = None
    s_stride = s_rows = s_off = d_off = 0
    if shared is not None:
        sg, su, sd = shared["gate"], shared["up"], shared["down"]
        s_stride, s_rows = shared["row_stride"], shared["rows"]
        s_off, d_off = shared.get("offset_bytes", 0), shared.get("down_offset_bytes", 0)
        ys = shared["ys"]
        for t, name in ((sg, "shared gate"), (su, "shared up")):
            _cuda(t, name, torch.uint8)
            _need(t, name, _weight_extent(s_rows, hidden, s_stride), s_off)
        _cuda(sd, "shared down", torch.uint8)
        _need(sd, "shared down", hidden * ROUND_BYTES, d_off)
        _cuda(ys, "ys", torch.float32)
        _need(ys, "ys", ncols * hidden * 4)
    call("moe_grouped_ffn_p64_noalloc", _ptr(w_gate), _ptr(w_up), _ptr(w_down), gu_stride, dn_stride,
         n_local_expert, hidden, inter, _ptr(xq), _ptr(grouping), ncols, topk, _ptr(y), _ptr(sg, s_off),
         _ptr(su, s_off), s_stride, s_rows, _ptr(sd, d_off), _ptr(ys), _stream(w_gate))
    return y


def moe_combine(y: torch.Tensor, ids: torch.Tensor, weights: torch.Tensor,
                out: torch.Tensor | None = None, shared: torch.Tensor | None = None) -> torch.Tensor:
    """out fp32 [ncols, n] = sum over unmasked slots of weights * y, plus
    shared [ncols, n] (the shared expert's output) when given; shared may be out."""
    _cuda(y, "y", torch.float32)
    _cuda(ids, "ids", torch.int32)
    _cuda(weights, "weights", torch.float32)
    ncols, topk, n = y.shape
    if not y.is_contiguous():
        raise ValueError("y must be contiguous [ncols, topk, n]")
    _need(ids, "ids", ncols * topk * 4)
    _need(weights, "weights", ncols * topk * 4)
    if out is None:
        out = torch.empty((ncols, n), dtype=torch.float32, device=y.device)
    _cuda(out, "out", torch.float32)
    _need(out, "out", ncols * n * 4)
    if shared is None:
        call("moe_combine", _ptr(y), _ptr(ids), _ptr(weights), ncols, topk, n, _ptr(out), _stream(y))
    else:
        _cuda(shared, "shared", torch.float32)
        if not shared.is_contiguous():
            raise ValueError("shared must be contiguous [ncols, n]")
        _need(shared, "shared", ncols * n * 4)
        call("moe_combine_shared", _ptr(y), _ptr(ids), _ptr(weights), ncols, topk, n, _ptr(shared),
             _ptr(out), _stream(y))
    return out


# ---------------------------------------------------------------------------
# synthetic weights (input generation; not part of the FFN path)
# ---------------------------------------------------------------------------

def synth_q8_0_fill(dst: torch.Tensor, n_mats: int, blocks_per_mat: int, mats_per_layer: int,
                    seed: int, layer0: int, expert0: int, matrix: int, offset_bytes: int = 0):
    _cuda(dst, "dst", torch.uint8)
    _need(dst, "dst", n_mats * blocks_per_mat * Q8_0_BLOCK_BYTES, offset_bytes)
    call("moeq8_synth_q8_0_fill", _ptr(dst, offset_bytes), n_mats, blocks_per_mat, mats_per_layer,
         seed, layer0, expert0, matrix, _stream(dst))
    return dst


def stream_read(buf: torch.Tensor, nbytes: int, sink: torch.Tensor, offset_bytes: int = 0):
    """Read nbytes of buf (from offset_bytes) once with a plain coalesced
    streaming kernel: the read ceiling a bandwidth-bound launch is compared
    with.  sink: a device tensor of at least 4 bytes."""
    _cuda(buf, "buf")
    _cuda(sink, "sink")
    _need(buf, "buf", nbytes, offset_bytes)
    _need(sink, "sink", 4)
    call("moeq8_stream_read", _ptr(buf, offset_bytes), nbytes, _ptr(sink), _stream(buf))


STREAM_READ_SHAPES = (8192, 16384, 32768, 65536)


def stream_read_shape(buf: torch.Tensor, nbytes: int, wg_bytes: int, sink: torch.Tensor,
                      offset_bytes: int = 0):
    """stream_read with wg_bytes (one of STREAM_READ_SHAPES) bytes a workgroup."""
    _cuda(buf, "buf")
    _cuda(sink, "sink")
    _need(buf, "buf", nbytes, offset_bytes)
    _need(sink, "sink", 4)
    call("moeq8_stream_read_shape", _ptr(buf, offset_bytes), nbytes, wg_bytes, _ptr(sink), _stream(buf))
