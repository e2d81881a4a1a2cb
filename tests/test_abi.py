"""The C-ABI library loads and exports every symbol include/*.h declares, and
host-side argument validation rejects bad calls before anything is enqueued
(CPU only: no compute call is made)."""

import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

import quantized_moe_expert_q8_amd as moeq8  # noqa: E402
from quantized_moe_expert_q8_amd import _lib  # noqa: E402


def _declared_functions():
    names = []
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w\s\*]*?\b([A-Za-z_]\w*)\s*\(", text, flags=re.M):
            if not m.group(0).lstrip().startswith(("#", "typedef", "enum", "struct")):
                names.append(m.group(1))
    return names


def test_header_declares_the_hot_path_calls():
    names = set(_declared_functions())
    for n in ("q8_1_quantize_rows", "mmvq_q8_0_glu_pair", "moe_route_topk", "moe_grouped_mmvq",
              "moe_combine", "mmvq_q8_0", "moe_grouping_bytes", "moe_grouped_gemm", "q8_block_encode",
              "q8_block_decode_sum"):
        assert n in names


def test_library_exports_every_declared_symbol():
    so = ctypes.CDLL(_lib.lib_path())
    declared = _declared_functions()
    assert len(declared) >= 12
    for name in declared:
        assert hasattr(so, name), name
        assert name in _lib.SIGNATURES, name


def test_abi_version_and_status_strings():
    L = moeq8.lib()
    assert L.moeq8_abi_version() == 1
    for st in (0, -1, -2, -3, -4, -99):
        assert L.moeq8_status_string(st)


def test_grouping_bytes():
    L = moeq8.lib()
    # header, expert[R], offset[R+1], route[R], 8 words of padding, rounded to
    # 4 words, then a 4-word table entry per group; whole 256-byte units
    assert L.moe_grouping_bytes(8, 8) == 2048           # 4*(208 + 4*64) = 1856 -> 2048
    assert L.moe_grouping_bytes(1, 8) == 512            # 4*(40 + 4*8) = 288 -> 512
    assert L.moe_grouping_bytes(0, 8) == 0 and L.moe_grouping_bytes(9, 8) == 0
    assert L.moe_grouping_bytes(1, 17) == 0


try:
    import torch
    _HAS_GPU = torch.cuda.is_available()
except Exception:  # pragma: no cover
    _HAS_GPU = False


# Fake, never-dereferenced addresses: every call below must be rejected on the
# host before a launch.  Skipped where a GPU is visible, so a validation bug
# can never turn one of these into a launch on real hardware.
P = 0x10000
cpu_only = pytest.mark.skipif(_HAS_GPU, reason="host-validation calls use fake pointers")


@cpu_only
@pytest.mark.parametrize("args,expect", [
    ((None, 68, 4, 64, 0, P, 1, P, None), -1),           # null weights
    ((P, 68, 4, 96, 0, P, 1, P, None), -1),              # K % 64
    ((P, 68, 4, 64, 0, P, 0, P, None), -1),              # ncols 0
    ((P, 68, 4, 64, 0, P, 9, P, None), -1),              # ncols 9
    ((P, 68, 4, 64, 1, P, 1, P, None), -2),              # odd block offset
    ((P + 2, 68, 4, 64, 0, P, 1, P, None), -2),          # misaligned weights
    ((P, 66, 4, 64, 0, P, 1, P, None), -2),              # row stride % 4
    ((P, 64, 4, 64, 0, P, 1, P, None), -1),              # row stride shorter than a row
    ((P, 68, -1, 64, 0, P, 1, P, None), -1),             # negative rows
    ((P, 68, 4, 64, 0, P + 1, 1, P, None), -2),          # misaligned activations
])
def test_mmvq_validation(args, expect):
    assert moeq8.lib().mmvq_q8_0(*args) == expect


@cpu_only
def test_other_validation():
    L = moeq8.lib()
    assert L.mmvq_q8_0(P, 68, 0, 64, 0, P, 1, P, None) == 0                      # n = 0: nothing to do
    assert L.mmvq_q8_0_glu_pair(P, None, 68, 4, 64, 0, P, 1, P, None, None, None) == -1
    assert L.q8_1_quantize_rows(P, 2, 48, 48, P, None) == -1                     # k % 32
    assert L.q8_1_quantize_rows(P, 2, 64, 32, P, None) == -1                     # stride < k
    assert L.q8_1_quantize_rows(P, 0, 64, 64, P, None) == 0
    assert L.q8_0_quantize_rows(P, 2, 64, 64, P + 1, None) == -2
    assert L.swiglu_ds4(None, P, 4, P, None) == -1
    assert L.moe_route_topk(P, None, None, 2, 8, 8, 9, P, P, P, None) == -1      # topk > n_expert
    assert L.moe_route_topk(P, None, None, 2, 8, 4, 2, P, P, P, None) == -1      # no owner map, n_local != n
    assert L.moe_route_topk(P, None, None, 2, 2048, 2048, 8, P, P, P, None) == -3
    assert L.moe_route_topk(P, None, None, 9, 8, 8, 2, P, P, P, None) == -1
    assert L.moe_grouped_mmvq(2, P, P, 0, 68, 1, 4, 64, P, P, 1, 1, P, None) == -1  # bad stage
    assert L.moe_grouped_mmvq(0, P, None, 272, 68, 1, 4, 64, P, P, 1, 1, P, None) == -1  # gate/up without up
    assert L.moe_grouped_mmvq(1, P, None, 270, 68, 2, 4, 64, P, P, 1, 1, P, None) == -2  # expert stride % 4
    assert L.moe_grouped_mmvq(1, P, None, 136, 68, 2, 4, 64, P, P, 1, 1, P, None) == -1  # experts overlap
    assert L.moe_grouped_gemm(0, P, P, 272, 68, 1, 48, 64, P, P, 1, 1, P, None) == -1   # n % 32
    assert L.moe_grouped_gemm(1, P, None, 272, 68, 1, 64, 96, P, P, 1, 1, P, None) == -1  # k % 64
    assert L.moe_grouped_gemm(0, P, None, 272, 68, 1, 64, 64, P, P, 1, 1, P, None) == -1  # no up matrix
    assert L.moe_grouped_gemm(1, P, None, 272, 68, 1, 64, 64, P, P, 1025, 1, P, None) == -1  # ncols
    assert L.moe_grouped_gemm(1, P, None, 270, 68, 2, 64, 64, P, P, 1, 1, P, None) == -2  # expert stride % 4
    assert L.moe_grouped_gemm(1, P, None, 272, 68, 1, 0, 64, P, P, 1, 1, P, None) == 0
    assert L.q8_block_encode(P, 2, 48, 48, P, None) == -1                        # n % 32
    assert L.q8_block_encode(P, 2, 64, 32, P, None) == -1                        # stride < n
    assert L.q8_block_encode(P + 2, 2, 64, 64, P, None) == -2
    assert L.q8_block_encode(P, 0, 64, 64, P, None) == 0
    assert L.q8_block_decode_sum(P, 0, 0, 2, 64, P, 64, None) == -1              # no ranks
    assert L.q8_block_decode_sum(P, 65, 1 << 20, 2, 64, P, 64, None) == -1       # too many ranks
    assert L.q8_block_decode_sum(P, 2, 100, 2, 64, P, 64, None) == -1            # ranks overlap
    assert L.q8_block_decode_sum(P, 2, 146, 2, 64, P, 64, None) == -2            # rank stride % 4
    assert L.q8_block_decode_sum(P, 2, 144, 0, 64, P, 64, None) == 0
    assert L.q4_quantize_rows(P, 2, 48, 48, P, None) == -1                       # k % 32
    assert L.q4_quantize_rows(P, 2, 64, 64, P + 1, None) == -2
    assert L.mmvq_q4(P, 34, 4, 64, 0, P, 1, P, None) == -2                       # row stride % 4
    assert L.mmvq_q4(P, 32, 4, 64, 0, P, 1, P, None) == -1                       # row shorter than a row
    assert L.mmvq_q4(P, 36, 4, 96, 0, P, 1, P, None) == -1                       # k % 64
    assert L.mmvq_q4_glu_pair(P, None, 36, 4, 64, 0, P, 1, P, None, None, None) == -1
    assert L.moe_grouped_mmvq_q4(5, P, P, 144, 36, 1, 4, 64, P, 0, P, 1, 1, P, None) == -1   # bad stage
    assert L.moe_grouped_mmvq_q4(0, P, None, 144, 36, 1, 4, 64, P, 0, P, 1, 1, P, None) == -1  # no up
    assert L.moe_combine(P, P, P, 0, 8, 16, P, None) == -1
    assert L.moe_combine(P, P, P, 1, 8, 0, P, None) == 0
    assert L.moe_combine_shared(P, P, P, 1, 8, 16, None, P, None) == -1         # no shared output
    assert L.moe_combine_shared(P, P, P, 1, 8, 16, P + 2, P, None) == -2        # misaligned shared
    assert L.moe_combine_shared(P, P, P, 1, 8, 0, P, P, None) == 0
    assert L.moeq8_synth_q8_0_fill(P + 1, 1, 1, 1, 0, 0, 0, 0, None) == -2
    assert L.moeq8_stream_read(P + 4, 64, P, None) == -2                         # misaligned buffer
    assert L.moeq8_stream_read(P, 24, P, None) == -2                             # bytes % 16
    assert L.moeq8_stream_read(P, 0, P, None) == 0
    # the routed FFN entry: columns, shapes of the packed layouts, alignment
    gu_s, dn_s = 1024 * 4352, 4096 * 1088
    assert L.moe_grouped_ffn_p64(P, P, P, gu_s, dn_s, 2, 4096, 1024, P, P, 0, 8, P, P,
                                 None, None, 0, 0, None, None, None, None) == -1            # no columns
    assert L.moe_grouped_ffn_p64(P, P, P, gu_s, dn_s, 2, 4096, 1024, P, P, 9, 8, P, P,
                                 None, None, 0, 0, None, None, None, None) == -1            # past 8 columns
    assert L.moe_grouped_ffn_p64(P, P, P, gu_s // 2, dn_s, 2, 2048, 1024, P, P, 1, 8, P, P,
                                 None, None, 0, 0, None, None, None, None) == -3            # not one segment a row
    assert L.moe_grouped_ffn_p64(P, P, P + 4, gu_s, dn_s, 2, 4096, 1024, P, P, 1, 8, P, P,
                                 None, None, 0, 0, None, None, None, None) == -2            # down off 16 bytes
    assert L.moe_grouped_ffn_p64(P, P, P, gu_s, dn_s, 2, 4096, 1024, P, P, 1, 8, P, P,
                                 P, None, 4352, 1024, P, P, P, None) == -1                  # shared up missing
    # its no-alloc form refuses what its memory cannot hold before anything else
    assert L.moe_grouped_ffn_p64_noalloc(P, P, P, gu_s, dn_s, 2, 4096, 2048, P, P, 8, 16, P,
                                         None, None, 0, 0, None, None, None) == -3          # h past 512 KiB
    assert L.moe_grouped_ffn_p64_noalloc(P, P, P, gu_s, dn_s, 2, 4096, 1024, P, P, 8, 8, P,
                                         P, P, 4352, 2048, P, P, None) == -3                # hs past 32 KiB
    assert L.moe_grouped_ffn_p64_noalloc(P, P, P, gu_s, dn_s, 2, 4096, 1024, P, P, 0, 8, P,
                                         None, None, 0, 0, None, None, None) == -1          # no columns
    assert L.moeq8_stream_read_shape(P, 64, 4096, P, None) == -1                # not a read shape
    assert L.moeq8_stream_read_shape(P, 24, 8192, P, None) == -2                # bytes % 16
    assert L.moeq8_stream_read_shape(P, 0, 16384, P, None) == 0
    assert L.moe_router_scores(None, 4, P, None) == -1
    assert L.moe_router_scores(P, -1, P, None) == -1
    assert L.moe_router_scores(P, 4, P + 2, None) == -2
    assert L.moe_router_scores(P, 0, P, None) == 0                                # nothing to do


def test_packed_layout_validation():
    """The packers and the packed stages reject on the host what they cannot
    read or write (no kernel runs: every case returns before a launch)."""
    L = moeq8.lib()
    Q = 0x10000000                                                               # far from P: no overlap
    rows = L.q8_0_pack64_rows
    assert rows(P, 2, 2048, 4352, Q, 4352, None) == -1                           # k % 4096
    assert rows(P, 2, 4096, 4000, Q, 8704, None) == -1                           # stride shorter than a row
    assert rows(P + 2, 2, 4096, 8704, Q, 8704, None) == -2
    assert rows(P, 2, 4096, 8704, P + 100, 8704, None) == -1                     # overlapping
    assert rows(P, 0, 4096, 8704, Q, 8704, None) == 0
    rounds = L.q8_0_pack64_rounds
    assert rounds(P, 6, 1024, 1088, Q, None) == -1                               # rows % 4
    assert rounds(P, 4, 1000, 1088, Q, None) == -1                               # k % 1024
    assert rounds(P, 4, 1024, 1000, Q, None) == -1                               # stride shorter than a row
    assert rounds(P + 2, 4, 1024, 1088, Q, None) == -2
    assert rounds(P, 0, 1024, 1088, Q, None) == 0
    ex = L.moe_grouped_mmvq_ex

    def gate_up(w_a, k, stride=8704):
        return ex(3, w_a, Q, 0, stride, 1, 4, k, P, 0, P, 1, 1, P,
                  None, None, 0, 0, 0, 0, None, 0, None, None)

    def down(n, k, stride):
        return ex(4, P, None, 0, stride, 1, n, k, P, k, P, 1, 1, P,
                  None, None, 0, 0, 0, 0, None, 0, None, None)

    assert gate_up(P, 2048) == -3                                                # one 4096-value segment a row
    assert gate_up(P + 4, 4096) == -2                                            # 16-byte aligned segments
    assert gate_up(P, 4096, 8708) == -2
    assert down(4, 2048, 2176) == -3                                             # k must be one 1024 round
    assert down(62, 1024, 1088) == -3                                            # whole quads of rows
    assert down(4, 1024, 2176) == -3                                             # contiguous 1088-byte rows
    gp = L.q8_0_pack_gemm_rows
    assert gp(P, 2, 128, 68 * 4, Q, 68 * 4, None) == -1                          # k % 256
    assert gp(P, 2, 256, 270, Q, 272, None) == -1                                # stride shorter than a row
    assert gp(P + 2, 2, 256, 272, Q, 272, None) == -2
    assert gp(P, 2, 256, 272, P + 100, 272, None) == -1                          # overlapping
    assert gp(P, 0, 256, 272, Q, 272, None) == 0
    gg = L.moe_grouped_gemm                                                      # the GEMM layout: staged form only
    assert gg(5, P, Q, 0, 68 * 2, 1, 32, 128, P, P, 1, 1, P, None) == -3         # k % 256
    assert gg(5, P + 4, Q, 0, 272, 1, 32, 256, P, P, 1, 1, P, None) == -3        # 16-byte alignment
    assert gg(6, P, None, 0, 272, 1, 32, 256, P, P, 1, 1, P, None) == -3         # down: whole 64-row tiles
    assert gg(7, P, Q, 0, 272, 1, 32, 256, P, P, 1, 1, P, None) == -1            # no such stage
    q4 = L.q4_pack64_rows
    assert q4(P, 2, 2048, 1152, Q, 1152, None) == -1                             # k % 4096
    assert q4(P, 2, 4096, 2300, Q, 4608, None) == -1                             # stride shorter than a row
    assert q4(P + 2, 2, 4096, 2304, Q, 2304, None) == -2
    assert q4(P, 2, 4096, 2304, Q, 2306, None) == -2                             # dword row strides
    assert q4(P, 2, 4096, 2304, P + 100, 2304, None) == -1                       # overlapping
    assert q4(P, 0, 4096, 2304, Q, 2304, None) == 0
    g4 = L.moe_grouped_mmvq_q4

    def gate_up4(w_a, k, stride=4608):
        return g4(3, w_a, Q, 0, stride, 1, 4, k, P, 0, P, 1, 1, P, None)

    def down4(n, k, stride):
        return g4(4, P, None, 0, stride, 1, n, k, P, k, P, 1, 1, P, None)

    assert gate_up4(P, 2048) == -3                                               # one 4096-value segment a row
    assert gate_up4(P + 4, 4096) == -2                                           # 16-byte aligned segments
    assert gate_up4(P, 4096, 4612) == -2
    assert down4(4, 2048, 1152) == -3                                            # k must be one 1024 round
    assert down4(62, 1024, 576) == -3                                            # whole quads of rows
    assert down4(4, 1024, 1152) == -3                                            # contiguous 576-byte rows


def test_ops_reject_out_of_bounds_views():
    """The torch layer refuses views that would read past a tensor (CPU tensors
    are refused first, so this needs no GPU)."""
    import torch
    w = torch.zeros(10, dtype=torch.uint8)
    with pytest.raises(ValueError):
        moeq8.mmvq_q8_0(w, w, 1, 64)


def test_synth_stream_key_host_matches_generator():
    import workloads
    L = moeq8.lib()
    for args in [(0, 0, 0, 0), (5, 42, 127, 2), (65535, 3, 9, 5)]:
        assert L.moeq8_synth_stream_key(*args) == workloads.stream_key(*args)


def test_wide_products_choice():
    from quantized_moe_expert_q8_amd import moe_layer as ml
    assert ml.wide_products_for(32, 8, 256) == "mmvq"       # one route per expert
    assert ml.wide_products_for(128, 8, 256) == "gemm"      # four routes per expert
    assert ml.wide_products_for(1024, 8, 256) == "gemm"
    assert ml.wide_products_for(8, 8, 16) == "gemm"
