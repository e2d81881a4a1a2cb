"""libmoeq8: quantized MoE expert FFN (Q8_0 x q8_1) on AMD MI355X (gfx950).

The compute runs in the HIP library libmoeq8.so (C ABI in include/moeq8.h);
this package only marshals torch tensors (device memory, streams) into it.
"""

from ._lib import MoeQ8Error, lib, lib_path  # noqa: F401
from . import ops  # noqa: F401
from .ops import (  # noqa: F401
    GATE_UP_SWIGLU,
    DOWN,
    DOWN_F32_ACT,
    GATE_UP_SWIGLU_P64,
    DOWN_F32_ACT_P64,
    GATE_UP_SWIGLU_G8,
    DOWN_G8,
    P64_K,
    Q8_0_BLOCK_BYTES,
    Q8_1_BLOCK_BYTES,
    q8_1_quantize_rows,
    q8_0_quantize_rows,
    q8_0_pack64_rows,
    q8_0_pack64_rounds,
    q4_pack64_rows,
    q8_0_pack_gemm_rows,
    mmvq_q8_0,
    mmvq_q8_0_glu_pair,
    swiglu_ds4,
    moe_grouping_bytes,
    moe_grouping_bytes_wide,
    moe_route_topk_wide,
    moe_group_routes,
    moe_route_topk,
    moe_grouped_mmvq,
    moe_grouped_gemm,
    moe_grouped_mmvq_ex,
    moe_route_topk_quantize,
    moe_router_scores,
    moe_combine,
    moe_grouped_ffn_p64,
    moe_grouped_ffn_p64_noalloc,
    EXCHANGE_BLOCK_BYTES,
    q8_block_encode,
    q8_block_decode_sum,
    Q4_BLOCK_BYTES,
    q4_quantize_rows,
    mmvq_q4,
    mmvq_q4_glu_pair,
    moe_grouped_mmvq_q4,
    synth_q8_0_fill,
    stream_read,
    stream_read_shape,
    STREAM_READ_SHAPES,
)
