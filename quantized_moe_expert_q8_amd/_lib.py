"""ctypes binding of libmoeq8.so (the in-tree HIP build).  No fallback: if the
library is missing or does not load, every call raises."""

from __future__ import annotations

import ctypes
import os

from .build import LIB_PATH

c_i32, c_i64, c_u32, c_u64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64
c_vp, c_fp, c_size = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t

# name -> (restype, argtypes); one entry per declaration in include/moeq8.h and
# include/moeq8_synth.h
SIGNATURES = {
    "moeq8_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moeq8_abi_version": (ctypes.c_int, []),
    "q8_1_quantize_rows": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, c_vp]),
    "q8_0_quantize_rows": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, c_vp]),
    "q8_0_pack64_rows": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp]),
    "q8_0_pack64_rounds": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, c_vp]),
    "q4_pack64_rows": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp]),
    "q8_0_pack_gemm_rows": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp]),
    "mmvq_q8_0": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_vp]),
    "mmvq_q8_0_glu_pair": (ctypes.c_int, [c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_vp, c_i64,
                                          c_vp, c_vp, c_vp, c_vp]),
    "swiglu_ds4": (ctypes.c_int, [c_vp, c_vp, c_i64, c_vp, c_vp]),
    "moe_grouping_bytes": (c_size, [c_i64, c_i32]),
    "moe_router_scores": (ctypes.c_int, [c_vp, c_i64, c_vp, c_vp]),
    "moe_route_topk": (ctypes.c_int, [c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i32, c_vp, c_vp,
                                      c_vp, c_vp]),
    "moe_grouped_mmvq": (ctypes.c_int, [c_i32, c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_i64,
                                        c_vp, c_vp, c_i64, c_i32, c_vp, c_vp]),
    "moe_grouped_gemm": (ctypes.c_int, [c_i32, c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_i64,
                                        c_vp, c_vp, c_i64, c_i32, c_vp, c_vp]),
    "moe_grouped_mmvq_ex": (ctypes.c_int, [c_i32, c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_i64,
                                           c_vp, c_i64, c_vp, c_i64, c_i32, c_vp, c_vp, c_vp, c_i64,
                                           c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_vp]),
    "moe_route_topk_quantize": (ctypes.c_int, [c_vp, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_i64,
                                               c_i64, c_i64, c_i32, c_vp, c_vp, c_vp, c_vp]),
    "moe_grouped_ffn_p64": (ctypes.c_int, [c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_i64, c_vp,
                                           c_vp, c_i64, c_i32, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64,
                                           c_vp, c_vp, c_vp, c_vp]),
    "moe_grouped_ffn_p64_noalloc": (ctypes.c_int, [c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_i64, c_vp,
                                                   c_vp, c_i64, c_i32, c_vp, c_vp, c_vp, c_i64, c_i64,
                                                   c_vp, c_vp, c_vp]),
    "moe_combine": (ctypes.c_int, [c_vp, c_vp, c_vp, c_i64, c_i32, c_i64, c_vp, c_vp]),
    "moe_combine_shared": (ctypes.c_int, [c_vp, c_vp, c_vp, c_i64, c_i32, c_i64, c_vp, c_vp, c_vp]),
    "q8_block_encode": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, c_vp]),
    "q8_block_decode_sum": (ctypes.c_int, [c_vp, c_i32, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp]),
    "q4_quantize_rows": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, c_vp]),
    "mmvq_q4": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_vp]),
    "mmvq_q4_glu_pair": (ctypes.c_int, [c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_vp, c_i64,
                                        c_vp, c_vp, c_vp, c_vp]),
    "moe_grouped_mmvq_q4": (ctypes.c_int, [c_i32, c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_i64,
                                           c_vp, c_i64, c_vp, c_i64, c_i32, c_vp, c_vp]),
    "moe_grouping_bytes_wide": (c_size, [c_i64, c_i32]),
    "moe_route_topk_wide": (ctypes.c_int, [c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i32, c_vp, c_vp,
                                           c_vp]),
    "moe_group_routes": (ctypes.c_int, [c_vp, c_i64, c_i32, c_i64, c_vp, c_vp]),
    "moeq8_synth_stream_key": (c_u64, [c_u32, c_u32, c_u32, c_u32]),
    "moeq8_synth_q8_0_fill": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i64, c_u32, c_u32, c_u32,
                                             c_u32, c_vp]),
    "moeq8_stream_read": (ctypes.c_int, [c_vp, c_i64, c_vp, c_vp]),
    "moeq8_stream_read_shape": (ctypes.c_int, [c_vp, c_i64, c_i64, c_vp, c_vp]),
}

_LIB = None


class MoeQ8Error(RuntimeError):
    def __init__(self, name: str, status: int):
        msg = lib().moeq8_status_string(status).decode()
        super().__init__(f"{name} failed with status {status}: {msg}")
        self.status = status


def lib_path() -> str:
    return os.environ.get("MOEQ8_LIB", LIB_PATH)


def lib():
    """Load libmoeq8.so once; raise if it is not built."""
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"libmoeq8 is not built ({path} missing): run __graft_entry__.build() "
                               "or python -m quantized_moe_expert_q8_amd.build")
        # torch first: its HIP runtime (same soname) then serves this library too,
        # so torch's streams and allocations are valid here
        import torch  # noqa: F401
        so = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(so, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = so
    return _LIB


def call(name: str, *args) -> int:
    st = getattr(lib(), name)(*args)
    if st != 0:
        raise MoeQ8Error(name, st)
    return st
