"""ctypes loader for libvarlen_attn.so (argument marshalling only).

Fails loudly when the library has not been built: there is no fallback
implementation in this package.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvarlen_attn.so")

VA_OK = 0
STATUS_NAMES = {
    0: "VA_OK", 1: "VA_ERR_NULL", 2: "VA_ERR_SHAPE", 3: "VA_ERR_DTYPE", 4: "VA_ERR_UNSUPPORTED",
    5: "VA_ERR_ALIAS", 6: "VA_ERR_ALIGN", 7: "VA_ERR_WORKSPACE", 8: "VA_ERR_HIP",
    9: "VA_ERR_DEVICE_CHECK",
}
VA_F32, VA_BF16, VA_F16 = 0, 1, 2

# every symbol include/varlen_attn.h declares
EXPORTED = [
    "varlen_attn_workspace_size", "varlen_attn_fwd_out", "varlen_attn_fwd",
    "varlen_attn_fwd_paged", "varlen_attn_free", "varlen_attn_plan", "varlen_attn_path",
    "varlen_attn_last_error", "varlen_attn_abi_version", "varlen_attn_bwd_workspace_size",
    "varlen_attn_bwd", "varlen_attn_merge", "varlen_attn_sparse_sharedkv",
    "varlen_attn_bwd_sinks_workspace_size", "varlen_attn_bwd_sinks", "varlen_attn_fwd_out_noalloc",
]


class VaProblem(ctypes.Structure):
    """Mirror of ``va_problem`` in include/varlen_attn.h."""
    _fields_ = [
        ("struct_size", ctypes.c_uint32), ("dtype", ctypes.c_int32), ("batch", ctypes.c_int32),
        ("total_q", ctypes.c_int32), ("total_k", ctypes.c_int32), ("num_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("max_seqlen_q", ctypes.c_int32), ("max_seqlen_k", ctypes.c_int32),
        ("scale", ctypes.c_float), ("causal", ctypes.c_int32), ("window_left", ctypes.c_int32),
        ("window_right", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
        ("block_size", ctypes.c_int32), ("block_table_stride", ctypes.c_int32),
        ("alibi_slopes", ctypes.c_void_p),
    ]


class VaSparseProblem(ctypes.Structure):
    """Mirror of ``va_sparse_problem`` in include/varlen_attn.h."""
    _fields_ = [(name, ctypes.c_uint32 if name == "struct_size" else
                 ctypes.c_float if name == "scale" else ctypes.c_int32) for name in (
        "struct_size", "dtype", "batch", "total_q", "num_heads", "num_kv_heads", "head_dim",
        "max_seqlen_kv", "scale", "window_left", "window_right", "topk", "cmp_ratio",
        "ori_num_blocks", "ori_block_size", "ori_block_table_stride",
        "cmp_num_blocks", "cmp_block_size", "cmp_block_table_stride", "cmp_attend_all")]


_lock = threading.Lock()
_lib = None


def load():
    """Returns the loaded library; raises if it was not built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m variable_length_attention_amd.build)")
        lib = ctypes.CDLL(LIB_PATH)
        vp, P = ctypes.c_void_p, ctypes.POINTER(VaProblem)
        lib.varlen_attn_workspace_size.argtypes = [P, ctypes.c_int]
        lib.varlen_attn_workspace_size.restype = ctypes.c_size_t
        lib.varlen_attn_fwd_out.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        lib.varlen_attn_fwd_out.restype = ctypes.c_int
        lib.varlen_attn_fwd_out_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.varlen_attn_fwd_out_noalloc.restype = ctypes.c_int
        lib.varlen_attn_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, ctypes.POINTER(vp),
                                        ctypes.POINTER(vp), vp]
        lib.varlen_attn_fwd.restype = ctypes.c_int
        lib.varlen_attn_fwd_paged.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                              ctypes.c_size_t, vp]
        lib.varlen_attn_fwd_paged.restype = ctypes.c_int
        lib.varlen_attn_free.argtypes = [vp, vp]
        lib.varlen_attn_free.restype = ctypes.c_int
        lib.varlen_attn_plan.argtypes = [P, ctypes.c_int, vp, vp, vp, ctypes.c_int32, vp, vp,
                                         ctypes.c_size_t, vp]
        lib.varlen_attn_plan.restype = ctypes.c_int
        lib.varlen_attn_path.argtypes = [P, ctypes.c_int]
        lib.varlen_attn_path.restype = ctypes.c_int
        lib.varlen_attn_last_error.argtypes = []
        lib.varlen_attn_last_error.restype = ctypes.c_char_p
        lib.varlen_attn_bwd_workspace_size.argtypes = [P]
        lib.varlen_attn_bwd_workspace_size.restype = ctypes.c_size_t
        lib.varlen_attn_bwd.argtypes = [P] + [vp] * 12 + [ctypes.c_size_t, vp]
        lib.varlen_attn_bwd.restype = ctypes.c_int
        lib.varlen_attn_bwd_sinks_workspace_size.argtypes = [P]
        lib.varlen_attn_bwd_sinks_workspace_size.restype = ctypes.c_size_t
        lib.varlen_attn_bwd_sinks.argtypes = [P] + [vp] * 6 + [ctypes.c_size_t, vp]
        lib.varlen_attn_bwd_sinks.restype = ctypes.c_int
        i32 = ctypes.c_int32
        lib.varlen_attn_merge.argtypes = [i32, i32, i32, i32, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, vp]
        lib.varlen_attn_merge.restype = ctypes.c_int
        lib.varlen_attn_sparse_sharedkv.argtypes = [ctypes.POINTER(VaSparseProblem)] + [vp] * 12
        lib.varlen_attn_sparse_sharedkv.restype = ctypes.c_int
        lib.varlen_attn_abi_version.argtypes = []
        lib.varlen_attn_abi_version.restype = ctypes.c_int
        _lib = lib
        return lib


def check(status: int) -> None:
    """Raises for a non-OK va_status, with the library's message."""
    if status == VA_OK:
        return
    msg = load().varlen_attn_last_error().decode(errors="replace")
    name = STATUS_NAMES.get(status, str(status))
    if status in (8, 9):
        raise RuntimeError(f"{name}: {msg}")
    raise ValueError(f"{name}: {msg}")
