"""ctypes declarations of the C ABI in include/tp_shard.h (libtpshard.so).

Loading fails loudly when the library has not been built: there is no
fallback implementation of any kernel.
"""

from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtpshard.so")

TP_OK, TP_E_ARG, TP_E_DIVIDE, TP_E_RANK, TP_E_NOMEM, TP_E_HIP, TP_E_KV_FULL, TP_E_STATE = 0, -1, -2, -3, -4, -5, -6, -7
TP_E_SCRATCH = -8
TP_NOALLOC_SCRATCH_BYTES = 32 << 20
TP_F32, TP_BF16 = 0, 1
TP_STAGE_ATTN, TP_STAGE_MLP, TP_STAGE_PRENORM = 0, 1, 0x10
TP_ACT_SWIGLU, TP_ACT_GELU = 0, 1
TP_PROJ_PARTIAL, TP_PROJ_QKV, TP_PROJ_SWIGLU, TP_PROJ_GELU = 0, 1, 2, 3
# kernel kinds of the shard's event timer (TP_K_*)
KERNEL_KINDS = ["rmsnorm", "gemm_qkv", "attn_prefill", "gemm_out", "gemm_up", "gemm_down", "gemv_qkv",
                "attn_decode", "gemv_out", "gemv_up", "gemv_down", "reduce_norm"]


class tp_opts(C.Structure):
    _fields_ = [("dtype", C.c_int), ("act", C.c_int), ("rmsnorm", C.c_int), ("eps", C.c_float),
                ("rope", C.c_int), ("rope_theta", C.c_float), ("decode_fp8", C.c_int)]


class tp_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down", "g1", "g2")]


# (name, restype, argtypes) for every function the header declares
SIGNATURES = [
    ("tp_shard_create", C.c_int, [C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.POINTER(tp_opts),
                                  C.POINTER(C.c_void_p)]),
    ("tp_shard_load_weights", C.c_int, [C.c_void_p, C.POINTER(tp_weights), C.c_void_p]),
    ("tp_shard_reserve", C.c_int, [C.c_void_p, C.c_longlong]),
    ("tp_kv_create", C.c_int, [C.c_void_p, C.c_int, C.c_int, C.POINTER(C.c_void_p)]),
    ("tp_kv_view", C.c_int, [C.c_void_p, C.POINTER(C.c_void_p), C.POINTER(C.c_void_p)]),
    ("tp_kv_set_len", C.c_int, [C.c_void_p, C.c_int]),
    ("tp_kv_get_len", C.c_int, [C.c_void_p, C.POINTER(C.c_int)]),
    ("tp_kv_set_len_async", C.c_int, [C.c_void_p, C.c_int, C.c_void_p]),
    ("tp_kv_get_len_stream", C.c_int, [C.c_void_p, C.POINTER(C.c_int), C.c_void_p]),
    ("tp_shard_forward_prefill", C.c_int, [C.c_void_p, C.c_int, C.c_void_p, C.c_int, C.c_int, C.c_void_p,
                                           C.c_void_p, C.c_void_p]),
    ("tp_shard_forward_prefill_reduce", C.c_int, [C.c_void_p, C.c_int, C.c_void_p, C.c_int, C.c_int, C.c_void_p,
                                                  C.POINTER(C.c_void_p), C.c_void_p, C.c_void_p, C.c_void_p]),
    ("tp_shard_forward_decode", C.c_int, [C.c_void_p, C.c_int, C.c_void_p, C.c_int, C.c_void_p, C.c_void_p,
                                          C.c_void_p]),
    ("tp_shard_forward_decode_noalloc", C.c_int, [C.c_void_p, C.c_int, C.c_void_p, C.c_int, C.c_void_p,
                                                  C.c_void_p, C.c_void_p]),
    ("tp_shard_forward_decode_reduce", C.c_int, [C.c_void_p, C.c_int, C.c_void_p, C.c_int, C.c_void_p,
                                                 C.POINTER(C.c_void_p), C.c_void_p, C.c_void_p, C.c_void_p]),
    ("tp_partial_reduce", C.c_int, [C.POINTER(C.c_void_p), C.c_int, C.c_void_p, C.c_void_p, C.c_longlong, C.c_int,
                                    C.c_void_p]),
    ("tp_shard_debug_view", C.c_int, [C.c_void_p, C.c_int, C.POINTER(C.c_void_p)]),
    ("tp_kv_create_paged", C.c_int, [C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_int, C.POINTER(C.c_void_p)]),
    ("tp_kv_set_block_table", C.c_int, [C.c_void_p, C.c_void_p]),
    ("tp_shard_reduce_norm", C.c_int, [C.c_void_p, C.c_int, C.POINTER(C.c_void_p), C.c_int, C.c_void_p, C.c_void_p,
                                       C.c_void_p, C.c_longlong, C.c_void_p]),
    ("tp_partial_reduce_scatter", C.c_int, [C.c_void_p, C.c_int, C.c_int, C.c_void_p, C.c_void_p, C.c_longlong,
                                            C.c_int, C.c_int, C.c_void_p]),
    ("tp_all_gather", C.c_int, [C.c_void_p, C.c_int, C.c_longlong, C.c_int, C.c_int, C.c_void_p, C.c_void_p]),
    ("tp_shard_norm", C.c_int, [C.c_void_p, C.c_int, C.c_void_p, C.c_longlong, C.c_void_p, C.c_void_p]),
    ("tp_shard_fp8_view", C.c_int, [C.c_void_p, C.c_int, C.POINTER(C.c_void_p), C.POINTER(C.c_void_p),
                                    C.POINTER(C.c_int), C.POINTER(C.c_int)]),
    ("tp_tune_set_gemm_config", C.c_int, [C.c_int]),
    ("tp_tune_set_attn_groups", C.c_int, [C.c_int]),
    ("tp_tune_set_attn_kernel", C.c_int, [C.c_int]),
    ("tp_tune_gemm_plan", C.c_int, [C.c_int, C.c_int, C.c_int, C.c_int, C.POINTER(C.c_int), C.POINTER(C.c_int),
                                    C.POINTER(C.c_int)]),
    ("tp_tune_set_gemm_split", C.c_int, [C.c_int, C.c_int, C.c_int]),
    ("tp_tune_set_decode_chunk", C.c_int, [C.c_int]),
    ("tp_tune_set_decode_attn", C.c_int, [C.c_int]),
    ("tp_shard_timing", C.c_int, [C.c_void_p, C.c_int]),
    ("tp_shard_timing_read", C.c_int, [C.c_void_p, C.c_int, C.POINTER(C.c_double), C.POINTER(C.c_longlong)]),
    ("tp_shard_destroy", None, [C.c_void_p]),
    ("tp_kv_destroy", None, [C.c_void_p]),
    ("tp_status_string", C.c_char_p, [C.c_int]),
]

_lib = None


def lib():
    """The loaded library; raises if it is missing (run build() first)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m tensor_transformer_layer_tp_amd.build` (no fallback exists)")
        L = C.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class TPError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({lib().tp_status_string(status).decode()})")


def check(status: int, where: str) -> None:
    if status != TP_OK:
        raise TPError(status, where)
