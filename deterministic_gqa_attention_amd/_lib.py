"""ctypes view of ``include/rla_attn.h`` (librla_attn.so).

The library is required: loading fails loudly if it has not been built, and no
call here has a CPU or PyTorch fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librla_attn.so")

RLA_OK = 0
STATUS_NAMES = {0: "RLA_OK", 1: "RLA_ERR_NULL_POINTER", 2: "RLA_ERR_BAD_SHAPE", 3: "RLA_ERR_UNSUPPORTED",
                4: "RLA_ERR_DUPLICATE_BLOCK", 5: "RLA_ERR_WORKSPACE_TOO_SMALL", 6: "RLA_ERR_HIP"}
RLA_DT_BF16, RLA_DT_FP32 = 0, 1
RLA_ORDER_GLOBAL_BLOCK_INDEX, RLA_ORDER_ARRIVAL = 0, 1
RLA_MAX_PARTS = 512

# Every function include/rla_attn.h declares.
EXPORTS = ("rla_attn_prefill", "rla_attn_prefill_chunked", "rla_attn_prefill_paged", "rla_attn_decode_paged",
           "rla_merge_states", "rla_attn_backward", "rla_lm_head_logprobs", "rla_decode_workspace_bytes",
           "rla_chunked_workspace_bytes", "rla_backward_workspace_bytes", "rla_lm_head_workspace_bytes",
           "rla_attn_decode_paged_static", "rla_last_error", "rla_core_id")
RLA_DECODE_STATIC_SCRATCH_BYTES = 132 << 20


class RlaParams(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("kv_block_size", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("causal", ctypes.c_int32),
                ("merge_order", ctypes.c_int32), ("acc_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32)]


class RlaPartials(ctypes.Structure):
    _fields_ = [("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("global_block_index", ctypes.POINTER(ctypes.c_int64)), ("n_parts", ctypes.c_int32),
                ("rows", ctypes.c_int64)]


class RlaShard(ctypes.Structure):
    _fields_ = [("kv_blocks", ctypes.POINTER(ctypes.c_int64)), ("n_kv_blocks", ctypes.c_int32),
                ("q_begin", ctypes.c_int64), ("q_count", ctypes.c_int64),
                ("partials", ctypes.POINTER(RlaPartials))]


class RLAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH):
    """Load librla_attn.so once.  Raises if it is missing (build it with
    ``python -m deterministic_gqa_attention_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m deterministic_gqa_attention_amd.build`")
    lib = ctypes.CDLL(path)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    pp = ctypes.POINTER(RlaParams)
    lib.rla_attn_prefill.argtypes = [pp, P, P, P, i32, i32, ctypes.POINTER(RlaShard), P, P, P]
    lib.rla_attn_prefill.restype = ctypes.c_int
    lib.rla_attn_prefill_chunked.argtypes = [pp, P, P, P, i32, i32, i32, i32, ctypes.POINTER(RlaShard), P, sz, P, P,
                                             P]
    lib.rla_attn_prefill_chunked.restype = ctypes.c_int
    lib.rla_attn_prefill_paged.argtypes = [pp, P, P, P, i64, i32, P, i32, i32, i32, i32, P, P, P]
    lib.rla_attn_prefill_paged.restype = ctypes.c_int
    lib.rla_attn_decode_paged.argtypes = [pp, P, P, P, i64, i32, P, i32, P, ctypes.POINTER(ctypes.c_int32),
                                          i32, i32, P, sz, P, P, P]
    lib.rla_attn_decode_paged.restype = ctypes.c_int
    lib.rla_attn_decode_paged_static.argtypes = [pp, P, P, P, i64, i32, P, i32, P, ctypes.POINTER(ctypes.c_int32),
                                                 i32, i32, P, P, P]
    lib.rla_attn_decode_paged_static.restype = ctypes.c_int
    lib.rla_attn_backward.argtypes = [pp, P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, P, P, P, P, sz, P]
    lib.rla_attn_backward.restype = ctypes.c_int
    lib.rla_lm_head_logprobs.argtypes = [P, i32, P, P, i32, i32, i32, P, P, P, sz, P]
    lib.rla_lm_head_logprobs.restype = ctypes.c_int
    lib.rla_merge_states.argtypes = [pp, ctypes.POINTER(RlaPartials), P, P, P]
    lib.rla_merge_states.restype = ctypes.c_int
    lib.rla_decode_workspace_bytes.argtypes = [pp, i32, i32]
    lib.rla_decode_workspace_bytes.restype = sz
    lib.rla_chunked_workspace_bytes.argtypes = [pp, i32, i32, i32, i32]
    lib.rla_chunked_workspace_bytes.restype = sz
    lib.rla_backward_workspace_bytes.argtypes = [pp, i32, i32]
    lib.rla_backward_workspace_bytes.restype = sz
    lib.rla_lm_head_workspace_bytes.argtypes = [i32, i32]
    lib.rla_lm_head_workspace_bytes.restype = sz
    lib.rla_last_error.argtypes = []
    lib.rla_last_error.restype = ctypes.c_char_p
    lib.rla_core_id.argtypes = []
    lib.rla_core_id.restype = ctypes.c_char_p
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != RLA_OK:
        msg = load().rla_last_error().decode(errors="replace")
        raise RLAError(status, msg)
