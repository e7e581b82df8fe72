"""ctypes binding of the C boundary declared in ``include/ua.h``.

Argument marshalling only: every step of the forward pass runs in the HIP
library ``libua.so``.  Importing this module fails loudly when the library
has not been built (``python -m varlen_attention_serving_amd.build``); there
is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

# Device memory and streams come from torch, whose wheel carries its own HIP
# runtime.  Load it first so libua.so binds to that same runtime instead of
# pulling a second copy into the process.
import torch  # noqa: F401

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libua.so")

UA_OK, UA_ERR_INVALID_ARG, UA_ERR_UNSUPPORTED, UA_ERR_WORKSPACE, UA_ERR_HIP = range(5)
UA_DTYPE_BF16, UA_DTYPE_F16, UA_DTYPE_FP8_E4M3 = range(3)
UA_FLAG_CAUSAL = 1 << 0
UA_FLAG_SOFTCAP = 1 << 1
UA_FLAG_ALIBI = 1 << 2
UA_FLAG_WINDOW = 1 << 3
UA_FLAG_SINKS = 1 << 4
UA_FLAG_QQ_BIAS = 1 << 5
UA_FLAG_DENSE_KV = 1 << 6
UA_FLAG_BF16_PARTIALS = 1 << 7
UA_FLAG_FORCE_2D = 1 << 8
UA_FLAG_FORCE_3D = 1 << 9
UA_FLAG_PERSISTENT = 1 << 10
UA_PARTIAL_F32, UA_PARTIAL_BF16 = 0, 1
UA_MAX_MERGE_SETS = 8

STATUS_NAMES = {UA_OK: "UA_OK", UA_ERR_INVALID_ARG: "UA_ERR_INVALID_ARG",
                UA_ERR_UNSUPPORTED: "UA_ERR_UNSUPPORTED", UA_ERR_WORKSPACE: "UA_ERR_WORKSPACE",
                UA_ERR_HIP: "UA_ERR_HIP"}

# every symbol include/ua.h declares
EXPORTS = ("ua_create_problem", "ua_workspace_size", "ua_query_plan", "ua_run",
           "ua_run_no_alloc", "ua_merge", "ua_destroy_problem", "ua_last_error", "ua_version")


class ua_problem_desc_t(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("scale", ctypes.c_float),
        ("softcap", ctypes.c_float),
        ("window", ctypes.c_int32),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
        ("num_blocks", ctypes.c_int64),
        ("max_num_seqs", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("max_total_q", ctypes.c_int64),
        ("max_seqlen_k", ctypes.c_int32),
        ("split_segment_tiles", ctypes.c_int32),
        ("num_cus", ctypes.c_int32),
    ]


class ua_run_args_t(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("k_cache", ctypes.c_void_p),
        ("v_cache", ctypes.c_void_p),
        ("o", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("cu_seqlens_q", ctypes.c_void_p),
        ("alibi_slopes", ctypes.c_void_p),
        ("sinks", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("num_seqs", ctypes.c_int32),
        ("max_seqlen_q", ctypes.c_int32),
        ("total_q", ctypes.c_int64),
        ("max_seqlen_k", ctypes.c_int32),
        ("block_table_stride", ctypes.c_int32),
        ("q_stride_tok", ctypes.c_int64),
        ("o_stride_tok", ctypes.c_int64),
        ("timing_events", ctypes.c_void_p * 3),
        ("lse", ctypes.c_void_p),
        ("qq_bias", ctypes.c_void_p),
        ("qq_bias_stride", ctypes.c_int32),
        ("cu_seqlens_k", ctypes.c_void_p),
        ("partial_o", ctypes.c_void_p),
        ("partial_lse", ctypes.c_void_p),
        ("partial_dtype", ctypes.c_int32),
    ]


class ua_merge_args_t(ctypes.Structure):
    _fields_ = [
        ("num_sets", ctypes.c_int32),
        ("partial_dtype", ctypes.c_int32),
        ("partial_o", ctypes.c_void_p * UA_MAX_MERGE_SETS),
        ("partial_lse", ctypes.c_void_p * UA_MAX_MERGE_SETS),
        ("total_q", ctypes.c_int64),
        ("num_q_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("o_dtype", ctypes.c_int32),
        ("o_stride_tok", ctypes.c_int64),
        ("o", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("sinks", ctypes.c_void_p),
    ]


class ua_plan_info_t(ctypes.Structure):
    _fields_ = [
        ("path", ctypes.c_int32),
        ("block_m", ctypes.c_int32),
        ("block_q", ctypes.c_int32),
        ("tile_n", ctypes.c_int32),
        ("waves", ctypes.c_int32),
        ("num_segments", ctypes.c_int32),
        ("tiles_per_segment", ctypes.c_int32),
        ("grid", ctypes.c_int32 * 3),
        ("use_i64_kv", ctypes.c_int32),
        ("stream_k", ctypes.c_int32),
        ("class_split", ctypes.c_int32),
    ]


class UaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m varlen_attention_serving_amd.build` (no fallback exists)")
    L = ctypes.CDLL(LIB_PATH)
    vp = ctypes.c_void_p
    L.ua_create_problem.argtypes = [ctypes.POINTER(ua_problem_desc_t), ctypes.POINTER(vp)]
    L.ua_create_problem.restype = ctypes.c_int
    L.ua_workspace_size.argtypes = [vp]
    L.ua_workspace_size.restype = ctypes.c_size_t
    L.ua_query_plan.argtypes = [vp, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                ctypes.c_int32, ctypes.POINTER(ua_plan_info_t)]
    L.ua_query_plan.restype = ctypes.c_int
    L.ua_run.argtypes = [vp, ctypes.POINTER(ua_run_args_t), vp]
    L.ua_run.restype = ctypes.c_int
    L.ua_run_no_alloc.argtypes = [vp, ctypes.POINTER(ua_run_args_t), vp]
    L.ua_run_no_alloc.restype = ctypes.c_int
    L.ua_merge.argtypes = [ctypes.POINTER(ua_merge_args_t), vp]
    L.ua_merge.restype = ctypes.c_int
    L.ua_destroy_problem.argtypes = [vp]
    L.ua_destroy_problem.restype = None
    L.ua_last_error.argtypes = []
    L.ua_last_error.restype = ctypes.c_char_p
    L.ua_version.argtypes = []
    L.ua_version.restype = ctypes.c_char_p
    return L


lib = _load()


def ua_last_error() -> str:
    return lib.ua_last_error().decode()


def ua_version() -> str:
    return lib.ua_version().decode()


def _check(status: int):
    if status != UA_OK:
        raise UaError(status, ua_last_error())


def ua_create_problem(desc: ua_problem_desc_t) -> int:
    h = ctypes.c_void_p()
    _check(lib.ua_create_problem(ctypes.byref(desc), ctypes.byref(h)))
    return h.value


def ua_workspace_size(problem) -> int:
    return int(lib.ua_workspace_size(problem))


def ua_query_plan(problem, num_seqs: int, total_q: int, max_seqlen_q: int,
                  max_seqlen_k: int) -> ua_plan_info_t:
    info = ua_plan_info_t()
    _check(lib.ua_query_plan(problem, num_seqs, total_q, max_seqlen_q, max_seqlen_k,
                             ctypes.byref(info)))
    return info


def ua_run(problem, args: ua_run_args_t, stream) -> None:
    _check(lib.ua_run(problem, ctypes.byref(args), stream))


def ua_run_no_alloc(problem, args: ua_run_args_t, stream) -> None:
    _check(lib.ua_run_no_alloc(problem, ctypes.byref(args), stream))


def ua_merge(args: ua_merge_args_t, stream) -> None:
    _check(lib.ua_merge(ctypes.byref(args), stream))


def ua_destroy_problem(problem) -> None:
    lib.ua_destroy_problem(problem)
