"""fp64 CPU oracle for unified paged attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path never does: it runs
the HIP library and fails loudly when that is missing.

The arithmetic lives in ``ua_oracle.c`` (plain loops over the definition in
"Unified paged attention on gfx950, from the math up", section 1).  This
module builds it with gcc and marshals numpy arrays into it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ua_oracle.c")
_LIB = os.path.join(_HERE, "libua_oracle.so")


class UaoProblem(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("use_softcap", ctypes.c_int32),
        ("use_alibi", ctypes.c_int32),
        ("use_window", ctypes.c_int32),
        ("use_sinks", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("block_table_stride", ctypes.c_int32),
        ("q_stride_tok", ctypes.c_int64),
        ("scale", ctypes.c_double),
        ("softcap", ctypes.c_double),
        ("k_scale", ctypes.c_double),
        ("v_scale", ctypes.c_double),
        ("use_qq_bias", ctypes.c_int32),
        ("qq_bias_stride", ctypes.c_int32),
        ("qq_bias", ctypes.c_void_p),
    ]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, IEEE semantics, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def open_library(path: str):
    """Load a compiled oracle and declare its entry points."""
    L = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    L.uao_attention.argtypes = [ctypes.POINTER(UaoProblem), vp, vp, vp, vp, vp, vp, vp, vp,
                                vp, vp, ctypes.c_int]
    L.uao_attention.restype = ctypes.c_int
    L.uao_rows.argtypes = [ctypes.POINTER(UaoProblem), vp, vp, vp, vp, vp, vp, vp, vp, vp,
                           ctypes.c_int64, vp, vp, ctypes.c_int]
    L.uao_rows.restype = ctypes.c_int
    L.uao_decode.argtypes = [ctypes.c_int, ctypes.c_uint32]
    L.uao_decode.restype = ctypes.c_double
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = open_library(_LIB)
    return _lib


def default_threads() -> int:
    """Host threads for the oracle: the affinity set, capped by OMP_NUM_THREADS."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _problem(w) -> UaoProblem:
    qq = getattr(w, "qq_bias", None)
    p = UaoProblem(
        num_seqs=w.num_seqs, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
        head_dim=w.head_dim, block_size=w.block_size, q_dtype=w.q_dtype, kv_dtype=w.kv_dtype,
        causal=int(w.causal), use_softcap=int(w.softcap > 0), use_alibi=int(w.use_alibi),
        use_window=int(w.window > 0), use_sinks=int(w.use_sinks), window=int(w.window),
        block_table_stride=int(w.block_table.shape[1]),
        q_stride_tok=int(w.num_q_heads * w.head_dim), scale=float(w.scale),
        softcap=float(w.softcap), k_scale=float(w.k_scale), v_scale=float(w.v_scale))
    if qq is not None:
        qq = np.ascontiguousarray(qq, dtype=np.float32)
        p._qq_keep = qq  # the struct holds a raw pointer: keep the array alive with it
        p.use_qq_bias = 1
        p.qq_bias_stride = int(qq.shape[1])
        p.qq_bias = qq.ctypes.data
    return p


def _arrays(w):
    arrs = [np.ascontiguousarray(w.q), np.ascontiguousarray(w.k_cache),
            np.ascontiguousarray(w.v_cache), np.ascontiguousarray(w.block_table, np.int32),
            np.ascontiguousarray(w.seq_lens, np.int32),
            np.ascontiguousarray(w.cu_seqlens_q, np.int32),
            None if w.alibi_slopes is None else np.ascontiguousarray(w.alibi_slopes, np.float32),
            None if w.sinks is None else np.ascontiguousarray(w.sinks, np.float32)]
    return arrs


def attention(w, nthreads: Optional[int] = None, return_lse: bool = False):
    """All rows of workload ``w``: fp64 O [T_q, H_q, d] (and LSE [T_q, H_q])."""
    p = _problem(w)
    arrs = _arrays(w)
    out = np.zeros((w.total_q, w.num_q_heads, w.head_dim), dtype=np.float64)
    lse = np.zeros((w.total_q, w.num_q_heads), dtype=np.float64) if return_lse else None
    rc = lib().uao_attention(ctypes.byref(p), *[_ptr(a) for a in arrs], _ptr(out), _ptr(lse),
                             nthreads or default_threads())
    if rc:
        raise RuntimeError("oracle rejected the workload")
    return (out, lse) if return_lse else out


def rows(w, rows_idx: np.ndarray, nthreads: Optional[int] = None, return_lse: bool = False):
    """Selected rows (token * H_q + head): fp64 O [n, d] (and LSE [n])."""
    p = _problem(w)
    arrs = _arrays(w)
    r = np.ascontiguousarray(rows_idx, dtype=np.int64)
    out = np.zeros((r.shape[0], w.head_dim), dtype=np.float64)
    lse = np.zeros(r.shape[0], dtype=np.float64) if return_lse else None
    rc = lib().uao_rows(ctypes.byref(p), *[_ptr(a) for a in arrs], _ptr(r), r.shape[0],
                        _ptr(out), _ptr(lse), nthreads or default_threads())
    if rc:
        raise RuntimeError("oracle rejected the workload")
    return (out, lse) if return_lse else out


def decode(dtype: int, bits: int) -> float:
    """The oracle's exact decoder of one stored value."""
    return float(lib().uao_decode(int(dtype), int(bits)))
