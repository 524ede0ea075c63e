"""fp64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers.  The GPU path never
imports, links or runs anything here, and this package imports nothing
from the GPU path.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP), which
writes out the textbook definition that the FlashAttention-4 pages say the
fused kernel reaches exactly (Tencent Cloud, "AI Infra 系列 第六章 GPU 性能工程
（二）", section 7: the rescaling trick only skips work that does not change
the result).  This module only marshals numpy arrays into it.

All functions take and return float64 numpy arrays laid out [B][H][S][D]
(LSE: [B][H][S]).  Inputs are expected to be the exact fp64 upcast of the
bf16 values the GPU sees.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_default = None

_dp = ctypes.POINTER(ctypes.c_double)
_lp = ctypes.POINTER(ctypes.c_long)


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        compile_source(_SRC, _LIB)
    return _LIB


def _bind(lib):
    lib.oracle_attn_fwd.argtypes = [_dp, _dp, _dp, ctypes.c_long, ctypes.c_long,
                                    ctypes.c_long, ctypes.c_long, ctypes.c_double,
                                    ctypes.c_int, _dp, _dp]
    lib.oracle_attn_fwd_rows.argtypes = [_dp, _lp, ctypes.c_long, _dp, _dp,
                                         ctypes.c_long, ctypes.c_long, ctypes.c_double,
                                         ctypes.c_int, _dp, _dp]
    lib.oracle_attn_bwd_head.argtypes = [_dp, _dp, _dp, _dp, ctypes.c_long,
                                         ctypes.c_long, ctypes.c_double, ctypes.c_int,
                                         _dp, _dp, _dp, _dp, _dp]
    lib.oracle_attn_bwd.argtypes = [_dp, _dp, _dp, _dp, ctypes.c_long, ctypes.c_long,
                                    ctypes.c_long, ctypes.c_long, ctypes.c_double,
                                    ctypes.c_int, _dp, _dp, _dp]
    lib.oracle_attn_bwd_causal_tail.argtypes = [_dp, _dp, ctypes.c_long, _dp, _dp,
                                                ctypes.c_long, ctypes.c_long, ctypes.c_double,
                                                _dp, _dp, _dp]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    return lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_dp)


class Oracle:
    """The oracle's entry points bound to one compiled copy of oracle.c."""

    def __init__(self, lib_path: str):
        self.path = lib_path
        self._lib = _bind(ctypes.CDLL(lib_path))

    def max_threads(self) -> int:
        """Threads the oracle's parallel loops use."""
        return int(self._lib.oracle_max_threads())

    def set_threads(self, n: int) -> None:
        self._lib.oracle_set_threads(int(n))

    def attn_fwd(self, q, k, v, scale: float, causal: bool):
        """Forward over [B,H,S,D]: returns (O [B,H,S,D], LSE [B,H,S]) in fp64."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
            raise ValueError("q, k, v must share one [B,H,S,D] shape")
        B, H, S, D = q.shape
        o = np.empty_like(q)
        lse = np.empty((B, H, S), dtype=np.float64)
        rc = self._lib.oracle_attn_fwd(_ptr(q), _ptr(k), _ptr(v), B, H, S, D, float(scale),
                                       int(bool(causal)), _ptr(o), _ptr(lse))
        if rc:
            raise RuntimeError("oracle_attn_fwd failed (%d)" % rc)
        return o, lse

    def attn_fwd_rows(self, q_rows, pos, k, v, scale: float, causal: bool):
        """Forward for selected query rows of ONE head.

        q_rows [n,D], pos [n] (sequence positions), k, v [S,D].
        Returns (O_rows [n,D], LSE_rows [n]).
        """
        q_rows, k, v = _f64(q_rows), _f64(k), _f64(v)
        pos = np.ascontiguousarray(pos, dtype=np.int64)
        n, D = q_rows.shape
        S = k.shape[0]
        if k.shape != (S, D) or v.shape != (S, D) or pos.shape != (n,):
            raise ValueError("shape mismatch")
        o = np.empty((n, D), dtype=np.float64)
        lse = np.empty((n,), dtype=np.float64)
        rc = self._lib.oracle_attn_fwd_rows(_ptr(q_rows), pos.ctypes.data_as(_lp), n, _ptr(k),
                                            _ptr(v), S, D, float(scale), int(bool(causal)),
                                            _ptr(o), _ptr(lse))
        if rc:
            raise RuntimeError("oracle_attn_fwd_rows failed (%d)" % rc)
        return o, lse

    def attn_bwd_head(self, q, k, v, do, scale: float, causal: bool):
        """Backward for ONE head ([S,D] each) with the oracle's own forward.

        Returns (dQ, dK, dV, O, LSE).
        """
        q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
        S, D = q.shape
        outs = [np.empty_like(q) for _ in range(4)]
        lse = np.empty((S,), dtype=np.float64)
        rc = self._lib.oracle_attn_bwd_head(_ptr(q), _ptr(k), _ptr(v), _ptr(do), S, D,
                                            float(scale), int(bool(causal)), _ptr(outs[0]),
                                            _ptr(outs[1]), _ptr(outs[2]), _ptr(outs[3]),
                                            _ptr(lse))
        if rc:
            raise RuntimeError("oracle_attn_bwd_head failed (%d)" % rc)
        return outs[0], outs[1], outs[2], outs[3], lse

    def attn_bwd_causal_tail(self, q_tail, do_tail, k, v, scale: float):
        """Causal backward for the last n rows and keys of ONE head.

        q_tail, do_tail [n,D] are rows S-n .. S-1; k, v [S,D] the whole head.
        Returns (dQ, dK, dV) of rows / keys S-n .. S-1, each [n,D].
        """
        q_tail, do_tail, k, v = _f64(q_tail), _f64(do_tail), _f64(k), _f64(v)
        n, D = q_tail.shape
        S = k.shape[0]
        if do_tail.shape != (n, D) or k.shape != (S, D) or v.shape != (S, D) or n > S:
            raise ValueError("shape mismatch")
        outs = [np.empty((n, D), dtype=np.float64) for _ in range(3)]
        rc = self._lib.oracle_attn_bwd_causal_tail(_ptr(q_tail), _ptr(do_tail), n, _ptr(k),
                                                   _ptr(v), S, D, float(scale), _ptr(outs[0]),
                                                   _ptr(outs[1]), _ptr(outs[2]))
        if rc:
            raise RuntimeError("oracle_attn_bwd_causal_tail failed (%d)" % rc)
        return outs[0], outs[1], outs[2]

    def attn_bwd(self, q, k, v, do, scale: float, causal: bool):
        """Backward over [B,H,S,D]: returns (dQ, dK, dV)."""
        q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
        B, H, S, D = q.shape
        dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
        rc = self._lib.oracle_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(do), B, H, S, D,
                                       float(scale), int(bool(causal)), _ptr(dq), _ptr(dk),
                                       _ptr(dv))
        if rc:
            raise RuntimeError("oracle_attn_bwd failed (%d)" % rc)
        return dq, dk, dv


def compile_source(src: str, out: str) -> str:
    """Compile a copy of the oracle's C source (plain gcc, no fast-math)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-fno-fast-math", "-ffp-contract=off", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def default() -> Oracle:
    global _default
    with _lock:
        if _default is None:
            build()
            _default = Oracle(_LIB)
    return _default


def max_threads() -> int:
    return default().max_threads()


def set_threads(n: int) -> None:
    default().set_threads(n)


def attn_fwd(q, k, v, scale: float, causal: bool):
    return default().attn_fwd(q, k, v, scale, causal)


def attn_fwd_rows(q_rows, pos, k, v, scale: float, causal: bool):
    return default().attn_fwd_rows(q_rows, pos, k, v, scale, causal)


def attn_bwd_head(q, k, v, do, scale: float, causal: bool):
    return default().attn_bwd_head(q, k, v, do, scale, causal)


def attn_bwd(q, k, v, do, scale: float, causal: bool):
    return default().attn_bwd(q, k, v, do, scale, causal)


def attn_bwd_causal_tail(q_tail, do_tail, k, v, scale: float):
    return default().attn_bwd_causal_tail(q_tail, do_tail, k, v, scale)


def fwd_flops(B: int, H: int, S: int, D: int, causal: bool) -> float:
    """Algorithmic forward FLOPs (4*B*H*S^2*D, halved when causal)."""
    f = 4.0 * B * H * S * S * D
    return f / 2 if causal else f


def rows_flops(pos, S: int, D: int, causal: bool) -> float:
    """Exact algorithmic FLOPs for a set of forward rows: 4*D per visible key."""
    pos = np.asarray(pos, dtype=np.int64)
    keys = (pos + 1) if causal else np.full(pos.shape, S)
    return float(4.0 * D * keys.sum())
