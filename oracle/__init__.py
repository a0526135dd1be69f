"""fp64 CPU oracle for exact scaled-dot-product attention (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never touches it, and it never touches the product path:
the two share no code.  See ``oracle.c`` for what each entry point computes
and which passage of the pages it follows.

The wrappers take float64 numpy arrays in [B, H, N, d] layout (any array that
``np.ascontiguousarray(x, dtype=np.float64)`` accepts) and return float64
arrays.  Inputs that came from bf16/fp16 tensors are widened exactly.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_default = None

# -O2 without fast-math: IEEE fp64 with libm exp/log, no reassociation.
_CFLAGS = ["-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", "-Wall", "-Wextra"]


def compile_source(src: str, out: str) -> str:
    """Compile a C source of the oracle's form into a shared library."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", *_CFLAGS, src, "-o", tmp, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (the checker, not the product)."""
    if force or not os.path.exists(_LIB):
        compile_source(_SRC, _LIB)
    return _LIB


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor: widen on the host, exactly
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _shape(Q, K):
    if Q.ndim != 4 or K.ndim != 4:
        raise ValueError("expected [B, H, N, d] arrays")
    B, H, Nq, d = Q.shape
    if K.shape[0] != B or K.shape[1] != H or K.shape[3] != d:
        raise ValueError("Q and K disagree in B, H or d")
    return B, H, Nq, K.shape[2], d


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError("%s failed (rc=%d)" % (what, rc))


class Oracle:
    """ctypes front end of one compiled oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P = ctypes.POINTER(ctypes.c_double)
        I64 = ctypes.c_int64
        PI = ctypes.POINTER(ctypes.c_int64)
        D, I = ctypes.c_double, ctypes.c_int
        lib.oracle_fwd.argtypes = [P, P, P, I64, I64, I64, I64, I64, D, I, P, P, P]
        lib.oracle_fwd_rows.argtypes = [P, P, P, I64, I64, I64, I64, I64, D, I, PI, I64, P, P]
        lib.oracle_bwd.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, D, I, P, P, P, P, P]
        lib.oracle_online_row.argtypes = [P, P, I64, I64, I64, I64, P, P, P]
        lib.oracle_tiled_fwd.argtypes = [P, P, P, I64, I64, I64, I64, I64, D, I, I64, P, P]
        lib.oracle_num_threads.argtypes = []
        U32P = ctypes.POINTER(ctypes.c_uint32)
        U8P = ctypes.POINTER(ctypes.c_uint8)
        lib.oracle_philox4x32_10.argtypes = [U32P, U32P, U32P]
        lib.oracle_philox4x32_10.restype = None
        lib.oracle_dropout_keep.argtypes = [I64, I64, I64, I64, I, ctypes.c_uint64, I64, U8P]
        lib.oracle_fwd_dropout.argtypes = [P, P, P, I64, I64, I64, I64, I64, D, I, U8P, D, P, P]
        lib.oracle_bwd_dropout.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, D, I, U8P, D, P, P, P, P, P]
        for name in ("oracle_fwd", "oracle_fwd_rows", "oracle_bwd", "oracle_online_row",
                     "oracle_tiled_fwd", "oracle_num_threads", "oracle_dropout_keep", "oracle_fwd_dropout",
                     "oracle_bwd_dropout"):
            getattr(lib, name).restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def fwd(self, Q, K, V, scale: float, causal: bool = False, want_probs: bool = False):
        """Untiled forward.  Returns (O, LSE) or (O, LSE, P)."""
        Q, K, V = _f64(Q), _f64(K), _f64(V)
        B, H, Nq, Nk, d = _shape(Q, K)
        if V.shape != K.shape:
            raise ValueError("V must have K's shape")
        O = np.empty((B, H, Nq, d))
        LSE = np.empty((B, H, Nq))
        Pm = np.empty((B, H, Nq, Nk)) if want_probs else None
        _check(self.lib.oracle_fwd(_ptr(Q), _ptr(K), _ptr(V), B, H, Nq, Nk, d, float(scale),
                                   int(bool(causal)), _ptr(O), _ptr(LSE),
                                   _ptr(Pm) if want_probs else None), "oracle_fwd")
        return (O, LSE, Pm) if want_probs else (O, LSE)

    def fwd_rows(self, Q, K, V, rows, scale: float, causal: bool = False):
        """Forward for selected query rows.  rows: int array [B*H, R] (or [R],
        the same rows for every head).  Returns O_rows [B*H, R, d], LSE_rows [B*H, R]."""
        Q, K, V = _f64(Q), _f64(K), _f64(V)
        B, H, Nq, Nk, d = _shape(Q, K)
        rows = np.asarray(rows, dtype=np.int64)
        if rows.ndim == 1:
            rows = np.broadcast_to(rows, (B * H, rows.shape[0]))
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        if rows.shape[0] != B * H:
            raise ValueError("rows must be [B*H, R]")
        R = rows.shape[1]
        O = np.empty((B * H, R, d))
        LSE = np.empty((B * H, R))
        _check(self.lib.oracle_fwd_rows(_ptr(Q), _ptr(K), _ptr(V), B, H, Nq, Nk, d, float(scale),
                                        int(bool(causal)),
                                        rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), R,
                                        _ptr(O), _ptr(LSE)), "oracle_fwd_rows")
        return O, LSE

    def bwd(self, Q, K, V, dO, scale: float, causal: bool = False):
        """Backward.  Returns (dQ, dK, dV, O, LSE)."""
        Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
        B, H, Nq, Nk, d = _shape(Q, K)
        if dO.shape != Q.shape or V.shape != K.shape:
            raise ValueError("dO must have Q's shape and V K's shape")
        dQ, dK, dV = np.empty_like(Q), np.empty_like(K), np.empty_like(V)
        O, LSE = np.empty_like(Q), np.empty((B, H, Nq))
        _check(self.lib.oracle_bwd(_ptr(Q), _ptr(K), _ptr(V), _ptr(dO), B, H, Nq, Nk, d, float(scale),
                                   int(bool(causal)), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(O), _ptr(LSE)),
               "oracle_bwd")
        return dQ, dK, dV, O, LSE

    def online_row(self, scores, values, tile: int, ntiles: int = -1):
        """Running-state recurrence for one row; returns (m, l, u) after `ntiles`
        tiles (all tiles when ntiles < 0), u unnormalised."""
        s = _f64(scores).reshape(-1)
        v = _f64(values)
        n, dv = v.shape
        if s.shape[0] != n:
            raise ValueError("scores and values disagree in length")
        m, l = ctypes.c_double(), ctypes.c_double()
        u = np.empty(dv)
        _check(self.lib.oracle_online_row(_ptr(s), _ptr(v), n, dv, int(tile), int(ntiles),
                                          ctypes.byref(m), ctypes.byref(l), _ptr(u)), "oracle_online_row")
        return m.value, l.value, u

    def tiled_fwd(self, Q, K, V, scale: float, causal: bool = False, tile: int = 64):
        """Forward through the running-state recurrence in key tiles of `tile`."""
        Q, K, V = _f64(Q), _f64(K), _f64(V)
        B, H, Nq, Nk, d = _shape(Q, K)
        O = np.empty((B, H, Nq, d))
        LSE = np.empty((B, H, Nq))
        _check(self.lib.oracle_tiled_fwd(_ptr(Q), _ptr(K), _ptr(V), B, H, Nq, Nk, d, float(scale),
                                         int(bool(causal)), int(tile), _ptr(O), _ptr(LSE)),
               "oracle_tiled_fwd")
        return O, LSE

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    # ---- dropout (see oracle.c: inverted dropout on P, Philox4x32-10 keep mask)

    def philox4x32_10(self, ctr, key):
        """Philox4x32-10 of a 4-word counter and a 2-word key; returns 4 uint32."""
        c = np.ascontiguousarray(ctr, dtype=np.uint32)
        k = np.ascontiguousarray(key, dtype=np.uint32)
        out = np.empty(4, dtype=np.uint32)
        U32P = ctypes.POINTER(ctypes.c_uint32)
        self.lib.oracle_philox4x32_10(c.ctypes.data_as(U32P), k.ctypes.data_as(U32P), out.ctypes.data_as(U32P))
        return out

    def dropout_keep(self, B, H, Nq, Nk, t: int, seed: int, bh0: int = 0):
        """uint8 keep mask [B, H, Nq, Nk] for drop threshold t (rate t/256), for
        the B*H heads starting at flat head index bh0."""
        keep = np.empty((B, H, Nq, Nk), dtype=np.uint8)
        _check(self.lib.oracle_dropout_keep(B, H, Nq, Nk, int(t), ctypes.c_uint64(int(seed) & (2 ** 64 - 1)),
                                            int(bh0), keep.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))),
               "oracle_dropout_keep")
        return keep

    def fwd_dropout(self, Q, K, V, keep, keep_scale: float, scale: float, causal: bool = False):
        """Forward with dropout on P under the given keep mask.  Returns (O, LSE)."""
        Q, K, V = _f64(Q), _f64(K), _f64(V)
        B, H, Nq, Nk, d = _shape(Q, K)
        keep = np.ascontiguousarray(keep, dtype=np.uint8)
        if keep.shape != (B, H, Nq, Nk):
            raise ValueError("keep must be [B, H, Nq, Nk]")
        O = np.empty((B, H, Nq, d))
        LSE = np.empty((B, H, Nq))
        _check(self.lib.oracle_fwd_dropout(_ptr(Q), _ptr(K), _ptr(V), B, H, Nq, Nk, d, float(scale),
                                           int(bool(causal)), keep.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
                                           float(keep_scale), _ptr(O), _ptr(LSE)), "oracle_fwd_dropout")
        return O, LSE

    def bwd_dropout(self, Q, K, V, dO, keep, keep_scale: float, scale: float, causal: bool = False):
        """Backward with dropout on P.  Returns (dQ, dK, dV, O, LSE)."""
        Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
        B, H, Nq, Nk, d = _shape(Q, K)
        keep = np.ascontiguousarray(keep, dtype=np.uint8)
        if keep.shape != (B, H, Nq, Nk):
            raise ValueError("keep must be [B, H, Nq, Nk]")
        dQ, dK, dV = np.empty_like(Q), np.empty_like(K), np.empty_like(V)
        O, LSE = np.empty_like(Q), np.empty((B, H, Nq))
        _check(self.lib.oracle_bwd_dropout(_ptr(Q), _ptr(K), _ptr(V), _ptr(dO), B, H, Nq, Nk, d, float(scale),
                                           int(bool(causal)), keep.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
                                           float(keep_scale), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(O), _ptr(LSE)),
               "oracle_bwd_dropout")
        return dQ, dK, dV, O, LSE


def load() -> Oracle:
    """The oracle built from oracle.c (compiled on first use if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB):
            build(force=True)
        _default = Oracle(_LIB)
    return _default


def fwd(*a, **k):
    return load().fwd(*a, **k)


def fwd_rows(*a, **k):
    return load().fwd_rows(*a, **k)


def bwd(*a, **k):
    return load().bwd(*a, **k)


def online_row(*a, **k):
    return load().online_row(*a, **k)


def tiled_fwd(*a, **k):
    return load().tiled_fwd(*a, **k)


def num_threads() -> int:
    return load().num_threads()


def philox4x32_10(*a, **k):
    return load().philox4x32_10(*a, **k)


def dropout_keep(*a, **k):
    return load().dropout_keep(*a, **k)


def fwd_dropout(*a, **k):
    return load().fwd_dropout(*a, **k)


def bwd_dropout(*a, **k):
    return load().bwd_dropout(*a, **k)
