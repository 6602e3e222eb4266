"""Python face of the fp64 CPU attention oracle — TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this module.  The GPU library never calls it, and the two share
no code.  The arithmetic lives in ``attention_oracle.c`` (the plain definition
of exact attention from the one formula printed on the pages "FlashAttention
(HI)" / "FlashAttention (TL)", section on the problems of standard attention);
this file only builds that C file with gcc and marshals numpy arrays into it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attention_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(src: str = _SRC, out: str = _LIB, extra_flags: tuple = ()) -> str:
    """Compile an oracle C source into a shared library with gcc/OpenMP."""
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11",
           *extra_flags, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _bind(lib):
    i64, dbl, pd = ctypes.c_int64, ctypes.c_double, ctypes.POINTER(ctypes.c_double)
    lib.oracle_attention.argtypes = [pd, pd, pd, i64, i64, i64, i64,
                                     ctypes.c_int, dbl, pd, pd]
    lib.oracle_attention.restype = ctypes.c_int
    lib.oracle_attention_rows.argtypes = [pd, pd, pd, i64, i64, i64, i64,
                                          ctypes.c_int, dbl,
                                          ctypes.POINTER(ctypes.c_int64), i64,
                                          pd, pd]
    lib.oracle_attention_rows.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    return lib


def load(path: str | None = None):
    """Load (building first if absent) the oracle library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _f64(x) -> np.ndarray:
    """Exact widening to a contiguous fp64 numpy array (torch or numpy input)."""
    if hasattr(x, "detach"):  # torch tensor: widen through fp32/fp64 on the CPU
        import torch
        x = x.detach().to("cpu")
        if x.dtype not in (torch.float64,):
            x = x.to(torch.float64)
        x = x.numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def attention(q, k, v, causal: bool, scale: float, lib=None):
    """Full oracle: q, k, v of shape [B, H, N, d] -> (o [B,H,N,d], lse [B,H,N]) in fp64."""
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    B, H, N, d = q.shape
    o = np.empty((B, H, N, d), np.float64)
    lse = np.empty((B, H, N), np.float64)
    rc = lib.oracle_attention(_ptr(q), _ptr(k), _ptr(v), B, H, N, d,
                              int(bool(causal)), float(scale), _ptr(o), _ptr(lse))
    if rc != 0:
        raise RuntimeError("oracle_attention failed")
    return o, lse


def attention_rows(q, k, v, causal: bool, scale: float, rows, lib=None):
    """Selected rows: rows are flat indices (b*H + h)*N + i.  Returns (o [R,d], lse [R])."""
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    B, H, N, d = q.shape
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    o = np.empty((rows.size, d), np.float64)
    lse = np.empty((rows.size,), np.float64)
    rc = lib.oracle_attention_rows(_ptr(q), _ptr(k), _ptr(v), B, H, N, d,
                                   int(bool(causal)), float(scale),
                                   rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                   rows.size, _ptr(o), _ptr(lse))
    if rc != 0:
        raise RuntimeError("oracle_attention_rows failed")
    return o, lse


def gqa_kv_index(H: int, Hkv: int) -> np.ndarray:
    """K/V head used by each of the H query heads when Hkv K/V heads are shared:
    consecutive query heads form a group of H / Hkv that shares one K/V head
    (multi-query attention for Hkv = 1, "FlashAttention (HI)", section on
    development and further research; grouping consecutive heads is the
    plain generalisation)."""
    if Hkv < 1 or H % Hkv != 0:
        raise ValueError("Hkv must divide H")
    return np.arange(H) // (H // Hkv)


def attention_gqa(q, k, v, causal: bool, scale: float, lib=None):
    """Grouped K/V heads: q [B, H, N, d], k and v [B, Hkv, N, d].  Each query head
    attends with the K/V head gqa_kv_index gives it; the rest is `attention`."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 4 or k.ndim != 4 or k.shape != v.shape or k.shape[0] != q.shape[0] \
            or k.shape[2:] != q.shape[2:]:
        raise ValueError("q must be [B, H, N, d] and k, v one [B, Hkv, N, d] shape")
    idx = gqa_kv_index(q.shape[1], k.shape[1])
    return attention(q, np.ascontiguousarray(k[:, idx]), np.ascontiguousarray(v[:, idx]),
                     causal, scale, lib)


def num_threads(lib=None) -> int:
    return int((lib or load()).oracle_num_threads())
