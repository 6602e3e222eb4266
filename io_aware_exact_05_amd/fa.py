"""ctypes binding of libfa.so (include/fa.h): argument marshalling only.

Every step of the attention pass runs in the library's HIP kernels; this module
turns torch tensors into device pointers and a stream handle, calls the C
entry point of the same name, and turns a non-zero status into an exception.
There is no fallback: if libfa.so is missing or fails to load, import fails.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# FA_LIB may name another build of the same library (tile-tuning builds).
LIB_PATH = os.environ.get("FA_LIB") or os.path.join(_PKG, "libfa.so")

# fa_dtype values
FA_F32, FA_F16, FA_BF16, FA_E4M3 = 0, 1, 2, 3
DTYPE_CODE = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}

# fa_status values
FA_OK = 0
STATUS_NAMES = {0: "FA_OK", -1: "FA_ERR_NULL", -2: "FA_ERR_SHAPE", -3: "FA_ERR_DTYPE",
                -4: "FA_ERR_HEADDIM", -5: "FA_ERR_ALIGN", -6: "FA_ERR_ARG",
                -7: "FA_ERR_ALIAS", -8: "FA_ERR_LAUNCH"}

# Every symbol include/fa.h declares.
EXPORTS = ("fa_fwd", "fa_status_string", "fa_abi_version")


class FaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m io_aware_exact_05_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.fa_fwd.restype = i
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_abi_version.argtypes = []
    lib.fa_abi_version.restype = i
    return lib


_lib = _load()


def status_string(status: int) -> str:
    return _lib.fa_status_string(int(status)).decode()


def abi_version() -> int:
    return int(_lib.fa_abi_version())


def _check(status: int):
    if status != FA_OK:
        msg = status_string(status)
        if status == -8:
            raise FaError(status, msg)
        raise FaError(status, msg)


def _stream_handle(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def fa_fwd_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, B: int, H: int,
               N: int, d: int, causal: int, scale: float, dtype: int, stream: int = 0) -> int:
    """Direct call of the C entry point with integer pointers; returns the status."""
    return int(_lib.fa_fwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, int(B), int(H), int(N),
                           int(d), int(causal), float(scale), int(dtype), stream))


def fa_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
           lse: torch.Tensor, causal: bool, scale: float, stream=None) -> None:
    """fa_fwd on caller-owned device tensors q, k, v, o [B,H,N,d] and lse [B,H,N] fp32."""
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape or o.shape != q.shape:
        raise ValueError("q, k, v, o must share one [B, H, N, d] shape")
    if q.dtype not in DTYPE_CODE or k.dtype != q.dtype or v.dtype != q.dtype or o.dtype != q.dtype:
        raise ValueError("q, k, v, o must share one dtype among float32, float16, bfloat16")
    B, H, N, d = q.shape
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must be float32 of shape [B, H, N]")
    _check(fa_fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                      B, H, N, d, int(bool(causal)), scale, DTYPE_CODE[q.dtype],
                      _stream_handle(stream)))


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
              scale: float | None = None, stream=None):
    """Allocate o and lse with torch and run fa_fwd.  Returns (o, lse)."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    fa_fwd(q, k, v, o, lse, causal, scale, stream)
    return o, lse
