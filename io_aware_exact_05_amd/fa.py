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
                -7: "FA_ERR_ALIAS", -8: "FA_ERR_LAUNCH", -9: "FA_ERR_SCRATCH"}

# FA_KVCACHE_SCRATCH_BYTES: the static scratch of fa_fwd_kvcache_noalloc, per device
KVCACHE_SCRATCH_BYTES = 16 << 20

# Every symbol include/fa.h declares.
EXPORTS = ("fa_fwd", "fa_fwd_gqa", "fa_bwd", "fa_bwd_gqa", "fa_bwd_workspace_bytes",
           "fa_fwd_kvcache", "fa_fwd_kvcache_workspace_bytes", "fa_fwd_kvcache_noalloc",
           "fa_fwd_fp8", "fa_quantize_e4m3",
           "fa_status_string", "fa_abi_version")


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
    lib.fa_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    lib.fa_fwd_gqa.restype = i
    sz = ctypes.c_size_t
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f, i, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd_gqa.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, f, i,
                               vp]
    lib.fa_bwd_gqa.restype = i
    lib.fa_bwd_workspace_bytes.argtypes = [i, i, i]
    lib.fa_bwd_workspace_bytes.restype = sz
    lib.fa_fwd_kvcache.argtypes = [vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, i, f, i, vp]
    lib.fa_fwd_kvcache.restype = i
    lib.fa_fwd_kvcache_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.fa_fwd_kvcache_workspace_bytes.restype = sz
    lib.fa_fwd_kvcache_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp]
    lib.fa_fwd_kvcache_noalloc.restype = i
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
    lib.fa_fwd_fp8.restype = i
    lib.fa_quantize_e4m3.argtypes = [vp, vp, vp, i, i, i, i, i, i, vp, vp]
    lib.fa_quantize_e4m3.restype = i
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


def fa_fwd_gqa_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, B: int, H: int,
                   Hkv: int, N: int, d: int, causal: int, scale: float, dtype: int,
                   stream: int = 0) -> int:
    """Direct call of fa_fwd_gqa with integer pointers; returns the status."""
    return int(_lib.fa_fwd_gqa(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, int(B), int(H), int(Hkv),
                               int(N), int(d), int(causal), float(scale), int(dtype), stream))


def fa_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
           lse: torch.Tensor, causal: bool, scale: float, stream=None) -> None:
    """Forward pass on caller-owned device tensors: q, o [B,H,N,d], k, v [B,Hkv,N,d] with
    Hkv dividing H (Hkv = H: fa_fwd; fewer: fa_fwd_gqa), lse [B,H,N] fp32."""
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dim() != 4 or o.shape != q.shape or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q, o must be [B, H, N, d] and k, v one [B, Hkv, N, d] shape")
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape[0] != B or tuple(k.shape[2:]) != (N, d) or Hkv < 1 or H % Hkv != 0:
        raise ValueError("k, v must be [B, Hkv, N, d] with Hkv dividing H")
    if q.dtype not in DTYPE_CODE or k.dtype != q.dtype or v.dtype != q.dtype or o.dtype != q.dtype:
        raise ValueError("q, k, v, o must share one dtype among float32, float16, bfloat16")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must be float32 of shape [B, H, N]")
    if Hkv == H:
        status = fa_fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                            B, H, N, d, int(bool(causal)), scale, DTYPE_CODE[q.dtype],
                            _stream_handle(stream))
    else:
        status = fa_fwd_gqa_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                lse.data_ptr(), B, H, Hkv, N, d, int(bool(causal)), scale,
                                DTYPE_CODE[q.dtype], _stream_handle(stream))
    _check(status)


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
              scale: float | None = None, stream=None):
    """Allocate o and lse with torch and run the forward pass (k, v may have fewer heads than
    q, their count dividing H).  Returns (o, lse)."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    fa_fwd(q, k, v, o, lse, causal, scale, stream)
    return o, lse


# ----------------------------------------------------------------------------
# backward pass
# ----------------------------------------------------------------------------

def bwd_workspace_bytes(B: int, H: int, N: int) -> int:
    return int(_lib.fa_bwd_workspace_bytes(int(B), int(H), int(N)))


def fa_bwd_raw(q, k, v, o, dout, lse, dq, dk, dv, ws, ws_bytes, B, H, N, d, causal, scale, dtype,
               stream=0) -> int:
    """Direct call of fa_bwd with integer pointers; returns the status."""
    return int(_lib.fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, ws, ws_bytes, int(B), int(H), int(N),
                           int(d), int(causal), float(scale), int(dtype), stream))


def fa_bwd_gqa_raw(q, k, v, o, dout, lse, dq, dk, dv, ws, ws_bytes, B, H, Hkv, N, d, causal, scale,
                   dtype, stream=0) -> int:
    """Direct call of fa_bwd_gqa with integer pointers; returns the status."""
    return int(_lib.fa_bwd_gqa(q, k, v, o, dout, lse, dq, dk, dv, ws, ws_bytes, int(B), int(H),
                               int(Hkv), int(N), int(d), int(causal), float(scale), int(dtype),
                               stream))


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, causal: bool, scale: float,
           stream=None) -> None:
    """Backward pass on caller-owned device tensors: q, o, dout, dq [B,H,N,d]; k, v, dk, dv
    [B,Hkv,N,d] (Hkv dividing H); lse [B,H,N] fp32 from the forward; workspace a uint8
    device tensor of at least bwd_workspace_bytes(B, H, N) bytes."""
    named = (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("lse", lse), ("dq", dq),
             ("dk", dk), ("dv", dv), ("workspace", workspace))
    for name, t in named:
        _dev(name, t)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, H, N, d] and k [B, Hkv, N, d]")
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape[0] != B or tuple(k.shape[2:]) != (N, d) or Hkv < 1 or H % Hkv != 0:
        raise ValueError("k, v must be [B, Hkv, N, d] with Hkv dividing H")
    for name, t in (("o", o), ("dout", dout), ("dq", dq)):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must match q in shape and dtype")
    for name, t in (("v", v), ("dk", dk), ("dv", dv)):
        if t.shape != k.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must match k in shape and q in dtype")
    if q.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("the backward pass takes float16 or bfloat16")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must be float32 of shape [B, H, N]")
    wsb = workspace.numel() * workspace.element_size()
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), wsb)
    tail = (d, int(bool(causal)), scale, DTYPE_CODE[q.dtype], _stream_handle(stream))
    if Hkv == H:
        status = fa_bwd_raw(*args, B, H, N, *tail)
    else:
        status = fa_bwd_gqa_raw(*args, B, H, Hkv, N, *tail)
    _check(status)


def attention_bwd(q, k, v, o, dout, lse, causal: bool = False, scale: float | None = None,
                  stream=None):
    """Allocate dq, dk, dv and the workspace with torch and run the backward pass.
    Returns (dq, dk, dv)."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    B, H, N, _ = q.shape
    ws = torch.empty(bwd_workspace_bytes(B, H, N), dtype=torch.uint8, device=q.device)
    fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, ws, causal, scale, stream)
    return dq, dk, dv


# ----------------------------------------------------------------------------
# attention over a key/value cache (decoding)
# ----------------------------------------------------------------------------

def kvcache_workspace_bytes(B: int, H: int, Hkv: int, Nq: int, Nkv: int, d: int) -> int:
    return int(_lib.fa_fwd_kvcache_workspace_bytes(int(B), int(H), int(Hkv), int(Nq), int(Nkv),
                                                   int(d)))


def fa_fwd_kvcache_raw(q, k, v, o, lse, ws, ws_bytes, B, H, Hkv, Nq, Nkv, d, causal, scale, dtype,
                       stream=0) -> int:
    """Direct call of fa_fwd_kvcache with integer pointers; returns the status."""
    return int(_lib.fa_fwd_kvcache(q, k, v, o, lse, ws, ws_bytes, int(B), int(H), int(Hkv),
                                   int(Nq), int(Nkv), int(d), int(causal), float(scale),
                                   int(dtype), stream))


def fa_fwd_kvcache_noalloc_raw(q, k, v, o, lse, B, H, Hkv, Nq, Nkv, d, causal, scale, dtype,
                               stream=0) -> int:
    """Direct call of fa_fwd_kvcache_noalloc with integer pointers; returns the status."""
    return int(_lib.fa_fwd_kvcache_noalloc(q, k, v, o, lse, int(B), int(H), int(Hkv), int(Nq),
                                           int(Nkv), int(d), int(causal), float(scale), int(dtype),
                                           stream))


def _kvcache_shapes(q, k, v, o, lse):
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse)):
        _dev(name, t)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape or o.shape != q.shape:
        raise ValueError("q, o must be [B, H, Nq, d] and k, v one [B, Hkv, Nkv, d] shape")
    B, H, Nq, d = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k, v must be [B, Hkv, Nkv, d]")
    if q.dtype not in (torch.float16, torch.bfloat16) or any(t.dtype != q.dtype for t in (k, v, o)):
        raise ValueError("q, k, v, o must share float16 or bfloat16")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, Nq):
        raise ValueError("lse must be float32 of shape [B, H, Nq]")
    return B, H, Hkv, Nq, Nkv, d


def fa_fwd_kvcache(q, k, v, o, lse, workspace, causal: bool, scale: float, stream=None) -> None:
    """q, o [B,H,Nq,d]; k, v [B,Hkv,Nkv,d]; lse [B,H,Nq] fp32; workspace a uint8 device tensor
    of at least kvcache_workspace_bytes(...) bytes (or None when that is 0)."""
    B, H, Hkv, Nq, Nkv, d = _kvcache_shapes(q, k, v, o, lse)
    wp, wb = 0, 0
    if workspace is not None:
        _dev("workspace", workspace)
        wp, wb = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check(fa_fwd_kvcache_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              lse.data_ptr(), wp or None, wb, B, H, Hkv, Nq, Nkv, d,
                              int(bool(causal)), scale, DTYPE_CODE[q.dtype],
                              _stream_handle(stream)))


def fa_fwd_kvcache_noalloc(q, k, v, o, lse, causal: bool, scale: float, stream=None) -> None:
    """fa_fwd_kvcache with the library's static per-device scratch as the workspace: the call
    allocates nothing.  Calls that overlap in time on one device race on that scratch."""
    B, H, Hkv, Nq, Nkv, d = _kvcache_shapes(q, k, v, o, lse)
    _check(fa_fwd_kvcache_noalloc_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                      lse.data_ptr(), B, H, Hkv, Nq, Nkv, d, int(bool(causal)),
                                      scale, DTYPE_CODE[q.dtype], _stream_handle(stream)))


def attention_kvcache(q, k, v, causal: bool = False, scale: float | None = None, stream=None):
    """Allocate o, lse and the workspace with torch and run fa_fwd_kvcache.  Returns (o, lse)."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    B, H, Nq, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    nb = kvcache_workspace_bytes(B, H, k.shape[1], Nq, k.shape[2], d)
    ws = torch.empty(nb, dtype=torch.uint8, device=q.device) if nb else None
    fa_fwd_kvcache(q, k, v, o, lse, ws, causal, scale, stream)
    return o, lse


# ----------------------------------------------------------------------------
# fp8 (OCP e4m3fn) path
# ----------------------------------------------------------------------------

def fa_fwd_fp8_raw(q8, k8, v8, qd, kd, vd, o, lse, B, H, N, d, causal, scale, stream=0) -> int:
    """Direct call of fa_fwd_fp8 with integer pointers; returns the status."""
    return int(_lib.fa_fwd_fp8(q8, k8, v8, qd, kd, vd, o, lse, int(B), int(H), int(N), int(d),
                               int(causal), float(scale), stream))


def fa_quantize_e4m3_raw(x, x8, descale, B, H, N, d, block_rows, rotate, signs, stream=0) -> int:
    """Direct call of fa_quantize_e4m3 with integer pointers; returns the status."""
    return int(_lib.fa_quantize_e4m3(x, x8, descale, int(B), int(H), int(N), int(d),
                                     int(block_rows), int(rotate), signs, stream))


def _dev(name, t, dtype=None):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}")


def fa_quantize_e4m3(x: torch.Tensor, x8: torch.Tensor, descale: torch.Tensor,
                     rotate: bool = False, signs: torch.Tensor | None = None,
                     stream=None) -> None:
    """x fp32 [B,H,N,d] -> x8 (uint8 codes, same shape) and descale fp32 [B,H,ceil(N/128)]."""
    _dev("x", x, torch.float32)
    _dev("x8", x8, torch.uint8)
    _dev("descale", descale, torch.float32)
    if signs is not None:
        _dev("signs", signs, torch.float32)
    B, H, N, d = x.shape
    if tuple(x8.shape) != (B, H, N, d) or tuple(descale.shape) != (B, H, (N + 127) // 128):
        raise ValueError("x8 must match x and descale must be [B, H, ceil(N/128)]")
    _check(fa_quantize_e4m3_raw(x.data_ptr(), x8.data_ptr(), descale.data_ptr(), B, H, N, d, 128,
                                int(bool(rotate)), signs.data_ptr() if signs is not None else None,
                                _stream_handle(stream)))


def quantize_e4m3(x: torch.Tensor, rotate: bool = False, signs: torch.Tensor | None = None,
                  stream=None):
    """Allocate and quantise: returns (x8 uint8 [B,H,N,d], descale fp32 [B,H,ceil(N/128)])."""
    B, H, N, d = x.shape
    x8 = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    desc = torch.empty((B, H, (N + 127) // 128), dtype=torch.float32, device=x.device)
    fa_quantize_e4m3(x, x8, desc, rotate, signs, stream)
    return x8, desc


def fa_fwd_fp8(q8, k8, v8, q_descale, k_descale, v_descale, o, lse, causal: bool, scale: float,
               stream=None) -> None:
    """fa_fwd_fp8 on device tensors: codes uint8 [B,H,N,d], descales fp32, o bf16, lse fp32."""
    for name, t in (("q8", q8), ("k8", k8), ("v8", v8)):
        _dev(name, t, torch.uint8)
    for name, t in (("q_descale", q_descale), ("k_descale", k_descale), ("v_descale", v_descale)):
        _dev(name, t, torch.float32)
    _dev("o", o, torch.bfloat16)
    _dev("lse", lse, torch.float32)
    B, H, N, d = q8.shape
    if k8.shape != q8.shape or v8.shape != q8.shape or o.shape != q8.shape:
        raise ValueError("q8, k8, v8, o must share one [B, H, N, d] shape")
    nb = (N + 127) // 128
    for t in (q_descale, k_descale, v_descale):
        if tuple(t.shape) != (B, H, nb):
            raise ValueError("descales must be [B, H, ceil(N/128)]")
    if tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must be [B, H, N]")
    _check(fa_fwd_fp8_raw(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), q_descale.data_ptr(),
                          k_descale.data_ptr(), v_descale.data_ptr(), o.data_ptr(), lse.data_ptr(),
                          B, H, N, d, int(bool(causal)), scale, _stream_handle(stream)))


def attention_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                  scale: float | None = None, rotate: bool = True,
                  signs: torch.Tensor | None = None, stream=None):
    """fp32 Q, K, V -> quantise (Q and K rotated with the same signs when rotate) -> fp8
    attention.  Returns (o bf16, lse fp32)."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    q8, qd = quantize_e4m3(q, rotate, signs, stream)
    k8, kd = quantize_e4m3(k, rotate, signs, stream)
    v8, vd = quantize_e4m3(v, False, None, stream)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    fa_fwd_fp8(q8, k8, v8, qd, kd, vd, o, lse, causal, scale, stream)
    return o, lse
