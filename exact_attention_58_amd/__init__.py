"""Python binding of the MI355X exact attention library (libfa_mi355x.so).

Argument marshalling only: every step of the forward and backward passes runs in the HIP kernels
behind the C ABI declared in include/fa.h. PyTorch is used for device memory and
streams. There is no fallback: if the library is missing, the calls raise.

    fa_fwd(q, k, v, o, lse, scale, causal, stream=None)   # C-ABI fa_fwd on torch tensors
    fa_select_config(dtype, B, H, Nq, Nk, d, causal, num_cus=256) -> dict   # num_cus=None: current device
    fa_status_str(code) -> str
    attention(q, k, v, scale=None, causal=False) -> (o, lse)  # allocates o and lse
    fa_fwd_config(q, k, v, o, lse, scale, causal, cfg, stream=None)   # cfg: {"Br","Bc","waves"}
    fa_tune_fwd(q, k, v, o, lse, scale, causal, reps=10, stream=None) -> cfg dict
    fa_tune_clear()
    fa_fwd_varlen(q, k, v, o, lse, cu_q, cu_k, max_q, max_k, scale, causal, stream=None)
    attention_varlen(q, k, v, cu_q, cu_k, max_q=None, max_k=None, scale=None, causal=False)
    fa_bwd(q, k, v, o, lse, do, dq, dk, dv, delta, scale, causal, stream=None)
    attention_bwd(q, k, v, o, lse, do, scale=None, causal=False) -> (dq, dk, dv)
    fa_bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, scale, causal, stream=None)  # no workspace
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfa_mi355x.so")

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
FA_OK, FA_EINVAL, FA_EUNSUPPORTED, FA_ELAUNCH = 0, 1, 2, 3
EXPORTED = ("fa_fwd", "fa_fwd_varlen", "fa_fwd_config", "fa_tune_fwd", "fa_tune_clear", "fa_bwd",
            "fa_bwd_noalloc", "fa_status_str", "fa_select_config", "fa_select_config_cus", "fa_version")
ABI_VERSION = 2
DTYPE_NAMES = {"f32": FA_F32, "f16": FA_F16, "bf16": FA_BF16}

_lock = threading.Lock()
_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, what: str = "fa_fwd"):
        self.status = status
        super().__init__(f"{what}: {fa_status_str(status)}")


def is_built() -> bool:
    return os.path.exists(LIB_PATH)


def ensure_built() -> str:
    """Builds the library only if no build is present (tests, smoke and bench use this)."""
    if not is_built():
        from . import build as _build
        _build.build()
    return LIB_PATH


def lib():
    """The loaded shared library; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with `python -m exact_attention_58_amd.build`")
            L = ctypes.CDLL(LIB_PATH)
            i64, vp = ctypes.c_int64, ctypes.c_void_p
            L.fa_fwd.restype = ctypes.c_int
            L.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float,
                                 ctypes.c_int, ctypes.c_int, vp]
            L.fa_fwd_varlen.restype = ctypes.c_int
            L.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64,
                                        ctypes.c_float, ctypes.c_int, ctypes.c_int, vp]
            L.fa_fwd_config.restype = ctypes.c_int
            L.fa_fwd_config.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
            ip_ = ctypes.POINTER(ctypes.c_int)
            L.fa_tune_fwd.restype = ctypes.c_int
            L.fa_tune_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, ip_, ip_, ip_, ip_, ip_]
            L.fa_tune_clear.restype = None
            L.fa_tune_clear.argtypes = []
            L.fa_bwd.restype = ctypes.c_int
            L.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                 ctypes.c_float, ctypes.c_int, ctypes.c_int, vp]
            L.fa_status_str.restype = ctypes.c_char_p
            L.fa_status_str.argtypes = [ctypes.c_int]
            L.fa_bwd_noalloc.restype = ctypes.c_int
            L.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                         ctypes.c_float, ctypes.c_int, ctypes.c_int, vp]
            ip = ctypes.POINTER(ctypes.c_int)
            L.fa_select_config.restype = ctypes.c_int
            L.fa_select_config.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, ctypes.c_int, ip, ip, ip]
            L.fa_select_config_cus.restype = ctypes.c_int
            L.fa_select_config_cus.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, ctypes.c_int,
                                               ctypes.c_int, ip, ip, ip, ip]
            L.fa_version.restype = ctypes.c_int
            L.fa_version.argtypes = []
            if L.fa_version() < ABI_VERSION:
                raise RuntimeError(f"{LIB_PATH} is interface version {L.fa_version()}, older than "
                                   f"{ABI_VERSION}: rebuild it with `python -m exact_attention_58_amd.build`")
            _lib = L
    return _lib


def fa_status_str(code: int) -> str:
    return lib().fa_status_str(int(code)).decode()


def fa_select_config(dtype, B, H, Nq, Nk, d, causal, num_cus: int | None = 256) -> dict:
    """The tile configuration fa_fwd would launch: {"Br", "Bc", "waves"} (+ "dpad" when
    num_cus is given). num_cus=None asks the C-ABI fa_select_config for the current device;
    a number calls the pure fa_select_config_cus with that compute-unit count."""
    dt = DTYPE_NAMES.get(dtype, dtype)
    if num_cus is None:
        out = [ctypes.c_int(0) for _ in range(3)]
        rc = lib().fa_select_config(int(dt), B, H, Nq, Nk, d, int(bool(causal)),
                                    *[ctypes.byref(x) for x in out])
        if rc != FA_OK:
            raise FaError(rc, "fa_select_config")
        return dict(zip(("Br", "Bc", "waves"), (x.value for x in out)))
    out = [ctypes.c_int(0) for _ in range(4)]
    rc = lib().fa_select_config_cus(int(dt), B, H, Nq, Nk, d, int(bool(causal)), int(num_cus),
                                    *[ctypes.byref(x) for x in out])
    if rc != FA_OK:
        raise FaError(rc, "fa_select_config_cus")
    return dict(zip(("Br", "Bc", "waves", "dpad"), (x.value for x in out)))


def _torch_dtype_code(t):
    import torch
    codes = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def fa_fwd(q, k, v, o, lse, scale: float, causal: bool, stream=None) -> None:
    """Calls the C-ABI fa_fwd on contiguous [B,H,N,d] device tensors (o, lse preallocated).

    stream: a torch.cuda.Stream, a raw hipStream_t int, or None for torch's current stream.
    """
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B,H,N,d]")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if tuple(k.shape) != (B, H, Nk, d) or tuple(v.shape) != (B, H, Nk, d):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if tuple(o.shape) != (B, H, Nq, d) or tuple(lse.shape) != (B, H, Nq):
        raise ValueError("o must be [B,H,Nq,d] and lse [B,H,Nq]")
    if not (q.dtype == k.dtype == v.dtype == o.dtype) or lse.dtype != torch.float32:
        raise TypeError("q, k, v, o must share one dtype; lse must be float32")
    dev = q.device
    if any(t.device != dev for t in (k, v, o, lse)):
        raise ValueError("all tensors must be on one device")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(dev):
        rc = lib().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                          B, H, Nq, Nk, d, float(scale), int(bool(causal)), _torch_dtype_code(q),
                          handle)
    if rc != FA_OK:
        raise FaError(rc)


def _check_dense(q, k, v, o, lse):
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B,H,N,d]")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if tuple(k.shape) != (B, H, Nk, d) or tuple(v.shape) != (B, H, Nk, d):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if tuple(o.shape) != (B, H, Nq, d) or tuple(lse.shape) != (B, H, Nq):
        raise ValueError("o must be [B,H,Nq,d] and lse [B,H,Nq]")
    if not (q.dtype == k.dtype == v.dtype == o.dtype) or lse.dtype != torch.float32:
        raise TypeError("q, k, v, o must share one dtype; lse must be float32")
    if any(t.device != q.device for t in (k, v, o, lse)):
        raise ValueError("all tensors must be on one device")
    return B, H, Nq, Nk, d


def _stream_handle(stream, dev):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def fa_fwd_config(q, k, v, o, lse, scale: float, causal: bool, cfg: dict, stream=None) -> None:
    """fa_fwd with an explicit tile configuration: a dict with Br, Bc, waves and optionally
    the knobs occ (workgroups per CU, 0 = no cap) and group (causal dispatch group, 0 =
    built-in), as fa_tune_fwd returns it."""
    import torch
    B, H, Nq, Nk, d = _check_dense(q, k, v, o, lse)
    handle = _stream_handle(stream, q.device)
    with torch.cuda.device(q.device):
        rc = lib().fa_fwd_config(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                 B, H, Nq, Nk, d, float(scale), int(bool(causal)), _torch_dtype_code(q),
                                 int(cfg["Br"]), int(cfg["Bc"]), int(cfg["waves"]),
                                 int(cfg.get("occ", 0)), int(cfg.get("group", 0)), handle)
    if rc != FA_OK:
        raise FaError(rc, "fa_fwd_config")


def fa_tune_fwd(q, k, v, o, lse, scale: float, causal: bool, reps: int = 10, stream=None) -> dict:
    """Times every tile configuration for this problem, records the fastest for later fa_fwd
    calls on the same problem and returns it (blocks until the timed launches finish)."""
    import torch
    B, H, Nq, Nk, d = _check_dense(q, k, v, o, lse)
    handle = _stream_handle(stream, q.device)
    out = [ctypes.c_int(0) for _ in range(5)]
    with torch.cuda.device(q.device):
        rc = lib().fa_tune_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                               B, H, Nq, Nk, d, float(scale), int(bool(causal)), _torch_dtype_code(q),
                               int(reps), handle, *[ctypes.byref(x) for x in out])
    if rc != FA_OK:
        raise FaError(rc, "fa_tune_fwd")
    return dict(zip(("Br", "Bc", "waves", "occ", "group"), (x.value for x in out)))


def fa_tune_clear() -> None:
    lib().fa_tune_clear()


def attention(q, k, v, scale: float | None = None, causal: bool = False, stream=None):
    """Allocates o and lse (torch.empty) and runs fa_fwd; returns (o, lse)."""
    import torch
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    fa_fwd(q, k, v, o, lse, scale, causal, stream)
    return o, lse


def fa_fwd_varlen(q, k, v, o, lse, cu_q, cu_k, max_q: int, max_k: int, scale: float, causal: bool,
                  stream=None) -> None:
    """Calls the C-ABI fa_fwd_varlen on packed sequences: q, o [H, Tq, d], k, v [H, Tk, d],
    lse [H, Tq] float32, cu_q, cu_k int32 device tensors of B+1 offsets; max_q, max_k the
    longest query and key sequence."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), ("cu_q", cu_q), ("cu_k", cu_k)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [H, total, d]")
    H, Tq, d = q.shape
    Tk = k.shape[1]
    if tuple(k.shape) != (H, Tk, d) or tuple(v.shape) != (H, Tk, d):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if tuple(o.shape) != (H, Tq, d) or tuple(lse.shape) != (H, Tq):
        raise ValueError("o must be [H,Tq,d] and lse [H,Tq]")
    if cu_q.dim() != 1 or cu_q.shape != cu_k.shape or cu_q.numel() < 2:
        raise ValueError("cu_q and cu_k must be 1-D with B+1 entries each")
    if cu_q.dtype != torch.int32 or cu_k.dtype != torch.int32:
        raise TypeError("cu_q and cu_k must be int32")
    if not (q.dtype == k.dtype == v.dtype == o.dtype) or lse.dtype != torch.float32:
        raise TypeError("q, k, v, o must share one dtype; lse must be float32")
    dev = q.device
    if any(t.device != dev for t in (k, v, o, lse, cu_q, cu_k)):
        raise ValueError("all tensors must be on one device")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(dev):
        rc = lib().fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                 cu_q.data_ptr(), cu_k.data_ptr(), cu_q.numel() - 1, H, Tq, Tk,
                                 int(max_q), int(max_k), d, float(scale), int(bool(causal)),
                                 _torch_dtype_code(q), handle)
    if rc != FA_OK:
        raise FaError(rc, "fa_fwd_varlen")


def attention_varlen(q, k, v, cu_q, cu_k, max_q: int | None = None, max_k: int | None = None,
                     scale: float | None = None, causal: bool = False, stream=None):
    """Allocates o and lse and runs fa_fwd_varlen; returns (o, lse). Missing maxima are read
    from the offsets (a device-to-host copy)."""
    import torch
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    if max_q is None:
        max_q = max(1, int((cu_q[1:] - cu_q[:-1]).max().item()))
    if max_k is None:
        max_k = max(1, int((cu_k[1:] - cu_k[:-1]).max().item()))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    fa_fwd_varlen(q, k, v, o, lse, cu_q, cu_k, max_q, max_k, scale, causal, stream)
    return o, lse


def _check_bwd(q, k, v, o, lse, do, dq, dk, dv, delta):
    import torch
    named = [("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), ("do", do), ("dq", dq), ("dk", dk), ("dv", dv)]
    if delta is not None:
        named.append(("delta", delta))
    for name, t in named:
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B,H,N,d]")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if tuple(k.shape) != (B, H, Nk, d) or tuple(v.shape) != (B, H, Nk, d):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    shapes = [("o", o, (B, H, Nq, d)), ("do", do, (B, H, Nq, d)), ("dq", dq, (B, H, Nq, d)),
              ("dk", dk, (B, H, Nk, d)), ("dv", dv, (B, H, Nk, d)), ("lse", lse, (B, H, Nq))]
    if delta is not None:
        shapes.append(("delta", delta, (B, H, Nq)))
    for name, t, shape in shapes:
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must be {list(shape)}")
    if not all(t.dtype == q.dtype for t in (k, v, o, do, dq, dk, dv)):
        raise TypeError("q, k, v, o, do, dq, dk, dv must share one dtype")
    if lse.dtype != torch.float32 or (delta is not None and delta.dtype != torch.float32):
        raise TypeError("lse and delta must be float32")
    if any(t.device != q.device for _, t in named):
        raise ValueError("all tensors must be on one device")
    return B, H, Nq, Nk, d


def fa_bwd(q, k, v, o, lse, do, dq, dk, dv, delta, scale: float, causal: bool, stream=None) -> None:
    """Calls the C-ABI fa_bwd on contiguous device tensors (gradients and the fp32 [B,H,Nq]
    workspace `delta` preallocated)."""
    import torch
    B, H, Nq, Nk, d = _check_bwd(q, k, v, o, lse, do, dq, dk, dv, delta)
    handle = _stream_handle(stream, q.device)
    with torch.cuda.device(q.device):
        rc = lib().fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                          do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                          B, H, Nq, Nk, d, float(scale), int(bool(causal)), _torch_dtype_code(q), handle)
    if rc != FA_OK:
        raise FaError(rc, "fa_bwd")


def fa_bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, scale: float, causal: bool, stream=None) -> None:
    """Calls the C-ABI fa_bwd_noalloc: fa_bwd with the library's own row-term workspace (no
    `delta`; at most 1048576 query rows B*H*Nq; overlapping calls on one GPU race)."""
    import torch
    B, H, Nq, Nk, d = _check_bwd(q, k, v, o, lse, do, dq, dk, dv, None)
    handle = _stream_handle(stream, q.device)
    with torch.cuda.device(q.device):
        rc = lib().fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                  do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                  B, H, Nq, Nk, d, float(scale), int(bool(causal)), _torch_dtype_code(q),
                                  handle)
    if rc != FA_OK:
        raise FaError(rc, "fa_bwd_noalloc")


def attention_bwd(q, k, v, o, lse, do, scale: float | None = None, causal: bool = False, stream=None):
    """Allocates dq, dk, dv and the workspace (torch.empty) and runs fa_bwd; returns (dq, dk, dv)."""
    import torch
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    delta = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    fa_bwd(q, k, v, o, lse, do, dq, dk, dv, delta, scale, causal, stream)
    return dq, dk, dv
