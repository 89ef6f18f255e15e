"""fp64 CPU oracle for exact attention: the forward (ctypes wrapper over attn_oracle.c) and
its gradients (attention_bwd, numpy on full matrices).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does, and this
package imports nothing from the product.

The oracle evaluates the plain definition of softmax attention in fp64 on inputs
upcast exactly from their storage dtype: scores = scale * q.k (page
"flash_attention_2.cu", forward kernel), top-left causal mask j <= i (same page,
causal guard), softmax by max / exp / sum, O = P.V / l and L = m + ln(l) (same
page, final normalisation). No tiling and no online recurrence.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "libattn_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile attn_oracle.c with gcc (no fast-math: IEEE fp64 throughout)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
           "-ffp-contract=off", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            lib = ctypes.CDLL(_LIB)
            f = lib.attn_oracle_fwd
            f.restype = ctypes.c_int
            dp = ctypes.POINTER(ctypes.c_double)
            i64 = ctypes.c_int64
            f.argtypes = [dp, dp, dp, i64, i64, i64, i64, i64, ctypes.c_double, ctypes.c_int,
                          ctypes.POINTER(ctypes.c_int64), i64, dp, dp, ctypes.c_int]
            _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def attention_fwd(q, k, v, scale: float, causal: bool, rows=None, threads: int | None = None):
    """Exact attention forward in fp64.

    q: [B,H,Nq,d], k and v: [B,H,Nk,d] (anything np.asarray turns into float64 exactly:
    numpy arrays or CPU torch tensors already upcast with .double()).
    rows: None for every row (returns O [B,H,Nq,d], L [B,H,Nq]) or an int64 array of flat
    row ids (b*H + h)*Nq + i (returns O [len(rows), d], L [len(rows)]).
    """
    q = np.ascontiguousarray(np.asarray(q, dtype=np.float64))
    k = np.ascontiguousarray(np.asarray(k, dtype=np.float64))
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float64))
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B,H,N,d]")
    B, H, Nq, d = q.shape
    if k.shape != (B, H, k.shape[2], d) or v.shape != k.shape:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    Nk = k.shape[2]
    if rows is None:
        nrows = B * H * Nq
        o = np.empty((B, H, Nq, d), dtype=np.float64)
        lse = np.empty((B, H, Nq), dtype=np.float64)
        rows_p = None
    else:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows.size
        o = np.empty((nrows, d), dtype=np.float64)
        lse = np.empty((nrows,), dtype=np.float64)
        rows_p = rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    lib = _load()
    dp = ctypes.POINTER(ctypes.c_double)
    rc = lib.attn_oracle_fwd(q.ctypes.data_as(dp), k.ctypes.data_as(dp), v.ctypes.data_as(dp),
                             B, H, Nq, Nk, d, float(scale), int(bool(causal)), rows_p, nrows,
                             o.ctypes.data_as(dp), lse.ctypes.data_as(dp),
                             int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"attn_oracle_fwd failed with status {rc}")
    return o, lse


def attention_bwd(q, k, v, do, scale: float, causal: bool, o=None):
    """Exact gradients of the attention forward in fp64 (numpy, whole score matrix per head).

    For O = softmax(S) V with S = scale * Q K^T (top-left causal mask: key j visible to query
    i iff j <= i) and an upstream gradient dO, the chain rule gives, per (b, h):

        P  = softmax(S) row by row            (exp(S - rowmax) / rowsum)
        dV = P^T dO
        dP = dO V^T
        dS = P * (dP - rowsum(P * dP))        (the softmax Jacobian applied row by row)
        dQ = scale * dS K
        dK = scale * dS^T Q

    These are the gradients the backward kernel of page "flash_attention_2.cu" accumulates
    (its dV, dP, dS = P (dP - D), dQ and dK updates); here they are written out on full
    matrices with no tiling, no recomputation from L and no online recurrence. rowsum(P dP)
    equals rowsum(dO * O) exactly in real arithmetic.

    o: None, or the forward output as the caller stored it ([B,H,Nq,d]). That page's backward
    kernel forms its row term from the stored output, D_i = rowsum(dO_i * O_i); given o, the
    row term is that sum over o (equal to rowsum(P dP) when o is the exact output). A stored
    output rounded to 16 bits then enters D exactly as it enters the kernels.

    q: [B,H,Nq,d], k, v: [B,H,Nk,d], do: [B,H,Nq,d]. Returns dq, dk, dv (fp64).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    if q.ndim != 4 or k.shape[:2] != q.shape[:2] or v.shape != k.shape or do.shape != q.shape \
            or k.shape[3] != q.shape[3]:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape} do{do.shape}")
    if o is not None:
        o = np.asarray(o, dtype=np.float64)
        if o.shape != q.shape:
            raise ValueError(f"o must be shaped like q: {o.shape} vs {q.shape}")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    visible = np.ones((Nq, Nk), dtype=bool)
    if causal:
        visible = np.arange(Nk)[None, :] <= np.arange(Nq)[:, None]
    for b in range(B):
        for h in range(H):
            s = scale * (q[b, h] @ k[b, h].T)
            s = np.where(visible, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            p = e / e.sum(axis=1, keepdims=True)
            dv[b, h] = p.T @ do[b, h]
            dp = do[b, h] @ v[b, h].T
            if o is None:
                D = (p * dp).sum(axis=1, keepdims=True)
            else:
                D = (do[b, h] * o[b, h]).sum(axis=1, keepdims=True)
            ds = p * (dp - D)
            dq[b, h] = scale * (ds @ k[b, h])
            dk[b, h] = scale * (ds.T @ q[b, h])
    return dq, dk, dv


def attention_fwd_varlen(q, k, v, cu_q, cu_k, scale: float, causal: bool,
                         threads: int | None = None):
    """Exact attention forward over a packed batch of sequences of different lengths (fp64).

    Page "Meta's xFormers has Attention kernel written in CUTLASS" (the grouped-GEMM
    discussion) asks for fixed and variable sequence lengths in one kernel. Read plainly:
    each sequence of the batch is its own attention problem, and sequences never see each
    other's keys.

    q: [H, Tq, d]; k, v: [H, Tk, d]; every head's rows hold the sequences back to back.
    cu_q, cu_k: B+1 offsets, nondecreasing, from 0 to Tq (resp. Tk). Sequence b owns query
    rows cu_q[b]:cu_q[b+1] and key rows cu_k[b]:cu_k[b+1]. The causal mask uses the
    sequence's own positions (key j visible to query i iff j <= i, both counted from the
    sequence start). A sequence with queries but no keys has an empty softmax sum: its
    rows get O = 0 and L = ln 0 = -inf.

    Each sequence goes through attention_fwd on its own slices. Returns O [H, Tq, d] and
    L [H, Tq].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    if q.ndim != 3 or k.ndim != 3 or v.shape != k.shape or k.shape[0] != q.shape[0] \
            or k.shape[2] != q.shape[2]:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    H, Tq, d = q.shape
    Tk = k.shape[1]
    for name, cu, total in (("cu_q", cu_q, Tq), ("cu_k", cu_k, Tk)):
        if cu.ndim != 1 or cu.size < 2 or cu[0] != 0 or cu[-1] != total or np.any(np.diff(cu) < 0):
            raise ValueError(f"{name} must run from 0 to {total} without decreasing")
    if cu_q.size != cu_k.size:
        raise ValueError("cu_q and cu_k must describe the same number of sequences")
    o = np.zeros((H, Tq, d), dtype=np.float64)
    lse = np.full((H, Tq), -np.inf, dtype=np.float64)
    for b in range(cu_q.size - 1):
        qs, qe, ks, ke = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if qe == qs or ke == ks:
            continue  # no rows, or rows with an empty softmax (O = 0, L = -inf as set)
        ob, lb = attention_fwd(q[None, :, qs:qe], k[None, :, ks:ke], v[None, :, ks:ke],
                               scale, causal, threads=threads)
        o[:, qs:qe] = ob[0]
        lse[:, qs:qe] = lb[0]
    return o, lse
