"""fa_bwd_noalloc: the backward entry point that allocates nothing (its row-term workspace is
the library's own device array). CPU: its argument checks, including the row limit, run before
any HIP call. GPU: its gradients equal fa_bwd's, bit for bit, on two calls in a row, the second
smaller, with outputs pre-filled with NaN."""
import ctypes

import pytest
import torch

import exact_attention_58_amd as fa
from exact_attention_58_amd.workloads import make_random

P = 4096  # non-null aligned fake pointer: only passed with arguments the checks reject
MAX_ROWS = 1 << 20


@pytest.fixture(scope="module")
def L():
    fa.ensure_built()
    return fa.lib()


def call_noalloc(L, q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, H=1, Nq=8, Nk=8, d=64,
                 scale=0.125, causal=0, dtype=2):
    return L.fa_bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, B, H, Nq, Nk, d, ctypes.c_float(scale),
                            causal, dtype, None)


@pytest.mark.parametrize("kw", [
    dict(q=None), dict(lse=None), dict(do=None), dict(dq=None), dict(dv=None), dict(B=0), dict(d=0),
    dict(dtype=3), dict(scale=float("nan")), dict(dv=P + 1), dict(lse=P + 2),
])
def test_noalloc_invalid_arguments(L, kw):
    assert call_noalloc(L, **kw) == fa.FA_EINVAL


@pytest.mark.parametrize("kw", [
    dict(d=136),
    dict(B=1, H=1, Nq=MAX_ROWS + 1),          # one query row past the workspace
    dict(B=4, H=16, Nq=MAX_ROWS // 64 + 1),
])
def test_noalloc_unsupported(L, kw):
    assert call_noalloc(L, **kw) == fa.FA_EUNSUPPORTED


def _case(B, H, Nq, Nk, d, dt, causal, seed):
    dev = torch.device("cuda:0")
    q = make_random((B, H, Nq, d), dt, seed).to(dev)
    k = make_random((B, H, Nk, d), dt, seed + 1).to(dev)
    v = make_random((B, H, Nk, d), dt, seed + 2).to(dev)
    do = make_random((B, H, Nq, d), dt, seed + 3).to(dev)
    o, lse = fa.attention(q, k, v, causal=causal)
    return q, k, v, o, lse, do


def _grads(fn, q, k, v, o, lse, do, causal):
    dq = torch.full_like(q, float("nan"))
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    fn(dq, dk, dv)
    torch.cuda.synchronize()
    return dq, dk, dv


@pytest.mark.gpu
@pytest.mark.parametrize("dt,d,causal", [("bf16", 64, False), ("f16", 128, True), ("f32", 96, True)])
def test_noalloc_matches_fa_bwd_on_two_calls(dt, d, causal):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.ensure_built()
    fa.lib()
    scale = d ** -0.5
    # the second call is smaller: the shared workspace keeps the first call's row terms past
    # the second call's rows, which must not leak into its gradients
    for i, (B, H, Nq, Nk) in enumerate(((2, 4, 1000, 900), (1, 2, 300, 200))):
        print(f"fa_bwd_noalloc call {i}: B={B} H={H} Nq={Nq} Nk={Nk} d={d} {dt} causal={causal}", flush=True)
        q, k, v, o, lse, do = _case(B, H, Nq, Nk, d, dt, causal, 500 + 10 * i + d)
        ref = _grads(lambda dq, dk, dv: fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv,
                                                  torch.empty_like(lse), scale, causal), q, k, v, o, lse, do, causal)
        got = _grads(lambda dq, dk, dv: fa.fa_bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, scale, causal),
                     q, k, v, o, lse, do, causal)
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.isfinite(a.float()).all(), name
            assert torch.equal(a, b), (i, name, float((a.float() - b.float()).abs().max()))
