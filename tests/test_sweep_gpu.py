"""GPU parity on a seeded random sweep of problems, forward and backward, against the fp64 oracle.

The cases are drawn once from a fixed seed: dtype, head dim (any 1..256 for 16-bit inputs,
1..128 for fp32, plus the tile-boundary dims), batch and heads, query and key lengths, the
causal flag, the scale (negative and off 1/sqrt(d) included) and buffers one element off
16-byte alignment. The small cases compare every row and, for d <= 128, the gradients; the
large cases (grids that reach the ping-pong kernel and the fp32 128-key tiles) compare a
sample of flat rows the oracle computes one by one; the medium cases sit between the two
(grids near one workgroup per CU up to several per CU), with gradients where the oracle's
full score matrices stay small.

Tolerances as elsewhere: O <= 1e-4 (fp32) / 2e-2 (fp16, bf16) max-abs, L <= 1e-3; gradients
max|err| <= 1e-4 (fp32) / 2e-2 (16-bit) of the larger of max|ref| and a thousandth of the
gradient's largest possible summand.
"""
import math
import random
import sys

import numpy as np
import pytest
import torch

import exact_attention_58_amd as fa
import oracle
from exact_attention_58_amd.workloads import DTYPES, make_random

pytestmark = pytest.mark.gpu

TOL_O = {"f32": 1e-4, "f16": 2e-2, "bf16": 2e-2}
TOL_L = 1e-3
TOL_G = {"f32": 1e-4, "f16": 2e-2, "bf16": 2e-2}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.ensure_built()
    fa.lib()


def draw_cases(seed, n, large, mid=False):
    rng = random.Random(seed)
    out = []
    for i in range(n):
        dt = rng.choice(["f32", "f16", "bf16", "bf16"])
        if mid:
            d = rng.choice([16, 32, 40, 48, 64, 80, 96, 112, 128] if dt != "f32" else [32, 64, 96, 128])
            B, H = rng.randint(1, 16), rng.randint(1, 32)
            Nq, Nk = rng.randint(128, 1536), rng.randint(128, 1536)
        elif large:
            d = rng.choice([40, 48, 64, 96, 128] if dt != "f32" else [32, 40, 64])
            B, H = rng.randint(1, 4), rng.randint(8, 32)
            Nq, Nk = rng.randint(1024, 5000), rng.randint(1024, 5000)
        else:
            dmax = 128 if dt == "f32" else 256
            dims = [32, 40, 48, 64, 96, 128] + ([160, 256] if dt != "f32" else [])
            d = rng.choice([rng.randint(1, dmax), rng.choice(dims)])
            B, H = rng.randint(1, 3), rng.randint(1, 6)
            hi = 3000 if rng.random() < 0.3 else 700
            Nq, Nk = rng.randint(1, hi), rng.randint(1, hi)
        causal = rng.random() < 0.5
        misalign = rng.random() < 0.2
        scale = rng.choice([1.0, 1.0, 0.5, 2.0, -1.0]) / math.sqrt(d)
        out.append((dt, B, H, Nq, Nk, d, causal, misalign, round(scale, 6), 7000 + 131 * i + (1 if large else 2 if mid else 0)))
    return out


SMALL = draw_cases(20261203, 60, large=False)
LARGE = draw_cases(20261204, 24, large=True)
MID = draw_cases(20261205, 20, large=False, mid=True)


def on_device(t, misalign):
    """A device copy of t, one element past an aligned allocation when misalign is set."""
    if not misalign:
        return t.cuda()
    flat = torch.empty(t.numel() + 1, dtype=t.dtype, device="cuda")
    view = flat[1:].view(t.shape)
    view.copy_(t.cuda())
    return view


def check_case(case, sample_rows):
    dt, B, H, Nq, Nk, d, causal, misalign, scale, seed = case
    q = make_random((B, H, Nq, d), dt, seed)
    k = make_random((B, H, Nk, d), dt, seed + 1)
    v = make_random((B, H, Nk, d), dt, seed + 2)
    qd, kd, vd = (on_device(t, misalign) for t in (q, k, v))
    o = on_device(torch.full(q.shape, float("nan"), dtype=DTYPES[dt]), misalign)
    lse = torch.full(q.shape[:-1], float("nan"), dtype=torch.float32, device="cuda")
    fa.fa_fwd(qd, kd, vd, o, lse, scale, causal)
    torch.cuda.synchronize()
    nr = B * H * Nq
    rows = None
    if sample_rows:
        rng = np.random.default_rng(seed)
        rows = np.unique(np.concatenate([rng.choice(nr, size=min(nr, 96), replace=False), [0, nr - 1]])).astype(np.int64)
    o_ref, l_ref = oracle.attention_fwd(q.double(), k.double(), v.double(), scale, causal, rows=rows)
    got_o, got_l = o.double().cpu().numpy(), lse.double().cpu().numpy()
    if rows is not None:
        got_o, got_l = got_o.reshape(nr, d)[rows], got_l.reshape(nr)[rows]
    what = f"{case}"
    assert np.all(np.isfinite(got_o)), what
    oe = float(np.max(np.abs(got_o - o_ref)))
    # rows that see no key have L = -inf on both sides
    assert np.array_equal(np.isneginf(got_l), np.isneginf(l_ref)), what
    fin = np.isfinite(l_ref)
    le = float(np.max(np.abs(got_l[fin] - l_ref[fin]))) if fin.any() else 0.0
    say(f"  {what}: max|dO| {oe:.2e} max|dL| {le:.2e}")
    assert oe <= TOL_O[dt] and le <= TOL_L, (what, oe, le)
    return q, k, v, qd, kd, vd, o, lse


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "-".join(map(str, c[:8])))
def test_sweep_small(case):
    dt, B, H, Nq, Nk, d, causal, misalign, scale, seed = case
    q, k, v, qd, kd, vd, o, lse = check_case(case, sample_rows=False)
    if d > 128:
        return
    do = make_random((B, H, Nq, d), dt, seed + 3)
    dod = on_device(do, misalign)
    dq, dk, dv = (on_device(torch.zeros_like(t), misalign) for t in (q, k, v))
    fa.fa_bwd(qd, kd, vd, o, lse, dod, dq, dk, dv, torch.empty_like(lse), scale, causal)
    torch.cuda.synchronize()
    want = oracle.attention_bwd(q.double(), k.double(), v.double(), do.double(), scale, causal,
                                o=o.double().cpu().numpy())
    rn = lambda t: float(torch.as_tensor(t).double().norm(dim=-1).max())
    term = {"dq": abs(scale) * rn(do) * rn(v) * rn(k), "dk": abs(scale) * rn(do) * rn(v) * rn(q), "dv": rn(do)}
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        got = got.double().cpu().numpy()
        assert np.all(np.isfinite(got)), (case, name)
        mag = max(float(np.max(np.abs(ref))), 1e-3 * term[name])
        err = float(np.max(np.abs(got - ref)))
        assert err == 0.0 or err / mag <= TOL_G[dt], (case, name, err / mag)


@pytest.mark.parametrize("case", LARGE, ids=lambda c: "-".join(map(str, c[:8])))
def test_sweep_large(case):
    check_case(case, sample_rows=True)


@pytest.mark.parametrize("case", MID, ids=lambda c: "-".join(map(str, c[:8])))
def test_sweep_medium(case):
    """Medium grids (B up to 16, H up to 32, 128-1536 rows and keys): the key split near one
    workgroup per CU, the 4-wave kernel at three waves per SIMD, and the 8-wave backward
    workgroups. Forward on sampled rows when large; gradients in full up to 2^26 scores."""
    dt, B, H, Nq, Nk, d, causal, misalign, scale, seed = case
    big = B * H * Nq * Nk * d > 2 ** 31
    q, k, v, qd, kd, vd, o, lse = check_case(case, sample_rows=big)
    if B * H * Nq * Nk > 2 ** 26:
        return
    do = make_random((B, H, Nq, d), dt, seed + 3)
    dod = on_device(do, misalign)
    dq, dk, dv = (on_device(torch.zeros_like(t), misalign) for t in (q, k, v))
    fa.fa_bwd(qd, kd, vd, o, lse, dod, dq, dk, dv, torch.empty_like(lse), scale, causal)
    torch.cuda.synchronize()
    want = oracle.attention_bwd(q.double(), k.double(), v.double(), do.double(), scale, causal,
                                o=o.double().cpu().numpy())
    rn = lambda t: float(torch.as_tensor(t).double().norm(dim=-1).max())
    term = {"dq": abs(scale) * rn(do) * rn(v) * rn(k), "dk": abs(scale) * rn(do) * rn(v) * rn(q), "dv": rn(do)}
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        got = got.double().cpu().numpy()
        assert np.all(np.isfinite(got)), (case, name)
        mag = max(float(np.max(np.abs(ref))), 1e-3 * term[name])
        err = float(np.max(np.abs(got - ref)))
        assert err == 0.0 or err / mag <= TOL_G[dt], (case, name, err / mag)
