"""GPU parity of the backward pass (fa_bwd through the C ABI) against the fp64 oracle.

Flow: the forward on the GPU gives O and L; fa_bwd takes them with an upstream gradient dO;
oracle.attention_bwd computes the exact gradients from q, k, v and dO, with the row term
D = rowsum(dO * O) formed from the same stored O the kernels read (the backward kernel of page
"flash_attention_2.cu" takes D from the stored output; for 16-bit inputs that output is
rounded, and the rounding reaches the gradients through D whatever the kernel does).

Tolerance (per gradient tensor, normalised by its largest magnitude): max|d - d_ref| <=
2e-2 * max|d_ref| for fp16/bf16 inputs (measured worst 6.4e-3). The kernels round P and dS to the input type for
the products that consume them and round the results, each a relative error of at most
2^-9 (bf16) per term, and the row term D = rowsum(dO * O) reads the forward's rounded O.
fp32 inputs: max|d - d_ref| <= 1e-4 * max|d_ref|, the forward's fp32 bound (1e-4 on O of
order one) carried to each gradient's own scale. Every step is fp32 with fp32 accumulation;
what the backward takes from the forward (O for D, L for P) carries the forward's errors, at
most a few 1e-6.
A gradient that cancels to (nearly) zero is normalised by a thousandth of the largest single
summand it can have instead (dQ: scale |dO| |V| |K| with row norms; dK: scale |dO| |V| |Q|;
dV: |dO|): rounding errors scale with the summands, not with what is left after they cancel
(one query and one key give dK = 0 exactly, since D = dO . O = dO . V).
"""
import math
import sys

import numpy as np
import pytest
import torch

import exact_attention_58_amd as fa
import oracle
from exact_attention_58_amd.workloads import make_random

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f16": 2e-2, "f32": 1e-4}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.ensure_built()
    fa.lib()


def offset_copy(t, elems):
    """A contiguous device copy of t whose data starts `elems` elements past an aligned
    allocation (so its rows are not 16-byte aligned)."""
    flat = torch.empty(t.numel() + elems, dtype=t.dtype, device="cuda")
    view = flat[elems:].view(t.shape)
    view.copy_(t.cuda())
    return view


def run_case(dt, B, H, Nq, Nk, d, causal, seed, scale=None, heads=None, misalign=0):
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    q = make_random((B, H, Nq, d), dt, seed)
    k = make_random((B, H, Nk, d), dt, seed + 1)
    v = make_random((B, H, Nk, d), dt, seed + 2)
    do = make_random((B, H, Nq, d), dt, seed + 3)
    qd, kd, vd, dod = (offset_copy(t, misalign) for t in (q, k, v, do))
    o, lse = fa.attention(qd, kd, vd, scale=scale, causal=causal)
    if misalign:
        o = offset_copy(o, misalign)
        dq, dk, dv = (offset_copy(torch.zeros_like(t), misalign) for t in (qd, kd, vd))
        fa.fa_bwd(qd, kd, vd, o, lse, dod, dq, dk, dv, torch.empty_like(lse), scale, causal)
    else:
        dq, dk, dv = fa.attention_bwd(qd, kd, vd, o, lse, dod, scale=scale, causal=causal)
    torch.cuda.synchronize()
    dq, dk, dv = (t.double().cpu().numpy() for t in (dq, dk, dv))
    o_host = o.double().cpu().numpy()
    if heads is not None:  # compare a subset of (b, h) slices at large sizes
        sel = lambda t: t.reshape(B * H, *t.shape[2:])[heads][None]
        q, k, v, do = (torch.from_numpy(sel(t.double().numpy())) for t in (q, k, v, do))
        dq, dk, dv, o_host = sel(dq), sel(dk), sel(dv), sel(o_host)
    want = oracle.attention_bwd(q.double(), k.double(), v.double(), do.double(), scale, causal, o=o_host)
    what = f"{dt} B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal} misalign={misalign}"
    rn = lambda t: float(torch.as_tensor(t).double().norm(dim=-1).max())
    term = {"dq": abs(scale) * rn(do) * rn(v) * rn(k), "dk": abs(scale) * rn(do) * rn(v) * rn(q), "dv": rn(do)}
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        assert np.all(np.isfinite(got)), (what, name)
        mag = max(float(np.max(np.abs(ref))), 1e-3 * term[name])
        err = float(np.max(np.abs(got - ref)))
        rel = err / mag if mag > 0 else err
        say(f"  {what} {name}: max|err| {err:.3e}  max|ref| {mag:.3e}  normalised {rel:.3e}")
        assert rel <= TOL[dt] or err == 0.0, (what, name, rel)


SHAPES = [(1, 1), (17, 63), (64, 65), (129, 127), (200, 1000), (300, 300), (256, 256)]


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [32, 64, 96, 128])
@pytest.mark.parametrize("Nq,Nk", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_shapes(dt, d, Nq, Nk, causal):
    run_case(dt, 1, 2, Nq, Nk, d, causal, seed=1000 + Nq + 7 * Nk + d)


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [1, 5, 36, 40, 100, 127])
@pytest.mark.parametrize("Nq,Nk", [(17, 63), (129, 127), (200, 333)])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_ragged_head_dims(dt, d, Nq, Nk, causal):
    """Head dims off the 16-byte row (masked loads and stores on every tensor)."""
    run_case(dt, 1, 2, Nq, Nk, d, causal, seed=3000 + Nq + 7 * Nk + d)


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_unaligned_buffers(dt, causal):
    """Every buffer one element past 16-byte alignment (the element-wise load path)."""
    run_case(dt, 2, 2, 150, 170, 64, causal, seed=4000 + causal, misalign=1)


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_bwd_batch_heads_and_scales(dt):
    run_case(dt, 2, 3, 150, 190, 64, False, seed=77, scale=0.05)
    run_case(dt, 2, 3, 150, 190, 64, True, seed=78, scale=-0.2)


def test_bwd_causal_more_keys_than_queries():
    """Keys past the last query get no gradient (top-left causal)."""
    run_case("bf16", 1, 1, 100, 300, 64, True, seed=91)


def test_bwd_full_size_heads():
    """bf16 d=128 at the benchmark's sequence length (two heads checked against the oracle)."""
    run_case("bf16", 1, 4, 4096, 4096, 128, False, seed=5, heads=[0, 3])
    run_case("bf16", 1, 4, 4096, 4096, 128, True, seed=6, heads=[1, 2])


def test_bwd_full_size_heads_f32():
    """fp32 at the pages' benchmark shape per head (N=4096, d=64) and at d=128, two heads each."""
    run_case("f32", 1, 4, 4096, 4096, 64, False, seed=7, scale=0.125, heads=[0, 3])
    run_case("f32", 1, 2, 4096, 4096, 128, True, seed=8, heads=[0, 1])


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("d", [32, 64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_wide_grids(dt, d, causal):
    """Grids of two or more 256-row workgroups per CU (4 x 32 heads, 1000 queries, 1100 keys:
    512 and 640 of them on 256 CUs) take the 8-wave dQ and (d <= 96) dK/dV workgroups, a single
    head the 4-wave ones. Two heads against the oracle, and every sampled head's gradients
    equal bit for bit to those of the same head run alone from the same O and L."""
    B, H, Nq, Nk, seed = 4, 32, 1000, 1100, 400 + d + (1 if causal else 0)
    scale = 1.0 / math.sqrt(d)
    q = make_random((B, H, Nq, d), dt, seed)
    k = make_random((B, H, Nk, d), dt, seed + 1)
    v = make_random((B, H, Nk, d), dt, seed + 2)
    do = make_random((B, H, Nq, d), dt, seed + 3)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = fa.attention(qd, kd, vd, scale=scale, causal=causal)
    dq, dk, dv = fa.attention_bwd(qd, kd, vd, o, lse, dod, scale=scale, causal=causal)
    torch.cuda.synchronize()
    heads = [0, 77, B * H - 1]
    flat = lambda t: t.reshape(B * H, *t.shape[2:])
    for h in heads:
        one = [flat(t)[h][None, None].contiguous() for t in (qd, kd, vd, o, lse, dod)]
        g1 = [torch.full_like(t, float("nan")) for t in one[:3]]
        fa.fa_bwd(*one, *g1, torch.empty_like(one[4]), scale, causal)
        torch.cuda.synchronize()
        for name, wide, alone in zip(("dq", "dk", "dv"), (dq, dk, dv), g1):
            assert torch.equal(flat(wide)[h], alone[0, 0]), (dt, d, causal, h, name)
    sel = lambda t: t.reshape(B * H, *t.shape[2:])[heads[:2]][None]
    qs, ks, vs, dos = (torch.from_numpy(sel(t.double().numpy())) for t in (q, k, v, do))
    want = oracle.attention_bwd(qs, ks, vs, dos, scale, causal, o=sel(o.double().cpu().numpy()))
    rn = lambda t: float(torch.as_tensor(t).double().norm(dim=-1).max())
    term = {"dq": scale * rn(dos) * rn(vs) * rn(ks), "dk": scale * rn(dos) * rn(vs) * rn(qs), "dv": rn(dos)}
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        got = sel(got.double().cpu().numpy())
        mag = max(float(np.max(np.abs(ref))), 1e-3 * term[name])
        err = float(np.max(np.abs(got - ref)))
        say(f"  wide {dt} d={d} causal={causal} {name}: normalised {err / mag:.3e}")
        assert err / mag <= TOL[dt], (dt, d, causal, name, err / mag)
