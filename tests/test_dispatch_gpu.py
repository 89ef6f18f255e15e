"""GPU parity for causal grids whose batch-head pairs reach the XCDs in groups with a partial
last group.

Causal grids deal their workgroups to the 8 XCDs so that each XCD runs the heaviest query (or
key) tiles of a group of pairs first. That order is a bijection from workgroup ids to
(pair, tile); a slip in it would leave some rows unwritten or written twice. These shapes
put 5 pairs on every XCD, so the groups (4 pairs, then 1) do not divide the pairs evenly.
Every output row is compared with the fp64 oracle. Outputs start as NaN, so a row no
workgroup writes fails. Tolerances are those of the dense parity tests: O max-abs 1e-4
(fp32) and 2e-2 (fp16/bf16), L 1e-3. Gradients: max|err| <= 2e-2 * max|ref| per tensor.
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

TOL_O = {"f32": 1e-4, "f16": 2e-2, "bf16": 2e-2}
TOL_L = 1e-3


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.ensure_built()
    fa.lib()


# (dtype, B, H, N, d, kernel waves the selector must pick): 40 pairs = 5 per XCD
CASES = [
    ("bf16", 5, 8, 4352, 128, 8),  # ping-pong kernel: 17 query tiles of 256, groups of 4 pairs
    ("bf16", 5, 8, 2048, 64, 4),   # 4-wave kernel (causal, <= 4096 keys): 16 tiles, groups of 4
    ("f16", 5, 8, 2048, 36, 4),    # 4-wave kernel (d % 8 != 0): 16 tiles of 128, groups of 4
    ("f32", 5, 8, 2048, 64, 4),    # fp32 two-way key split: 32 tiles of 64 (dispatch groups of 128)
    ("f32", 5, 8, 256, 64, 4),     # fp32 four-way key split: 8 tiles of 32, one group of 5 pairs
]


@pytest.mark.parametrize("dt,B,H,N,d,waves", CASES)
def test_causal_grouped_dispatch_forward(dt, B, H, N, d, waves):
    cfg = fa.fa_select_config(dt, B, H, N, N, d, True)
    assert cfg["waves"] == waves, cfg
    scale = 1.0 / math.sqrt(d)
    q = make_random((B, H, N, d), dt, 4100 + d)
    k = make_random((B, H, N, d), dt, 4101 + d)
    v = make_random((B, H, N, d), dt, 4102 + d)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=qd.device)
    say(f"causal grouped dispatch: {dt} B={B} H={H} N={N} d={d} cfg={cfg}")
    fa.fa_fwd(qd, kd, vd, o, lse, scale, True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_fwd(q.double(), k.double(), v.double(), scale, True)
    og, lg = o.double().cpu().numpy(), lse.double().cpu().numpy()
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg)), "rows left unwritten"
    o_err, l_err = float(np.max(np.abs(og - o_ref))), float(np.max(np.abs(lg - l_ref)))
    say(f"  max|dO|={o_err:.3e}  max|dL|={l_err:.3e}")
    assert o_err <= TOL_O[dt] and l_err <= TOL_L


def test_causal_grouped_dispatch_backward():
    # dK/dV: 16 key tiles of 128 per pair, dQ: 16 query tiles of 128, groups of 4 pairs
    dt, B, H, N, d = "bf16", 5, 8, 2048, 64
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = (make_random((B, H, N, d), dt, 4200 + i) for i in range(4))
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = fa.attention(qd, kd, vd, scale=scale, causal=True)
    dq, dk, dv = (torch.full_like(qd, float("nan")) for _ in range(3))
    delta = torch.empty((B, H, N), dtype=torch.float32, device=qd.device)
    say(f"causal grouped dispatch backward: {dt} B={B} H={H} N={N} d={d}")
    fa.fa_bwd(qd, kd, vd, o, lse, dod, dq, dk, dv, delta, scale, True)
    torch.cuda.synchronize()
    want = oracle.attention_bwd(q.double(), k.double(), v.double(), do.double(), scale, True)
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        g = got.double().cpu().numpy()
        assert np.all(np.isfinite(g)), (name, "rows left unwritten")
        mag = float(np.max(np.abs(ref)))
        err = float(np.max(np.abs(g - ref)))
        say(f"  {name}: max|err| {err:.3e}  max|ref| {mag:.3e}")
        assert err <= 2e-2 * mag
