"""GPU checks of the tile-configuration entry points: every kernel a problem admits (forced
through fa_fwd_config) against the fp64 oracle on the same inputs, and fa_tune_fwd's record
steering later fa_fwd calls.

Tolerances as for the forward: O max-abs <= 1e-4 (fp32) and <= 2e-2 (fp16/bf16), L <= 1e-3.
The kernels are deterministic (no atomics), so "fa_fwd launched configuration X" is checked
as bit-equality with fa_fwd_config(X) on the same inputs.
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
ALL = [{"Br": 256, "Bc": 64, "waves": 8}, {"Br": 256, "Bc": 128, "waves": 8}, {"Br": 128, "Bc": 64, "waves": 4},
       {"Br": 64, "Bc": 64, "waves": 4}, {"Br": 128, "Bc": 32, "waves": 4},
       {"Br": 128, "Bc": 128, "waves": 4}, {"Br": 64, "Bc": 128, "waves": 4}, {"Br": 32, "Bc": 32, "waves": 4}]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.ensure_built()
    fa.lib()
    fa.fa_tune_clear()
    yield
    fa.fa_tune_clear()


def admitted(dt, d, causal):
    """The configurations fa_fwd_config accepts for contiguous (16-byte aligned) tensors."""
    dpad = (d + 31) // 32 * 32
    if dt == "f32":
        bc = 32 if dpad > 96 else 64
        split = [] if dpad > 96 else [{"Br": 64, "Bc": bc, "waves": 4}, {"Br": 32, "Bc": 32, "waves": 4}]
        # 128-key tiles for 128-row workgroups up to d = 64 (16-byte rows: d % 4 == 0)
        bc128 = 128 if dpad <= 64 and d % 4 == 0 else bc
        return [{"Br": 128, "Bc": bc128, "waves": 4}] + split
    bc = 32 if dpad > 224 else 128 if dpad <= 32 else 64
    out = [{"Br": 128, "Bc": bc, "waves": 4}]
    if d % 8 == 0 and dpad <= 128:
        out.append({"Br": 256, "Bc": 128 if dpad <= 64 else 64, "waves": 8})
    if dpad <= 128:
        out.append({"Br": 64, "Bc": bc, "waves": 4})
    return out


def inputs(dt, B, H, Nq, Nk, d, seed):
    q = make_random((B, H, Nq, d), dt, seed)
    k = make_random((B, H, Nk, d), dt, seed + 1)
    v = make_random((B, H, Nk, d), dt, seed + 2)
    return q, k, v


CASES = [
    ("bf16", 1, 2, 300, 700, 64, False), ("bf16", 1, 2, 300, 700, 64, True),
    ("f16", 2, 2, 257, 513, 128, False), ("f16", 1, 2, 129, 1000, 96, False),
    ("bf16", 1, 1, 200, 200, 200, True), ("bf16", 1, 2, 100, 90, 40, False),
    ("f32", 1, 2, 300, 700, 64, False), ("f32", 1, 1, 100, 300, 128, True),
    ("bf16", 1, 2, 200, 300, 256, False), ("f16", 1, 1, 150, 170, 250, True),
    ("bf16", 1, 2, 300, 700, 32, True), ("f16", 2, 2, 257, 513, 24, False), ("f32", 1, 2, 200, 300, 32, True),
    ("f32", 1, 2, 200, 500, 96, False), ("f32", 1, 2, 150, 400, 37, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_every_admitted_config_matches_oracle(case):
    dt, B, H, Nq, Nk, d, causal = case
    q, k, v = inputs(dt, B, H, Nq, Nk, d, 300 + Nq + d)
    scale = 1.0 / math.sqrt(d)
    o_ref, l_ref = oracle.attention_fwd(q.double(), k.double(), v.double(), scale, causal)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    ok = admitted(dt, d, causal)
    for cfg in ALL:
        o = torch.empty_like(qd)
        lse = torch.empty(qd.shape[:-1], dtype=torch.float32, device="cuda")
        if cfg not in ok:
            with pytest.raises(fa.FaError) as e:
                fa.fa_fwd_config(qd, kd, vd, o, lse, scale, causal, cfg)
            assert e.value.status == fa.FA_EUNSUPPORTED
            continue
        fa.fa_fwd_config(qd, kd, vd, o, lse, scale, causal, cfg)
        torch.cuda.synchronize()
        oe = float(np.max(np.abs(o.double().cpu().numpy() - o_ref)))
        le = float(np.max(np.abs(lse.double().cpu().numpy() - l_ref)))
        say(f"  {case} {cfg}: max|dO| {oe:.3e} max|dL| {le:.3e}")
        assert oe <= TOL_O[dt] and le <= TOL_L, (case, cfg)


@pytest.mark.parametrize("case", [("bf16", 2, 4, 1000, 3001, 64, False), ("f16", 1, 8, 700, 700, 128, True),
                                  ("bf16", 1, 2, 300, 700, 96, False)],
                         ids=lambda c: "-".join(map(str, c)))
def test_tune_record_steers_fa_fwd(case):
    dt, B, H, Nq, Nk, d, causal = case
    q, k, v = (t.cuda() for t in inputs(dt, B, H, Nq, Nk, d, 500 + d))
    scale = 1.0 / math.sqrt(d)
    fa.fa_tune_clear()
    rule = fa.fa_select_config(dt, B, H, Nq, Nk, d, causal, num_cus=torch.cuda.get_device_properties(0).multi_processor_count)
    rule = {k_: rule[k_] for k_ in ("Br", "Bc", "waves")}

    def run(cfg=None):
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")
        if cfg is None:
            fa.fa_fwd(q, k, v, o, lse, scale, causal)
        else:
            fa.fa_fwd_config(q, k, v, o, lse, scale, causal, cfg)
        torch.cuda.synchronize()
        return o, lse

    o0, l0 = run()
    o_r, l_r = run(rule)
    assert torch.equal(o0, o_r) and torch.equal(l0, l_r)  # untuned: the built-in choice
    ot = torch.empty_like(q)
    lt = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")
    best = fa.fa_tune_fwd(q, k, v, ot, lt, scale, causal, reps=3)
    say(f"  {case}: built-in {rule}, tuned {best}")
    assert {k_: best[k_] for k_ in ("Br", "Bc", "waves")} in admitted(dt, d, causal)
    assert best["occ"] in ((0, 1) if best["waves"] == 4 else (0,))
    assert best["group"] in ((0, 16, 32, 64, 128) if causal and B * H % 8 == 0 else (0,))
    o1, l1 = run()
    o_b, l_b = run(best)
    assert torch.equal(o1, o_b) and torch.equal(l1, l_b)    # tuned: the recorded choice
    assert torch.equal(ot, o_b) and torch.equal(lt, l_b)    # the tuning call's own output
    fa.fa_tune_clear()
    o2, l2 = run()
    assert torch.equal(o2, o_r) and torch.equal(l2, l_r)    # cleared: built-in again


KNOB_CASES = [
    ("bf16", 1, 8, 1024, 1024, 128, True),   # 8 pairs: one per XCD, grouped causal order
    ("f16", 2, 8, 1000, 1000, 64, True),     # 16 pairs, ragged last tile
    ("f32", 1, 8, 700, 700, 64, True),
    ("f16", 2, 4, 600, 900, 96, False),      # non-causal: group has no effect
]
KNOBS = [dict(occ=1), dict(occ=2), dict(group=8), dict(group=16), dict(group=128), dict(group=1024),
         dict(occ=1, group=32)]


@pytest.mark.parametrize("case", KNOB_CASES, ids=lambda c: "-".join(map(str, c)))
def test_knobs_leave_results_bit_identical(case):
    """The occupancy cap and the causal dispatch group move workgroups, never arithmetic:
    every admitted configuration with every knob setting equals its knob-free result bit for
    bit, and the knob-free result matches the oracle. Outputs start as NaN, so a tile that no
    workgroup writes under some group size fails."""
    dt, B, H, Nq, Nk, d, causal = case
    q, k, v = inputs(dt, B, H, Nq, Nk, d, 700 + Nq + d)
    scale = 1.0 / math.sqrt(d)
    o_ref, l_ref = oracle.attention_fwd(q.double(), k.double(), v.double(), scale, causal)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()

    def run(cfg):
        o = torch.full_like(qd, float("nan"))
        lse = torch.full(qd.shape[:-1], float("nan"), dtype=torch.float32, device="cuda")
        fa.fa_fwd_config(qd, kd, vd, o, lse, scale, causal, cfg)
        torch.cuda.synchronize()
        return o, lse

    for cfg in admitted(dt, d, causal):
        o0, l0 = run(cfg)
        oe = float(np.max(np.abs(o0.double().cpu().numpy() - o_ref)))
        le = float(np.max(np.abs(l0.double().cpu().numpy() - l_ref)))
        say(f"  {case} {cfg}: max|dO| {oe:.3e} max|dL| {le:.3e}")
        assert oe <= TOL_O[dt] and le <= TOL_L, (case, cfg)
        for knob in KNOBS:
            o1, l1 = run({**cfg, **knob})
            assert torch.equal(o0, o1) and torch.equal(l0, l1), (case, cfg, knob)
