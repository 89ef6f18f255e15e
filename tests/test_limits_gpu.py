"""GPU checks at the largest sizes the forward accepts: one head whose key or query count
times d sits just under 2^31 (the int32 row-index limit inside a head), and a grid of 65536
batch-heads.

Inputs are seeded and synthetic, drawn on the device (a host copy of several GiB of keys
would add nothing). Expected values come from closed forms that hold at any size and from
the fp64 oracle on sampled rows:
- identical key rows give every visible key the same weight, so O_i is the mean of the value
  rows and L_i = scale*q_i.k + ln(Nk); the value rows follow an integer pattern whose mean
  is computed exactly on the host;
- value rows of ones give O = 1 for any weights;
- with few keys, a sample of query rows (the last rows included) goes through the oracle.
Tolerances as for the forward: O <= 2e-2 (fp16/bf16), <= 1e-4 (fp32); L <= 1e-3.
"""
import math
import sys

import numpy as np
import pytest
import torch

import exact_attention_58_amd as fa
import oracle

pytestmark = pytest.mark.gpu

INT32_MAX = 2 ** 31 - 1
DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
TOL_O = {"f32": 1e-4, "f16": 2e-2, "bf16": 2e-2}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.ensure_built()
    fa.lib()


def randn(shape, dt, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(DT[dt])


def pattern_rows(n, d, dt, col_offset):
    """V[j, c] = ((7j + 3c) mod 13 - 6) / 8 (+ (c mod 5) / 4 with col_offset), exact in every
    dtype, and its column means. The first term sums to zero over every 13 rows, so the
    running sums stay small; the optional column term gives each column its own mean."""
    j = torch.arange(n, device="cuda", dtype=torch.int32)[:, None]
    c = torch.arange(d, device="cuda", dtype=torch.int32)[None, :]
    v = ((7 * j + 3 * c) % 13 - 6).to(torch.float32) / 8
    if col_offset:
        v = v + (c % 5).to(torch.float32) / 4
    v = v.to(DT[dt])
    # (7j + 3c) mod 13 has period 13 in j
    full, rest = divmod(n, 13)
    mean = np.zeros(d)
    for cc in range(d):
        vals = [((7 * jj + 3 * cc) % 13 - 6) / 8 for jj in range(13)]
        mean[cc] = (full * sum(vals) + sum(vals[:rest])) / n + ((cc % 5) / 4 if col_offset else 0.0)
    return v, mean


CONFIGS = {"built-in": None, "ping-pong": {"Br": 256, "Bc": 64, "waves": 8}}


@pytest.mark.parametrize("cfg", list(CONFIGS))
def test_longest_key_sequence_bf16(cfg):
    """Nk * d just under 2^31 (Nk = 2^24 - 1, d = 128): identical keys, patterned values."""
    d, Nk, Nq = 128, INT32_MAX // 128, 256
    say(f"  Nk={Nk} d={d} Nq={Nq} config={cfg}")
    q = randn((1, 1, Nq, d), "bf16", 11)
    krow = randn((1, 1, 1, d), "bf16", 12)
    k = krow.expand(1, 1, Nk, d).contiguous()
    v, vmean = pattern_rows(Nk, d, "bf16", True)
    v = v.view(1, 1, Nk, d)
    scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((1, 1, Nq), dtype=torch.float32, device="cuda")
    if CONFIGS[cfg] is None:
        fa.fa_fwd(q, k, v, o, lse, scale, False)
    else:
        fa.fa_fwd_config(q, k, v, o, lse, scale, False, CONFIGS[cfg])
    torch.cuda.synchronize()
    qh = q[0, 0].double().cpu().numpy()
    kh = krow[0, 0, 0].double().cpu().numpy()
    l_want = scale * (qh @ kh) + math.log(Nk)
    l_err = float(np.max(np.abs(lse[0, 0].double().cpu().numpy() - l_want)))
    o_err = float(np.max(np.abs(o[0, 0].double().cpu().numpy() - vmean[None, :])))
    say(f"    max|dO| {o_err:.3e}  max|dL| {l_err:.3e}")
    assert o_err <= TOL_O["bf16"] and l_err <= 1e-3
    del k, v


def test_longest_key_sequence_random_keys_unit_values():
    """Random keys over Nk = 2^24 - 1, value rows of ones: O = 1 for every row, causal too."""
    d, Nk, Nq = 128, INT32_MAX // 128, 256
    q = randn((1, 1, Nq, d), "bf16", 21)
    k = randn((1, 1, Nk, d), "bf16", 22)
    v = torch.ones((1, 1, Nk, d), dtype=torch.bfloat16, device="cuda")
    for causal in (False, True):
        o, lse = fa.attention(q, k, v, causal=causal)
        torch.cuda.synchronize()
        err = float((o.double() - 1.0).abs().max())
        say(f"  causal={causal}: max|O - 1| {err:.3e}")
        assert err <= TOL_O["bf16"] and bool(torch.isfinite(lse).all())
    del k, v


def test_longest_key_sequence_f32():
    """fp32 at Nk * d just under 2^31 (Nk = 2^25 - 1, d = 64): identical keys."""
    d, Nk, Nq = 64, INT32_MAX // 64, 128
    q = randn((1, 1, Nq, d), "f32", 31)
    krow = randn((1, 1, 1, d), "f32", 32)
    k = krow.expand(1, 1, Nk, d).contiguous()
    v, vmean = pattern_rows(Nk, d, "f32", False)
    v = v.view(1, 1, Nk, d)
    o, lse = fa.attention(q, k, v, scale=0.125)
    torch.cuda.synchronize()
    l_want = 0.125 * (q[0, 0].double().cpu().numpy() @ krow[0, 0, 0].double().cpu().numpy()) + math.log(Nk)
    l_err = float(np.max(np.abs(lse[0, 0].double().cpu().numpy() - l_want)))
    o_err = float(np.max(np.abs(o[0, 0].double().cpu().numpy() - vmean[None, :])))
    say(f"  max|dO| {o_err:.3e}  max|dL| {l_err:.3e}")
    assert o_err <= TOL_O["f32"] and l_err <= 1e-3
    del k, v


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_longest_query_sequence(dt):
    """Nq * d just under 2^31 (d = 128 for bf16, 64 for fp32) with 64 keys; sampled rows,
    the last rows of the index range included, against the oracle (causal and not)."""
    d = 128 if dt == "bf16" else 64
    Nq, Nk = INT32_MAX // d, 64
    q = randn((1, 1, Nq, d), dt, 41)
    k = randn((1, 1, Nk, d), dt, 42)
    v = randn((1, 1, Nk, d), dt, 43)
    scale = 1.0 / math.sqrt(d)
    kh, vh = k.double().cpu().numpy(), v.double().cpu().numpy()
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 62, 63, 64, Nq // 2, Nq - 2, Nq - 1],
                                     rng.integers(0, Nq, 120)]))
    late = rows[rows >= Nk - 1]
    for causal in (False, True):
        o, lse = fa.attention(q, k, v, scale=scale, causal=causal)
        torch.cuda.synchronize()
        idx = torch.from_numpy(rows).cuda()
        og = o[0, 0].index_select(0, idx).double().cpu().numpy()
        lg = lse[0, 0].index_select(0, idx).double().cpu().numpy()
        qs = q[0, 0].index_select(0, idx).double().cpu().numpy()[None, None]
        # non-causal rows are independent of their position; causal rows at or past Nk - 1
        # see every key, and the first Nk rows are checked as the head of the sequence
        o_ref, l_ref = oracle.attention_fwd(qs, kh, vh, scale, False)
        sel = np.ones(len(rows), bool) if not causal else rows >= Nk - 1
        o_err = float(np.max(np.abs(og[sel] - o_ref[0, 0][sel])))
        l_err = float(np.max(np.abs(lg[sel] - l_ref[0, 0][sel])))
        if causal:
            head = q[:, :, :Nk].double().cpu().numpy()
            oh, lh = oracle.attention_fwd(head, kh, vh, scale, True)
            o_err = max(o_err, float(np.max(np.abs(o[0, 0, :Nk].double().cpu().numpy() - oh[0, 0]))))
            l_err = max(l_err, float(np.max(np.abs(lse[0, 0, :Nk].double().cpu().numpy() - lh[0, 0]))))
        say(f"  {dt} causal={causal}: {len(rows)} rows ({len(late)} past Nk-1), max|dO| {o_err:.3e} max|dL| {l_err:.3e}")
        assert o_err <= TOL_O[dt] and l_err <= 1e-3
        del o, lse


def test_many_batch_heads():
    """B * H = 65536 small heads (grid of 65536 workgroups); 64 sampled heads vs the oracle."""
    B, H, N, d = 128, 512, 16, 32
    q, k, v = (randn((B, H, N, d), "bf16", 50 + i) for i in range(3))
    o, lse = fa.attention(q, k, v, causal=True)
    torch.cuda.synchronize()
    heads = torch.from_numpy(np.random.default_rng(7).choice(B * H, 64, replace=False)).cuda()
    pick = lambda t: t.reshape(B * H, *t.shape[2:]).index_select(0, heads).double().cpu().numpy()[None]
    o_ref, l_ref = oracle.attention_fwd(pick(q), pick(k), pick(v), 1.0 / math.sqrt(d), True)
    o_err = float(np.max(np.abs(pick(o) - o_ref)))
    l_err = float(np.max(np.abs(pick(lse) - l_ref)))
    say(f"  65536 heads: max|dO| {o_err:.3e} max|dL| {l_err:.3e}")
    assert o_err <= TOL_O["bf16"] and l_err <= 1e-3
