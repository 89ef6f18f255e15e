"""Pins for the fp64 CPU oracle (runs on the CPU, no GPU).

The oracle is checked against things other than itself:
  * hand-derived worked examples (tests/golden/hand_worked.json),
  * a 50-digit decimal brute force written with a different formulation
    (weights as 1 / sum_k exp(s_k - s_j), L as ln(sum exp(s)) without a max shift),
  * library routines: torch's fp64 CPU scaled_dot_product_attention for O and
    scipy.special.logsumexp for L,
  * closed forms and invariants that follow from the definition of softmax attention
    (page "flash_attention_2.cu", forward kernel; causal guard keeps the diagonal).
"""
import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest
import scipy.special
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def rng(seed):
    return np.random.default_rng(seed)


def _val(x):
    """Parse the golden file's exact values: numbers, 'a/b', 'lnX', 'ln(a/b)', '-lnX'."""
    if isinstance(x, (int, float)):
        return float(x)
    s = x.replace(" ", "")
    neg = s.startswith("-")
    if neg:
        s = s[1:]
    if s.startswith("ln"):
        arg = s[2:].strip("()")
        val = math.log(_val(arg))
    elif "/" in s:
        a, b = s.split("/")
        val = float(a) / float(b)
    else:
        val = float(s)
    return -val if neg else val


def _tree(x):
    if isinstance(x, list):
        return [_tree(e) for e in x]
    return _val(x)


# ---------------------------------------------------------------- worked examples

def test_hand_worked_examples():
    data = json.load(open(os.path.join(HERE, "golden", "hand_worked.json")))
    assert len(data["cases"]) >= 5
    for case in data["cases"]:
        q, k, v = (np.array(_tree(case[n]), dtype=np.float64) for n in ("q", "k", "v"))
        o_ref = np.array(_tree(case["o"]))
        l_ref = np.array(_tree(case["lse"]))
        o, lse = oracle.attention_fwd(q, k, v, _val(case["scale"]), case["causal"], threads=2)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-14, err_msg=case["name"])
        np.testing.assert_allclose(lse, l_ref, rtol=0, atol=1e-14, err_msg=case["name"])


# ---------------------------------------------------------------- decimal brute force

getcontext().prec = 50


def decimal_attention(q, k, v, scale, causal):
    """Softmax attention at 50 digits, weight_j = 1 / sum_k exp(s_k - s_j), L = ln(sum_k exp(s_k))."""
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    sc = Decimal(float(scale))
    o = np.zeros((B, H, Nq, d))
    L = np.zeros((B, H, Nq))
    for b in range(B):
        for h in range(H):
            Kd = [[Decimal(float(x)) for x in k[b, h, j]] for j in range(Nk)]
            Vd = [[Decimal(float(x)) for x in v[b, h, j]] for j in range(Nk)]
            for i in range(Nq):
                qi = [Decimal(float(x)) for x in q[b, h, i]]
                keys = [j for j in range(Nk) if (not causal or j <= i)]
                s = {j: sc * sum(qi[c] * Kd[j][c] for c in range(d)) for j in keys}
                for c in range(d):
                    acc = Decimal(0)
                    for j in keys:
                        denom = sum((s[kk] - s[j]).exp() for kk in keys)
                        acc += Vd[j][c] / denom
                    o[b, h, i, c] = float(acc)
                L[b, h, i] = float(sum(s[j].exp() for j in keys).ln())
    return o, L


@pytest.mark.parametrize("Nq", [1, 3, 7])
@pytest.mark.parametrize("Nk", [1, 4, 9])
@pytest.mark.parametrize("d", [1, 2, 5])
@pytest.mark.parametrize("causal", [False, True])
def test_decimal_brute_force(Nq, Nk, d, causal):
    seed = 1000 + 97 * Nq + 13 * Nk + 5 * d + int(causal)
    r = rng(seed)
    B, H = 2, 2
    for scale in (1.0 / math.sqrt(d), 0.7, 0.0, -0.3):
        q = r.standard_normal((B, H, Nq, d))
        k = r.standard_normal((B, H, Nk, d))
        v = r.standard_normal((B, H, Nk, d))
        o, L = oracle.attention_fwd(q, k, v, scale, causal, threads=3)
        o_ref, L_ref = decimal_attention(q, k, v, scale, causal)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(L, L_ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_decimal_brute_force_large_magnitude(causal):
    """Scores of several hundred: exp overflows fp64 without the max shift."""
    r = rng(77 + causal)
    q = 30 * r.standard_normal((1, 2, 5, 3))
    k = 30 * r.standard_normal((1, 2, 6, 3))
    v = r.standard_normal((1, 2, 6, 3))
    o, L = oracle.attention_fwd(q, k, v, 1.0, causal, threads=2)
    assert np.abs(L).max() > 500
    o_ref, L_ref = decimal_attention(q, k, v, 1.0, causal)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, L_ref, rtol=1e-14, atol=0)


# ---------------------------------------------------------------- library routines

def _mask(Nq, Nk, causal):
    if not causal:
        return np.ones((Nq, Nk), dtype=bool)
    return np.arange(Nk)[None, :] <= np.arange(Nq)[:, None]


@pytest.mark.parametrize("shape,causal,scale", [
    ((2, 3, 37, 53, 24), False, 0.21),
    ((2, 3, 37, 53, 24), True, 0.21),
    ((1, 2, 64, 40, 7), True, -0.5),
    ((3, 1, 11, 130, 96), False, 1 / math.sqrt(96)),
    ((1, 1, 129, 129, 128), True, 1 / math.sqrt(128)),
])
def test_against_torch_sdpa_and_scipy_logsumexp(shape, causal, scale):
    B, H, Nq, Nk, d = shape
    r = rng(sum(shape) + causal)
    q = r.standard_normal((B, H, Nq, d))
    k = r.standard_normal((B, H, Nk, d))
    v = r.standard_normal((B, H, Nk, d))
    o, L = oracle.attention_fwd(q, k, v, scale, causal, threads=4)
    m = torch.from_numpy(_mask(Nq, Nk, causal))
    o_t = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=m, scale=scale)
    np.testing.assert_allclose(o, o_t.numpy(), rtol=0, atol=1e-12)
    s = scale * np.matmul(q, np.swapaxes(k, -1, -2))
    s = np.where(_mask(Nq, Nk, causal), s, -np.inf)
    L_ref = scipy.special.logsumexp(s, axis=-1)
    np.testing.assert_allclose(L, L_ref, rtol=0, atol=1e-12)


def test_lse_against_fsum():
    """L against an fp64 logsumexp written with math.fsum, row by row."""
    r = rng(5)
    q = r.standard_normal((1, 1, 9, 16))
    k = r.standard_normal((1, 1, 21, 16))
    v = r.standard_normal((1, 1, 21, 16))
    _, L = oracle.attention_fwd(q, k, v, 0.25, True, threads=2)
    for i in range(9):
        s = [0.25 * math.fsum(q[0, 0, i, c] * k[0, 0, j, c] for c in range(16)) for j in range(i + 1)]
        mx = max(s)
        ref = mx + math.log(math.fsum(math.exp(x - mx) for x in s))
        assert abs(L[0, 0, i] - ref) < 1e-13


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("causal", [False, True])
def test_v_ones_gives_ones(causal):
    r = rng(11)
    q = r.standard_normal((2, 2, 13, 8))
    k = r.standard_normal((2, 2, 17, 8))
    o, _ = oracle.attention_fwd(q, k, np.ones((2, 2, 17, 8)), 0.4, causal, threads=2)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_v(causal):
    r = rng(12)
    Nq, Nk, d = 10, 14, 6
    q = r.standard_normal((1, 2, Nq, d))
    kvec = r.standard_normal((1, 2, 1, d))
    k = np.repeat(kvec, Nk, axis=2)
    v = r.standard_normal((1, 2, Nk, d))
    scale = 0.6
    o, L = oracle.attention_fwd(q, k, v, scale, causal, threads=2)
    for h in range(2):
        for i in range(Nq):
            cnt = min(i + 1, Nk) if causal else Nk
            np.testing.assert_allclose(o[0, h, i], v[0, h, :cnt].mean(axis=0), rtol=0, atol=1e-13)
            ref = scale * float(q[0, h, i] @ kvec[0, h, 0]) + math.log(cnt)
            assert abs(L[0, h, i] - ref) < 1e-12


def test_causal_row0_is_v0():
    r = rng(13)
    q = r.standard_normal((2, 3, 5, 4))
    k = r.standard_normal((2, 3, 7, 4))
    v = r.standard_normal((2, 3, 7, 4))
    o, L = oracle.attention_fwd(q, k, v, 0.9, True, threads=2)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(L[:, :, 0], 0.9 * np.einsum("bhc,bhc->bh", q[:, :, 0], k[:, :, 0]),
                               rtol=0, atol=1e-14)


def test_zero_scale_gives_mean_and_log_count():
    r = rng(14)
    q = r.standard_normal((1, 1, 6, 5))
    k = r.standard_normal((1, 1, 9, 5))
    v = r.standard_normal((1, 1, 9, 5))
    o, L = oracle.attention_fwd(q, k, v, 0.0, False, threads=1)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0].mean(0), (6, 5)), rtol=0, atol=1e-14)
    np.testing.assert_allclose(L, math.log(9), rtol=0, atol=1e-14)


def test_single_key_broadcasts_v0():
    r = rng(15)
    q = r.standard_normal((2, 1, 4, 3))
    k = r.standard_normal((2, 1, 1, 3))
    v = r.standard_normal((2, 1, 1, 3))
    for causal in (False, True):
        o, L = oracle.attention_fwd(q, k, v, 1.3, causal, threads=1)
        np.testing.assert_array_equal(o, np.broadcast_to(v, o.shape))
        np.testing.assert_allclose(L, 1.3 * np.einsum("bhic,bhc->bhi", q, k[:, :, 0]), rtol=0, atol=1e-14)


def test_duplicated_keys_add_ln2():
    r = rng(16)
    q = r.standard_normal((1, 2, 8, 12))
    k = r.standard_normal((1, 2, 11, 12))
    v = r.standard_normal((1, 2, 11, 12))
    o1, L1 = oracle.attention_fwd(q, k, v, 0.3, False, threads=2)
    o2, L2 = oracle.attention_fwd(q, np.concatenate([k, k], 2), np.concatenate([v, v], 2), 0.3, False, threads=2)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-14)
    np.testing.assert_allclose(L2, L1 + math.log(2), rtol=0, atol=1e-13)


def test_permuting_keys_and_values_together():
    r = rng(17)
    q = r.standard_normal((1, 1, 9, 7))
    k = r.standard_normal((1, 1, 15, 7))
    v = r.standard_normal((1, 1, 15, 7))
    perm = r.permutation(15)
    o1, L1 = oracle.attention_fwd(q, k, v, 0.5, False, threads=2)
    o2, L2 = oracle.attention_fwd(q, k[:, :, perm], v[:, :, perm], 0.5, False, threads=2)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-14)
    np.testing.assert_allclose(L2, L1, rtol=0, atol=1e-14)


def test_causal_row_equals_prefix_attention():
    r = rng(18)
    q = r.standard_normal((1, 1, 12, 5))
    k = r.standard_normal((1, 1, 12, 5))
    v = r.standard_normal((1, 1, 12, 5))
    o, L = oracle.attention_fwd(q, k, v, 0.8, True, threads=2)
    for i in range(12):
        oi, Li = oracle.attention_fwd(q[:, :, i:i + 1], k[:, :, :i + 1], v[:, :, :i + 1], 0.8, False, threads=1)
        np.testing.assert_allclose(o[0, 0, i], oi[0, 0, 0], rtol=0, atol=1e-15)
        np.testing.assert_allclose(L[0, 0, i], Li[0, 0, 0], rtol=0, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_hard_attention_selects_one_value_row(causal):
    """Orthonormal keys and one-hot queries with a huge scale: row i picks V[pi(i)] exactly.

    A swapped index (query vs key, or q vs k operand) picks a different row.
    """
    d = Nk = 8
    Nq = 8
    r = rng(19 + causal)
    pi = np.array([r.integers(0, i + 1) if causal else r.integers(0, Nk) for i in range(Nq)])
    q = np.zeros((1, 1, Nq, d))
    q[0, 0, np.arange(Nq), pi] = 1.0
    k = np.eye(d)[None, None]
    v = r.standard_normal((1, 1, Nk, d))
    o, L = oracle.attention_fwd(q, k, v, 200.0, causal, threads=1)
    np.testing.assert_allclose(o[0, 0], v[0, 0, pi], rtol=0, atol=1e-60)
    np.testing.assert_allclose(L[0, 0], 200.0, rtol=0, atol=1e-60)


def test_row_subset_matches_full():
    r = rng(20)
    q = r.standard_normal((2, 3, 19, 9))
    k = r.standard_normal((2, 3, 23, 9))
    v = r.standard_normal((2, 3, 23, 9))
    o, L = oracle.attention_fwd(q, k, v, 0.35, True, threads=3)
    rows = np.array([0, 5, 18, 19, 57, 2 * 3 * 19 - 1])
    o_s, L_s = oracle.attention_fwd(q, k, v, 0.35, True, rows=rows, threads=2)
    np.testing.assert_array_equal(o_s, o.reshape(-1, 9)[rows])
    np.testing.assert_array_equal(L_s, L.reshape(-1)[rows])


def test_bad_arguments_raise():
    q = np.zeros((1, 1, 2, 3))
    with pytest.raises(ValueError):
        oracle.attention_fwd(q, np.zeros((1, 1, 2, 4)), np.zeros((1, 1, 2, 4)), 1.0, False)
    with pytest.raises(RuntimeError):
        oracle.attention_fwd(q, q, q, 1.0, False, rows=[7])
