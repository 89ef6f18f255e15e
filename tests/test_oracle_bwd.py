"""Pins for the fp64 backward oracle (oracle.attention_bwd), checked against things other than
itself: central finite differences of the forward oracle (a separate C implementation),
torch autograd in fp64 through an explicit softmax, and closed forms of the gradients.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def loss(q, k, v, g, scale, causal):
    """sum(O * G): its gradient w.r.t. q, k, v is the backward pass with dO = G."""
    o, _ = oracle.attention_fwd(q, k, v, scale, causal)
    return float(np.sum(o * g))


def numeric_grad(x, f, h=1e-5):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        old = x[idx]
        x[idx] = old + h
        fp = f()
        x[idx] = old - h
        fm = f()
        x[idx] = old
        g[idx] = (fp - fm) / (2 * h)
    return g


@pytest.mark.parametrize("B,H,Nq,Nk,d", [(1, 1, 3, 4, 2), (1, 2, 4, 3, 3), (2, 1, 5, 5, 2)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [0.7, -0.4, 0.0])
def test_finite_differences(B, H, Nq, Nk, d, causal, scale):
    q = rand((B, H, Nq, d), 1)
    k = rand((B, H, Nk, d), 2)
    v = rand((B, H, Nk, d), 3)
    g = rand((B, H, Nq, d), 4)
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, scale, causal)
    f = lambda: loss(q, k, v, g, scale, causal)
    for got, x in ((dq, q), (dk, k), (dv, v)):
        want = numeric_grad(x, f)
        assert np.max(np.abs(got - want)) < 1e-7


def torch_grads(q, k, v, g, scale, causal):
    qt, kt, vt = (torch.tensor(t, dtype=torch.float64, requires_grad=True) for t in (q, k, v))
    s = scale * (qt @ kt.transpose(-1, -2))
    if causal:
        Nq, Nk = s.shape[-2:]
        mask = torch.arange(Nk)[None, :] > torch.arange(Nq)[:, None]
        s = s.masked_fill(mask, float("-inf"))
    o = torch.softmax(s, dim=-1) @ vt
    (o * torch.tensor(g, dtype=torch.float64)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("shape,causal,scale", [
    ((2, 3, 17, 23, 8), False, 1 / math.sqrt(8)),
    ((1, 2, 31, 31, 16), True, 0.25),
    ((1, 1, 40, 9, 5), True, -0.6),
    ((1, 1, 9, 40, 5), False, 1.3),
])
def test_against_torch_autograd(shape, causal, scale):
    B, H, Nq, Nk, d = shape
    q = rand((B, H, Nq, d), 11)
    k = rand((B, H, Nk, d), 12)
    v = rand((B, H, Nk, d), 13)
    g = rand((B, H, Nq, d), 14)
    got = oracle.attention_bwd(q, k, v, g, scale, causal)
    want = torch_grads(q, k, v, g, scale, causal)
    for a, b in zip(got, want):
        assert np.max(np.abs(a - b)) < 1e-11


@pytest.mark.parametrize("causal", [False, True])
def test_identical_value_rows_give_zero_dq_dk(causal):
    """O = v for every query whatever the weights, so S gets no gradient."""
    q = rand((1, 2, 6, 4), 21)
    k = rand((1, 2, 7, 4), 22)
    row = rand((4,), 23)
    v = np.broadcast_to(row, (1, 2, 7, 4)).copy()
    g = rand((1, 2, 6, 4), 24)
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, 0.8, causal)
    assert np.max(np.abs(dq)) < 1e-13 and np.max(np.abs(dk)) < 1e-13
    # dV_j = sum_i P_ij dO_i; the weights of each row sum to 1, so sum_j dV_j = sum_i dO_i
    assert np.allclose(dv.sum(axis=2), g.sum(axis=2), atol=1e-13)


def test_zero_scale_uniform_weights():
    q = rand((1, 1, 5, 3), 31)
    k = rand((1, 1, 8, 3), 32)
    v = rand((1, 1, 8, 3), 33)
    g = rand((1, 1, 5, 3), 34)
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, 0.0, False)
    assert np.max(np.abs(dq)) == 0.0 and np.max(np.abs(dk)) == 0.0
    want = np.broadcast_to(g.sum(axis=2, keepdims=True) / 8, dv.shape)
    assert np.allclose(dv, want, atol=1e-14)


def test_single_key():
    q = rand((1, 1, 4, 3), 41)
    k = rand((1, 1, 1, 3), 42)
    v = rand((1, 1, 1, 3), 43)
    g = rand((1, 1, 4, 3), 44)
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, 0.9, False)
    assert np.max(np.abs(dq)) < 1e-15 and np.max(np.abs(dk)) < 1e-15
    assert np.allclose(dv[0, 0, 0], g[0, 0].sum(axis=0), atol=1e-14)


def test_causal_keys_past_the_last_query_get_no_gradient():
    """Top-left causal with Nk > Nq: keys j >= Nq are visible to no query."""
    q = rand((1, 1, 4, 3), 51)
    k = rand((1, 1, 9, 3), 52)
    v = rand((1, 1, 9, 3), 53)
    g = rand((1, 1, 4, 3), 54)
    _, dk, dv = oracle.attention_bwd(q, k, v, g, 0.5, True)
    assert np.all(dk[0, 0, 4:] == 0.0) and np.all(dv[0, 0, 4:] == 0.0)
    assert np.max(np.abs(dk[0, 0, :4])) > 0 and np.max(np.abs(dv[0, 0, :4])) > 0


def test_row_term_equals_do_dot_o():
    """rowsum(P * dP) = rowsum(dO * O): the D term the kernels read from O (forward oracle)."""
    q = rand((1, 2, 7, 5), 61)
    k = rand((1, 2, 9, 5), 62)
    v = rand((1, 2, 9, 5), 63)
    g = rand((1, 2, 7, 5), 64)
    o, _ = oracle.attention_fwd(q, k, v, 0.6, True)
    d_fwd = (g * o).sum(axis=-1)
    s = 0.6 * np.einsum("bhqd,bhkd->bhqk", q, k)
    s = np.where(np.arange(9)[None, :] <= np.arange(7)[:, None], s, -np.inf)
    p = np.exp(s - s.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    dp = np.einsum("bhqd,bhkd->bhqk", g, v)
    assert np.allclose((p * dp).sum(-1), d_fwd, atol=1e-13)


def test_bad_shapes_raise():
    q = rand((1, 1, 3, 2), 1)
    with pytest.raises(ValueError):
        oracle.attention_bwd(q, rand((1, 1, 4, 3), 2), rand((1, 1, 4, 3), 3), q, 1.0, False)
    with pytest.raises(ValueError):
        oracle.attention_bwd(q, rand((1, 1, 4, 2), 2), rand((1, 1, 4, 2), 3), rand((1, 1, 4, 2), 4), 1.0, False)


def _probs(q, k, scale, causal):
    """Softmax weights written out separately (numpy, per head)."""
    s = scale * np.einsum("bhqd,bhkd->bhqk", q, k)
    if causal:
        Nq, Nk = s.shape[-2:]
        s = np.where(np.arange(Nk)[None, :] <= np.arange(Nq)[:, None], s, -np.inf)
    p = np.exp(s - s.max(-1, keepdims=True))
    return p / p.sum(-1, keepdims=True)


@pytest.mark.parametrize("causal", [False, True])
def test_stored_output_equal_to_exact_output_changes_nothing(causal):
    """Given the exact forward output, the row term rowsum(dO * O) equals rowsum(P * dP), so the
    gradients are those of the chain rule (page "flash_attention_2.cu", backward kernel: D from
    the stored output)."""
    q, k, v, g = rand((2, 2, 6, 5), 71), rand((2, 2, 8, 5), 72), rand((2, 2, 8, 5), 73), rand((2, 2, 6, 5), 74)
    o, _ = oracle.attention_fwd(q, k, v, 0.45, causal)
    for a, b in zip(oracle.attention_bwd(q, k, v, g, 0.45, causal, o=o), oracle.attention_bwd(q, k, v, g, 0.45, causal)):
        assert np.max(np.abs(a - b)) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_stored_output_perturbation_moves_gradients_by_the_closed_form(causal):
    """A stored output o + E changes the row term by dD_i = sum_c dO_ic E_ic. dS = P (dP - D) is
    linear in D, so dQ moves by -scale dD_i sum_j P_ij k_j, dK by -scale sum_i P_ij dD_i q_i,
    and dV not at all."""
    scale = 0.6
    q, k, v, g = rand((1, 2, 7, 4), 81), rand((1, 2, 9, 4), 82), rand((1, 2, 9, 4), 83), rand((1, 2, 7, 4), 84)
    o, _ = oracle.attention_fwd(q, k, v, scale, causal)
    e = rand(o.shape, 85, 1e-2)
    base = oracle.attention_bwd(q, k, v, g, scale, causal, o=o)
    moved = oracle.attention_bwd(q, k, v, g, scale, causal, o=o + e)
    p = _probs(q, k, scale, causal)
    dD = (g * e).sum(-1)  # [B,H,Nq]
    want_dq = -scale * dD[..., None] * np.einsum("bhqk,bhkd->bhqd", p, k)
    want_dk = -scale * np.einsum("bhqk,bhq,bhqd->bhkd", p, dD, q)
    assert np.max(np.abs((moved[0] - base[0]) - want_dq)) < 1e-12
    assert np.max(np.abs((moved[1] - base[1]) - want_dk)) < 1e-12
    assert np.max(np.abs(moved[2] - base[2])) < 1e-12
