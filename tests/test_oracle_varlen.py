"""Pins for the packed variable-length oracle (oracle.attention_fwd_varlen).

Checked against things other than its own route (per-sequence calls of the C forward):
- a block-diagonal softmax over the whole packed score matrix in numpy, where a segment id per
  row decides which keys a query sees (a wrong offset, a sequence that leaks into the next
  one, or a causal mask in packed instead of per-sequence positions fails it);
- the dense forward on a [B,H,N,d] batch whose sequences all have one length, repacked;
- closed forms: one key per sequence gives O = that key's value row and L = scale q.k;
  a sequence with queries but no keys gives O = 0 and L = -inf.
"""
import numpy as np
import pytest

import oracle


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def offsets(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)


def block_diagonal(q, k, v, lq, lk, scale, causal):
    """Whole packed matrix, mask from segment ids and in-sequence positions."""
    seg_q = np.repeat(np.arange(len(lq)), lq)
    seg_k = np.repeat(np.arange(len(lk)), lk)
    pos_q = np.concatenate([np.arange(n) for n in lq]) if len(lq) else np.zeros(0, int)
    pos_k = np.concatenate([np.arange(n) for n in lk]) if len(lk) else np.zeros(0, int)
    visible = seg_q[:, None] == seg_k[None, :]
    if causal:
        visible &= pos_k[None, :] <= pos_q[:, None]
    H, Tq, d = q.shape
    o = np.zeros((H, Tq, d))
    lse = np.full((H, Tq), -np.inf)
    for h in range(H):
        s = scale * np.einsum("id,jd->ij", q[h], k[h])
        for i in range(Tq):
            sel = visible[i]
            if not sel.any():
                continue
            row = s[i, sel]
            m = row.max()
            w = np.exp(row - m)
            o[h, i] = w @ v[h][sel] / w.sum()
            lse[h, i] = m + np.log(w.sum())
    return o, lse


CASES = [
    ([5, 1, 7], [5, 1, 7]),
    ([3, 0, 8, 2], [4, 6, 8, 1]),     # an empty query sequence
    ([4, 3], [0, 5]),                 # queries with no keys
    ([1, 1, 1], [9, 2, 3]),
    ([12], [3]),
]


@pytest.mark.parametrize("lq,lk", CASES)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [0.6, -1.1])
def test_block_diagonal_softmax(lq, lk, causal, scale):
    H, d = 2, 5
    q = rand((H, sum(lq), d), 1)
    k = rand((H, sum(lk), d), 2)
    v = rand((H, sum(lk), d), 3)
    o, lse = oracle.attention_fwd_varlen(q, k, v, offsets(lq), offsets(lk), scale, causal)
    wo, wl = block_diagonal(q, k, v, lq, lk, scale, causal)
    assert np.max(np.abs(o - wo)) < 1e-12
    fin = np.isfinite(wl)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.max(np.abs(lse[fin] - wl[fin]), initial=0.0) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_match_dense(causal):
    B, H, N, d = 3, 2, 9, 4
    q = rand((B, H, N, d), 11)
    k = rand((B, H, N, d), 12)
    v = rand((B, H, N, d), 13)
    pack = lambda t: t.transpose(1, 0, 2, 3).reshape(H, B * N, d)
    cu = offsets([N] * B)
    o, lse = oracle.attention_fwd_varlen(pack(q), pack(k), pack(v), cu, cu, 0.4, causal)
    wo, wl = oracle.attention_fwd(q, k, v, 0.4, causal)
    assert np.max(np.abs(o - pack(wo))) < 1e-13
    assert np.max(np.abs(lse - wl.transpose(1, 0, 2).reshape(H, B * N))) < 1e-13


def test_single_key_sequences():
    lq, lk = [3, 2, 4], [1, 1, 1]
    q = rand((1, 9, 3), 21)
    k = rand((1, 3, 3), 22)
    v = rand((1, 3, 3), 23)
    o, lse = oracle.attention_fwd_varlen(q, k, v, offsets(lq), offsets(lk), 0.7, False)
    seg = np.repeat(np.arange(3), lq)
    assert np.allclose(o[0], v[0][seg], atol=1e-15)
    assert np.allclose(lse[0], 0.7 * np.sum(q[0] * k[0][seg], axis=1), atol=1e-14)


def test_queries_without_keys():
    q = rand((2, 6, 3), 31)
    k = rand((2, 4, 3), 32)
    v = rand((2, 4, 3), 33)
    o, lse = oracle.attention_fwd_varlen(q, k, v, [0, 2, 6], [0, 0, 4], 1.0, True)
    assert np.all(o[:, :2] == 0.0) and np.all(lse[:, :2] == -np.inf)
    assert np.all(np.isfinite(lse[:, 2:]))


@pytest.mark.parametrize("cu_q,cu_k", [
    ([0, 3, 2, 4], [0, 1, 2, 3]),   # decreasing
    ([1, 2, 4], [0, 1, 3]),         # does not start at 0
    ([0, 2, 3], [0, 1, 3]),         # does not end at Tq
    ([0, 4], [0, 1, 3]),            # different sequence counts
])
def test_bad_offsets_raise(cu_q, cu_k):
    q = rand((1, 4, 2), 1)
    k = rand((1, 3, 2), 2)
    with pytest.raises(ValueError):
        oracle.attention_fwd_varlen(q, k, k, cu_q, cu_k, 1.0, False)
