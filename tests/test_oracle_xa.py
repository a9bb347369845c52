"""Pins of the XAttention-mode oracle against things other than itself: brute
force over the full score matrix, the stride-1 special case, the softmax
normalisation, invariances, exhaustive search for the threshold selection, and
library attention for the all-kept and forced-only cases.  A plausible mistake
in the oracle (main diagonal instead of antidiagonal, a missing 1/S, a shifted
block index, a greedy order that drops the forced blocks, a > for a >=) fails
one of them."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import ea_oracle as orc
from oracle import xa_oracle as xa

FACTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def test_page_facts_threshold_and_configs():
    assert xa.xa_plan.__kwdefaults__["tau"] == FACTS["xa_threshold"]["value"]
    assert sorted(xa.HEAD_CONFIGS) == sorted(FACTS["head_configs"]["value"])
    # "{retrieval mode}-{sparse mode}": router mode 0 is the retrieval head
    for name, (m0, m1) in xa.HEAD_CONFIGS.items():
        r, s = name.split("-")
        assert {"FA": 0, "XA": 2}[r] == m0 and {"SSA": 1, "XA": 2}[s] == m1


@pytest.mark.parametrize("L,S", [(37, 4), (40, 8), (16, 8), (9, 3)])
def test_antidiagonal_brute_force(L, S):
    # every S x S tile of the zero-padded Q K^T, summed over r + c = S - 1
    d = 5
    q, k = _rand(1, L, d), _rand(2, L, d)
    n = -(-L // S)
    full = np.zeros((n * S, n * S))
    full[:L, :L] = q @ k.T
    want = np.zeros((n, n))
    for a in range(n):
        for c in range(n):
            for r in range(S):
                want[a, c] += full[a * S + r, c * S + (S - 1 - r)]
    np.testing.assert_allclose(xa.antidiagonal_scores(q, k, S), want, rtol=1e-12, atol=1e-12)


def test_antidiagonal_is_not_the_main_diagonal():
    # a query group whose last row alone matches the key group's first row
    d, S = 4, 4
    q = np.zeros((8, d))
    k = np.zeros((8, d))
    q[3] = [1, 0, 0, 0]   # row aS + S-1 of group 0
    k[0] = [1, 0, 0, 0]   # row cS + 0 of group 0
    D = xa.antidiagonal_scores(q, k, S)
    assert D[0, 0] == 1.0 and D.sum() == 1.0
    q2 = np.zeros((8, d))
    q2[0] = [1, 0, 0, 0]  # main-diagonal partner: not on the antidiagonal
    assert xa.antidiagonal_scores(q2, k, S).sum() == 0.0


def test_stride_one_is_the_score_matrix():
    q, k = _rand(3, 23, 6), _rand(4, 23, 6)
    np.testing.assert_allclose(xa.antidiagonal_scores(q, k, 1), q @ k.T, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("L", [300, 256, 129])
def test_block_mass_rows_sum_to_group_rows(L):
    # each group row's softmax sums to 1 over the visible groups
    B, S = 32, 4
    q, k = _rand(5, L, 8), _rand(6, L, 8)
    A = xa.block_mass(q, k, block=B, stride=S)
    nb = -(-L // B)
    n = -(-L // S)
    rows = np.array([min(B // S, n - i * (B // S)) for i in range(nb)])
    np.testing.assert_allclose(A.sum(axis=1), rows, rtol=1e-12)
    assert np.all(np.triu(A, 1) == 0) and np.all(A[np.tril_indices(nb)] > 0)


def test_block_mass_matches_softmax_of_scaled_groups():
    # stride 1 and block 1: A is the causal softmax of Q K^T / sqrt(d) itself
    L, d = 12, 5
    q, k = _rand(7, L, d), _rand(8, L, d)
    A = xa.block_mass(q, k, block=1, stride=1)
    ref = torch.softmax(torch.tensor(q @ k.T / math.sqrt(d)).masked_fill(
        torch.triu(torch.ones(L, L, dtype=torch.bool), 1), -math.inf), dim=1).numpy()
    np.testing.assert_allclose(A, ref, rtol=1e-12, atol=1e-15)


def test_block_mass_uses_one_over_stride():
    # one group per block: A is the causal softmax of the antidiagonal sums
    # divided by S (the mean of the S products), nothing else
    L, d, S = 16, 3, 4
    q, k = _rand(9, L, d), _rand(10, L, d)
    A = xa.block_mass(q, k, block=S, stride=S, scale=1.0)
    D = xa.antidiagonal_scores(q, k, S) / S
    n = D.shape[0]
    D = np.where(np.tril(np.ones((n, n), bool)), D, -np.inf)
    P = np.exp(D - D.max(1, keepdims=True))
    P /= P.sum(1, keepdims=True)
    np.testing.assert_allclose(A, P, rtol=1e-12)


def test_block_mass_key_shift_invariance():
    # a constant added to every key row adds the same amount to a group row's
    # scores, which its softmax removes
    L, d = 200, 8
    q, k = _rand(11, L, d), _rand(12, L, d)
    A0 = xa.block_mass(q, k, block=32, stride=8)
    A1 = xa.block_mass(q, k + _rand(13, d)[None, :] * 3.0, block=32, stride=8)
    np.testing.assert_allclose(A0, A1, rtol=1e-9, atol=1e-12)


def _exhaustive(a, i, tau):
    """Smallest subsets containing blocks 0 and i with mass >= tau * total;
    returns (size, best mass among subsets of that size)."""
    a = np.asarray(a[:i + 1], np.float64)
    target = tau * a.sum()
    free = list(range(1, i))
    for r in range(len(free) + 1):
        best = None
        for extra in itertools.combinations(free, r):
            m = a[[0, i, *extra]].sum() if i > 0 else a[0]
            if m >= target and (best is None or m > best):
                best = m
        if best is not None:
            return len({0, i}) + r, best
    raise AssertionError


@pytest.mark.parametrize("seed", range(8))
def test_selection_is_minimal(seed):
    r = np.random.default_rng(100 + seed)
    i = int(r.integers(1, 10))
    a = r.exponential(size=i + 1) ** 2
    for tau in (0.3, 0.9, 0.99):
        keep = xa.select_row(a, i, tau)
        size, best = _exhaustive(a, i, tau)
        assert keep[0] and keep[i]
        assert keep.sum() == size
        assert a[keep].sum() >= tau * a.sum()
        assert math.isclose(a[keep].sum(), best, rel_tol=1e-12)


def test_selection_extremes_and_ties():
    a = np.array([0.1, 0.2, 0.2, 0.2, 0.3])
    assert xa.select_row(a, 4, 1.0).all()
    assert xa.select_row(a, 4, 0.0).tolist() == [True, False, False, False, True]
    # 0.4 forced, 0.2 more needed to reach 0.6: one of the three equal blocks,
    # the lowest index
    assert xa.select_row(a, 4, 0.6).tolist() == [True, True, False, False, True]
    assert xa.select_row(np.array([1.0]), 0, 0.9).tolist() == [True]


def test_needle_block_is_selected():
    # one far key block aligned with a late query block carries its mass
    L, d, B, S = 1024, 16, 128, 8
    q, k = _rand(14, L, d) * 0.1, _rand(15, L, d) * 0.1
    u = np.zeros(d)
    u[0] = 1.0
    q[7 * B:] += 6.0 * u
    k[3 * B:4 * B] += 6.0 * u
    A = xa.block_mass(q, k, block=B, stride=S)
    sel = xa.select(A, 0.9)
    assert sel[7].tolist() == [True, False, False, True, False, False, False, True]


def _sdpa(q, k, v, mask):
    s = torch.tensor(q) @ torch.tensor(k).T / math.sqrt(q.shape[1])
    s = s.masked_fill(~torch.tensor(mask), -math.inf)
    return (torch.softmax(s, 1) @ torch.tensor(v)).numpy()


def _case(seed, L=300, Hq=4, Hkv=2, d=8):
    Q, K, V = _rand(seed, L, Hq, d), _rand(seed + 1, L, Hkv, d), _rand(seed + 2, L, Hkv, d)
    return Q, K, V, np.array([0, L])


def test_xa_attention_tau_one_is_causal_attention():
    Q, K, V, cu = _case(20)
    cm = np.array([[2, 2]])
    plan = xa.xa_plan(Q, K, cm, cu, block=32, stride=4, tau=1.0)
    O, _ = xa.hybrid_attention_xa(Q, K, V, cm, cu, plan, xa_block=32)
    L = Q.shape[0]
    causal = np.tril(np.ones((L, L), bool))
    for hq in range(4):
        np.testing.assert_allclose(O[:, hq], _sdpa(Q[:, hq], K[:, hq // 2], V[:, hq // 2], causal),
                                   rtol=1e-10, atol=1e-12)


def test_xa_attention_tau_zero_is_sink_plus_own_block():
    Q, K, V, cu = _case(30)
    cm = np.array([[2, 0]])
    plan = xa.xa_plan(Q, K, cm, cu, block=32, stride=4, tau=0.0)
    O, lse = xa.hybrid_attention_xa(Q, K, V, cm, cu, plan, xa_block=32)
    L = Q.shape[0]
    i, j = np.arange(L)[:, None], np.arange(L)[None, :]
    mask = (j <= i) & ((j < 32) | (j // 32 == i // 32))
    for hq in (0, 1):
        np.testing.assert_allclose(O[:, hq], _sdpa(Q[:, hq], K[:, 0], V[:, 0], mask),
                                   rtol=1e-10, atol=1e-12)
    # the FA KV head is untouched by XA: the plain hybrid oracle agrees
    O2, lse2 = orc.hybrid_attention(Q, K, V, np.array([[0, 0]]), cu)
    np.testing.assert_allclose(O[:, 2:], O2[:, 2:], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse[:, 2:], lse2[2:].T, rtol=1e-12)


def test_xa_rows_subset_matches_full():
    Q, K, V, cu = _case(40, L=260)
    cm = np.array([[2, 1]])
    plan = xa.xa_plan(Q, K, cm, cu, block=32, stride=8, tau=0.9)
    O, lse = xa.hybrid_attention_xa(Q, K, V, cm, cu, plan, xa_block=32, window_blocks=1)
    toks = [0, 31, 32, 100, 259]
    O2, lse2 = xa.hybrid_attention_xa(Q, K, V, cm, cu, plan, xa_block=32, window_blocks=1,
                                      tokens=toks, heads=[1, 3])
    np.testing.assert_allclose(O2, O[toks][:, [1, 3]], rtol=1e-13)
    np.testing.assert_allclose(lse2, lse[toks][:, [1, 3]], rtol=1e-13)


def test_xa_effective_flops_counts_selected_pairs():
    # tau = 1 keeps every causal block: the FA count; SA heads as before
    Q, K, V, cu = _case(50, L=300)
    cm = np.array([[2, 1]])
    plan = xa.xa_plan(Q, K, cm, cu, block=128, stride=8, tau=1.0)
    got = xa.xa_effective_flops(cm, cu, 4, 2, 8, plan, window_blocks=1)
    fa = orc.effective_flops(np.array([[0, 1]]), cu, 4, 2, 8, window_blocks=1)
    assert got == fa


def test_block_mass_rows_is_block_mass():
    # the row-restricted form used at full size agrees with the whole matrix
    L, d = 700, 8
    q, k = _rand(60, L, d), _rand(61, L, d)
    A = xa.block_mass(q, k, block=64, stride=8)
    rows = [0, 3, 10]
    np.testing.assert_allclose(xa.block_mass_rows(q, k, rows, block=64, stride=8), A[rows],
                               rtol=1e-12, atol=1e-15)
