"""Pins of the CPU oracle against things other than itself: values the pages
state, closed forms, textbook/library special cases, invariants and brute force
on tiny inputs.  Each test names what it pins and why a plausible mistake in
the oracle (a dropped term, a wrong sign or index, a transposed operand) would
fail it."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import ea_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")
FACTS = json.load(open(GOLDEN))


def _rand(seed, *shape, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _weights(seed, d, th, rh, std=0.3):
    r = np.random.default_rng(seed)
    return {
        "w1": r.standard_normal((th, d)) * std, "b1": r.standard_normal(th) * std,
        "w2": r.standard_normal((d, th)) * std, "b2": r.standard_normal(d) * std,
        "w3": r.standard_normal((rh, d)) * std, "b3": r.standard_normal(rh) * std,
        "w4": r.standard_normal((2, rh)) * std, "b4": r.standard_normal(2) * std,
    }


# ----------------------------------------------------------------------------
# Router
# ----------------------------------------------------------------------------

def test_page_facts_pool_len_and_modes():
    # the oracle's defaults and conventions are the pages' numbers
    assert orc.boundary_pool.__defaults__[0] == FACTS["pool_len"]["value"]
    assert orc.route.__defaults__[0] == FACTS["pool_len"]["value"]
    d, th, rh = 8, 16, 4
    w = _weights(0, d, th, rh)
    w["w4"][:] = 0.0
    K = _rand(1, 50, 3, d)
    cu = np.array([0, 50])
    w["b4"] = np.array([1.0, 0.0])
    m, z = orc.route(K, cu, w)
    assert (m == FACTS["mode_fa"]["value"]).all() and z.shape[-1] == FACTS["logits_columns"]["value"]
    w["b4"] = np.array([0.0, 1.0])
    m, _ = orc.route(K, cu, w)
    assert (m == FACTS["mode_sa"]["value"]).all()


def test_router_param_count_matches_page_and_draws():
    # 128 -> 1024 -> 128 task MLP, 128 -> 64 -> 2 router MLP: about 0.27M per layer
    n = orc.router_param_count(128, 1024, 64)
    assert n == 271682
    f = FACTS["router_params_per_layer_at_head_dim_128"]
    assert abs(n - f["value"]) / f["value"] < f["rel_tol"]
    # the closed form equals the number of values the generator actually draws
    from workloads.gen import draw_router_weights
    w = draw_router_weights(0, 128, 1024, 64, 0.02)
    assert sum(a.size for a in w.values()) == n


def test_argmax_tie_goes_to_fa():
    d = 8
    w = _weights(2, d, 16, 4)
    w["w4"][:] = 0.0
    w["b4"] = np.array([0.25, 0.25])
    m, z = orc.route(_rand(3, 300, 2, d), np.array([0, 300]), w)
    assert (z[..., 0] == z[..., 1]).all() and (m == 0).all()


def test_gelu_textbook_values():
    # GELU(x) = x Phi(x): Phi(0) = 1/2, Phi(1) = 0.8413447460685429 (normal table),
    # Phi(x) + Phi(-x) = 1 so GELU(x) - GELU(-x) = x, and GELU(x) -> x, GELU(-x) -> 0
    assert orc.gelu(0.0) == 0.0
    assert abs(orc.gelu(1.0) - 0.8413447460685429) < 1e-15
    assert abs(orc.gelu(-1.0) - (0.8413447460685429 - 1.0)) < 1e-15
    x = np.linspace(-6, 6, 97)
    np.testing.assert_allclose(orc.gelu(x) - orc.gelu(-x), x, atol=1e-14)
    assert abs(orc.gelu(10.0) - 10.0) < 1e-12 and abs(orc.gelu(-10.0)) < 1e-12


def test_router_matches_torch_modules():
    # nn.Linear / exact GELU in float64 compose to the same logits
    d, th, rh = 16, 64, 8
    w = _weights(4, d, th, rh)
    x = _rand(5, 7, d)
    net = torch.nn.Sequential(
        torch.nn.Linear(d, th), torch.nn.GELU(approximate="none"), torch.nn.Linear(th, d),
        torch.nn.Linear(d, rh), torch.nn.GELU(approximate="none"), torch.nn.Linear(rh, 2),
    ).double()
    with torch.no_grad():
        for lin, (wn, bn) in zip([net[0], net[2], net[3], net[5]],
                                 [("w1", "b1"), ("w2", "b2"), ("w3", "b3"), ("w4", "b4")]):
            lin.weight.copy_(torch.from_numpy(w[wn]))
            lin.bias.copy_(torch.from_numpy(w[bn]))
        z_ref = net(torch.from_numpy(x)).numpy()
    np.testing.assert_allclose(orc.router_logits(x, w), z_ref, rtol=0, atol=1e-13)


def test_boundary_pool_bruteforce_and_union():
    d = 4
    for L in [0, 1, 57, 100, 150, 199, 200, 201, 333]:
        K = _rand(L + 7, L, 2, d)
        out = orc.boundary_pool(K, np.array([0, L]), pool_len=100)
        for g in range(2):
            rows = sorted(set(range(min(100, L))) | set(range(max(0, L - 100), L)))
            if L == 0:
                assert (out[0, g] == 0).all()
                continue
            acc = [0.0] * d
            for t in rows:
                for c in range(d):
                    acc[c] += float(K[t, g, c])
            np.testing.assert_allclose(out[0, g], np.array(acc) / len(rows), rtol=0, atol=1e-14)
            # below 200 tokens nothing is counted twice
            assert len(rows) == min(L, 200)


def test_boundary_pool_locality_and_head_permutation():
    d, L = 8, 1000
    K = _rand(11, L, 4, d)
    cu = np.array([0, L])
    a = orc.boundary_pool(K, cu)
    K2 = K.copy()
    K2[100:L - 100] = 1e6  # the middle of the sequence does not reach the router
    np.testing.assert_array_equal(orc.boundary_pool(K2, cu), a)
    K3 = K.copy()
    K3[99] += 1.0          # the last pooled head row does
    assert not np.array_equal(orc.boundary_pool(K3, cu), a)
    perm = np.array([2, 0, 3, 1])
    w = _weights(12, d, 32, 4)
    np.testing.assert_array_equal(orc.router_logits(orc.boundary_pool(K[:, perm], cu), w),
                                  orc.router_logits(a, w)[:, perm])


def test_route_varlen_independent_sequences():
    d = 8
    w = _weights(13, d, 32, 4)
    lens = [250, 0, 90, 400]
    cu = np.concatenate([[0], np.cumsum(lens)])
    K = _rand(14, cu[-1], 3, d)
    m, z = orc.route(K, cu, w)
    for b, L in enumerate(lens):
        if L == 0:
            assert (z[b] == 0).all() and (m[b] == 0).all()
            continue
        mb, zb = orc.route(K[cu[b]:cu[b + 1]], np.array([0, L]), w)
        np.testing.assert_array_equal(zb[0], z[b])


# ----------------------------------------------------------------------------
# Sparse geometry
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("L,block,ns,rho,keep", [
    (512, 64, 1, 0.2, 2),        # N = 8
    (32768, 64, 2, 0.2, 102),    # N = 512
    (131072, 64, 1, 0.2, 410),   # N = 2048
    (262144, 64, 4, 0.1, 410),   # N = 4096
    (100, 64, 1, 0.2, 2),        # N = 2: at least one window block
    (64 * 5, 64, 0, 0.3, 2),     # 1.5 rounds half up
])
def test_sa_geometry_closed_form(L, block, ns, rho, keep):
    n_sink, w = orc.sa_geometry(L, block, ns, 0, rho)
    assert n_sink == ns and n_sink + w == keep and w >= 1


def test_keep_fraction_matches_page_example():
    rho = FACTS["sa_keep_fraction_example"]["value"]
    for L in [32768, 131072, 262144]:
        ns, w = orc.sa_geometry(L, 64, 1, 0, rho)
        N = L // 64
        assert abs((ns + w) / N - rho) <= 0.5 / N + 1e-12


def test_visible_block_count_closed_form():
    # sum over query blocks of visible key blocks = K(K+1)/2 + (N-K)K for SA, N(N+1)/2 for FA
    for L, ns, rho in [(32768, 2, 0.2), (4096, 1, 0.2), (64 * 37 + 5, 3, 0.3)]:
        n_sink, w = orc.sa_geometry(L, 64, ns, 0, rho)
        N = -(-L // 64)
        Kk = n_sink + w
        count = 0
        for qb in range(N):
            kb = np.arange(qb + 1)
            count += int(orc.visible(qb * 64 + 63, kb * 64, 1, n_sink, w, 64).sum())
        assert count == Kk * (Kk + 1) // 2 + (N - Kk) * Kk
    n_sink, w = orc.sa_geometry(32768, 64, 2, 0, 0.2)
    assert n_sink + w == 102 and 102 * 103 // 2 + 410 * 102 == 47073


def test_effective_flops_closed_forms():
    # all-FA, one 32K sequence, 32 query heads, d = 128: 4 d Hq 64^2 N(N+1)/2
    N = 512
    cu = np.array([0, 32768])
    fa = orc.effective_flops(np.zeros((1, 8), np.int8), cu, 32, 8, 128, n_sink=2)
    assert fa == 4 * 128 * 32 * 64 * 64 * N * (N + 1) // 2
    sa = orc.effective_flops(np.ones((1, 8), np.int8), cu, 32, 8, 128, n_sink=2)
    assert sa == 4 * 128 * 32 * 64 * 64 * 47073
    # a ragged tail: L = 100 -> blocks of 64 and 36 rows
    cu = np.array([0, 100])
    fa = orc.effective_flops(np.zeros((1, 1), np.int8), cu, 1, 1, 4)
    assert fa == 4 * 4 * (64 * 64 + 36 * 64 + 36 * 36)


# ----------------------------------------------------------------------------
# Attention
# ----------------------------------------------------------------------------

def _brute(Q, K, V, modes, L, block, ns, w, scale, G):
    """Pure-Python double loop over (i, j) with the visibility written out."""
    Hq, d = Q.shape[1], Q.shape[2]
    O = np.zeros((L, Hq, d))
    for h in range(Hq):
        g = h // G
        for i in range(L):
            js = []
            for j in range(i + 1):
                if modes[0, g] == 0 or j // block < ns or i // block - j // block < w:
                    js.append(j)
            s = [scale * sum(float(Q[i, h, c]) * float(K[j, g, c]) for c in range(d)) for j in js]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            tot = sum(e)
            for c in range(d):
                O[i, h, c] = sum(e[t] * float(V[js[t], g, c]) for t in range(len(js))) / tot
    return O


@pytest.mark.parametrize("modes", [[0, 0], [1, 1], [0, 1], [1, 0]])
def test_attention_bruteforce_tiny(modes):
    L, Hq, Hkv, d, block, ns, w = 45, 4, 2, 3, 8, 1, 2
    Q, K, V = _rand(20, L, Hq, d), _rand(21, L, Hkv, d), _rand(22, L, Hkv, d)
    m = np.array([modes], np.int8)
    O, _ = orc.hybrid_attention(Q, K, V, m, np.array([0, L]), block=block, n_sink=ns,
                                window_blocks=w, chunk=16)
    ref = _brute(Q, K, V, m, L, block, ns, w, 1 / math.sqrt(d), Hq // Hkv)
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)


def _sdpa(Q, K, V, causal=True):
    q = torch.from_numpy(Q).permute(1, 0, 2)[None]
    k = torch.from_numpy(K).permute(1, 0, 2)[None]
    v = torch.from_numpy(V).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, enable_gqa=True)
    return o[0].permute(1, 0, 2).numpy()


def test_all_fa_equals_sdpa():
    L, Hq, Hkv, d = 300, 8, 2, 16
    Q, K, V = _rand(30, L, Hq, d), _rand(31, L, Hkv, d), _rand(32, L, Hkv, d)
    O, LSE = orc.hybrid_attention(Q, K, V, np.zeros((1, Hkv), np.int8), np.array([0, L]), chunk=64)
    np.testing.assert_allclose(O, _sdpa(Q, K, V), rtol=0, atol=1e-12)
    # LSE against torch.logsumexp of the masked scores
    s = torch.einsum("ihc,jhc->hij", torch.from_numpy(Q[:, :1]), torch.from_numpy(K[:, :1])) / math.sqrt(d)
    s = s.masked_fill(torch.triu(torch.ones(L, L, dtype=torch.bool), 1), float("-inf"))
    np.testing.assert_allclose(LSE[0], torch.logsumexp(s[0], -1).numpy(), atol=1e-12)


def test_window_covering_sequence_equals_fa():
    L, Hq, Hkv, d = 200, 4, 2, 8
    Q, K, V = _rand(33, L, Hq, d), _rand(34, L, Hkv, d), _rand(35, L, Hkv, d)
    cu = np.array([0, L])
    fa, _ = orc.hybrid_attention(Q, K, V, np.zeros((1, 2), np.int8), cu, block=16)
    for ns, w in [(0, 13), (2, 11), (0, 40)]:
        sa, _ = orc.hybrid_attention(Q, K, V, np.ones((1, 2), np.int8), cu, block=16,
                                     n_sink=ns, window_blocks=w)
        np.testing.assert_allclose(sa, fa, rtol=0, atol=1e-13)


def test_single_block_window_is_blockwise_sdpa():
    # n_sink = 0, w = 1: each 64-token block attends causally to itself only
    L, Hq, Hkv, d = 64 * 3 + 20, 4, 1, 8
    Q, K, V = _rand(36, L, Hq, d), _rand(37, L, Hkv, d), _rand(38, L, Hkv, d)
    sa, _ = orc.hybrid_attention(Q, K, V, np.ones((1, 1), np.int8), np.array([0, L]),
                                 n_sink=0, window_blocks=1)
    for s in range(0, L, 64):
        e = min(L, s + 64)
        np.testing.assert_allclose(sa[s:e], _sdpa(Q[s:e], K[s:e], V[s:e]), rtol=0, atol=1e-12)


def test_rows_before_window_edge_equal_fa():
    L, Hq, Hkv, d = 64 * 10, 2, 1, 8
    Q, K, V = _rand(39, L, Hq, d), _rand(40, L, Hkv, d), _rand(41, L, Hkv, d)
    cu = np.array([0, L])
    fa, _ = orc.hybrid_attention(Q, K, V, np.zeros((1, 1), np.int8), cu)
    sa, _ = orc.hybrid_attention(Q, K, V, np.ones((1, 1), np.int8), cu, n_sink=1, window_blocks=3)
    np.testing.assert_allclose(sa[:64 * 4], fa[:64 * 4], rtol=0, atol=1e-13)
    assert np.abs(sa[64 * 4:] - fa[64 * 4:]).max() > 1e-3


def _visible_range_sum(i, mode, ns, w, block, f):
    """Closed-form count and sums of f(j) = j, j^2 over the keys row i sees."""
    def s1(a, b):  # sum of j for j in [a, b)
        return (b - a) * (a + b - 1) / 2 if b > a else 0.0

    def s2(a, b):  # sum of j^2 for j in [a, b)
        g = lambda n: (n - 1) * n * (2 * n - 1) / 6  # noqa: E731  sum_{j<n} j^2
        return g(b) - g(a) if b > a else 0.0
    if mode == 0:
        ranges = [(0, i + 1)]
    else:
        lo = max(0, (i // block - w + 1) * block)
        ranges = [(0, min(ns * block, lo)), (lo, i + 1)]
    n = sum(max(0, b - a) for a, b in ranges)
    return n, sum(s1(a, b) for a, b in ranges), sum(s2(a, b) for a, b in ranges)


@pytest.mark.parametrize("mode,ns,w", [(0, 1, 1), (1, 1, 1), (1, 2, 3), (1, 0, 2), (1, 4, 1)])
def test_zero_query_gives_mean_of_visible_values(mode, ns, w):
    # Q = 0: every visible score is 0, so O_i is the plain mean of the visible V
    # rows and LSE_i = ln(count); with V[j] = (j, j^2) both follow in closed form
    L, block = 64 * 9 + 13, 64
    Q = np.zeros((L, 1, 2))
    K = _rand(42, L, 1, 2)
    V = np.stack([np.arange(L), np.arange(L) ** 2], axis=1)[:, None, :].astype(np.float64)
    O, LSE = orc.hybrid_attention(Q, K, V, np.array([[mode]], np.int8), np.array([0, L]),
                                  n_sink=ns, window_blocks=w)
    for i in range(L):
        n, a, b = _visible_range_sum(i, mode, ns, w, block, None)
        assert abs(O[i, 0, 0] - a / n) < 1e-9 * max(1, a / n)
        assert abs(O[i, 0, 1] - b / n) < 1e-9 * max(1, b / n)
        assert abs(LSE[0, i] - math.log(n)) < 1e-12


def test_constant_v_and_weights_sum_to_one():
    L, Hq, Hkv, d = 150, 2, 1, 8
    Q, K = _rand(43, L, Hq, d), _rand(44, L, Hkv, d)
    V = np.full((L, Hkv, d), 0.375)
    for mode in [0, 1]:
        m = np.array([[mode]], np.int8)
        O, _ = orc.hybrid_attention(Q, K, V, m, np.array([0, L]), block=16, n_sink=1, window_blocks=2)
        np.testing.assert_allclose(O, 0.375, rtol=0, atol=1e-15)
        P = orc.attention_weights(Q, K, m, L, 1, G=2, block=16, n_sink=1, window_blocks=2)
        np.testing.assert_allclose(P.sum(1), 1.0, atol=1e-14)
        i, j = np.meshgrid(np.arange(L), np.arange(L), indexing="ij")
        vis = orc.visible(i, j, mode, 1, 2, 16)
        assert (P[~vis] == 0).all() and (P[vis] > 0).all()


def test_constant_key_shift_leaves_output_unchanged():
    L, Hq, Hkv, d = 257, 4, 2, 16
    Q, K, V = _rand(45, L, Hq, d), _rand(46, L, Hkv, d), _rand(47, L, Hkv, d)
    cu = np.array([0, L])
    m = np.array([[0, 1]], np.int8)
    O1, L1 = orc.hybrid_attention(Q, K, V, m, cu)
    c = _rand(48, 1, Hkv, d) * 3
    O2, L2 = orc.hybrid_attention(Q, K + c, V, m, cu)
    np.testing.assert_allclose(O2, O1, rtol=0, atol=1e-12)
    assert np.abs(L2 - L1).max() > 1e-3  # LSE moves by q.c * scale


def test_varlen_equals_concatenated_single_runs():
    Hq, Hkv, d = 4, 2, 8
    lens = [130, 1, 0, 200]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = cu[-1]
    Q, K, V = _rand(49, T, Hq, d), _rand(50, T, Hkv, d), _rand(51, T, Hkv, d)
    modes = np.array([[0, 1], [1, 1], [0, 0], [1, 0]], np.int8)
    O, LSE = orc.hybrid_attention(Q, K, V, modes, cu, block=16, n_sink=1, keep_fraction=0.3)
    for b, L in enumerate(lens):
        if L == 0:
            continue
        s, e = cu[b], cu[b + 1]
        ob, lb = orc.hybrid_attention(Q[s:e], K[s:e], V[s:e], modes[b:b + 1], np.array([0, L]),
                                      block=16, n_sink=1, keep_fraction=0.3)
        np.testing.assert_array_equal(O[s:e], ob)
        np.testing.assert_array_equal(LSE[:, s:e], lb)


def test_rows_api_equals_full():
    Hq, Hkv, d = 4, 2, 8
    lens = [300, 77]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = cu[-1]
    Q, K, V = _rand(52, T, Hq, d), _rand(53, T, Hkv, d), _rand(54, T, Hkv, d)
    modes = np.array([[0, 1], [1, 0]], np.int8)
    O, LSE = orc.hybrid_attention(Q, K, V, modes, cu)
    toks = [0, 5, 63, 64, 299, 300, 376]
    heads = [0, 3]
    o, l = orc.hybrid_attention_rows(Q, K, V, modes, cu, toks, heads)
    np.testing.assert_allclose(o, O[toks][:, heads], atol=1e-14)
    np.testing.assert_allclose(l, LSE[heads][:, toks].T, atol=1e-14)
