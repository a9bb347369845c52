"""Pins of the oracle's training forward (Gumbel-Softmax routing with
straight-through hard decisions, and the dual-mode attention it mixes) against
closed forms, the Gumbel-max property, textbook attention and invariants."""
import math

import numpy as np
import torch

from oracle import ea_oracle as orc
from workloads import gen


def _rand(seed, *shape, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ----------------------------------------------------------------------------
# Gumbel-Softmax routing
# ----------------------------------------------------------------------------

def test_gumbel_route_exact_values():
    # softmax((0, ln 3) / 1) = (1/4, 3/4); the same at tau = 2 with doubled logits
    r, m = orc.gumbel_route(np.array([[0.0, math.log(3.0)]]), None, 1.0)
    np.testing.assert_allclose(r, [[0.25, 0.75]], atol=1e-7)
    assert m.tolist() == [1]
    r, m = orc.gumbel_route(np.array([[0.0, 2 * math.log(3.0)]]), None, 2.0)
    np.testing.assert_allclose(r, [[0.25, 0.75]], atol=1e-7)
    # (ln 3, 0) reversed: FA wins
    r, m = orc.gumbel_route(np.array([[math.log(3.0), 0.0]]), None, 1.0)
    np.testing.assert_allclose(r, [[0.75, 0.25]], atol=1e-7)
    assert m.tolist() == [0]


def test_gumbel_route_is_logistic_of_the_noisy_margin():
    # two classes: softmax(y)[1] = 1 / (1 + exp(y0 - y1)), y = (z + g) / tau
    z, g = _rand(1, 50, 2, scale=2.0), _rand(2, 50, 2)
    for tau in (0.3, 1.0, 4.0):
        r, m = orc.gumbel_route(z, g, tau)
        y = (z.astype(np.float32) + g.astype(np.float32)) / np.float32(tau)
        want = 1.0 / (1.0 + np.exp(y[:, 0].astype(np.float64) - y[:, 1].astype(np.float64)))
        np.testing.assert_allclose(r[:, 1], want, rtol=0, atol=1e-12)
        np.testing.assert_allclose(r.sum(-1), 1.0, atol=1e-15)
        assert np.array_equal(m, (r[:, 1] > r[:, 0]).astype(np.int8))


def test_gumbel_route_tie_goes_to_fa_and_low_temperature_is_one_hot():
    r, m = orc.gumbel_route(np.array([[1.5, 1.5], [-2.0, -2.0]]), None, 0.7)
    assert m.tolist() == [0, 0]
    np.testing.assert_allclose(r, 0.5, atol=0)
    z, g = _rand(3, 40, 2), _rand(4, 40, 2)
    r, m = orc.gumbel_route(z, g, 1e-3)
    hard = np.stack([1 - m, m], -1)
    keep = np.abs((z + g)[:, 1] - (z + g)[:, 0]) > 0.05   # margins well above tau
    np.testing.assert_allclose(r[keep], hard[keep], atol=1e-12)


def test_gumbel_noise_statistics_and_gumbel_max_property():
    g = gen.draw_gumbel(5, (400000, 2)).astype(np.float64)
    # standard Gumbel: mean = Euler-Mascheroni gamma, variance = pi^2 / 6
    assert abs(g.mean() - 0.5772156649) < 0.005
    assert abs(g.var() - math.pi ** 2 / 6) < 0.01
    # argmax(z + g) is distributed as softmax(z): the hard decisions of the
    # Gumbel-Softmax router sample SA with probability sigmoid(z1 - z0)
    z = np.tile(np.array([[0.3, 1.1]]), (g.shape[0], 1))
    _, m = orc.gumbel_route(z, g, 1.0)
    p = 1.0 / (1.0 + math.exp(0.3 - 1.1))
    assert abs(m.mean() - p) < 4 * math.sqrt(p * (1 - p) / len(m))


def test_ste_forward_value_is_the_hard_decision():
    z, g = _rand(6, 64, 2), _rand(7, 64, 2)
    r_soft, m = orc.gumbel_route(z, g, 0.5)
    r = orc.ste_weights(r_soft, m)
    np.testing.assert_allclose(r, np.stack([1 - m, m], -1), rtol=0, atol=1e-15)


# ----------------------------------------------------------------------------
# Dual-mode attention
# ----------------------------------------------------------------------------

def _sdpa(Q, K, V):
    q = torch.from_numpy(Q).permute(1, 0, 2)[None]
    k = torch.from_numpy(K).permute(1, 0, 2)[None]
    v = torch.from_numpy(V).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, enable_gqa=True)
    return o[0].permute(1, 0, 2).numpy()


def _case(seed, lengths, Hq, Hkv, d):
    T = int(sum(lengths))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    Q, K, V = _rand(seed, T, Hq, d), _rand(seed + 1, T, Hkv, d), _rand(seed + 2, T, Hkv, d)
    z, g = _rand(seed + 3, len(lengths), Hkv, 2), _rand(seed + 4, len(lengths), Hkv, 2)
    r_soft, m = orc.gumbel_route(z, g, 1.0)
    return Q, K, V, cu, r_soft, m


def test_dual_fa_output_is_causal_sdpa_and_sa_is_blockwise_for_a_one_block_window():
    Q, K, V, cu, r_soft, m = _case(10, [333], 8, 2, 16)
    O, O_fa, O_sa, L_fa, L_sa = orc.dual_attention(Q, K, V, cu, r_soft, m, n_sink=0,
                                                   window_blocks=1)
    np.testing.assert_allclose(O_fa, _sdpa(Q, K, V), rtol=0, atol=1e-12)
    for s in range(0, 333, 64):
        e = min(333, s + 64)
        np.testing.assert_allclose(O_sa[s:e], _sdpa(Q[s:e], K[s:e], V[s:e]), rtol=0, atol=1e-12)


def test_dual_lse_superset_and_covering_window():
    Q, K, V, cu, r_soft, m = _case(20, [700, 90], 4, 2, 8)
    _, O_fa, O_sa, L_fa, L_sa = orc.dual_attention(Q, K, V, cu, r_soft, m, n_sink=1,
                                                   window_blocks=2)
    # FA sees a superset of SA's keys: its log-sum-exp is never smaller
    assert (L_fa >= L_sa - 1e-12).all()
    # rows whose causal keys all lie in sinks + window: both modes agree
    np.testing.assert_allclose(O_sa[:192], O_fa[:192], rtol=0, atol=1e-13)
    np.testing.assert_allclose(O_sa[700:790], O_fa[700:790], rtol=0, atol=1e-13)
    assert np.abs(O_sa[192:700] - O_fa[192:700]).max() > 1e-3
    # and the merge identity the fused kernel relies on: the FA sum of
    # exponentials is the SA one plus that of the keys SA leaves out
    assert (np.exp(L_fa[:, 192:700]) > np.exp(L_sa[:, 192:700]) * (1 + 1e-9)).all()


def test_dual_mix_selects_by_hard_decision_per_kv_group():
    Q, K, V, cu, _, _ = _case(30, [150, 260], 8, 4, 8)
    m = np.array([[0, 1, 1, 0], [1, 0, 0, 1]], np.int8)
    r_soft = np.full((2, 4, 2), 0.5)
    O, O_fa, O_sa, _, _ = orc.dual_attention(Q, K, V, cu, r_soft, m, n_sink=1, window_blocks=1)
    G = 2
    for b in range(2):
        s0, e0 = cu[b], cu[b + 1]
        for hq in range(8):
            want = O_sa if m[b, hq // G] else O_fa
            np.testing.assert_allclose(O[s0:e0, hq], want[s0:e0, hq], rtol=0, atol=1e-15)


def test_dual_rows_api_equals_full():
    Q, K, V, cu, r_soft, m = _case(40, [200, 130], 8, 2, 8)
    full = orc.dual_attention(Q, K, V, cu, r_soft, m, n_sink=1, window_blocks=1)
    toks = np.array([0, 5, 63, 64, 199, 200, 201, 329])
    heads = [0, 3, 7]
    rows = orc.dual_attention_rows(Q, K, V, cu, r_soft, m, toks, heads, n_sink=1, window_blocks=1)
    for k in range(3):
        np.testing.assert_allclose(rows[k], full[k][toks][:, heads], rtol=0, atol=1e-14)
    for k in range(3, 5):
        np.testing.assert_allclose(rows[k], full[k][heads][:, toks].T, rtol=0, atol=1e-14)


# ----------------------------------------------------------------------------
# Decode
# ----------------------------------------------------------------------------

def test_decode_is_the_last_prefill_row():
    # decoding token L of a sequence equals row L of the prefill of length L + 1
    lengths = [1, 64, 65, 200, 777]
    Hq, Hkv, d = 4, 2, 16
    q_new = _rand(50, len(lengths), Hq, d)
    Kh = [_rand(60 + i, L + 1, Hkv, d) for i, L in enumerate(lengths)]
    Vh = [_rand(80 + i, L + 1, Hkv, d) for i, L in enumerate(lengths)]
    modes = np.array([[0, 1], [1, 0], [1, 1], [0, 1], [1, 0]], np.int8)
    for geom in (dict(n_sink=1, keep_fraction=0.2), dict(n_sink=2, window_blocks=3),
                 dict(n_sink=0, window_blocks=1)):
        O, LSE = orc.decode_attention(q_new, Kh, Vh, modes, **geom)
        for b, L in enumerate(lengths):
            Q = np.zeros((L + 1, Hq, d))
            Q[L] = q_new[b]
            full, full_lse = orc.hybrid_attention(Q, Kh[b], Vh[b], modes[b:b + 1],
                                                  np.array([0, L + 1]), **geom)
            np.testing.assert_allclose(O[b], full[L], rtol=0, atol=1e-13)
            np.testing.assert_allclose(LSE[b], full_lse[:, L], rtol=0, atol=1e-13)


def test_decode_fa_is_sdpa_over_the_history():
    L, Hq, Hkv, d = 300, 8, 2, 16
    q_new = _rand(90, 1, Hq, d)
    Kh, Vh = [_rand(91, L + 1, Hkv, d)], [_rand(92, L + 1, Hkv, d)]
    O, _ = orc.decode_attention(q_new, Kh, Vh, np.zeros((1, Hkv), np.int8))
    q = torch.from_numpy(q_new[0])[:, None]                        # [Hq, 1, d]
    k = torch.from_numpy(Kh[0]).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
    v = torch.from_numpy(Vh[0]).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v)[:, 0]
    np.testing.assert_allclose(O[0], ref.numpy(), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# Backward
# ----------------------------------------------------------------------------

def _torch_grads(Q, K, V, dO, modes, cu, geom, scale=None):
    """Reference gradients by torch autograd through an explicitly masked
    float64 softmax attention, one (sequence, head) at a time."""
    T, Hq, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    q = torch.tensor(Q, requires_grad=True)
    k = torch.tensor(K, requires_grad=True)
    v = torch.tensor(V, requires_grad=True)
    outs = []
    for b in range(len(cu) - 1):
        s0, e0 = int(cu[b]), int(cu[b + 1])
        L = e0 - s0
        if L == 0:
            continue
        ns, w = orc.sa_geometry(L, 64, geom.get("n_sink", 1), geom.get("window_blocks", 0),
                                geom.get("keep_fraction", 0.2))
        i = torch.arange(L)[:, None]
        j = torch.arange(L)[None, :]
        for hq in range(Hq):
            g = hq // G
            m = j <= i
            if modes[b, g]:
                m = m & ((j // 64 < ns) | (i // 64 - j // 64 < w))
            sc = (q[s0:e0, hq] @ k[s0:e0, g].T) * scale
            p = torch.softmax(sc.masked_fill(~m, float("-inf")), dim=-1)
            o = p @ v[s0:e0, g]
            outs.append((o * torch.from_numpy(dO[s0:e0, hq])).sum())
    torch.stack(outs).sum().backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


def test_backward_matches_autograd():
    lengths = [150, 0, 333, 64]
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    Hq, Hkv, d = 4, 2, 16
    Q, K, V, dO = _rand(100, T, Hq, d), _rand(101, T, Hkv, d), _rand(102, T, Hkv, d), _rand(103, T, Hq, d)
    modes = np.array([[0, 1], [1, 0], [1, 1], [0, 1]], np.int8)
    for geom in (dict(n_sink=1, window_blocks=2), dict(n_sink=0, window_blocks=1),
                 dict(n_sink=1, keep_fraction=0.3)):
        got = orc.hybrid_attention_backward(Q, K, V, dO, modes, cu, **geom)
        ref = _torch_grads(Q, K, V, dO, modes, cu, geom)
        for a, r in zip(got, ref):
            np.testing.assert_allclose(a, r, rtol=0, atol=1e-11)


def test_backward_rows_match_autograd_at_selected_rows():
    # the sampled-row backward against torch autograd of the masked-softmax
    # forward: ragged lengths, an empty sequence, FA and SA heads, sinks,
    # keys near a sequence end (few rows see them) and at its start (all do)
    lengths = [150, 0, 333, 64]
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    Hq, Hkv, d = 4, 2, 16
    Q, K, V, dO = _rand(140, T, Hq, d), _rand(141, T, Hkv, d), _rand(142, T, Hkv, d), _rand(143, T, Hq, d)
    modes = np.array([[0, 1], [1, 0], [1, 1], [0, 1]], np.int8)
    qt = np.array([0, 5, 149, 150, 200, 482, 483, 546])
    kt = np.array([0, 63, 64, 149, 150, 151, 300, 482, 483, 500, 546])
    for geom in (dict(n_sink=1, window_blocks=2), dict(n_sink=0, window_blocks=1),
                 dict(n_sink=1, keep_fraction=0.3)):
        dq, dk, dv = orc.hybrid_attention_backward_rows(Q, K, V, dO, modes, cu, qt, kt, chunk=37,
                                                        **geom)
        ref = _torch_grads(Q, K, V, dO, modes, cu, geom)
        np.testing.assert_allclose(dq, ref[0][qt], rtol=0, atol=1e-11)
        np.testing.assert_allclose(dk, ref[1][kt], rtol=0, atol=1e-11)
        np.testing.assert_allclose(dv, ref[2][kt], rtol=0, atol=1e-11)
    # and every row selected = the full backward
    full = orc.hybrid_attention_backward(Q, K, V, dO, modes, cu, n_sink=1, window_blocks=2)
    allt = np.arange(T)
    rows = orc.hybrid_attention_backward_rows(Q, K, V, dO, modes, cu, allt, allt, n_sink=1,
                                              window_blocks=2)
    for a, r in zip(rows, full):
        np.testing.assert_allclose(a, r, rtol=0, atol=1e-11)


def test_backward_finite_differences():
    L, Hq, Hkv, d = 70, 2, 1, 4
    cu = np.array([0, L])
    Q, K, V, dO = _rand(110, L, Hq, d), _rand(111, L, Hkv, d), _rand(112, L, Hkv, d), _rand(113, L, Hq, d)
    modes = np.array([[1]], np.int8)
    geom = dict(n_sink=0, window_blocks=1)

    def loss(Qx, Kx, Vx):
        O, _ = orc.hybrid_attention(Qx, Kx, Vx, modes, cu, **geom)
        return float((O * dO).sum())

    dQ, dK, dV = orc.hybrid_attention_backward(Q, K, V, dO, modes, cu, **geom)
    rng = np.random.default_rng(5)
    eps = 1e-6
    for arr, grad in ((Q, dQ), (K, dK), (V, dV)):
        for _ in range(6):
            ix = tuple(int(rng.integers(0, n)) for n in arr.shape)
            a = arr.copy()
            a[ix] += eps
            up = loss(*(a if x is arr else x for x in (Q, K, V)))
            a[ix] -= 2 * eps
            dn = loss(*(a if x is arr else x for x in (Q, K, V)))
            assert abs((up - dn) / (2 * eps) - grad[ix]) < 1e-6


def test_backward_invariants():
    # a constant shift of K per (sequence, head) leaves O unchanged, so the
    # keys' gradient sums to zero over the visible keys of every row:
    # sum_j dS_ij = 0, hence sum over keys of dK = scale * sum_ij dS_ij q_i = 0
    L, Hq, Hkv, d = 200, 4, 2, 8
    cu = np.array([0, L])
    Q, K, V, dO = _rand(120, L, Hq, d), _rand(121, L, Hkv, d), _rand(122, L, Hkv, d), _rand(123, L, Hq, d)
    for modes in (np.array([[0, 1]], np.int8), np.array([[1, 1]], np.int8)):
        dQ, dK, dV = orc.hybrid_attention_backward(Q, K, V, dO, modes, cu, n_sink=1,
                                                   window_blocks=1)
        np.testing.assert_allclose(dK.sum(axis=0), 0.0, atol=1e-10)
        # dV sums dO over the queries weighted by probabilities that sum to 1 per row
        np.testing.assert_allclose(dV.sum(axis=0),
                                   dO.reshape(L, Hkv, Hq // Hkv, d).sum(axis=(0, 2)), atol=1e-10)


def test_router_logit_grad_matches_autograd_through_the_ste():
    # torch autograd through y = (z + g) / tau, r_soft = softmax(y),
    # r = onehot(argmax) - r_soft.detach() + r_soft, O = r0 O_FA + r1 O_SA,
    # loss = <dO, O>
    lengths = [40, 0, 77]
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    Hq, Hkv, d = 6, 2, 8
    dO, O_fa, O_sa = _rand(130, T, Hq, d), _rand(131, T, Hq, d), _rand(132, T, Hq, d)
    z, g = _rand(133, 3, Hkv, 2), _rand(134, 3, Hkv, 2)
    tau = 0.7
    r_soft, modes = orc.gumbel_route(z, g, tau)
    dz, dr = orc.router_logit_grad(dO, O_fa, O_sa, cu, r_soft, tau)
    zt = torch.tensor(z.astype(np.float32).astype(np.float64), requires_grad=True)
    y = (zt + torch.tensor(g.astype(np.float32).astype(np.float64))) / float(np.float32(tau))
    rs = torch.softmax(y, dim=-1)
    hard = torch.nn.functional.one_hot(rs.argmax(-1), 2).double()
    r = hard - rs.detach() + rs
    loss = 0.0
    G = Hq // Hkv
    for b in range(3):
        s0, e0 = cu[b], cu[b + 1]
        for hq in range(Hq):
            rb = r[b, hq // G]
            o = rb[0] * torch.from_numpy(O_fa[s0:e0, hq]) + rb[1] * torch.from_numpy(O_sa[s0:e0, hq])
            loss = loss + (o * torch.from_numpy(dO[s0:e0, hq])).sum()
    loss.backward()
    # the oracle rounds y = (z + g) / tau to float32 (the precision the hard
    # decision is taken in); autograd runs in float64: 2^-24 relative apart
    np.testing.assert_allclose(dz, zt.grad.numpy(), rtol=1e-6, atol=1e-9)
    # dr itself: an empty sequence has none; dz sums to zero over the two modes
    assert np.all(dr[1] == 0)
    np.testing.assert_allclose(dz.sum(-1), 0.0, atol=1e-12)
