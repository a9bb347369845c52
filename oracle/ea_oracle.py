"""Plain CPU oracle for the head-routed hybrid attention prefill of Elastic Attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU
baseline leg may import this module.  The product path (the HIP library and its
Python binding) never does, and shares no code, header, table or helper with it.

What is computed, and where the pages define it:

* Boundary pooling of the Key states over the first and last ``pool_len``
  (= 100) tokens of a sequence, per KV head -> x'_K in R^{H x d'}
  ("Elastic Attention: Test-time Adaptive Sparsity Ratios for Efficient
  Transformers", router paragraph on Fig. 3(c) and the boundary-pooling
  paragraph of the implementation details; "Technical Summary: Elastic
  Attention", Sec. 2.1).
* Task MLP then router MLP -> logits z in R^{H x 2} (same passages).
* Hard routing r_hard = argmax over the two columns, 0 = FA, 1 = SA (router
  paragraph on Fig. 3(b) and the Gumbel-Softmax paragraph: inference uses
  hard decisions).
* Backward: gradients of the layer output with respect to Q, K and V, every
  head in its routed mode (the chain rule through the FA / SA equations).
* Decode: the newest token of each sequence attends to its history with the
  same visibility as the last row of the prefill of that longer sequence.
* Training-time routing: r_soft = Gumbel-Softmax of z (softmax over the two
  modes of (z + g) / tau, g standard Gumbel noise, tau the annealed
  temperature), r_hard = argmax of r_soft, and the straight-through estimator
  r = r_hard - sg(r_soft) + r_soft whose forward value is r_hard (the
  Gumbel-Softmax and STE paragraphs of the method section; "Technical
  Summary: Elastic Attention", Sec. 2.2).  The training forward computes each
  head in both modes and mixes the two outputs with r (dual-mode forward).
* Per KV head either full causal attention (FA equation of the preliminaries)
  or sparse attention over a retained subset of K/V (SA equation); query heads
  share their group's K/V and mode (GQA footnote of the hybrid-head equation);
  head outputs are concatenated along features (router paragraph, Fig. 3(b)).

Readings where the pages are silent (the display equations did not survive):
the softmax scale is 1/sqrt(d); attention is causal; the pooling operator is
the arithmetic mean over the union of the boundary rows; the MLP activation is
the exact (erf) GELU; one router is shared by all KV heads of a layer; an
argmax tie goes to FA; the sparse pattern is static: ``n_sink`` attention-sink
blocks plus a causal local window of ``w`` blocks of 64 tokens, sized so that
sinks + window keep ``round(rho * N)`` of the N key blocks.

Every function is written for clarity, not speed: float64 throughout, a
two-pass softmax over explicitly masked score rows, no tiling, no online
rescaling, no fusion.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf

# ----------------------------------------------------------------------------
# Router
# ----------------------------------------------------------------------------


def boundary_rows(L: int, pool_len: int) -> np.ndarray:
    """Sequence-local indices pooled for a sequence of length L: the first
    ``pool_len`` and the last ``pool_len`` tokens, as a set (a token in both
    ranges counts once)."""
    head = np.arange(min(pool_len, L))
    tail = np.arange(max(0, L - pool_len), L)
    return np.union1d(head, tail)


def boundary_pool(K: np.ndarray, cu_seqlens: np.ndarray, pool_len: int = 100) -> np.ndarray:
    """x'_K[b, g, :] = mean of K over the boundary rows of sequence b, KV head g.

    K: [T, Hkv, d] (any float dtype).  Returns float64 [B, Hkv, d]; a sequence
    of length 0 pools to zeros."""
    B = len(cu_seqlens) - 1
    T, Hkv, d = K.shape
    out = np.zeros((B, Hkv, d), dtype=np.float64)
    for b in range(B):
        s, e = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        L = e - s
        if L <= 0:
            continue
        idx = s + boundary_rows(L, pool_len)
        out[b] = K[idx].astype(np.float64).sum(axis=0) / len(idx)
    return out


def gelu(x: np.ndarray) -> np.ndarray:
    """GELU(x) = x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)), float64."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def linear(x: np.ndarray, W: np.ndarray, b: np.ndarray) -> np.ndarray:
    """y = x W^T + b with W in [out, in] layout, float64."""
    return np.asarray(x, np.float64) @ np.asarray(W, np.float64).T + np.asarray(b, np.float64)


def router_logits(xp: np.ndarray, w: dict) -> np.ndarray:
    """Task MLP then router MLP, row-wise over the last axis.

    t = W2 GELU(W1 x' + b1) + b2;  z = W4 GELU(W3 t + b3) + b4."""
    t = linear(gelu(linear(xp, w["w1"], w["b1"])), w["w2"], w["b2"])
    return linear(gelu(linear(t, w["w3"], w["b3"])), w["w4"], w["b4"])


def route(K: np.ndarray, cu_seqlens: np.ndarray, w: dict, pool_len: int = 100):
    """Hard FA/SA decision per (sequence, KV head).

    Returns (modes int8 [B, Hkv] with 0 = FA and 1 = SA, logits float64
    [B, Hkv, 2]).  A tie goes to FA.  An empty sequence gets mode 0 and zero
    logits."""
    xp = boundary_pool(K, cu_seqlens, pool_len)
    z = router_logits(xp, w)
    lengths = np.diff(np.asarray(cu_seqlens, dtype=np.int64))
    z[lengths == 0] = 0.0
    modes = (z[..., 1] > z[..., 0]).astype(np.int8)
    return modes, z


def router_param_count(d: int, task_hidden: int, router_hidden: int) -> int:
    """Parameters of the two MLPs (weights and biases)."""
    return (task_hidden * d + task_hidden) + (d * task_hidden + d) + \
        (router_hidden * d + router_hidden) + (2 * router_hidden + 2)


# ----------------------------------------------------------------------------
# Sparse-attention geometry and visibility
# ----------------------------------------------------------------------------


def sa_geometry(L: int, block: int, n_sink: int, window_blocks: int, keep_fraction: float):
    """(n_sink, w) for a sequence of length L.

    N = ceil(L / block) key blocks.  With an explicit ``window_blocks`` > 0 the
    window is that; otherwise the retained block count is
    keep = max(n_sink + 1, floor(rho * N + 1/2)) with rho the float32 value of
    ``keep_fraction`` evaluated in double, and w = keep - n_sink."""
    N = -(-int(L) // int(block))
    if window_blocks > 0:
        return int(n_sink), int(window_blocks)
    rho = float(np.float32(keep_fraction))
    keep = max(int(n_sink) + 1, int(math.floor(rho * N + 0.5)))
    return int(n_sink), int(keep - n_sink)


def visible(i, j, mode: int, n_sink: int, w: int, block: int):
    """Whether sequence-local query i may attend to key j.

    FA: causal (j <= i).  SA: causal and (key block is a sink block, or the
    query's block is fewer than w blocks after the key's block)."""
    i = np.asarray(i)
    j = np.asarray(j)
    causal = j <= i
    if mode == 0:
        return causal
    qb = i // block
    kb = j // block
    return causal & ((kb < n_sink) | ((qb - kb) < w))


# ----------------------------------------------------------------------------
# Attention
# ----------------------------------------------------------------------------


def _attend(q, pos, Kseq, Vseq, mode, n_sink, w, block, scale, return_weights=False):
    """Two-pass softmax attention of query rows ``q`` [n, d] at sequence
    positions ``pos`` [n] over one sequence's keys/values [L, d]; float64."""
    q = np.asarray(q, np.float64)
    jmax = int(pos.max()) + 1
    Kc = np.asarray(Kseq[:jmax], np.float64)
    Vc = np.asarray(Vseq[:jmax], np.float64)
    s = (q @ Kc.T) * scale
    mask = visible(pos[:, None], np.arange(jmax)[None, :], mode, n_sink, w, block)
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ Vc) / l
    lse = (m + np.log(l))[:, 0]
    if return_weights:
        return o, lse, p / l
    return o, lse


def _scale(d, softmax_scale):
    return 1.0 / math.sqrt(d) if not softmax_scale else float(np.float32(softmax_scale))


def hybrid_attention(Q, K, V, modes, cu_seqlens, *, block=64, n_sink=1, window_blocks=0,
                     keep_fraction=0.2, softmax_scale=0.0, chunk=512):
    """Full output of the hybrid layer.

    Q [T, Hq, d], K/V [T, Hkv, d] (values as float32 or float64), modes int8
    [B, Hkv].  Query head hq reads KV head hq // (Hq / Hkv) and that head's
    mode.  Returns (O float64 [T, Hq, d], LSE float64 [Hq, T]) with natural-log
    LSE = m + ln(sum exp(s - m))."""
    T, Hq, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    scale = _scale(d, softmax_scale)
    O = np.zeros((T, Hq, d), dtype=np.float64)
    LSE = np.zeros((Hq, T), dtype=np.float64)
    for b in range(len(cu_seqlens) - 1):
        s0, e0 = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        L = e0 - s0
        if L <= 0:
            continue
        ns, w = sa_geometry(L, block, n_sink, window_blocks, keep_fraction)
        for hq in range(Hq):
            g = hq // G
            mode = int(modes[b, g])
            for r0 in range(0, L, chunk):
                r1 = min(L, r0 + chunk)
                pos = np.arange(r0, r1)
                o, lse = _attend(Q[s0 + r0:s0 + r1, hq], pos, K[s0:e0, g], V[s0:e0, g], mode,
                                 ns, w, block, scale)
                O[s0 + r0:s0 + r1, hq] = o
                LSE[hq, s0 + r0:s0 + r1] = lse
    return O, LSE


def hybrid_attention_rows(Q, K, V, modes, cu_seqlens, tokens, heads, *, block=64, n_sink=1,
                          window_blocks=0, keep_fraction=0.2, softmax_scale=0.0):
    """The same output at selected global token indices and query heads only.

    Returns (O float64 [len(tokens), len(heads), d], LSE float64
    [len(tokens), len(heads)])."""
    T, Hq, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    scale = _scale(d, softmax_scale)
    tokens = np.asarray(tokens, dtype=np.int64)
    seg = np.searchsorted(np.asarray(cu_seqlens, np.int64), tokens, side="right") - 1
    O = np.zeros((len(tokens), len(heads), d), dtype=np.float64)
    LSE = np.zeros((len(tokens), len(heads)), dtype=np.float64)
    for b in np.unique(seg):
        s0, e0 = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        L = e0 - s0
        ns, w = sa_geometry(L, block, n_sink, window_blocks, keep_fraction)
        sel = np.nonzero(seg == b)[0]
        pos = tokens[sel] - s0
        for hi, hq in enumerate(heads):
            g = hq // G
            o, lse = _attend(Q[tokens[sel], hq], pos, K[s0:e0, g], V[s0:e0, g], int(modes[b, g]),
                             ns, w, block, scale)
            O[sel, hi] = o
            LSE[sel, hi] = lse
    return O, LSE


def attention_weights(Q, K, modes, L, hq, *, G, block=64, n_sink=1, window_blocks=0,
                      keep_fraction=0.2, softmax_scale=0.0):
    """The L x L row-stochastic weight matrix of query head hq for a single
    sequence of length L starting at token 0 (small cases only)."""
    d = Q.shape[2]
    g = hq // G
    ns, w = sa_geometry(L, block, n_sink, window_blocks, keep_fraction)
    Vdummy = np.zeros((L, 1))
    _, _, P = _attend(Q[:L, hq], np.arange(L), K[:L, g], Vdummy, int(modes[0, g]), ns, w, block,
                      _scale(d, softmax_scale), return_weights=True)
    return P


# ----------------------------------------------------------------------------
# Backward of the hybrid layer
# ----------------------------------------------------------------------------


def hybrid_attention_backward(Q, K, V, dO, modes, cu_seqlens, *, block=64, n_sink=1,
                              window_blocks=0, keep_fraction=0.2, softmax_scale=0.0):
    """Gradients of the hybrid layer's output O with respect to Q, K and V for
    an upstream gradient dO, every head in its routed mode (the FA or SA
    equation; a head's K/V are shared by its G query heads).

    Per head, with S = scale Q K^T over the visible pairs (others -inf),
    P = softmax(S) row-wise and O = P V, the chain rule gives
    dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(P * dP)), dQ = scale dS K,
    dK = scale dS^T Q; rowsum(P * dP) = rowsum(dO * O).  dK and dV of a KV head
    sum over its query heads.  Returns (dQ [T, Hq, d], dK, dV [T, Hkv, d]),
    float64."""
    T, Hq, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    scale = _scale(d, softmax_scale)
    dQ = np.zeros((T, Hq, d), dtype=np.float64)
    dK = np.zeros((T, Hkv, d), dtype=np.float64)
    dV = np.zeros((T, Hkv, d), dtype=np.float64)
    for b in range(len(cu_seqlens) - 1):
        s0, e0 = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        L = e0 - s0
        if L <= 0:
            continue
        ns, w = sa_geometry(L, block, n_sink, window_blocks, keep_fraction)
        idx = np.arange(L)
        for hq in range(Hq):
            g = hq // G
            mask = visible(idx[:, None], idx[None, :], int(modes[b, g]), ns, w, block)
            q = np.asarray(Q[s0:e0, hq], np.float64)
            k = np.asarray(K[s0:e0, g], np.float64)
            v = np.asarray(V[s0:e0, g], np.float64)
            do = np.asarray(dO[s0:e0, hq], np.float64)
            s = np.where(mask, (q @ k.T) * scale, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            dp = do @ v.T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dQ[s0:e0, hq] = scale * (ds @ k)
            dK[s0:e0, g] += scale * (ds.T @ q)
            dV[s0:e0, g] += p.T @ do
    return dQ, dK, dV


def _row_grad_stats(q, do, pos, Kseq, Vseq, mode, n_sink, w, block, scale):
    """For query rows ``q``/``do`` [n, d] at sequence positions ``pos``, over
    their whole visible key set: the probabilities P [n, jmax], dP = dO V^T
    and D = rowsum(P * dP) (= rowsum(dO * O)); float64, two-pass softmax."""
    jmax = int(pos.max()) + 1
    Kc = np.asarray(Kseq[:jmax], np.float64)
    Vc = np.asarray(Vseq[:jmax], np.float64)
    s = (np.asarray(q, np.float64) @ Kc.T) * scale
    mask = visible(pos[:, None], np.arange(jmax)[None, :], mode, n_sink, w, block)
    s = np.where(mask, s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    dp = np.asarray(do, np.float64) @ Vc.T
    D = (p * dp).sum(axis=1, keepdims=True)
    return p, dp, D


def hybrid_attention_backward_rows(Q, K, V, dO, modes, cu_seqlens, q_tokens, k_tokens, *,
                                   block=64, n_sink=1, window_blocks=0, keep_fraction=0.2,
                                   softmax_scale=0.0, chunk=64):
    """hybrid_attention_backward at selected rows only.

    dQ at the global token indices ``q_tokens`` (every query head), and dK, dV
    at the global token indices ``k_tokens`` (every KV head).  Same chain rule:
    for a query row i, dQ_i = scale sum_j P_ij (dP_ij - D_i) k_j over its
    visible keys; for a key j of KV head g, dV_j = sum over the group's query
    heads and the rows i that see j of P_ij dO_i, and dK_j = scale sum of
    P_ij (dP_ij - D_i) q_i.  Each row's P and D come from its full visible
    key set, so the cost is that of the rows involved.  Returns (dQ
    [len(q_tokens), Hq, d], dK, dV [len(k_tokens), Hkv, d]), float64."""
    T, Hq, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    scale = _scale(d, softmax_scale)
    cu = np.asarray(cu_seqlens, np.int64)
    q_tokens = np.asarray(q_tokens, np.int64)
    k_tokens = np.asarray(k_tokens, np.int64)
    dQ = np.zeros((len(q_tokens), Hq, d), dtype=np.float64)
    dK = np.zeros((len(k_tokens), Hkv, d), dtype=np.float64)
    dV = np.zeros((len(k_tokens), Hkv, d), dtype=np.float64)
    qseg = np.searchsorted(cu, q_tokens, side="right") - 1
    kseg = np.searchsorted(cu, k_tokens, side="right") - 1
    for b in np.unique(np.concatenate([qseg, kseg])):
        s0, e0 = int(cu[b]), int(cu[b + 1])
        L = e0 - s0
        ns, w = sa_geometry(L, block, n_sink, window_blocks, keep_fraction)
        qsel = np.nonzero(qseg == b)[0]
        ksel = np.nonzero(kseg == b)[0]
        kpos = k_tokens[ksel] - s0
        for hq in range(Hq):
            g = hq // G
            mode = int(modes[b, g])
            Kb, Vb = K[s0:e0, g], V[s0:e0, g]
            if len(qsel):
                pos = q_tokens[qsel] - s0
                p, dp, D = _row_grad_stats(Q[q_tokens[qsel], hq], dO[q_tokens[qsel], hq], pos, Kb,
                                           Vb, mode, ns, w, block, scale)
                dQ[qsel, hq] = scale * ((p * (dp - D)) @ np.asarray(Kb[:p.shape[1]], np.float64))
            if len(ksel):
                # rows that see at least one selected key
                i_all = np.arange(int(kpos.min()), L)
                sees = visible(i_all[:, None], kpos[None, :], mode, ns, w, block).any(axis=1)
                rows = i_all[sees]
                for r0 in range(0, len(rows), chunk):
                    pos = rows[r0:r0 + chunk]
                    p, dp, D = _row_grad_stats(Q[s0 + pos, hq], dO[s0 + pos, hq], pos, Kb, Vb, mode,
                                               ns, w, block, scale)
                    cols = np.minimum(kpos, p.shape[1] - 1)
                    inside = kpos < p.shape[1]
                    pk = np.where(inside[None, :], p[:, cols], 0.0)          # [rows, keys]
                    dsk = pk * (np.where(inside[None, :], dp[:, cols], 0.0) - D)
                    dV[ksel, g] += pk.T @ np.asarray(dO[s0 + pos, hq], np.float64)
                    dK[ksel, g] += scale * (dsk.T @ np.asarray(Q[s0 + pos, hq], np.float64))
    return dQ, dK, dV


# ----------------------------------------------------------------------------
# Decode: one new token per sequence
# ----------------------------------------------------------------------------


def decode_attention(q_new, K_hist, V_hist, modes, *, block=64, n_sink=1, window_blocks=0,
                     keep_fraction=0.2, softmax_scale=0.0):
    """Attention of each sequence's newest token over its whole history.

    q_new [B, Hq, d]; K_hist[b], V_hist[b] [L_b + 1, Hkv, d] hold the keys and
    values of positions 0..L_b, the last row being the new token's.  The query
    at position L_b sees keys as the last row of a sequence of length L_b + 1
    in the prefill (FA and SA equations; the SA window is that of length
    L_b + 1).  Returns (O float64 [B, Hq, d], LSE float64 [B, Hq])."""
    B, Hq, d = q_new.shape
    Hkv = K_hist[0].shape[1]
    G = Hq // Hkv
    scale = _scale(d, softmax_scale)
    O = np.zeros((B, Hq, d), dtype=np.float64)
    LSE = np.zeros((B, Hq), dtype=np.float64)
    for b in range(B):
        n = K_hist[b].shape[0]
        ns, w = sa_geometry(n, block, n_sink, window_blocks, keep_fraction)
        pos = np.array([n - 1])
        for hq in range(Hq):
            g = hq // G
            o, lse = _attend(q_new[b, hq][None], pos, K_hist[b][:, g], V_hist[b][:, g],
                             int(modes[b, g]), ns, w, block, scale)
            O[b, hq] = o[0]
            LSE[b, hq] = lse[0]
    return O, LSE


# ----------------------------------------------------------------------------
# Training forward: Gumbel-Softmax routing with straight-through hard decisions,
# and the dual-mode attention it mixes
# ----------------------------------------------------------------------------


def gumbel_route(z, g, tau: float):
    """Routing of the training forward for logits z [..., 2] and noise g [..., 2].

    y = (z + g) / tau, taken in float32 as the library takes it, so that the
    hard decision is made in one precision on both sides; r_soft = softmax(y)
    over the last axis (float64 from the float32 y); r_hard = argmax of r_soft,
    which is the argmax of y (softmax is monotone), a tie going to FA (index 0).
    Returns (r_soft float64 [..., 2], modes int8 [...])."""
    z32 = np.asarray(z, dtype=np.float32)
    g32 = np.zeros_like(z32) if g is None else np.asarray(g, dtype=np.float32)
    y = (z32 + g32) / np.float32(tau)
    y64 = y.astype(np.float64)
    e = np.exp(y64 - y64.max(axis=-1, keepdims=True))
    r_soft = e / e.sum(axis=-1, keepdims=True)
    modes = (y[..., 1] > y[..., 0]).astype(np.int8)
    return r_soft, modes


def ste_weights(r_soft, modes):
    """Straight-through mixing weights r = r_hard - sg(r_soft) + r_soft, as
    their forward values (the stop-gradient is the identity in a forward
    pass), float64 [..., 2]; r_hard is the one-hot of ``modes``."""
    r_hard = np.stack([1 - np.asarray(modes), np.asarray(modes)], axis=-1).astype(np.float64)
    return r_hard - r_soft + r_soft


def dual_attention(Q, K, V, cu_seqlens, r_soft, modes, *, block=64, n_sink=1, window_blocks=0,
                   keep_fraction=0.2, softmax_scale=0.0):
    """Dual-mode training forward of one layer: every query head in both modes.

    O_FA = the FA output of every head, O_SA = the SA output of every head (the
    FA and SA equations, all heads), and the layer output mixes them per
    (sequence, KV head) with the straight-through weights of ``r_soft`` and
    ``modes``: O = r[0] O_FA + r[1] O_SA.  Returns (O, O_FA, O_SA, LSE_FA,
    LSE_SA), float64, O's [T, Hq, d] and LSE's [Hq, T]."""
    B = len(cu_seqlens) - 1
    Hkv = K.shape[1]
    geom = dict(block=block, n_sink=n_sink, window_blocks=window_blocks,
                keep_fraction=keep_fraction, softmax_scale=softmax_scale)
    O_fa, L_fa = hybrid_attention(Q, K, V, np.zeros((B, Hkv), np.int8), cu_seqlens, **geom)
    O_sa, L_sa = hybrid_attention(Q, K, V, np.ones((B, Hkv), np.int8), cu_seqlens, **geom)
    O = _mix(O_fa, O_sa, cu_seqlens, ste_weights(r_soft, modes))
    return O, O_fa, O_sa, L_fa, L_sa


def _mix(O_fa, O_sa, cu_seqlens, r):
    T, Hq, _ = O_fa.shape
    G = Hq // r.shape[1]
    O = np.zeros_like(O_fa)
    for b in range(len(cu_seqlens) - 1):
        s0, e0 = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        for hq in range(Hq):
            rb = r[b, hq // G]
            O[s0:e0, hq] = rb[0] * O_fa[s0:e0, hq] + rb[1] * O_sa[s0:e0, hq]
    return O


def router_logit_grad(dO, O_fa, O_sa, cu_seqlens, r_soft, tau: float):
    """Gradient of the loss with respect to the routing logits z through the
    straight-through estimator, for the upstream gradient dO of the mixed
    output O = r[0] O_FA + r[1] O_SA.

    The STE passes the gradient of r straight to r_soft: dr[b, g, m] =
    sum over the tokens of sequence b and the query heads of KV head g of
    <dO, O_m>.  Through r_soft = softmax((z + g) / tau):
    dz = r_soft * (dr - <dr, r_soft>) / tau.  Returns (dz, dr) float64
    [B, Hkv, 2]."""
    T, Hq, d = dO.shape
    B = len(cu_seqlens) - 1
    Hkv = r_soft.shape[1]
    G = Hq // Hkv
    dr = np.zeros((B, Hkv, 2), dtype=np.float64)
    for b in range(B):
        s0, e0 = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        for hq in range(Hq):
            g = hq // G
            do = np.asarray(dO[s0:e0, hq], np.float64)
            dr[b, g, 0] += float((do * np.asarray(O_fa[s0:e0, hq], np.float64)).sum())
            dr[b, g, 1] += float((do * np.asarray(O_sa[s0:e0, hq], np.float64)).sum())
    rs = np.asarray(r_soft, np.float64)
    dz = rs * (dr - (dr * rs).sum(axis=-1, keepdims=True)) / float(np.float32(tau))
    return dz, dr


def dual_attention_rows(Q, K, V, cu_seqlens, r_soft, modes, tokens, heads, *, block=64, n_sink=1,
                        window_blocks=0, keep_fraction=0.2, softmax_scale=0.0):
    """dual_attention at selected global token indices and query heads only.

    Returns (O, O_FA, O_SA) float64 [len(tokens), len(heads), d] and (LSE_FA,
    LSE_SA) float64 [len(tokens), len(heads)]."""
    B = len(cu_seqlens) - 1
    Hkv = K.shape[1]
    G = Q.shape[1] // Hkv
    geom = dict(block=block, n_sink=n_sink, window_blocks=window_blocks,
                keep_fraction=keep_fraction, softmax_scale=softmax_scale)
    O_fa, L_fa = hybrid_attention_rows(Q, K, V, np.zeros((B, Hkv), np.int8), cu_seqlens, tokens,
                                       heads, **geom)
    O_sa, L_sa = hybrid_attention_rows(Q, K, V, np.ones((B, Hkv), np.int8), cu_seqlens, tokens,
                                       heads, **geom)
    tokens = np.asarray(tokens, dtype=np.int64)
    seg = np.searchsorted(np.asarray(cu_seqlens, np.int64), tokens, side="right") - 1
    r = ste_weights(r_soft, modes)
    O = np.zeros_like(O_fa)
    for ti, b in enumerate(seg):
        for hi, hq in enumerate(heads):
            rb = r[b, hq // G]
            O[ti, hi] = rb[0] * O_fa[ti, hi] + rb[1] * O_sa[ti, hi]
    return O, O_fa, O_sa, L_fa, L_sa


# ----------------------------------------------------------------------------
# Effective FLOPs
# ----------------------------------------------------------------------------


def effective_flops(modes, cu_seqlens, Hq, Hkv, d, *, block=64, n_sink=1, window_blocks=0,
                    keep_fraction=0.2) -> int:
    """4 d * sum over query heads and visible (query block, key block) pairs of
    rows(qb) * cols(kb); a pair is visible when any (i, j) in it is visible, and
    a partly visible (diagonal or window-edge) pair counts in full."""
    G = Hq // Hkv
    total = 0
    for b in range(len(cu_seqlens) - 1):
        L = int(cu_seqlens[b + 1]) - int(cu_seqlens[b])
        if L <= 0:
            continue
        ns, w = sa_geometry(L, block, n_sink, window_blocks, keep_fraction)
        N = -(-L // block)
        size = np.minimum(block, L - block * np.arange(N))
        for g in range(Hkv):
            mode = int(modes[b, g])
            acc = 0
            for qb in range(N):
                kb = np.arange(qb + 1)
                # block-level visibility: the last row of the query block sees key
                # block kb's first key iff some pair of the two blocks is visible
                ok = visible(qb * block + size[qb] - 1, kb * block, mode, ns, w, block)
                acc += int(size[qb]) * int(size[kb][ok].sum())
            total += G * acc
    return 4 * d * total
