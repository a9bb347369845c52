"""Plain CPU oracle for the XAttention (XA) head mode of the hybrid layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU
baseline leg may import this module.  The product path (the HIP library and its
Python binding) never does, and shares no code, header, table or helper with it.

Where it comes from.  "Elastic Attention: Test-time Adaptive Sparsity Ratios for
Efficient Transformers" (experimental setup, baselines paragraph) runs the
sparse or the retrieval heads in XAttention mode with threshold tau = 0.9 and
XAttention's other hyperparameters at their defaults, and names head
configurations "{retrieval-head mode}-{sparse-head mode}" (FA-SSA, FA-XA,
XA-SSA); its efficiency summary quotes the largest prefill speedup for XA-SSA.
The pages do not define XAttention itself; its steps are restated here from
its own paper, "XAttention: Block Sparse Attention with Antidiagonal Scoring"
(Xu et al., 2025), method section (antidiagonal scoring, then threshold block
selection), with its default block size 128 and stride 8:

1. Antidiagonal score.  Cut the query and key positions of one head into
   groups of S (the stride).  The score of query group a against key group c
   is the sum over the antidiagonal of that S x S tile of Q K^T:
   sum_{t=0..S-1} <q[aS + S-1-t], k[cS + t]>.
2. Normalise.  Scale by 1/sqrt(d) and by 1/S (the mean of the S terms), mask
   key groups after the query group (causal at group level, the diagonal group
   kept), and take a softmax over each group row.
3. Block mass.  Sum the normalised group scores inside each block x block
   tile: A[i, j] for query block i and key block j (B/S group rows and
   columns per tile).
4. Threshold selection.  For query block i, keep the smallest set of key
   blocks j <= i whose mass reaches tau times the row's total, taking blocks
   in decreasing mass.

Readings where neither text fixes a detail (each listed in the design notes):

* Positions past the sequence end inside the last group read as zero vectors
  (they add nothing to an antidiagonal sum); a group row or column exists for
  every group holding at least one real position.
* The first key block (the attention-sink block) and the diagonal block are
  always kept and count toward the mass; the rest is taken greedily in
  decreasing mass, ties to the lower block index, until the kept mass is at
  least tau * total.
* GQA: the selection is made per query head, each against its group's keys.
* Attention of an XA head is then causal softmax attention over the keys of
  its kept blocks (the diagonal block causally masked); float64, two-pass.

Everything is float64 and written for clarity: one strided product per
antidiagonal offset, explicit masks, a two-pass softmax, a Python loop for the
greedy selection.
"""
from __future__ import annotations

import math

import numpy as np

from .ea_oracle import sa_geometry, visible

# Head configurations: computation mode of router mode 0 (retrieval head) and
# router mode 1 (sparse head).  0 = FA, 1 = SA (sink + local window), 2 = XA.
HEAD_CONFIGS = {
    "FA-SSA": (0, 1),
    "FA-XA": (0, 2),
    "XA-SSA": (2, 1),
}
MODE_FA, MODE_SA, MODE_XA = 0, 1, 2


def computation_modes(modes, config: str) -> np.ndarray:
    """Per (sequence, KV head) computation mode of a router decision array."""
    table = np.asarray(HEAD_CONFIGS[config], dtype=np.int64)
    return table[np.asarray(modes, dtype=np.int64)]


def antidiagonal_scores(q: np.ndarray, k: np.ndarray, stride: int) -> np.ndarray:
    """Step 1 for one query head: q [L, d], k [L, d] -> D [n, n] with
    n = ceil(L / S) and D[a, c] = sum_t <q[aS + S-1-t], k[cS + t]>, positions
    at or past L reading as zero."""
    L, d = q.shape
    S = int(stride)
    n = -(-L // S)
    qp = np.zeros((n * S, d))
    kp = np.zeros((n * S, d))
    qp[:L] = q
    kp[:L] = k
    D = np.zeros((n, n))
    for t in range(S):
        # rows aS + (S-1-t) of q against rows cS + t of k, for every a and c
        D += qp[S - 1 - t::S] @ kp[t::S].T
    return D


def block_mass(q: np.ndarray, k: np.ndarray, *, block: int = 128, stride: int = 8,
               scale: float | None = None) -> np.ndarray:
    """Steps 2 and 3 for one query head of one sequence: A [nb, nb] with
    nb = ceil(L / block); A[i, j] = 0 for j > i.  Row i sums to the number of
    group rows in query block i."""
    L, d = q.shape
    S = int(stride)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    D = antidiagonal_scores(np.asarray(q, np.float64), np.asarray(k, np.float64), S)
    n = D.shape[0]
    logits = D * (scale / S)
    a = np.arange(n)
    logits = np.where(a[None, :] <= a[:, None], logits, -np.inf)
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    p /= p.sum(axis=1, keepdims=True)
    R = block // S
    nb = -(-L // block)
    A = np.zeros((nb, nb))
    for i in range(nb):
        for j in range(i + 1):
            A[i, j] = p[i * R:(i + 1) * R, j * R:(j + 1) * R].sum()
    return A


def block_mass_rows(q: np.ndarray, k: np.ndarray, rows, *, block: int = 128, stride: int = 8,
                    scale: float | None = None) -> np.ndarray:
    """Rows ``rows`` (query blocks) of ``block_mass`` without forming the whole
    group score matrix: the same three steps restricted to the group rows of
    those blocks.  Returns [len(rows), nb]."""
    L, d = q.shape
    S = int(stride)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    n = -(-L // S)
    nb = -(-L // block)
    R = block // S
    qp = np.zeros((n * S, d))
    kp = np.zeros((n * S, d))
    qp[:L] = np.asarray(q, np.float64)
    kp[:L] = np.asarray(k, np.float64)
    out = np.zeros((len(rows), nb))
    for ri, i in enumerate(rows):
        a = np.arange(i * R, min((i + 1) * R, n))
        D = np.zeros((len(a), n))
        for t in range(S):
            D += qp[a * S + S - 1 - t] @ kp[t::S].T
        logits = np.where(np.arange(n)[None, :] <= a[:, None], D * (scale / S), -np.inf)
        p = np.exp(logits - logits.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        for j in range(i + 1):
            out[ri, j] = p[:, j * R:(j + 1) * R].sum()
    return out


def select_row(mass_row: np.ndarray, i: int, tau: float) -> np.ndarray:
    """Step 4 for query block i: bool [i + 1] of kept key blocks."""
    a = np.asarray(mass_row[:i + 1], np.float64)
    keep = np.zeros(i + 1, dtype=bool)
    keep[0] = True
    keep[i] = True
    target = float(tau) * a.sum()
    got = a[keep].sum()
    for j in sorted(range(1, i), key=lambda x: (-a[x], x)):
        if got >= target:
            break
        keep[j] = True
        got += a[j]
    return keep


def select(A: np.ndarray, tau: float) -> np.ndarray:
    """Step 4 for every query block of one head: bool [nb, nb] (lower
    triangular)."""
    nb = A.shape[0]
    sel = np.zeros((nb, nb), dtype=bool)
    for i in range(nb):
        sel[i, :i + 1] = select_row(A[i], i, tau)
    return sel


def xa_plan(Q, K, cmodes, cu_seqlens, *, block=128, stride=8, tau=0.9, softmax_scale=0.0):
    """Block masses and selections of every XA query head.

    ``cmodes`` [B, Hkv] are computation modes (2 = XA).  Returns a dict
    (b, hq) -> (A [nb, nb], sel [nb, nb]) over the XA heads only."""
    T, Hq, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d) if not softmax_scale else float(np.float32(softmax_scale))
    out = {}
    for b in range(len(cu_seqlens) - 1):
        s0, e0 = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        if e0 <= s0:
            continue
        for hq in range(Hq):
            g = hq // G
            if int(cmodes[b, g]) != MODE_XA:
                continue
            A = block_mass(Q[s0:e0, hq], K[s0:e0, g], block=block, stride=stride, scale=scale)
            out[(b, hq)] = (A, select(A, tau))
    return out


def xa_visible(i, j, sel: np.ndarray, block: int):
    """Whether sequence-local query i sees key j under a selection."""
    i = np.asarray(i)
    j = np.asarray(j)
    return (j <= i) & sel[i // block, j // block]


def hybrid_attention_xa(Q, K, V, cmodes, cu_seqlens, plan, *, block=64, n_sink=1,
                        window_blocks=0, keep_fraction=0.2, softmax_scale=0.0, xa_block=128,
                        tokens=None, heads=None):
    """Output of the layer with FA, SA and XA heads (computation modes
    ``cmodes``), XA heads following the selections in ``plan`` (from
    ``xa_plan``).  With ``tokens`` / ``heads`` given, only those global token
    indices and query heads are computed.

    Returns (O float64 [n_tok, n_heads, d], LSE float64 [n_tok, n_heads])."""
    T, Hq, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d) if not softmax_scale else float(np.float32(softmax_scale))
    tokens = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    heads = list(range(Hq)) if heads is None else list(heads)
    seg = np.searchsorted(np.asarray(cu_seqlens, np.int64), tokens, side="right") - 1
    O = np.zeros((len(tokens), len(heads), d))
    LSE = np.zeros((len(tokens), len(heads)))
    for b in np.unique(seg):
        s0, e0 = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        L = e0 - s0
        ns, w = sa_geometry(L, block, n_sink, window_blocks, keep_fraction)
        rows = np.nonzero(seg == b)[0]
        pos = tokens[rows] - s0
        for hi, hq in enumerate(heads):
            g = hq // G
            mode = int(cmodes[b, g])
            jmax = int(pos.max()) + 1
            jj = np.arange(jmax)[None, :]
            if mode == MODE_XA:
                mask = xa_visible(pos[:, None], jj, plan[(b, hq)][1], xa_block)
            else:
                mask = visible(pos[:, None], jj, mode, ns, w, block)
            s = (np.asarray(Q[tokens[rows], hq], np.float64)
                 @ np.asarray(K[s0:s0 + jmax, g], np.float64).T) * scale
            s = np.where(mask, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            l = p.sum(axis=1, keepdims=True)
            O[rows, hi] = (p @ np.asarray(V[s0:s0 + jmax, g], np.float64)) / l
            LSE[rows, hi] = (m + np.log(l))[:, 0]
    return O, LSE


def xa_effective_flops(cmodes, cu_seqlens, Hq, Hkv, d, plan, *, block=64, n_sink=1,
                       window_blocks=0, keep_fraction=0.2, xa_block=128) -> int:
    """4 d * sum over query heads of visible (64-query block, 64-key block)
    pairs of rows * cols, partly visible pairs counted in full; an XA head's
    pair is visible when its 128-blocks are selected and it is causal."""
    G = Hq // Hkv
    total = 0
    for b in range(len(cu_seqlens) - 1):
        L = int(cu_seqlens[b + 1]) - int(cu_seqlens[b])
        if L <= 0:
            continue
        ns, w = sa_geometry(L, block, n_sink, window_blocks, keep_fraction)
        N = -(-L // block)
        size = np.minimum(block, L - block * np.arange(N))
        for hq in range(Hq):
            g = hq // G
            mode = int(cmodes[b, g])
            for qb in range(N):
                kb = np.arange(qb + 1)
                last = qb * block + size[qb] - 1
                if mode == MODE_XA:
                    ok = plan[(b, hq)][1][last // xa_block, (kb * block) // xa_block]
                else:
                    ok = visible(last, kb * block, mode, ns, w, block)
                total += int(size[qb]) * int(size[kb][ok].sum())
    return 4 * d * total
