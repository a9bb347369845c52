"""Host-side bookkeeping for reporting: the sparse window per sequence and the
effective FLOP count of a routed layer (closed forms; no device work).

Effective FLOPs count only the 64 x 64 (query block, key block) pairs the
fused kernel computes: 4 * d * rows * cols per pair and query head (two
matrix products of 2 * rows * cols * d each), a partly masked diagonal or
window-edge pair counted in full.  For a sequence of N key blocks, an FA head
computes key blocks 0..qb for query block qb and an SA head
min(qb + 1, n_sink + w) of them.
"""
from __future__ import annotations

import math

import numpy as np

BLOCK = 64
MI355X_BF16_DENSE_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 FLOP/clk/CU
MI355X_FP32_MATRIX_TFLOPS = 157.3
MI355X_HBM_GBPS = 8000.0


def window_blocks(L: int, n_sink: int, keep_fraction: float, window_blocks: int = 0) -> int:
    """w for a sequence of length L (same rule as the library: keep =
    max(n_sink + 1, floor(rho * N + 1/2)) in double on the float32 rho)."""
    if window_blocks > 0:
        return int(window_blocks)
    N = -(-int(L) // BLOCK)
    rho = float(np.float32(keep_fraction))
    return max(int(n_sink) + 1, int(math.floor(rho * N + 0.5))) - int(n_sink)


def _pair_sum(L: int, keep: int | None) -> int:
    """Sum over visible (qb, kb) pairs of rows(qb) * cols(kb); keep=None for FA."""
    N = -(-L // BLOCK)
    last = L - (N - 1) * BLOCK            # rows of the last block
    full = BLOCK * BLOCK
    if keep is None or keep >= N:
        # all pairs kb <= qb: (N-1)N/2 pairs of full blocks among the first N-1
        # query blocks, N-1 pairs of (last rows x 64) and one (last x last)
        return (N - 1) * N // 2 * full + (N - 1) * last * BLOCK + last * last
    # SA: query block qb sees min(qb + 1, keep) key blocks, all of 64 columns
    # except the diagonal block of the last query block
    s = 0
    # query blocks 0..N-2 (64 rows each)
    k = keep
    first = min(N - 1, k)                  # qb < k: qb + 1 blocks
    s += full * (first * (first + 1) // 2)
    s += full * max(0, N - 1 - k) * k
    # last query block: min(N, k) blocks, the last one (its own) with `last` columns
    nl = min(N, k)
    s += last * (BLOCK * (nl - 1) + last)
    return s


def effective_flops(modes, lengths, Hq: int, Hkv: int, d: int, *, n_sink: int,
                    keep_fraction: float, window_blocks_: int = 0) -> int:
    """EF of a routed layer; modes int [B, Hkv], lengths [B]."""
    G = Hq // Hkv
    total = 0
    for b, L in enumerate(lengths):
        L = int(L)
        if L <= 0:
            continue
        w = window_blocks(L, n_sink, keep_fraction, window_blocks_)
        n_fa = int((np.asarray(modes[b]) == 0).sum())
        n_sa = Hkv - n_fa
        total += G * (n_fa * _pair_sum(L, None) + n_sa * _pair_sum(L, n_sink + w))
    return 4 * d * total


def msr(modes) -> float:
    """Share of (sequence, KV head) pairs routed to sparse attention."""
    m = np.asarray(modes)
    return float((m != 0).mean())


XA_BLOCK = 128
# computation mode (0 FA, 1 SA, 2 XA) of router decisions 0 / 1 per head configuration
HEAD_CONFIG_MODES = {"FA-SSA": (0, 1), "FA-XA": (0, 2), "XA-SSA": (2, 1)}


def computation_modes(modes, config: str) -> np.ndarray:
    """[B, Hkv] computation modes of router decisions ``modes`` under ``config``."""
    return np.asarray(HEAD_CONFIG_MODES[config], dtype=np.int64)[np.asarray(modes, dtype=np.int64)]


def xa_head_pairs(keep: np.ndarray, L: int) -> int:
    """Sum of rows * cols over the (64-query block, 64-key block) pairs an XA
    head computes, given its keep flags ``keep`` [nb, nb] over 128-token blocks
    (row i: key blocks kept for query block i): causal pairs whose 128-blocks
    are kept, partly masked ones counted in full."""
    N = -(-int(L) // BLOCK)
    size = np.minimum(BLOCK, int(L) - BLOCK * np.arange(N)).astype(np.int64)
    total = 0
    for qb in range(N):
        i = qb // (XA_BLOCK // BLOCK)
        kb = np.arange(qb + 1)
        ok = np.asarray(keep[i, kb // (XA_BLOCK // BLOCK)], dtype=bool)
        total += int(size[qb]) * int(size[kb][ok].sum())
    return total


def xa_effective_flops(cmodes, keep, lengths, Hq: int, Hkv: int, d: int, *, n_sink: int,
                       keep_fraction: float, window_blocks_: int = 0) -> int:
    """EF of a layer with FA (0), SA (1) and XA (2) computation modes
    ``cmodes`` [B, Hkv]; ``keep`` [B, Hq, nqb, nqb] holds the XA heads' keep
    flags (as written by ea_xa_prefill)."""
    G = Hq // Hkv
    total = 0
    for b, L in enumerate(lengths):
        L = int(L)
        if L <= 0:
            continue
        w = window_blocks(L, n_sink, keep_fraction, window_blocks_)
        for g in range(Hkv):
            m = int(cmodes[b][g])
            if m == 0:
                total += G * _pair_sum(L, None)
            elif m == 1:
                total += G * _pair_sum(L, n_sink + w)
            else:
                for hq in range(g * G, (g + 1) * G):
                    total += xa_head_pairs(keep[b, hq], L)
    return 4 * d * total


def xa_selection_flops(cmodes, lengths, Hq: int, Hkv: int, d: int, stride: int = 8) -> int:
    """Matrix FLOPs of the XA selection: per XA query head and query block i,
    i + 1 key blocks of 16 x 16 group scores over S * d products, each
    scored once."""
    G = Hq // Hkv
    per_tile = 2 * (XA_BLOCK // stride) ** 2 * stride * d
    total = 0
    for b, L in enumerate(lengths):
        nb = -(-int(L) // XA_BLOCK)
        n_xa = int((np.asarray(cmodes[b]) == 2).sum()) * G
        total += n_xa * per_tile * (nb * (nb + 1) // 2)
    return total
