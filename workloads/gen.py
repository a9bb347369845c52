"""Seeded draws for the hybrid-prefill workloads.

Everything here is input construction: normal draws, sequence lengths, the
router's random weights, which KV heads a workload wants sparse, and the
encoding of float32 values as bfloat16 bit patterns (round to nearest, ties to
even).  The per-(sequence, KV head) key offsets and the final-bias override
that steer routing are *stored values* read from ``route_control.json``; the
script that computes them lives with the oracle and is the only code that
writes that file.

Random streams.  Every tensor has its own stream id and is drawn in fixed
chunks of rows, chunk ``c`` of stream ``s`` under seed ``seed`` coming from
``PCG64(SeedSequence([seed, s, c]))``.  The result is independent of how many
threads fill the chunks.
"""
from __future__ import annotations

import json
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

from .configs import Workload

STREAM = {
    "q": 1, "k": 2, "v": 3, "lowrank_a": 4, "lowrank_b": 5,
    "w1": 6, "b1": 7, "w2": 8, "b2": 9, "w3": 10, "b3": 11, "w4": 12, "b4": 13,
    "lengths": 14, "heads": 15, "gumbel": 16, "hitter_dir": 17, "hitter_blocks": 18,
}
HITTER_BLOCK = 128
CHUNK_ROWS = 4096
CONTROL_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "route_control.json")


def _threads() -> int:
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


def _rng(seed: int, stream: int, chunk: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(stream), int(chunk)])))


# ----------------------------------------------------------------------------
# bfloat16 encoding
# ----------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> the float32 values they encode (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# chunked normal draws
# ----------------------------------------------------------------------------

def _draw_rows(seed, stream, n_rows, row_shape, std, out_dtype, post=None):
    """Draw ``n_rows`` rows of N(0, std^2) float32, optionally post-process each
    chunk in place (``post(chunk, row0)``), and store as float32 or bf16 bits."""
    row_shape = tuple(row_shape)
    out = np.empty((n_rows,) + row_shape, dtype=np.uint16 if out_dtype == "bf16" else np.float32)
    n_chunks = (n_rows + CHUNK_ROWS - 1) // CHUNK_ROWS

    def fill(c):
        r0 = c * CHUNK_ROWS
        r1 = min(n_rows, r0 + CHUNK_ROWS)
        x = _rng(seed, stream, c).standard_normal((r1 - r0,) + row_shape, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        if post is not None:
            post(x, r0)
        out[r0:r1] = bf16_bits(x) if out_dtype == "bf16" else x

    if n_chunks <= 1:
        for c in range(n_chunks):
            fill(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out


def normal(seed: int, stream: int, shape, std: float = 1.0) -> np.ndarray:
    """A float32 N(0, std^2) array of ``shape`` from stream ``stream``."""
    shape = tuple(shape)
    return _draw_rows(seed, stream, shape[0], shape[1:], std, "f32")


def draw_router_weights(seed: int, d: int, task_hidden: int, router_hidden: int, std: float):
    """Router parameters in nn.Linear layout ``[out, in]``, all N(0, std^2), float32.

    Shapes: task MLP d -> task_hidden -> d, router MLP d -> router_hidden -> 2.
    """
    shapes = {
        "w1": (task_hidden, d), "b1": (task_hidden,),
        "w2": (d, task_hidden), "b2": (d,),
        "w3": (router_hidden, d), "b3": (router_hidden,),
        "w4": (2, router_hidden), "b4": (2,),
    }
    w = {}
    for name, shp in shapes.items():
        x = _rng(seed, STREAM[name]).standard_normal(shp, dtype=np.float32)
        w[name] = (x * np.float32(std)).astype(np.float32)
    return w


def draw_lengths(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    """Sequence lengths floor(exp(U(ln lo, ln hi))), int64."""
    u = _rng(seed, STREAM["lengths"]).uniform(np.log(lo), np.log(hi), size=n)
    return np.floor(np.exp(u)).astype(np.int64)


def draw_gumbel(seed: int, shape) -> np.ndarray:
    """Standard Gumbel(0, 1) noise, float32, from its own stream (the noise the
    Gumbel-Softmax router draws during training, passed in as an input)."""
    return _rng(seed, STREAM["gumbel"]).gumbel(0.0, 1.0, size=tuple(shape)).astype(np.float32)


def draw_sa_heads(seed: int, counts, Hkv: int):
    """For each sequence b, a seeded subset of ``counts[b]`` KV heads meant to be sparse.

    Returns an int8 array [B, Hkv] of target modes (1 = sparse)."""
    rng = _rng(seed, STREAM["heads"])
    t = np.zeros((len(counts), Hkv), dtype=np.int8)
    for b, k in enumerate(counts):
        perm = rng.permutation(Hkv)
        t[b, perm[:k]] = 1
    return t


# ----------------------------------------------------------------------------
# cases
# ----------------------------------------------------------------------------

@dataclass
class Case:
    dtype: str
    seed: int
    lengths: np.ndarray            # int64 [B]
    cu_seqlens: np.ndarray         # int32 [B+1]
    Hq: int
    Hkv: int
    d: int
    q: np.ndarray                  # [T, Hq, d]: uint16 bf16 bits, or float32
    k: np.ndarray                  # [T, Hkv, d]
    v: np.ndarray                  # [T, Hkv, d]
    weights: dict                  # router parameters, float32, nn.Linear layout
    pool_len: int = 100
    block: int = 64
    n_sink: int = 1
    keep_fraction: float = 0.2
    window_blocks: int = 0
    softmax_scale: float = 0.0     # 0 means 1/sqrt(d)
    target_modes: np.ndarray | None = None   # int8 [B, Hkv] the workload aims for, or None
    name: str = "custom"
    meta: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return len(self.lengths)

    @property
    def T(self) -> int:
        return int(self.cu_seqlens[-1])

    def _f32(self, a):
        return bf16_bits_to_f32(a) if self.dtype == "bf16" else a

    def q_f32(self):
        return self._f32(self.q)

    def k_f32(self):
        return self._f32(self.k)

    def v_f32(self):
        return self._f32(self.v)


def load_control():
    if not os.path.exists(CONTROL_PATH):
        return {}
    with open(CONTROL_PATH) as f:
        return json.load(f)


def _cu(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    if cu[-1] >= 2**31:
        raise ValueError("total tokens must fit in int32")
    return cu.astype(np.int32)


def _make_k(seed, T, Hkv, d, std, lowrank, cu, shift, out_dtype, extra=None):
    """K = std*N(0,1) [+ A B^T low-rank term per head] [+ per-(seq, head) offset]
    [+ whatever ``extra(x, r0)`` adds]."""
    lr_b = None
    if lowrank:
        # B: [Hkv, d, r] ~ N(0, 1/r) so the low-rank term has unit variance per element.
        lr_b = (_rng(seed, STREAM["lowrank_b"]).standard_normal((Hkv, d, lowrank), dtype=np.float32)
                * np.float32(1.0 / np.sqrt(lowrank))).astype(np.float32)

    def post(x, r0):
        n = x.shape[0]
        if lr_b is not None:
            c = r0 // CHUNK_ROWS
            a = _rng(seed, STREAM["lowrank_a"], c).standard_normal((n, lowrank), dtype=np.float32)
            x += np.einsum("tr,hdr->thd", a, lr_b).astype(np.float32)
        if shift is not None:
            seg = np.searchsorted(cu, np.arange(r0, r0 + n), side="right") - 1
            x += shift[seg]
        if extra is not None:
            extra(x, r0)

    return _draw_rows(seed, STREAM["k"], T, (Hkv, d), std, out_dtype, post)


def hitter_layout(seed, lengths, Hkv, d, frac, pool_len=100):
    """Heavy-hitter structure: a unit direction per KV head, and the
    sequence-local 128-token key blocks that carry it (each with probability
    ``frac``, never a block holding one of the first or last ``pool_len``
    tokens, so the router's pooled keys are untouched).  Returns
    (u float32 [Hkv, d], list of bool arrays per sequence)."""
    u = _rng(seed, STREAM["hitter_dir"]).standard_normal((Hkv, d), dtype=np.float32)
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    blocks = []
    r = _rng(seed, STREAM["hitter_blocks"])
    for L in np.asarray(lengths, dtype=np.int64):
        n = -(-int(L) // HITTER_BLOCK)
        hb = r.random(n) < frac
        j = np.arange(n)
        first_ok = j * HITTER_BLOCK >= pool_len
        last_ok = (j + 1) * HITTER_BLOCK <= int(L) - pool_len
        blocks.append(hb & first_ok & last_ok)
    return u, blocks


def custom_case(seed, lengths, Hq, Hkv, d, dtype="bf16", *, task_hidden=None, router_hidden=None,
                w_std=0.05, q_std=1.0, k_std=1.0, v_std=1.0, lowrank=0, n_sink=1,
                keep_fraction=0.2, window_blocks=0, pool_len=100, block=64, k_shift=None,
                b4=None, softmax_scale=0.0, hitters=None, name="custom") -> Case:
    """A case of arbitrary shape.  ``k_shift`` is an optional float32 [B, Hkv, d]
    offset added to every K row of that sequence and head before rounding.
    ``hitters`` = (frac, strength) adds strength * u_g to every query row of
    KV group g and to the key rows of the heavy-hitter blocks of
    ``hitter_layout`` (before rounding), so that those blocks draw most of
    every query's attention."""
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = _cu(lengths)
    T = int(cu[-1])
    task_hidden = task_hidden or 4 * d
    router_hidden = router_hidden or max(2, d // 2)
    qpost = kpost = None
    if hitters is not None:
        frac, strength = hitters
        u, hblocks = hitter_layout(seed, lengths, Hkv, d, frac, pool_len)
        G = Hq // Hkv
        uq = np.float32(strength) * np.repeat(u, G, axis=0)          # [Hq, d]
        hit = np.concatenate([np.repeat(hb, HITTER_BLOCK)[:int(L)]
                              for hb, L in zip(hblocks, lengths)]) if len(lengths) else np.zeros(0, bool)
        uk = np.float32(strength) * u                                 # [Hkv, d]

        def qpost(x, r0):
            x += uq[None]

        def kpost(x, r0):
            x[hit[r0:r0 + x.shape[0]]] += uk[None]
    q = _draw_rows(seed, STREAM["q"], T, (Hq, d), q_std, dtype, qpost)
    k = _make_k(seed, T, Hkv, d, k_std, lowrank, cu,
                None if k_shift is None else np.asarray(k_shift, dtype=np.float32), dtype, kpost)
    v = _draw_rows(seed, STREAM["v"], T, (Hkv, d), v_std, dtype)
    w = draw_router_weights(seed, d, task_hidden, router_hidden, w_std)
    if b4 is not None:
        w["b4"] = np.asarray(b4, dtype=np.float32)
    return Case(dtype=dtype, seed=int(seed), lengths=lengths, cu_seqlens=cu, Hq=Hq, Hkv=Hkv, d=d,
                q=q, k=k, v=v, weights=w, pool_len=pool_len, block=block, n_sink=n_sink,
                keep_fraction=keep_fraction, window_blocks=window_blocks,
                softmax_scale=softmax_scale, name=name)


def workload_lengths(wl: Workload, seed: int) -> np.ndarray:
    if wl.seq_lens is not None:
        return np.asarray(wl.seq_lens, dtype=np.int64)
    lo, hi = wl.varlen_range
    return draw_lengths(seed, wl.n_seqs, lo, hi)


def build_case(wl: Workload, seed: int | None = None, *, control: bool = True,
               hitters=None) -> Case:
    """The seeded inputs of workload ``wl``.

    With ``control`` the stored routing controls (seed actually used, final
    router bias, per-(sequence, KV head) key offsets) are applied, so the
    router produces ``target_modes``.  Without it the raw draws are returned
    (this is what the script that computes the controls starts from)."""
    ctl = load_control().get(wl.name) if control else None
    if ctl is not None and seed is None:
        seed = int(ctl["seed"])
    if seed is None:
        seed = wl.start_seed
    lengths = workload_lengths(wl, seed)
    shift = None
    b4 = None
    target = None
    if ctl is not None and int(ctl["seed"]) == int(seed):
        if ctl.get("shift") is not None:
            shift = np.asarray(ctl["shift"], dtype=np.float32)
        if ctl.get("b4") is not None:
            b4 = ctl["b4"]
        if ctl.get("target_modes") is not None:
            target = np.asarray(ctl["target_modes"], dtype=np.int8)
    c = custom_case(seed, lengths, wl.Hq, wl.Hkv, wl.d, wl.dtype, task_hidden=wl.task_hidden,
                    router_hidden=wl.router_hidden, w_std=wl.w_std, q_std=wl.q_std,
                    k_std=wl.k_std, v_std=wl.v_std, lowrank=wl.lowrank, n_sink=wl.n_sink,
                    keep_fraction=wl.keep_fraction, pool_len=wl.pool_len, block=wl.block,
                    k_shift=shift, b4=b4, hitters=hitters, name=wl.name)
    if target is None and wl.sa_heads is not None:
        target = draw_sa_heads(seed, wl.sa_heads, wl.Hkv)
    c.target_modes = target
    return c


def workload_k(wl: Workload, seed: int, shift=None):
    """Only the K tensor of workload ``wl`` (as ``build_case`` would draw it with
    the given key offsets), plus its lengths and cu_seqlens."""
    lengths = workload_lengths(wl, seed)
    cu = _cu(lengths)
    k = _make_k(seed, int(cu[-1]), wl.Hkv, wl.d, wl.k_std, wl.lowrank, cu,
                None if shift is None else np.asarray(shift, dtype=np.float32), wl.dtype)
    return lengths, cu, k
