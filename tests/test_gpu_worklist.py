"""The device-built work list (through the C ABI).

- The order the counting sort writes equals NumPy's stable argsort of the
  items' band keys, and every key is the band of its item's recorded cost.
- Each item's recorded cost is the number of 64-key blocks its rows can see,
  counted here from the visibility rule (the reading of the SA pattern stated
  in the oracle: sinks plus a causal local window, per 64-token block).
- The attention result does not depend on the list order: a permuted order
  gives bitwise the same O and LSE (every item is computed on its own, with no
  reduction across items; the fused single pass of "Technical Summary:
  Elastic Attention", Sec. 2.3)."""
import numpy as np
import pytest
import torch

import full_attention_long_amd as ea
from gpu_helpers import note, to_device
from workloads import gen
from workloads.configs import WORKLOADS

pytestmark = pytest.mark.gpu

ITEM_WORDS = 5
BAND_SHIFT = 5
N_BINS = 1024


def _plan(c, modes_np, max_seqlen, n_sink, keep, window_blocks=0):
    dv = to_device(c)
    B, T = len(c.lengths), int(c.cu_seqlens[-1])
    modes = torch.from_numpy(np.ascontiguousarray(modes_np, np.int8)).cuda()
    code = 1 if c.dtype == "bf16" else 0
    need = ea.ea_hybrid_prefill_workspace_size(B, T, max_seqlen, c.Hq, c.Hkv, c.d, code)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ea.ea_hybrid_prefill_plan(modes, dv["cu"], T, max_seqlen, c.Hq, c.Hkv, c.d, code, ws,
                              n_sink=n_sink, window_blocks=window_blocks, keep_fraction=keep)
    torch.cuda.synchronize()
    lay = ea.ea_hybrid_prefill_plan_layout(B, T, max_seqlen, c.Hq, c.Hkv, c.d, code)
    return dv, modes, ws, lay


def _read_list(ws, lay):
    h = ws.cpu().numpy()
    n = lay["n_slots"]
    tiles = int(h[:4].view(np.int32)[0])
    items = h[lay["items"]:lay["items"] + 4 * ITEM_WORDS * n].view(np.int32).reshape(n, ITEM_WORDS)
    keys = h[lay["keys"]:lay["keys"] + 4 * n].view(np.uint32)
    order = h[lay["order"]:lay["order"] + 4 * n].view(np.int32)
    return tiles, items, keys, order


def _visible_blocks(mode, qb0, qb1, n_sink, w):
    """Key blocks some row of query blocks qb0..qb1 can see (FA 0 / SA 1)."""
    seen = set()
    for qb in range(qb0, qb1 + 1):
        for kb in range(qb + 1):
            if mode == 0 or kb < n_sink or qb - kb < w:
                seen.add(kb)
    return len(seen)


def _window(L, n_sink, keep, window_blocks):
    if window_blocks > 0:
        return window_blocks
    N = -(-L // 64)
    return max(n_sink + 1, int(np.floor(np.float64(np.float32(keep)) * N + 0.5))) - n_sink


def _check_list(c, modes_np, max_seqlen, n_sink, keep, window_blocks=0, check_costs=True):
    note(f"work list {c.name} lengths={list(c.lengths)[:8]} Hq={c.Hq} Hkv={c.Hkv}")
    _, _, ws, lay = _plan(c, modes_np, max_seqlen, n_sink, keep, window_blocks)
    tiles, items, keys, order = _read_list(ws, lay)
    n_real = tiles * c.Hkv
    maxcost = -(-max_seqlen // 64)
    # the sort: a permutation, equal to the stable argsort of the keys
    np.testing.assert_array_equal(order, np.argsort(keys, kind="stable"))
    # keys: band of the recorded cost for real items, the empty key after them
    cost = items[:n_real, 3]
    want = np.minimum((maxcost - np.minimum(cost, maxcost)) >> BAND_SHIFT, N_BINS - 2)
    np.testing.assert_array_equal(keys[:n_real], want.astype(np.uint32))
    assert (keys[n_real:] == min((maxcost >> BAND_SHIFT) + 1, N_BINS - 1)).all()
    # every (sequence, KV head, tile) appears exactly once
    G = c.Hq // c.Hkv
    BMq = 256 // G
    want_tiles = sorted((b, g, t) for b, L in enumerate(c.lengths) for g in range(c.Hkv)
                        for t in range(-(-int(L) // BMq)))
    got_tiles = sorted(map(tuple, items[:n_real, :3].tolist()))
    assert got_tiles == want_tiles
    if check_costs:
        for b, g, qt, cst, mode in items[:n_real].tolist():
            L = int(c.lengths[b])
            p0, p1 = qt * BMq, min(qt * BMq + BMq, L) - 1
            assert mode == int(modes_np[b, g])
            w = _window(L, n_sink, keep, window_blocks)
            assert cst == _visible_blocks(mode, p0 // 64, p1 // 64, n_sink, w), (b, g, qt)
    return tiles


def test_list_small_varlen_costs_and_order():
    c = gen.custom_case(61, [300, 0, 1, 777, 64, 129, 2500], 8, 2, 128, "bf16")
    rng = np.random.default_rng(3)
    modes = rng.integers(0, 2, size=(7, 2)).astype(np.int8)
    _check_list(c, modes, 2500, 1, 0.2)
    _check_list(c, modes, 2500, 2, 0.3)
    _check_list(c, modes, 3500, 0, 0.2, window_blocks=1)


@pytest.mark.parametrize("name", ["qwen4b_s128k_sa2", "varlen8"])
def test_list_full_size_order(name):
    wl = WORKLOADS[name]
    seed = int(gen.load_control()[name]["seed"])
    lengths = gen.workload_lengths(wl, seed)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    # shapes only: the list depends on lengths, heads, modes and geometry
    c = gen.Case(dtype="bf16", seed=seed, lengths=np.asarray(lengths, np.int64), cu_seqlens=cu,
                 Hq=wl.Hq, Hkv=wl.Hkv, d=wl.d, q=np.zeros((1, wl.Hq, wl.d), np.uint16),
                 k=np.zeros((1, wl.Hkv, wl.d), np.uint16), v=np.zeros((1, wl.Hkv, wl.d), np.uint16),
                 weights={}, pool_len=100, name=name)
    modes = np.asarray(gen.load_control()[name]["target_modes"], np.int8)
    _check_list(c, modes, int(max(lengths)), wl.n_sink, wl.keep_fraction, check_costs=False)


def test_permuted_list_order_gives_identical_output():
    c = gen.custom_case(62, [3000, 130, 1777], 8, 2, 128, "bf16")
    modes = np.array([[0, 1], [1, 0], [1, 1]], np.int8)
    dv, m, ws, lay = _plan(c, modes, 3000, 1, 0.2)
    note("permuted order: planned order")
    O1, l1 = ea.ea_hybrid_prefill_run(dv["q"], dv["k"], dv["v"], m, dv["cu"], 3000, ws)
    torch.cuda.synchronize()
    tiles, _, _, order = _read_list(ws, lay)
    n_real = tiles * c.Hkv
    perm = order.copy()
    perm[:n_real] = np.random.default_rng(5).permutation(order[:n_real])
    assert not np.array_equal(perm, order)
    o0 = lay["order"]
    ws[o0:o0 + 4 * perm.size] = torch.from_numpy(perm.view(np.uint8).copy()).cuda()
    note("permuted order: shuffled order")
    O2, l2 = ea.ea_hybrid_prefill_run(dv["q"], dv["k"], dv["v"], m, dv["cu"], 3000, ws)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(l1, l2)
