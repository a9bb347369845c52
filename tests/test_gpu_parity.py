"""GPU parity of the HIP path against the CPU oracle (through the C ABI).

Routing decisions must match bit for bit (every case here has
|z0 - z1| >= 1e-3, or is compared only where the oracle margin leaves the
argmax well posed); logits within 1e-5; O within max-abs 1e-5 for fp32 and
max-abs 2e-2 / mean-abs 1e-3 for bf16; LSE within 1e-4."""
import numpy as np
import pytest
import torch

from gpu_helpers import (LSE_TOL, compare_o, gpu_prefill, gpu_route, note, o_to_numpy,
                         to_device)
from oracle import ea_oracle as orc
from workloads import gen
from workloads.configs import WORKLOADS

pytestmark = pytest.mark.gpu


def oracle_full(c, modes):
    return orc.hybrid_attention(c.q_f32(), c.k_f32(), c.v_f32(), modes, c.cu_seqlens,
                                n_sink=c.n_sink, window_blocks=c.window_blocks,
                                keep_fraction=c.keep_fraction, softmax_scale=c.softmax_scale)


def check_full(c, modes, **kw):
    note(f"prefill {c.name} dtype={c.dtype} lengths={list(c.lengths)} Hq={c.Hq} Hkv={c.Hkv} "
         f"d={c.d} modes={modes.tolist()} ns={c.n_sink} rho={c.keep_fraction} wb={c.window_blocks}")
    O, lse = gpu_prefill(c, modes, **kw)
    ref_o, ref_lse = oracle_full(c, modes)
    compare_o(o_to_numpy(O), ref_o, c.dtype)
    lse = lse.cpu().numpy()
    assert np.abs(lse - ref_lse).max() <= LSE_TOL
    return O


# ----------------------------------------------------------------------------
# Router
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(WORKLOADS))
def test_route_workloads_bit_exact(name):
    wl = WORKLOADS[name]
    ctl = gen.load_control()[name]
    seed = int(ctl["seed"])
    shift = None if ctl["shift"] is None else np.asarray(ctl["shift"], np.float32)
    lengths, cu, k = gen.workload_k(wl, seed, shift)
    w = gen.draw_router_weights(seed, wl.d, wl.task_hidden, wl.router_hidden, wl.w_std)
    if ctl["b4"] is not None:
        w["b4"] = np.asarray(ctl["b4"], np.float32)
    c = gen.Case(dtype=wl.dtype, seed=seed, lengths=lengths, cu_seqlens=cu, Hq=wl.Hq, Hkv=wl.Hkv,
                 d=wl.d, q=k[:1], k=k, v=k[:1], weights=w, pool_len=wl.pool_len, name=name)
    note(f"route {name}")
    modes, logits = gpu_route(c)
    kf = c.k_f32()
    ref_modes, ref_z = orc.route(kf, cu, w, wl.pool_len)
    np.testing.assert_array_equal(modes, ref_modes)
    np.testing.assert_array_equal(modes, np.asarray(ctl["target_modes"], np.int8))
    assert np.abs(logits - ref_z).max() <= 1e-5


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64), ("bf16", 64), ("f32", 128)])
def test_route_varlen_edge_lengths(dtype, d):
    lengths = [0, 1, 150, 199, 200, 201, 5000, 0]
    c = gen.custom_case(11, lengths, 4, 4, d, dtype, w_std=0.2)
    note(f"route varlen dtype={dtype} d={d}")
    modes, logits = gpu_route(c)
    ref_modes, ref_z = orc.route(c.k_f32(), c.cu_seqlens, c.weights, c.pool_len)
    assert np.abs(logits - ref_z).max() <= 1e-5
    posed = np.abs(ref_z[..., 0] - ref_z[..., 1]) > 1e-4
    np.testing.assert_array_equal(modes[posed], ref_modes[posed])
    assert (modes[np.array(lengths) == 0] == 0).all()
    assert (logits[np.array(lengths) == 0] == 0).all()


@pytest.mark.parametrize("d,task_hidden,router_hidden", [(64, 100, 7), (128, 1000, 65), (96, 37, 3)])
def test_route_odd_mlp_widths(d, task_hidden, router_hidden):
    # widths that fill neither the eight output rows a wave takes per pass
    # nor the 64-lane stride over the input axis
    c = gen.custom_case(13, [333, 1200], 4, 2, d, "bf16", task_hidden=task_hidden,
                        router_hidden=router_hidden, w_std=0.2)
    note(f"route widths d={d} task={task_hidden} router={router_hidden}")
    modes, logits = gpu_route(c)
    ref_modes, ref_z = orc.route(c.k_f32(), c.cu_seqlens, c.weights, c.pool_len)
    assert np.abs(logits - ref_z).max() <= 1e-5
    posed = np.abs(ref_z[..., 0] - ref_z[..., 1]) > 1e-4
    np.testing.assert_array_equal(modes[posed], ref_modes[posed])


def test_route_reads_only_boundary_rows():
    c = gen.custom_case(12, [1000, 700], 4, 2, 128, "bf16", w_std=0.2)
    note("route locality")
    m1, z1 = gpu_route(c)
    k = c.k.copy()
    k[100:900] = 0x7FC0  # bf16 NaN in rows the router must not read
    k[1000 + 100:1000 + 600] = 0x7FC0
    c.k = k
    m2, z2 = gpu_route(c)
    np.testing.assert_array_equal(z1, z2)
    np.testing.assert_array_equal(m1, m2)


# ----------------------------------------------------------------------------
# Hybrid prefill, small cases against the full oracle output
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("modes", [None, [[0, 0]], [[1, 1]], [[0, 1]], [[1, 0]]])
def test_prefill_tiny_f32(modes):
    c = gen.build_case(WORKLOADS["tiny_f32_s512"])
    m = c.target_modes if modes is None else np.array(modes, np.int8)
    check_full(c, m)


CASES = [
    # lengths, Hq, Hkv, d, dtype, n_sink, rho, window_blocks
    ([1000], 8, 2, 128, "bf16", 1, 0.2, 0),
    ([1000], 8, 2, 128, "bf16", 2, 0.3, 0),
    ([300, 0, 1, 777, 64, 129], 8, 2, 128, "bf16", 1, 0.2, 0),
    ([2000], 4, 4, 128, "bf16", 1, 0.2, 0),        # G = 1: 128 positions per tile
    ([1500], 16, 2, 128, "bf16", 1, 0.2, 0),       # G = 8: 16 positions per tile
    ([700], 6, 2, 64, "bf16", 1, 0.25, 0),         # G = 3: 42 positions, tiles straddle blocks
    ([1000, 333], 8, 2, 64, "bf16", 1, 0.2, 0),
    ([3000], 8, 1, 128, "bf16", 0, 0.2, 1),        # n_sink = 0, w = 1: block-local attention
    ([2500], 8, 2, 128, "bf16", 1, 0.2, 100),      # window covers the sequence: SA == FA
    ([4100], 8, 2, 128, "bf16", 4, 0.1, 0),
    ([600, 33], 8, 2, 128, "f32", 1, 0.2, 0),
    ([513, 64, 65], 4, 2, 64, "f32", 2, 0.3, 0),
    ([1200], 4, 1, 128, "f32", 1, 0.2, 0),
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_prefill_small(case):
    lengths, Hq, Hkv, d, dtype, ns, rho, wb = case
    c = gen.custom_case(100 + len(lengths) + Hq + d, lengths, Hq, Hkv, d, dtype, n_sink=ns,
                        keep_fraction=rho, window_blocks=wb)
    rng = np.random.default_rng(7)
    modes = rng.integers(0, 2, size=(len(lengths), Hkv)).astype(np.int8)
    modes[0, 0] = 1
    if Hkv > 1:
        modes[0, 1] = 0
    check_full(c, modes)


def test_window_covering_sequence_equals_fa_bitwise():
    c = gen.custom_case(5, [2500], 8, 2, 128, "bf16", n_sink=1, window_blocks=100)
    note("SA with a window covering the sequence vs FA")
    o_sa, _ = gpu_prefill(c, np.array([[1, 1]], np.int8))
    o_fa, _ = gpu_prefill(c, np.array([[0, 0]], np.int8))
    assert torch.equal(o_sa, o_fa)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_constant_v(dtype):
    c = gen.custom_case(6, [900, 130], 8, 2, 128, dtype)
    val = 0.375
    c.v = gen.bf16_bits(np.full(c.v.shape, val, np.float32)) if dtype == "bf16" else \
        np.full(c.v.shape, val, np.float32)
    note(f"constant V {dtype}")
    O, _ = gpu_prefill(c, np.array([[0, 1], [1, 0]], np.int8))
    err = np.abs(o_to_numpy(O) - val).max()
    assert err <= (2e-3 if dtype == "bf16" else 1e-6), err


def test_nan_outside_visible_blocks_never_reaches_output():
    # sequence 0 is followed by a sequence of NaNs (its ragged last block must
    # not read past its end) and has NaN in key blocks that only some query
    # tiles of its SA head can see; every other row must match the clean run
    L0, L1, ns = 64 * 20 + 37, 300, 1
    c = gen.custom_case(8, [L0, L1], 8, 2, 128, "bf16", n_sink=ns, window_blocks=2)
    modes = np.array([[1, 0], [0, 0]], np.int8)
    note("NaN isolation: clean run")
    clean, _ = gpu_prefill(c, modes)
    nan = np.uint16(0x7FC0)
    k, v = c.k.copy(), c.v.copy()
    k[L0:], v[L0:] = nan, nan
    bad = [5, 6]  # key blocks of the SA KV head (head 0) poisoned
    for kb in bad:
        k[kb * 64:(kb + 1) * 64, 0] = nan
        v[kb * 64:(kb + 1) * 64, 0] = nan
    c.k, c.v = k, v
    note("NaN isolation: poisoned run")
    dirty, _ = gpu_prefill(c, modes)
    clean, dirty = clean.float().cpu().numpy(), dirty.float().cpu().numpy()
    qb = np.arange(L0) // 64
    sees_bad = np.zeros(L0, bool)
    for kb in bad:
        sees_bad |= (qb >= kb) & (qb - kb < 2)
    G = 4
    np.testing.assert_array_equal(dirty[:L0][~sees_bad][:, :G], clean[:L0][~sees_bad][:, :G])
    np.testing.assert_array_equal(dirty[:L0, G:], clean[:L0, G:])
    assert np.isnan(dirty[:L0][sees_bad][:, :G]).any()   # the poisoned rows did read NaN


def test_bitwise_deterministic():
    c = gen.custom_case(9, [3000, 1000], 8, 2, 128, "bf16")
    modes = np.array([[0, 1], [1, 1]], np.int8)
    note("determinism")
    a, la = gpu_prefill(c, modes)
    b, lb = gpu_prefill(c, modes)
    assert torch.equal(a, b) and torch.equal(la, lb)


# ----------------------------------------------------------------------------
# Full workload sizes (the bench's configuration): route + prefill, sampled rows
# ----------------------------------------------------------------------------

def sample_rows(lengths, cu, rng, per_seq=6):
    toks = []
    for b, L in enumerate(lengths):
        L = int(L)
        if L == 0:
            continue
        cand = {0, min(L - 1, 63), min(L - 1, 64), L // 2 + 17, max(0, L - 65), L - 1}
        cand |= set(rng.integers(0, L, size=per_seq).tolist())
        toks += [int(cu[b]) + t for t in sorted(cand) if t < L]
    return np.array(toks)


@pytest.mark.parametrize("name", ["llama8b_s32k", "qwen4b_s128k_sa2", "qwen4b_s128k_sa6",
                                  "extrap_s256k", "varlen8"])
def test_full_size_sampled(name):
    wl = WORKLOADS[name]
    note(f"full size {name}: generating")
    c = gen.build_case(wl)
    dv = to_device(c)
    note(f"full size {name}: route")
    modes, _ = gpu_route(c, dv)
    np.testing.assert_array_equal(modes, c.target_modes)
    note(f"full size {name}: prefill T={c.T}")
    O, lse = gpu_prefill(c, modes, dv)
    del dv
    rng = np.random.default_rng(1)
    toks = sample_rows(c.lengths, c.cu_seqlens, rng, per_seq=4 if c.B > 1 else 8)
    G = c.Hq // c.Hkv
    heads = [g * G + (g % G) for g in range(c.Hkv)]
    tt = torch.from_numpy(toks).cuda()
    got = O[tt][:, heads].float().cpu().numpy()
    got_lse = lse[heads][:, tt].T.cpu().numpy()
    note(f"full size {name}: oracle on {len(toks)} rows x {len(heads)} heads")
    ref, ref_lse = orc.hybrid_attention_rows(c.q_f32(), c.k_f32(), c.v_f32(), modes, c.cu_seqlens,
                                             toks, heads, n_sink=c.n_sink,
                                             keep_fraction=c.keep_fraction)
    compare_o(got, ref, c.dtype)
    assert np.abs(got_lse - ref_lse).max() <= LSE_TOL
    assert bool(torch.isfinite(O).all())


def test_plan_then_run_equals_one_shot_and_plan_is_reusable():
    import full_attention_long_amd as ea
    from gpu_helpers import max_seqlen
    c = gen.custom_case(13, [1500, 0, 700], 8, 2, 128, "bf16")
    modes = np.array([[1, 0], [0, 1], [0, 1]], np.int8)
    note("plan/run vs one-shot")
    one, lone = gpu_prefill(c, modes)
    dv = to_device(c)
    m = torch.from_numpy(modes).cuda()
    n = ea.ea_hybrid_prefill_workspace_size(c.B, c.T, max_seqlen(c), c.Hq, c.Hkv, c.d, 1)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    ea.ea_hybrid_prefill_plan(m, dv["cu"], c.T, max_seqlen(c), c.Hq, c.Hkv, c.d, 1, ws)
    for _ in range(2):
        o, l = ea.ea_hybrid_prefill_run(dv["q"], dv["k"], dv["v"], m, dv["cu"], max_seqlen(c), ws)
        torch.cuda.synchronize()
        assert torch.equal(o, one) and torch.equal(l, lone)


def test_run_over_unplanned_workspace_writes_nothing():
    import full_attention_long_amd as ea
    from gpu_helpers import max_seqlen
    c = gen.custom_case(14, [900], 8, 2, 128, "bf16")
    dv = to_device(c)
    m = torch.zeros((1, 2), dtype=torch.int8, device="cuda")
    n = ea.ea_hybrid_prefill_workspace_size(c.B, c.T, max_seqlen(c), c.Hq, c.Hkv, c.d, 1)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    out = torch.full_like(dv["q"], 7.0)
    note("run over a zeroed (unplanned) workspace")
    ea.ea_hybrid_prefill_run(dv["q"], dv["k"], dv["v"], m, dv["cu"], max_seqlen(c), ws, out=out,
                             with_lse=False)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
