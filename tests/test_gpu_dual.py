"""GPU parity of the training forward (Gumbel-Softmax routing with
straight-through hard decisions, and the dual-mode attention) against the CPU
oracle, through the C ABI.

Hard decisions must match bit for bit (both sides take them in float32 on the
same inputs); r_soft within 1e-6; O, O_FA, O_SA within max-abs 1e-5 (fp32) or
2e-2 / mean-abs 1e-3 (bf16); LSEs within 1e-4."""
import numpy as np
import pytest
import torch

import full_attention_long_amd as ea
from gpu_helpers import LSE_TOL, compare_o, dev_tensor, max_seqlen, note, o_to_numpy, to_device
from oracle import ea_oracle as orc
from workloads import gen
from workloads.configs import WORKLOADS

pytestmark = pytest.mark.gpu


def _route_inputs(seed, B, Hkv, scale=2.0):
    z = gen.normal(seed, 20, (B, Hkv, 2), std=scale)
    g = gen.draw_gumbel(seed, (B, Hkv, 2))
    return z, g


@pytest.mark.parametrize("tau", [0.1, 0.5, 1.0, 3.0])
def test_gumbel_route_matches_oracle(tau):
    z, g = _route_inputs(11, 64, 8)
    # a few exact ties and near-ties
    z[0, 0] = [0.25, 0.25]
    g[0, 0] = [0.0, 0.0]
    z[0, 1] = [1.0, np.nextafter(np.float32(1.0), np.float32(2.0))]
    g[0, 1] = [0.0, 0.0]
    note(f"gumbel route tau={tau}")
    for noise in (g, None):
        zt = torch.from_numpy(z).cuda()
        gt = None if noise is None else torch.from_numpy(noise).cuda()
        r_soft, modes = ea.ea_gumbel_route(zt, tau, gumbel=gt)
        torch.cuda.synchronize()
        ref_r, ref_m = orc.gumbel_route(z, noise, tau)
        np.testing.assert_array_equal(modes.cpu().numpy(), ref_m)
        np.testing.assert_allclose(r_soft.cpu().numpy(), ref_r, rtol=0, atol=1e-6)
        if noise is None:
            assert ref_m[0, 0] == 0  # an exact tie goes to FA on both sides


CASES = [
    # lengths, Hq, Hkv, d, dtype, n_sink, rho, window_blocks
    ([1000], 8, 2, 128, "bf16", 1, 0.2, 0),
    ([300, 0, 1, 777, 64, 129], 8, 2, 128, "bf16", 1, 0.2, 0),
    ([2000], 4, 4, 128, "bf16", 1, 0.2, 0),        # G = 1: tiles of 256 positions, 4 blocks
    ([700], 6, 2, 64, "bf16", 1, 0.25, 0),         # G = 3: tiles straddle blocks
    ([1500], 16, 2, 128, "bf16", 2, 0.3, 0),
    ([3000], 8, 1, 128, "bf16", 0, 0.2, 1),        # n_sink = 0, w = 1: middle = all but the diagonal
    ([2500], 8, 2, 128, "bf16", 1, 0.2, 100),      # window covers the sequence: empty middle set
    ([600, 33], 8, 2, 128, "f32", 1, 0.2, 0),
    ([513, 64, 65], 4, 2, 64, "f32", 2, 0.3, 0),
    ([1200], 4, 1, 128, "f32", 0, 0.2, 1),
]


def _gpu_dual(c, modes, dv=None):
    dv = dv or to_device(c)
    m = None if modes is None else torch.from_numpy(np.ascontiguousarray(modes, np.int8)).cuda()
    res = ea.ea_dual_prefill(dv["q"], dv["k"], dv["v"], dv["cu"], max_seqlen(c), modes=m,
                             n_sink=c.n_sink, window_blocks=c.window_blocks,
                             keep_fraction=c.keep_fraction, softmax_scale=c.softmax_scale)
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_dual_prefill_small(case):
    lengths, Hq, Hkv, d, dtype, ns, rho, wb = case
    c = gen.custom_case(300 + len(lengths) + Hq + d, lengths, Hq, Hkv, d, dtype, n_sink=ns,
                        keep_fraction=rho, window_blocks=wb)
    z, g = _route_inputs(5 + Hq, len(lengths), Hkv)
    r_soft, modes = orc.gumbel_route(z, g, 0.7)
    note(f"dual {dtype} lengths={lengths} Hq={Hq} Hkv={Hkv} d={d} ns={ns} rho={rho} wb={wb}")
    O, O_fa, O_sa, lse_fa, lse_sa = _gpu_dual(c, modes)
    ref = orc.dual_attention(c.q_f32(), c.k_f32(), c.v_f32(), c.cu_seqlens, r_soft, modes,
                             n_sink=ns, window_blocks=wb, keep_fraction=rho)
    for got, want, what in [(O, ref[0], "O"), (O_fa, ref[1], "O_FA"), (O_sa, ref[2], "O_SA")]:
        compare_o(o_to_numpy(got), want, dtype, what)
    assert np.abs(lse_fa.cpu().numpy() - ref[3]).max() <= LSE_TOL
    assert np.abs(lse_sa.cpu().numpy() - ref[4]).max() <= LSE_TOL


def test_dual_sa_is_the_routed_sa_bitwise_and_mix_selects():
    c = gen.custom_case(41, [1777, 300], 8, 2, 128, "bf16", n_sink=1, keep_fraction=0.2)
    dv = to_device(c)
    modes = np.array([[1, 0], [0, 1]], np.int8)
    note("dual vs routed forward")
    O, O_fa, O_sa, lse_fa, lse_sa = _gpu_dual(c, modes, dv)
    m_sa = torch.ones((2, 2), dtype=torch.int8, device="cuda")
    m_fa = torch.zeros((2, 2), dtype=torch.int8, device="cuda")
    R_sa, L_sa = ea.ea_hybrid_prefill(dv["q"], dv["k"], dv["v"], m_sa, dv["cu"], max_seqlen(c))
    R_fa, L_fa = ea.ea_hybrid_prefill(dv["q"], dv["k"], dv["v"], m_fa, dv["cu"], max_seqlen(c))
    torch.cuda.synchronize()
    # the SA items are the routed forward's SA items: same blocks, same order
    assert torch.equal(O_sa, R_sa) and torch.equal(lse_sa, L_sa)
    # the merged FA output agrees with the one-pass FA forward to bf16 rounding
    assert (O_fa.float() - R_fa.float()).abs().max().item() <= 8e-3
    assert (lse_fa - L_fa).abs().max().item() <= 1e-5
    # the mix is a per-(sequence, KV head) selection
    cu = c.cu_seqlens
    for b in range(2):
        for hq in range(8):
            src = O_sa if modes[b, hq // 4] else O_fa
            assert torch.equal(O[cu[b]:cu[b + 1], hq], src[cu[b]:cu[b + 1], hq])
    # without modes there is no mix and the rest is unchanged
    O2, O_fa2, O_sa2, _, _ = _gpu_dual(c, None, dv)
    assert O2 is None and torch.equal(O_fa2, O_fa) and torch.equal(O_sa2, O_sa)


def test_dual_full_size_sampled():
    wl = WORKLOADS["qwen4b_s128k_sa6"]
    note("dual full size qwen4b_s128k: generating")
    c = gen.build_case(wl)
    dv = to_device(c)
    z, g = _route_inputs(9, c.B, c.Hkv)
    r_soft, modes = orc.gumbel_route(z, g, 1.0)
    note(f"dual full size qwen4b_s128k: prefill T={c.T}")
    O, O_fa, O_sa, lse_fa, lse_sa = _gpu_dual(c, modes, dv)
    del dv
    L = int(c.lengths[0])
    rng = np.random.default_rng(3)
    toks = np.unique(np.concatenate([[0, 63, 64, 26239, 26240, 26304, L - 1],
                                     rng.integers(0, L, 6)]))
    heads = [0, 5, 10, 15, 21, 31]
    tt = torch.from_numpy(toks).cuda()
    note(f"dual full size: oracle on {len(toks)} rows x {len(heads)} heads")
    ref = orc.dual_attention_rows(c.q_f32(), c.k_f32(), c.v_f32(), c.cu_seqlens, r_soft, modes,
                                  toks, heads, n_sink=c.n_sink, keep_fraction=c.keep_fraction)
    for got, want, what in [(O, ref[0], "O"), (O_fa, ref[1], "O_FA"), (O_sa, ref[2], "O_SA")]:
        compare_o(got[tt][:, heads].float().cpu().numpy(), want, c.dtype, what)
    assert np.abs(lse_fa[heads][:, tt].T.cpu().numpy() - ref[3]).max() <= LSE_TOL
    assert np.abs(lse_sa[heads][:, tt].T.cpu().numpy() - ref[4]).max() <= LSE_TOL
    for t in (O, O_fa, O_sa, lse_fa, lse_sa):
        assert bool(torch.isfinite(t).all())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_router_logit_grad_matches_oracle(dtype):
    lengths = [700, 0, 1, 333]
    c = gen.custom_case(61, lengths, 8, 2, 64, dtype, n_sink=1, keep_fraction=0.25)
    z, g = _route_inputs(17, len(lengths), 2)
    tau = 0.6
    zt, gt = torch.from_numpy(z).cuda(), torch.from_numpy(g).cuda()
    r_soft, modes = ea.ea_gumbel_route(zt, tau, gumbel=gt)
    note(f"router logit grad {dtype}")
    O, O_fa, O_sa, _, _ = _gpu_dual(c, modes.cpu().numpy())
    dOn = gen.normal(5, 40, (c.T, 8, 64))
    dO = dev_tensor(gen.bf16_bits(dOn) if dtype == "bf16" else dOn, dtype)
    dz, dr = ea.ea_router_logit_grad(dO, O_fa, O_sa, torch.from_numpy(c.cu_seqlens).cuda(),
                                     int(max(lengths)), r_soft, tau)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy()  # noqa: E731
    ref_dz, ref_dr = orc.router_logit_grad(f(dO), f(O_fa), f(O_sa), c.cu_seqlens,
                                           r_soft.cpu().numpy(), tau)
    s = max(float(np.abs(ref_dr).max()), 1e-30)
    assert np.abs(dr.cpu().numpy() - ref_dr).max() <= 1e-5 * s
    assert np.abs(dz.cpu().numpy() - ref_dz).max() <= 1e-5 * max(float(np.abs(ref_dz).max()), 1e-30) + 1e-6
    assert np.all(dr.cpu().numpy()[1] == 0)            # the empty sequence
    # reproducible bit for bit
    dz2, _ = ea.ea_router_logit_grad(dO, O_fa, O_sa, torch.from_numpy(c.cu_seqlens).cuda(),
                                     int(max(lengths)), r_soft, tau)
    assert torch.equal(dz, dz2)
