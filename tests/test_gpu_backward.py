"""GPU parity of the hybrid-layer backward (dQ, dK, dV) against the CPU
oracle, through the C ABI.  The forward's O and LSE come from the library's
own forward on the same inputs, as in a training step; the oracle uses its
exact values.  Gradients are compared relative to the largest reference
magnitude of each tensor: max-abs error <= 1.5e-2 and mean-abs error <= 1.5e-3
of it (bf16 operands, float32 accumulation)."""
import numpy as np
import pytest
import torch

import full_attention_long_amd as ea
from gpu_helpers import dev_tensor, max_seqlen, note, to_device
from oracle import ea_oracle as orc
from workloads import gen

pytestmark = pytest.mark.gpu

REL_MAX, REL_MEAN = 1.5e-2, 1.5e-3


def compare_grad(got, ref, what):
    g = got.float().cpu().numpy().astype(np.float64)
    scale = max(float(np.abs(ref).max()), 1e-30)
    err = np.abs(g - ref)
    mx, mean = float(err.max()) / scale, float(err.mean()) / scale
    note(f"{what}: max-abs {mx:.2e} mean-abs {mean:.2e} of max |ref| {scale:.3e}")
    assert np.isfinite(g).all(), f"{what}: non-finite"
    assert mx <= REL_MAX, f"{what}: max-abs {mx:.2e} of max |ref| > {REL_MAX}"
    assert mean <= REL_MEAN, f"{what}: mean-abs {mean:.2e} of max |ref| > {REL_MEAN}"


CASES = [
    # lengths, Hq, Hkv, d, n_sink, rho, window_blocks
    ([1000], 8, 2, 128, 1, 0.2, 0),
    ([300, 0, 1, 777, 64, 129], 8, 2, 128, 1, 0.2, 0),
    ([2000], 4, 4, 128, 1, 0.2, 0),          # G = 1: query tiles of 256 positions
    ([700], 6, 2, 64, 1, 0.25, 0),           # G = 3
    ([1500], 16, 2, 128, 2, 0.3, 0),
    ([1300], 8, 1, 128, 0, 0.2, 1),          # n_sink = 0, w = 1
    ([900, 455], 8, 2, 64, 1, 0.2, 100),     # window covers the sequence: SA == FA
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_backward_small(case):
    lengths, Hq, Hkv, d, ns, rho, wb = case
    c = gen.custom_case(500 + len(lengths) + Hq + d, lengths, Hq, Hkv, d, "bf16", n_sink=ns,
                        keep_fraction=rho, window_blocks=wb)
    rng = np.random.default_rng(11)
    modes = rng.integers(0, 2, size=(len(lengths), Hkv)).astype(np.int8)
    modes[0, 0] = 1
    if Hkv > 1:
        modes[0, 1] = 0
    dob = gen.bf16_bits(gen.normal(77 + Hq, 30, (c.T, Hq, d)))
    note(f"backward lengths={lengths} Hq={Hq} Hkv={Hkv} d={d} ns={ns} rho={rho} wb={wb} "
         f"modes={modes.tolist()}")
    dv = to_device(c)
    m = torch.from_numpy(modes).cuda()
    geom = dict(n_sink=ns, window_blocks=wb, keep_fraction=rho)
    O, lse = ea.ea_hybrid_prefill(dv["q"], dv["k"], dv["v"], m, dv["cu"], max_seqlen(c), **geom)
    dO = dev_tensor(dob, "bf16")
    dQ, dK, dV = ea.ea_hybrid_backward(dv["q"], dv["k"], dv["v"], O, dO, lse, m, dv["cu"],
                                       max_seqlen(c), **geom)
    torch.cuda.synchronize()
    ref = orc.hybrid_attention_backward(c.q_f32(), c.k_f32(), c.v_f32(),
                                        gen.bf16_bits_to_f32(dob), modes, c.cu_seqlens, **geom)
    for got, r, what in zip((dQ, dK, dV), ref, ("dQ", "dK", "dV")):
        compare_grad(got, r, what)


def test_backward_bitwise_deterministic():
    c = gen.custom_case(9, [1777], 8, 2, 128, "bf16", n_sink=1, keep_fraction=0.2)
    dv = to_device(c)
    m = torch.tensor([[1, 0]], dtype=torch.int8, device="cuda")
    O, lse = ea.ea_hybrid_prefill(dv["q"], dv["k"], dv["v"], m, dv["cu"], max_seqlen(c))
    dO = torch.randn_like(dv["q"].float()).to(torch.bfloat16)
    a = ea.ea_hybrid_backward(dv["q"], dv["k"], dv["v"], O, dO, lse, m, dv["cu"], max_seqlen(c))
    b = ea.ea_hybrid_backward(dv["q"], dv["k"], dv["v"], O, dO, lse, m, dv["cu"], max_seqlen(c))
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("name", ["qwen4b_s128k_sa2"])
def test_backward_full_size_sampled(name):
    """The 128K layer the backward is benchmarked on: dQ at sampled rows of
    every query head of one FA and one SA KV group (rows at the start, the
    middle and the end, where dQ sums over up to 131K keys), and dK, dV at
    keys in the last three 64-key blocks of both groups (each summed over the
    rows that see it, across the group's four query heads).  The oracle forms
    its own P, dP and D for every row involved (hybrid_attention_backward_rows,
    pinned to autograd on small cases)."""
    from workloads.configs import WORKLOADS
    wl = WORKLOADS[name]
    note(f"backward full size {name}: generating")
    c = gen.build_case(wl)
    modes = np.asarray(c.target_modes, np.int8)
    L, G = c.T, c.Hq // c.Hkv
    dob = gen._draw_rows(901, 31, c.T, (c.Hq, c.d), 1.0, "bf16")
    dv = to_device(c)
    m = torch.from_numpy(modes).cuda()
    geom = dict(n_sink=c.n_sink, keep_fraction=c.keep_fraction)
    note(f"backward full size {name}: forward and backward on the GPU, T={c.T}")
    O, lse = ea.ea_hybrid_prefill(dv["q"], dv["k"], dv["v"], m, dv["cu"], L, **geom)
    dO = dev_tensor(dob, "bf16")
    dQ, dK, dV = ea.ea_hybrid_backward(dv["q"], dv["k"], dv["v"], O, dO, lse, m, dv["cu"], L, **geom)
    torch.cuda.synchronize()
    del dv, O, lse, dO
    rng = np.random.default_rng(21)
    qt = np.unique(np.concatenate([[0, 63, 64, 4000, L // 2 + 17, L - 65, L - 64, L - 1],
                                   rng.integers(0, L, size=8)]))
    kt = np.unique(np.concatenate([[L - 192, L - 129, L - 128, L - 65, L - 64, L - 1],
                                   rng.integers(L - 192, L, size=6)]))
    groups = [int(np.nonzero(modes[0] == 0)[0][0]), int(np.nonzero(modes[0] == 1)[0][0])]
    qf, kf, vf = c.q_f32(), c.k_f32(), c.v_f32()
    dof = gen.bf16_bits_to_f32(dob)
    tq, tk = torch.from_numpy(qt).cuda(), torch.from_numpy(kt).cuda()
    for g in groups:
        hs = list(range(g * G, (g + 1) * G))
        note(f"backward full size {name}: oracle for KV group {g} (mode {modes[0, g]}), "
             f"{len(qt)} query rows, {len(kt)} keys")
        ref_dq, ref_dk, ref_dv = orc.hybrid_attention_backward_rows(
            np.ascontiguousarray(qf[:, hs]), np.ascontiguousarray(kf[:, [g]]),
            np.ascontiguousarray(vf[:, [g]]), np.ascontiguousarray(dof[:, hs]), modes[:, [g]],
            c.cu_seqlens, qt, kt, **geom)
        compare_grad(dQ[tq][:, hs], ref_dq, f"dQ group {g}")
        compare_grad(dK[tk][:, [g]], ref_dk, f"dK group {g}")
        compare_grad(dV[tk][:, [g]], ref_dv, f"dV group {g}")
