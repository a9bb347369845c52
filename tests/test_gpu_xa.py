"""GPU parity of the XAttention (XA) head mode against the CPU oracle, through
the C ABI.

Block masses (float32 on the GPU, float64 in the oracle) must agree within
2e-4.  The keep decisions are integers decided by float sums, so they are
compared where the oracle's decision is not a near-tie (the kept mass before
the last kept block and the mass at the stopping point both at least 1e-3 away
from the target, and the last kept and first dropped candidates at least 1e-3
apart): there they must match exactly, and near-ties must be rare.  Outputs
are compared against the oracle's attention over the oracle's own selection,
on every row of FA / SA heads and on the XA rows whose keep row matched:
max-abs 2e-2, mean-abs 1e-3 (bf16), LSE 1e-4."""
import numpy as np
import pytest
import torch

import full_attention_long_amd as ea
from gpu_helpers import LSE_TOL, compare_o, max_seqlen, note, o_to_numpy, to_device
from oracle import xa_oracle as xa
from workloads import gen
from workloads.configs import WORKLOADS

pytestmark = pytest.mark.gpu

MASS_TOL = 2e-4
TIE = 1e-3


def robust(row, i, tau):
    """Whether the oracle's keep decision for query block i is clear of ties."""
    a = np.asarray(row[:i + 1], np.float64)
    if i < 2:
        return True
    target = tau * a.sum()
    cand = sorted(range(1, i), key=lambda j: (-a[j], j))
    vals = a[cand]
    got = a[0] + a[i] + np.concatenate([[0.0], np.cumsum(vals)])  # before candidate p
    k = int(np.argmax(got >= target)) if (got >= target).any() else len(vals)
    if k < len(vals) and got[k] - target <= TIE:
        return False
    if k >= 1 and target - got[k - 1] <= TIE:
        return False
    if 1 <= k < len(vals) and vals[k - 1] - vals[k] <= TIE:
        return False
    return True


def run_xa(c, modes, config, tau, dv=None):
    dv = dv or to_device(c)
    m = torch.from_numpy(np.ascontiguousarray(modes, np.int8)).cuda()
    nqb = -(-max_seqlen(c) // 128)
    mass = torch.full((c.B, c.Hq, nqb, nqb), -1.0, dtype=torch.float32, device="cuda")
    keep = torch.full((c.B, c.Hq, nqb, nqb), 7, dtype=torch.uint8, device="cuda")
    O, lse = ea.ea_xa_prefill(dv["q"], dv["k"], dv["v"], m, dv["cu"], max_seqlen(c),
                              head_config=config, threshold=tau, n_sink=c.n_sink,
                              window_blocks=c.window_blocks, keep_fraction=c.keep_fraction,
                              mass=mass, keep=keep)
    torch.cuda.synchronize()
    return O, lse, mass.cpu().numpy(), keep.cpu().numpy()


def check_plan(c, cmodes, mass, keep, plan, tau):
    """Masses within MASS_TOL; keep rows equal where robust.  Returns the set of
    (b, hq, i) rows whose keep row matched, and the count of near-tie rows."""
    matched, ties, rows = set(), 0, 0
    G = c.Hq // c.Hkv
    for (b, hq), (A, sel) in plan.items():
        nb = A.shape[0]
        for i in range(nb):
            rows += 1
            got = mass[b, hq, i, :i + 1]
            err = np.abs(got - A[i, :i + 1]).max()
            assert err <= MASS_TOL, f"mass b={b} hq={hq} i={i}: {err:.2e}"
            gk = keep[b, hq, i, :i + 1].astype(bool)
            assert gk[0] and gk[i], f"forced blocks b={b} hq={hq} i={i}"
            if (gk == sel[i, :i + 1]).all():
                matched.add((b, hq, i))
            elif robust(A[i], i, tau):
                raise AssertionError(f"keep row b={b} hq={hq} i={i} differs away from a tie: "
                                     f"{np.nonzero(gk != sel[i, :i + 1])[0][:8]}")
            else:
                ties += 1
    # heads that are not XA leave the outputs untouched
    for b in range(c.B):
        for hq in range(c.Hq):
            if cmodes[b, hq // G] != xa.MODE_XA:
                assert (mass[b, hq] == -1.0).all() and (keep[b, hq] == 7).all()
    assert ties <= max(2, rows // 50), f"{ties} near-tie rows of {rows}"
    return matched


class Bf16View:
    """float32 values of a bf16-bit array, converted only where indexed (the
    full-size case reads a few rows and heads of multi-GiB tensors)."""

    def __init__(self, bits):
        self.bits = bits
        self.shape = bits.shape

    def __getitem__(self, idx):
        return gen.bf16_bits_to_f32(np.ascontiguousarray(self.bits[idx]))


def compare_rows(c, cmodes, O, lse, plan, matched, tokens=None, heads=None):
    """O / LSE against the oracle on FA/SA heads and matched XA rows."""
    G = c.Hq // c.Hkv
    tokens = np.arange(c.T) if tokens is None else np.asarray(tokens)
    heads = list(range(c.Hq)) if heads is None else list(heads)
    ref_o, ref_l = xa.hybrid_attention_xa(Bf16View(c.q), Bf16View(c.k), Bf16View(c.v), cmodes,
                                          c.cu_seqlens,
                                          plan, n_sink=c.n_sink, window_blocks=c.window_blocks,
                                          keep_fraction=c.keep_fraction, tokens=tokens, heads=heads)
    seg = np.searchsorted(c.cu_seqlens, tokens, side="right") - 1
    pos = tokens - c.cu_seqlens[seg]
    tt = torch.from_numpy(tokens).cuda()
    got_o = O[tt][:, heads].float().cpu().numpy()
    got_l = lse[heads][:, tt].T.cpu().numpy()
    ok = np.ones((len(tokens), len(heads)), bool)
    for hi, hq in enumerate(heads):
        for ti in range(len(tokens)):
            b = int(seg[ti])
            if cmodes[b, hq // G] == xa.MODE_XA and (b, hq, int(pos[ti]) // 128) not in matched:
                ok[ti, hi] = False
    assert ok.mean() > 0.9
    compare_o(got_o[ok], ref_o[ok], "bf16")
    assert np.abs(got_l[ok] - ref_l[ok]).max() <= LSE_TOL


CASES = [
    # lengths, Hq, Hkv, d, config, modes (per sequence), tau, hitters
    ([3000], 8, 2, 128, "XA-SSA", [[0, 1]], 0.9, None),
    ([1500, 700, 129], 8, 4, 64, "FA-XA", [[1, 0, 1, 1], [0, 1, 1, 0], [1, 1, 1, 1]], 0.9, None),
    ([2049], 16, 2, 128, "XA-SSA", [[0, 0]], 0.5, None),
    ([1000, 3], 32, 2, 64, "FA-XA", [[1, 1], [1, 0]], 0.7, None),
    ([4096], 8, 2, 128, "XA-SSA", [[0, 1]], 0.0, None),
    ([2000], 8, 2, 128, "FA-XA", [[1, 1]], 1.0, None),
    ([6000], 8, 2, 128, "XA-SSA", [[0, 0]], 0.9, (0.1, 8.0)),
    ([5000, 1100], 16, 4, 128, "FA-XA", [[1, 0, 1, 1], [1, 1, 0, 1]], 0.9, (0.05, 8.0)),
    ([0, 50, 1300, 7], 8, 2, 128, "XA-SSA", [[0, 0], [0, 1], [0, 0], [1, 0]], 0.9, None),
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_xa_prefill_small(case):
    lengths, Hq, Hkv, d, config, modes, tau, hitters = case
    c = gen.custom_case(700 + Hq + d + len(lengths), lengths, Hq, Hkv, d, "bf16", n_sink=1,
                        keep_fraction=0.2, hitters=hitters)
    modes = np.asarray(modes, np.int8)
    cmodes = xa.computation_modes(modes, config)
    note(f"xa {config} lengths={lengths} Hq={Hq} Hkv={Hkv} d={d} tau={tau} hitters={hitters}")
    O, lse, mass, keep = run_xa(c, modes, config, tau)
    plan = xa.xa_plan(c.q_f32(), c.k_f32(), cmodes, c.cu_seqlens, tau=tau)
    matched = check_plan(c, cmodes, mass, keep, plan, tau)
    compare_rows(c, cmodes, O, lse, plan, matched)


def test_xa_fa_ssa_config_is_the_routed_prefill_bitwise():
    # with no XA head the XA entry point runs the routed prefill's work
    c = gen.custom_case(77, [3333, 500], 8, 2, 128, "bf16", n_sink=1, keep_fraction=0.2)
    dv = to_device(c)
    modes = np.array([[1, 0], [0, 1]], np.int8)
    note("xa FA-SSA vs routed prefill")
    O, lse, mass, keep = run_xa(c, modes, "FA-SSA", 0.9, dv)
    m = torch.from_numpy(modes).cuda()
    R, RL = ea.ea_hybrid_prefill(dv["q"], dv["k"], dv["v"], m, dv["cu"], max_seqlen(c))
    torch.cuda.synchronize()
    assert torch.equal(O, R) and torch.equal(lse, RL)
    assert (mass == -1.0).all() and (keep == 7).all()


def test_xa_full_size_sampled():
    wl = WORKLOADS["qwen4b_s128k_sa2"]
    note("xa full size qwen4b_s128k XA-SSA: generating")
    c = gen.build_case(wl, hitters=(0.1, 8.0))
    modes = c.target_modes
    cmodes = xa.computation_modes(modes, "XA-SSA")
    dv = to_device(c)
    note(f"xa full size: prefill T={c.T}")
    O, lse, mass, keep = run_xa(c, modes, "XA-SSA", 0.9, dv)
    del dv
    L = int(c.lengths[0])
    nb = L // 128
    xa_heads = [hq for hq in range(c.Hq) if cmodes[0, hq // 4] == xa.MODE_XA]
    heads = [xa_heads[0], xa_heads[-1], next(h for h in range(c.Hq) if h not in xa_heads)]
    rows = [0, 1, 204, 511, nb - 1]
    scale = 1.0 / np.sqrt(c.d)
    plan = {}
    matched = set()
    note(f"xa full size: oracle masses of {len(rows)} query blocks x heads {heads[:2]}")
    for hq in heads[:2]:
        A = xa.block_mass_rows(Bf16View(c.q)[:, hq], Bf16View(c.k)[:, hq // 4], rows, scale=scale)
        sel = np.zeros((nb, nb), bool)
        for ri, i in enumerate(rows):
            err = np.abs(mass[0, hq, i, :i + 1] - A[ri, :i + 1]).max()
            assert err <= MASS_TOL, f"mass hq={hq} i={i}: {err:.2e}"
            sel[i, :i + 1] = xa.select_row(A[ri], i, 0.9)
            gk = keep[0, hq, i, :i + 1].astype(bool)
            if (gk == sel[i, :i + 1]).all():
                matched.add((0, hq, i))
            else:
                assert not robust(A[ri], i, 0.9), f"keep row hq={hq} i={i} differs away from a tie"
        plan[(0, hq)] = (None, sel)
    # sparsity of the selection the kernel made: far below dense on this input
    dens = (keep[0, xa_heads] == 1).sum() / (len(xa_heads) * nb * (nb + 1) / 2)
    note(f"xa full size: kept-block density {dens:.3f}")
    assert dens < 0.5
    toks = np.array([i * 128 + o for i in rows for o in (0, 77, 127)])
    compare_rows(c, cmodes, O, lse, plan, matched, tokens=toks, heads=heads)
    assert bool(torch.isfinite(O).all()) and bool(torch.isfinite(lse).all())


def test_xa_long_rows_sort_in_half_batches():
    """A sequence of more than 1,025 XA blocks at d = 64: each row then has
    2,048 sort slots, two rows no longer fit one key tile, and the selection
    sorts its rows four at a time.  Masses and keep rows of sampled query
    blocks against the oracle, and the keep flags of every row are a valid
    selection: blocks 0 and i kept, nothing past i."""
    L = 1100 * 128 + 45
    c = gen.custom_case(131, [L], 8, 2, 64, "bf16", n_sink=1, keep_fraction=0.2,
                        hitters=(0.1, 8.0))
    modes = np.array([[1, 1]], np.int8)  # FA-XA: both KV heads in XA mode
    cmodes = xa.computation_modes(modes, "FA-XA")
    note(f"xa long rows d=64 L={L}")
    O, lse, mass, keep = run_xa(c, modes, "FA-XA", 0.9)
    nb = -(-L // 128)
    rows = [0, 2, 700, 1026, nb - 1]
    scale = 1.0 / np.sqrt(c.d)
    for hq in (0, 5):
        A = xa.block_mass_rows(Bf16View(c.q)[:, hq], Bf16View(c.k)[:, hq // 4], rows, scale=scale)
        for ri, i in enumerate(rows):
            err = np.abs(mass[0, hq, i, :i + 1] - A[ri, :i + 1]).max()
            assert err <= MASS_TOL, f"mass hq={hq} i={i}: {err:.2e}"
            want = xa.select_row(A[ri], i, 0.9)
            gk = keep[0, hq, i, :i + 1].astype(bool)
            if not (gk == want).all():
                assert not robust(A[ri], i, 0.9), f"keep row hq={hq} i={i} differs away from a tie"
    k = keep[0]
    assert (k[:, np.arange(nb), 0] == 1).all() and (k[:, np.arange(nb), np.arange(nb)] == 1).all()
    iu, ju = np.triu_indices(nb, 1)
    il, jl = np.tril_indices(nb)
    assert (k[:, iu, ju] == 7).all() and np.isin(k[:, il, jl], (0, 1)).all()
    assert bool(torch.isfinite(O).all()) and bool(torch.isfinite(lse).all())


def test_xa_plan_and_run_equal_the_one_shot_call():
    c = gen.custom_case(91, [2500, 900], 8, 2, 128, "bf16", n_sink=1, keep_fraction=0.2,
                        hitters=(0.1, 8.0))
    dv = to_device(c)
    modes = np.array([[0, 1], [1, 0]], np.int8)
    note("xa plan + run vs one-shot")
    O, lse, mass, keep = run_xa(c, modes, "XA-SSA", 0.9, dv)
    m = torch.from_numpy(modes).cuda()
    ws = torch.empty(ea.ea_xa_prefill_workspace_size(c.B, c.T, max_seqlen(c), c.Hq, c.Hkv, c.d, 1),
                     dtype=torch.uint8, device="cuda")
    ea.ea_xa_prefill_plan(dv["q"], dv["k"], m, dv["cu"], max_seqlen(c), ws, head_config="XA-SSA")
    O2, lse2 = ea.ea_xa_prefill_run(dv["q"], dv["k"], dv["v"], m, dv["cu"], max_seqlen(c), ws,
                                    head_config="XA-SSA")
    # a second run over the same plan gives the same result
    O3, lse3 = ea.ea_xa_prefill_run(dv["q"], dv["k"], dv["v"], m, dv["cu"], max_seqlen(c), ws,
                                    head_config="XA-SSA")
    torch.cuda.synchronize()
    assert torch.equal(O, O2) and torch.equal(lse, lse2)
    assert torch.equal(O2, O3) and torch.equal(lse2, lse3)
