"""The bench's closed-form effective-FLOP count and window rule agree with the
oracle's brute-force count over the visibility predicate."""
import numpy as np
import pytest

from full_attention_long_amd import metrics
from oracle import ea_oracle as orc


@pytest.mark.parametrize("lengths,ns,rho,wb", [
    ([32768], 2, 0.2, 0), ([512], 1, 0.2, 0), ([1000, 1, 64, 65, 0, 4097], 1, 0.2, 0),
    ([777, 3000], 0, 0.3, 0), ([5000], 3, 0.2, 7), ([200], 4, 0.1, 0), ([12345, 64 * 40], 2, 0.15, 0),
])
def test_effective_flops_matches_oracle(lengths, ns, rho, wb):
    rng = np.random.default_rng(len(lengths) * 7 + ns)
    B, Hkv, Hq, d = len(lengths), 4, 8, 128
    modes = rng.integers(0, 2, size=(B, Hkv)).astype(np.int8)
    modes[0, 0], modes[0, 1] = 0, 1
    cu = np.concatenate([[0], np.cumsum(lengths)])
    ref = orc.effective_flops(modes, cu, Hq, Hkv, d, n_sink=ns, keep_fraction=rho, window_blocks=wb)
    got = metrics.effective_flops(modes, lengths, Hq, Hkv, d, n_sink=ns, keep_fraction=rho,
                                  window_blocks_=wb)
    assert got == ref


@pytest.mark.parametrize("L", [1, 63, 64, 65, 512, 32768, 131072, 262144, 4097 * 64 + 3])
@pytest.mark.parametrize("ns,rho", [(1, 0.2), (2, 0.2), (4, 0.1), (0, 0.35)])
def test_window_rule_matches_oracle(L, ns, rho):
    assert metrics.window_blocks(L, ns, rho) == orc.sa_geometry(L, 64, ns, 0, rho)[1]


def test_headline_effective_flops():
    # 128K, 32/8 heads, d = 128, 6 of 8 KV heads sparse at rho = 0.2, one sink block
    m = np.array([[1, 1, 0, 1, 0, 1, 1, 1]])
    ef = metrics.effective_flops(m, [131072], 32, 8, 128, n_sink=1, keep_fraction=0.2)
    assert abs(ef - 7.324e13) / 7.324e13 < 1e-3


def test_xa_effective_flops_matches_oracle_count():
    # host bookkeeping of an XA layer vs the oracle's count over the same keep flags
    from oracle import xa_oracle as xo
    from full_attention_long_amd import metrics as mt
    rng = np.random.default_rng(5)
    lengths = np.array([1000, 300, 129])
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    Hq, Hkv, d = 8, 4, 64
    modes = np.array([[1, 0, 1, 1], [0, 1, 1, 0], [1, 1, 1, 1]], np.int8)
    for cfg in ("FA-XA", "XA-SSA", "FA-SSA"):
        cm = mt.computation_modes(modes, cfg)
        assert np.array_equal(cm, xo.computation_modes(modes, cfg))
        nqb = -(-int(lengths.max()) // 128)
        keep = np.zeros((3, Hq, nqb, nqb), np.uint8)
        plan = {}
        for b, L in enumerate(lengths):
            nb = -(-int(L) // 128)
            for hq in range(Hq):
                if cm[b, hq // 2] != 2:
                    continue
                sel = np.tril(rng.random((nb, nb)) < 0.4)
                sel[:, 0] = True
                sel[np.arange(nb), np.arange(nb)] = True
                sel = np.tril(sel)
                keep[b, hq, :nb, :nb] = sel
                plan[(b, hq)] = (None, sel)
        got = mt.xa_effective_flops(cm, keep, lengths, Hq, Hkv, d, n_sink=1, keep_fraction=0.2)
        want = xo.xa_effective_flops(cm, cu, Hq, Hkv, d, plan)
        assert got == want, cfg


def test_xa_selection_flops_closed_form():
    # one scoring of every causal 16 x 16 group tile (S = 8, d = 128):
    # 2 * 16 * 16 * 8 * 128 FLOP per tile, nb (nb + 1) / 2 tiles per XA query head
    from full_attention_long_amd import metrics as mt
    cm = np.array([[2, 1], [0, 2]])
    lengths = np.array([1024, 300])
    got = mt.xa_selection_flops(cm, lengths, 8, 2, 128)
    tile = 2 * 16 * 16 * 8 * 128
    assert got == 4 * tile * (8 * 9 // 2) + 4 * tile * (3 * 4 // 2)
