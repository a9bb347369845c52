"""The seeded generator: determinism, the bf16 encoding, and that the stored
routing controls make the oracle router produce each workload's target split
with the required margin."""
import numpy as np
import pytest
import torch

from oracle.ea_oracle import route
from workloads import gen
from workloads.configs import WORKLOADS


def test_same_seed_same_draws_any_thread_count(monkeypatch):
    a = gen.custom_case(7, [5000, 3000], 4, 2, 64, "bf16")
    monkeypatch.setattr(gen, "_threads", lambda: 1)
    b = gen.custom_case(7, [5000, 3000], 4, 2, 64, "bf16")
    for x, y in [(a.q, b.q), (a.k, b.k), (a.v, b.v)]:
        np.testing.assert_array_equal(x, y)
    c = gen.custom_case(8, [5000, 3000], 4, 2, 64, "bf16")
    assert not np.array_equal(a.q, c.q)


def test_bf16_encoding_is_round_to_nearest_even():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 10
    x = np.concatenate([x, np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3e38, -2.5e-39],
                                    np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(gen.bf16_bits(x), ref)
    back = gen.bf16_bits_to_f32(gen.bf16_bits(x))
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_varlen_lengths_in_range_and_ragged():
    wl = WORKLOADS["varlen8"]
    lens = gen.workload_lengths(wl, wl.start_seed)
    assert len(lens) == 8 and lens.min() >= 4096 and lens.max() < 65536
    assert (lens % 64 != 0).any()


def test_value_distributions():
    c = gen.custom_case(3, [20000], 4, 2, 128, "bf16", k_std=0.5)
    assert abs(c.q_f32().std() - 1.0) < 0.01 and abs(c.k_f32().std() - 0.5) < 0.01
    c = gen.custom_case(3, [20000], 4, 2, 128, "bf16", lowrank=8)
    assert abs(c.k_f32().std() - np.sqrt(2.0)) < 0.05


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_stored_controls_give_target_routing_with_margin(name):
    wl = WORKLOADS[name]
    ctl = gen.load_control()[name]
    seed = int(ctl["seed"])
    shift = None if ctl["shift"] is None else np.asarray(ctl["shift"], np.float32)
    lengths, cu, k = gen.workload_k(wl, seed, shift)
    kf = gen.bf16_bits_to_f32(k) if wl.dtype == "bf16" else k
    w = gen.draw_router_weights(seed, wl.d, wl.task_hidden, wl.router_hidden, wl.w_std)
    if ctl["b4"] is not None:
        w["b4"] = np.asarray(ctl["b4"], np.float32)
    modes, z = route(kf, cu, w, wl.pool_len)
    np.testing.assert_array_equal(modes, np.asarray(ctl["target_modes"], np.int8))
    assert np.abs(z[..., 0] - z[..., 1]).min() >= 1e-3
    if wl.sa_heads is not None:
        assert list(modes.sum(axis=1)) == list(wl.sa_heads)


def test_build_case_applies_controls():
    wl = WORKLOADS["tiny_f32_s512"]
    c = gen.build_case(wl)
    assert c.dtype == "f32" and c.q.dtype == np.float32 and c.T == 512
    assert c.target_modes is not None and c.target_modes.shape == (1, 2)
