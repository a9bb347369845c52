"""GPU parity of decoding with the mode-aware KV cache against the CPU oracle,
through the C ABI: a prompt batch goes into the cache, then several decode
steps each append one token per sequence and attend; every step's output is
compared with the oracle over the full (never evicted) history.

O within max-abs 2e-2 / mean-abs 1e-3 (bf16), LSE within 1e-4."""
import numpy as np
import pytest
import torch

import full_attention_long_amd as ea
from gpu_helpers import LSE_TOL, compare_o, dev_tensor, note
from oracle import ea_oracle as orc
from workloads import gen
from workloads.configs import WORKLOADS

pytestmark = pytest.mark.gpu


def _bf16(seed, stream, shape):
    x = gen.normal(seed, stream, shape)
    return gen.bf16_bits(x), gen.bf16_bits_to_f32(gen.bf16_bits(x))


def run_decode(lengths, Hq, Hkv, d, modes, steps, *, max_len, check_every=1, seed=0, **geom):
    B = len(lengths)
    T = int(sum(lengths))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    kb, kf = _bf16(seed, 101, (T, Hkv, d))
    vb, vf = _bf16(seed, 102, (T, Hkv, d))
    cache = ea.KVCache(torch.from_numpy(modes), max_len, d, n_sink=geom.get("n_sink", 1),
                       window_blocks=geom.get("window_blocks", 0),
                       keep_fraction=geom.get("keep_fraction", 0.2))
    note(f"decode lengths={lengths} Hq={Hq} Hkv={Hkv} d={d} modes={modes.tolist()} geom={geom} "
         f"max_len={max_len} bytes={cache.nbytes}")
    cache.prefill(dev_tensor(kb, "bf16"), dev_tensor(vb, "bf16"), torch.from_numpy(cu).cuda())
    torch.cuda.synchronize()
    assert cache.lengths.cpu().tolist() == list(lengths)
    Kh = [kf[cu[b]:cu[b + 1]] for b in range(B)]
    Vh = [vf[cu[b]:cu[b + 1]] for b in range(B)]
    for step in range(steps):
        qb_, qf = _bf16(seed + step, 201, (B, Hq, d))
        knb, knf = _bf16(seed + step, 202, (B, Hkv, d))
        vnb, vnf = _bf16(seed + step, 203, (B, Hkv, d))
        O, lse = cache.decode(dev_tensor(qb_, "bf16"), dev_tensor(knb, "bf16"),
                              dev_tensor(vnb, "bf16"))
        torch.cuda.synchronize()
        Kh = [np.concatenate([Kh[b], knf[b:b + 1]]) for b in range(B)]
        Vh = [np.concatenate([Vh[b], vnf[b:b + 1]]) for b in range(B)]
        if step % check_every == 0 or step == steps - 1:
            ref, ref_lse = orc.decode_attention(qf, Kh, Vh, modes, **geom)
            compare_o(O.float().cpu().numpy(), ref, "bf16", f"O step {step}")
            assert np.abs(lse.cpu().numpy() - ref_lse).max() <= LSE_TOL, f"LSE step {step}"
    assert cache.lengths.cpu().tolist() == [L + steps for L in lengths]
    return cache


@pytest.mark.parametrize("d", [128, 64])
def test_decode_ring_wraps_fixed_window(d):
    # window of 2 blocks + 1 sink: SA slots are 3-block rings that wrap many times
    lengths = [100, 1000, 64 * 9 + 3, 1]
    modes = np.array([[1, 0], [1, 1], [0, 1], [1, 0]], np.int8)
    run_decode(lengths, 8, 2, d, modes, 140, max_len=2048, check_every=7, n_sink=1,
               window_blocks=2)


def test_decode_keep_fraction_window_grows():
    # w follows the length: 0.2 of the blocks; SA ring sized for max_len
    lengths = [1500, 3000]
    modes = np.array([[1, 1, 0, 1], [0, 1, 1, 1]], np.int8)
    run_decode(lengths, 16, 4, 128, modes, 130, max_len=4096, check_every=13, n_sink=1,
               keep_fraction=0.2)


def test_decode_gqa_shapes_and_sinks():
    # G = 16 (the most the decode MFMA packs), 2 sink blocks, n_sink = 0 elsewhere
    modes = np.array([[1], [0]], np.int8)
    run_decode([700, 64], 16, 1, 128, modes, 66, max_len=1024, check_every=11, n_sink=2,
               window_blocks=3)
    run_decode([333], 3, 1, 64, np.array([[1]], np.int8), 70, max_len=640, check_every=9,
               n_sink=0, window_blocks=1)


def test_decode_full_sequence_outputs_zero_and_keeps_length():
    modes = np.array([[0, 1]], np.int8)
    cache = run_decode([126], 4, 2, 64, modes, 2, max_len=128, n_sink=1, window_blocks=1)
    q = torch.zeros((1, 4, 64), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 2, 64), dtype=torch.bfloat16, device="cuda")
    O, lse = cache.decode(q + 1, kv, kv)
    torch.cuda.synchronize()
    assert cache.lengths.cpu().tolist() == [128]
    assert torch.equal(O, torch.zeros_like(O)) and bool(torch.isinf(lse).all())


def test_decode_full_size_128k():
    # the headline layer's K/V as the prompt, then 3 decode steps; max_len
    # L + 64 makes 129 chunks of 16 blocks and the new tokens land in the last
    # one, past the 128 chunks the merge kernel holds in registers
    wl = WORKLOADS["qwen4b_s128k_sa6"]
    note("decode 128K: generating")
    c = gen.build_case(wl)
    L = int(c.lengths[0])
    cache = ea.KVCache(torch.from_numpy(c.target_modes), L + 64, c.d, n_sink=c.n_sink,
                       keep_fraction=c.keep_fraction)
    fa_bytes = ea.ea_kvcache_bytes(cache.desc, torch.zeros_like(torch.from_numpy(c.target_modes)))
    assert cache.nbytes < 0.45 * fa_bytes       # 6 of 8 KV heads keep ~0.2 of their blocks
    note("decode 128K: prefill into the cache")
    cache.prefill(dev_tensor(c.k, "bf16"), dev_tensor(c.v, "bf16"),
                  torch.from_numpy(c.cu_seqlens.astype(np.int32)).cuda())
    kf, vf = c.k_f32(), c.v_f32()
    Kh, Vh = [kf], [vf]
    for step in range(3):
        qb_, qf = _bf16(7 + step, 201, (1, c.Hq, c.d))
        knb, knf = _bf16(7 + step, 202, (1, c.Hkv, c.d))
        vnb, vnf = _bf16(7 + step, 203, (1, c.Hkv, c.d))
        note(f"decode 128K: step {step}")
        O, lse = cache.decode(dev_tensor(qb_, "bf16"), dev_tensor(knb, "bf16"),
                              dev_tensor(vnb, "bf16"))
        torch.cuda.synchronize()
        Kh = [np.concatenate([Kh[0], knf])]
        Vh = [np.concatenate([Vh[0], vnf])]
        ref, ref_lse = orc.decode_attention(qf, Kh, Vh, c.target_modes, n_sink=c.n_sink,
                                            keep_fraction=c.keep_fraction)
        compare_o(O.float().cpu().numpy(), ref, "bf16", f"O step {step}")
        assert np.abs(lse.cpu().numpy() - ref_lse).max() <= LSE_TOL
