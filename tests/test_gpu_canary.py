"""Guard-band canaries around every output and workspace buffer.

Each buffer the library writes (O, LSE, the workspace, the dual-mode outputs,
the backward gradients, the KV cache and decode outputs, the XA masses and
keep flags) is carved out of a larger allocation whose 4 KiB before and after
are filled with a byte pattern; after the call the pattern must be intact, so
no kernel writes past the ends of what it was given (the fused pass writes
every head in place in the caller's layout, "Technical Summary: Elastic
Attention", Sec. 2.3).  Outputs are also compared with the oracle, so the
guarded layout changes nothing."""
import numpy as np
import pytest
import torch

import full_attention_long_amd as ea
from gpu_helpers import LSE_TOL, compare_o, note, o_to_numpy, to_device
from oracle import ea_oracle as orc
from workloads import gen

pytestmark = pytest.mark.gpu

GUARD = 4096
PATTERN = 0xA5


class Guarded:
    """Tensors carved out of pattern-filled allocations with guard bands."""

    def __init__(self):
        self.bufs = []

    def new(self, shape, dtype):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        buf = torch.full((n + 2 * GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
        self.bufs.append((buf, n))
        return buf[GUARD:GUARD + n].view(dtype).view(*shape) if n else buf[GUARD:GUARD].view(dtype)

    def bytes(self, n):
        return self.new((max(int(n), 1),), torch.uint8)

    def check(self):
        torch.cuda.synchronize()
        for i, (buf, n) in enumerate(self.bufs):
            front = buf[:GUARD].cpu().numpy()
            back = buf[GUARD + n:].cpu().numpy()
            assert (front == PATTERN).all(), f"buffer {i}: write before its start"
            assert (back == PATTERN).all(), f"buffer {i}: write past its end"


PREFILL = [
    # lengths, Hq, Hkv, d, dtype
    ([300, 0, 1, 777, 64, 129], 8, 2, 128, "bf16"),
    ([700], 6, 2, 64, "bf16"),
    ([1500], 16, 2, 128, "bf16"),
    ([513, 64, 65], 4, 2, 64, "f32"),
]


@pytest.mark.parametrize("case", PREFILL, ids=[f"p{i}" for i in range(len(PREFILL))])
def test_prefill_guards(case):
    lengths, Hq, Hkv, d, dtype = case
    c = gen.custom_case(71 + Hq + d, lengths, Hq, Hkv, d, dtype)
    modes_np = np.random.default_rng(2).integers(0, 2, size=(len(lengths), Hkv)).astype(np.int8)
    dv = to_device(c)
    T = int(c.cu_seqlens[-1])
    ms = max(1, int(max(lengths)))
    g = Guarded()
    O = g.new(tuple(dv["q"].shape), dv["q"].dtype)
    lse = g.new((Hq, T), torch.float32)
    code = 1 if dtype == "bf16" else 0
    ws = g.bytes(ea.ea_hybrid_prefill_workspace_size(len(lengths), T, ms, Hq, Hkv, d, code))
    modes = torch.from_numpy(modes_np).cuda()
    note(f"canary prefill {case}")
    ea.ea_hybrid_prefill(dv["q"], dv["k"], dv["v"], modes, dv["cu"], ms, out=O, lse=lse, workspace=ws)
    g.check()
    ref_o, ref_lse = orc.hybrid_attention(c.q_f32(), c.k_f32(), c.v_f32(), modes_np, c.cu_seqlens,
                                          n_sink=1, keep_fraction=0.2)
    compare_o(o_to_numpy(O), ref_o, dtype)
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= LSE_TOL


def test_dual_and_backward_guards():
    lengths, Hq, Hkv, d = [900, 130, 64], 8, 2, 128
    c = gen.custom_case(73, lengths, Hq, Hkv, d, "bf16")
    dv = to_device(c)
    T = int(c.cu_seqlens[-1])
    modes = torch.tensor([[0, 1], [1, 0], [1, 1]], dtype=torch.int8, device="cuda")
    g = Guarded()
    outs = [g.new((T, Hq, d), torch.bfloat16) for _ in range(3)]
    lses = [g.new((Hq, T), torch.float32) for _ in range(2)]
    ws = g.bytes(ea.ea_dual_prefill_workspace_size(3, T, 900, Hq, Hkv, d, 1))
    note("canary dual")
    ea.ea_dual_prefill(dv["q"], dv["k"], dv["v"], dv["cu"], 900, modes=modes, out=outs[0],
                       out_fa=outs[1], out_sa=outs[2], lse_fa=lses[0], lse_sa=lses[1], workspace=ws)
    g.check()
    note("canary backward")
    O, lse = ea.ea_hybrid_prefill(dv["q"], dv["k"], dv["v"], modes, dv["cu"], 900)
    dO = torch.randn_like(O)
    g2 = Guarded()
    dQ = g2.new((T, Hq, d), torch.bfloat16)
    dK = g2.new((T, Hkv, d), torch.bfloat16)
    dV = g2.new((T, Hkv, d), torch.bfloat16)
    wsb = g2.bytes(ea.ea_hybrid_backward_workspace_size(3, T, 900, Hq, Hkv, d, 1))
    ea.ea_hybrid_backward(dv["q"], dv["k"], dv["v"], O, dO, lse, modes, dv["cu"], 900, dQ=dQ, dK=dK,
                          dV=dV, workspace=wsb)
    g2.check()
    assert bool(torch.isfinite(dQ.float()).all()) and bool(torch.isfinite(dK.float()).all())


def test_decode_guards():
    lengths, Hq, Hkv, d, max_len = [200, 70], 8, 2, 128, 1024
    B = len(lengths)
    modes_h = torch.tensor([[0, 1], [1, 0]], dtype=torch.int8)
    desc = ea.KVCacheDesc(B, Hkv, d, max_len, 1, 2, 0.2)
    g = Guarded()
    cache = g.bytes(ea.ea_kvcache_bytes(desc, modes_h))
    note("canary decode")
    ea.ea_kvcache_init(desc, modes_h.cuda(), cache)
    T = sum(lengths)
    cu = torch.tensor([0, lengths[0], T], dtype=torch.int32, device="cuda")
    K = torch.randn(T, Hkv, d, device="cuda").to(torch.bfloat16)
    V = torch.randn(T, Hkv, d, device="cuda").to(torch.bfloat16)
    ea.ea_kvcache_prefill(desc, cache, K, V, cu)
    out = g.new((B, Hq, d), torch.bfloat16)
    lse = g.new((B, Hq), torch.float32)
    ws = g.bytes(ea.ea_decode_workspace_size(desc, Hq))
    for step in range(3):
        q = torch.randn(B, Hq, d, device="cuda").to(torch.bfloat16)
        kn = torch.randn(B, Hkv, d, device="cuda").to(torch.bfloat16)
        vn = torch.randn(B, Hkv, d, device="cuda").to(torch.bfloat16)
        ea.ea_decode_step(desc, cache, q, kn, vn, out=out, lse=lse, workspace=ws)
    g.check()
    assert bool(torch.isfinite(out.float()).all())


def test_xa_guards():
    lengths, Hq, Hkv, d = [1000, 300], 8, 2, 128
    c = gen.custom_case(75, lengths, Hq, Hkv, d, "bf16")
    dv = to_device(c)
    T = int(c.cu_seqlens[-1])
    nqb = -(-1000 // 128)
    modes = torch.tensor([[0, 1], [1, 0]], dtype=torch.int8, device="cuda")
    g = Guarded()
    O = g.new((T, Hq, d), torch.bfloat16)
    lse = g.new((Hq, T), torch.float32)
    mass = g.new((2, Hq, nqb, nqb), torch.float32)
    keep = g.new((2, Hq, nqb, nqb), torch.uint8)
    ws = g.bytes(ea.ea_xa_prefill_workspace_size(2, T, 1000, Hq, Hkv, d, 1))
    for cfg in ["XA-SSA", "FA-XA"]:
        note(f"canary XA {cfg}")
        ea.ea_xa_prefill(dv["q"], dv["k"], dv["v"], modes, dv["cu"], 1000, head_config=cfg, out=O,
                         lse=lse, mass=mass, keep=keep, workspace=ws)
        g.check()
    assert bool(torch.isfinite(O.float()).all())
