"""Device-content checks of the planner (through the C ABI).

Every invalid case below stays inside its buffers even if it were not
checked (a mode of 2 reads as SA; the bad offsets only shorten, drop or
re-slice sequences inside [0, T)), so a failing check cannot make a kernel
read or write out of bounds.  Each case must leave the outputs exactly as they
were (filled with a sentinel beforehand) and report the failed check: through
ea_workspace_status by default, from the call itself under EA_VALIDATE=1.
Paper passage of the mode check: the router paragraph on Fig. 3(b) of
"Elastic Attention: Test-time Adaptive Sparsity Ratios for Efficient
Transformers" (the hard decision per KV head is 0 or 1)."""
import re

import pytest
import torch

import full_attention_long_amd as ea
from gpu_helpers import note, to_device
from workloads import gen

pytestmark = pytest.mark.gpu

SENTINEL = 7.0
T = 1000


def _case():
    # one 1000-token sequence; the cu variants below re-slice its rows
    return gen.custom_case(41, [T], 8, 2, 128, "bf16", w_std=0.2)


def _prefill(dv, modes, cu, max_seqlen, ws):
    O = torch.full_like(dv["q"], SENTINEL)
    lse = torch.full((dv["q"].shape[1], T), SENTINEL, dtype=torch.float32, device="cuda")
    ea.ea_hybrid_prefill(dv["q"], dv["k"], dv["v"], modes, cu, max_seqlen, n_sink=1,
                         keep_fraction=0.2, out=O, lse=lse, workspace=ws)
    return O, lse


BAD = [
    # name, cu offsets (B + 1), modes per sequence, max_seqlen, message
    ("mode", [0, T], [[0, 2]], T, "mode value"),
    ("cu_order", [0, 600, 500, T], [[0, 1], [1, 0], [0, 0]], T, "decreases"),
    ("cu_end", [0, 500, 900], [[0, 1], [1, 1]], T, "cu_seqlens[B]"),
    ("cu_start", [100, 500, T], [[0, 1], [1, 0]], T, "cu_seqlens[0]"),
    ("seqlen", [0, T], [[1, 0]], T - 64, "max_seqlen"),
]


def _inputs(cu_list, modes_list):
    cu = torch.tensor(cu_list, dtype=torch.int32, device="cuda")
    modes = torch.tensor(modes_list, dtype=torch.int8, device="cuda")
    return cu, modes


@pytest.mark.parametrize("name,cu_list,modes_list,max_seqlen,msg", BAD, ids=[b[0] for b in BAD])
def test_prefill_rejects_invalid_contents(monkeypatch, name, cu_list, modes_list, max_seqlen, msg):
    c = _case()
    dv = to_device(c)
    cu, modes = _inputs(cu_list, modes_list)
    B = len(cu_list) - 1
    need = ea.ea_hybrid_prefill_workspace_size(B, T, max_seqlen, 8, 2, 128, 1)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    note(f"validate prefill {name} (status read afterwards)")
    monkeypatch.delenv("EA_VALIDATE", raising=False)
    O, lse = _prefill(dv, modes, cu, max_seqlen, ws)
    with pytest.raises(ea.EAError, match=re.escape(msg)):
        ea.ea_workspace_status(ws)
    assert bool((O.float() == SENTINEL).all()) and bool((lse == SENTINEL).all())
    note(f"validate prefill {name} (EA_VALIDATE=1)")
    monkeypatch.setenv("EA_VALIDATE", "1")
    with pytest.raises(ea.EAError, match=re.escape(msg)):
        _prefill(dv, modes, cu, max_seqlen, ws)
    torch.cuda.synchronize()


def test_valid_contents_pass_and_match(monkeypatch):
    c = _case()
    dv = to_device(c)
    cu, modes = _inputs([0, 600, T], [[0, 1], [1, 0]])
    need = ea.ea_hybrid_prefill_workspace_size(2, T, 600, 8, 2, 128, 1)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    note("validate prefill valid (both ways)")
    monkeypatch.delenv("EA_VALIDATE", raising=False)
    O0, lse0 = _prefill(dv, modes, cu, 600, ws)
    ea.ea_workspace_status(ws)
    monkeypatch.setenv("EA_VALIDATE", "1")
    O1, lse1 = _prefill(dv, modes, cu, 600, ws)
    torch.cuda.synchronize()
    assert torch.equal(O0, O1) and torch.equal(lse0, lse1)
    assert bool((O0.float() != SENTINEL).any())


def test_plan_run_dual_xa_backward_reject_bad_mode(monkeypatch):
    c = _case()
    dv = to_device(c)
    cu, modes = _inputs([0, T], [[2, 0]])
    monkeypatch.setenv("EA_VALIDATE", "1")
    q, k, v = dv["q"], dv["k"], dv["v"]
    note("validate plan")
    ws = torch.zeros(ea.ea_hybrid_prefill_workspace_size(1, T, T, 8, 2, 128, 1), dtype=torch.uint8,
                     device="cuda")
    with pytest.raises(ea.EAError, match="mode value"):
        ea.ea_hybrid_prefill_plan(modes, cu, T, T, 8, 2, 128, 1, ws)
    note("validate run on the rejected plan")
    O = torch.full_like(q, SENTINEL)
    with pytest.raises(ea.EAError, match="mode value"):
        ea.ea_hybrid_prefill_run(q, k, v, modes, cu, T, ws, out=O)
    note("validate dual")
    outs = [torch.full_like(q, SENTINEL) for _ in range(3)]
    lses = [torch.full((8, T), SENTINEL, dtype=torch.float32, device="cuda") for _ in range(2)]
    with pytest.raises(ea.EAError, match="mode value"):
        ea.ea_dual_prefill(q, k, v, cu, T, modes=modes, out=outs[0], out_fa=outs[1], out_sa=outs[2],
                           lse_fa=lses[0], lse_sa=lses[1])
    note("validate XA")
    with pytest.raises(ea.EAError, match="mode value"):
        ea.ea_xa_prefill(q, k, v, modes, cu, T, head_config="XA-SSA", out=outs[0], lse=lses[0])
    note("validate backward")
    grads = [torch.full_like(q, SENTINEL), torch.full_like(k, SENTINEL), torch.full_like(v, SENTINEL)]
    with pytest.raises(ea.EAError, match="mode value"):
        ea.ea_hybrid_backward(q, k, v, q, q, lses[0], modes, cu, T, dQ=grads[0], dK=grads[1],
                              dV=grads[2])
    torch.cuda.synchronize()
    for t in [O, *outs, *lses, *grads]:
        assert bool((t.float() == SENTINEL).all())


def test_route_and_cache_fill_check_cu_on_host(monkeypatch):
    c = _case()
    dv = to_device(c)
    monkeypatch.setenv("EA_VALIDATE", "1")
    cu_bad = torch.tensor([0, 600, 500, T], dtype=torch.int32, device="cuda")
    note("validate route")
    with pytest.raises(ea.EAError, match="decreases"):
        ea.ea_route(dv["k"], cu_bad, dv["w"], pool_len=100)
    note("validate cache fill")
    modes = torch.zeros((1, 2), dtype=torch.int8)
    cache = ea.KVCache(modes, T - 64, 128, n_sink=1, keep_fraction=0.2)
    cu_long = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    with pytest.raises(ea.EAError, match="max_seqlen"):
        cache.prefill(dv["k"], dv["v"], cu_long)
    torch.cuda.synchronize()
