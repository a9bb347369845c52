"""Host-side argument checks of the Python binding (no GPU needed).

The C ABI receives bare device pointers, so the binding is where a tensor of
the wrong shape or dtype must be refused; these tests pass CPU tensors, which
reach the shape and dtype checks first and the device check last."""
import pytest
import torch

from full_attention_long_amd import binding as ea
from full_attention_long_amd.binding import EAError

T, HQ, HKV, D, B = 200, 8, 2, 64, 2


def _qkv(dtype=torch.bfloat16):
    return (torch.zeros(T, HQ, D, dtype=dtype), torch.zeros(T, HKV, D, dtype=dtype),
            torch.zeros(T, HKV, D, dtype=dtype))


def _cu():
    return torch.tensor([0, 120, T], dtype=torch.int32)


def _modes():
    return torch.zeros(B, HKV, dtype=torch.int8)


def _weights(d=D, h1=32, h3=16):
    f = torch.float32
    return {"w1": torch.zeros(h1, d, dtype=f), "b1": torch.zeros(h1, dtype=f),
            "w2": torch.zeros(d, h1, dtype=f), "b2": torch.zeros(d, dtype=f),
            "w3": torch.zeros(h3, d, dtype=f), "b3": torch.zeros(h3, dtype=f),
            "w4": torch.zeros(2, h3, dtype=f), "b4": torch.zeros(2, dtype=f)}


def _raises(match, fn, *args, **kw):
    with pytest.raises(EAError, match=match):
        fn(*args, **kw)


def test_route_checks_weight_shapes_and_dtypes():
    K = _qkv()[1]
    w = _weights()
    w["w2"] = torch.zeros(D, 31)
    _raises("w2 must have shape", ea.ea_route, K, _cu(), w)
    w = _weights()
    w["b4"] = torch.zeros(3)
    _raises("b4 must have shape", ea.ea_route, K, _cu(), w)
    w = _weights()
    w["w3"] = w["w3"].double()
    _raises("w3 must be of dtype", ea.ea_route, K, _cu(), w)
    _raises("K must be of dtype", ea.ea_route, K.half(), _cu(), _weights())
    _raises("cu_seqlens must be of dtype", ea.ea_route, K, _cu().long(), _weights())
    _raises("modes must have shape", ea.ea_route, K, _cu(), _weights(),
            modes=torch.zeros(B, HKV + 1, dtype=torch.int8))
    _raises("logits must have shape", ea.ea_route, K, _cu(), _weights(),
            logits=torch.zeros(B, HKV, 3))
    # well-formed metadata reaches the device check
    _raises("contiguous device tensor", ea.ea_route, K, _cu(), _weights())


def test_prefill_checks_shapes_and_dtypes():
    Q, K, V = _qkv()
    _raises("K must have shape", ea.ea_hybrid_prefill, Q, K[:-1], V, _modes(), _cu(), 120)
    _raises("V must be of dtype", ea.ea_hybrid_prefill, Q, K, V.float(), _modes(), _cu(), 120)
    _raises("modes must be of dtype", ea.ea_hybrid_prefill, Q, K, V, _modes().int(), _cu(), 120)
    _raises("modes must have shape", ea.ea_hybrid_prefill, Q, K, V, _modes()[:1], _cu(), 120)
    _raises("out must be of dtype", ea.ea_hybrid_prefill, Q, K, V, _modes(), _cu(), 120,
            out=torch.zeros(T, HQ, D))
    _raises("lse must have shape", ea.ea_hybrid_prefill, Q, K, V, _modes(), _cu(), 120,
            lse=torch.zeros(T, HQ))
    _raises("cu_seqlens must hold", ea.ea_hybrid_prefill, Q, K, V, _modes(),
            torch.zeros(1, dtype=torch.int32), 120)
    _raises("workspace must be of dtype", ea.ea_hybrid_prefill_run, Q, K, V, _modes(), _cu(), 120,
            torch.zeros(16, dtype=torch.int32))
    _raises("modes must have shape", ea.ea_hybrid_prefill_plan, _modes(), _cu(), T, 120, HQ,
            HKV + 1, D, ea.EA_BF16, torch.zeros(16, dtype=torch.uint8))
    _raises("contiguous device tensor", ea.ea_hybrid_prefill, Q, K, V, _modes(), _cu(), 120,
            workspace=torch.zeros(16, dtype=torch.uint8))


def test_backward_dual_xa_and_grad_check_shapes():
    Q, K, V = _qkv()
    lse = torch.zeros(HQ, T)
    _raises("dO must have shape", ea.ea_hybrid_backward, Q, K, V, Q, Q[:-1], lse, _modes(), _cu(),
            120)
    _raises("lse must be of dtype", ea.ea_hybrid_backward, Q, K, V, Q, Q, lse.double(), _modes(),
            _cu(), 120)
    _raises("dK must have shape", ea.ea_hybrid_backward, Q, K, V, Q, Q, lse, _modes(), _cu(), 120,
            dK=torch.zeros_like(Q))
    _raises("lse_fa must have shape", ea.ea_dual_prefill, Q, K, V, _cu(), 120,
            lse_fa=torch.zeros(HQ, T + 1))
    _raises("mass must have shape", ea.ea_xa_prefill, Q, K, V, _modes(), _cu(), 120,
            mass=torch.zeros(B, HQ, 2, 2), workspace=torch.zeros(16, dtype=torch.uint8))
    r = torch.zeros(B, HKV, 2)
    _raises("O_sa must have shape", ea.ea_router_logit_grad, Q, Q, Q[:, :4], _cu(), 120, r, 1.0)
    _raises("dz must have shape", ea.ea_router_logit_grad, Q, Q, Q, _cu(), 120, r, 1.0,
            dz=torch.zeros(B, HKV))


def test_decode_checks_shapes():
    desc = ea.KVCacheDesc(B, HKV, D, 1024, 1, 0, 0.2)
    cache = torch.zeros(64, dtype=torch.uint8)
    q = torch.zeros(B, HQ, D, dtype=torch.bfloat16)
    kn = torch.zeros(B, HKV, D, dtype=torch.bfloat16)
    _raises("q must have shape", ea.ea_decode_step, desc, cache, q[:, :, :32], kn, kn)
    _raises("k_new must have shape", ea.ea_decode_step, desc, cache, q, kn[:1], kn)
    _raises("v_new must be of dtype", ea.ea_decode_step, desc, cache, q, kn, kn.float())
    _raises("cu_seqlens must have shape", ea.ea_kvcache_prefill, desc, cache,
            torch.zeros(T, HKV, D, dtype=torch.bfloat16), torch.zeros(T, HKV, D, dtype=torch.bfloat16),
            torch.tensor([0, T], dtype=torch.int32))
    _raises("contiguous device tensor", ea.ea_decode_step, desc, cache, q, kn, kn)
