"""ctypes binding of libea (argument marshalling only).

Every step of the routed hybrid prefill runs in the library's HIP kernels;
this module only converts torch device tensors to pointers and sizes, provides
outputs and workspace as torch allocations, and turns error codes into
exceptions.  It has no CPU fallback: without the built library it raises.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libea.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "ea.h")

EA_OK, EA_ERR_INVALID_ARG, EA_ERR_UNSUPPORTED, EA_ERR_WORKSPACE, EA_ERR_HIP = 0, -1, -2, -3, -4
EA_F32, EA_BF16 = 0, 1


class EAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libea status {status}: {message}")
        self.status = status


class RouterDesc(ctypes.Structure):
    _fields_ = [
        ("head_dim", ctypes.c_int32), ("task_hidden", ctypes.c_int32),
        ("router_hidden", ctypes.c_int32), ("pool_len", ctypes.c_int32),
        ("w1", ctypes.c_void_p), ("b1", ctypes.c_void_p), ("w2", ctypes.c_void_p),
        ("b2", ctypes.c_void_p), ("w3", ctypes.c_void_p), ("b3", ctypes.c_void_p),
        ("w4", ctypes.c_void_p), ("b4", ctypes.c_void_p),
    ]


class SparsityParams(ctypes.Structure):
    _fields_ = [
        ("block", ctypes.c_int32), ("n_sink_blocks", ctypes.c_int32),
        ("window_blocks", ctypes.c_int32), ("keep_fraction", ctypes.c_float),
        ("softmax_scale", ctypes.c_float),
    ]


class XAParams(ctypes.Structure):
    _fields_ = [
        ("block", ctypes.c_int32), ("stride", ctypes.c_int32),
        ("threshold", ctypes.c_float), ("head_config", ctypes.c_int32),
    ]


EA_HEADS_FA_SSA, EA_HEADS_FA_XA, EA_HEADS_XA_SSA = 0, 1, 2
HEAD_CONFIGS = {"FA-SSA": EA_HEADS_FA_SSA, "FA-XA": EA_HEADS_FA_XA, "XA-SSA": EA_HEADS_XA_SSA}


class KVCacheDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("max_len", ctypes.c_int32), ("n_sink_blocks", ctypes.c_int32),
        ("window_blocks", ctypes.c_int32), ("keep_fraction", ctypes.c_float),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libea.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m full_attention_long_amd.build` "
            "(there is no fallback implementation)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.ea_abi_version.restype = i32
    L.ea_abi_version.argtypes = []
    L.ea_last_error.restype = ctypes.c_char_p
    L.ea_last_error.argtypes = []
    L.ea_workspace_status.restype = i32
    L.ea_workspace_status.argtypes = [vp, sz, vp]
    L.ea_route.restype = i32
    L.ea_route.argtypes = [vp, i32, vp, i32, i32, ctypes.POINTER(RouterDesc), vp, vp, vp]
    L.ea_hybrid_prefill_workspace_size.restype = sz
    L.ea_hybrid_prefill_workspace_size.argtypes = [i32, i64, i32, i32, i32, i32, i32]
    L.ea_hybrid_prefill.restype = i32
    L.ea_hybrid_prefill.argtypes = [vp, vp, vp, i32, vp, vp, i32, i64, i32, i32, i32, i32,
                                    ctypes.POINTER(SparsityParams), vp, vp, vp, sz, vp]
    L.ea_hybrid_prefill_noalloc_max_workspace.restype = sz
    L.ea_hybrid_prefill_noalloc_max_workspace.argtypes = []
    L.ea_hybrid_prefill_noalloc.restype = i32
    L.ea_hybrid_prefill_noalloc.argtypes = [vp, vp, vp, i32, vp, vp, i32, i64, i32, i32, i32, i32,
                                            ctypes.POINTER(SparsityParams), vp, vp, vp]
    L.ea_hybrid_prefill_plan_layout.restype = i32
    L.ea_hybrid_prefill_plan_layout.argtypes = [i32, i64, i32, i32, i32, i32, i32,
                                                ctypes.POINTER(i64), ctypes.POINTER(i64),
                                                ctypes.POINTER(i64), ctypes.POINTER(i64)]
    L.ea_hybrid_prefill_plan.restype = i32
    L.ea_hybrid_prefill_plan.argtypes = [vp, vp, i32, i64, i32, i32, i32, i32, i32,
                                         ctypes.POINTER(SparsityParams), vp, sz, vp]
    L.ea_hybrid_prefill_run.restype = i32
    L.ea_hybrid_prefill_run.argtypes = [vp, vp, vp, i32, vp, vp, i32, i64, i32, i32, i32, i32,
                                        ctypes.POINTER(SparsityParams), vp, vp, vp, sz, vp]
    L.ea_gumbel_route.restype = i32
    L.ea_gumbel_route.argtypes = [vp, vp, ctypes.c_float, i32, vp, vp, vp]
    L.ea_dual_prefill_workspace_size.restype = sz
    L.ea_dual_prefill_workspace_size.argtypes = [i32, i64, i32, i32, i32, i32, i32]
    L.ea_dual_prefill.restype = i32
    L.ea_dual_prefill.argtypes = [vp, vp, vp, i32, vp, vp, i32, i64, i32, i32, i32, i32,
                                  ctypes.POINTER(SparsityParams), vp, vp, vp, vp, vp, vp, sz, vp]
    cd = ctypes.POINTER(KVCacheDesc)
    L.ea_kvcache_bytes.restype = sz
    L.ea_kvcache_bytes.argtypes = [cd, vp]
    L.ea_kvcache_init.restype = i32
    L.ea_kvcache_init.argtypes = [cd, vp, vp, sz, vp]
    L.ea_kvcache_prefill.restype = i32
    L.ea_kvcache_prefill.argtypes = [cd, vp, sz, vp, vp, vp, i64, vp]
    L.ea_decode_workspace_size.restype = sz
    L.ea_decode_workspace_size.argtypes = [cd, i32]
    L.ea_decode_step.restype = i32
    L.ea_decode_step.argtypes = [cd, vp, sz, vp, vp, vp, i32, ctypes.c_float, vp, vp, vp, sz, vp]
    L.ea_hybrid_backward_workspace_size.restype = sz
    L.ea_hybrid_backward_workspace_size.argtypes = [i32, i64, i32, i32, i32, i32, i32]
    L.ea_hybrid_backward.restype = i32
    L.ea_hybrid_backward.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, vp, i32, i64, i32, i32, i32,
                                     i32, ctypes.POINTER(SparsityParams), vp, vp, vp, vp, sz, vp]
    L.ea_router_logit_grad_workspace_size.restype = sz
    L.ea_router_logit_grad_workspace_size.argtypes = [i32, i32, i32]
    L.ea_router_logit_grad.restype = i32
    L.ea_router_logit_grad.argtypes = [vp, vp, vp, i32, vp, i32, i64, i32, i32, i32, i32, vp,
                                       ctypes.c_float, vp, vp, vp, sz, vp]
    L.ea_xa_prefill_workspace_size.restype = sz
    L.ea_xa_prefill_workspace_size.argtypes = [i32, i64, i32, i32, i32, i32, i32]
    L.ea_xa_prefill.restype = i32
    L.ea_xa_prefill.argtypes = [vp, vp, vp, i32, vp, vp, i32, i64, i32, i32, i32, i32,
                                ctypes.POINTER(SparsityParams), ctypes.POINTER(XAParams), vp, vp,
                                vp, vp, vp, sz, vp]
    L.ea_xa_prefill_plan.restype = i32
    L.ea_xa_prefill_plan.argtypes = [vp, vp, i32, vp, vp, i32, i64, i32, i32, i32, i32,
                                     ctypes.POINTER(SparsityParams), ctypes.POINTER(XAParams), vp,
                                     vp, vp, sz, vp]
    L.ea_xa_prefill_run.restype = i32
    L.ea_xa_prefill_run.argtypes = [vp, vp, vp, i32, vp, vp, i32, i64, i32, i32, i32, i32,
                                    ctypes.POINTER(SparsityParams), ctypes.POINTER(XAParams), vp,
                                    vp, vp, sz, vp]
    L.ea_mfma_probe.restype = i32
    L.ea_mfma_probe.argtypes = [vp, i32, i32, ctypes.c_uint32, ctypes.POINTER(i64), vp]
    _lib = L
    return L


def header_functions() -> list[str]:
    """Names of the functions include/ea.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:ea_status|size_t|int32_t|const char\*)\s+(ea_\w+)\s*\(",
                                 text, re.M)))


def _check(status: int):
    if status != EA_OK:
        raise EAError(status, lib().ea_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return EA_BF16
    if t.dtype == torch.float32:
        return EA_F32
    raise EAError(EA_ERR_UNSUPPORTED, f"unsupported dtype {t.dtype}")


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, name):
    if t is None or not t.is_cuda or not t.is_contiguous():
        raise EAError(EA_ERR_INVALID_ARG, f"{name} must be a contiguous device tensor")
    return t


def _meta(t, name, dtypes=None, shape=None, ndim=None):
    """Checks a tensor argument's dtype and shape.  The C ABI receives bare
    pointers, so this is the last place a buffer of the wrong size or element
    type can be refused before a kernel reads or writes past its end."""
    if t is None:
        raise EAError(EA_ERR_INVALID_ARG, f"{name} is required")
    if ndim is not None and t.dim() != ndim:
        raise EAError(EA_ERR_INVALID_ARG, f"{name} must have {ndim} dimensions (got {t.dim()})")
    if dtypes is not None and t.dtype not in dtypes:
        raise EAError(EA_ERR_INVALID_ARG, f"{name} must be of dtype {' or '.join(map(str, dtypes))} "
                                          f"(got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise EAError(EA_ERR_INVALID_ARG, f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return t


def _float_types():
    import torch
    return (torch.bfloat16, torch.float32)


def _check_cu(cu_seqlens):
    """cu_seqlens: int32 [B + 1], B >= 1; returns B."""
    import torch
    _meta(cu_seqlens, "cu_seqlens", (torch.int32,), ndim=1)
    if cu_seqlens.numel() < 2:
        raise EAError(EA_ERR_INVALID_ARG, "cu_seqlens must hold B + 1 >= 2 offsets")
    return cu_seqlens.numel() - 1


def _check_qkv(Q, K, V):
    """Q [T, Hq, d] and K, V [T, Hkv, d] of one floating dtype; returns T, Hq, Hkv, d."""
    _meta(Q, "Q", _float_types(), ndim=3)
    T, Hq, d = Q.shape
    _meta(K, "K", (Q.dtype,), ndim=3)
    Hkv = K.shape[1]
    _meta(K, "K", shape=(T, Hkv, d))
    if V is not None:
        _meta(V, "V", (Q.dtype,), shape=(T, Hkv, d))
    return T, Hq, Hkv, d


def ea_abi_version() -> int:
    return int(lib().ea_abi_version())


def ea_last_error() -> str:
    return lib().ea_last_error().decode()


def ea_workspace_status(workspace, stream=None):
    """Raise EAError if the plan in ``workspace`` (uint8 device tensor) failed
    the planner's device-content checks; waits for ``stream``."""
    import torch
    _meta(workspace, "workspace", (torch.uint8,), ndim=1)
    _dev(workspace, "workspace")
    _check(lib().ea_workspace_status(_ptr(workspace), workspace.numel(), _stream(stream)))


def ea_route(K, cu_seqlens, weights: dict, *, pool_len: int = 100, modes=None, logits=None,
             with_logits: bool = True, stream=None):
    """Hard FA/SA modes (int8 [B, Hkv]) and logits (float32 [B, Hkv, 2]) from K [T, Hkv, d]."""
    import torch
    _meta(K, "K", _float_types(), ndim=3)
    B = _check_cu(cu_seqlens)
    Hkv, d = K.shape[1], K.shape[2]
    f32 = (torch.float32,)
    w1 = _meta(weights.get("w1"), "w1", f32, ndim=2)
    w3 = _meta(weights.get("w3"), "w3", f32, ndim=2)
    H1, H3 = w1.shape[0], w3.shape[0]
    for k, shape in [("w1", (H1, d)), ("b1", (H1,)), ("w2", (d, H1)), ("b2", (d,)),
                     ("w3", (H3, d)), ("b3", (H3,)), ("w4", (2, H3)), ("b4", (2,))]:
        _meta(weights.get(k), k, f32, shape=shape)
    if modes is not None:
        _meta(modes, "modes", (torch.int8,), shape=(B, Hkv))
    if logits is not None:
        _meta(logits, "logits", f32, shape=(B, Hkv, 2))
    _dev(K, "K")
    _dev(cu_seqlens, "cu_seqlens")
    w = {k: _dev(weights[k], k) for k in ["w1", "b1", "w2", "b2", "w3", "b3", "w4", "b4"]}
    desc = RouterDesc(d, w["w1"].shape[0], w["w3"].shape[0], pool_len,
                      *[w[k].data_ptr() for k in ["w1", "b1", "w2", "b2", "w3", "b3", "w4", "b4"]])
    if modes is None:
        modes = torch.empty((B, Hkv), dtype=torch.int8, device=K.device)
    if logits is None and with_logits:
        logits = torch.empty((B, Hkv, 2), dtype=torch.float32, device=K.device)
    _check(lib().ea_route(_ptr(K), _dtype_code(K), _ptr(cu_seqlens), B, Hkv, ctypes.byref(desc),
                          _ptr(modes), _ptr(logits), _stream(stream)))
    return modes, logits


def ea_hybrid_prefill_workspace_size(B, total_tokens, max_seqlen, Hq, Hkv, head_dim, dtype_code):
    return int(lib().ea_hybrid_prefill_workspace_size(B, total_tokens, max_seqlen, Hq, Hkv,
                                                      head_dim, dtype_code))


def _prefill_args(Q, K, V, modes, cu_seqlens, out, lse, with_lse, workspace, max_seqlen):
    import torch
    T, Hq, Hkv, d = _check_qkv(Q, K, V)
    B = _check_cu(cu_seqlens)
    _meta(modes, "modes", (torch.int8,), shape=(B, Hkv))
    if out is not None:
        _meta(out, "out", (Q.dtype,), shape=Q.shape)
    if lse is not None:
        _meta(lse, "lse", (torch.float32,), shape=(Hq, T))
    if workspace is not None:
        _meta(workspace, "workspace", (torch.uint8,), ndim=1)
    for t, n in [(Q, "Q"), (K, "K"), (V, "V"), (modes, "modes"), (cu_seqlens, "cu_seqlens")]:
        _dev(t, n)
    if workspace is not None:
        _dev(workspace, "workspace")
    code = _dtype_code(Q)
    if out is None:
        out = torch.empty_like(Q)
    if lse is None and with_lse:
        lse = torch.empty((Hq, T), dtype=torch.float32, device=Q.device)
    if workspace is None:
        need = ea_hybrid_prefill_workspace_size(B, T, max_seqlen, Hq, Hkv, d, code)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=Q.device)
    return T, Hq, Hkv, d, B, code, out, lse, workspace


def ea_hybrid_prefill(Q, K, V, modes, cu_seqlens, max_seqlen: int, *, n_sink: int = 1,
                      window_blocks: int = 0, keep_fraction: float = 0.2,
                      softmax_scale: float = 0.0, block: int = 64, out=None, lse=None,
                      with_lse: bool = True, workspace=None, stream=None):
    """O [T, Hq, d] (and LSE float32 [Hq, T]) of the fused hybrid attention forward."""
    T, Hq, Hkv, d, B, code, out, lse, workspace = _prefill_args(
        Q, K, V, modes, cu_seqlens, out, lse, with_lse, workspace, max_seqlen)
    sp = SparsityParams(block, n_sink, window_blocks, keep_fraction, softmax_scale)
    _check(lib().ea_hybrid_prefill(_ptr(Q), _ptr(K), _ptr(V), code, _ptr(modes), _ptr(cu_seqlens),
                                   B, T, max_seqlen, Hq, Hkv, d, ctypes.byref(sp), _ptr(out),
                                   _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out, lse


def ea_hybrid_prefill_noalloc(Q, K, V, modes, cu_seqlens, max_seqlen: int, *, n_sink: int = 1,
                              window_blocks: int = 0, keep_fraction: float = 0.2,
                              softmax_scale: float = 0.0, block: int = 64, out, lse=None,
                              stream=None):
    """ea_hybrid_prefill into caller-provided ``out`` (and ``lse``) with the
    library's static workspace: the call allocates nothing (not even here)."""
    import torch
    T, Hq, Hkv, d = _check_qkv(Q, K, V)
    B = _check_cu(cu_seqlens)
    _meta(modes, "modes", (torch.int8,), shape=(B, Hkv))
    _meta(out, "out", (Q.dtype,), shape=Q.shape)
    if lse is not None:
        _meta(lse, "lse", (torch.float32,), shape=(Hq, T))
    for t, n in [(Q, "Q"), (K, "K"), (V, "V"), (modes, "modes"), (cu_seqlens, "cu_seqlens"),
                 (out, "out")]:
        _dev(t, n)
    sp = SparsityParams(block, n_sink, window_blocks, keep_fraction, softmax_scale)
    _check(lib().ea_hybrid_prefill_noalloc(_ptr(Q), _ptr(K), _ptr(V), _dtype_code(Q), _ptr(modes),
                                           _ptr(cu_seqlens), B, T, max_seqlen, Hq, Hkv, d,
                                           ctypes.byref(sp), _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


def ea_hybrid_prefill_noalloc_max_workspace() -> int:
    return int(lib().ea_hybrid_prefill_noalloc_max_workspace())


def ea_hybrid_prefill_plan_layout(B, total_tokens, max_seqlen, Hq, Hkv, head_dim, dtype_code):
    """Byte offsets of the item records, sort keys and list order inside a
    planned workspace, and the number of list slots (a dict)."""
    out = [ctypes.c_int64(0) for _ in range(4)]
    _check(lib().ea_hybrid_prefill_plan_layout(B, total_tokens, max_seqlen, Hq, Hkv, head_dim,
                                               dtype_code, *[ctypes.byref(o) for o in out]))
    return {"items": out[0].value, "keys": out[1].value, "order": out[2].value,
            "n_slots": out[3].value}


def ea_hybrid_prefill_plan(modes, cu_seqlens, total_tokens: int, max_seqlen: int, Hq: int, Hkv: int,
                           head_dim: int, dtype_code: int, workspace, *, n_sink: int = 1,
                           window_blocks: int = 0, keep_fraction: float = 0.2,
                           softmax_scale: float = 0.0, block: int = 64, stream=None):
    """Build the cost-ordered work list into ``workspace`` (a uint8 device tensor)."""
    import torch
    B = _check_cu(cu_seqlens)
    _meta(modes, "modes", (torch.int8,), shape=(B, Hkv))
    _meta(workspace, "workspace", (torch.uint8,), ndim=1)
    _dev(modes, "modes")
    _dev(cu_seqlens, "cu_seqlens")
    _dev(workspace, "workspace")
    sp = SparsityParams(block, n_sink, window_blocks, keep_fraction, softmax_scale)
    _check(lib().ea_hybrid_prefill_plan(_ptr(modes), _ptr(cu_seqlens), B, total_tokens, max_seqlen,
                                        Hq, Hkv, head_dim, dtype_code, ctypes.byref(sp),
                                        _ptr(workspace), workspace.numel(), _stream(stream)))
    return workspace


def ea_hybrid_prefill_run(Q, K, V, modes, cu_seqlens, max_seqlen: int, workspace, *,
                          n_sink: int = 1, window_blocks: int = 0, keep_fraction: float = 0.2,
                          softmax_scale: float = 0.0, block: int = 64, out=None, lse=None,
                          with_lse: bool = True, stream=None):
    """The attention launch alone, over a workspace ``ea_hybrid_prefill_plan`` filled."""
    T, Hq, Hkv, d, B, code, out, lse, workspace = _prefill_args(
        Q, K, V, modes, cu_seqlens, out, lse, with_lse, workspace, max_seqlen)
    sp = SparsityParams(block, n_sink, window_blocks, keep_fraction, softmax_scale)
    _check(lib().ea_hybrid_prefill_run(_ptr(Q), _ptr(K), _ptr(V), code, _ptr(modes),
                                       _ptr(cu_seqlens), B, T, max_seqlen, Hq, Hkv, d,
                                       ctypes.byref(sp), _ptr(out), _ptr(lse), _ptr(workspace),
                                       workspace.numel(), _stream(stream)))
    return out, lse


def ea_xa_prefill_workspace_size(B, total_tokens, max_seqlen, Hq, Hkv, head_dim, dtype_code):
    return int(lib().ea_xa_prefill_workspace_size(B, total_tokens, max_seqlen, Hq, Hkv, head_dim,
                                                  dtype_code))


def ea_xa_prefill(Q, K, V, modes, cu_seqlens, max_seqlen: int, *, head_config="XA-SSA",
                  threshold: float = 0.9, xa_block: int = 128, stride: int = 8, n_sink: int = 1,
                  window_blocks: int = 0, keep_fraction: float = 0.2, softmax_scale: float = 0.0,
                  block: int = 64, out=None, lse=None, with_lse: bool = True, mass=None,
                  keep=None, workspace=None, stream=None):
    """O [T, Hq, d] (and LSE float32 [Hq, T]) of the hybrid prefill with XA heads.

    ``head_config`` is "FA-SSA", "FA-XA" or "XA-SSA" (or its ea_head_config
    code).  ``mass`` / ``keep`` (float32 / uint8 [B, Hq, nqb, nqb] device
    tensors, nqb = ceil(max_seqlen / xa_block)) receive the XA heads' block
    masses and keep flags when given."""
    import torch
    T, Hq, Hkv, d = _check_qkv(Q, K, V)
    B = _check_cu(cu_seqlens)
    _check_xa_outputs(mass, keep, B, Hq, max_seqlen, xa_block)
    code = _dtype_code(Q)
    if workspace is None:
        need = ea_xa_prefill_workspace_size(B, T, max_seqlen, Hq, Hkv, d, code)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=Q.device)
    T, Hq, Hkv, d, B, code, out, lse, workspace = _prefill_args(
        Q, K, V, modes, cu_seqlens, out, lse, with_lse, workspace, max_seqlen)
    for t, n in [(mass, "mass"), (keep, "keep")]:
        if t is not None:
            _dev(t, n)
    sp = SparsityParams(block, n_sink, window_blocks, keep_fraction, softmax_scale)
    xp = _xa_params(head_config, threshold, xa_block, stride)
    _check(lib().ea_xa_prefill(_ptr(Q), _ptr(K), _ptr(V), code, _ptr(modes), _ptr(cu_seqlens), B, T,
                               max_seqlen, Hq, Hkv, d, ctypes.byref(sp), ctypes.byref(xp), _ptr(out),
                               _ptr(lse), _ptr(mass), _ptr(keep), _ptr(workspace),
                               workspace.numel(), _stream(stream)))
    return out, lse


def _check_xa_outputs(mass, keep, B, Hq, max_seqlen, xa_block):
    """mass float32 / keep uint8 [B, Hq, nqb, nqb], nqb = ceil(max_seqlen / xa_block)."""
    import torch
    nqb = (max_seqlen + xa_block - 1) // xa_block if xa_block > 0 else 0
    for t, n, dt in [(mass, "mass", torch.float32), (keep, "keep", torch.uint8)]:
        if t is not None:
            _meta(t, n, (dt,), shape=(B, Hq, nqb, nqb))


def _xa_params(head_config, threshold, xa_block, stride):
    cfg = HEAD_CONFIGS[head_config] if isinstance(head_config, str) else int(head_config)
    return XAParams(xa_block, stride, threshold, cfg)


def ea_xa_prefill_plan(Q, K, modes, cu_seqlens, max_seqlen: int, workspace, *,
                       head_config="XA-SSA", threshold: float = 0.9, xa_block: int = 128,
                       stride: int = 8, n_sink: int = 1, window_blocks: int = 0,
                       keep_fraction: float = 0.2, softmax_scale: float = 0.0, block: int = 64,
                       mass=None, keep=None, stream=None):
    """XA selection and work list into ``workspace`` (uint8 device tensor of
    ``ea_xa_prefill_workspace_size`` bytes)."""
    import torch
    T, Hq, Hkv, d = _check_qkv(Q, K, None)
    B = _check_cu(cu_seqlens)
    _meta(modes, "modes", (torch.int8,), shape=(B, Hkv))
    _meta(workspace, "workspace", (torch.uint8,), ndim=1)
    _check_xa_outputs(mass, keep, B, Hq, max_seqlen, xa_block)
    for t, n in [(Q, "Q"), (K, "K"), (modes, "modes"), (cu_seqlens, "cu_seqlens"),
                 (workspace, "workspace"), (mass, "mass"), (keep, "keep")]:
        if t is not None or n not in ("mass", "keep"):
            _dev(t, n)
    sp = SparsityParams(block, n_sink, window_blocks, keep_fraction, softmax_scale)
    xp = _xa_params(head_config, threshold, xa_block, stride)
    _check(lib().ea_xa_prefill_plan(_ptr(Q), _ptr(K), _dtype_code(Q), _ptr(modes), _ptr(cu_seqlens),
                                    cu_seqlens.numel() - 1, T, max_seqlen, Hq, K.shape[1], d,
                                    ctypes.byref(sp), ctypes.byref(xp), _ptr(mass), _ptr(keep),
                                    _ptr(workspace), workspace.numel(), _stream(stream)))
    return workspace


def ea_xa_prefill_run(Q, K, V, modes, cu_seqlens, max_seqlen: int, workspace, *,
                      head_config="XA-SSA", threshold: float = 0.9, xa_block: int = 128,
                      stride: int = 8, n_sink: int = 1, window_blocks: int = 0,
                      keep_fraction: float = 0.2, softmax_scale: float = 0.0, block: int = 64,
                      out=None, lse=None, with_lse: bool = True, stream=None):
    """The attention launch over a workspace ``ea_xa_prefill_plan`` filled."""
    T, Hq, Hkv, d, B, code, out, lse, workspace = _prefill_args(
        Q, K, V, modes, cu_seqlens, out, lse, with_lse, workspace, max_seqlen)
    sp = SparsityParams(block, n_sink, window_blocks, keep_fraction, softmax_scale)
    xp = _xa_params(head_config, threshold, xa_block, stride)
    _check(lib().ea_xa_prefill_run(_ptr(Q), _ptr(K), _ptr(V), code, _ptr(modes), _ptr(cu_seqlens),
                                   B, T, max_seqlen, Hq, Hkv, d, ctypes.byref(sp), ctypes.byref(xp),
                                   _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                   _stream(stream)))
    return out, lse


def ea_hybrid_backward_workspace_size(B, total_tokens, max_seqlen, Hq, Hkv, head_dim, dtype_code):
    return int(lib().ea_hybrid_backward_workspace_size(B, total_tokens, max_seqlen, Hq, Hkv,
                                                       head_dim, dtype_code))


def ea_hybrid_backward(Q, K, V, O, dO, lse, modes, cu_seqlens, max_seqlen: int, *, n_sink: int = 1,
                       window_blocks: int = 0, keep_fraction: float = 0.2,
                       softmax_scale: float = 0.0, block: int = 64, dQ=None, dK=None, dV=None,
                       workspace=None, stream=None):
    """(dQ, dK, dV) of the hybrid layer for the upstream gradient dO, given the
    forward's O and LSE (bf16 tensors; LSE float32 [Hq, T])."""
    import torch
    T, Hq, Hkv, d = _check_qkv(Q, K, V)
    B = _check_cu(cu_seqlens)
    _meta(O, "O", (Q.dtype,), shape=Q.shape)
    _meta(dO, "dO", (Q.dtype,), shape=Q.shape)
    _meta(lse, "lse", (torch.float32,), shape=(Hq, T))
    _meta(modes, "modes", (torch.int8,), shape=(B, Hkv))
    for t, n, like in [(dQ, "dQ", Q), (dK, "dK", K), (dV, "dV", V)]:
        if t is not None:
            _meta(t, n, (Q.dtype,), shape=like.shape)
    for t, n in [(Q, "Q"), (K, "K"), (V, "V"), (O, "O"), (dO, "dO"), (lse, "lse"),
                 (modes, "modes"), (cu_seqlens, "cu_seqlens")]:
        _dev(t, n)
    code = _dtype_code(Q)
    dQ = torch.empty_like(Q) if dQ is None else dQ
    dK = torch.empty_like(K) if dK is None else dK
    dV = torch.empty_like(V) if dV is None else dV
    if workspace is None:
        need = ea_hybrid_backward_workspace_size(B, T, max_seqlen, Hq, Hkv, d, code)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=Q.device)
    sp = SparsityParams(block, n_sink, window_blocks, keep_fraction, softmax_scale)
    _check(lib().ea_hybrid_backward(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO), _ptr(lse), code,
                                    _ptr(modes), _ptr(cu_seqlens), B, T, max_seqlen, Hq, Hkv, d,
                                    ctypes.byref(sp), _ptr(dQ), _ptr(dK), _ptr(dV),
                                    _ptr(workspace), workspace.numel(), _stream(stream)))
    return dQ, dK, dV


def ea_router_logit_grad_workspace_size(B: int, max_seqlen: int, Hkv: int) -> int:
    return int(lib().ea_router_logit_grad_workspace_size(B, max_seqlen, Hkv))


def ea_router_logit_grad(dO, O_fa, O_sa, cu_seqlens, max_seqlen: int, r_soft, tau: float, *,
                         dz=None, dr=None, with_dr: bool = True, workspace=None, stream=None):
    """(dz, dr) float32 [B, Hkv, 2]: the routing logits' gradient through the
    straight-through estimator and the Gumbel-Softmax."""
    import torch
    _meta(dO, "dO", _float_types(), ndim=3)
    T, Hq, d = dO.shape
    _meta(O_fa, "O_fa", (dO.dtype,), shape=dO.shape)
    _meta(O_sa, "O_sa", (dO.dtype,), shape=dO.shape)
    B = _check_cu(cu_seqlens)
    _meta(r_soft, "r_soft", (torch.float32,), ndim=3)
    Hkv = r_soft.shape[1]
    _meta(r_soft, "r_soft", shape=(B, Hkv, 2))
    for t, n in [(dz, "dz"), (dr, "dr")]:
        if t is not None:
            _meta(t, n, (torch.float32,), shape=(B, Hkv, 2))
    for t, n in [(dO, "dO"), (O_fa, "O_fa"), (O_sa, "O_sa"), (cu_seqlens, "cu_seqlens"),
                 (r_soft, "r_soft")]:
        _dev(t, n)
    dz = torch.empty_like(r_soft) if dz is None else dz
    if dr is None and with_dr:
        dr = torch.empty_like(r_soft)
    if workspace is None:
        workspace = torch.empty(max(1, ea_router_logit_grad_workspace_size(B, max_seqlen, Hkv)),
                                dtype=torch.uint8, device=dO.device)
    _check(lib().ea_router_logit_grad(_ptr(dO), _ptr(O_fa), _ptr(O_sa), _dtype_code(dO),
                                      _ptr(cu_seqlens), B, T, max_seqlen, Hq, Hkv, d,
                                      _ptr(r_soft), float(tau), _ptr(dz), _ptr(dr),
                                      _ptr(workspace), workspace.numel(), _stream(stream)))
    return dz, dr


def ea_gumbel_route(logits, tau: float, *, gumbel=None, r_soft=None, modes=None,
                    with_soft: bool = True, stream=None):
    """Training-time routing of float32 logits [..., 2]: r_soft = softmax((logits +
    gumbel) / tau) and the hard modes (int8 [...], 1 = SA) of the straight-through
    estimator."""
    import torch
    _dev(logits, "logits")
    if logits.dtype != torch.float32 or logits.shape[-1] != 2:
        raise ValueError("logits must be float32 [..., 2]")
    if gumbel is not None:
        _dev(gumbel, "gumbel")
        if gumbel.shape != logits.shape or gumbel.dtype != torch.float32:
            raise ValueError("gumbel must be float32 of the logits' shape")
    if r_soft is not None:
        _meta(r_soft, "r_soft", (torch.float32,), shape=logits.shape)
    if modes is not None:
        _meta(modes, "modes", (torch.int8,), shape=logits.shape[:-1])
    n = logits.numel() // 2
    if modes is None:
        modes = torch.empty(logits.shape[:-1], dtype=torch.int8, device=logits.device)
    if r_soft is None and with_soft:
        r_soft = torch.empty_like(logits)
    _check(lib().ea_gumbel_route(_ptr(logits), _ptr(gumbel), float(tau), n, _ptr(r_soft),
                                 _ptr(modes), _stream(stream)))
    return r_soft, modes


def ea_dual_prefill_workspace_size(B, total_tokens, max_seqlen, Hq, Hkv, head_dim, dtype_code):
    return int(lib().ea_dual_prefill_workspace_size(B, total_tokens, max_seqlen, Hq, Hkv,
                                                    head_dim, dtype_code))


def ea_dual_prefill(Q, K, V, cu_seqlens, max_seqlen: int, *, modes=None, n_sink: int = 1,
                    window_blocks: int = 0, keep_fraction: float = 0.2, softmax_scale: float = 0.0,
                    block: int = 64, out=None, out_fa=None, out_sa=None, lse_fa=None, lse_sa=None,
                    workspace=None, stream=None):
    """Dual-mode (training) forward: every head in both modes.

    Returns (O, O_FA, O_SA, LSE_FA, LSE_SA); O (the straight-through mix, the
    hard decision's output per (sequence, KV head)) only when ``modes`` is
    given, else None."""
    import torch
    T, Hq, Hkv, d = _check_qkv(Q, K, V)
    B = _check_cu(cu_seqlens)
    if modes is not None:
        _meta(modes, "modes", (torch.int8,), shape=(B, Hkv))
    for t, n in [(out, "out"), (out_fa, "out_fa"), (out_sa, "out_sa")]:
        if t is not None:
            _meta(t, n, (Q.dtype,), shape=Q.shape)
    for t, n in [(lse_fa, "lse_fa"), (lse_sa, "lse_sa")]:
        if t is not None:
            _meta(t, n, (torch.float32,), shape=(Hq, T))
    for t, n in [(Q, "Q"), (K, "K"), (V, "V"), (cu_seqlens, "cu_seqlens")]:
        _dev(t, n)
    if modes is not None:
        _dev(modes, "modes")
    code = _dtype_code(Q)
    if out is None and modes is not None:
        out = torch.empty_like(Q)
    out_fa = torch.empty_like(Q) if out_fa is None else out_fa
    out_sa = torch.empty_like(Q) if out_sa is None else out_sa
    lse_fa = torch.empty((Hq, T), dtype=torch.float32, device=Q.device) if lse_fa is None else lse_fa
    lse_sa = torch.empty((Hq, T), dtype=torch.float32, device=Q.device) if lse_sa is None else lse_sa
    if workspace is None:
        need = ea_dual_prefill_workspace_size(B, T, max_seqlen, Hq, Hkv, d, code)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=Q.device)
    sp = SparsityParams(block, n_sink, window_blocks, keep_fraction, softmax_scale)
    _check(lib().ea_dual_prefill(_ptr(Q), _ptr(K), _ptr(V), code, _ptr(modes), _ptr(cu_seqlens),
                                 B, T, max_seqlen, Hq, Hkv, d, ctypes.byref(sp), _ptr(out),
                                 _ptr(out_fa), _ptr(out_sa), _ptr(lse_fa), _ptr(lse_sa),
                                 _ptr(workspace), workspace.numel(), _stream(stream)))
    return out, out_fa, out_sa, lse_fa, lse_sa


def ea_kvcache_bytes(desc: KVCacheDesc, modes_host) -> int:
    """Bytes of a cache for ``desc`` and the routing ``modes_host`` (a CPU int8
    tensor [B, Hkv])."""
    import torch
    if modes_host.is_cuda or modes_host.dtype != torch.int8 or not modes_host.is_contiguous():
        raise ValueError("modes_host must be a contiguous CPU int8 tensor")
    return int(lib().ea_kvcache_bytes(ctypes.byref(desc), ctypes.c_void_p(modes_host.data_ptr())))


def ea_kvcache_init(desc: KVCacheDesc, modes, cache, *, stream=None):
    import torch
    _meta(modes, "modes", (torch.int8,), shape=(desc.B, desc.Hkv))
    _meta(cache, "cache", (torch.uint8,), ndim=1)
    _dev(modes, "modes")
    _dev(cache, "cache")
    _check(lib().ea_kvcache_init(ctypes.byref(desc), _ptr(modes), _ptr(cache), cache.numel(),
                                 _stream(stream)))
    return cache


def ea_kvcache_prefill(desc: KVCacheDesc, cache, K, V, cu_seqlens, *, stream=None):
    import torch
    _meta(cache, "cache", (torch.uint8,), ndim=1)
    _meta(K, "K", (torch.bfloat16,), ndim=3)
    _meta(K, "K", shape=(K.shape[0], desc.Hkv, desc.head_dim))
    _meta(V, "V", (torch.bfloat16,), shape=K.shape)
    _meta(cu_seqlens, "cu_seqlens", (torch.int32,), shape=(desc.B + 1,))
    for t, n in [(cache, "cache"), (K, "K"), (V, "V"), (cu_seqlens, "cu_seqlens")]:
        _dev(t, n)
    _check(lib().ea_kvcache_prefill(ctypes.byref(desc), _ptr(cache), cache.numel(), _ptr(K),
                                    _ptr(V), _ptr(cu_seqlens), K.shape[0], _stream(stream)))
    return cache


def ea_decode_workspace_size(desc: KVCacheDesc, Hq: int) -> int:
    return int(lib().ea_decode_workspace_size(ctypes.byref(desc), Hq))


def ea_decode_step(desc: KVCacheDesc, cache, q, k_new, v_new, *, softmax_scale: float = 0.0,
                   out=None, lse=None, with_lse: bool = True, workspace=None, stream=None):
    """Append (k_new, v_new) [B, Hkv, d] at each sequence's length and attend
    with q [B, Hq, d]; returns (O [B, Hq, d] bf16, LSE float32 [B, Hq])."""
    import torch
    _meta(cache, "cache", (torch.uint8,), ndim=1)
    _meta(q, "q", (torch.bfloat16,), ndim=3)
    Hq = q.shape[1]
    _meta(q, "q", shape=(desc.B, Hq, desc.head_dim))
    _meta(k_new, "k_new", (torch.bfloat16,), shape=(desc.B, desc.Hkv, desc.head_dim))
    _meta(v_new, "v_new", (torch.bfloat16,), shape=(desc.B, desc.Hkv, desc.head_dim))
    if out is not None:
        _meta(out, "out", (torch.bfloat16,), shape=q.shape)
    if lse is not None:
        _meta(lse, "lse", (torch.float32,), shape=(desc.B, Hq))
    for t, n in [(cache, "cache"), (q, "q"), (k_new, "k_new"), (v_new, "v_new")]:
        _dev(t, n)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and with_lse:
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(1, ea_decode_workspace_size(desc, Hq)), dtype=torch.uint8,
                                device=q.device)
    _check(lib().ea_decode_step(ctypes.byref(desc), _ptr(cache), cache.numel(), _ptr(q),
                                _ptr(k_new), _ptr(v_new), Hq, float(softmax_scale), _ptr(out),
                                _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out, lse


class KVCache:
    """A mode-aware KV cache in one device buffer (bf16, blocks of 64 tokens).

    FA heads keep every block; SA heads keep their sink blocks and a ring of
    the window at ``max_len``.  ``lengths`` views the per-sequence token counts
    kept in the buffer's header."""

    def __init__(self, modes, max_len: int, head_dim: int, *, n_sink: int = 1,
                 window_blocks: int = 0, keep_fraction: float = 0.2, stream=None):
        import torch
        B, Hkv = modes.shape
        self.desc = KVCacheDesc(B, Hkv, head_dim, max_len, n_sink, window_blocks, keep_fraction)
        m_host = modes.detach().to("cpu", torch.int8).contiguous()
        m_dev = m_host.cuda()
        self.nbytes = ea_kvcache_bytes(self.desc, m_host)
        if self.nbytes == 0:
            raise EAError(EA_ERR_INVALID_ARG, ea_last_error() or "invalid cache descriptor")
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device="cuda")
        ea_kvcache_init(self.desc, m_dev, self.buf, stream=stream)
        self.workspace = None

    @property
    def lengths(self):
        return self.buf[:4 * self.desc.B].view(torch_int32())

    def prefill(self, K, V, cu_seqlens, *, stream=None):
        return ea_kvcache_prefill(self.desc, self.buf, K, V, cu_seqlens, stream=stream)

    def decode(self, q, k_new, v_new, **kw):
        import torch
        if self.workspace is None:
            self.workspace = torch.empty(max(1, ea_decode_workspace_size(self.desc, q.shape[1])),
                                         dtype=torch.uint8, device="cuda")
        kw.setdefault("workspace", self.workspace)
        return ea_decode_step(self.desc, self.buf, q, k_new, v_new, **kw)


def torch_int32():
    import torch
    return torch.int32


def ea_mfma_probe(out, n_workgroups: int, iters: int, *, seed: int = 1, stream=None) -> int:
    """Launch the matrix-core ceiling probe into ``out`` (float32 device tensor
    of n_workgroups * 512 elements); returns the FLOPs the launch performs."""
    _dev(out, "out")
    import torch
    if out.dtype != torch.float32 or out.numel() < n_workgroups * 512:
        raise ValueError("out must be float32 with at least n_workgroups * 512 elements")
    flops = ctypes.c_int64(0)
    _check(lib().ea_mfma_probe(_ptr(out), n_workgroups, iters, seed & 0xFFFFFFFF,
                               ctypes.byref(flops), _stream(stream)))
    return flops.value
