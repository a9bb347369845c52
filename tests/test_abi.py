"""The C ABI without a GPU: every declared symbol is exported, the workspace
size is a pure host computation, and every host-checkable error returns its
status before anything is launched (the pointers below are never
dereferenced: validation fails first)."""
import ctypes

import pytest

import full_attention_long_amd as ea
from full_attention_long_amd import binding as bnd

FAKE = 0x100000  # 256-byte aligned, never dereferenced by a failing call


def test_every_header_function_is_exported():
    names = ea.header_functions()
    assert set(names) == {"ea_abi_version", "ea_last_error", "ea_route",
                          "ea_hybrid_prefill_workspace_size", "ea_hybrid_prefill",
                          "ea_hybrid_prefill_plan", "ea_hybrid_prefill_run", "ea_mfma_probe",
                          "ea_gumbel_route", "ea_dual_prefill_workspace_size", "ea_dual_prefill",
                          "ea_kvcache_bytes", "ea_kvcache_init", "ea_kvcache_prefill",
                          "ea_decode_workspace_size", "ea_decode_step",
                          "ea_hybrid_backward_workspace_size", "ea_hybrid_backward",
                          "ea_router_logit_grad_workspace_size", "ea_router_logit_grad",
                          "ea_xa_prefill_workspace_size", "ea_xa_prefill",
                          "ea_xa_prefill_plan", "ea_xa_prefill_run", "ea_workspace_status",
                          "ea_hybrid_prefill_plan_layout", "ea_hybrid_prefill_noalloc",
                          "ea_hybrid_prefill_noalloc_max_workspace"}
    L = ea.lib()
    for n in names:
        assert hasattr(L, n), n
    assert ea.ea_abi_version() == 2


def test_workspace_size_bounds():
    ws = ea.ea_hybrid_prefill_workspace_size(1, 131072, 131072, 32, 8, 128, bnd.EA_BF16)
    items = 8 * (131072 // 64 + 1)            # query tiles of 64 positions x 4 heads
    per_item = 20 + 4 + 4                     # item record + sort key + sorted order
    assert items * per_item <= ws <= items * per_item + 4 * 2**20
    # no copy of K, V or Q: the workspace does not grow with head_dim or dtype
    assert ea.ea_hybrid_prefill_workspace_size(1, 1000, 1000, 32, 8, 128, bnd.EA_F32) == \
        ea.ea_hybrid_prefill_workspace_size(1, 1000, 1000, 32, 8, 64, bnd.EA_BF16)
    # invalid sizes -> 0
    assert ea.ea_hybrid_prefill_workspace_size(0, 1000, 1000, 32, 8, 128, 1) == 0
    assert ea.ea_hybrid_prefill_workspace_size(1, 1000, 1000, 30, 8, 128, 1) == 0
    assert ea.ea_hybrid_prefill_workspace_size(1, 1000, 1000, 32, 8, 96, 1) == 0
    assert ea.ea_hybrid_prefill_workspace_size(1, 2**31, 1000, 32, 8, 128, 1) == 0


def _prefill(**kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, dtype=1, modes=FAKE, cu=FAKE, B=1, T=1000, max_seqlen=1000,
             Hq=8, Hkv=2, d=128, block=64, n_sink=1, window=0, keep=0.2, scale=0.0, O=FAKE,
             lse=None, ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    sp = bnd.SparsityParams(a["block"], a["n_sink"], a["window"], a["keep"], a["scale"])
    st = ea.lib().ea_hybrid_prefill(a["Q"], a["K"], a["V"], a["dtype"], a["modes"], a["cu"], a["B"],
                                    a["T"], a["max_seqlen"], a["Hq"], a["Hkv"], a["d"],
                                    ctypes.byref(sp), a["O"], a["lse"], a["ws"], a["ws_bytes"], None)
    return st, ea.ea_last_error()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(Q=None), -1, "null pointer"),
    (dict(modes=None), -1, "null pointer"),
    (dict(O=None), -1, "null pointer"),
    (dict(B=0), -1, "B must be"),
    (dict(Hq=6, Hkv=4), -1, "multiple of Hkv"),
    (dict(Hq=512, Hkv=1), -2, "Hq / Hkv"),
    (dict(d=96), -2, "head_dim"),
    (dict(dtype=7), -2, "dtype"),
    (dict(block=128), -2, "block"),
    (dict(n_sink=-1), -1, "n_sink"),
    (dict(n_sink=2**24 + 1), -1, "n_sink"),
    (dict(window=-2), -1, "window_blocks"),
    (dict(window=2**31 - 1), -1, "window_blocks"),
    (dict(keep=0.0), -1, "keep_fraction"),
    (dict(keep=1.5), -1, "keep_fraction"),
    (dict(scale=-1.0), -1, "softmax_scale"),
    (dict(scale=float("nan")), -1, "softmax_scale"),
    (dict(max_seqlen=0), -1, "max_seqlen"),
    (dict(max_seqlen=2000), -1, "max_seqlen"),
    (dict(T=2**31), -1, "total_tokens"),
    (dict(T=2**30, max_seqlen=2**20, Hq=32, Hkv=8), -2, "2^31"),
    (dict(ws=None), -3, "workspace"),
    (dict(ws_bytes=1024), -3, "workspace"),
    (dict(ws=FAKE + 16), -1, "256-byte"),
    (dict(Q=FAKE + 2), -1, "16-byte"),
])
def test_prefill_host_errors(kw, status, msg):
    st, err = _prefill(**kw)
    assert st == status and msg in err, (st, err)


def test_prefill_zero_tokens_is_a_no_op():
    st, err = _prefill(T=0, max_seqlen=0)
    assert st == 0 and err == ""


def _route(**kw):
    a = dict(K=FAKE, dtype=1, cu=FAKE, B=1, Hkv=8, modes=FAKE, d=128, th=512, rh=64, pool=100,
             w=FAKE)
    a.update(kw)
    desc = bnd.RouterDesc(a["d"], a["th"], a["rh"], a["pool"], *([a["w"]] * 8))
    st = ea.lib().ea_route(a["K"], a["dtype"], a["cu"], a["B"], a["Hkv"], ctypes.byref(desc),
                           a["modes"], None, None)
    return st, ea.ea_last_error()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(K=None), -1, "null pointer"),
    (dict(modes=None), -1, "null pointer"),
    (dict(w=None), -1, "router weight"),
    (dict(B=0), -1, "B and Hkv"),
    (dict(d=300), -2, "head_dim"),
    (dict(th=5000), -2, "task_hidden"),
    (dict(rh=2000), -2, "router_hidden"),
    (dict(pool=0), -1, "pool_len"),
    (dict(dtype=3), -2, "dtype"),
])
def test_route_host_errors(kw, status, msg):
    st, err = _route(**kw)
    assert st == status and msg in err, (st, err)


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(bnd, "_lib", None)
    monkeypatch.setattr(bnd, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        bnd.lib()


def test_plan_and_run_host_errors():
    L = ea.lib()
    sp = bnd.SparsityParams(64, 1, 0, 0.2, 0.0)
    # plan: null modes, bad block, small workspace
    assert L.ea_hybrid_prefill_plan(None, FAKE, 1, 1000, 1000, 8, 2, 128, 1, ctypes.byref(sp),
                                    FAKE, 1 << 40, None) == -1
    assert "null pointer" in ea.ea_last_error()
    bad = bnd.SparsityParams(32, 1, 0, 0.2, 0.0)
    assert L.ea_hybrid_prefill_plan(FAKE, FAKE, 1, 1000, 1000, 8, 2, 128, 1, ctypes.byref(bad),
                                    FAKE, 1 << 40, None) == -2
    assert L.ea_hybrid_prefill_plan(FAKE, FAKE, 1, 1000, 1000, 8, 2, 128, 1, ctypes.byref(sp),
                                    FAKE, 16, None) == -3
    # run: null Q, misaligned O
    assert L.ea_hybrid_prefill_run(None, FAKE, FAKE, 1, FAKE, FAKE, 1, 1000, 1000, 8, 2, 128,
                                   ctypes.byref(sp), FAKE, None, FAKE, 1 << 40, None) == -1
    assert L.ea_hybrid_prefill_run(FAKE, FAKE, FAKE, 1, FAKE, FAKE, 1, 1000, 1000, 8, 2, 128,
                                   ctypes.byref(sp), FAKE + 4, None, FAKE, 1 << 40, None) == -1
    assert "16-byte" in ea.ea_last_error()
    # zero tokens: nothing to do
    assert L.ea_hybrid_prefill_plan(FAKE, FAKE, 1, 0, 0, 8, 2, 128, 1, ctypes.byref(sp),
                                    FAKE, 1 << 40, None) == 0


def test_mfma_probe_host_errors():
    L = ea.lib()
    flops = ctypes.c_int64(0)
    cases = [
        (dict(out=None, n=256, iters=10), "null pointer"),
        (dict(out=FAKE, n=0, iters=10), "n_workgroups"),
        (dict(out=FAKE, n=2**20 + 1, iters=10), "n_workgroups"),
        (dict(out=FAKE, n=256, iters=0), "iters"),
        (dict(out=FAKE, n=256, iters=2**26 + 1), "iters"),
        (dict(out=FAKE + 4, n=256, iters=10), "aligned"),
    ]
    for c, msg in cases:
        st = L.ea_mfma_probe(c["out"], c["n"], c["iters"], 1, ctypes.byref(flops), None)
        assert st == bnd.EA_ERR_INVALID_ARG, (c, st)
        assert msg in ea.ea_last_error(), (c, ea.ea_last_error())


def test_gumbel_route_host_errors():
    L = ea.lib()
    cases = [
        ((None, None, 1.0, 4, FAKE, FAKE), "null pointer"),
        ((FAKE, None, 1.0, 4, FAKE, None), "null pointer"),
        ((FAKE, None, 1.0, -1, FAKE, FAKE), "n must be"),
        ((FAKE, None, 0.0, 4, FAKE, FAKE), "tau"),
        ((FAKE, None, -1.0, 4, FAKE, FAKE), "tau"),
        ((FAKE, None, float("inf"), 4, FAKE, FAKE), "tau"),
        ((FAKE, None, float("nan"), 4, FAKE, FAKE), "tau"),
    ]
    for args, msg in cases:
        assert L.ea_gumbel_route(*args, None) == bnd.EA_ERR_INVALID_ARG, args
        assert msg in ea.ea_last_error(), (args, ea.ea_last_error())
    # n = 0: nothing to launch
    assert L.ea_gumbel_route(FAKE, None, 1.0, 0, FAKE, FAKE, None) == 0


def test_dual_workspace_holds_two_entries_per_tile():
    one = ea.ea_hybrid_prefill_workspace_size(1, 131072, 131072, 32, 8, 128, bnd.EA_BF16)
    two = ea.ea_dual_prefill_workspace_size(1, 131072, 131072, 32, 8, 128, bnd.EA_BF16)
    items = 8 * (131072 // 64 + 1)
    assert two - one >= items * (20 + 8) - 4096
    assert ea.ea_dual_prefill_workspace_size(1, 1000, 1000, 30, 8, 128, 1) == 0


def test_dual_prefill_host_errors():
    L = ea.lib()
    sp = bnd.SparsityParams(64, 1, 0, 0.2, 0.0)
    A, B2, C, D2, E2, F2 = FAKE, FAKE + 256, FAKE + 512, FAKE + 768, FAKE + 1024, FAKE + 1280

    def call(modes=A, O=B2, O_fa=C, O_sa=D2, lse_fa=E2, lse_sa=F2, ws_bytes=1 << 40, sp_=sp):
        return L.ea_dual_prefill(A, A, A, 1, modes, A, 1, 1000, 1000, 8, 2, 128,
                                 ctypes.byref(sp_), O, O_fa, O_sa, lse_fa, lse_sa, A, ws_bytes,
                                 None)

    assert call(O_sa=None) == -1 and "null pointer" in ea.ea_last_error()
    assert call(lse_fa=None) == -1
    assert call(O_fa=None) == -1
    assert call(modes=None) == -1 and "modes is required" in ea.ea_last_error()
    assert call(O_sa=C) == -1 and "alias" in ea.ea_last_error()
    assert call(O=D2) == -1 and "alias" in ea.ea_last_error()
    assert call(lse_sa=E2) == -1 and "alias" in ea.ea_last_error()
    assert call(O_sa=D2 + 4) == -1 and "16-byte" in ea.ea_last_error()
    assert call(ws_bytes=16) == -3
    assert call(sp_=bnd.SparsityParams(32, 1, 0, 0.2, 0.0)) == -2
    # modes may be null when the mix is not requested; zero tokens launch nothing
    assert L.ea_dual_prefill(A, A, A, 1, None, A, 1, 0, 0, 8, 2, 128, ctypes.byref(sp), None, C,
                             D2, E2, F2, A, 1 << 40, None) == 0


def _desc(**kw):
    d = dict(B=1, Hkv=2, head_dim=128, max_len=131072, n_sink_blocks=1, window_blocks=0,
             keep_fraction=0.2)
    d.update(kw)
    return bnd.KVCacheDesc(*[d[k] for k in ["B", "Hkv", "head_dim", "max_len", "n_sink_blocks",
                                            "window_blocks", "keep_fraction"]])


def test_kvcache_bytes_mode_aware():
    import torch
    blk = 2 * 64 * 128 * 2                      # K and V rows of one 64-token block
    fa_fa = ea.ea_kvcache_bytes(_desc(), torch.zeros((1, 2), dtype=torch.int8))
    fa_sa = ea.ea_kvcache_bytes(_desc(), torch.tensor([[0, 1]], dtype=torch.int8))
    # FA slot: all 2048 blocks; SA slot: 1 sink + w(2048) = 409 window blocks
    assert fa_fa - fa_sa == (2048 - 410) * blk
    header = fa_fa - 2 * 2048 * blk
    assert 0 < header <= 4096
    # a window that covers the sequence keeps every block
    small = _desc(max_len=640, window_blocks=20)
    assert ea.ea_kvcache_bytes(small, torch.tensor([[1, 1]], dtype=torch.int8)) == \
        ea.ea_kvcache_bytes(small, torch.zeros((1, 2), dtype=torch.int8))
    # a fixed window: sinks + window
    fixed = _desc(max_len=64 * 100, window_blocks=7, n_sink_blocks=2)
    assert ea.ea_kvcache_bytes(fixed, torch.zeros((1, 2), dtype=torch.int8)) - \
        ea.ea_kvcache_bytes(fixed, torch.tensor([[0, 1]], dtype=torch.int8)) == (100 - 9) * blk
    # invalid descriptors -> 0
    z = torch.zeros((1, 2), dtype=torch.int8)
    for bad in (dict(head_dim=96), dict(keep_fraction=0.0), dict(max_len=0), dict(B=0),
                dict(n_sink_blocks=-1), dict(max_len=2**21 + 1)):
        assert ea.ea_kvcache_bytes(_desc(**bad), z) == 0, bad


def test_kvcache_and_decode_host_errors():
    L = ea.lib()
    d = _desc()
    ws = ea.ea_decode_workspace_size(d, 8)
    assert ws >= 1 * 8 * 128 * 128 * 4          # chunk partials: B x Hq x chunks x d floats
    A = FAKE
    assert L.ea_kvcache_init(ctypes.byref(d), None, A, 1 << 30, None) == -1
    assert L.ea_kvcache_init(ctypes.byref(d), A, A + 16, 1 << 30, None) == -1
    assert "256-byte" in ea.ea_last_error()
    assert L.ea_kvcache_init(ctypes.byref(d), A, A, 16, None) == -3
    assert L.ea_kvcache_prefill(ctypes.byref(d), A, 1 << 30, None, A, A, 10, None) == -1

    def step(Hq=8, scale=0.0, ws_bytes=ws, q=A, d_=d):
        return L.ea_decode_step(ctypes.byref(d_), A, 1 << 30, q, A, A, Hq, scale, A, None, A,
                                ws_bytes, None)

    assert step(q=None) == -1
    assert step(Hq=7) == -1 and "multiple" in ea.ea_last_error()
    assert step(Hq=2 * 17) == -2 and "16" in ea.ea_last_error()
    assert step(scale=-1.0) == -1
    assert step(ws_bytes=16) == -3
    assert step(q=A + 8) == -1 and "16-byte" in ea.ea_last_error()
    assert step(d_=_desc(head_dim=80)) == -2


def test_backward_host_errors():
    L = ea.lib()
    sp = bnd.SparsityParams(64, 1, 0, 0.2, 0.0)
    A = FAKE
    ws = ea.ea_hybrid_backward_workspace_size(1, 1000, 1000, 8, 2, 128, bnd.EA_BF16)
    assert ws > ea.ea_hybrid_prefill_workspace_size(1, 1000, 1000, 8, 2, 128, bnd.EA_BF16) + 2 * 8 * 1000 * 4 - 1

    def call(dtype=1, dO=A, lse=A, dQ=A, ws_bytes=ws, O=A):
        return L.ea_hybrid_backward(A, A, A, O, dO, lse, dtype, A, A, 1, 1000, 1000, 8, 2, 128,
                                    ctypes.byref(sp), dQ, A, A, A, ws_bytes, None)

    assert call(dtype=0) == -2 and "bf16" in ea.ea_last_error()
    assert call(dO=None) == -1
    assert call(lse=None) == -1
    assert call(O=None) == -1
    assert call(dQ=A + 8) == -1 and "16-byte" in ea.ea_last_error()
    assert call(ws_bytes=ws - 1) == -3


def test_xa_workspace_holds_the_selection_lists():
    one = ea.ea_hybrid_prefill_workspace_size(1, 131072, 131072, 32, 8, 128, bnd.EA_BF16)
    xa = ea.ea_xa_prefill_workspace_size(1, 131072, 131072, 32, 8, 128, bnd.EA_BF16)
    nqb = 131072 // 128
    tri = nqb * (nqb + 1) // 2
    # counts [Hkv, nqb], the triangular lists [Hkv, tri] of int32, the XA rows
    # [Hkv], and the selection's float32 scratch [Hq, tri, 16]
    need = 4 * 8 * nqb + 4 * 8 * tri + 4 * 8 + 4 * 32 * tri * 16
    assert need <= xa - one <= need + 1024
    assert ea.ea_xa_prefill_workspace_size(1, 1000, 1000, 30, 8, 128, 1) == 0


def test_xa_prefill_host_errors():
    L = ea.lib()
    A = FAKE

    def call(dtype=1, Hq=8, Hkv=2, d=128, T=1000, max_seqlen=1000, xa=(128, 8, 0.9, 2),
             ws_bytes=1 << 40, modes=A, O=A):
        sp = bnd.SparsityParams(64, 1, 0, 0.2, 0.0)
        xp = None if xa is None else ctypes.byref(bnd.XAParams(*xa))
        return L.ea_xa_prefill(A, A, A, dtype, modes, A, 1, T, max_seqlen, Hq, Hkv, d,
                               ctypes.byref(sp), xp, O, None, None, None, A, ws_bytes, None)

    assert call(xa=None) == -1 and "null XA" in ea.ea_last_error()
    assert call(xa=(64, 8, 0.9, 2)) == -2 and "block" in ea.ea_last_error()
    assert call(xa=(128, 16, 0.9, 2)) == -2 and "stride" in ea.ea_last_error()
    assert call(xa=(128, 8, 1.5, 2)) == -1 and "threshold" in ea.ea_last_error()
    assert call(xa=(128, 8, float("nan"), 2)) == -1
    assert call(xa=(128, 8, 0.9, 3)) == -1 and "head configuration" in ea.ea_last_error()
    assert call(dtype=0) == -2 and "EA_BF16" in ea.ea_last_error()
    assert call(Hq=2, Hkv=2) == -2 and "power of two" in ea.ea_last_error()
    assert call(Hq=24, Hkv=2) == -2
    assert call(Hq=64, Hkv=2, d=64) == -2
    assert call(T=600000, max_seqlen=600000, Hq=4, Hkv=2, d=64) == -2 and "too long" in ea.ea_last_error()
    assert call(modes=None) == -1
    assert call(O=None) == -1
    assert call(ws_bytes=16) == -3
    # zero tokens launch nothing
    assert call(T=0, max_seqlen=0) == 0
    # the two halves validate the same way
    sp = bnd.SparsityParams(64, 1, 0, 0.2, 0.0)
    xp = bnd.XAParams(128, 8, 0.9, 2)
    assert L.ea_xa_prefill_plan(A, A, 0, A, A, 1, 1000, 1000, 8, 2, 128, ctypes.byref(sp),
                                ctypes.byref(xp), None, None, A, 1 << 40, None) == -2
    assert L.ea_xa_prefill_plan(None, A, 1, A, A, 1, 1000, 1000, 8, 2, 128, ctypes.byref(sp),
                                ctypes.byref(xp), None, None, A, 1 << 40, None) == -1
    assert L.ea_xa_prefill_run(A, A, A, 1, A, A, 1, 1000, 1000, 8, 2, 128, ctypes.byref(sp),
                               None, A, None, A, 1 << 40, None) == -1
    assert L.ea_xa_prefill_run(A, A, None, 1, A, A, 1, 1000, 1000, 8, 2, 128, ctypes.byref(sp),
                               ctypes.byref(xp), A, None, A, 1 << 40, None) == -1


def test_workspace_status_host_errors():
    L = ea.lib()
    assert L.ea_workspace_status(None, 4096, None) == bnd.EA_ERR_INVALID_ARG
    assert "null pointer" in ea.ea_last_error()
    assert L.ea_workspace_status(FAKE, 16, None) == bnd.EA_ERR_WORKSPACE
    assert "at least" in ea.ea_last_error()


def test_cache_desc_rejects_huge_geometry():
    L = ea.lib()
    for ns, wb in [(2**24 + 1, 0), (1, 2**31 - 1)]:
        desc = bnd.KVCacheDesc(1, 8, 128, 4096, ns, wb, 0.2)
        assert L.ea_kvcache_init(ctypes.byref(desc), FAKE, FAKE, 1 << 30, None) == bnd.EA_ERR_INVALID_ARG
        assert "2^24" in ea.ea_last_error() or "16777216" in ea.ea_last_error()


def test_plan_layout_is_inside_the_workspace():
    for args in [(1, 131072, 131072, 32, 8, 128, 1), (3, 5000, 4000, 8, 2, 64, 0)]:
        lay = ea.ea_hybrid_prefill_plan_layout(*args)
        ws = ea.ea_hybrid_prefill_workspace_size(*args)
        n = lay["n_slots"]
        assert lay["items"] + 20 * n <= ws and lay["keys"] + 4 * n <= ws and lay["order"] + 4 * n <= ws
        spans = sorted([(lay["items"], 20 * n), (lay["keys"], 4 * n), (lay["order"], 4 * n)])
        assert all(a + la <= b for (a, la), (b, _) in zip(spans, spans[1:]))
        assert spans[0][0] >= 256          # after the header
    with pytest.raises(ea.EAError):
        ea.ea_hybrid_prefill_plan_layout(0, 10, 10, 8, 2, 64, 1)


def test_noalloc_rejects_sizes_beyond_its_static_workspace():
    L = ea.lib()
    cap = ea.ea_hybrid_prefill_noalloc_max_workspace()
    assert cap == 4 << 20
    sp = bnd.SparsityParams(64, 1, 0, 0.2, 0.0)
    # 4M tokens x 8 KV heads need far more than 4 MiB of work list
    st = L.ea_hybrid_prefill_noalloc(FAKE, FAKE, FAKE, 1, FAKE, FAKE, 1, 2**22, 2**17, 32, 8, 128,
                                     ctypes.byref(sp), FAKE, None, None)
    assert st == bnd.EA_ERR_WORKSPACE and "static workspace" in ea.ea_last_error()
    # the 128K headline layer fits
    assert ea.ea_hybrid_prefill_workspace_size(1, 131072, 131072, 32, 8, 128, 1) <= cap
    # invalid sizes are rejected before any device call
    st = L.ea_hybrid_prefill_noalloc(FAKE, FAKE, FAKE, 1, FAKE, FAKE, 0, 10, 10, 8, 2, 128,
                                     ctypes.byref(sp), FAKE, None, None)
    assert st == bnd.EA_ERR_INVALID_ARG
