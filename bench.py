"""Throughput of the routed hybrid attention prefill on one MI355X.

One step = the whole hot path of one transformer layer's attention, run once
for each routing mix of the headline workload, on inputs already resident in
device memory: the router (boundary pooling, task MLP, router MLP, argmax),
the cost-ordered work list, and the fused FA/SA attention forward.  The
headline workload is the 128K-token Qwen3-4B-shaped layer (32 query heads, 8
KV heads, d = 128, bf16, one sequence) in its two routing mixes, 2 of 8 and 6
of 8 KV heads sparse, so one step is two layers.  `value` is effective TFLOP/s
over the whole step: the effective FLOPs of both layers (only the computed
64 x 64 FA/SA blocks count, the router's few MFLOP do not) over the step time.

`roofline` is the attention kernel alone: its effective FLOPs per launch over
its average launch time, from HIP events recorded on the stream it runs on,
against the MI355X dense bf16 MFMA peak.  `traffic` is that kernel's HBM bytes
per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE counters (scaled by what the
same counters read for an elementwise kernel of known size), read from
profiles/attention_traffic.json when it was taken on the current kernel
source, else null.  `mfma_busy` is the share of SIMD-cycles in which that
kernel's matrix pipe is busy (rocprofv3 SQ_VALU_MFMA_BUSY_CYCLES over
GRBM_GUI_ACTIVE x 1024 SIMDs / 8 XCDs), from
profiles/attention_sq_counters.json under the same source-hash rule.  `mfma_loop_tflops` is the practical ceiling beside the
data-sheet peak: the library's MFMA-loop probe (8 waves per CU issuing
back-to-back bf16 MFMAs with no memory traffic) at whatever clock the board
holds under that load, measured in the same run.

Prints one JSON line.  --gpus must be 1: the path is measured on one GPU.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import re
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "hybrid prefill effective TFLOP/s + ms/layer at 128K; % bf16 MFMA roofline"
DEFAULT_RUNS = ["qwen4b_s128k_sa2", "qwen4b_s128k_sa6"]
# The sources that decide the attention kernel's memory traffic: the kernel,
# the work-list order that places its workgroups on the XCDs, and the
# constants of the shared header that those two use (with the constants their
# definitions use in turn).
ATTN_SRCS = [os.path.join(ROOT, "full_attention_long_amd", "csrc", f)
             for f in ("ea_attention.hip", "ea_worklist.hip")]
ATTN_HEADER = os.path.join(ROOT, "full_attention_long_amd", "csrc", "ea_internal.h")
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "attention_traffic.json")
SQ_JSON = os.path.join(ROOT, "profiles", "attention_sq_counters.json")
N_XCD, N_SIMD = 8, 1024   # MI355X: 8 XCDs, 256 CUs x 4 SIMDs
ATTN_KERNEL = "attention_kernel"
CALIB_KERNEL = "bitwise_not"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def mfma_probe(target_ms: float = 100.0, launches: int = 3) -> dict:
    """Practical bf16 matrix-core ceiling: the library's MFMA-loop probe (one
    workgroup of 8 waves per CU, back-to-back 32x32x16 bf16 MFMAs, no memory
    traffic) timed with HIP events on the current stream."""
    import torch

    import full_attention_long_amd as ea
    n = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(n * 512, dtype=torch.float32, device="cuda")
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def timed(iters):
        a, b = E(), E()
        a.record()
        flops = ea.ea_mfma_probe(out, n, iters)
        b.record()
        torch.cuda.synchronize()
        return flops, a.elapsed_time(b)

    timed(2000)
    _, ms = timed(20000)
    iters = max(1000, int(20000 * target_ms / max(ms, 1e-3)))
    timed(iters)  # settle the clock under the full-length load
    res = [timed(iters) for _ in range(launches)]
    ms = float(np.median([r[1] for r in res]))
    flops = res[0][0]
    assert bool(torch.isfinite(out).all()), "probe checksums not finite"
    return {"tflops": round(flops / (ms * 1e-3) / 1e12, 1), "ms": round(ms, 3),
            "workgroups": n, "iters": iters}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    texts = []
    for path in ATTN_SRCS:
        with open(path, "rb") as f:
            data = f.read()
        h.update(data)
        texts.append(data.decode())
    defs, code = {}, []
    with open(ATTN_HEADER) as f:
        for ln in f:
            m = re.match(r"\s*constexpr int (k\w+)\s*=", ln)
            if m:
                defs[m.group(1)] = ln.strip()
            else:
                code.append(ln.split("//")[0])  # the header's own code (its helpers)
    used, todo = set(), "\n".join(texts + code)
    while True:
        new = {k for k in defs if k not in used and re.search(r"\b%s\b" % k, todo)}
        if not new:
            break
        used |= new
        todo = "\n".join(defs[k] for k in new)
    h.update("\n".join(defs[k] for k in sorted(used)).encode())
    return h.hexdigest()[:16]


class Layer:
    """One routed layer's device-resident inputs, outputs and workspace."""

    def __init__(self, name):
        import torch

        import full_attention_long_amd as ea
        from workloads import gen
        from workloads.configs import WORKLOADS

        self.name = name
        log(f"{name}: generating inputs")
        self.case = c = gen.build_case(WORKLOADS[name])
        bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()  # noqa: E731
        self.q, self.k, self.v = bf(c.q), bf(c.k), bf(c.v)
        self.cu = torch.from_numpy(c.cu_seqlens).cuda()
        self.w = {n: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
                  for n, a in c.weights.items()}
        self.maxlen = int(c.lengths.max())
        self.O = torch.empty_like(self.q)
        self.lse = torch.empty((c.Hq, c.T), dtype=torch.float32, device="cuda")
        self.modes = torch.empty((c.B, c.Hkv), dtype=torch.int8, device="cuda")
        self.logits = torch.empty((c.B, c.Hkv, 2), dtype=torch.float32, device="cuda")
        nbytes = ea.ea_hybrid_prefill_workspace_size(c.B, c.T, self.maxlen, c.Hq, c.Hkv, c.d, 1)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        self.geom = dict(n_sink=c.n_sink, keep_fraction=c.keep_fraction)

    def step(self, ev=None):
        """Router, work list, attention; ev = 4 events bracketing route / plan / run."""
        import full_attention_long_amd as ea
        c = self.case
        if ev is not None:
            ev[0].record()
        ea.ea_route(self.k, self.cu, self.w, pool_len=c.pool_len, modes=self.modes,
                    logits=self.logits)
        if ev is not None:
            ev[1].record()
        ea.ea_hybrid_prefill_plan(self.modes, self.cu, c.T, self.maxlen, c.Hq, c.Hkv, c.d, 1,
                                  self.ws, **self.geom)
        if ev is not None:
            ev[2].record()
        ea.ea_hybrid_prefill_run(self.q, self.k, self.v, self.modes, self.cu, self.maxlen, self.ws,
                                 out=self.O, lse=self.lse, **self.geom)
        if ev is not None:
            ev[3].record()


def stored_traffic():
    """HBM bytes per attention launch per workload from the stored counter
    summary, if it was taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_JSON) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return t


def stored_sq():
    """Matrix-pipe utilisation of the attention kernel from the stored SQ
    counter summary, if it was taken on the current kernel source; else None."""
    try:
        with open(SQ_JSON) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return t


def cpu_info():
    """Host CPU model and the cores this process may run on."""
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def pin_blas(cores):
    """Limit the BLAS thread pools to `cores` threads (returns the limiter)."""
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=cores)
    except Exception:  # pragma: no cover
        return None


def cpu_baseline(cases, budget_s=12.0):
    """The oracle on a bounded sample of the same layers: 64-row query blocks
    of one query head at seeded positions, alternating between the layers,
    until ~budget_s of CPU time is spent; effective FLOPs of the sample over
    its wall time."""
    from full_attention_long_amd import metrics
    from oracle import ea_oracle as orc

    model, cores = cpu_info()
    limiter = pin_blas(cores)
    rng = np.random.default_rng(0)
    f32 = [(c.q_f32(), c.k_f32(), c.v_f32()) for c in cases]
    total_flops = sum(metrics.effective_flops(c.target_modes, c.lengths, c.Hq, c.Hkv, c.d,
                                              n_sink=c.n_sink, keep_fraction=c.keep_fraction)
                      for c in cases)
    done_flops, units, t_used = 0, 0, 0.0
    while t_used < budget_s and units < 512:
        ci = units % len(cases)
        c = cases[ci]
        qf, kf, vf = f32[ci]
        L = int(c.lengths[0])
        G = c.Hq // c.Hkv
        w = metrics.window_blocks(L, c.n_sink, c.keep_fraction)
        g = (units // len(cases)) % c.Hkv
        hq = g * G + (units // (len(cases) * c.Hkv)) % G
        qb = int(rng.integers(0, L // 64))
        toks = np.arange(qb * 64, min(L, qb * 64 + 64))
        t0 = time.perf_counter()
        orc.hybrid_attention_rows(qf, kf, vf, c.target_modes, c.cu_seqlens, toks, [hq],
                                  n_sink=c.n_sink, keep_fraction=c.keep_fraction)
        t_used += time.perf_counter() - t0
        nvis = qb + 1 if c.target_modes[0, g] == 0 else min(qb + 1, c.n_sink + w)
        done_flops += 4 * c.d * len(toks) * 64 * nvis
        units += 1
    if limiter is not None:
        limiter.restore_original_limits()
    frac = done_flops / total_flops
    return {
        "value": round(done_flops / t_used / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
        "kind": "oracle", "precision": "float64", "cpu_model": model,
        "sample_fraction": round(frac, 6), "extrapolated": bool(frac < 0.05),
        "sample": f"{units} query blocks of 64 rows x one query head at seeded positions, "
                  f"alternating {'+'.join(c.name for c in cases)} ({100 * frac:.3f}% of the "
                  f"step's effective FLOPs; the rate is extrapolated from it); float64 two-pass "
                  f"softmax over the visible keys on {cores} cores (BLAS threads pinned to "
                  f"them); {t_used:.1f} s of CPU",
    }


def cpu_baseline_dual(c, budget_s=12.0):
    """The oracle's dual-mode forward on a bounded sample of the layer: 64-row
    query blocks of one query head at seeded positions, each computed in both
    modes, until ~budget_s of CPU time is spent; the FA FLOPs of the sample
    (the dual forward's effective work) over its wall time."""
    from oracle import ea_oracle as orc

    model, cores = cpu_info()
    limiter = pin_blas(cores)
    rng = np.random.default_rng(0)
    qf, kf, vf = c.q_f32(), c.k_f32(), c.v_f32()
    L = int(c.lengths[0])
    r_soft = np.full((c.B, c.Hkv, 2), 0.5)
    modes = np.zeros((c.B, c.Hkv), np.int8)
    done_flops, units, t_used = 0, 0, 0.0
    while t_used < budget_s and units < 512:
        hq = units % c.Hq
        qb = int(rng.integers(0, L // 64))
        toks = np.arange(qb * 64, min(L, qb * 64 + 64))
        t0 = time.perf_counter()
        orc.dual_attention_rows(qf, kf, vf, c.cu_seqlens, r_soft, modes, toks, [hq],
                                n_sink=c.n_sink, keep_fraction=c.keep_fraction)
        t_used += time.perf_counter() - t0
        done_flops += 4 * c.d * len(toks) * 64 * (qb + 1)
        units += 1
    if limiter is not None:
        limiter.restore_original_limits()
    return {
        "value": round(done_flops / t_used / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
        "kind": "oracle", "precision": "float64", "cpu_model": model, "extrapolated": True,
        "sample": f"{units} query blocks of 64 rows x one query head at seeded positions of "
                  f"{c.name}, each in both modes; float64 two-pass softmax on {cores} cores; "
                  f"{t_used:.1f} s of CPU",
    }


def bench_dual(args):
    """Dual-mode (training) forward of one layer: router logits, Gumbel-Softmax
    hard decisions, and the dual attention (work list, one attention launch
    over every head's SA set and the rest of its causal blocks, merge); prints
    one JSON line of its own."""
    import torch

    import full_attention_long_amd as ea
    from full_attention_long_amd import metrics
    from workloads import gen
    name = args.runs.split(",")[0]
    ly = Layer(name)
    c = ly.case
    noise = torch.from_numpy(gen.draw_gumbel(c.seed, (c.B, c.Hkv, 2))).cuda()
    r_soft = torch.empty((c.B, c.Hkv, 2), dtype=torch.float32, device="cuda")
    O_fa, O_sa = torch.empty_like(ly.q), torch.empty_like(ly.q)
    lse_fa = torch.empty((c.Hq, c.T), dtype=torch.float32, device="cuda")
    lse_sa = torch.empty_like(lse_fa)
    nbytes = ea.ea_dual_prefill_workspace_size(c.B, c.T, ly.maxlen, c.Hq, c.Hkv, c.d, 1)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        ea.ea_route(ly.k, ly.cu, ly.w, pool_len=c.pool_len, modes=ly.modes, logits=ly.logits)
        ea.ea_gumbel_route(ly.logits, args.tau, gumbel=noise, r_soft=r_soft, modes=ly.modes)
        if ev is not None:
            ev[1].record()
        ea.ea_dual_prefill(ly.q, ly.k, ly.v, ly.cu, ly.maxlen, modes=ly.modes, out=ly.O,
                           out_fa=O_fa, out_sa=O_sa, lse_fa=lse_fa, lse_sa=lse_sa, workspace=ws,
                           **ly.geom)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ef = metrics.effective_flops(np.zeros((c.B, c.Hkv), np.int8), c.lengths, c.Hq, c.Hkv, c.d,
                                 n_sink=c.n_sink, keep_fraction=c.keep_fraction)
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    evs = [[E() for _ in range(3)] for _ in range(args.steps)]
    start, stop = E(), E()
    torch.cuda.synchronize()
    start.record()
    for s in range(args.steps):
        step(evs[s])
    stop.record()
    torch.cuda.synchronize()
    step_ms = start.elapsed_time(stop) / args.steps
    seg = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2])] for e in evs])
    route_ms, dual_ms = seg.mean(axis=0)
    log(f"dual {name}: step {step_ms:.3f} ms (routing {route_ms:.3f}, dual forward {dual_ms:.3f})")
    probe = mfma_probe()
    achieved = ef / (dual_ms * 1e-3) / 1e12
    peak = metrics.MI355X_BF16_DENSE_TFLOPS
    out = {
        "metric": "dual-mode training forward effective TFLOP/s at 128K (FA FLOPs of every head)",
        "value": round(ef / (step_ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name + ":dual", "seq_len": ly.maxlen, "Hq": c.Hq, "Hkv": c.Hkv,
                   "d": c.d, "tau": args.tau, "effective_flops": int(ef),
                   "routing_ms": round(float(route_ms), 4),
                   "dual_forward_ms": round(float(dual_ms), 4),
                   "sa_kv_heads": int(ly.modes.sum().item())},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None,
                     "kernel": "ea_dual_prefill (work list + ea::attention_kernel_bf16<128, false> + "
                               "dual_merge_kernel)",
                     "mfma_loop_tflops": probe["tflops"],
                     "frac_of_mfma_loop": round(achieved / probe["tflops"], 4)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_dual(c, args.cpu_budget)
    print(json.dumps(out), flush=True)


def decode_bytes(lengths, modes, Hq, Hkv, d, n_sink, keep_fraction, window_blocks=0):
    """Algorithmic HBM bytes of one decode step: the K and V rows every query
    must read (FA: all of the sequence; SA: sink blocks and the window, as for
    the last row of the prefill of the longer sequence), the new K/V rows
    written, q read, O written (bf16) and the LSE (fp32)."""
    from full_attention_long_amd import metrics
    total = 0
    for b, L in enumerate(lengths):
        n = int(L) + 1                      # history including the new token
        N = -(-n // 64)
        w = window_blocks or metrics.window_blocks(n, n_sink, keep_fraction)
        qb = (n - 1) // 64
        for g in range(Hkv):
            if modes[b, g] == 0:
                keys = n
            else:
                ws = max(0, qb - w + 1)
                sinks = min(n_sink, ws) * 64
                keys = sinks + (n - ws * 64)
            total += keys * d * 2 * 2
        del N
    B = len(lengths)
    total += B * Hkv * d * 2 * 2             # new K/V rows
    total += B * Hq * d * 2 * 2 + B * Hq * 4  # q in, O out, LSE
    return total


def bench_decode(args):
    """Decode steps over a mode-aware KV cache holding a long prompt: one
    token per sequence per step (append + split attention + combine); prints
    one JSON line of its own with the HBM roofline of the step."""
    import torch

    import full_attention_long_amd as ea
    from workloads import gen
    from workloads.configs import WORKLOADS
    lines = []
    for name in args.runs.split(","):
        c = gen.build_case(WORKLOADS[name])
        modes = c.target_modes
        lengths = [int(x) for x in c.lengths]
        max_len = max(lengths) + args.steps + args.warmup + 64
        cache = ea.KVCache(torch.from_numpy(modes), max_len, c.d, n_sink=c.n_sink,
                           keep_fraction=c.keep_fraction)
        fa_bytes = ea.ea_kvcache_bytes(cache.desc, torch.zeros_like(torch.from_numpy(modes)))
        bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()  # noqa: E731
        cache.prefill(bf(c.k), bf(c.v), torch.from_numpy(c.cu_seqlens.astype(np.int32)).cuda())
        B, Hq, Hkv, d = c.B, c.Hq, c.Hkv, c.d
        g = torch.Generator(device="cuda").manual_seed(1)
        q = torch.randn((B, Hq, d), generator=g, device="cuda").to(torch.bfloat16)
        kn = torch.randn((B, Hkv, d), generator=g, device="cuda").to(torch.bfloat16)
        vn = torch.randn((B, Hkv, d), generator=g, device="cuda").to(torch.bfloat16)
        O = torch.empty_like(q)
        lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        for _ in range(args.warmup):
            cache.decode(q, kn, vn, out=O, lse=lse)
        torch.cuda.synchronize()
        start_len = cache.lengths.cpu().numpy().copy()
        E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
        evs = [(E(), E()) for _ in range(args.steps)]
        for s in range(args.steps):
            evs[s][0].record()
            cache.decode(q, kn, vn, out=O, lse=lse)
            evs[s][1].record()
        torch.cuda.synchronize()
        ms = np.array([a.elapsed_time(b) for a, b in evs])
        nbytes = np.mean([decode_bytes(start_len + s, modes, Hq, Hkv, d, c.n_sink,
                                       c.keep_fraction) for s in range(args.steps)])
        med = float(np.median(ms))
        gbps = nbytes / (med * 1e-3) / 1e9
        log(f"decode {name}: {med * 1e3:.1f} us per step, {nbytes / 1e6:.1f} MB -> {gbps:.0f} GB/s; "
            f"cache {cache.nbytes / 2**20:.0f} MiB vs {fa_bytes / 2**20:.0f} MiB all-FA")
        lines.append({"workload": name, "B": B, "context": max(lengths), "Hq": Hq, "Hkv": Hkv,
                      "d": d, "sa_kv_heads": int(modes.sum()), "step_us_median": round(med * 1e3, 2),
                      "bytes_per_step": int(nbytes), "gbps": round(gbps, 1),
                      "cache_bytes": int(cache.nbytes), "cache_bytes_all_fa": int(fa_bytes)})
        del cache
        torch.cuda.empty_cache()
    tot_bytes = sum(r["bytes_per_step"] for r in lines)
    tot_us = sum(r["step_us_median"] for r in lines)
    gbps = tot_bytes / (tot_us * 1e-6) / 1e9
    peak = 8000.0
    out = {
        "metric": "decode step HBM throughput over the mode-aware KV cache (GB/s)",
        "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(tot_us / len(lines) / 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "+".join(r["workload"] for r in lines) + ":decode", "runs": lines},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": peak, "unit": "GB/s",
                     "frac": round(gbps / peak, 4), "traffic": None,
                     "kernel": "ea_decode_step (append + decode_attn_kernel + combine)"},
    }
    print(json.dumps(out), flush=True)


def bench_backward(args):
    """Backward of each --runs layer (work list, D / LSE pass, dQ kernel, dK/dV
    kernel) after its forward; effective FLOPs = 2.5x the forward's (the five
    products S, dP, dV, dQ, dK over the visible blocks).  Prints one JSON line
    of its own."""
    import torch

    import full_attention_long_amd as ea
    from full_attention_long_amd import metrics
    runs = []
    tot_ef = tot_ms = 0.0
    for name in args.runs.split(","):
        ly = Layer(name)
        c = ly.case
        ly.step()
        torch.cuda.synchronize()
        g = torch.Generator(device="cuda").manual_seed(3)
        dO = torch.randn(ly.q.shape, generator=g, device="cuda").to(torch.bfloat16)
        dQ, dK, dV = torch.empty_like(ly.q), torch.empty_like(ly.k), torch.empty_like(ly.v)
        nbytes = ea.ea_hybrid_backward_workspace_size(c.B, c.T, ly.maxlen, c.Hq, c.Hkv, c.d, 1)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

        def bwd():
            ea.ea_hybrid_backward(ly.q, ly.k, ly.v, ly.O, dO, ly.lse, ly.modes, ly.cu, ly.maxlen,
                                  dQ=dQ, dK=dK, dV=dV, workspace=ws, **ly.geom)

        for _ in range(args.warmup):
            bwd()
        torch.cuda.synchronize()
        E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
        evs = [(E(), E()) for _ in range(args.steps)]
        for s in range(args.steps):
            evs[s][0].record()
            bwd()
            evs[s][1].record()
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
        ef = 2.5 * metrics.effective_flops(ly.modes.cpu().numpy(), c.lengths, c.Hq, c.Hkv, c.d,
                                           n_sink=c.n_sink, keep_fraction=c.keep_fraction)
        log(f"backward {name}: {ms:.3f} ms, {ef / (ms * 1e-3) / 1e12:.1f} TFLOP/s")
        runs.append({"workload": name, "backward_ms": round(ms, 4), "effective_flops": int(ef),
                     "tflops": round(ef / (ms * 1e-3) / 1e12, 3),
                     "sa_kv_heads": int(ly.modes.sum().item())})
        tot_ef += ef
        tot_ms += ms
        del ly, dO, dQ, dK, dV, ws
        torch.cuda.empty_cache()
    value = tot_ef / (tot_ms * 1e-3) / 1e12
    probe = mfma_probe()
    peak = metrics.MI355X_BF16_DENSE_TFLOPS
    out = {
        "metric": "hybrid-layer backward effective TFLOP/s at 128K (2.5x forward FLOPs)",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(tot_ms / len(runs), 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "+".join(r["workload"] for r in runs) + ":backward", "runs": runs},
        "roofline": {"bound": "mfma", "achieved": round(value, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(value / peak, 4), "traffic": None,
                     "kernel": "ea_hybrid_backward (bwd_pre + bwd_dq_kernel + bwd_dkv_kernel)",
                     "mfma_loop_tflops": probe["tflops"],
                     "frac_of_mfma_loop": round(value / probe["tflops"], 4)},
    }
    print(json.dumps(out), flush=True)


def cpu_baseline_xa(c, cmodes, budget_s=12.0):
    """The oracle's XA path on a bounded sample of the layer: for XA query
    heads at seeded query blocks, the block masses of that block row, its
    selection, and the attention of its 128 rows over the kept blocks, until
    ~budget_s of CPU time is spent; the sample's computed-block FLOPs over its
    wall time."""
    from oracle import xa_oracle as xo

    model, cores = cpu_info()
    limiter = pin_blas(cores)
    from workloads import gen
    rng = np.random.default_rng(0)
    G = c.Hq // c.Hkv
    L = int(c.lengths[0])
    nb = -(-L // 128)
    xa_heads = [hq for hq in range(c.Hq) if cmodes[0, hq // G] == xo.MODE_XA]
    qh = {hq: gen.bf16_bits_to_f32(np.ascontiguousarray(c.q[:, hq])) for hq in xa_heads[:2]}
    kh = {g: gen.bf16_bits_to_f32(np.ascontiguousarray(c.k[:, g])) for g in {h // G for h in qh}}
    vh = {g: gen.bf16_bits_to_f32(np.ascontiguousarray(c.v[:, g])) for g in kh}
    done_flops, units, t_used = 0, 0, 0.0
    while t_used < budget_s and units < 256:
        hq = list(qh)[units % len(qh)]
        g = hq // G
        i = int(rng.integers(0, nb))
        t0 = time.perf_counter()
        A = xo.block_mass_rows(qh[hq], kh[g], [i])
        keep = xo.select_row(A[0], i, 0.9)
        rows = np.arange(i * 128, min(L, i * 128 + 128))
        cols = np.concatenate([np.arange(j * 128, min(L, j * 128 + 128)) for j in np.nonzero(keep)[0]])
        s_ = (qh[hq][rows].astype(np.float64) @ kh[g][cols].astype(np.float64).T) / np.sqrt(c.d)
        s_ = np.where(cols[None, :] <= rows[:, None], s_, -np.inf)
        p = np.exp(s_ - s_.max(axis=1, keepdims=True))
        _ = (p @ vh[g][cols].astype(np.float64)) / p.sum(axis=1, keepdims=True)
        t_used += time.perf_counter() - t0
        done_flops += 4 * c.d * len(rows) * len(cols)
        units += 1
    if limiter is not None:
        limiter.restore_original_limits()
    return {
        "value": round(done_flops / t_used / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
        "kind": "oracle", "precision": "float64", "cpu_model": model, "extrapolated": True,
        "sample": f"{units} XA query blocks of 128 rows x one query head at seeded positions of "
                  f"{c.name}: block masses of the row, threshold selection, float64 attention "
                  f"over the kept blocks; FLOPs of the kept blocks; {cores} cores; {t_used:.1f} s "
                  f"of CPU",
    }


def bench_xa(args):
    """Hybrid prefill with XAttention heads (one layer): router, XA selection +
    work list (plan), fused attention (run).  Effective FLOPs count the blocks
    the heads compute (XA heads: the kept ones).  Also times an all-FA prefill
    of the same inputs for the speedup over full attention.  Prints one JSON
    line of its own."""
    import torch

    import full_attention_long_amd as ea
    from full_attention_long_amd import metrics
    from workloads import gen
    from workloads.configs import WORKLOADS
    name = args.runs.split(",")[0]
    hitters = None if args.xa_plain else (0.1, 8.0)
    log(f"xa {name} {args.xa_config} hitters={hitters}: generating inputs")
    c = gen.build_case(WORKLOADS[name], hitters=hitters)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()  # noqa: E731
    q, k, v = bf(c.q), bf(c.k), bf(c.v)
    cu = torch.from_numpy(c.cu_seqlens).cuda()
    w = {n: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda() for n, a in c.weights.items()}
    maxlen = int(c.lengths.max())
    O = torch.empty_like(q)
    lse = torch.empty((c.Hq, c.T), dtype=torch.float32, device="cuda")
    modes = torch.empty((c.B, c.Hkv), dtype=torch.int8, device="cuda")
    logits = torch.empty((c.B, c.Hkv, 2), dtype=torch.float32, device="cuda")
    ws = torch.empty(ea.ea_xa_prefill_workspace_size(c.B, c.T, maxlen, c.Hq, c.Hkv, c.d, 1),
                     dtype=torch.uint8, device="cuda")
    xg = dict(head_config=args.xa_config, threshold=args.xa_tau, n_sink=c.n_sink,
              keep_fraction=c.keep_fraction)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        ea.ea_route(k, cu, w, pool_len=c.pool_len, modes=modes, logits=logits)
        if ev is not None:
            ev[1].record()
        ea.ea_xa_prefill_plan(q, k, modes, cu, maxlen, ws, **xg)
        if ev is not None:
            ev[2].record()
        ea.ea_xa_prefill_run(q, k, v, modes, cu, maxlen, ws, out=O, lse=lse, **xg)
        if ev is not None:
            ev[3].record()

    for _ in range(max(1, args.warmup)):  # the routing check below reads a step's modes
        step()
    torch.cuda.synchronize()
    m = modes.cpu().numpy()
    assert np.array_equal(m, c.target_modes), f"{name}: routing differs from the target"
    cm = metrics.computation_modes(m, args.xa_config)
    nqb = -(-maxlen // 128)
    keep = torch.zeros((c.B, c.Hq, nqb, nqb), dtype=torch.uint8, device="cuda")
    ea.ea_xa_prefill_plan(q, k, modes, cu, maxlen, ws, keep=keep, **xg)
    torch.cuda.synchronize()
    keep_np = keep.cpu().numpy()
    del keep
    ef = metrics.xa_effective_flops(cm, keep_np, c.lengths, c.Hq, c.Hkv, c.d, n_sink=c.n_sink,
                                    keep_fraction=c.keep_fraction)
    sel_flops = metrics.xa_selection_flops(cm, c.lengths, c.Hq, c.Hkv, c.d)
    xa_rows = [(b, hq) for b in range(c.B) for hq in range(c.Hq) if cm[b, hq // (c.Hq // c.Hkv)] == 2]
    tri = sum((-(-int(c.lengths[b]) // 128)) * (-(-int(c.lengths[b]) // 128) + 1) // 2 for b, _ in xa_rows)
    density = float(sum(int(np.tril(keep_np[b, hq]).sum()) for b, hq in xa_rows)) / max(1, tri)
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    evs = [[E() for _ in range(4)] for _ in range(args.steps)]
    start, stop = E(), E()
    torch.cuda.synchronize()
    start.record()
    for s_ in range(args.steps):
        step(evs[s_])
    stop.record()
    torch.cuda.synchronize()
    step_ms = start.elapsed_time(stop) / args.steps
    seg = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3])]
                    for e in evs])
    route_ms, plan_ms, run_ms = seg.mean(axis=0)
    # the same inputs under full attention on every head
    fa_modes = torch.zeros_like(modes)
    wsf = torch.empty(ea.ea_hybrid_prefill_workspace_size(c.B, c.T, maxlen, c.Hq, c.Hkv, c.d, 1),
                      dtype=torch.uint8, device="cuda")
    for _ in range(2):
        ea.ea_hybrid_prefill(q, k, v, fa_modes, cu, maxlen, out=O, lse=lse, workspace=wsf,
                             n_sink=c.n_sink, keep_fraction=c.keep_fraction)
    torch.cuda.synchronize()
    a_, b_ = E(), E()
    a_.record()
    n_fa = max(2, args.steps // 4)
    for _ in range(n_fa):
        ea.ea_hybrid_prefill(q, k, v, fa_modes, cu, maxlen, out=O, lse=lse, workspace=wsf,
                             n_sink=c.n_sink, keep_fraction=c.keep_fraction)
    b_.record()
    torch.cuda.synchronize()
    fa_ms = a_.elapsed_time(b_) / n_fa
    log(f"xa {name} {args.xa_config}: step {step_ms:.3f} ms (route {route_ms:.3f}, selection + "
        f"list {plan_ms:.3f}, attention {run_ms:.3f}); kept density {density:.3f}; all-FA "
        f"{fa_ms:.3f} ms -> {fa_ms / step_ms:.2f}x")
    probe = mfma_probe()
    peak = metrics.MI355X_BF16_DENSE_TFLOPS
    achieved = ef / (run_ms * 1e-3) / 1e12
    out = {
        "metric": "hybrid prefill with XAttention heads at 128K: effective TFLOP/s on the computed "
                  "blocks, ms/layer, speedup over full attention",
        "value": round(ef / (step_ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{name}:{args.xa_config}" + ("" if hitters is None else ":hitters"),
                   "seq_len": maxlen, "Hq": c.Hq, "Hkv": c.Hkv, "d": c.d,
                   "xa_threshold": args.xa_tau, "xa_block": 128, "xa_stride": 8,
                   "hitters": None if hitters is None else {"block_fraction": hitters[0],
                                                            "strength": hitters[1]},
                   "xa_kv_heads": int((cm == 2).sum()), "sa_kv_heads": int((cm == 1).sum()),
                   "kept_block_density": round(density, 4), "effective_flops": int(ef),
                   "route_ms": round(float(route_ms), 4),
                   "xa_selection_and_list_ms": round(float(plan_ms), 4),
                   "xa_selection_flops": int(sel_flops),
                   "xa_selection_tflops": round(sel_flops / (plan_ms * 1e-3) / 1e12, 3),
                   "attention_ms": round(float(run_ms), 4),
                   "all_fa_prefill_ms": round(fa_ms, 4),
                   "speedup_over_full_attention": round(fa_ms / step_ms, 3)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None,
                     "kernel": "ea::attention_kernel_bf16<128, true>",
                     "avg_launch_ms": round(float(run_ms), 4), "flops_per_launch": float(ef),
                     "mfma_loop_tflops": probe["tflops"],
                     "frac_of_mfma_loop": round(achieved / probe["tflops"], 4)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_xa(c, cm, args.cpu_budget)
    print(json.dumps(out), flush=True)


def calibrate(mib):
    """One elementwise kernel of known traffic (reads and writes mib MiB), so
    that profiler byte counters can be scaled to bytes."""
    import torch
    n = mib * 2**20 // 4
    src = torch.ones(n, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    log(f"calibration: {CALIB_KERNEL} over {n * 4} bytes in, {n * 4} bytes out")
    del src, dst


def summarize_counters(pmc_dirs, calib_mib, layers_flops, out_path):
    """Turn rocprofv3 --pmc CSV output (one directory per counter) into the
    stored traffic summary: mean KiB per attention dispatch per counter, scaled
    by expected / measured KiB of the calibration kernel."""
    import csv
    res = {}
    for d in pmc_dirs:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        rows = []
        for fn in files:
            with open(fn) as f:
                rows += list(csv.DictReader(f))
        for counter in {r["Counter_Name"] for r in rows}:
            att = [float(r["Counter_Value"]) for r in rows
                   if r["Counter_Name"] == counter and ATTN_KERNEL in r["Kernel_Name"]]
            cal = [float(r["Counter_Value"]) for r in rows
                   if r["Counter_Name"] == counter and CALIB_KERNEL in r["Kernel_Name"]]
            if not att or not cal:
                raise SystemExit(f"{counter}: attention {len(att)} / calibration {len(cal)} rows")
            factor = calib_mib * 1024.0 / (sum(cal) / len(cal))
            res[counter] = {"attention_kib_per_dispatch": sum(att) / len(att),
                            "dispatches": len(att), "calibration_kib": sum(cal) / len(cal),
                            "expected_calibration_kib": calib_mib * 1024.0, "scale": factor,
                            "bytes_per_dispatch": sum(att) / len(att) * 1024.0 * factor}
    total = sum(v["bytes_per_dispatch"] for v in res.values())
    out = {"kernel": ATTN_KERNEL, "kernel_source_sha256_16": kernel_source_hash(),
           "counters": res, "hbm_bytes_per_launch": total, "layers": layers_flops}
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def summarize_sq(pmc_dirs, layers, out_path):
    """Turn rocprofv3 --pmc CSV output holding SQ_VALU_MFMA_BUSY_CYCLES and
    GRBM_GUI_ACTIVE (any further counters are kept too) into the stored
    matrix-pipe summary: means per attention dispatch and the busy share of
    SIMD-cycles."""
    import csv
    means = {}
    for d in pmc_dirs:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        rows = []
        for fn in files:
            with open(fn) as f:
                rows += list(csv.DictReader(f))
        for counter in {r["Counter_Name"] for r in rows}:
            att = [float(r["Counter_Value"]) for r in rows
                   if r["Counter_Name"] == counter and ATTN_KERNEL in r["Kernel_Name"]]
            if att:
                means[counter] = {"per_dispatch": sum(att) / len(att), "dispatches": len(att)}
    need = ["SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"]
    if any(n not in means for n in need):
        raise SystemExit(f"need counters {need}; found {sorted(means)}")
    simd_cycles = means["GRBM_GUI_ACTIVE"]["per_dispatch"] / N_XCD * N_SIMD
    busy = means["SQ_VALU_MFMA_BUSY_CYCLES"]["per_dispatch"] / simd_cycles
    out = {"kernel": ATTN_KERNEL, "kernel_source_sha256_16": kernel_source_hash(),
           "counters": means, "simd_cycles_per_dispatch": simd_cycles,
           "mfma_busy": busy, "layers": layers}
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--runs", default=",".join(DEFAULT_RUNS),
                    help="comma-separated workload names; one step runs each once")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--dual", action="store_true",
                    help="measure the dual-mode (training) forward of the first --runs workload "
                         "instead (default qwen4b_s128k_sa6)")
    ap.add_argument("--tau", type=float, default=1.0, help="Gumbel-Softmax temperature (--dual)")
    ap.add_argument("--backward", action="store_true",
                    help="measure the hybrid-layer backward of each --runs workload instead")
    ap.add_argument("--decode", action="store_true",
                    help="measure decode steps over a mode-aware KV cache holding each --runs "
                         "workload as the prompt instead (default qwen4b_s128k_sa2,sa6 and "
                         "varlen8)")
    ap.add_argument("--xa", action="store_true",
                    help="measure the prefill with XAttention heads of the first --runs workload "
                         "instead (default qwen4b_s128k_sa2)")
    ap.add_argument("--xa-config", default="XA-SSA", choices=["XA-SSA", "FA-XA", "FA-SSA"])
    ap.add_argument("--xa-tau", type=float, default=0.9, help="XAttention threshold (--xa)")
    ap.add_argument("--xa-plain", action="store_true",
                    help="--xa on the workload's plain inputs (no heavy-hitter key blocks)")
    ap.add_argument("--calibrate-mib", type=int, default=0,
                    help="first run one elementwise kernel that reads and writes this many MiB "
                         "(for scaling profiler byte counters)")
    ap.add_argument("--summarize-counters", nargs="+", default=None, metavar="PMC_DIR",
                    help="no GPU work: turn rocprofv3 --pmc output directories of a run made with "
                         "--calibrate-mib into profiles/attention_traffic.json")
    ap.add_argument("--summarize-sq", nargs="+", default=None, metavar="PMC_DIR",
                    help="no GPU work: turn rocprofv3 --pmc output directories holding "
                         "SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE into "
                         "profiles/attention_sq_counters.json")
    args = ap.parse_args()
    if args.summarize_sq:
        summarize_sq(args.summarize_sq, args.runs, SQ_JSON)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.calibrate_mib or 1024, args.runs,
                           TRAFFIC_JSON)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the hybrid prefill "
              "runs and is measured on a single GPU's share of the work", file=sys.stderr)
        sys.exit(2)
    import torch

    import full_attention_long_amd as ea
    from full_attention_long_amd import metrics
    ea.lib()
    torch.cuda.set_device(0)
    if args.calibrate_mib:
        calibrate(args.calibrate_mib)
    if args.backward:
        bench_backward(args)
        return
    if args.decode:
        if args.runs == ",".join(DEFAULT_RUNS):
            args.runs = "qwen4b_s128k_sa2,qwen4b_s128k_sa6,varlen8"
        bench_decode(args)
        return
    if args.xa:
        if args.runs == ",".join(DEFAULT_RUNS):
            args.runs = "qwen4b_s128k_sa2"
        bench_xa(args)
        return
    if args.dual:
        if args.runs == ",".join(DEFAULT_RUNS):
            args.runs = "qwen4b_s128k_sa6"
        bench_dual(args)
        return
    layers = [Layer(n) for n in args.runs.split(",")]

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        for ly in layers:
            ly.step()
    torch.cuda.synchronize()
    efs = []
    for ly in layers:
        m = ly.modes.cpu().numpy()
        c = ly.case
        assert np.array_equal(m, c.target_modes), f"{ly.name}: routing differs from the target"
        efs.append(metrics.effective_flops(m, c.lengths, c.Hq, c.Hkv, c.d, n_sink=c.n_sink,
                                           keep_fraction=c.keep_fraction))

    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    evs = [[[E() for _ in range(4)] for _ in layers] for _ in range(args.steps)]
    start, stop = E(), E()
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for s in range(args.steps):
        for li, ly in enumerate(layers):
            ly.step(evs[s][li])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = start.elapsed_time(stop) / args.steps

    runs = []
    for li, ly in enumerate(layers):
        c = ly.case
        seg = np.array([[evs[s][li][k].elapsed_time(evs[s][li][k + 1]) for k in range(3)]
                        for s in range(args.steps)])
        route_ms, plan_ms, attn_ms = seg.mean(axis=0)
        attn_med = float(np.median(seg[:, 2]))
        layer_ms = float(seg.sum(axis=1).mean())
        m = ly.modes.cpu().numpy()
        runs.append({
            "workload": ly.name, "seq_len": ly.maxlen, "tokens": int(c.T), "Hq": c.Hq,
            "Hkv": c.Hkv, "d": c.d, "sa_kv_heads": int(m.sum()), "msr": metrics.msr(m),
            "n_sink": c.n_sink, "keep_fraction": c.keep_fraction,
            "effective_flops": int(efs[li]), "ms_per_layer": round(layer_ms, 4),
            "route_ms": round(float(route_ms), 4), "plan_ms": round(float(plan_ms), 4),
            "attention_ms": round(float(attn_ms), 4),
            "attention_ms_median": round(attn_med, 4),
            "effective_tflops": round(efs[li] / (layer_ms * 1e-3) / 1e12, 3),
            "attention_tflops": round(efs[li] / (attn_ms * 1e-3) / 1e12, 3),
            "seed": c.seed,
        })
        log(f"{ly.name}: layer {layer_ms:.3f} ms (route {route_ms:.3f}, plan {plan_ms:.3f}, "
            f"attention {attn_ms:.3f}) -> {runs[-1]['effective_tflops']:.1f} TFLOP/s")
    log("matrix-core ceiling probe")
    probe = mfma_probe()
    log(f"probe: {probe['tflops']:.1f} TFLOP/s ({probe['ms']:.1f} ms per launch)")
    tot_ef = float(sum(efs))
    value = tot_ef / (step_ms * 1e-3) / 1e12
    attn_sum = sum(r["attention_ms"] for r in runs)
    achieved = tot_ef / (attn_sum * 1e-3) / 1e12
    peak = metrics.MI355X_BF16_DENSE_TFLOPS
    tr = stored_traffic()
    traffic = None
    if tr is not None:
        traffic = round(float(tr["hbm_bytes_per_launch"]), 0)
    sq = stored_sq()
    mfma_busy = round(float(sq["mfma_busy"]), 4) if sq is not None else None
    log(f"step {step_ms:.3f} ms (wall {wall / args.steps * 1e3:.3f} ms), {value:.1f} TFLOP/s; "
        f"attention {achieved:.1f} TFLOP/s = {100 * achieved / peak:.1f}% of peak")
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "+".join(ly.name for ly in layers),
            "layers_per_step": len(layers),
            "ms_per_layer": round(step_ms / len(layers), 4),
            "pct_bf16_roofline": round(100 * value / peak, 2),
            "runs": runs,
        },
        "roofline": {
            "bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": traffic, "mfma_busy": mfma_busy,
            "kernel": "ea::attention_kernel_bf16<128, false>",
            "avg_launch_ms": round(attn_sum / len(runs), 4),
            "flops_per_launch": round(tot_ef / len(runs), 0),
            "traffic_gbps": (round(traffic / (attn_sum / len(runs) * 1e-3) / 1e9, 1)
                             if traffic is not None else None),
            "mfma_loop_tflops": probe["tflops"],
            "frac_of_mfma_loop": round(achieved / probe["tflops"], 4),
        },
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline([ly.case for ly in layers], args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
