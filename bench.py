"""Throughput of the routed hybrid attention prefill on one MI355X.

One step = one layer's whole hot path on device-resident inputs: the router
(boundary pooling, task MLP, router MLP, argmax), the device work list, the
V transpose and the fused FA/SA attention forward.  The default workload is
the 128K-token Qwen3-4B-shaped layer (32 query heads, 8 KV heads, d = 128,
bf16), measured in both routing mixes it is specified with (2 of 8 and 6 of 8
KV heads sparse); `value` is the combined effective TFLOP/s of the two
layers: their effective FLOPs over their summed step times.  Effective FLOPs
count only the computed 64 x 64 FA/SA blocks.

Prints one JSON line.  --gpus must be 1 (the path runs on one GPU).
"""
from __future__ import annotations

import argparse
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


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def device_inputs(case):
    import torch
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()  # noqa: E731
    return {
        "q": dev(case.q), "k": dev(case.k), "v": dev(case.v),
        "cu": torch.from_numpy(case.cu_seqlens).cuda(),
        "w": {n: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
              for n, a in case.weights.items()},
    }


def measure(name, steps, warmup):
    import torch

    import full_attention_long_amd as ea
    from full_attention_long_amd import metrics
    from workloads import gen
    from workloads.configs import WORKLOADS

    wl = WORKLOADS[name]
    log(f"{name}: generating inputs")
    case = gen.build_case(wl)
    dv = device_inputs(case)
    T, Hq, Hkv, d = case.T, case.Hq, case.Hkv, case.d
    maxlen = int(case.lengths.max())
    O = torch.empty_like(dv["q"])
    lse = torch.empty((Hq, T), dtype=torch.float32, device="cuda")
    modes = torch.empty((case.B, Hkv), dtype=torch.int8, device="cuda")
    logits = torch.empty((case.B, Hkv, 2), dtype=torch.float32, device="cuda")
    ws = torch.empty(ea.ea_hybrid_prefill_workspace_size(case.B, T, maxlen, Hq, Hkv, d, 1),
                     dtype=torch.uint8, device="cuda")

    def step(ev=None):
        ea.ea_route(dv["k"], dv["cu"], dv["w"], pool_len=case.pool_len, modes=modes, logits=logits)
        if ev is not None:
            ev[0].record()
        ea.ea_hybrid_prefill(dv["q"], dv["k"], dv["v"], modes, dv["cu"], maxlen, n_sink=case.n_sink,
                             keep_fraction=case.keep_fraction, out=O, lse=lse, workspace=ws)
        if ev is not None:
            ev[1].record()

    log(f"{name}: warmup {warmup}")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    m = modes.cpu().numpy()
    assert np.array_equal(m, case.target_modes), "routing differs from the workload's target"
    ef = metrics.effective_flops(m, case.lengths, Hq, Hkv, d, n_sink=case.n_sink,
                                 keep_fraction=case.keep_fraction)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"{name}: timing {steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        step(evs[i])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = start.elapsed_time(stop) / steps
    prefill_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    log(f"{name}: {step_ms:.3f} ms/step, prefill call {prefill_ms:.3f} ms, wall {wall:.2f} s")
    res = {
        "workload": name, "seq_len": int(maxlen), "tokens": int(T), "Hq": Hq, "Hkv": Hkv, "d": d,
        "sa_kv_heads": int(m.sum()), "msr": metrics.msr(m), "n_sink": case.n_sink,
        "keep_fraction": case.keep_fraction, "effective_flops": int(ef),
        "ms_per_layer": step_ms, "prefill_ms": prefill_ms,
        "effective_tflops": ef / (step_ms * 1e-3) / 1e12,
        "prefill_effective_tflops": ef / (prefill_ms * 1e-3) / 1e12,
        "seed": case.seed,
    }
    res["pct_bf16_roofline"] = 100.0 * res["effective_tflops"] / metrics.MI355X_BF16_DENSE_TFLOPS
    del dv, O, lse, ws
    torch.cuda.empty_cache()
    return res, case


def cpu_baseline(case, budget_s=12.0):
    """The oracle on a bounded sample of the same layer: 64-row query blocks of
    one query head per KV head, at seeded positions, until ~budget_s of CPU time
    has been spent; effective FLOPs of the sample over its wall time."""
    from full_attention_long_amd import metrics
    from oracle import ea_oracle as orc

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    L = int(case.lengths[0])
    G = case.Hq // case.Hkv
    modes = case.target_modes
    w = metrics.window_blocks(L, case.n_sink, case.keep_fraction)
    rng = np.random.default_rng(0)
    qf, kf, vf = case.q_f32(), case.k_f32(), case.v_f32()
    done_flops, units, t_used = 0, 0, 0.0
    while t_used < budget_s and units < 256:
        g = units % case.Hkv
        hq = g * G + (units // case.Hkv) % G
        qb = int(rng.integers(0, L // 64))
        toks = np.arange(qb * 64, min(L, qb * 64 + 64))
        t0 = time.perf_counter()
        orc.hybrid_attention_rows(qf, kf, vf, modes, case.cu_seqlens, toks, [hq],
                                  n_sink=case.n_sink, keep_fraction=case.keep_fraction)
        t_used += time.perf_counter() - t0
        nvis = qb + 1 if modes[0, g] == 0 else min(qb + 1, case.n_sink + w)
        done_flops += 4 * case.d * len(toks) * 64 * nvis
        units += 1
    return {
        "value": done_flops / t_used / 1e12, "unit": "TFLOP/s", "cores": int(cores),
        "kind": "oracle",
        "sample": f"{units} query blocks of 64 rows (one query head each, seeded positions) of "
                  f"{case.name}; float64 two-pass softmax; {t_used:.1f} s; "
                  f"cpu {platform.processor() or platform.machine()}",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--runs", default=",".join(DEFAULT_RUNS),
                    help="comma-separated workload names measured together")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run one plain device-to-device copy of this many MiB (a kernel of "
                         "known traffic, to scale profiler byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the hybrid prefill "
              "runs and is measured on a single GPU's share of the work", file=sys.stderr)
        sys.exit(2)
    import torch

    import full_attention_long_amd as ea
    from full_attention_long_amd import metrics
    ea.lib()
    torch.cuda.set_device(0)
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib * 2**20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy of {n} bytes done")
        del src, dst
    runs, cases = [], []
    for name in args.runs.split(","):
        r, c = measure(name, args.steps, args.warmup)
        runs.append(r)
        cases.append(c)
    tot_ef = sum(r["effective_flops"] for r in runs)
    tot_ms = sum(r["ms_per_layer"] for r in runs)
    tot_prefill = sum(r["prefill_ms"] for r in runs)
    value = tot_ef / (tot_ms * 1e-3) / 1e12
    achieved = tot_ef / (tot_prefill * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(tot_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "+".join(r["workload"] for r in runs),
            "layers_per_step": len(runs),
            "pct_bf16_roofline": round(100 * value / metrics.MI355X_BF16_DENSE_TFLOPS, 2),
            "runs": runs,
        },
        "roofline": {
            "bound": "mfma", "achieved": round(achieved, 3),
            "peak": metrics.MI355X_BF16_DENSE_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / metrics.MI355X_BF16_DENSE_TFLOPS, 4), "traffic": None,
            "kernel": "attention_kernel<bf16, 128> (timed as the ea_hybrid_prefill call: work "
                      "list + V transpose + attention)",
        },
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(cases[-1], args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
