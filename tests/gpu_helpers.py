"""Shared plumbing of the GPU tests: move a seeded case to the device, run the
library through its binding, and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import full_attention_long_amd as ea
from workloads.gen import Case

# O tolerances against the float64 oracle on the same (bf16- or fp32-valued) inputs
TOL = {"f32": {"max": 1e-5, "mean": 1e-6}, "bf16": {"max": 2e-2, "mean": 1e-3}}
LSE_TOL = 1e-4


def note(msg: str):
    """Print (and flush) what the next GPU step is, so a failing run names its case."""
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def dev_tensor(a: np.ndarray, dtype: str):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def to_device(c: Case):
    d = {
        "q": dev_tensor(c.q, c.dtype),
        "k": dev_tensor(c.k, c.dtype),
        "v": dev_tensor(c.v, c.dtype),
        "cu": torch.from_numpy(c.cu_seqlens.astype(np.int32)).cuda(),
        "w": {k: torch.from_numpy(np.ascontiguousarray(v, np.float32)).cuda()
              for k, v in c.weights.items()},
    }
    return d


def max_seqlen(c: Case) -> int:
    return max(1, int(c.lengths.max()) if len(c.lengths) else 1)


def gpu_route(c: Case, dv=None):
    dv = dv or to_device(c)
    modes, logits = ea.ea_route(dv["k"], dv["cu"], dv["w"], pool_len=c.pool_len)
    torch.cuda.synchronize()
    return modes.cpu().numpy(), logits.cpu().numpy()


def gpu_prefill(c: Case, modes: np.ndarray, dv=None, **kw):
    dv = dv or to_device(c)
    m = torch.from_numpy(np.ascontiguousarray(modes, np.int8)).cuda()
    O, lse = ea.ea_hybrid_prefill(dv["q"], dv["k"], dv["v"], m, dv["cu"], max_seqlen(c),
                                  n_sink=c.n_sink, window_blocks=c.window_blocks,
                                  keep_fraction=c.keep_fraction, softmax_scale=c.softmax_scale, **kw)
    torch.cuda.synchronize()
    return O, lse


def o_to_numpy(O):
    return O.float().cpu().numpy()


def compare_o(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "O"):
    err = np.abs(got.astype(np.float64) - ref)
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    tol = TOL[dtype]
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert mx <= tol["max"], f"{what}: max-abs {mx:.3e} > {tol['max']:.1e} (mean {mean:.3e})"
    assert mean <= tol["mean"], f"{what}: mean-abs {mean:.3e} > {tol['mean']:.1e}"
    return mx, mean
