"""Build libea.so (gfx950) in-tree with hipcc.

Usage: python -m full_attention_long_amd.build [-v]
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libea.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["ea_api.hip", "ea_route.hip", "ea_worklist.hip", "ea_attention.hip", "ea_dual.hip", "ea_decode.hip", "ea_backward.hip", "ea_probe.hip", "ea_xa.hip"]
# The attention kernels never rely on NaN semantics (masked scores are set to
# -inf by selects on integer conditions); without NaN handling a row max is
# one v_max3 per two scores instead of a canonicalize + max per score.
EXTRA = {"ea_attention.hip": ["-fno-honor-nans"]}
ARCH = "gfx950"


def hipcc() -> str:
    for c in [os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"]:
        if c and os.path.exists(c):
            return c
    return "hipcc"


def flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
        # keep packed fp32 (v_pk_*_f32) out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
    ]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout or "") + (r.stderr or "")
    # hipcc's host pass does not know the packed-fp32 feature; that warning is expected
    out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out:
        print(out, flush=True)


def build(verbose: bool = False) -> str:
    """Compile every source and link libea.so; always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([cc, *flags(), *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(min(len(cmds), 8)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv[1:]))
