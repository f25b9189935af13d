"""Builds libinvattn.so (HIP for gfx950 + the host page table) in-tree with hipcc.

python -m invariant_attention_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libinvattn.so")
SOURCES = ["kv_append.hip", "decode.hip", "prefill.hip", "layer_ops.hip", "probe.hip", "capi.hip", "pool.cpp"]
HEADERS = ["arith.hpp", "pages.hpp", "launch.hpp", "errors.hpp"]

# -ffp-contract=off: no implicit FMA contraction -- the arithmetic order is the one
# written in arith.hpp.  The packed-fp32 feature is turned off for the device pass.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-fast-math",
    "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def build(verbose: bool = False) -> str:
    """Compile every source into libinvattn.so (always rebuilds)."""
    include = os.path.join(os.path.dirname(HERE), "include")
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIP_FLAGS, "-shared", "-I", include, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(line for line in proc.stderr.splitlines() if noise not in line)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    _write_build_info()
    return LIB


def _write_build_info() -> None:
    """Records the git commit the library was built from (build_info.json, beside the library), for
    runs on a copy of the tree that has no .git."""
    import json
    try:
        sha = subprocess.run(["git", "rev-parse", "--short", "HEAD"], cwd=os.path.dirname(HERE), capture_output=True,
                             text=True, timeout=10).stdout.strip() or None
    except Exception:
        sha = None
    with open(os.path.join(HERE, "build_info.json"), "w") as f:
        json.dump({"git": sha}, f)


if __name__ == "__main__":
    print(build(verbose=True))
