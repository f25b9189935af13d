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


# Per-source device flags.  The prefill kernel runs one wave per SIMD with two
# 16-row blocks per wave and holds more state than the 256 architectural VGPRs;
# with its MFMA accumulators forced to architectural VGPRs, the per-tile
# rescale and the split merge touch no accumulation registers (AGPRs), and
# the merged split state is what lives there.
FILE_FLAGS = {"prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def build(verbose: bool = False) -> str:
    """Compile every source into libinvattn.so (always rebuilds)."""
    import shutil
    import tempfile
    include = os.path.join(os.path.dirname(HERE), "include")
    tmp = LIB + ".tmp%d" % os.getpid()
    noise = "'-packed-fp32-ops' is not a recognized feature"
    objdir = tempfile.mkdtemp(prefix="invattn_build_")
    try:
        # One object per source (compiled in parallel, each with its own flags), then one link.
        procs, objs = [], []
        for src in SOURCES:
            obj = os.path.join(objdir, src + ".o")
            cmd = [hipcc(), *HIP_FLAGS, *FILE_FLAGS.get(src, []), "-I", include, "-c", "-o", obj,
                   os.path.join(CSRC, src)]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
            objs.append(obj)
        errs = []
        for src, p in procs:
            _, e = p.communicate()
            e = "\n".join(line for line in e.splitlines() if noise not in line)
            if p.returncode != 0:
                errs.append(f"{src}:\n{e}")
            elif verbose and e.strip():
                print(e, file=sys.stderr)
        if errs:
            raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
        cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
        if verbose:
            print(" ".join(cmd), flush=True)
        proc = subprocess.run(cmd, capture_output=True, text=True)
        if proc.returncode != 0:
            raise RuntimeError("hipcc link failed:\n" + proc.stderr)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
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
