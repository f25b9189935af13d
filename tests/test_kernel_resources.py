"""Every kernel of the library keeps its state in registers and LDS: compiled for gfx950, no kernel
has a private (scratch) segment or spills vector registers.  A register array indexed by a lane-varying
value, or too many live values, sends the kernel's state to scratch memory, which multiplies the
memory traffic of a bandwidth-bound kernel; this catches it on the CPU, without a GPU."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "invariant_attention_amd", "csrc")
SOURCES = sorted(f for f in os.listdir(CSRC)
                 if f.endswith(".hip") and "__global__" in open(os.path.join(CSRC, f)).read())


def _file_flags(source):
    import importlib.util
    spec = importlib.util.spec_from_file_location("ia_build", os.path.join(ROOT, "invariant_attention_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.FILE_FLAGS.get(source, [])


def _hipcc():
    cand = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return cand if os.path.exists(cand) else shutil.which("hipcc")


@pytest.mark.parametrize("source", SOURCES)
def test_no_scratch_and_no_spills(source, tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc is not available")
    out = tmp_path / (source + ".s")
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off", "-fno-fast-math",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *_file_flags(source),
           "-I", os.path.join(ROOT, "include"),
           "--cuda-device-only", "-S", "-o", str(out), os.path.join(CSRC, source)]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    assert proc.returncode == 0, proc.stderr[-2000:]
    text = out.read_text()
    n_kernels = len(re.findall(r"^\s*\.amdhsa_kernel\s", text, re.M))
    segments = [int(x) for x in re.findall(r"^\s*\.private_segment_fixed_size:\s+(\d+)", text, re.M)]
    assert n_kernels > 0 and len(segments) == n_kernels, (n_kernels, segments)
    names = re.findall(r"^\s*\.amdhsa_kernel\s+(\S+)", text, re.M)
    scratch = [n for n, line in zip(names, re.findall(r"^\s*\.amdhsa_private_segment_fixed_size\s+(\d+)", text, re.M))
               if int(line) != 0]
    assert not scratch and not any(segments), f"kernels with a private (scratch) segment: {scratch}"
    # Scalar spills go to lanes of vector registers (no memory); vector spills would go to scratch.
    spills = re.findall(r"^\s*\.vgpr_spill_count:\s+([1-9]\d*)", text, re.M)
    assert not spills, f"vector register spills in {source}: {spills}"
