"""Build the HIP library in-tree with hipcc for gfx950.

    python -m bit_quantized_matmul_q4_amd.build          # libq4.so (+ the test probe library)

Outputs, next to this file:
  libq4.so       the C-ABI product library (include/q4.h)
  libq4probe.so  MFMA / conversion probe kernels used only by the GPU tests
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libq4.so")
PROBE_LIB = os.path.join(HERE, "libq4probe.so")
ARCH = os.environ.get("Q4_OFFLOAD_ARCH", "gfx950")

# No fast-math, no FMA contraction (the reduction order uses explicit fmaf),
# and no packed fp32 instructions.  Matrix-core results go to ordinary vector
# registers (the accumulator-register form costs a read-back per element).
# No sinking of common code out of branches: it merges the tree stack's
# per-level writes into one store with a computed address, which moves the
# whole stack to scratch memory.
COMMON_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-mllvm", "-simplifycfg-sink-common=false",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _compile(sources, out, extra=()):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *COMMON_FLAGS, *extra, "-x", "hip", *sources, "-o", tmp]
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the gfx950 feature flag; that warning is harmless
    noise = "is not a recognized feature for this target"
    lines = [ln for ln in proc.stdout.splitlines() if noise not in ln]
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (proc.returncode, "\n".join(lines)))
    if lines:
        sys.stderr.write("\n".join(lines) + "\n")
    os.replace(tmp, out)
    return out


def build_library() -> str:
    return _compile([os.path.join(CSRC, "q4_kernels.hip"), os.path.join(CSRC, "q4_api.cpp")], LIB)


def build_probe() -> str:
    return _compile([os.path.join(CSRC, "q4_probe.hip")], PROBE_LIB)


def build_all() -> None:
    build_library()
    build_probe()


if __name__ == "__main__":
    build_all()
    print(LIB)
    print(PROBE_LIB)
