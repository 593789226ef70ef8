"""Build the gfx950 C-ABI library pack_rr_helper_amd/librr.so with hipcc.

The library links only the HIP runtime: no torch, no Python.  Device code is
compiled for gfx950 with FMA contraction off (the reductions add and then
scale, each rounded once, in a fixed order), fp32 denormals kept, packed fp32
instructions disabled, and scalar kernel arguments preloaded into registers.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "librr.so")
SOURCES = [os.path.join(CSRC, "rr_kernels.hip"), os.path.join(CSRC, "rr_api.cpp")]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # scalar kernel arguments (the single-segment reduction's pointers, length
    # and scale) arrive preloaded in SGPRs instead of through scalar loads
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def build(out=LIB, defines=()):
    """Compile every source into one shared library at ``out``."""
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *[f"-D{d}" for d in defines], "-o", tmp, *SOURCES]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError(f"hipcc failed ({proc.returncode}): {' '.join(cmd)}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
