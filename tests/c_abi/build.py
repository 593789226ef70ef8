"""Build tests/c_abi/rr_abi_example: a plain C11 program that drives the relay
library through include/rr.h (no Python, no torch) and checks it against the
oracle's C library.  gcc links it against librr.so, liboracle.so and the HIP
runtime, with run paths relative to the binary so the tree can move."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "rr_abi_example.c")
EXE = os.path.join(HERE, "rr_abi_example")
LIBRR = os.path.join(ROOT, "pack_rr_helper_amd", "librr.so")
LIBORC = os.path.join(ROOT, "oracle", "liboracle.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(out=EXE):
    for lib in (LIBRR, LIBORC):
        if not os.path.exists(lib):
            raise RuntimeError(f"{lib} is missing: build the libraries first")
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           SRC, "-o", out + ".tmp", LIBRR, LIBORC, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-Wl,-rpath,$ORIGIN/../../pack_rr_helper_amd", "-Wl,-rpath,$ORIGIN/../../oracle"]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"gcc failed ({proc.returncode}):\n{proc.stdout}{proc.stderr}")
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build())
