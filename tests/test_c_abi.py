"""The library used from plain C: tests/c_abi/rr_abi_example.c includes only
include/rr.h and the HIP runtime header, allocates with hipMalloc and checks
the results against the oracle's C library (see that file)."""
import importlib.util
import os
import subprocess

import pytest

_spec = importlib.util.spec_from_file_location(
    "rr_c_abi_build", os.path.join(os.path.dirname(__file__), "c_abi", "build.py"))
c_abi_build = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(c_abi_build)


@pytest.fixture(scope="module")
def example():
    exe = c_abi_build.EXE
    newest_input = max(os.path.getmtime(p) for p in
                       (c_abi_build.SRC, c_abi_build.LIBRR, c_abi_build.LIBORC))
    if not os.path.exists(exe) or os.path.getmtime(exe) < newest_input:
        c_abi_build.build()
    return exe


def run(exe, mode, timeout):
    print(f"[c-abi] {mode}", flush=True)
    proc = subprocess.run([exe, mode], capture_output=True, text=True, timeout=timeout)
    return proc.returncode, proc.stdout + proc.stderr


def test_c_program_host_checks(example):
    rc, out = run(example, "host", 60)
    assert rc == 0, out
    assert "host checks passed" in out


@pytest.mark.gpu
def test_c_program_gpu_parity(example):
    rc, out = run(example, "gpu", 120)
    assert rc == 0, out
    for what in ("A=2 allreduce helpers", "A=4 reduce-scatter pass 1", "all-to-all pack + unpack",
                 "one recorded plan"):
        assert what in out and "bit-exact" in out, out
    assert "gpu checks passed" in out
