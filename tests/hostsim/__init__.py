"""TEST INFRASTRUCTURE: build and load libhostsim.so, the product's C-ABI
layer (pack_rr_helper_amd/csrc/rr_api.cpp) linked with a host-memory replay
of the kernels' index arithmetic (sim_launch.cpp)."""
import ctypes
import fcntl
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIB = os.path.join(HERE, "libhostsim.so")
SOURCES = [os.path.join(HERE, "sim_launch.cpp"),
           os.path.join(ROOT, "pack_rr_helper_amd", "csrc", "rr_api.cpp")]
HEADERS = [os.path.join(ROOT, "pack_rr_helper_amd", "csrc", "rr_internal.h"),
           os.path.join(ROOT, "include", "rr.h")]


# a variant with at most 5 tiles per launch: batches and single moves or
# items longer than that continue in further launches
CAPPED_LIB = os.path.join(HERE, "libhostsim_cap5.so")
CAPPED_DEFINES = ("RR_MAX_TILES_PER_LAUNCH=5",)
# variants in which every copy call takes the long-call tiling (the library
# switches to it only for calls that move hundreds of MiB)
LONG_LIB = os.path.join(HERE, "libhostsim_long.so")
LONG_DEFINES = ("RR_COPY_LONG_BYTES=1",)
CAPPED_LONG_LIB = os.path.join(HERE, "libhostsim_cap5_long.so")


def build(lib=LIB, defines=()):
    tmp = f"{lib}.{os.getpid()}.tmp"   # private to this process: parallel test workers may build too
    subprocess.run(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__",
                    *[f"-D{d}" for d in defines],
                    "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "pack_rr_helper_amd", "csrc"),
                    "-o", tmp, *SOURCES, "-L/opt/rocm/lib", "-lamdhip64"], check=True)
    os.replace(tmp, lib)
    return lib


class Sim:
    def __init__(self, capped=False, long_copies=False):
        lib, defines = {(False, False): (LIB, ()), (True, False): (CAPPED_LIB, CAPPED_DEFINES),
                        (False, True): (LONG_LIB, LONG_DEFINES),
                        (True, True): (CAPPED_LONG_LIB, CAPPED_DEFINES + LONG_DEFINES)}[(capped, long_copies)]
        # one builder at a time; the others wait and then find the library fresh
        with open(lib + ".lock", "w") as lk:
            fcntl.flock(lk, fcntl.LOCK_EX)
            if not os.path.exists(lib) or any(os.path.getmtime(s) > os.path.getmtime(lib)
                                              for s in SOURCES + HEADERS):
                build(lib, defines)
        self.long_copies = long_copies
        self.L = ctypes.CDLL(lib)
        self.L.sim_message.restype = ctypes.c_char_p
        self.L.sim_register.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int]
        self.L.rr_last_error.restype = ctypes.c_char_p
        self.keep = []

    def reset(self):
        self.L.sim_reset()
        self.keep = []

    def buf(self, a, writable=True):
        """Register a numpy array (its whole byte range) as a buffer."""
        assert a.flags.c_contiguous
        self.L.sim_register(ctypes.c_void_p(a.ctypes.data), a.nbytes, int(writable))
        self.keep.append(a)
        return a

    def register(self, addr, nbytes, writable=True):
        """Register a raw host address range (memory the caller keeps alive)."""
        self.L.sim_register(ctypes.c_void_p(addr), nbytes, int(writable))

    def check(self):
        assert self.L.sim_violations() == 0, self.L.sim_message().decode()

    def call(self, name, *args):
        st = getattr(self.L, name)(*args)
        if st != 0:
            raise RuntimeError(f"{name} -> {st}: {self.L.rr_last_error().decode()}")
        self.check()


def ptr(a, off_elems=0):
    return ctypes.c_void_p(a.ctypes.data + off_elems * a.itemsize)


def parr(*ps):
    return (ctypes.c_void_p * len(ps))(*[p.value if isinstance(p, ctypes.c_void_p) else p for p in ps])
