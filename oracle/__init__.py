"""CPU oracle for the sharded relay hot path -- TEST INFRASTRUCTURE ONLY.

Only tests/, ``__graft_entry__.smoke()`` and the CPU-baseline leg of bench.py
may import this package.  It wraps the plain C oracle (oracle.c, built by
oracle/build.py with gcc) over numpy arrays.  It shares no code with the HIP
library and never consumes anything the HIP library produced.

Array conventions: fp32 buffers are ``numpy.float32``; bf16 buffers are raw
bit patterns in ``numpy.uint16``.  dtype codes: 0 = fp32, 1 = bf16.
Op codes: 0 = SUM, 1 = AVG.  Collective codes: 0 = allreduce,
1 = reduce-scatter, 2 = all-to-all.

Every function is pinned in tests/test_oracle_*.py against something other
than itself: printed constants and closed forms from the pull request's
description, exact rational brute force (oracle/brute.py), invariants, and
library routines (torch's CPU bf16 conversion, numpy's IEEE fp32 adds).
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32, BF16 = 0, 1
SUM, AVG = 0, 1
ALLREDUCE, REDUCE_SCATTER, ALLTOALL = 0, 1, 2

_lib = None


class Geom(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "chunk", "relay_total", "direct_off", "direct_len", "dirA_off", "dirA_len",
        "dirB_off", "dirB_len", "dslice", "helper_elems")] + [
        ("pure_direct", ctypes.c_int32), ("status", ctypes.c_int32)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_ if n != "status"}


def lib():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path):
            _build.build()
        _lib = ctypes.CDLL(path)
        _setup(_lib)
    return _lib


def _setup(L):
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    pp = ctypes.POINTER(ctypes.c_void_p)
    sig = {
        "orc_bf16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
        "orc_f32_to_bf16": (ctypes.c_uint16, [ctypes.c_float]),
        "orc_passthrough_helper_size": (i64, [i64, i32, i32]),
        "orc_geometry": (ctypes.c_int, [i32, i32, i32, i32, i64, i32, i32, ctypes.POINTER(Geom)]),
        "orc_ar2_helper": (None, [ctypes.c_int, ctypes.c_int, vp, vp, i64, vp]),
        "orc_ar4_helper": (None, [ctypes.c_int, ctypes.c_int, ctypes.c_int, pp, i64, vp]),
        "orc_ar_active": (None, [ctypes.c_int] * 6 + [i64, ctypes.c_int, pp, vp]),
        "orc_rs2_active": (None, [ctypes.c_int, ctypes.c_int, vp, vp, i64, vp]),
        "orc_rs4_pass1": (None, [ctypes.c_int, ctypes.c_int, i64, vp, vp]),
        "orc_rs4_pass2": (None, [ctypes.c_int] * 5 + [i64, ctypes.c_int, pp, pp, vp]),
        "orc_a2a_pack": (None, [ctypes.c_int, ctypes.c_int, i64, i64, ctypes.c_int, pp, pp]),
        "orc_a2a_unpack": (None, [ctypes.c_int, ctypes.c_int, i64, i64, ctypes.c_int, pp, pp]),
        "orc_ar2_group": (ctypes.c_int, [ctypes.c_int] * 4 + [i64, vp, vp, vp, vp, vp]),
        "orc_rs2_group": (ctypes.c_int, [ctypes.c_int] * 4 + [i64, vp, vp, vp, vp, vp]),
        "orc_ar4_group": (ctypes.c_int, [ctypes.c_int] * 4 + [i64, pp, pp, vp]),
        "orc_rs4_group": (ctypes.c_int, [ctypes.c_int] * 4 + [i64, pp, pp, vp]),
        "orc_a2a_group": (ctypes.c_int, [ctypes.c_int] * 4 + [i64, pp, pp, vp]),
        "orc_plain_sum": (None, [ctypes.c_int] * 3 + [pp, i64, i64, vp]),
        "orc_plain_all_to_all": (None, [ctypes.c_int, ctypes.c_int, i64, ctypes.c_int, pp, vp]),
        "orc_bf16_to_f32_array": (None, [vp, vp, i64]),
        "orc_f32_to_bf16_array": (None, [vp, vp, i64]),
        "orc_abi_version": (ctypes.c_int, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args


# --------------------------------------------------------------------------
# helpers
# --------------------------------------------------------------------------

def np_dtype(dt):
    return np.float32 if dt == F32 else np.uint16


def _p(a):
    assert a.flags.c_contiguous
    return ctypes.c_void_p(a.ctypes.data)


def _pa(arrs):
    return (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])


def _check(a, dt):
    if a.dtype != np_dtype(dt):
        raise TypeError(f"expected {np_dtype(dt)} array, got {a.dtype}")
    if not a.flags.c_contiguous:
        raise ValueError("arrays must be C-contiguous")


def esize(dt):
    return 4 if dt == F32 else 2


# --------------------------------------------------------------------------
# codec and geometry
# --------------------------------------------------------------------------

def bf16_to_f32(bits):
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, np.float32)
    lib().orc_bf16_to_f32_array(_p(bits), _p(out), bits.size)
    return out


def f32_to_bf16(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_f32_to_bf16_array(_p(x), _p(out), x.size)
    return out


def passthrough_helper_size(count_g, A, num_chunks):
    return lib().orc_passthrough_helper_size(count_g, A, num_chunks)


def geometry(A, H, numChunks, permille, count, coll, dtype):
    """Returns the geometry dict, or None when the arguments are rejected."""
    g = Geom()
    rc = lib().orc_geometry(A, H, numChunks, permille, count, coll, dtype, ctypes.byref(g))
    return None if rc else g.as_dict()


# --------------------------------------------------------------------------
# steps
# --------------------------------------------------------------------------

def ar2_helper(dt, op, slot0, slot1):
    _check(slot0, dt), _check(slot1, dt)
    assert slot0.size == slot1.size
    out = np.empty_like(slot0)
    lib().orc_ar2_helper(dt, op, _p(slot0), _p(slot1), slot0.size, _p(out))
    return out


def ar4_helper(dt, op, slots):
    for s in slots:
        _check(s, dt)
        assert s.size == slots[0].size
    out = np.empty_like(slots[0])
    lib().orc_ar4_helper(dt, op, len(slots), _pa(slots), slots[0].size, _p(out))
    return out


def ar_active(dt, op, A, H, numChunks, permille, count, a, x, out):
    """Writes active a's direct-sum region of ``out`` in place."""
    for s in x:
        _check(s, dt)
        assert s.size == count
    _check(out, dt)
    lib().orc_ar_active(dt, op, A, H, numChunks, permille, count, a, _pa(x), _p(out))
    return out


def rs2_active(dt, op, blk0, blk1):
    _check(blk0, dt), _check(blk1, dt)
    out = np.empty_like(blk0)
    lib().orc_rs2_active(dt, op, _p(blk0), _p(blk1), blk0.size, _p(out))
    return out


def rs4_pass1(dt, A, chunk, scratch):
    _check(scratch, dt)
    assert scratch.size >= A * (A - 1) * chunk
    out = np.empty(A * chunk, np_dtype(dt))
    lib().orc_rs4_pass1(dt, A, chunk, _p(scratch), _p(out))
    return out


def rs4_pass2(dt, op, A, H, permille, R, o, blk, red):
    for b in blk:
        _check(b, dt)
    for r in red:
        _check(r, dt)
    out = np.empty(R, np_dtype(dt))
    lib().orc_rs4_pass2(dt, op, A, H, permille, R, o, _pa(blk), _pa(red), _p(out))
    return out


def a2a_pack(es, A, seg, chunk, h, src):
    dst = [np.empty((A - 1) * chunk * es, np.uint8) for _ in range(A)]
    src = [np.ascontiguousarray(s).view(np.uint8) for s in src]
    lib().orc_a2a_pack(es, A, seg, chunk, h, _pa(src), _pa(dst))
    return dst


def a2a_unpack(es, A, seg, chunk, h, recv, out):
    """Scatters into the byte views of ``out`` in place."""
    recv = [np.ascontiguousarray(r).view(np.uint8) for r in recv]
    outb = [o.view(np.uint8) for o in out]
    lib().orc_a2a_unpack(es, A, seg, chunk, h, _pa(recv), _pa(outb))
    return out


# --------------------------------------------------------------------------
# whole-group compositions
# --------------------------------------------------------------------------

def ar2_group(dt, op, H, numChunks, count, x0, x1):
    out0, out1 = np.empty_like(x0), np.empty_like(x1)
    scratch = np.empty(2 * max(count, 1), np_dtype(dt))
    rc = lib().orc_ar2_group(dt, op, H, numChunks, count, _p(x0), _p(x1), _p(out0), _p(out1), _p(scratch))
    if rc:
        raise ValueError("bad geometry")
    return out0, out1


def rs2_group(dt, op, H, numChunks, R, x0, x1):
    out0, out1 = np.empty(R, np_dtype(dt)), np.empty(R, np_dtype(dt))
    scratch = np.empty(4 * max(R, 1), np_dtype(dt))
    rc = lib().orc_rs2_group(dt, op, H, numChunks, R, _p(x0), _p(x1), _p(out0), _p(out1), _p(scratch))
    if rc:
        raise ValueError("bad geometry")
    return out0, out1


def ar4_group(dt, op, H, permille, count, x):
    out = [np.empty_like(a) for a in x]
    scratch = np.empty(2 * max(count, 1) + 5 * count, np_dtype(dt))
    rc = lib().orc_ar4_group(dt, op, H, permille, count, _pa(x), _pa(out), _p(scratch))
    if rc:
        raise ValueError("bad geometry")
    return out


def rs4_group(dt, op, H, permille, R, x):
    out = [np.empty(R, np_dtype(dt)) for _ in x]
    scratch = np.empty(2 * R + 4 * R + 16, np_dtype(dt))
    rc = lib().orc_rs4_group(dt, op, H, permille, R, _pa(x), _pa(out), _p(scratch))
    if rc:
        raise ValueError("bad geometry")
    return out


def a2a_group(es, A, H, numChunks, seg, src):
    srcb = [np.ascontiguousarray(s).view(np.uint8) for s in src]
    out = [np.empty(A * seg * es, np.uint8) for _ in range(A)]
    scratch = np.empty(A * (A - 1) * seg * es + 16, np.uint8)
    rc = lib().orc_a2a_group(es, A, H, numChunks, seg, _pa(srcb), _pa(out), _p(scratch))
    if rc:
        raise ValueError("bad geometry")
    return out


def plain_sum(dt, op, x, off, n):
    """RND(sum_s x_s[off:off+n] / D), D = A for AVG: the exact sum, rounded once."""
    for s in x:
        _check(s, dt)
    out = np.empty(n, np_dtype(dt))
    lib().orc_plain_sum(dt, op, len(x), _pa(x), off, n, _p(out))
    return out


def plain_all_to_all(es, A, seg, d, src):
    srcb = [np.ascontiguousarray(s).view(np.uint8) for s in src]
    out = np.empty(A * seg * es, np.uint8)
    lib().orc_plain_all_to_all(es, A, seg, d, _pa(srcb), _p(out))
    return out
