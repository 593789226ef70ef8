"""Host-side tests of the C ABI (no GPU): the library loads and exports every
symbol include/rr.h declares, its geometry agrees with the oracle's
independently written geometry, and every validation path returns its error
before any HIP call.  Pointers here are fake addresses that are never
dereferenced: each call is rejected (or is a documented no-op) before a kernel
could be enqueued."""
import ctypes
import os
import re

import pytest
import torch

import pack_rr_helper_amd as rr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rr.h")
AR, RS, A2A = 0, 1, 2
F32, BF16 = 0, 1
SUM, AVG = 0, 1
OK, EINVAL, EALIAS = 0, 1, 2


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(rr.library_path):
        from pack_rr_helper_amd import build
        build.build()
    return rr.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rr_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert {"rr_helper_reduce", "rr_active_add_scale", "rr_rs_multi_reduce", "rr_a2a_pack",
            "rr_a2a_unpack", "rr_geometry", "rr_last_error", "rr_abi_version"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert L.rr_abi_version() == 1


def relay(A, H, nc=0, pm=500, count=0):
    return ctypes.byref(rr._Relay(A, H, nc, pm, count))


def ptrs(*addrs):
    return (ctypes.c_void_p * len(addrs))(*addrs)


def err(L):
    return L.rr_last_error().decode()


# --------------------------------------------------------------------------
# geometry: two independent implementations agree
# --------------------------------------------------------------------------

GEOM_CASES = [(A, H, nc, pm, count, coll, dt)
              for (A, H, nc, pm) in [(2, 6, 8, 0), (2, 6, 9, 0), (2, 2, 4, 0), (4, 4, 5, 500),
                                     (4, 4, 6, 780), (4, 4, 5, 250), (4, 2, 3, 1000)]
              for count in [0, 5, 1023, 1024, 7 * 128 * 1000, 2 ** 20 - 1, 2 ** 20, 2 ** 25 + 3,
                            2 ** 27, 12002982488]
              for coll in (AR, RS, A2A) for dt in (F32, BF16)]


def test_geometry_agrees_with_the_oracle(L, orc):
    checked = 0
    for (A, H, nc, pm, count, coll, dt) in GEOM_CASES:
        ref = orc.geometry(A, H, nc, pm, count, coll, dt)
        try:
            got = rr.rr_geometry(rr.Relay(A, H, nc, pm, count), coll, dt)
        except rr.RRError as e:
            assert ref is None, (A, H, nc, pm, count, coll, dt, str(e))
            continue
        assert ref is not None, (A, H, nc, pm, count, coll, dt)
        assert got == ref, (A, H, nc, pm, count, coll, dt)
        checked += 1
    assert checked > 300


def test_passthrough_size_matches_the_oracle(L, orc):
    for t in (0, 1, 895999, 896000, 12002982488, 2 ** 40 + 17):
        for A, nc in ((2, 7), (4, 5), (2, 8), (8, 2)):
            assert rr.rr_passthrough_helper_size(t, A, nc) == orc.passthrough_helper_size(t, A, nc)
    assert L.rr_passthrough_helper_size(-1, 2, 7) == -1
    # near the int64 limit the size is still exact (no overflowing product)
    big = 2 ** 63 - 1
    for A, nc in ((2, 7), (8, 2), (2 ** 31 - 1, 1), (4, 5)):
        per_slot = (big // nc) // 128 * 128
        assert L.rr_passthrough_helper_size(big, A, nc) == min(big, A * per_slot)


@pytest.mark.parametrize("A,H,nc,pm,count,coll,dt", [
    (3, 5, 8, 0, 4096, AR, BF16), (2, 0, 8, 0, 4096, AR, BF16), (2, 6, 7, 0, 4096, AR, BF16),
    (4, 4, 4, 0, 4096, A2A, BF16), (4, 4, 0, 0, 4096, AR, BF16), (4, 4, 0, 1001, 4096, RS, BF16),
    (2, 6, 8, 0, -1, AR, BF16), (2, 6, 8, 0, 4096, 3, BF16), (2, 6, 8, 0, 4096, AR, 2),
    (4, 4, 0, 600, 2 ** 22, RS, BF16),
    (2, 6, 8, 0, 2 ** 48 + 1, AR, BF16), (4, 4, 0, 1000, 2 ** 62, AR, F32),
    (4, 4, 5, 0, 2 ** 63 - 1, A2A, F32),
])
def test_geometry_rejections(L, A, H, nc, pm, count, coll, dt):
    g = rr._Geom()
    assert L.rr_geometry(relay(A, H, nc, pm, count), coll, dt, ctypes.byref(g)) == EINVAL
    assert err(L)


# --------------------------------------------------------------------------
# validation of the compute entry points (no HIP call is reached)
# --------------------------------------------------------------------------

B = 1 << 40        # a fake, 256-byte aligned "device" address, never dereferenced
MB = 1 << 20


def test_helper_reduce_rejections(L):
    r2 = relay(2, 6, 8, 0, 8 * MB)
    s = ptrs(B, B + 16 * MB)
    assert L.rr_helper_reduce(r2, RS, BF16, SUM, 0, s, 2, B + 64 * MB, None) == EINVAL
    assert "passthrough" in err(L)
    assert L.rr_helper_reduce(relay(4, 4, 0, 500, 8 * MB), RS, BF16, SUM, 0, ptrs(B, B, B, B), 4,
                              B, None) == EINVAL
    assert L.rr_helper_reduce(r2, A2A, BF16, SUM, 0, s, 2, B + 64 * MB, None) == EINVAL
    assert L.rr_helper_reduce(r2, AR, BF16, 2, 0, s, 2, B + 64 * MB, None) == EINVAL      # op
    assert L.rr_helper_reduce(r2, AR, BF16, SUM, 6, s, 2, B + 64 * MB, None) == EINVAL    # helper
    assert L.rr_helper_reduce(r2, AR, BF16, SUM, 0, s, 3, B + 64 * MB, None) == EINVAL    # nSlots
    assert L.rr_helper_reduce(r2, AR, BF16, SUM, 0, ptrs(B, 0), 2, B + 64 * MB, None) == EINVAL
    assert L.rr_helper_reduce(r2, AR, BF16, SUM, 0, s, 2, None, None) == EINVAL
    assert L.rr_helper_reduce(r2, AR, BF16, SUM, 0, ptrs(B + 1, B + 16 * MB), 2, B + 64 * MB,
                              None) == EINVAL                                            # misaligned
    assert L.rr_helper_reduce(r2, AR, F32, SUM, 0, ptrs(B + 2, B + 16 * MB), 2, B + 64 * MB,
                              None) == EINVAL
    # partial overlap of the output with a slot
    assert L.rr_helper_reduce(r2, AR, BF16, SUM, 0, s, 2, B + 2, None) == EALIAS


def test_zero_chunk_helper_is_a_no_op(L):
    # count below numChunks*128: pure direct, the helper returns before any launch
    assert L.rr_helper_reduce(relay(2, 6, 8, 0, 1000), AR, BF16, AVG, 3, ptrs(B, B), 2, B,
                              None) == OK
    assert L.rr_helper_reduce(relay(4, 4, 0, 500, 1000), AR, BF16, AVG, 0, ptrs(B, B, B, B), 4,
                              B, None) == OK                       # under the 2 MiB floor
    assert L.rr_rs_multi_reduce(relay(4, 4, 0, 500, 1000), BF16, SUM, 1, 0, ptrs(B), 1, B,
                                None) == OK
    r = relay(4, 4, 5, 0, 600)
    assert L.rr_a2a_pack(r, BF16, 0, ptrs(B, B, B, B), ptrs(B, B, B, B), None) == OK
    assert L.rr_a2a_unpack(r, BF16, 0, ptrs(B, B, B, B), ptrs(B, B, B, B), None) == OK


def test_active_add_scale_rejections(L):
    r2 = relay(2, 6, 8, 0, 8 * MB)
    ins = ptrs(B, B + 64 * MB)
    assert L.rr_active_add_scale(r2, A2A, BF16, SUM, 0, ins, 2, B + 128 * MB, None) == EINVAL
    assert L.rr_active_add_scale(relay(4, 4, 0, 500, 8 * MB), RS, BF16, SUM, 0,
                                 ptrs(B, B, B, B), 4, B, None) == EINVAL
    assert "rr_rs_multi_reduce" in err(L)
    assert L.rr_active_add_scale(r2, AR, BF16, SUM, 2, ins, 2, B + 128 * MB, None) == EINVAL
    assert L.rr_active_add_scale(r2, AR, BF16, SUM, 0, ins, 3, B + 128 * MB, None) == EINVAL
    # output overlapping the other input by a partial range
    assert L.rr_active_add_scale(r2, AR, BF16, SUM, 0, ins, 2, B + 64 * MB + 256, None) == EALIAS


def test_rs_multi_reduce_rejections(L):
    r4 = relay(4, 4, 0, 500, 4 * MB)
    assert L.rr_rs_multi_reduce(relay(2, 6, 8, 0, 4 * MB), BF16, SUM, 1, 0, ptrs(B), 1, B,
                                None) == EINVAL
    assert L.rr_rs_multi_reduce(r4, BF16, SUM, 3, 0, ptrs(B), 1, B, None) == EINVAL
    assert L.rr_rs_multi_reduce(r4, BF16, SUM, 1, 4, ptrs(B), 1, B, None) == EINVAL
    assert L.rr_rs_multi_reduce(r4, BF16, SUM, 1, 0, ptrs(B), 2, B, None) == EINVAL
    # pass 1 output inside the 12 input chunks
    assert L.rr_rs_multi_reduce(r4, BF16, SUM, 1, 0, ptrs(B), 1, B + 1024, None) == EALIAS
    assert L.rr_rs_multi_reduce(r4, BF16, SUM, 2, 4, ptrs(*[B] * 8), 8, B, None) == EINVAL
    assert L.rr_rs_multi_reduce(r4, BF16, SUM, 2, 0, ptrs(*[B] * 7), 7, B, None) == EINVAL
    # pass 2 output partially overlapping a helper's reduced chunk
    blocks = [B + i * 16 * MB for i in range(4)]
    reds = [B + 64 * MB + i * MB for i in range(4)]
    assert L.rr_rs_multi_reduce(r4, BF16, SUM, 2, 0, ptrs(*blocks, *reds), 8, B + 64 * MB + 512,
                                None) == EALIAS


def test_a2a_rejections(L):
    r = relay(4, 4, 5, 0, 1 * MB)
    src = ptrs(*[B + i * 8 * MB for i in range(4)])
    dst = ptrs(*[B + 64 * MB + i * 2 * MB for i in range(4)])
    assert L.rr_a2a_pack(r, BF16, 4, src, dst, None) == EINVAL                      # helper
    assert L.rr_a2a_pack(relay(4, 4, 4, 0, MB), BF16, 0, src, dst, None) == EINVAL  # numChunks
    # in-place (a dst inside a source) is forbidden: an all-to-all never writes into its own inputs
    assert L.rr_a2a_pack(r, BF16, 0, src, ptrs(B, B + 66 * MB, B + 68 * MB, B + 70 * MB),
                         None) == EALIAS
    assert L.rr_a2a_pack(r, BF16, 0, src, ptrs(B + 64 * MB, B + 64 * MB, B + 68 * MB, B + 70 * MB),
                         None) == EALIAS
    assert L.rr_a2a_unpack(r, BF16, 0, dst, ptrs(*[B + 64 * MB + i * 8 * MB for i in range(4)]),
                           None) == EALIAS
    assert L.rr_a2a_unpack(r, BF16, 0, dst, ptrs(B, B, B + 16 * MB, B + 24 * MB), None) == EALIAS


def test_binding_refuses_host_tensors_before_the_abi(L):
    x = torch.zeros(4096, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device memory"):
        rr.rr_helper_reduce(rr.Relay(2, 6, 8, 0, 4096), AR, BF16, SUM, 0, [x, x], x)
    with pytest.raises(ValueError):
        rr.rr_geometry(rr.Relay(3, 5, 8, 0, 4096), AR, BF16)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(rr, "_lib", None)
    monkeypatch.setattr(rr, "library_path", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        rr.load()


def test_error_messages_are_per_thread(L):
    """rr_last_error() is thread-local: threads failing at the same time with
    different arguments each read back the message of their own call."""
    import threading
    bad = {t: relay(3 + 2 * t, 5, 8, 0, 4096) for t in range(8)}   # A = 3, 5, 7, ... all rejected
    got, start = {}, threading.Barrier(8)

    def work(t):
        start.wait()
        for _ in range(200):
            g = rr._Geom()
            assert L.rr_geometry(bad[t], 0, 1, ctypes.byref(g)) == EINVAL
            msg = L.rr_last_error().decode()
            if f"A={3 + 2 * t}:" not in msg:
                got[t] = msg
                return
        got[t] = "ok"

    threads = [threading.Thread(target=work, args=(t,)) for t in range(8)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert all(v == "ok" for v in got.values()), got
    assert len(got) == 8
