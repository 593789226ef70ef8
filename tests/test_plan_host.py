"""Plans (rr_plan_bytes / rr_plan_begin / rr_plan_end / rr_plan_launch in
include/rr.h), driven through the host replay of the kernels (libhostsim.so
links the product's C-ABI layer): recorded calls validate but launch nothing,
a launched plan produces the oracle's bytes from the buffers' current
contents, and every misuse is rejected before anything runs."""
import ctypes
import threading

import numpy as np
import pytest

from pack_rr_helper_amd import _Relay
from pack_rr_helper_amd import synth
from tests.hostsim import Sim, parr, ptr

AR, RS, A2A = 0, 1, 2
BF16 = 1
SUM, AVG = 0, 1
OK, EINVAL = 0, 1


@pytest.fixture(scope="module")
def sim():
    s = Sim()
    L = s.L
    L.rr_plan_bytes.restype = ctypes.c_size_t
    L.rr_plan_bytes.argtypes = [ctypes.c_int32]
    L.rr_plan_begin.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    L.rr_plan_end.argtypes = [ctypes.POINTER(ctypes.c_int32)]
    L.rr_plan_launch.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    L.rr_plan_append.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    return s


def rel(A, H, nc=0, pm=500, count=0):
    return ctypes.byref(_Relay(A, H, nc, pm, count))


def plan_buf(sim, launches):
    n = sim.L.rr_plan_bytes(launches)
    assert n > 0
    return np.zeros((n + 7) // 8, np.uint64), n


def begin(sim, buf, n):
    return sim.L.rr_plan_begin(ctypes.c_void_p(buf.ctypes.data), n)


def end(sim):
    k = ctypes.c_int32(-1)
    return sim.L.rr_plan_end(ctypes.byref(k)), k.value


def launch(sim, buf, off=0):
    return sim.L.rr_plan_launch(ctypes.c_void_p(buf.ctypes.data + off), None)


class Group:
    """Buffers of an A=2 reduce-scatter owner, a batched A=2 allreduce
    helper call (three chunks, three groups in the fused call) and an A=4
    all-to-all pack, registered with the replay."""

    def __init__(self, sim, seed):
        self.sim = sim
        self.R = 8 * 128 * 6 + 13
        self.x = [sim.buf(synth.as_bf16_bits(synth.normal(self.R, seed, r)), writable=False) for r in range(2)]
        self.out = sim.buf(np.zeros(self.R, np.uint16))
        self.count = 8 * 128 * 10
        self.c = 128 * 10
        self.s = [sim.buf(synth.as_bf16_bits(synth.normal(self.count, seed + 1, r)), writable=False)
                  for r in range(2)]
        self.hout = [sim.buf(np.zeros(self.c, np.uint16)) for _ in range(3)]
        self.seg = 5 * 128 * 4 + 8
        self.src = [sim.buf(synth.bits16(4 * self.seg, seed + 2, r), writable=False) for r in range(4)]
        self.ac = 128 * 4
        self.dst = [sim.buf(np.zeros(3 * self.ac, np.uint16)) for _ in range(4)]

    def owner(self):
        return self.sim.L.rr_active_add_scale(rel(2, 6, 8, 0, self.R), RS, BF16, AVG, 0,
                                              parr(ptr(self.x[0]), ptr(self.x[1])), 2, ptr(self.out), None)

    def helpers(self):
        jobs = (_HelperJob * 3)()
        for h in range(3):
            jobs[h].relay, jobs[h].helper, jobs[h].nSlots = _Relay(2, 6, 8, 0, self.count), h, 2
            jobs[h].slots[0] = ptr(self.s[0], h * self.c).value
            jobs[h].slots[1] = ptr(self.s[1], h * self.c).value
            jobs[h].out = ptr(self.hout[h]).value
        return self.sim.L.rr_helper_reduce_many(AR, BF16, SUM, jobs, 3, None)

    def pack(self):
        return self.sim.L.rr_a2a_pack(rel(4, 4, 5, 0, self.seg), BF16, 2, parr(*[ptr(s) for s in self.src]),
                                      parr(*[ptr(d) for d in self.dst]), None)

    def calls(self):
        return [self.owner(), self.helpers(), self.pack()]

    def check(self, orc):
        assert np.array_equal(self.out, orc.rs2_active(BF16, AVG, self.x[0].copy(), self.x[1].copy()))
        for h in range(3):
            sl = slice(h * self.c, (h + 1) * self.c)
            assert np.array_equal(self.hout[h], orc.ar2_helper(BF16, SUM, self.s[0][sl].copy(), self.s[1][sl].copy()))
        ref = orc.a2a_pack(2, 4, self.seg, self.ac, 2, [s.copy() for s in self.src])
        for d in range(4):
            assert np.array_equal(self.dst[d].view(np.uint8), ref[d])

    def untouched(self):
        return not self.out.any() and not any(h.any() for h in self.hout) and not any(d.any() for d in self.dst)


from pack_rr_helper_amd import _HelperJob  # noqa: E402  (ctypes job layout only)


def test_recorded_calls_launch_only_when_the_plan_is_launched(sim, orc):
    sim.reset()
    g = Group(sim, 70)
    buf, n = plan_buf(sim, 8)
    assert begin(sim, buf, n) == OK
    assert g.calls() == [OK, OK, OK]
    assert sim.L.sim_launches() == 0 and g.untouched()
    st, k = end(sim)
    assert st == OK and k == 3       # one launch per call here
    assert launch(sim, buf) == OK
    assert sim.L.sim_launches() == 3
    g.check(orc)
    sim.check()
    # the plan reads the buffers' contents at launch time: new inputs, new outputs
    for x in g.x + g.s + g.src:
        x[:] = np.roll(x, 7)
    assert launch(sim, buf) == OK
    g.check(orc)
    # a byte copy of the plan is the same plan
    copy = buf.copy()
    for x in g.x:
        x[:] = np.roll(x, 3)
    assert launch(sim, copy) == OK
    g.check(orc)
    sim.check()


def test_rejected_call_records_nothing(sim):
    sim.reset()
    g = Group(sim, 71)
    buf, n = plan_buf(sim, 4)
    assert begin(sim, buf, n) == OK
    # A=3 is outside the method: rejected before anything is recorded
    st = sim.L.rr_active_add_scale(rel(3, 5, 8, 0, g.R), RS, BF16, AVG, 0, parr(ptr(g.x[0]), ptr(g.x[1])), 2,
                                   ptr(g.out), None)
    assert st == EINVAL
    assert end(sim) == (OK, 0)
    assert launch(sim, buf) == OK and sim.L.sim_launches() == 0 and g.untouched()


def test_a_full_plan_is_unusable(sim):
    sim.reset()
    g = Group(sim, 72)
    buf, n = plan_buf(sim, 2)
    assert begin(sim, buf, n) == OK
    sts = g.calls()
    assert sts[:2] == [OK, OK] and sts[2] == EINVAL
    assert b"plan buffer holds 2 launches" in sim.L.rr_last_error()
    st, k = end(sim)
    assert st == EINVAL and k == 2
    assert launch(sim, buf) == EINVAL
    assert sim.L.sim_launches() == 0 and g.untouched()


def test_plan_misuse_is_rejected(sim):
    sim.reset()
    buf, n = plan_buf(sim, 4)
    assert sim.L.rr_plan_bytes(0) == 0 and sim.L.rr_plan_bytes(4097) == 0
    assert sim.L.rr_plan_bytes(2) > sim.L.rr_plan_bytes(1)
    assert end(sim)[0] == EINVAL                                   # not recording
    assert sim.L.rr_plan_begin(None, n) == EINVAL                  # null buffer
    assert begin(sim, buf, sim.L.rr_plan_bytes(1) - 1) == EINVAL   # holds no launch
    assert sim.L.rr_plan_begin(ctypes.c_void_p(buf.ctypes.data + 4), n - 8) == EINVAL  # misaligned
    assert launch(sim, np.zeros(512, np.uint64)) == EINVAL         # not a plan
    assert launch(sim, buf, 4) == EINVAL                           # misaligned plan
    assert begin(sim, buf, n) == OK
    assert begin(sim, buf, n) == EINVAL                            # already recording
    assert launch(sim, buf) == EINVAL                              # still being recorded
    assert end(sim) == (OK, 0)
    assert launch(sim, buf) == OK                                  # an empty plan launches nothing
    assert sim.L.sim_launches() == 0


def test_recording_belongs_to_its_thread(sim, orc):
    """A call made on another thread while this one records is launched at
    once, not recorded."""
    sim.reset()
    g = Group(sim, 73)
    buf, n = plan_buf(sim, 4)
    assert begin(sim, buf, n) == OK
    out = {}
    t = threading.Thread(target=lambda: out.setdefault("st", g.calls()))
    t.start()
    t.join()
    assert out["st"] == [OK, OK, OK] and sim.L.sim_launches() == 3
    g.check(orc)
    assert end(sim) == (OK, 0)


def test_plans_append(sim, orc):
    """Plans appended into a finished plan launch all their launches in
    order; appending beyond the room, to itself, or an unfinished or broken
    plan is rejected and changes nothing."""
    sim.reset()
    g = Group(sim, 74)
    append = lambda dst, n, src: sim.L.rr_plan_append(ctypes.c_void_p(dst.ctypes.data), n,
                                                      ctypes.c_void_p(src.ctypes.data))
    a, na = plan_buf(sim, 2)
    b, nb = plan_buf(sim, 1)
    whole, nw = plan_buf(sim, 4)
    assert begin(sim, a, na) == OK and [g.owner(), g.helpers()] == [OK, OK] and end(sim) == (OK, 2)
    assert begin(sim, b, nb) == OK and g.pack() == OK and end(sim) == (OK, 1)
    assert begin(sim, whole, nw) == OK
    assert append(whole, nw, a) == EINVAL         # still being recorded
    assert end(sim) == (OK, 0)
    assert append(whole, nw, a) == OK and append(whole, nw, b) == OK
    assert append(whole, nw, whole) == EINVAL     # itself
    assert append(whole, nw, a) == EINVAL         # 3 + 2 > 4: no room, nothing changed
    assert append(whole, sim.L.rr_plan_bytes(3), b) == EINVAL  # the buffer stated holds 3
    assert sim.L.sim_launches() == 0 and g.untouched()
    assert launch(sim, whole) == OK and sim.L.sim_launches() == 3
    g.check(orc)
    sim.check()
    # a broken plan cannot be appended
    c, nc_ = plan_buf(sim, 1)
    assert begin(sim, c, nc_) == OK and g.owner() == OK and g.pack() == EINVAL and end(sim)[0] == EINVAL
    d, nd = plan_buf(sim, 4)
    assert begin(sim, d, nd) == OK and end(sim) == (OK, 0)
    assert append(d, nd, c) == EINVAL
