"""Host-logic tests: every entry point of the C ABI, driven through
libhostsim.so on host buffers, must (a) touch only the registered buffers when
its segment tables are replayed with the kernels' index arithmetic and
(b) produce the oracle's bytes.  Covers ragged tails, zero chunks, views at
every 2-byte misalignment (realigned reductions and copies), in-place
aliases and segment tables large enough to split a call into several
launches."""
import ctypes

import numpy as np
import pytest

from pack_rr_helper_amd import synth
from pack_rr_helper_amd import _Relay
from tests.hostsim import Sim, parr, ptr

AR, RS, A2A = 0, 1, 2
F32, BF16 = 0, 1
SUM, AVG = 0, 1


@pytest.fixture(scope="module")
def sim():
    return Sim()


def rel(A, H, nc=0, pm=500, count=0):
    return ctypes.byref(_Relay(A, H, nc, pm, count))


def bits(n, seed, rank):
    return synth.as_bf16_bits(synth.normal(n, seed, rank))


def padded(a, lead):
    """a copy of a placed `lead` elements into a larger buffer (misaligned view)."""
    big = np.zeros(a.size + lead + 16, a.dtype)
    big[lead:lead + a.size] = a
    return big


@pytest.mark.parametrize("dt", [F32, BF16])
@pytest.mark.parametrize("count", [8 * 128 * 6 + 8, 2 ** 16 + 8 * 37 + 5, 900])
@pytest.mark.parametrize("lead", [0, 3])
def test_ar2_helper_and_active(sim, orc, dt, count, lead):
    sim.reset()
    A, H, nc = 2, 6, 8
    g = orc.geometry(A, H, nc, 0, count, AR, dt)
    c = g["chunk"]
    xs = [synth.uniform(count, -1, 1, 0, r) for r in range(A)]
    if dt == BF16:
        xs = [synth.as_bf16_bits(x) for x in xs]
    bx = [sim.buf(padded(x, lead), writable=False) for x in xs]
    for k in range(H):
        out = sim.buf(np.zeros(max(c, 1) + 8, xs[0].dtype))
        sim.call("rr_helper_reduce", rel(A, H, nc, 0, count), AR, dt, AVG, k,
                 parr(ptr(bx[0], lead + k * c), ptr(bx[1], lead + k * c)), 2, ptr(out, 1 if lead else 0), None)
        if c:
            ref = orc.ar2_helper(dt, AVG, xs[0][k * c:(k + 1) * c].copy(), xs[1][k * c:(k + 1) * c].copy())
            o = 1 if lead else 0
            assert np.array_equal(out[o:o + c], ref)
    for a in range(A):
        out = sim.buf(np.full(count + lead + 8, 7, xs[0].dtype))
        sim.call("rr_active_add_scale", rel(A, H, nc, 0, count), AR, dt, SUM, a,
                 parr(ptr(bx[0], lead), ptr(bx[1], lead)), 2, ptr(out, lead), None)
        ref = orc.ar_active(dt, SUM, A, H, nc, 0, count, a, xs, np.full(count, 7, xs[0].dtype))
        assert np.array_equal(out[lead:lead + count], ref)
        assert np.all(out[:lead] == 7) and np.all(out[lead + count:] == 7)


@pytest.mark.parametrize("R", [8 * 128 * 3 + 40, 100])
def test_rs2_active_in_place(sim, orc, R):
    sim.reset()
    x0, x1 = bits(2 * R, 1, 0), bits(2 * R, 1, 1)
    own = sim.buf(x0.copy())
    peer = sim.buf(x1[:R].copy(), writable=False)
    sim.call("rr_active_add_scale", rel(2, 6, 8, 0, R), RS, BF16, AVG, 0,
             parr(ptr(own), ptr(peer)), 2, ptr(own), None)
    assert np.array_equal(own[:R], orc.rs2_active(BF16, AVG, x0[:R].copy(), x1[:R].copy()))
    assert np.array_equal(own[R:], x0[R:])


@pytest.mark.parametrize("count", [2 ** 20 + 4 * 128 + 12, 2 ** 19 + 3])
def test_ar4_helper_and_active(sim, orc, count):
    sim.reset()
    A, H = 4, 4
    xs = [synth.as_bf16_bits(synth.uniform(count, -2, 2, 3, r)) for r in range(A)]
    bx = [sim.buf(x.copy(), writable=False) for x in xs]
    g = orc.geometry(A, H, 0, 500, count, AR, BF16)
    c = g["chunk"]
    for h in range(H):
        out = sim.buf(np.zeros(max(c, 1), np.uint16))
        sim.call("rr_helper_reduce", rel(A, H, 0, 500, count), AR, BF16, AVG, h,
                 parr(*[ptr(b, h * c) for b in bx]), 4, ptr(out), None)
        if c:
            ref = orc.ar4_helper(BF16, AVG, [x[h * c:(h + 1) * c].copy() for x in xs])
            assert np.array_equal(out[:c], ref)
    for a in range(A):
        out = sim.buf(np.zeros(count, np.uint16))
        sim.call("rr_active_add_scale", rel(A, H, 0, 500, count), AR, BF16, AVG, a,
                 parr(*[ptr(b) for b in bx]), 4, ptr(out), None)
        ref = orc.ar_active(BF16, AVG, A, H, 0, 500, count, a, xs, np.zeros(count, np.uint16))
        assert np.array_equal(out, ref)


@pytest.mark.parametrize("H,R,lead", [(4, 8 * 128 * 4 + 24, 0), (4, 8 * 128 * 2 + 5, 1), (24, 48 * 128 * 2 + 40, 3)])
def test_rs4_passes(sim, orc, H, R, lead):
    """H=24 makes pass 2 exceed one segment table (24 offload slices and 25
    direct pieces), here with misaligned views."""
    sim.reset()
    A = 4
    g = orc.geometry(A, H, 0, 500, R, RS, BF16)
    c = g["chunk"]
    scratch = bits(A * (A - 1) * c, 2, 9)
    sbuf = sim.buf(padded(scratch, lead), writable=False)
    red = sim.buf(np.zeros(A * c + lead + 8, np.uint16))
    sim.call("rr_rs_multi_reduce", rel(A, H, 0, 500, R), BF16, SUM, 1, 0, parr(ptr(sbuf, lead)), 1,
             ptr(red, lead), None)
    assert np.array_equal(red[lead:lead + A * c], orc.rs4_pass1(BF16, A, c, scratch))
    blk = [bits(R, 2, s) for s in range(A)]
    reds = [bits(c, 3, h) for h in range(H)]
    # H=24: every view shares one misalignment (element-wise head and tail,
    # no realignment); otherwise the views disagree modulo 16 bytes and the
    # inputs are realigned.
    bl = [lead if (H == 24 or s % 2) else 0 for s in range(A)]
    ol = lead if H == 24 else 0
    bb = [sim.buf(padded(b, bl[s]), writable=False) for s, b in enumerate(blk)]
    rb = [sim.buf(padded(r, lead), writable=False) for r in reds]
    for o in range(A):
        out = sim.buf(np.zeros(R + 16, np.uint16))
        launches0 = sim.L.sim_launches()
        sim.call("rr_rs_multi_reduce", rel(A, H, 0, 500, R), BF16, AVG, 2, o,
                 parr(*[ptr(b, bl[s]) for s, b in enumerate(bb)], *[ptr(r, lead) for r in rb]),
                 A + H, ptr(out, ol), None)
        assert np.array_equal(out[ol:ol + R], orc.rs4_pass2(BF16, AVG, A, H, 500, R, o, blk, reds))
        if H == 24:
            assert sim.L.sim_launches() - launches0 >= 2


@pytest.fixture(scope="module", params=["default", "long"])
def copy_sim(request):
    """The replay with the default copy tiling, and with the long-call tiling
    (4 KiB tiles for aligned moves) that the library takes for calls of
    hundreds of MiB, forced here for every call."""
    return Sim(long_copies=request.param == "long")


def _tiling_used(sim, long_copies):
    n_long, n_default = sim.L.sim_copy_launches(1), sim.L.sim_copy_launches(0)
    assert (n_long > 0 and n_default == 0) if long_copies else (n_long == 0 and n_default > 0)


def _copy_call(sim, name, *args):
    """Issues one copy call; checks that it took the long-call tiling exactly
    when the library forces it and none of its moves is realigned (every launch
    in the aligned-only kernels), and the long call's non-temporal stores
    exactly when the library forces it.  Returns whether it took the long
    tiling (False for a call with nothing to move)."""
    L = sim.L
    before = (L.sim_copy_launches(1), L.sim_copy_launches(0), L.sim_shifted_copy_launches(),
              L.sim_nt_copy_launches(1))
    sim.call(name, *args)
    n_long, n_default, n_shifted, n_nt = (L.sim_copy_launches(1) - before[0], L.sim_copy_launches(0) - before[1],
                                          L.sim_shifted_copy_launches() - before[2],
                                          L.sim_nt_copy_launches(1) - before[3])
    if n_long + n_default == 0:  # nothing to move
        return False
    assert n_nt == (n_long + n_default if sim.long_copies else 0)
    want_long = sim.long_copies and n_shifted == 0
    assert (n_long > 0 and n_default == 0) if want_long else n_long == 0
    return want_long


@pytest.mark.parametrize("seg,lead", [(5 * 128 * 4 + 8, 0), (5 * 128 * 2 + 3, 0), (5 * 128 * 3, 5), (400, 0),
                                      (5 * 128 * 9 + 8, 0)])
@pytest.mark.parametrize("es", [2, 4])
def test_a2a_pack_unpack(copy_sim, orc, seg, lead, es):
    sim = copy_sim
    sim.reset()
    A, H, nc = 4, 4, 5
    dt = BF16 if es == 2 else F32
    c = orc.geometry(A, H, nc, 0, seg, A2A, dt)["chunk"]
    npdt = np.uint16 if es == 2 else np.uint32
    src = [synth.rng(4, s).integers(0, 2 ** (8 * es), A * seg, dtype=npdt) for s in range(A)]
    sb = [sim.buf(padded(s, lead), writable=False) for s in src]
    outs = [sim.buf(np.full(A * seg + 16, 0x5A, npdt)) for _ in range(A)]
    longs = []
    for h in range(H):
        dst = [sim.buf(np.zeros(max((A - 1) * c, 1) + 8, npdt)) for _ in range(A)]
        longs.append(_copy_call(sim, "rr_a2a_pack", rel(A, H, nc, 0, seg), dt, h, parr(*[ptr(b, lead) for b in sb]),
                                parr(*[ptr(d) for d in dst]), None))
        ref = orc.a2a_pack(es, A, seg, c, h, src)
        for d in range(A):
            assert np.array_equal(dst[d][:(A - 1) * c].view(np.uint8), ref[d])
        recv = [sim.buf(d.copy(), writable=False) for d in dst]
        longs.append(_copy_call(sim, "rr_a2a_unpack", rel(A, H, nc, 0, seg), dt, h,
                                parr(*[ptr(r) for r in recv]), parr(*[ptr(o, 1) for o in outs]), None))
    expect = [np.full(A * seg, 0x5A, npdt) for _ in range(A)]
    for h in range(H):
        orc.a2a_unpack(es, A, seg, c, h, orc.a2a_pack(es, A, seg, c, h, src), expect)
    for d in range(A):
        assert np.array_equal(outs[d][1:1 + A * seg], expect[d])
        assert outs[d][0] == 0x5A and np.all(outs[d][1 + A * seg:] == 0x5A)
    if c > 0 and lead == 0 and (seg * es) % 16 == 0:
        # every pack move is aligned: the long-call tiling runs where forced
        assert any(longs) == sim.long_copies


# --------------------------------------------------------------------------
# batched multi-group calls
# --------------------------------------------------------------------------

import pack_rr_helper_amd as _rr  # noqa: E402  (ctypes job layouts only)


def _relay(A, H, nc, pm, count):
    return _Relay(A, H, nc, pm, count)


def test_helper_many_heterogeneous_groups_one_launch(sim, orc):
    """Three A=2 groups of different sizes and one zero-chunk group in one
    call: one launch, each group's helper output equal to the oracle's."""
    sim.reset()
    counts = [8 * 128 * 12 + 5, 8 * 128 * 3, 900, 8 * 128 * 7 + 3]
    jobs = (_rr._HelperJob * len(counts))()
    refs, outs = [], []
    for j, n in enumerate(counts):
        x = [sim.buf(bits(n, 20 + j, a), writable=False) for a in range(2)]
        c = orc.geometry(2, 6, 8, 0, n, AR, BF16)["chunk"]
        h = j % 6
        out = sim.buf(np.zeros(max(c, 1), np.uint16))
        jobs[j].relay, jobs[j].helper, jobs[j].nSlots = _relay(2, 6, 8, 0, n), h, 2
        jobs[j].slots[0], jobs[j].slots[1] = ptr(x[0], h * c).value, ptr(x[1], h * c).value
        jobs[j].out = ptr(out).value
        outs.append((out, c))
        refs.append(orc.ar2_helper(BF16, AVG, x[0][h * c:(h + 1) * c].copy(), x[1][h * c:(h + 1) * c].copy())
                    if c else None)
    L0 = sim.L.sim_launches()
    sim.call("rr_helper_reduce_many", AR, BF16, AVG, jobs, len(counts), None)
    assert sim.L.sim_launches() - L0 == 1
    for (out, c), ref in zip(outs, refs):
        if c:
            assert np.array_equal(out[:c], ref)
        else:
            assert np.all(out == 0)


def test_active_many_mixes_a2_and_a4_groups(sim, orc):
    sim.reset()
    n2, n4 = 8 * 128 * 5 + 17, 2 ** 20 + 4 * 128 * 3
    x2 = [sim.buf(bits(n2, 30, a), writable=False) for a in range(2)]
    x4 = [sim.buf(bits(n4, 31, a), writable=False) for a in range(4)]
    o2 = [sim.buf(np.zeros(n2, np.uint16)) for _ in range(2)]
    o4 = [sim.buf(np.zeros(n4, np.uint16)) for _ in range(4)]
    specs = [(_relay(2, 6, 8, 0, n2), a, x2, o2[a]) for a in range(2)] + \
            [(_relay(4, 4, 0, 500, n4), a, x4, o4[a]) for a in range(4)]
    jobs = (_rr._ActiveJob * len(specs))()
    for j, (r, a, xs, o) in enumerate(specs):
        jobs[j].relay, jobs[j].activeIdx, jobs[j].nIn = r, a, len(xs)
        for i, x in enumerate(xs):
            jobs[j].inp[i] = ptr(x).value
        jobs[j].out = ptr(o).value
    sim.call("rr_active_add_scale_many", AR, BF16, AVG, jobs, len(specs), None)
    for a in range(2):
        assert np.array_equal(o2[a], orc.ar_active(BF16, AVG, 2, 6, 8, 0, n2, a, x2, np.zeros(n2, np.uint16)))
    for a in range(4):
        assert np.array_equal(o4[a], orc.ar_active(BF16, AVG, 4, 4, 0, 500, n4, a, x4, np.zeros(n4, np.uint16)))


def test_phase_reduce_runs_a4_helper_and_active_slices_in_one_launch(sim, orc):
    """The A=4 allreduce phase of one rank: its helper slice of the other
    group and its own direct slice, one call, one launch, each output equal
    to the oracle's; then every helper and active job of a group at once."""
    sim.reset()
    # above the 2 MiB pure-direct floor; every slice starts 16-byte aligned
    # (other offsets take a second, realigning launch) and the last active
    # slice has a 3-element tail
    A, H, n = 4, 4, 2 ** 20 + 2 ** 15 + 3
    xs = [synth.as_bf16_bits(synth.uniform(n, -2, 2, 3, r)) for r in range(A)]
    ys = [synth.as_bf16_bits(synth.uniform(n, -2, 2, 4, r)) for r in range(A)]
    bx = [sim.buf(x.copy(), writable=False) for x in xs]
    by = [sim.buf(y.copy(), writable=False) for y in ys]
    c = orc.geometry(A, H, 0, 500, n, AR, BF16)["chunk"]
    assert c > 0

    def helper_jobs(hs, src):
        jobs = (_rr._HelperJob * len(hs))()
        outs = []
        for j, h in enumerate(hs):
            o = sim.buf(np.zeros(c, np.uint16))
            jobs[j].relay, jobs[j].helper, jobs[j].nSlots = _relay(A, H, 0, 500, n), h, A
            for i, b in enumerate(src):
                jobs[j].slots[i] = ptr(b, h * c).value
            jobs[j].out = ptr(o).value
            outs.append(o)
        return jobs, outs

    def active_jobs(as_, src):
        jobs = (_rr._ActiveJob * len(as_))()
        outs = []
        for j, a in enumerate(as_):
            o = sim.buf(np.zeros(n, np.uint16))
            jobs[j].relay, jobs[j].activeIdx, jobs[j].nIn = _relay(A, H, 0, 500, n), a, A
            for i, b in enumerate(src):
                jobs[j].inp[i] = ptr(b).value
            jobs[j].out = ptr(o).value
            outs.append(o)
        return jobs, outs

    for hs, as_ in (([1], [2]), (list(range(H)), list(range(A)))):
        hj, ho = helper_jobs(hs, by)     # the other group's offload region
        aj, ao = active_jobs(as_, bx)    # this group's direct slices
        L0 = sim.L.sim_launches()
        sim.call("rr_phase_reduce_many", AR, BF16, AVG, hj, len(hs), aj, len(as_), None)
        assert sim.L.sim_launches() - L0 == 1
        for h, o in zip(hs, ho):
            assert np.array_equal(o, orc.ar4_helper(BF16, AVG, [y[h * c:(h + 1) * c].copy() for y in ys]))
        for a, o in zip(as_, ao):
            assert np.array_equal(o, orc.ar_active(BF16, AVG, A, H, 0, 500, n, a, xs, np.zeros(n, np.uint16)))

    # a helper job reading what an active job writes (active 0's direct
    # slice starts after the H relay chunks) names the active job with its
    # number after the helper jobs'; an empty call launches nothing
    hj, _ = helper_jobs([0], by)
    aj, ao = active_jobs([0], bx)
    hj[0].slots[1] = ptr(ao[0], H * c).value
    L = sim.L
    L0 = L.sim_launches()
    assert L.rr_phase_reduce_many(AR, BF16, AVG, hj, 1, aj, 1, None) == 2      # RR_EALIAS
    assert L.rr_last_error().decode().startswith("jobs 0 and 1: ")
    aj[0].activeIdx = 7
    assert L.rr_phase_reduce_many(AR, BF16, AVG, hj, 1, aj, 1, None) == 1      # RR_EINVAL
    assert L.rr_last_error().decode().startswith("job 1:")
    assert L.rr_phase_reduce_many(AR, BF16, AVG, None, 0, None, 0, None) == 0
    assert L.rr_phase_reduce_many(AR, BF16, AVG, None, 1, None, 0, None) == 1
    assert L.sim_launches() == L0


def test_many_rejects_cross_job_overlap_and_names_the_job(sim):
    sim.reset()
    n = 8 * 128 * 4
    x = [sim.buf(bits(n, 40, a), writable=False) for a in range(2)]
    out = sim.buf(np.zeros(2 * n, np.uint16))
    jobs = (_rr._HelperJob * 2)()
    c = n // 8
    for j in range(2):
        jobs[j].relay, jobs[j].helper, jobs[j].nSlots = _relay(2, 6, 8, 0, n), j, 2
        jobs[j].slots[0], jobs[j].slots[1] = ptr(x[0], j * c).value, ptr(x[1], j * c).value
        jobs[j].out = ptr(out, j * 64).value           # job 1's output overlaps job 0's
    L = sim.L
    L0 = L.sim_launches()
    assert L.rr_helper_reduce_many(AR, BF16, AVG, jobs, 2, None) == 2    # RR_EALIAS
    assert L.rr_last_error().decode() == "jobs 0 and 1: two output ranges overlap"
    # job 1 reading job 0's output
    jobs[1].out = ptr(out, n).value
    jobs[1].slots[1] = ptr(out, 16).value
    assert L.rr_helper_reduce_many(AR, BF16, AVG, jobs, 2, None) == 2
    assert L.rr_last_error().decode().startswith("jobs 0 and 1: an output range overlaps")
    # an alias within one job is named like any other invalid job
    jobs[1].slots[1] = ptr(x[1], c).value
    jobs[1].out = ptr(x[1], c + 1).value
    assert L.rr_helper_reduce_many(AR, BF16, AVG, jobs, 2, None) == 2
    assert L.rr_last_error().decode().startswith("job 1: an output range overlaps")
    jobs[1].out = ptr(out, n).value
    jobs[1].helper = 9
    assert L.rr_helper_reduce_many(AR, BF16, AVG, jobs, 2, None) == 1    # RR_EINVAL
    assert L.rr_last_error().decode().startswith("job 1:")
    assert L.sim_launches() == L0


def test_rs_and_a2a_many_match_single_calls(sim, orc):
    sim.reset()
    A, H, R = 4, 4, 8 * 128 * 3 + 16
    c = orc.geometry(A, H, 0, 500, R, RS, BF16)["chunk"]
    xs = [bits(A * R, 50, s) for s in range(A)]
    bx = [sim.buf(x, writable=False) for x in xs]
    scratch = [sim.buf(np.concatenate([xs[s][o * R + h * c:o * R + (h + 1) * c] for o in range(A)
                                       for s in range(A) if s != o] + [np.zeros(4 * c + 16, np.uint16)]))
               for h in range(H)]
    jobs = (_rr._RsJob * H)()
    keep = []
    for h in range(H):
        p = parr(ptr(scratch[h]))
        keep.append(p)
        jobs[h].relay, jobs[h].pass_, jobs[h].idx, jobs[h].nIn = _relay(A, H, 0, 500, R), 1, h, 1
        jobs[h].inp = ctypes.cast(p, ctypes.POINTER(ctypes.c_void_p))
        jobs[h].out = ptr(scratch[h], 12 * c).value
    sim.call("rr_rs_multi_reduce_many", BF16, SUM, jobs, H, None)
    outs = [sim.buf(np.zeros(R, np.uint16)) for _ in range(A)]
    jobs2 = (_rr._RsJob * A)()
    for o in range(A):
        p = parr(*[ptr(b, o * R) for b in bx], *[ptr(scratch[h], 12 * c + o * c) for h in range(H)])
        keep.append(p)
        jobs2[o].relay, jobs2[o].pass_, jobs2[o].idx, jobs2[o].nIn = _relay(A, H, 0, 500, R), 2, o, A + H
        jobs2[o].inp = ctypes.cast(p, ctypes.POINTER(ctypes.c_void_p))
        jobs2[o].out = ptr(outs[o]).value
    L0 = sim.L.sim_launches()
    sim.call("rr_rs_multi_reduce_many", BF16, SUM, jobs2, A, None)
    assert sim.L.sim_launches() - L0 == 1
    ref = orc.rs4_group(BF16, SUM, H, 500, R, xs)
    for o in range(A):
        assert np.array_equal(outs[o], ref[o])
    # all-to-all: the four helper slices' packs and unpacks as two calls
    seg = 5 * 128 * 3 + 8
    cc = orc.geometry(A, H, 5, 0, seg, A2A, BF16)["chunk"]
    src = [sim.buf(synth.bits16(A * seg, 51, s), writable=False) for s in range(A)]
    packed = [[sim.buf(np.zeros(3 * cc, np.uint16)) for _ in range(A)] for _ in range(H)]
    out = [sim.buf(np.zeros(A * seg, np.uint16)) for _ in range(A)]
    for name, ins, outs_ in (("rr_a2a_pack_many", lambda h: src, lambda h: packed[h]),
                             ("rr_a2a_unpack_many", lambda h: packed[h], lambda h: out)):
        aj = (_rr._A2AJob * H)()
        for h in range(H):
            pi, po = parr(*[ptr(b) for b in ins(h)]), parr(*[ptr(b) for b in outs_(h)])
            keep += [pi, po]
            aj[h].relay, aj[h].helper = _relay(A, H, 5, 0, seg), h
            aj[h].inp = ctypes.cast(pi, ctypes.POINTER(ctypes.c_void_p))
            aj[h].out = ctypes.cast(po, ctypes.POINTER(ctypes.c_void_p))
        sim.call(name, BF16, aj, H, None)
    expect = [np.zeros(A * seg, np.uint16) for _ in range(A)]
    for h in range(H):
        orc.a2a_unpack(2, A, seg, cc, h, orc.a2a_pack(2, A, seg, cc, h, src), expect)
    for d in range(A):
        assert np.array_equal(out[d], expect[d])


# --------------------------------------------------------------------------
# randomized: geometry, sizes, ops, dtypes, misalignment, batching
# --------------------------------------------------------------------------

def _rand_case(rng):
    A = int(rng.choice([2, 4]))
    H = int(rng.integers(1, 7)) if A == 2 else int(rng.integers(1, 5))
    dt = int(rng.choice([F32, BF16]))
    op = int(rng.choice([SUM, AVG]))
    return A, H, dt, op


@pytest.mark.parametrize("seed", range(48))
def test_random_active_and_helper_calls_match_the_oracle(sim, orc, seed):
    rng = np.random.default_rng(1000 + seed)
    sim.reset()
    A, H, dt, op = _rand_case(rng)
    npdt = np.float32 if dt == F32 else np.uint16
    es = 4 if dt == F32 else 2
    nc = H + 2 + int(rng.integers(0, 3)) if A == 2 else 0
    pm = int(rng.choice([250, 500, 780, 1000])) if A == 4 else 0
    count = int(rng.integers(0, 3 * 2 ** 20 // es)) if A == 4 else int(rng.integers(0, 40000))
    g = orc.geometry(A, H, nc, pm, count, AR, dt)
    assert g is not None
    lead = int(rng.integers(0, 8))
    def mk(r):
        x = synth.normal(count, 2000 + seed, r)
        return x if dt == F32 else synth.as_bf16_bits(x)
    xs = [mk(r) for r in range(A)]
    bx = [sim.buf(padded(x, lead if rng.random() < 0.5 else 0), writable=False) for x in xs]
    leads = [(b.size - 16 - x.size) for b, x in zip(bx, xs)]
    rel = _Relay(A, H, nc, pm, count)
    # actives, batched
    jobs = (_rr._ActiveJob * A)()
    outs = []
    for a in range(A):
        o = sim.buf(np.zeros(count + 8, npdt))
        outs.append(o)
        jobs[a].relay, jobs[a].activeIdx, jobs[a].nIn = rel, a, A
        for s in range(A):
            jobs[a].inp[s] = ptr(bx[s], leads[s]).value
        jobs[a].out = ptr(o).value
    sim.call("rr_active_add_scale_many", AR, dt, op, jobs, A, None)
    for a in range(A):
        ref = orc.ar_active(dt, op, A, H, nc, pm, count, a, xs, np.zeros(count, npdt))
        assert np.array_equal(outs[a][:count].view(np.uint8), ref.view(np.uint8)), (A, H, dt, count, a)
    # helpers, one batched call over every helper
    c = g["chunk"]
    hj = (_rr._HelperJob * H)()
    houts = []
    for h in range(H):
        o = sim.buf(np.zeros(max(c, 1) + 8, npdt))
        houts.append(o)
        hj[h].relay, hj[h].helper, hj[h].nSlots = rel, h, A
        for s in range(A):
            hj[h].slots[s] = ptr(bx[s], leads[s] + h * c).value
        hj[h].out = ptr(o, 1 if rng.random() < 0.3 else 0).value
    sim.call("rr_helper_reduce_many", AR, dt, op, hj, H, None)
    for h in range(H):
        if not c:
            continue
        sl = [x[h * c:(h + 1) * c].copy() for x in xs]
        ref = orc.ar2_helper(dt, op, *sl) if A == 2 else orc.ar4_helper(dt, op, sl)
        o = houts[h]
        start = (hj[h].out - o.ctypes.data) // es
        assert np.array_equal(o[start:start + c].view(np.uint8), ref.view(np.uint8)), (A, H, dt, count, h)


@pytest.mark.parametrize("seed", range(32))
def test_random_all_to_all_round_trip(sim, orc, seed):
    rng = np.random.default_rng(3000 + seed)
    sim.reset()
    A = int(rng.choice([2, 4]))
    H = int(rng.integers(1, 7)) if A == 2 else int(rng.integers(1, 5))
    nc = (H + 2 if A == 2 else H + 1) + int(rng.integers(0, 4))
    es = int(rng.choice([2, 4]))
    dt = BF16 if es == 2 else F32
    npdt = np.uint16 if es == 2 else np.uint32
    seg = int(rng.integers(0, 20000))
    c = orc.geometry(A, H, nc, 0, seg, A2A, dt)["chunk"]
    src = [rng.integers(0, 2 ** (8 * es), A * seg, dtype=npdt) for _ in range(A)]
    lead = int(rng.integers(0, 8))
    sb = [sim.buf(padded(s, lead), writable=False) for s in src]
    packed = [[sim.buf(np.zeros(max((A - 1) * c, 1) + 8, npdt)) for _ in range(A)] for _ in range(H)]
    out = [sim.buf(np.full(A * seg + 16, 7, npdt)) for _ in range(A)]
    keep = []
    for name, ins, outs_ in (("rr_a2a_pack_many", lambda h: [ptr(b, lead) for b in sb], lambda h: [ptr(p) for p in packed[h]]),
                             ("rr_a2a_unpack_many", lambda h: [ptr(p) for p in packed[h]], lambda h: [ptr(o, 3) for o in out])):
        aj = (_rr._A2AJob * H)()
        for h in range(H):
            pi, po = parr(*ins(h)), parr(*outs_(h))
            keep += [pi, po]
            aj[h].relay, aj[h].helper = _relay(A, H, nc, 0, seg), h
            aj[h].inp = ctypes.cast(pi, ctypes.POINTER(ctypes.c_void_p))
            aj[h].out = ctypes.cast(po, ctypes.POINTER(ctypes.c_void_p))
        sim.call(name, dt, aj, H, None)
    expect = [np.full(A * seg, 7, npdt) for _ in range(A)]
    for h in range(H):
        if c:
            orc.a2a_unpack(es, A, seg, c, h, orc.a2a_pack(es, A, seg, c, h, src), expect)
    for d in range(A):
        assert np.array_equal(out[d][3:3 + A * seg], expect[d]), (A, H, nc, es, seg, d)


# --------------------------------------------------------------------------
# launch forms
# --------------------------------------------------------------------------

def test_copy_batch_of_unequal_moves_fills_the_table(sim, orc):
    """Six pack jobs over groups of different segmentCounts (some 5 mod 8):
    72 chunk moves of 2-6 tiles.  The first launch holds a full 64-entry tile
    table in the mixed-mode kernel, the last 8 moves (of one job, equal)
    follow in a uniform mixed-mode launch; every job's bytes as the oracle's,
    every access inside the registered buffers."""
    sim.reset()
    A, H, nc = 4, 4, 5
    aj = (_rr._A2AJob * 6)()
    keep, outs, refs = [], [], []
    for j in range(6):
        seg = 5 * 128 * (40 + 24 * j) + (5 if j % 2 else 0)
        c = orc.geometry(A, H, nc, 0, seg, A2A, BF16)["chunk"]
        src = [sim.buf(synth.bits16(A * seg, 320 + j, s), writable=False) for s in range(A)]
        dst = [sim.buf(np.zeros((A - 1) * c, np.uint16)) for _ in range(A)]
        pi, po = parr(*[ptr(b) for b in src]), parr(*[ptr(b) for b in dst])
        keep += [pi, po]
        aj[j].relay, aj[j].helper = _relay(A, H, nc, 0, seg), j % H
        aj[j].inp = ctypes.cast(pi, ctypes.POINTER(ctypes.c_void_p))
        aj[j].out = ctypes.cast(po, ctypes.POINTER(ctypes.c_void_p))
        outs.append(dst)
        refs.append(orc.a2a_pack(2, A, seg, c, j % H, src))
    sim.call("rr_a2a_pack_many", BF16, aj, 6, None)
    assert sim.L.sim_launches() == 2
    assert [sim.L.sim_form_launches(1, f) for f in range(3)] == [1, 1, 0]
    assert sim.L.sim_shifted_copy_launches() == 2
    for j in range(6):
        for d in range(A):
            assert np.array_equal(outs[j][d].view(np.uint8), refs[j][d]), f"job {j} dest {d}"


def test_every_launch_form_is_replayed(sim, orc):
    """The library launches a batch in one of three forms (one segment with
    preloaded arguments, a uniform (tile, segment) grid, the tile table).  Each form, replayed here, writes the oracle's values and
    touches only the registered buffers."""
    def forms(copy):
        return [sim.L.sim_form_launches(copy, f) for f in range(3)]   # table, uniform, one

    sim.reset()
    # one aligned segment: an A=2 reduce-scatter owner over its whole block
    R = 8 * 128 * 20
    x0, x1 = bits(R, 41, 0), bits(R, 41, 1)
    a, b = sim.buf(x0.copy(), writable=False), sim.buf(x1.copy(), writable=False)
    out = sim.buf(np.zeros(R, np.uint16))
    sim.call("rr_active_add_scale", rel(2, 6, 8, 0, R), RS, BF16, AVG, 0, parr(ptr(a), ptr(b)), 2,
             ptr(out), None)
    assert np.array_equal(out, orc.rs2_active(BF16, AVG, x0.copy(), x1.copy()))
    assert forms(0) == [0, 0, 1]

    # equal segments: all six helpers of an A=2 group, three tiles each
    n = 8 * 8192 * 3
    xs = [sim.buf(bits(n, 42, s), writable=False) for s in range(2)]
    c = orc.geometry(2, 6, 8, 0, n, AR, BF16)["chunk"]
    jobs = (_rr._HelperJob * 6)()
    outs = [sim.buf(np.zeros(c, np.uint16)) for _ in range(6)]
    for h in range(6):
        jobs[h].relay, jobs[h].helper, jobs[h].nSlots = _relay(2, 6, 8, 0, n), h, 2
        jobs[h].slots[0], jobs[h].slots[1] = ptr(xs[0], h * c).value, ptr(xs[1], h * c).value
        jobs[h].out = ptr(outs[h]).value
    sim.call("rr_helper_reduce_many", AR, BF16, AVG, jobs, 6, None)
    for h in range(6):
        ref = orc.ar2_helper(BF16, AVG, xs[0][h * c:(h + 1) * c].copy(), xs[1][h * c:(h + 1) * c].copy())
        assert np.array_equal(outs[h], ref)
    assert forms(0) == [0, 1, 1]

    # every buffer 6 bytes past a 16-byte boundary: one realigning segment
    # (element-wise head and tail in tile 0), also in the single-segment form
    lead = 3
    xb = [sim.buf(padded(bits(R, 43, s), lead), writable=False) for s in range(2)]
    ob = sim.buf(np.zeros(R + lead + 16, np.uint16))
    sim.call("rr_active_add_scale", rel(2, 6, 8, 0, R), RS, BF16, SUM, 1,
             parr(ptr(xb[0], lead), ptr(xb[1], lead)), 2, ptr(ob, lead), None)
    ref = orc.rs2_active(BF16, SUM, xb[0][lead:lead + R].copy(), xb[1][lead:lead + R].copy())
    assert np.array_equal(ob[lead:lead + R], ref)
    assert forms(0) == [0, 1, 2]

    # unequal segments: helper jobs of two groups whose chunks span different
    # tile counts take the tile table
    counts = [8 * 8192 * 3, 8 * 8192 * 5 + 8 * 128]
    hj = (_rr._HelperJob * 2)()
    hrefs = []
    for j, n2 in enumerate(counts):
        xs2 = [sim.buf(bits(n2, 45 + j, s), writable=False) for s in range(2)]
        c2 = orc.geometry(2, 6, 8, 0, n2, AR, BF16)["chunk"]
        o2 = sim.buf(np.zeros(c2, np.uint16))
        hj[j].relay, hj[j].helper, hj[j].nSlots = _relay(2, 6, 8, 0, n2), 1, 2
        hj[j].slots[0], hj[j].slots[1] = ptr(xs2[0], c2).value, ptr(xs2[1], c2).value
        hj[j].out = ptr(o2).value
        hrefs.append((o2, orc.ar2_helper(BF16, AVG, xs2[0][c2:2 * c2].copy(), xs2[1][c2:2 * c2].copy())))
    sim.call("rr_helper_reduce_many", AR, BF16, AVG, hj, 2, None)
    for o2, ref2 in hrefs:
        assert np.array_equal(o2, ref2)
    assert forms(0) == [1, 1, 2]

    # copies: pack and unpack issue one segment per chunk move (tile 0 also
    # copies its head and tail bytes) and one launch per call, so the aligned
    # case (twelve aligned moves) and a ragged segmentCount (aligned and
    # realigned moves in the mixed-mode kernel) both run on the uniform grid
    A, H, nc = 4, 4, 5
    for seg, launches in ((5 * 128 * 40, 2), (5 * 128 * 40 + 3, 2)):   # chunks of several tiles
        before = forms(1)
        c = orc.geometry(A, H, nc, 0, seg, A2A, BF16)["chunk"]
        src = [sim.buf(bits(A * seg, 44, s), writable=False) for s in range(A)]
        dst = [sim.buf(np.zeros((A - 1) * c, np.uint16)) for _ in range(A)]
        sim.call("rr_a2a_pack", rel(A, H, nc, 0, seg), BF16, 2, parr(*[ptr(s) for s in src]),
                 parr(*[ptr(d) for d in dst]), None)
        ref = orc.a2a_pack(2, A, seg, c, 2, src)
        for d in range(A):
            assert np.array_equal(dst[d].view(np.uint8), ref[d])
        outs = [sim.buf(np.zeros(A * seg, np.uint16)) for _ in range(A)]
        recv = [sim.buf(d.copy(), writable=False) for d in dst]
        sim.call("rr_a2a_unpack", rel(A, H, nc, 0, seg), BF16, 2, parr(*[ptr(r) for r in recv]),
                 parr(*[ptr(o) for o in outs]), None)
        expect = [np.zeros(A * seg, np.uint16) for _ in range(A)]
        orc.a2a_unpack(2, A, seg, c, 2, ref, expect)
        for d in range(A):
            assert np.array_equal(outs[d], expect[d])
        after = forms(1)
        assert after[0] == before[0] and after[2] == before[2]
        assert after[1] - before[1] == launches


# --------------------------------------------------------------------------
# launches capped at 5 tiles: long moves and items continue in further launches
# --------------------------------------------------------------------------

@pytest.fixture(scope="module")
def capped():
    return Sim(capped=True)


@pytest.fixture(scope="module", params=["default", "long"])
def capped_copy(request):
    return Sim(capped=True, long_copies=request.param == "long")


@pytest.mark.parametrize("seg,out_lead", [(5 * 128 * 200, 0), (5 * 128 * 200 + 3, 0), (5 * 128 * 200, 1),
                                          (5 * 128 * 37 + 5, 3)])
def test_copies_longer_than_a_launch_continue(capped_copy, orc, seg, out_lead):
    """Each chunk move spans several body tiles (7 or 13 in the aligned
    moves, by tiling), more than one launch holds: the launcher cuts it after
    whole tiles, and the rest starts on a 16-byte destination boundary with the
    same source shift in the next launch."""
    sim = capped_copy
    sim.reset()
    A, H, nc, h = 4, 4, 5, 1
    c = orc.geometry(A, H, nc, 0, seg, A2A, BF16)["chunk"]
    src = [sim.buf(bits(A * seg, 60, s), writable=False) for s in range(A)]
    dst = [sim.buf(np.zeros((A - 1) * c, np.uint16)) for _ in range(A)]
    L0 = sim.L.sim_launches()
    sim.call("rr_a2a_pack", rel(A, H, nc, 0, seg), BF16, h, parr(*[ptr(s) for s in src]),
             parr(*[ptr(d) for d in dst]), None)
    tiles = -(-(c * 2) // 8192)
    assert sim.L.sim_launches() - L0 >= 12 * tiles // 5
    if seg % 8 == 0 and out_lead == 0:
        _tiling_used(sim, sim.long_copies)
    ref = orc.a2a_pack(2, A, seg, c, h, src)
    for d in range(A):
        assert np.array_equal(dst[d].view(np.uint8), ref[d])
    recv = [sim.buf(d.copy(), writable=False) for d in dst]
    outs = [sim.buf(np.full(A * seg + out_lead + 8, 0x3C, np.uint16)) for _ in range(A)]
    sim.call("rr_a2a_unpack", rel(A, H, nc, 0, seg), BF16, h, parr(*[ptr(r) for r in recv]),
             parr(*[ptr(o, out_lead) for o in outs]), None)
    expect = [np.full(A * seg, 0x3C, np.uint16) for _ in range(A)]
    orc.a2a_unpack(2, A, seg, c, h, ref, expect)
    for d in range(A):
        assert np.array_equal(outs[d][out_lead:out_lead + A * seg], expect[d])
        assert np.all(outs[d][:out_lead] == 0x3C) and np.all(outs[d][out_lead + A * seg:] == 0x3C)


@pytest.mark.parametrize("lead", [0, 3])
def test_reductions_longer_than_a_launch_continue(capped, orc, lead):
    sim = capped
    sim.reset()
    R = 8192 * 23 + 77                     # 23 vector tiles and a tail, plus a head when lead > 0
    x0, x1 = bits(R, 61, 0), bits(R, 61, 1)
    a = sim.buf(padded(x0, lead), writable=False)
    b = sim.buf(padded(x1, lead), writable=False)
    out = sim.buf(np.zeros(R + lead + 16, np.uint16))
    L0 = sim.L.sim_launches()
    sim.call("rr_active_add_scale", rel(2, 6, 8, 0, R), RS, BF16, AVG, 0, parr(ptr(a, lead), ptr(b, lead)), 2,
             ptr(out, lead), None)
    assert sim.L.sim_launches() - L0 >= 5
    assert np.array_equal(out[lead:lead + R], orc.rs2_active(BF16, AVG, x0, x1))
    assert np.all(out[:lead] == 0) and np.all(out[lead + R:] == 0)


# --------------------------------------------------------------------------
# aliasing rule on random overlapping views
# --------------------------------------------------------------------------

def _overlap(a, b):
    return a[0] < a[1] and b[0] < b[1] and a[0] < b[1] and b[0] < a[1]


@pytest.mark.parametrize("seed", range(200))
def test_random_views_follow_the_aliasing_rule(sim, orc, seed):
    """Random A=2 helper jobs over views of one buffer, on a coarse grid so
    that overlaps and exact in-place aliases are common: the call is accepted
    exactly when, checked pair by pair, no output overlaps another job's output
    or any input other than its own identical slot, and an accepted call
    writes the oracle's values."""
    sim.reset()
    rng = np.random.default_rng(7700 + seed)
    count = 8 * 256
    c = orc.geometry(2, 6, 8, 0, count, AR, BF16)["chunk"]
    N = 6 * c
    snap = bits(N, 70 + seed, 0)
    buf = sim.buf(snap.copy())
    grid = np.arange(0, N - c + 1, 64)
    jobs = []
    for _ in range(int(rng.integers(1, 6))):
        s0, s1 = (int(v) for v in rng.choice(grid, 2))
        out = s0 if rng.random() < 0.3 else int(rng.choice(grid))
        jobs.append((s0, s1, out))
    ok = True
    for i, (_, _, oi) in enumerate(jobs):
        o = (oi, oi + c)
        for j, (s0, s1, oj) in enumerate(jobs):
            for x in ((s0, s0 + c), (s1, s1 + c)):
                if _overlap(o, x) and not (i == j and o == x):
                    ok = False
            if j != i and _overlap(o, (oj, oj + c)):
                ok = False
    arr = (_rr._HelperJob * len(jobs))()
    for k, (s0, s1, o) in enumerate(jobs):
        arr[k].relay, arr[k].helper, arr[k].nSlots = _relay(2, 6, 8, 0, count), k, 2
        arr[k].slots[0], arr[k].slots[1] = ptr(buf, s0).value, ptr(buf, s1).value
        arr[k].out = ptr(buf, o).value
    st = sim.L.rr_helper_reduce_many(AR, BF16, AVG, arr, len(jobs), None)
    assert st == (0 if ok else 2), (jobs, sim.L.rr_last_error())
    sim.check()
    if ok:
        for s0, s1, o in jobs:
            ref = orc.ar2_helper(BF16, AVG, snap[s0:s0 + c].copy(), snap[s1:s1 + c].copy())
            assert np.array_equal(buf[o:o + c], ref)
