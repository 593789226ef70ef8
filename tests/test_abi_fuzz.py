"""Seeded argument fuzz of the C ABI on the host (no GPU), through
libhostsim.so: the library's validation and segment tables with a host replay
of the kernels' index arithmetic.  Each case draws a batch of jobs of one entry
point with random geometry, indices, input counts, element offsets, null or
misaligned pointers and in-place or partial aliases, and checks what must hold
whatever the arguments:

* every status is RR_OK, RR_EINVAL or RR_EALIAS, and a rejected call sets a
  message and leaves every byte of every buffer as it was;
* a job drawn with no fault injected is accepted;
* an accepted call's replay reads and writes only inside the buffers it was
  given, and leaves the buffers no output points into unchanged;
* the batched entry point agrees with its jobs called one by one: the first
  job whose arguments its single call rejects fails the batch with that
  call's status and message under the job's index; failing that, an alias
  the single call of a job finds over its items fails the batch under that
  job's index; otherwise the batch writes the same bytes as the single calls
  (the jobs' buffers are disjoint, so order does not matter).

Output values are checked against the oracle elsewhere; this test covers the
argument space around them."""
import ctypes
import re

import numpy as np
import pytest

from pack_rr_helper_amd import _A2AJob, _ActiveJob, _HelperJob, _Relay, _RsJob
from tests.hostsim import Sim

AR, RS, A2A = 0, 1, 2
F32, BF16 = 0, 1
SLACK = 300   # elements: the largest offset of a partially aliased output
OK, EINVAL, EALIAS = 0, 1, 2
KINDS = ("helper", "active", "rs", "pack", "unpack")
# aliases found over all items (or moves) of a call, after every job's
# arguments are accepted
WHOLE_CALL_ALIAS = ("two output ranges overlap",
                    "an output range overlaps an input range other than an exact in-place alias",
                    "two destination chunks overlap",
                    "a destination chunk overlaps a source chunk")


@pytest.fixture(scope="module")
def sims():
    return {False: Sim(), True: Sim(capped=True)}


class Case:
    """Buffers of one case, all registered with the replay as writable."""

    def __init__(self, sim, rng, es):
        self.sim, self.rng, self.es = sim, rng, es
        self.bufs = []
        self.out_targets = set()      # indices of buffers an output points into
        self.faulty = False           # a fault was injected somewhere in the job

    def fresh(self, nelem):
        # counts beyond this are only drawn as invalid (rejected) arguments; a
        # call that accepted one would show up as a replay access violation
        nelem = min(nelem, 1 << 23)
        lead = int(self.rng.integers(0, 8))
        nominal = (nelem + lead + 8) * self.es
        # SLACK more elements of memory past the registered range: room for an
        # output placed at a partial alias of this buffer (out_pointer)
        a = np.concatenate([self.rng.integers(0, 256, size=nominal, dtype=np.uint8),
                            np.zeros(SLACK * self.es, np.uint8)])
        self.sim.register(a.ctypes.data, nominal)
        self.bufs.append(a)
        return a.ctypes.data + lead * self.es

    def owner(self, p):
        for i, a in enumerate(self.bufs):
            if a.ctypes.data <= p < a.ctypes.data + a.nbytes:
                return i
        return None

    def pointer(self, nelem):
        """A device pointer for a read buffer: usually fresh and element
        aligned, sometimes null or not aligned to the element."""
        u = self.rng.random()
        if u < 0.02:
            self.faulty = True
            return 0
        if u < 0.04:
            self.faulty = True
            return self.fresh(nelem) + (1 if self.es == 2 else int(self.rng.choice([1, 2, 3])))
        return self.fresh(nelem)

    def out_pointer(self, nelem, inputs, in_place):
        """An output pointer: fresh, or an exact or partial alias of one of
        `inputs`; an exact alias is valid only for the pointers in `in_place`."""
        u = self.rng.random()
        p = None
        if inputs and u < 0.06:
            p = int(self.rng.choice(inputs))
            if not p or p not in in_place:
                self.faulty = True
        elif inputs and u < 0.09:
            p = int(self.rng.choice(inputs))
            p = p + int(self.rng.integers(1, SLACK)) * self.es if p else 0
            self.faulty = True
            # the caller's output buffer of nelem elements at p: a call may
            # accept it when the overlap misses every range it reads (an input
            # its geometry leaves unused), and then writes all of it
            if p:
                self.sim.register(p, min(nelem, 1 << 23) * self.es)   # the cap of fresh()
        else:
            p = self.pointer(nelem)
        o = self.owner(p) if p else None
        if o is not None:
            self.out_targets.add(o)
        return p

    def snapshot(self):
        return [a.copy() for a in self.bufs]

    def same_as(self, snap, only=None):
        idx = range(len(self.bufs)) if only is None else only
        return all(np.array_equal(self.bufs[i], snap[i]) for i in idx)

    def restore(self, snap):
        for a, s in zip(self.bufs, snap):
            a[...] = s


def pick(rng, good, bad, case, p_bad=0.06):
    if rng.random() < p_bad:
        case.faulty = True
        return int(rng.choice(bad))
    return int(rng.choice(good))


def draw_relay(rng, case, kind, dt):
    A = 4 if kind in ("rs", "pack", "unpack") else int(rng.choice([2, 4]))
    if kind == "active" and rng.random() < 0.3:
        A = 2                                   # A=2 reduce-scatter owner
    A = pick(rng, [A], [0, 1, 3, 8, -2], case, 0.03)
    H = pick(rng, list(range(1, 7)) if A == 2 else list(range(1, 5)), [0, -1], case, 0.03)
    coll = {"helper": AR, "active": RS if (A == 2 and rng.random() < 0.3) else AR, "rs": RS,
            "pack": A2A, "unpack": A2A}[kind]
    nc, pm = 0, 500
    if A == 2:
        nc = pick(rng, [H + 2 + int(rng.integers(0, 3))], [H + 1, 0, -1], case, 0.04)
    elif coll == A2A:
        nc = pick(rng, [H + 1 + int(rng.integers(0, 3))], [H, 0], case, 0.04)
    elif coll == RS:
        pm = pick(rng, [int(rng.integers(1, min(1000, 125 * max(H, 1)) + 1))],
                  [0, 1001, -3, 125 * max(H, 1) + 130], case, 0.04)
    else:
        pm = pick(rng, [int(rng.integers(1, 1001)), 500, 1000], [0, 1001], case, 0.04)
    es = 4 if dt == F32 else 2
    if A == 4 and coll == AR and rng.random() < 0.15:
        count = (2 << 20) // es + int(rng.integers(0, 5000))    # above the 2 MiB floor
    else:
        count = int(rng.integers(0, 3 * 1024)) if rng.random() < 0.5 else int(rng.integers(0, 20000))
    if rng.random() < 0.02:
        case.faulty = True
        count = int(rng.choice([-1, -4096, (1 << 48) + 1]))
    return coll, _Relay(A, H, nc, pm, count)


def draw_job(rng, case, kind, dt):
    coll, r = draw_relay(rng, case, kind, dt)
    A, H, n = r.A, r.H, max(r.count, 0)
    if kind == "helper":
        idx = pick(rng, list(range(max(H, 1))), [-1, max(H, 1), 99], case, 0.04)
        k = pick(rng, [A if A in (2, 4) else 2], [0, 1, 3, 5, 9], case, 0.03)
        slots = [case.pointer(n) for _ in range(4)]
        used = slots[:min(max(k, 0), 4)]
        out = case.out_pointer(n, used, in_place=used)
        return coll, dict(relay=r, helper=idx, nSlots=k, slots=slots, out=out)
    if kind == "active":
        idx = pick(rng, list(range(A if A in (2, 4) else 2)), [-1, 4, 7], case, 0.04)
        k = pick(rng, [A if A in (2, 4) else 2], [0, 1, 3, 5], case, 0.03)
        ins = [case.pointer(n) for _ in range(4)]
        used = ins[:min(max(k, 0), 4)]
        out = case.out_pointer(n, used, in_place=used)
        return coll, dict(relay=r, activeIdx=idx, nIn=k, inp=ins, out=out)
    if kind == "rs":
        ps = pick(rng, [1, 2], [0, 3], case, 0.03)
        idx = pick(rng, list(range(max(H, 1) if ps == 1 else 4)), [-1, 9], case, 0.04)
        want = 1 if ps == 1 else 4 + max(H, 0)
        k = pick(rng, [want], [want + 1, max(want - 1, 0), 0], case, 0.03)
        ins = [case.pointer(2 * n if (ps == 1 and i == 0) else n) for i in range(16)]
        # in place: pass 2 may write over the owner's own block exactly
        own = [ins[idx]] if ps == 2 and 0 <= idx < min(k, 4) else []
        out = case.out_pointer(n, ins[:min(max(k, 0), 16)], in_place=own)
        return coll, dict(relay=r, pass_=ps, idx=idx, nIn=k, inp=ins, out=out)
    # all-to-all pack (src, dst) or unpack (recv, out): never in place
    idx = pick(rng, list(range(max(H, 1))), [-1, max(H, 1)], case, 0.04)
    ins = [case.pointer(4 * n) for _ in range(4)]
    outs = [case.out_pointer(4 * n, ins, in_place=[]) for _ in range(4)]
    return coll, dict(relay=r, helper=idx, inp=ins, out=outs)


def pointer_array(ps):
    return (ctypes.c_void_p * len(ps))(*[p or None for p in ps])


def call_single(L, kind, coll, dt, op, j):
    r = ctypes.byref(j["relay"])
    if kind == "helper":
        return L.rr_helper_reduce(r, coll, dt, op, j["helper"], pointer_array(j["slots"]), j["nSlots"],
                                  ctypes.c_void_p(j["out"] or None), None)
    if kind == "active":
        return L.rr_active_add_scale(r, coll, dt, op, j["activeIdx"], pointer_array(j["inp"]), j["nIn"],
                                     ctypes.c_void_p(j["out"] or None), None)
    if kind == "rs":
        return L.rr_rs_multi_reduce(r, dt, op, j["pass_"], j["idx"], pointer_array(j["inp"]), j["nIn"],
                                    ctypes.c_void_p(j["out"] or None), None)
    f = L.rr_a2a_pack if kind == "pack" else L.rr_a2a_unpack
    return f(r, dt, j["helper"], pointer_array(j["inp"]), pointer_array(j["out"]), None)


def call_many(L, kind, coll, dt, op, jobs):
    keep = []
    if kind == "helper":
        arr = (_HelperJob * len(jobs))()
        for a, j in zip(arr, jobs):
            a.relay, a.helper, a.nSlots = j["relay"], j["helper"], j["nSlots"]
            for s in range(4):
                a.slots[s] = j["slots"][s] or None
            a.out = j["out"] or None
        return L.rr_helper_reduce_many(coll, dt, op, arr, len(jobs), None)
    if kind == "active":
        arr = (_ActiveJob * len(jobs))()
        for a, j in zip(arr, jobs):
            a.relay, a.activeIdx, a.nIn = j["relay"], j["activeIdx"], j["nIn"]
            for s in range(4):
                a.inp[s] = j["inp"][s] or None
            a.out = j["out"] or None
        return L.rr_active_add_scale_many(coll, dt, op, arr, len(jobs), None)
    if kind == "rs":
        arr = (_RsJob * len(jobs))()
        for a, j in zip(arr, jobs):
            ins = pointer_array(j["inp"])
            keep.append(ins)
            a.relay, a.pass_, a.idx, a.nIn = j["relay"], j["pass_"], j["idx"], j["nIn"]
            a.inp = ctypes.cast(ins, ctypes.POINTER(ctypes.c_void_p))
            a.out = j["out"] or None
        return L.rr_rs_multi_reduce_many(dt, op, arr, len(jobs), None)
    arr = (_A2AJob * len(jobs))()
    for a, j in zip(arr, jobs):
        ins, outs = pointer_array(j["inp"]), pointer_array(j["out"])
        keep += [ins, outs]
        a.relay, a.helper = j["relay"], j["helper"]
        a.inp = ctypes.cast(ins, ctypes.POINTER(ctypes.c_void_p))
        a.out = ctypes.cast(outs, ctypes.POINTER(ctypes.c_void_p))
    f = L.rr_a2a_pack_many if kind == "pack" else L.rr_a2a_unpack_many
    return f(dt, arr, len(jobs), None)


def run_case(sim, seed):
    rng = np.random.default_rng([7100, seed])
    sim.reset()
    L = sim.L
    kind = KINDS[seed % len(KINDS)]
    dt = int(rng.choice([F32, BF16]))
    op = int(rng.choice([0, 1])) if rng.random() > 0.03 else 2
    case = Case(sim, rng, 4 if dt == F32 else 2)
    jobs, colls, faulty = [], [], []
    for _ in range(int(rng.integers(1, 6))):
        case.faulty = op == 2
        coll, j = draw_job(rng, case, kind, dt)
        jobs.append(j)
        colls.append(coll)
        faulty.append(case.faulty)
    # a batch shares one collective; a job drawn for another one is a fault
    coll = colls[0]
    for i, c in enumerate(colls):
        faulty[i] = faulty[i] or c != coll
    where = f"seed {seed} kind {kind} dt {dt} op {op} coll {coll}"

    start = case.snapshot()
    statuses, messages = [], []
    for i, j in enumerate(jobs):
        before = case.snapshot()
        st = call_single(L, kind, coll, dt, op, j)
        msg = L.rr_last_error().decode()
        assert st in (OK, EINVAL, EALIAS), f"{where} job {i}: status {st}"
        sim.check()
        if st != OK:
            assert msg, f"{where} job {i}: status {st} with no message"
            assert case.same_as(before), f"{where} job {i}: a rejected call wrote memory"
        if not faulty[i]:
            assert st == OK, f"{where} job {i}: a job with no fault was rejected: {msg}"
        statuses.append(st)
        messages.append(msg)
    untouched = [i for i in range(len(case.bufs)) if i not in case.out_targets]
    assert case.same_as(start, untouched), f"{where}: a buffer no output points into changed"
    after_singles = case.snapshot()

    case.restore(start)
    st = call_many(L, kind, coll, dt, op, jobs)
    msg = L.rr_last_error().decode()
    sim.check()
    bad = [i for i, x in enumerate(statuses) if x != OK]
    by_args = [i for i in bad if messages[i] not in WHOLE_CALL_ALIAS]
    if by_args:
        j = by_args[0]
        assert st == statuses[j] and msg == f"job {j}: {messages[j]}", (where, st, msg, messages[j])
    elif bad:
        m = re.fullmatch(r"job (\d+): (.*)", msg)
        assert st == EALIAS and m, (where, st, msg)
        assert int(m[1]) in bad and m[2] == messages[int(m[1])], (where, msg, messages)
    if bad:
        assert case.same_as(start), f"{where}: a rejected batch wrote memory"
    else:
        assert st == OK, (where, st, msg)
        assert case.same_as(after_singles), f"{where}: the batch wrote other bytes than its jobs"
    return statuses


@pytest.mark.parametrize("block", range(8))
def test_fuzzed_arguments_keep_the_contract(sims, block):
    seen = {OK: 0, EINVAL: 0, EALIAS: 0}
    for seed in range(block * 80, block * 80 + 80):
        for st in run_case(sims[seed % 7 == 3], seed):
            seen[st] += 1
    # the draws reach every outcome in every block
    assert all(v > 0 for v in seen.values()), seen
