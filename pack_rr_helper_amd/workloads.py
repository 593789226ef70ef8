"""One-GPU synthesis of the relay hot path: every rank's and every helper's
buffers of one sparse group live in this GPU's HBM, and each role's local
kernel is launched through the C ABI exactly as that rank would launch it.

Point-to-point hops are not local work and are not launched here; a buffer a
rank would receive is represented by the bytes it would receive:

* a helper's slots are views of the active ranks' buffers (the scatter would
  copy exactly those bytes into the helper's scratch);
* an A=2 allreduce active reads the peer's direct region from its own receive
  buffer, filled once, untimed, as the direct exchange would fill it (so the
  two actives never share an input, as on two GPUs);
* the A=2 reduce-scatter peer block is the other active's block (the
  passthrough forwards and the direct exchange deliver it unchanged);
* the A=4 reduce-scatter helper scratch is filled once, untimed, with the
  (owner, source) chunks the scatter would deliver, owner-major;
* the all-to-all pack reads the source ranks' inputs directly, and unpack
  reads the per-destination buffers pack wrote.

Message size M is the per-active-rank input in bytes (the pull request's sweep
axis), bf16 unless stated.  Workload classes expose ``calls(stream)``: one
entry per role, ``(row, kernel, algorithmic_bytes, fn)`` with ``fn()``
issuing that role's work.  ``mode`` chooses which jobs a role's call covers:

* ``"share"``: the jobs one GPU runs for that role in the fused 8-GPU call,
  as one ``*_many`` call (one launch).  A GPU is a helper for the three other
  A=2 sparse groups (three helper jobs; chunks 0-2 of the simulated group
  stand in for the other groups' chunks) and runs one job in every other
  role (its own active epilogue, owner pass, A=4 helper slice, all-to-all
  helper slice);
* ``"group"`` (the default): every job of the simulated group in one call,
  2-4x one GPU's share -- the whole group's work in one launch;
* ``"job"``: one call (one launch) per job.

Calls are prepared once (checks and marshalling), so issuing one costs a single
C call.  ``run(stream)`` issues every entry.  Algorithmic bytes count every
input element read once and every output element written once.
"""
import torch

from . import (ALLREDUCE, ALLTOALL, AVG, BF16, F32, REDUCE_SCATTER, SUM, Relay, rr_a2a_pack,
               rr_a2a_pack_many, rr_a2a_unpack, rr_a2a_unpack_many, rr_active_add_scale,
               rr_active_add_scale_many, rr_geometry, rr_helper_reduce, rr_helper_reduce_many,
               rr_phase_reduce_many, rr_rs_multi_reduce, rr_rs_multi_reduce_many)

TORCH = {F32: torch.float32, BF16: torch.bfloat16}
ESIZE = {F32: 4, BF16: 2}
# Kernel families.  The library launches a batch in one of three forms (one
# aligned segment, a uniform grid of equal segments, a tile table), each its
# own kernel symbol running the same per-tile code; timings are reported per
# family: the reduction kernels of one element type, and the copy kernels
# (aligned and realigning).
COPY = "copy"


def reduce_kernel(dtype):
    return "reduce<bf16>" if dtype == BF16 else "reduce<f32>"


MODES = ("share", "group", "job")


class _Row:
    mode = "group"

    def _set_mode(self, mode):
        if mode not in MODES:
            raise ValueError(f"mode {mode!r}: one of {MODES}")
        self.mode = mode

    def calls(self, stream=None):
        key = id(stream) if stream is not None else None
        if getattr(self, "_calls_key", object()) != key:
            self._calls = self._build(stream)
            self._calls_key = key
            self._stream_ref = stream
        return self._calls

    def run(self, stream=None):
        for _, _, _, fn in self.calls(stream):
            fn()

    def bytes_per_step(self):
        return sum(b for _, _, b, _ in self.calls())

    def _roles(self, stream, row, kernel, per_job_bytes, jobs, many, single, share=1):
        """Entries for one role: one call over every job ("group"), over the
        first ``share`` jobs -- one GPU's share ("share"), or one per job."""
        if not jobs:
            return []
        if self.mode == "job":
            return [(row, kernel, b, single(job, stream=stream, prepare=True))
                    for b, job in zip(per_job_bytes, jobs)]
        n = len(jobs) if self.mode == "group" else min(share, len(jobs))
        return [(row, kernel, sum(per_job_bytes[:n]), many(jobs[:n], stream=stream, prepare=True))]


class AR2(_Row):
    """A=2 allreduce: reduce-at-helper (summary section 2) over the H relay
    chunks and the active epilogue over the direct region (section 1)."""

    def __init__(self, xs, dtype, op=AVG, H=6, numChunks=8, mode="group"):
        self.dtype, self.op = dtype, op
        self._set_mode(mode)
        self.count = xs[0].numel()
        self.relay = Relay(2, H, numChunks, 0, self.count)
        self.g = rr_geometry(self.relay, ALLREDUCE, dtype)
        c, self.es = self.g["chunk"], ESIZE[dtype]
        self.x = xs
        self.red = [torch.empty(max(c, 1), dtype=TORCH[dtype], device=xs[0].device) for _ in range(H)]
        self.out = [torch.empty_like(xs[0]) for _ in range(2)]
        # each active's copy of the other active's direct region, as received
        lo = self.g["direct_off"]
        self.recv = [torch.zeros_like(xs[0]) for _ in range(2)]
        self.recv[0][lo:].copy_(xs[1][lo:])
        self.recv[1][lo:].copy_(xs[0][lo:])

    def _build(self, stream):
        c, es, r, k = self.g["chunk"], self.es, self.relay, reduce_kernel(self.dtype)
        hjobs = [(r, h, [self.x[0][h * c:(h + 1) * c], self.x[1][h * c:(h + 1) * c]], self.red[h])
                 for h in range(r.H)] if c else []
        ins = [[self.x[0], self.recv[0]], [self.recv[1], self.x[1]]]   # source-rank order
        ajobs = [(r, a, ins[a], self.out[a]) for a in range(2)] if self.g["direct_len"] else []
        op, dt = self.op, self.dtype
        return (self._roles(stream, "ar2_helper", k, [3 * c * es] * len(hjobs), hjobs,
                            lambda j, **kw: rr_helper_reduce_many(ALLREDUCE, dt, op, j, **kw),
                            lambda j, **kw: rr_helper_reduce(j[0], ALLREDUCE, dt, op, *j[1:], **kw),
                            share=3)
                + self._roles(stream, "ar2_active", k, [3 * self.g["direct_len"] * es] * len(ajobs), ajobs,
                              lambda j, **kw: rr_active_add_scale_many(ALLREDUCE, dt, op, j, **kw),
                              lambda j, **kw: rr_active_add_scale(j[0], ALLREDUCE, dt, op, *j[1:], **kw)))

    def deliver_returns(self):
        """The helpers' return hop (a copy per active), for whole-group checks."""
        c = self.g["chunk"]
        for k in range(self.relay.H):
            for a in range(2):
                self.out[a][k * c:(k + 1) * c].copy_(self.red[k][:c])


class RS2(_Row):
    """A=2 reduce-scatter owner epilogue: the fused add + scale of the relayed
    and direct chunks over the whole recvCount block (reduce-scatter core
    commit, phases 3 and 5).  xs[a] holds 2 blocks of R."""

    def __init__(self, xs, dtype, op=AVG, H=6, numChunks=8, in_place=False, mode="group"):
        self.dtype, self.op = dtype, op
        self._set_mode(mode)
        self.R = R = xs[0].numel() // 2
        self.relay = Relay(2, H, numChunks, 0, R)
        self.x = xs
        if in_place:
            self.own = [xs[0][:R].clone(), xs[1][R:].clone()]
            self.out = self.own
        else:
            self.own = [xs[0][:R], xs[1][R:]]
            self.out = [torch.empty(R, dtype=TORCH[dtype], device=xs[0].device) for _ in range(2)]
        # the peer block as delivered: the other active's contribution, unsummed
        self.peer = [xs[1][:R], xs[0][R:]]

    def _build(self, stream):
        r, dt, op = self.relay, self.dtype, self.op
        jobs = [(r, 0, [self.own[0], self.peer[0]], self.out[0]),
                (r, 1, [self.peer[1], self.own[1]], self.out[1])] if self.R else []
        return self._roles(stream, "rs2_owner", reduce_kernel(dt), [3 * self.R * ESIZE[dt]] * len(jobs), jobs,
                           lambda j, **kw: rr_active_add_scale_many(REDUCE_SCATTER, dt, op, j, **kw),
                           lambda j, **kw: rr_active_add_scale(j[0], REDUCE_SCATTER, dt, op, *j[1:], **kw))


class AR4(_Row):
    """A=4 allreduce at an offload fraction (summary section 4): the H helpers
    reduce their position slices 4->1, the A actives reduce their direct
    slices.  Both happen in the same phase of the fused call (a rank is an
    active of its group and a helper of the other), so with ``phase`` the
    "share" and "group" forms issue them as one rr_phase_reduce_many call
    (row "ar4_phase"; one GPU's share is helper slice 0 and active slice 0);
    without it, and in the "job" form, each role is its own call."""

    def __init__(self, xs, dtype, op=AVG, H=4, permille=500, mode="group", phase=True):
        self.dtype, self.op, self.phase = dtype, op, phase
        self._set_mode(mode)
        self.count = xs[0].numel()
        self.relay = Relay(4, H, 0, permille, self.count)
        self.g = rr_geometry(self.relay, ALLREDUCE, dtype)
        c, self.es = self.g["chunk"], ESIZE[dtype]
        self.x = xs
        self.red = [torch.empty(max(c, 1), dtype=TORCH[dtype], device=xs[0].device) for _ in range(H)]
        self.out = [torch.empty_like(xs[0]) for _ in range(4)]

    def _build(self, stream):
        c, g, es, r, dt, op = self.g["chunk"], self.g, self.es, self.relay, self.dtype, self.op
        k = reduce_kernel(dt)
        hjobs = [(r, h, [x[h * c:(h + 1) * c] for x in self.x], self.red[h]) for h in range(r.H)] if c else []
        sizes = [g["dslice"] if a < 3 else g["direct_len"] - 3 * g["dslice"] for a in range(4)]
        ajobs = [(r, a, self.x, self.out[a]) for a in range(4) if sizes[a]]
        if self.phase and self.mode != "job":
            n = None if self.mode == "group" else 1
            hj, aj = hjobs[:n], ajobs[:n]
            if not hj and not aj:
                return []
            b = 5 * es * (c * len(hj) + sum(sizes[j[1]] for j in aj))
            return [("ar4_phase", k, b,
                     rr_phase_reduce_many(ALLREDUCE, dt, op, hj, aj, stream=stream, prepare=True))]
        return (self._roles(stream, "ar4_helper", k, [5 * c * es] * len(hjobs), hjobs,
                            lambda j, **kw: rr_helper_reduce_many(ALLREDUCE, dt, op, j, **kw),
                            lambda j, **kw: rr_helper_reduce(j[0], ALLREDUCE, dt, op, *j[1:], **kw))
                + self._roles(stream, "ar4_active", k, [5 * sizes[j[1]] * es for j in ajobs], ajobs,
                              lambda j, **kw: rr_active_add_scale_many(ALLREDUCE, dt, op, j, **kw),
                              lambda j, **kw: rr_active_add_scale(j[0], ALLREDUCE, dt, op, *j[1:], **kw)))

    def deliver(self):
        """Broadcast of the helpers' chunks and the all-gather of the direct
        slices (copies), for whole-group checks."""
        c, g = self.g["chunk"], self.g
        for h in range(self.relay.H):
            for a in range(4):
                self.out[a][h * c:(h + 1) * c].copy_(self.red[h][:c])
        for a in range(4):
            lo = g["direct_off"] + a * g["dslice"]
            hi = lo + g["dslice"] if a < 3 else self.count
            for b in range(4):
                if b != a:
                    self.out[b][lo:hi].copy_(self.out[a][lo:hi])


class RS4(_Row):
    """A=4 reduce-scatter, flat reduce-at-helper (summary section 6): pass 1 at
    each helper over its (owner, source) scratch, pass 2 at each owner.
    xs[s] holds A blocks of R."""

    def __init__(self, xs, dtype, op=SUM, H=4, permille=500, mode="group"):
        A = 4
        self.dtype, self.op = dtype, op
        self._set_mode(mode)
        self.R = R = xs[0].numel() // A
        self.relay = Relay(A, H, 0, permille, R)
        self.g = rr_geometry(self.relay, REDUCE_SCATTER, dtype)
        c, self.es = self.g["chunk"], ESIZE[dtype]
        self.x = xs
        dev = xs[0].device
        # helper scratch, 2R each: A*(A-1) chunks owner-major, then A reduced chunks
        self.scratch = [torch.empty(2 * R, dtype=TORCH[dtype], device=dev) for _ in range(H)]
        for h in range(H):
            for o in range(A):
                for j, s in enumerate(s for s in range(A) if s != o):
                    dst = (o * (A - 1) + j) * c
                    self.scratch[h][dst:dst + c].copy_(xs[s][o * R + h * c:o * R + (h + 1) * c])
        self.out = [torch.empty(R, dtype=TORCH[dtype], device=dev) for _ in range(A)]
        # every helper's reduced chunks as its pass 1 returns them, staged once:
        # an owner's pass 2 reads all H of them, while one GPU's share of the
        # step runs a single helper's pass 1
        if c:
            rr_rs_multi_reduce_many(dtype, op, [(self.relay, 1, h, [self.scratch[h]],
                                                 self.scratch[h][A * (A - 1) * c:]) for h in range(H)])

    def reduced(self, h, o):
        c, A = self.g["chunk"], 4
        base = A * (A - 1) * c
        return self.scratch[h][base + o * c:base + (o + 1) * c]

    def _build(self, stream):
        A, c, R, H, es, r = 4, self.g["chunk"], self.R, self.relay.H, self.es, self.relay
        dt, op, k = self.dtype, self.op, reduce_kernel(self.dtype)
        p1 = [(r, 1, h, [self.scratch[h]], self.scratch[h][A * (A - 1) * c:]) for h in range(H)] if c else []
        p2 = []
        for o in range(A if R else 0):
            blocks = [x[o * R:(o + 1) * R] for x in self.x]
            reds = [self.reduced(h, o) if c else blocks[0] for h in range(H)]
            p2.append((r, 2, o, blocks + reds, self.out[o]))
        many = lambda j, **kw: rr_rs_multi_reduce_many(dt, op, j, **kw)
        single = lambda j, **kw: rr_rs_multi_reduce(j[0], dt, op, *j[1:], **kw)
        return (self._roles(stream, "rs4_pass1", k, [(A * (A - 1) + A) * c * es] * len(p1), p1, many, single)
                + self._roles(stream, "rs4_pass2", k, [(3 * H * c + (A + 1) * (R - H * c)) * es] * len(p2),
                              p2, many, single))


class A2A(_Row):
    """A=4 all-to-all helper coalescing (reverted all-to-all paragraph): one
    pack and one unpack per helper slice.  src[s] holds A segments of seg."""

    def __init__(self, src, dtype=BF16, H=4, numChunks=5, mode="group"):
        A = 4
        self.dtype = dtype
        self._set_mode(mode)
        self.seg = src[0].numel() // A
        self.relay = Relay(A, H, numChunks, 0, self.seg)
        self.g = rr_geometry(self.relay, ALLTOALL, dtype)
        c, self.es = self.g["chunk"], ESIZE[dtype]
        self.src = src
        dev = src[0].device
        self.packed = [[torch.empty(max((A - 1) * c, 1), dtype=src[0].dtype, device=dev) for _ in range(A)]
                       for _ in range(H)]
        self.out = [torch.zeros_like(s) for s in src]

    def _build(self, stream):
        A, c, es, r, dt = 4, self.g["chunk"], self.es, self.relay, self.dtype
        kern = COPY
        pj = [(r, h, self.src, self.packed[h]) for h in range(r.H)] if c else []
        uj = [(r, h, self.packed[h], self.out) for h in range(r.H)] if c else []
        b = 2 * A * (A - 1) * c * es
        return (self._roles(stream, "a2a_pack", kern, [b] * len(pj), pj,
                            lambda j, **kw: rr_a2a_pack_many(dt, j, **kw),
                            lambda j, **kw: rr_a2a_pack(j[0], dt, *j[1:], **kw))
                + self._roles(stream, "a2a_unpack", kern, [b] * len(uj), uj,
                              lambda j, **kw: rr_a2a_unpack_many(dt, j, **kw),
                              lambda j, **kw: rr_a2a_unpack(j[0], dt, *j[1:], **kw)))


def message_shapes(M, es=2):
    """Element counts for a per-active-rank input of M bytes."""
    return {
        "ar2_count": M // es,
        "rs2_recv": M // (2 * es),
        "ar4_count": M // es,
        "rs4_recv": M // (4 * es),
        "a2a_seg": M // (4 * es),
    }
