"""Whole-node relay schedules, simulated on one GPU.

A schedule describes one fused sharded-relay collective on an 8-GPU node
(every sparse group at once): for each serialized group, the point-to-point
hops (source slice -> destination slice, each on one link in one direction)
and then the local steps every rank runs before the next group.  Every rank's
buffers live in this GPU's HBM; ``run_on_gpu`` moves each hop with a device
copy and runs each rank's local steps through the relay library (one batched
call per rank and role, as that rank would issue it).  The same description
feeds the per-link cost model: ``link_groups`` lists (src, dst, elements) per
group.

Schedules (pull request "Link-balance the sharded relay schedules (up to 3.2x
vs NCCL)", summary sections 1, 2, 4 and 6, and the reverted all-to-all
paragraph; layouts as in include/rr.h):

* ``a2_allreduce``: two groups, numChunks = H+2; helpers reduce at the helper
  and return one chunk to both actives; the direct region travels as dirA in
  group 1 and dirB in group 2.
* ``a2_reduce_scatter`` / ``a2_all_to_all`` / ``a2_all_gather``: the same
  two-group shape with passthrough helpers (slots forwarded unsummed).
* ``a4_allreduce``: offload ``permille`` of the buffer through the helpers
  (4 -> 1 at the helper, broadcast back), the rest reduce-scattered then
  all-gathered over the intra-group links.
* ``a4_reduce_scatter``: flat reduce-at-helper; the helper scratch keeps a
  separate chunk for every owner and every source other than that owner; the
  direct region travels half in each of the two groups.
* ``a2_allreduce_small``: the small-message path of summary section 3 -- one
  full exchange of the buffer (or, for comparison, a reduce-scatter swap then
  an all-gather swap), then the add + scale over the whole buffer.
* ``a4_all_gather``: summary section 5 -- two balanced groups: offload chunks
  reach the helpers in the first group and every other active in the second,
  so each cross link moves A-1 times more in the second group; sending one
  part of the direct region in the first group for every A-1 parts in the
  second evens the groups out.
* ``a4_all_to_all``: helper offload with per-destination coalescing; the
  gather (pack) and scatter (unpack) kernels stand in for the source->helper
  and helper->destination hops (the one-GPU collapse: the pack reads the
  sources, the unpack writes the destinations).

A=2 sparse groups are ranks {0,1},{2,3},{4,5},{6,7}; A=4 groups {0..3},{4..7}
(the consecutive layout of the 4-active allreduce commit).  The helpers of a
group are the other ranks in ascending order; helper index k is the position
in that list.
"""
from dataclasses import dataclass, field

from . import (ALLREDUCE, ALLTOALL, BF16, F32, REDUCE_SCATTER, Relay, rr_a2a_pack_many,
               rr_a2a_unpack_many, rr_active_add_scale_many, rr_geometry, rr_helper_reduce_many,
               rr_phase_reduce_many,
               rr_rs_multi_reduce_many)

NODE = 8


@dataclass(frozen=True)
class Ref:
    """Elements [off, off+n) of buffer ``buf`` on rank ``rank``."""
    rank: int
    buf: str
    off: int
    n: int


@dataclass
class Hop:
    src: Ref
    dst: Ref
    via: str = ""   # "" = a device copy; else moved by that local step kind


@dataclass
class Step:
    rank: int
    kind: str       # helper_reduce | active | rs_pass1 | rs_pass2 | a2a_pack | a2a_unpack | copy
    relay: Relay = None
    coll: int = ALLREDUCE
    idx: int = 0
    ins: list = field(default_factory=list)
    outs: list = field(default_factory=list)


@dataclass
class Group:
    hops: list = field(default_factory=list)
    after: list = field(default_factory=list)


@dataclass
class Schedule:
    name: str
    A: int
    dtype: int
    op: int
    buffers: dict              # (rank, buf) -> elements
    groups: list
    in_elems: int
    out_elems: int

    def link_groups(self):
        """[(src_rank, dst_rank, elements), ...] per group, for the cost model."""
        return [[(h.src.rank, h.dst.rank, h.src.n) for h in g.hops if h.src.rank != h.dst.rank]
                for g in self.groups]


def sparse_groups(A):
    return [list(range(g * A, (g + 1) * A)) for g in range(NODE // A)]


def helpers_of(act):
    return [r for r in range(NODE) if r not in act]


def _hop(hops, s, d, via=""):
    if s.n:
        assert s.n == d.n
        hops.append(Hop(s, d, via))


# --------------------------------------------------------------------------
# A = 2
# --------------------------------------------------------------------------

def _a2(kind, count, dtype, op, H, numChunks):
    """The two-group A=2 schedule shared by the four collectives (summary
    section 1): helper k takes chunk k of what each active sends towards the
    other; the direct region goes as dirA in group 1 and dirB in group 2.

    For active i of a group, ``send`` is the offset in its input of the data
    meant for the other active, and ``land(j)`` where the other active's data
    lands on active j (buffer, base offset)."""
    n = count
    if kind == "allreduce":
        send, land = (lambda i: 0), (lambda j: ("recv", 0))
        in_elems, out_elems = n, n
    elif kind == "reduce_scatter":       # block b of an input is destined for active b
        send, land = (lambda i: (1 - i) * n), (lambda j: ("recv", 0))
        in_elems, out_elems = 2 * n, n
    elif kind == "all_to_all":           # segment d of an input goes to active d
        send, land = (lambda i: (1 - i) * n), (lambda j: ("out", (1 - j) * n))
        in_elems, out_elems = 2 * n, 2 * n
    elif kind == "all_gather":           # output slot s holds active s's input
        send, land = (lambda i: 0), (lambda j: ("out", (1 - j) * n))
        in_elems, out_elems = n, 2 * n
    else:
        raise ValueError(kind)
    coll = REDUCE_SCATTER if kind == "reduce_scatter" else ALLREDUCE
    relay = Relay(2, H, numChunks, 0, n)
    g = rr_geometry(relay, coll, dtype)
    c = g["chunk"]
    bufs = {}
    for r in range(NODE):
        bufs[(r, "in")], bufs[(r, "out")] = in_elems, out_elems
        if kind in ("allreduce", "reduce_scatter"):
            bufs[(r, "recv")] = n
    g1, g2 = Group(), Group()
    for gi, act in enumerate(sparse_groups(2)):
        hs = f"hs{gi}"
        for k, h in enumerate(helpers_of(act)):
            if not c:
                break
            bufs[(h, hs)] = 2 * c
            for i, a in enumerate(act):
                _hop(g1.hops, Ref(a, "in", send(i) + k * c, c), Ref(h, hs, i * c, c))
            if kind == "allreduce":
                # reduce at the helper, return the one reduced chunk to both
                g1.after.append(Step(h, "helper_reduce", relay, coll, k,
                                     [Ref(h, hs, 0, c), Ref(h, hs, c, c)], [Ref(h, hs, 0, c)]))
                for a in act:
                    _hop(g2.hops, Ref(h, hs, 0, c), Ref(a, "out", k * c, c))
            else:
                # passthrough: slot i goes, unsummed, to the other active
                for i in range(2):
                    buf, base = land(1 - i)
                    _hop(g2.hops, Ref(h, hs, i * c, c), Ref(act[1 - i], buf, base + k * c, c))
        for grp, off, m in ((g1, g["dirA_off"], g["dirA_len"]), (g2, g["dirB_off"], g["dirB_len"])):
            for i, a in enumerate(act):
                buf, base = land(1 - i)
                _hop(grp.hops, Ref(a, "in", send(i) + off, m), Ref(act[1 - i], buf, base + off, m))
        for i, a in enumerate(act):
            if kind == "allreduce":
                ins = [Ref(a, "in", 0, n), Ref(a, "recv", 0, n)]
                g2.after.append(Step(a, "active", relay, coll, i, ins if i == 0 else ins[::-1],
                                     [Ref(a, "out", 0, n)]))
            elif kind == "reduce_scatter":
                ins = [Ref(a, "in", i * n, n), Ref(a, "recv", 0, n)]
                g2.after.append(Step(a, "active", relay, coll, i, ins if i == 0 else ins[::-1],
                                     [Ref(a, "out", 0, n)]))
            else:                        # the rank's own segment / slot stays local
                src_off = i * n if kind == "all_to_all" else 0
                g1.after.append(Step(a, "copy", ins=[Ref(a, "in", src_off, n)], outs=[Ref(a, "out", i * n, n)]))
    return Schedule(f"a2_{kind}", 2, dtype, op, bufs, [g1, g2], in_elems, out_elems)


def a2_allreduce(count, dtype=BF16, op=1, H=6, numChunks=8):
    return _a2("allreduce", count, dtype, op, H, numChunks)


def a2_reduce_scatter(R, dtype=BF16, op=1, H=6, numChunks=8):
    return _a2("reduce_scatter", R, dtype, op, H, numChunks)


def a2_all_to_all(seg, dtype=BF16, H=6, numChunks=8):
    return _a2("all_to_all", seg, dtype, 0, H, numChunks)


def a2_all_gather(S, dtype=BF16, H=6, numChunks=8):
    return _a2("all_gather", S, dtype, 0, H, numChunks)


def a2_allreduce_small(count, dtype=BF16, op=1, H=6, numChunks=8, exchange="full"):
    """exchange = "full": one group, each active sends its whole buffer to the
    other and both reduce all of it; "rs_ag": a reduce-scatter swap of halves,
    the half reduced by its owner, then an all-gather swap (two groups)."""
    relay = Relay(2, H, numChunks, 0, count)
    bufs = {}
    for r in range(NODE):
        bufs[(r, "in")] = bufs[(r, "out")] = bufs[(r, "recv")] = count
    groups = []
    if exchange == "full":
        g1 = Group()
        for act in sparse_groups(2):
            for i, a in enumerate(act):
                _hop(g1.hops, Ref(a, "in", 0, count), Ref(act[1 - i], "recv", 0, count))
            for i, a in enumerate(act):
                # the whole buffer as one block: the reduce-scatter form of the
                # two-input add + scale (it covers every element)
                ins = [Ref(a, "in", 0, count), Ref(a, "recv", 0, count)]
                g1.after.append(Step(a, "active", relay, REDUCE_SCATTER, i, ins if i == 0 else ins[::-1],
                                     [Ref(a, "out", 0, count)]))
        groups = [g1]
    elif exchange == "rs_ag":
        half = count // 2
        part = [(0, half), (half, count - half)]          # active i owns part i
        g1, g2 = Group(), Group()
        for act in sparse_groups(2):
            for i, a in enumerate(act):
                lo, n = part[1 - i]
                _hop(g1.hops, Ref(a, "in", lo, n), Ref(act[1 - i], "recv", lo, n))
                _hop(g2.hops, Ref(a, "out", part[i][0], part[i][1]), Ref(act[1 - i], "out", part[i][0], part[i][1]))
            for i, a in enumerate(act):
                lo, n = part[i]
                rel = Relay(2, H, numChunks, 0, n)
                ins = [Ref(a, "in", lo, n), Ref(a, "recv", lo, n)]
                g1.after.append(Step(a, "active", rel, REDUCE_SCATTER, i, ins if i == 0 else ins[::-1],
                                     [Ref(a, "out", lo, n)]))
        groups = [g1, g2]
    else:
        raise ValueError(exchange)
    return Schedule(f"a2_allreduce_small_{exchange}", 2, dtype, op, bufs, groups, count, count)


# --------------------------------------------------------------------------
# A = 4
# --------------------------------------------------------------------------

def a4_all_gather(S, dtype=BF16, H=4, numChunks=8):
    """Offload chunk = align_down(S/numChunks, 128) per helper; active a's
    slice k goes to helper k in group 1 and from there to the other actives in
    group 2.  The direct remainder is sent a quarter in group 1 and three
    quarters in group 2.  Output slot a of every active holds active a's
    input."""
    A = 4
    c = (S // numChunks) // 128 * 128
    if H * c > S:
        raise ValueError("offload chunks exceed the send count")
    d0 = H * c
    d1 = (S - d0) // A                  # the 1 : (A-1) split of the direct region
    bufs = {}
    for r in range(NODE):
        bufs[(r, "in")] = S
        bufs[(r, "out")] = A * S
    g1, g2 = Group(), Group()
    for gi, act in enumerate(sparse_groups(A)):
        hs = f"hs{gi}"
        for k, h in enumerate(helpers_of(act)):
            if not c:
                break
            bufs[(h, hs)] = A * c       # one chunk per source: the A-slot helper buffer
            for ai, a in enumerate(act):
                _hop(g1.hops, Ref(a, "in", k * c, c), Ref(h, hs, ai * c, c))
                for b in act:
                    if b != a:
                        _hop(g2.hops, Ref(h, hs, ai * c, c), Ref(b, "out", ai * S + k * c, c))
        for ai, a in enumerate(act):
            g1.after.append(Step(a, "copy", ins=[Ref(a, "in", 0, S)], outs=[Ref(a, "out", ai * S, S)]))
            for b in act:
                if b != a:
                    _hop(g1.hops, Ref(a, "in", d0, d1), Ref(b, "out", ai * S + d0, d1))
                    _hop(g2.hops, Ref(a, "in", d0 + d1, S - d0 - d1), Ref(b, "out", ai * S + d0 + d1, S - d0 - d1))
    return Schedule("a4_all_gather", A, dtype, 0, bufs, [g1, g2], S, A * S)


# --------------------------------------------------------------------------

def a4_allreduce(count, dtype=BF16, op=1, H=4, permille=500):
    A = 4
    relay = Relay(A, H, 0, permille, count)
    g = rr_geometry(relay, ALLREDUCE, dtype)
    c = g["chunk"]
    bufs = {}
    for r in range(NODE):
        bufs[(r, "in")] = bufs[(r, "out")] = count
    g1, g2 = Group(), Group()

    def dslice(i):
        lo = g["direct_off"] + i * g["dslice"]
        return lo, (g["dslice"] if i < A - 1 else g["direct_off"] + g["direct_len"] - lo)

    for gi, act in enumerate(sparse_groups(A)):
        hs = f"hs{gi}"
        for k, h in enumerate(helpers_of(act)):
            if not c:
                break
            bufs[(h, hs)] = (A + 1) * c
            for i, a in enumerate(act):
                _hop(g1.hops, Ref(a, "in", k * c, c), Ref(h, hs, i * c, c))
                _hop(g2.hops, Ref(h, hs, A * c, c), Ref(a, "out", k * c, c))
            g1.after.append(Step(h, "helper_reduce", relay, ALLREDUCE, k,
                                 [Ref(h, hs, i * c, c) for i in range(A)], [Ref(h, hs, A * c, c)]))
        for i, b in enumerate(act):
            lo, n = dslice(i)
            for j, a in enumerate(act):
                if a != b:
                    bufs[(b, f"peer{j}")] = count
                    _hop(g1.hops, Ref(a, "in", lo, n), Ref(b, f"peer{j}", lo, n))     # reduce-scatter
                    _hop(g2.hops, Ref(b, "out", lo, n), Ref(a, "out", lo, n))         # all-gather
            ins = [Ref(b, "in", 0, count) if j == i else Ref(b, f"peer{j}", 0, count) for j in range(A)]
            g1.after.append(Step(b, "active", relay, ALLREDUCE, i, ins, [Ref(b, "out", 0, count)]))
    return Schedule("a4_allreduce", A, dtype, op, bufs, [g1, g2], count, count)


def a4_reduce_scatter(R, dtype=BF16, op=0, H=4, permille=500):
    A = 4
    relay = Relay(A, H, 0, permille, R)
    g = rr_geometry(relay, REDUCE_SCATTER, dtype)
    c = g["chunk"]
    d0 = g["direct_off"]
    half = (R - d0) // 2
    bufs = {}
    for r in range(NODE):
        bufs[(r, "in")] = A * R
        bufs[(r, "out")] = R
        if c:
            bufs[(r, "reds")] = H * c
    g1, g2 = Group(), Group()
    for gi, act in enumerate(sparse_groups(A)):
        hs = f"hs{gi}"
        for k, h in enumerate(helpers_of(act)):
            if not c:
                break
            bufs[(h, hs)] = 2 * R
            for oi, o in enumerate(act):
                srcs = [s for s in act if s != o]
                for j, s in enumerate(srcs):
                    _hop(g1.hops, Ref(s, "in", oi * R + k * c, c), Ref(h, hs, (oi * (A - 1) + j) * c, c))
                _hop(g2.hops, Ref(h, hs, A * (A - 1) * c + oi * c, c), Ref(o, "reds", k * c, c))
            g1.after.append(Step(h, "rs_pass1", relay, REDUCE_SCATTER, k, [Ref(h, hs, 0, A * (A - 1) * c)],
                                 [Ref(h, hs, A * (A - 1) * c, A * c)]))
        for oi, o in enumerate(act):
            for si, s in enumerate(act):
                if s == o:
                    continue
                bufs[(o, f"peer{si}")] = R
                _hop(g1.hops, Ref(s, "in", oi * R + d0, half), Ref(o, f"peer{si}", d0, half))
                _hop(g2.hops, Ref(s, "in", oi * R + d0 + half, R - d0 - half),
                     Ref(o, f"peer{si}", d0 + half, R - d0 - half))
            blocks = [Ref(o, "in", oi * R, R) if si == oi else Ref(o, f"peer{si}", 0, R) for si in range(A)]
            reds = [Ref(o, "reds", k * c, c) for k in range(H)] if c else [blocks[0]] * H
            g2.after.append(Step(o, "rs_pass2", relay, REDUCE_SCATTER, oi, blocks + reds, [Ref(o, "out", 0, R)]))
    return Schedule("a4_reduce_scatter", A, dtype, op, bufs, [g1, g2], A * R, R)


def a4_all_to_all(seg, dtype=BF16, H=4, numChunks=5):
    A = 4
    relay = Relay(A, H, numChunks, 0, seg)
    g = rr_geometry(relay, ALLTOALL, dtype)
    c = g["chunk"]
    d0 = g["direct_off"]
    half = (seg - d0) // 2
    bufs = {}
    for r in range(NODE):
        bufs[(r, "in")] = bufs[(r, "out")] = A * seg
    g1, g2 = Group(), Group()
    for gi, act in enumerate(sparse_groups(A)):
        for k, h in enumerate(helpers_of(act)):
            if not c:
                break
            pd = [f"pd{gi}_{di}" for di in range(A)]
            for di, d in enumerate(act):
                bufs[(h, pd[di])] = (A - 1) * c
                for j, s in enumerate(s for s in act if s != d):
                    _hop(g1.hops, Ref(s, "in", di * seg + k * c, c), Ref(h, pd[di], j * c, c), via="a2a_pack")
                    si = act.index(s)
                    _hop(g2.hops, Ref(h, pd[di], j * c, c), Ref(d, "out", si * seg + k * c, c), via="a2a_unpack")
            g1.after.append(Step(h, "a2a_pack", relay, ALLTOALL, k, [Ref(s, "in", 0, A * seg) for s in act],
                                 [Ref(h, pd[di], 0, (A - 1) * c) for di in range(A)]))
            g2.after.append(Step(h, "a2a_unpack", relay, ALLTOALL, k, [Ref(h, pd[di], 0, (A - 1) * c) for di in range(A)],
                                 [Ref(d, "out", 0, A * seg) for d in act]))
        for di, d in enumerate(act):
            for si, s in enumerate(act):
                if s == d:
                    g1.after.append(Step(d, "copy", ins=[Ref(d, "in", di * seg, seg)],
                                         outs=[Ref(d, "out", di * seg, seg)]))
                    continue
                _hop(g1.hops, Ref(s, "in", di * seg + d0, half), Ref(d, "out", si * seg + d0, half))
                _hop(g2.hops, Ref(s, "in", di * seg + d0 + half, seg - d0 - half),
                     Ref(d, "out", si * seg + d0 + half, seg - d0 - half))
    return Schedule("a4_all_to_all", A, dtype, 0, bufs, [g1, g2], A * seg, A * seg)


# --------------------------------------------------------------------------
# execution on one GPU
# --------------------------------------------------------------------------

def run_on_gpu(s, inputs, stream=None):
    """Execute schedule ``s`` with every rank's buffers in this GPU's HBM.
    ``inputs[r]`` is rank r's input tensor; returns the ranks' output tensors."""
    import torch
    dev = inputs[0].device
    tdt = inputs[0].dtype
    buf = {key: torch.zeros(n, dtype=tdt, device=dev) for key, n in s.buffers.items()}
    for r in range(NODE):
        buf[(r, "in")].copy_(inputs[r])

    def view(ref):
        return buf[(ref.rank, ref.buf)][ref.off:ref.off + ref.n]

    def full(ref):       # kernels take buffers from the slice start to the buffer end
        return buf[(ref.rank, ref.buf)][ref.off:]

    for grp in s.groups:
        for h in grp.hops:
            if not h.via:
                view(h.dst).copy_(view(h.src))
        by_rank_kind = {}
        for st in grp.after:
            by_rank_kind.setdefault((st.rank, st.kind), []).append(st)
        # a rank's helper and active reductions of one phase (the fused A=4
        # allreduce: its position slice for the other group and its own direct
        # slice) go out as one call
        for rank in {r for r, _ in by_rank_kind}:
            hs, acts = by_rank_kind.get((rank, "helper_reduce")), by_rank_kind.get((rank, "active"))
            if hs and acts and len({st.coll for st in hs + acts}) == 1:
                by_rank_kind[(rank, "phase")] = (hs, acts)
                del by_rank_kind[(rank, "helper_reduce")], by_rank_kind[(rank, "active")]
        for (rank, kind), steps in sorted(by_rank_kind.items(), key=lambda kv: kv[0]):
            if kind == "copy":
                for st in steps:
                    view(st.outs[0]).copy_(view(st.ins[0]))
            elif kind == "phase":
                hs, acts = steps
                rr_phase_reduce_many(hs[0].coll, s.dtype, s.op,
                                     [(st.relay, st.idx, [full(x) for x in st.ins], full(st.outs[0]))
                                      for st in hs],
                                     [(st.relay, st.idx, [full(x) for x in st.ins], full(st.outs[0]))
                                      for st in acts], stream)
            elif kind == "helper_reduce":
                rr_helper_reduce_many(steps[0].coll, s.dtype, s.op,
                                      [(st.relay, st.idx, [full(x) for x in st.ins], full(st.outs[0]))
                                       for st in steps], stream)
            elif kind == "active":
                rr_active_add_scale_many(steps[0].coll, s.dtype, s.op,
                                         [(st.relay, st.idx, [full(x) for x in st.ins], full(st.outs[0]))
                                          for st in steps], stream)
            elif kind in ("rs_pass1", "rs_pass2"):
                p = 1 if kind == "rs_pass1" else 2
                rr_rs_multi_reduce_many(s.dtype, s.op,
                                        [(st.relay, p, st.idx, [full(x) for x in st.ins], full(st.outs[0]))
                                         for st in steps], stream)
            elif kind == "a2a_pack":
                rr_a2a_pack_many(s.dtype, [(st.relay, st.idx, [full(x) for x in st.ins],
                                            [full(x) for x in st.outs]) for st in steps], stream)
            elif kind == "a2a_unpack":
                rr_a2a_unpack_many(s.dtype, [(st.relay, st.idx, [full(x) for x in st.ins],
                                              [full(x) for x in st.outs]) for st in steps], stream)
            else:
                raise ValueError(f"unknown step kind {kind}")
    return [buf[(r, "out")] for r in range(NODE)]
