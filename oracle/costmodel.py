"""Per-link cost model of the sharded relay schedules -- TEST INFRASTRUCTURE ONLY.

Model (pull request "Link-balance the sharded relay schedules", Summary, "Cost
model used throughout"): every GPU pair of an 8-GPU node has exactly one link,
so each GPU has 7.  A schedule is a sequence of serialized groups; a group's
time is the largest number of elements carried by one (link, direction) in it,
and the schedule's time is the sum over its groups.

All sizes are exact ``Fraction``s of the per-rank element count, so the closed
forms the pull request prints can be compared exactly.

Schedules built here (ranks 0..7; sparse group g of A actives = ranks
[g*A, (g+1)*A); the helpers of a group are the other ranks in ascending order):
  * ``a2_three_group``: the A=2 schedule before the pull request: three
    serialized groups (scatter to the helpers, helper forwarding, and the
    direct active-to-active swap on its own), numChunks = H+1 (section 1).
  * ``a2_two_group``: the link-balanced A=2 schedule -- two groups, half of the
    direct region travelling inside each relay group; ``d`` is the direct size
    (section 1; numChunks = H+2 gives d = 2*count/8).
  * ``a4_allreduce``: A=4 allreduce with offload fraction p (section 4).
  * ``a4_all_to_all``: A=4 all-to-all helper offload with fraction p (the
    reverted experiment; the pull request prints only its 1.67x model figure,
    the two-group form here is a reconstruction that reproduces it).
  * ``nccl_allreduce_baseline`` / ``direct_all_to_all``: the baselines the
    ceilings are quoted against.
"""
from collections import defaultdict
from fractions import Fraction

NODE = 8


def link_cost(schedule, per_group=0):
    """Sum over groups of the max over (src, dst) of the elements carried,
    plus ``per_group`` for every serialized group boundary (the fixed cost
    that makes a latency-bound schedule prefer fewer groups, summary section 3)."""
    total = Fraction(0)
    for group in schedule:
        total += Fraction(per_group)
        load = defaultdict(Fraction)
        for src, dst, n in group:
            if src == dst:
                raise ValueError("a transfer needs two distinct ranks")
            if not (0 <= src < NODE and 0 <= dst < NODE):
                raise ValueError("rank out of range")
            load[(src, dst)] += Fraction(n)
        total += max(load.values(), default=Fraction(0))
    return total


def _groups(A):
    return [list(range(g * A, (g + 1) * A)) for g in range(NODE // A)]


def _helpers(actives):
    return [r for r in range(NODE) if r not in actives]


def a2_three_group(count=Fraction(1), fused=True):
    """numChunks = H+1: groups scatter, forward, direct; one chunk per link each."""
    sparse = _groups(2) if fused else _groups(2)[:1]
    H = NODE - 2
    c = Fraction(count) / (H + 1)
    g1, g2, g3 = [], [], []
    for a0, a1 in sparse:
        for h in _helpers([a0, a1]):
            g1 += [(a0, h, c), (a1, h, c)]          # scatter chunk k to helper k
            g2 += [(h, a1, c), (h, a0, c)]          # forward the other active's chunk
        g3 += [(a0, a1, c), (a1, a0, c)]            # direct exchange of chunk H
    return [g1, g2, g3]


def a2_two_group(count=Fraction(1), d=None, fused=True):
    """Two groups; relay region count - d over H helpers; the direct region d
    is split in two halves, sent with group 1 and group 2 respectively."""
    sparse = _groups(2) if fused else _groups(2)[:1]
    H = NODE - 2
    count = Fraction(count)
    d = count * 2 / (H + 2) if d is None else Fraction(d)
    c = (count - d) / H
    g1, g2 = [], []
    for a0, a1 in sparse:
        for h in _helpers([a0, a1]):
            g1 += [(a0, h, c), (a1, h, c)]          # scatter to the helper
            g2 += [(h, a0, c), (h, a1, c)]          # helper returns one chunk to each
        g1 += [(a0, a1, d / 2), (a1, a0, d / 2)]    # dirA rides with group 1
        g2 += [(a0, a1, d / 2), (a1, a0, d / 2)]    # dirB rides with group 2
    return [g1, g2]


def a4_allreduce(count=Fraction(1), p=Fraction(1, 2), fused=True):
    """Offload fraction p through H helpers, the rest reduce-scattered and
    all-gathered over the intra links; two groups."""
    A = 4
    sparse = _groups(A) if fused else _groups(A)[:1]
    H = NODE - A
    count, p = Fraction(count), Fraction(p)
    o = count * p / H                 # per-helper offload chunk
    ds = count * (1 - p) / A          # per-active direct slice
    g1, g2 = [], []
    for act in sparse:
        for a in act:
            for h in _helpers(act):
                g1.append((a, h, o))      # offload slice to its helper
                g2.append((h, a, o))      # reduced slice broadcast back
            for b in act:
                if b != a:
                    g1.append((a, b, ds))  # direct reduce-scatter
                    g2.append((a, b, ds))  # direct all-gather
    return [g1, g2]


def a4_all_to_all(seg=Fraction(1), p=Fraction(2, 5), fused=True):
    """Offload fraction p of every (source, dest) segment through the H helpers,
    the direct remainder split in halves over the two groups."""
    A = 4
    sparse = _groups(A) if fused else _groups(A)[:1]
    H = NODE - A
    seg, p = Fraction(seg), Fraction(p)
    c = seg * p / H
    dh = seg * (1 - p) / 2
    g1, g2 = [], []
    for act in sparse:
        for s in act:
            for d in act:
                if d == s:
                    continue
                for h in _helpers(act):
                    g1.append((s, h, c))   # source -> helper, slice h of segment d
                    g2.append((h, d, c))   # helper -> destination
                g1.append((s, d, dh))
                g2.append((s, d, dh))
    return [g1, g2]


def nccl_allreduce_baseline(count=Fraction(1), A=2):
    """Reduce-scatter then all-gather among the A actives over their A-1 intra
    links: each link direction carries count/A per phase."""
    count = Fraction(count)
    g = []
    for act in _groups(A):
        for a in act:
            for b in act:
                if a != b:
                    g.append((a, b, count / A))
    return [g, list(g)]


def direct_all_to_all(seg=Fraction(1), A=4):
    """Pure-direct all-to-all: every pair exchanges one segment in one group."""
    g = []
    for act in _groups(A):
        for s in act:
            for d in act:
                if s != d:
                    g.append((s, d, Fraction(seg)))
    return [g]
