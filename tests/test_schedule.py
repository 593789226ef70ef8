"""Whole-node relay schedules (pack_rr_helper_amd/schedule.py): the same
description is (a) executed on the host with the oracle's step functions and
checked against the plain collectives, (b) tallied by the link-cost model and
checked against the closed forms of the PR summary, and (c) executed on the
GPU through the relay library and checked against (a) bit for bit."""
from fractions import Fraction

import numpy as np
import pytest

import oracle as orc
from oracle import costmodel as cm
from pack_rr_helper_amd import schedule as S
from pack_rr_helper_amd import synth
from tests.sched_cpu import run_on_cpu

BF16, SUM, AVG = 1, 0, 1


def ords(b):
    b = b.astype(np.int32)
    return np.where(b & 0x8000, 0x8000 - (b & 0x7FFF) - 1, b + 0x8000)


def bf16_vals(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_rs4_bound(s, xs, r, got):
    """Owner r's A=4 reduce-scatter output within the error of its steps: on
    an offload slice the helper rounds the fp32 sum of the 3 other sources to
    bf16 (|err| <= u*|s|), the owner adds in fp32 and rounds once more; the
    direct region is one fp32 fold of 4 and one rounding.  u = 2^-8, e = 2^-24."""
    A, R = 4, s.out_elems
    act = next(g for g in S.sparse_groups(A) if r in g)
    o = act.index(r)
    vals = [bf16_vals(xs[a][o * R:(o + 1) * R]) for a in act]
    exact = sum(vals)
    other = sum(np.abs(v) for i, v in enumerate(vals) if i != o)
    u, e = 2.0 ** -8, 2.0 ** -24
    S_ = np.abs(exact - vals[o]) + 2 * e * other
    g = bf16_vals(got)
    bound = u / (1 - u) * np.abs(g) + e * (np.abs(vals[o]) + (1 + u) * S_) + u * S_ + 2 * e * other
    assert np.all(np.abs(g - exact) <= bound * (1 + 1e-9) + 3 * e * sum(np.abs(v) for v in vals))


def inputs(n, seed, ints=False):
    if ints:
        return [synth.as_bf16_bits(synth.small_ints(n, 16, seed, r)) for r in range(8)]
    return [synth.as_bf16_bits(synth.normal(n, seed, r)) for r in range(8)]


def expected(s, xs):
    """The plain collective each rank should end with."""
    outs = []
    for r in range(8):
        act = next(g for g in S.sparse_groups(s.A) if r in g)
        i = act.index(r)
        peers = [xs[a] for a in act]
        if s.name.endswith("allreduce"):
            outs.append(orc.plain_sum(BF16, s.op, peers, 0, s.in_elems))
        elif s.name.endswith("reduce_scatter"):
            outs.append(orc.plain_sum(BF16, s.op, peers, i * s.out_elems, s.out_elems))
        elif s.name.startswith("a2_allreduce_small"):
            outs.append(orc.plain_sum(BF16, s.op, peers, 0, s.in_elems))
        elif s.name.endswith("all_to_all"):
            outs.append(orc.plain_all_to_all(2, s.A, s.in_elems // s.A, i, peers).view(np.uint16))
        else:
            outs.append(np.concatenate(peers))
    return outs


CASES = [
    ("a2_allreduce", lambda n: S.a2_allreduce(n), 8 * 128 * 6 + 77),
    ("a2_allreduce_zero_chunk", lambda n: S.a2_allreduce(n), 700),
    ("a2_reduce_scatter", lambda n: S.a2_reduce_scatter(n // 2), 2 * (8 * 128 * 5 + 9)),
    ("a2_all_to_all", lambda n: S.a2_all_to_all(n // 2), 2 * (8 * 128 * 4 + 5)),
    ("a2_all_gather", lambda n: S.a2_all_gather(n), 8 * 128 * 3 + 11),
    ("a4_allreduce", lambda n: S.a4_allreduce(n), 2 ** 20 + 4 * 128 * 5 + 6),
    ("a4_allreduce_floor", lambda n: S.a4_allreduce(n), 5000),
    ("a4_reduce_scatter", lambda n: S.a4_reduce_scatter(n // 4, op=SUM), 4 * (8 * 128 * 4 + 24)),
    ("a4_all_to_all", lambda n: S.a4_all_to_all(n // 4), 4 * (5 * 128 * 6 + 3)),
    ("a2_allreduce_small_full", lambda n: S.a2_allreduce_small(n), 3000),
    ("a2_allreduce_small_rs_ag", lambda n: S.a2_allreduce_small(n, exchange="rs_ag"), 3001),
    ("a4_all_gather", lambda n: S.a4_all_gather(n), 8 * 128 * 5 + 19),
]


@pytest.mark.parametrize("name,mk,n", CASES, ids=[c[0] for c in CASES])
def test_schedule_on_cpu_is_the_plain_collective(name, mk, n):
    s = mk(n)
    for ints in (True, False):
        xs = inputs(s.in_elems, 70, ints)
        got = run_on_cpu(s, xs)
        exp = expected(s, xs)
        for r in range(8):
            if ints or not ("allreduce" in s.name or s.name.endswith("reduce_scatter")):
                assert np.array_equal(got[r], exp[r]), (name, r)
            elif s.name == "a4_reduce_scatter":
                assert_rs4_bound(s, xs, r, got[r])
            else:
                assert np.max(np.abs(ords(got[r]) - ords(exp[r]))) <= 1, (name, r)


def cost(s):
    return cm.link_cost([[(a, b, Fraction(m)) for a, b, m in g] for g in s.link_groups()])


def test_a2_schedules_cost_a_quarter_of_the_count():
    n = 8 * 128 * 1000
    for s in (S.a2_allreduce(n), S.a2_reduce_scatter(n), S.a2_all_to_all(n), S.a2_all_gather(n)):
        assert cost(s) == Fraction(n, 4), s.name
        # every (link, direction) carries exactly one chunk in each group
        for g in s.link_groups():
            load = {}
            for a, b, m in g:
                load[(a, b)] = load.get((a, b), 0) + m
            assert set(load.values()) == {n // 8}


def test_a4_allreduce_cost_matches_the_critical_path_formula():
    n = 4 * 128 * 1000 * 8
    for pm in (500, 780):
        s = S.a4_allreduce(n, permille=pm)
        p = Fraction(pm, 1000)
        assert cost(s) == 2 * max(p, 1 - p) * n / 4


def test_a4_all_to_all_cost_at_the_model_optimum():
    # offload 0.4 of every segment: numChunks = 10 gives chunk = seg/10 per helper
    seg = 10 * 128 * 50
    s = S.a4_all_to_all(seg, numChunks=10)
    assert cost(s) == Fraction(3, 5) * seg
    assert cost(S.a4_all_to_all(seg, numChunks=5)) > seg      # 0.8 offload loses to direct


def test_zero_chunk_schedule_has_no_helper_traffic():
    s = S.a2_allreduce(700)
    helpers = {(a, b) for g in s.link_groups() for a, b, m in g if (a // 2) != (b // 2)}
    assert not helpers


@pytest.mark.gpu
@pytest.mark.parametrize("name,mk,n", CASES, ids=[c[0] for c in CASES])
def test_schedule_on_gpu_matches_the_host_execution(name, mk, n):
    import torch
    print("[gpu-case] schedule", name, n, flush=True)
    s = mk(n)
    xs = inputs(s.in_elems, 71)
    dev = [synth.to_device(x, BF16) for x in xs]
    outs = S.run_on_gpu(s, dev)
    torch.cuda.synchronize()
    ref = run_on_cpu(s, xs)
    for r in range(8):
        assert np.array_equal(synth.to_host(outs[r]), ref[r]), (name, r)


def test_small_message_single_exchange_beats_rs_plus_ag():
    """Summary section 3: both move the whole buffer per link direction, but
    the reduce-scatter + all-gather form pays two group boundaries."""
    n = 4096
    full, rsag = S.a2_allreduce_small(n), S.a2_allreduce_small(n, exchange="rs_ag")
    assert len(full.groups) == 1 and len(rsag.groups) == 2
    assert cost(full) == cost(rsag) == n
    lat = Fraction(1)
    assert cm.link_cost([[(a, b, Fraction(m)) for a, b, m in g] for g in full.link_groups()], lat) < \
        cm.link_cost([[(a, b, Fraction(m)) for a, b, m in g] for g in rsag.link_groups()], lat)


def test_a4_all_gather_two_balanced_groups():
    """Summary section 5: forwarding offload chunks in the second group loads
    each cross link A-1 times as heavily as the first group does; giving the
    second group A-1 parts of the direct region for every part sent in the
    first evens the two groups out at half the pure-direct time."""
    S_ = 8 * 128 * 400
    s = S.a4_all_gather(S_)
    g1, g2 = s.link_groups()
    def peak(g, intra):
        load = {}
        for a, b, m in g:
            if (a // 4 == b // 4) == intra:
                load[(a, b)] = load.get((a, b), 0) + m
        return max(load.values())
    assert peak(g2, False) == 3 * peak(g1, False)          # cross: forwarding carries 3 sources
    assert peak(g1, True) == peak(g1, False) and peak(g2, True) == peak(g2, False)
    direct = Fraction(S_)                                    # pure direct: one group of S per link
    assert cost(s) == direct / 2
