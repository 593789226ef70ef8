"""The link-cost evaluator against the closed forms of the PR summary
(sections 1 and 4 and the reverted all-to-all paragraph)."""
import json
import os
from fractions import Fraction as F

from oracle import costmodel as cm

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "printed_values.json")))["cost_model"]


def test_a2_three_groups_cost_three_sevenths():
    for fused in (False, True):
        t = cm.link_cost(cm.a2_three_group(fused=fused))
        assert t == F(GOLD["a2_three_group_time"])
        assert round(float(t), 2) == GOLD["a2_three_group_time_printed"]


def test_a2_direct_link_idle_during_relay_groups():
    g = cm.a2_three_group(fused=False)
    direct = {(0, 1), (1, 0)}
    assert not any((s, d) in direct for s, d, _ in g[0] + g[1])
    assert all((s, d) in direct for s, d, _ in g[2])


def test_a2_two_groups_cost_a_quarter_and_the_optimum_is_count_over_4():
    for fused in (False, True):
        assert cm.link_cost(cm.a2_two_group(fused=fused)) == F(GOLD["a2_two_group_time"])
    grid = [F(k, 64) for k in range(1, 64)]
    costs = {d: cm.link_cost(cm.a2_two_group(d=d, fused=True)) for d in grid}
    best = min(costs, key=costs.get)
    assert best == F(GOLD["a2_optimal_direct"])
    assert costs[best] == F(1, 4)
    # at the optimum each (link, direction) moves one chunk in each of the two groups
    for group in cm.a2_two_group(fused=True):
        loads = {}
        for s, d, n in group:
            loads[(s, d)] = loads.get((s, d), 0) + n
        assert set(loads.values()) == {F(1, 8)}


def test_a2_ceilings_against_the_nccl_baseline():
    base = cm.link_cost(cm.nccl_allreduce_baseline(A=2))
    assert base == 1
    assert round(float(base / F(3, 7)), 2) == GOLD["a2_ceiling_before"]
    assert base / cm.link_cost(cm.a2_two_group()) == GOLD["a2_ceiling_after"]


def test_a4_allreduce_critical_path_and_ceilings():
    A = 4
    base = cm.link_cost(cm.nccl_allreduce_baseline(A=A))
    assert base == F(1, 2)
    for p in (F(780, 1000), F(1, 2), F(3, 10)):
        t = cm.link_cost(cm.a4_allreduce(p=p))
        assert t == 2 * max(p, 1 - p) / A
    c780 = base / cm.link_cost(cm.a4_allreduce(p=F(780, 1000)))
    c500 = base / cm.link_cost(cm.a4_allreduce(p=F(1, 2)))
    assert round(float(c780), 2) == GOLD["a4_allreduce_ceiling_780"]
    assert c500 == GOLD["a4_allreduce_ceiling_500"]
    # equal direct and offload regions minimise the critical path
    grid = [F(k, 100) for k in range(1, 100)]
    assert min(grid, key=lambda p: cm.link_cost(cm.a4_allreduce(p=p))) == F(1, 2)


def test_a4_all_to_all_model_ratio():
    base = cm.link_cost(cm.direct_all_to_all())
    grid = [F(k, 100) for k in range(1, 100)]
    best = min(grid, key=lambda p: cm.link_cost(cm.a4_all_to_all(p=p)))
    ratio = base / cm.link_cost(cm.a4_all_to_all(p=best))
    assert best == F(2, 5) and ratio == F(5, 3)
    assert round(float(ratio), 2) == GOLD["a4_all_to_all_model"]


def test_evaluator_rejects_self_links():
    import pytest
    with pytest.raises(ValueError):
        cm.link_cost([[(3, 3, 1)]])
