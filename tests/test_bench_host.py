"""Host-side logic of bench.py (no GPU): the kernel-code digest that guards
the stored HBM counter figures, the lookup of those figures, and the refusal
of more than one GPU."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_code_digest_ignores_comments_and_spacing_only():
    code = "__global__ void k(int *p)\n{\n    p[0] = 1;  // one\n}\n"
    same = "/* a kernel */\n__global__ void k(int *p) { p[0] = 1; }\n// end\n"
    changed = "__global__ void k(int *p)\n{\n    p[0] = 2;  // one\n}\n"
    assert bench.code_digest([code]) == bench.code_digest([same])
    assert bench.code_digest([code]) != bench.code_digest([changed])
    assert bench.code_digest([code, same]) != bench.code_digest([code])


def test_stored_traffic_is_used_only_for_its_own_workload():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as fh:
        t = json.load(fh)
    kernel = next(iter(t["kernels"]))
    k = t["kernels"][kernel]
    seq = (k["algorithmic_bytes_per_launch"], k["launches_per_step"])
    got = bench.traffic_for(kernel, t["message_mib"], t["variant"], *seq)
    if t["kernel_source_digest"] == bench.kernel_source_digest():
        assert got == k["hbm_bytes_per_launch"]
    else:
        assert got is None          # counters taken on other kernel code
    other = "group" if t["variant"] != "group" else "share"
    assert bench.traffic_for(kernel, t["message_mib"], other, *seq) is None
    assert bench.traffic_for(kernel, t["message_mib"] * 2, t["variant"], *seq) is None
    assert bench.traffic_for("no such kernel", t["message_mib"], t["variant"], *seq) is None
    # another launch sequence of the same kernel (other launches per step or
    # bytes per launch) gets no stored figure either
    assert bench.traffic_for(kernel, t["message_mib"], t["variant"], seq[0], seq[1] - 1) is None
    assert bench.traffic_for(kernel, t["message_mib"], t["variant"], seq[0] + 16, seq[1]) is None


def test_more_than_one_gpu_is_refused():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                          capture_output=True, text=True, timeout=120)
    assert proc.returncode == 2
    assert "one GPU" in proc.stderr and proc.stdout == ""


M2 = 2 << 20  # a 2 MiB bf16 message: every chunk formula divides evenly but the all-to-all's


def _role_bytes(jobs):
    out = {}
    for role, nb, _ in jobs:
        out[role] = out.get(role, 0) + nb
    return out


def test_oracle_jobs_cover_the_step_bytes_per_role():
    """The CPU baseline runs the same jobs as the GPU step: per role, the
    algorithmic bytes of one GPU's share (9M/8, 0.75M, 1.5M, 5M/8 + 5M/8 for
    the A=4 allreduce's helper and active slices in one phase, M/2, M and 24
    all-to-all chunks each way), 2-4x that for the group, and the group's
    bytes with the A=4 roles apart when every job is its own launch."""
    inp = bench.host_inputs(M2, rows=("ar2", "rs2", "ar4", "rs4", "a2a"))
    prep = bench.oracle_prep(inp, bench.BF16_CODE)
    a2a_chunk = (M2 // 8 // 5) // 128 * 128
    share = {"ar2_helper": 9 * M2 // 8, "ar2_active": 3 * M2 // 4, "rs2_owner": 3 * M2 // 2,
             "ar4_phase": 10 * M2 // 8, "rs4_pass1": M2 // 2, "rs4_pass2": M2,
             "a2a_pack": 24 * a2a_chunk * 2, "a2a_unpack": 24 * a2a_chunk * 2}
    assert _role_bytes(bench.oracle_jobs(inp, prep, bench.BF16_CODE, "share")) == share
    times = {"ar2_helper": 2, "ar2_active": 2, "rs2_owner": 2}
    group = {r: b * times.get(r, 4) for r, b in share.items()}
    assert _role_bytes(bench.oracle_jobs(inp, prep, bench.BF16_CODE, "group")) == group
    job = dict(group)
    job["ar4_helper"] = job["ar4_active"] = job.pop("ar4_phase") // 2
    assert _role_bytes(bench.oracle_jobs(inp, prep, bench.BF16_CODE, "job")) == job


def test_oracle_rates_cover_every_sweep_role():
    """The sweep's oracle column has a rate for every role it times: the A=4
    allreduce as its shared phase launch and as separate helper and active
    launches, beside every other role of one GPU's share."""
    rates = bench.oracle_role_rates(M2, "bf16", "share", budget_s=0.0)
    assert {"ar4_phase", "ar4_helper", "ar4_active"} <= set(rates)
    assert set(bench.STEP_MIX) <= set(rates)
    assert all(r["gbs"] > 0 and r["gbs_1t"] > 0 for r in rates.values())


def test_oracle_timers_run_on_one_and_several_threads():
    inp = bench.host_inputs(M2, rows=("ar2",))
    prep = bench.oracle_prep(inp, bench.BF16_CODE)
    jobs = lambda: bench.oracle_jobs(inp, prep, bench.BF16_CODE, "share")
    t, b, reps = bench.oracle_one_thread(jobs(), 0.0)
    assert reps == 1 and t > 0 and b == sum(nb for _, nb, _ in jobs())
    t, b, passes = bench.oracle_threads(jobs, 3, 0.0)
    assert passes == 3 and t > 0 and b == 3 * sum(nb for _, nb, _ in jobs())


def test_stand_in_step_covers_every_launch():
    """--calibrate-step gives every launch of the step a plain-stream stand-in
    whose read/write mix matches the role's algorithmic bytes: K inputs and
    one output for a K-input reduction, one and one for a copy."""
    inp = bench.host_inputs(M2, rows=("ar2", "rs2", "ar4", "rs4", "a2a"))
    prep = bench.oracle_prep(inp, bench.BF16_CODE)
    roles = {r for v in bench.VARIANTS for r, _, _ in bench.oracle_jobs(inp, prep, bench.BF16_CODE, v)}
    assert roles == set(bench.STEP_MIX)
    for role in ("ar2_helper", "rs2_owner", "ar4_active", "ar4_phase", "rs4_pass1", "a2a_pack"):
        R, W = bench.STEP_MIX[role]
        assert W == 1 and R == {"ar2": 2, "rs2": 2, "ar4": 4, "rs4": 3, "a2a": 1}[role[:3]]
