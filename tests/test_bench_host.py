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


def _traffic_file(tmp_path, digest=None):
    t = {"kernel_source_digest": digest or bench.kernel_source_digest(), "entries": [
        {"message_mib": 64.0, "variant": "share", "dtype": "bf16", "workload": bench.workload_name(64.0),
         "kernels": {"reduce<bf16>": {"hbm_bytes_per_launch": 1001, "algorithmic_bytes_per_launch": 1000,
                                      "launches_per_step": 6}}},
        {"message_mib": 1024.0, "variant": "group", "dtype": "bf16", "workload": bench.workload_name(1024.0),
         "kernels": {"copy": {"hbm_bytes_per_launch": 2002, "algorithmic_bytes_per_launch": 2000,
                              "launches_per_step": 2}}}]}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(t))
    return str(path)


def test_stored_traffic_is_used_only_for_its_own_workload(tmp_path):
    path = _traffic_file(tmp_path)
    get = lambda *a, **k: bench.traffic_for(*a, path=path, **k)
    assert get("reduce<bf16>", 64.0, "share", 1000, 6) == 1001
    assert get("copy", 1024.0, "group", 2000, 2) == 2002
    assert get("reduce<bf16>", 64.0, "group", 1000, 6) is None       # other variant
    assert get("reduce<bf16>", 128.0, "share", 1000, 6) is None      # other message
    assert get("reduce<bf16>", 64.0, "share", 1000, 6, "f32") is None  # other dtype
    assert get("copy", 64.0, "share", 1000, 6) is None               # no such kernel there
    # another launch sequence of the same kernel (other launches per step or
    # bytes per launch) gets no stored figure either
    assert get("reduce<bf16>", 64.0, "share", 1000, 5) is None
    assert get("reduce<bf16>", 64.0, "share", 1016, 6) is None
    # an entry of another workload at the same message (the ragged all-to-all
    # step) is not used for the plain step, and the other way round
    assert bench.traffic_for("reduce<bf16>", 64.0, "share", 1000, 6, path=path,
                             workload=bench.workload_name(64.0, "bf16", True)) is None
    # counters taken on other kernel code are never used
    stale = _traffic_file(tmp_path, digest="0" * 16)
    assert bench.traffic_for("reduce<bf16>", 64.0, "share", 1000, 6, path=stale) is None


def test_committed_traffic_matches_its_kernel_code():
    """The committed counter figures carry the digest of the kernel code they
    were taken on; bench.py uses them only while that code is unchanged."""
    with open(bench.TRAFFIC_JSON) as fh:
        t = json.load(fh)
    for e in t["entries"]:
        for kern, k in e["kernels"].items():
            got = bench.traffic_for(kern, e["message_mib"], e["variant"], k["algorithmic_bytes_per_launch"],
                                    k["launches_per_step"], e["dtype"], workload=e["workload"])
            assert got == (k["hbm_bytes_per_launch"] if t["kernel_source_digest"] == bench.kernel_source_digest()
                           else None)


_REL = "void rr::(anonymous namespace)::{}(rr::RedBatchT<8>)"


def _pmc_csv(path, counter, dispatches):
    lines = ['"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value"']
    for i, (name, v) in enumerate(dispatches, 1):
        lines.append(f'{i},"{name}","{counter}",{v}')
    path.write_text("\n".join(lines) + "\n")
    return str(path)


def test_traffic_from_scales_by_the_plain_copy_and_averages_the_timed_steps(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(tmp_path / "traffic.json"))
    red, cp = _REL.format("reduce_uniform_kernel<true, 8>"), _REL.format("copy_uniform_kernel<16>")
    order, algo = ["ar2_helper", "a2a_pack"], {"ar2_helper": 3 * 1024 * 100, "a2a_pack": 2 * 1024 * 50}
    run = {"steps": 2, "warmup": 1, "dtype": "bf16",
           "config": {"launch_order": order, "rows_bytes_per_launch": algo, "message_bytes": 64 << 20,
                      "variant": "share", "workload": "two launches"}}
    (tmp_path / "run.json").write_text("[bench] noise\n" + json.dumps(run) + "\n")
    # a relay launch while staging inputs, the copy of 256 MiB three times,
    # then warmup + 2 x 2 steps of the two launches
    setup = [(red, 999.0), ("__amd_rocclr_copyBuffer", 1.0)]
    fetch = setup + [("__amd_rocclr_copyBuffer", 256 * 1024 / 2)] * 3 + [(red, 100.0), (cp, 25.0)] * 5
    write = setup + [("__amd_rocclr_copyBuffer", 256 * 1024)] * 3 + [(red, 100.0), (cp, 50.0)] * 5
    args = type("A", (), {})()
    args.traffic_from = ",".join([_pmc_csv(tmp_path / "f.csv", "FETCH_SIZE", fetch),
                                  _pmc_csv(tmp_path / "w.csv", "WRITE_SIZE", write)])
    args.traffic_bench = str(tmp_path / "run.json")
    args.calibrate_copy_mib = 256.0
    bench.traffic_from(args)
    t = json.loads((tmp_path / "traffic.json").read_text())
    e = t["entries"][0]
    assert t["kernel_source_digest"] == bench.kernel_source_digest()
    assert e["fetch_scale"] == 2.0 and e["write_scale"] == 1.0
    assert [l["hbm_bytes"] for l in e["launches"]] == [300 * 1024, 100 * 1024]
    assert e["kernels"]["reduce<bf16>"] == {"hbm_bytes_per_launch": 300 * 1024,
                                            "algorithmic_bytes_per_launch": 300 * 1024, "launches_per_step": 1}
    assert e["kernels"]["copy"]["hbm_bytes_per_launch"] == 100 * 1024


def test_linear_fit_recovers_fixed_cost_and_bandwidth():
    t0, bw = 1.5e-6, 6.4e12
    samples = {"r": {m: (int(m * 2 ** 20), [t0 + m * 2 ** 20 / bw]) for m in (64.0, 128.0, 256.0, 512.0)}}
    row = bench.fit_table(samples)[0]
    assert abs(row["t0_us"] - 1.5) < 1e-3 and abs(row["bw_gbs"] - 6400.0) < 0.1 and row["r2"] > 0.99999
    a = row["at_ref"]
    assert abs(a["pct_of_peak"] / 100 - (bw / 8e12) * a["streaming_share"]) < 1e-3


def test_fit_from_trace_uses_only_launches_after_the_cache_clearing_read(tmp_path, capsys):
    evict = "void at::native::reduce_kernel<512, 1, at::native::ReduceOp<long, at::native::func_wrapper<long> > >"
    red = _REL.format("reduce_one_kernel<true, 2>")
    log, rows, ts = [], [], 0

    def disp(name, dur_ns):
        nonlocal ts
        rows.append((name, ts, ts + dur_ns))
        ts += dur_ns + 1000

    disp(red, 5)  # a launch made while staging inputs: not timed
    for role, t0_ns, bw in (("one_tile", 3560, None), ("a", 1000, 6400.0), ("b", 2000, 8000.0)):
        for mib in ((0.0,) if bw is None else (64.0, 128.0, 256.0, 512.0)):
            b = 768 if bw is None else int(mib * 2 ** 20)
            for rep in range(4):
                disp(evict, 200000)
                disp(red, t0_ns if bw is None else int(t0_ns + b / bw))
                log.append({"role": role, "message_mib": mib, "bytes": b, "warmup": rep < 2})
    lines = ['"Dispatch_Id","Kernel_Name","Start_Timestamp","End_Timestamp"']
    lines += [f'{i},"{n}",{a},{b}' for i, (n, a, b) in enumerate(rows, 1)]
    (tmp_path / "trace.csv").write_text("\n".join(lines) + "\n")
    (tmp_path / "log.json").write_text(json.dumps({"variant": "share", "launches": log}))
    args = type("A", (), {})()
    args.fit_trace, args.fit_log, args.sweep_out = str(tmp_path / "trace.csv"), str(tmp_path / "log.json"), \
        str(tmp_path / "fit.json")
    bench.fit_from_trace(args)
    fit = json.loads((tmp_path / "fit.json").read_text())
    assert fit["one_tile_us"] == 3.56
    got = {r["role"]: r for r in fit["roles"]}
    assert abs(got["a"]["t0_us"] - 1.0) < 0.01 and abs(got["a"]["bw_gbs"] - 6400) < 1
    assert abs(got["b"]["t0_us"] - 2.0) < 0.01 and abs(got["b"]["bw_gbs"] - 8000) < 1
    assert "| a |" in capsys.readouterr().out


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


def test_library_stand_in_follows_the_copy_store_policy():
    """The stand-in with the library's own policy per launch: reductions in
    the 16 KiB non-temporal pattern, copies moving under 256 MiB in 8 KiB
    tiles with agent-scope stores, larger ones non-temporal, and long ones in
    4 KiB tiles (8 KiB when ragged).  The sizes are the library's own."""
    import re
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "pack_rr_helper_amd", "csrc", "rr_internal.h")).read()
    for name, const in (("RR_COPY_LONG_BYTES", bench.COPY_LONG_BYTES),
                        ("RR_COPY_AGENT_MAX_BYTES", bench.COPY_AGENT_MAX_BYTES)):
        m = re.search(r"#define %s \(int64_t\(1\) << (\d+)\)" % name, hdr)
        assert m and const == 1 << int(m.group(1)), name
    long_b, wt_b = 2 * bench.COPY_LONG_BYTES, 2 * bench.COPY_AGENT_MAX_BYTES
    calls = [("ar4_phase", "reduce<bf16>", 84 << 20, None), ("a2a_pack", "copy", 80 << 20, None),
             ("a2a_unpack", "copy", long_b, None), ("a2a_pack", "copy", long_b - 2, None),
             ("a2a_pack", "copy", wt_b - 2, None)]
    names = lambda ragged: [bench.CALIB_PATTERNS[p] for p in bench.library_patterns(calls, ragged)]
    assert names(False) == ["relay", "tile8k_wt", "tile4k", "tile8k", "tile8k_wt"]
    assert names(True) == ["relay", "tile8k_wt", "tile8k", "tile8k", "tile8k_wt"]


def test_another_library_build_gets_no_stored_traffic(monkeypatch):
    """With --library the run measures another build, so the counter bytes
    stored for the default build are not attached."""
    key = ("reduce<bf16>", 64.0, "share", 68506965, 6)
    monkeypatch.setattr(bench, "CUSTOM_LIBRARY", "/tmp/other/librr.so")
    assert bench.traffic_for(*key) is None
