#!/usr/bin/env python3
"""Benchmark of the sharded relay hot path on one MI355X.

One step is one pass of every relay kernel of the method over one batch of
synthetic input at one message size M (per-active-rank input bytes, bf16),
in the fused 8-GPU collectives' layout (A=2: four sparse groups; A=4: two).
Consecutive steps use three independent sets of buffers in turn
(--buffer-sets), so no step finds its data left in the 256 MB Infinity Cache
by the step before:

  A=2 allreduce  (H=6, numChunks=8):  helper reduce-at-helper, active epilogue
  A=2 reduce-scatter:                 owner epilogue (recvCount = M/4 elems)
  A=4 allreduce  (H=4, 500 permille): helper 4->1 slice, active direct slice
  A=4 reduce-scatter (H=4):           helper pass 1, owner pass 2
  A=4 all-to-all (H=4, numChunks=5):  helper-slice pack and unpack (segmentCount = M/8)

--variant chooses the jobs each launch covers (one launch per role, except
that the A=4 allreduce's helper and active reductions, which a rank runs in
the same phase, share one launch):
  share  (default) one GPU's share of the fused call: a GPU is a helper for
         the three other A=2 groups (3 helper jobs) and runs one job in
         every other role; 8 launches per step;
  group  every job of one simulated group in one launch (2-4x a GPU's share);
  job    one launch per job of the group (34 launches per step).

Inputs are resident in HBM before timing starts.  ``value`` is the step's
algorithmic bytes (every input element read once, every output element
written once) divided by the step time of a first timed region with nothing
between the launches, in GB/s (10^9 bytes/s).  A second timed region puts a
timing-only HIP event between consecutive launches on their stream; less the
events' own cost per launch, it gives each launch's duration, and the kernel
family with the largest share of the step's time is reported against the
8 TB/s HBM peak in ``roofline``.  ``other_variants`` repeats the first timed
region with the launches of the other variants, and ``stand_in_step`` with
every launch replaced by a plain stream kernel of its read/write mix and bytes
(``--no-other-variants`` skips both; profiling runs use that flag so that they
hold only the named variant's relay launches).  ``cpu_baseline`` times the CPU oracle on
the same jobs, on the host's cores (up to 16 threads, the value) and on one
thread; the sweep records both oracle rates beside every row.

  python bench.py [--steps K] [--warmup W] [--message-mib M] [--variant share|group|job]
  python bench.py --sweep [--sweep-out FILE]   # per-role GB/s, 2 MiB .. 1 GiB, bf16 and fp32
  python bench.py --calibrate                  # plain read/write stream mixes alone
  python bench.py --calibrate-step             # the step beside plain streams of its mixes and bytes
  python bench.py --step-sweep [--sweep-out F] # both at 2 MiB .. 1 GiB messages, share and group
"""
import argparse
import hashlib
import json
import os
import platform
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0  # MI355X HBM3E, published
KERNEL_FORMS = {
    "reduce<bf16>": "reduce_one_kernel<bf16,K> (one aligned segment), reduce_uniform_kernel<bf16> "
                    "(equal segments), reduce_kernel<bf16> (tile table): one per-tile code, three "
                    "launch forms (reduce_shifted_*<bf16> realign views at other offsets; the "
                    "benchmark's buffers are aligned)",
    "reduce<f32>": "reduce_one_kernel<f32,K>, reduce_uniform_kernel<f32>, reduce_kernel<f32> "
                   "(reduce_shifted_*<f32> for views at other offsets)",
    "copy": "copy_uniform_kernel, copy_kernel (aligned moves only), copy_mixed_uniform_kernel, copy_mixed_kernel",
}
VARIANTS = {
    "share": "each role's launch covers one GPU's share of the fused 8-GPU call (3 A=2 helper "
             "jobs, one job in every other role; the A=4 allreduce's helper and active job share "
             "one launch)",
    "group": "each role's launch covers every job of one simulated group (2-4x one GPU's share)",
    "job": "one launch per job",
}
METRIC = "achieved HBM GB/s (and % of peak) of relay reduce/pack kernels, 2MB-1GB msgs"
MIB = 1 << 20
BF16_CODE, F32_CODE = 1, 0  # dtype codes of the C ABI and the oracle
# rows of the per-role sweep (one workload each; "ar4" times the A=4 allreduce's
# helper and active launches apart, "ar4_phase" the launch they share in the
# step; the _shifted rows place every input at an odd element offset, the
# a2a_ragged row has segmentCount = 5 mod 8)
SWEEP_ROWS = ("ar2", "rs2", "ar4", "ar4_phase", "rs4", "a2a", "a2a_ragged", "rs2_shifted", "ar4_shifted")


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--message-mib", type=float, default=64.0)
    p.add_argument("--dtype", choices=("bf16", "f32"), default="bf16",
                   help="buffer dtype of the step (the sweeps take --sweep-dtypes)")
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip the CPU oracle timings (the step's cpu_baseline, the sweep rows' oracle)")
    p.add_argument("--buffer-sets", type=int, default=3,
                   help="independent copies of every buffer, used by consecutive steps in turn "
                        "(3: no step finds its data left in a cache by the previous steps)")
    p.add_argument("--sizes", default="256,1024",
                   help="also time the step at these messages (MiB), share and group, each with its own "
                        "roofline block under 'sizes'; '' for none")
    p.add_argument("--device-inputs", action="store_true",
                   help="draw the step's inputs on the device (timing only) instead of seeded host arrays")
    p.add_argument("--traffic-from", default=None,
                   help="FETCH_CSV,WRITE_CSV: rocprofv3 --pmc passes of a --calibrate-copy-mib run; with "
                        "--traffic-bench, record that run's HBM bytes per launch in profiles/traffic.json")
    p.add_argument("--sweep-summary", default=None,
                   help="JSONL of a --sweep run: print its tables (GB/s, %% of peak, best, relay / fastest stand-in, "
                        "oracle rates) as markdown")
    p.add_argument("--ragged-a2a", action="store_true",
                   help="the step's all-to-all with segmentCount = 5 mod 8 (its chunk moves realigned)")
    p.add_argument("--trace-summary", default=None,
                   help="KERNEL_TRACE_CSV: with --traffic-bench naming the JSON line of the traced run, print "
                        "per-family kernel averages and the last step launch by launch")
    p.add_argument("--traffic-bench", default=None,
                   help="the JSON line bench.py printed in the FETCH_SIZE pass of --traffic-from")
    p.add_argument("--no-other-variants", action="store_true",
                   help="skip timing the other variants and the plain-stream stand-in step")
    p.add_argument("--calibrate-copy-mib", type=float, default=0.0,
                   help="run a plain device copy of this size first (HBM counter calibration)")
    p.add_argument("--variant", choices=("share", "group", "job"), default="share",
                   help="jobs per launch: one GPU's share of the fused call (default), the "
                        "whole simulated group, or one job")
    p.add_argument("--sweep", action="store_true", help="per-row sweep instead of the step benchmark")
    p.add_argument("--step-sweep", action="store_true",
                   help="the step and its plain-stream stand-in at each of --sweep-sizes")
    p.add_argument("--calibrate", action="store_true",
                   help="time plain read/write stream mixes (bench_calib.so) instead of the step")
    p.add_argument("--calibrate-step", action="store_true",
                   help="time the step beside a stand-in step of plain streams with the same mixes and bytes")
    p.add_argument("--calibrate-sizes", default="256,1024", help="MiB per stream")
    p.add_argument("--calibrate-out", default=None)
    p.add_argument("--calibrate-alone", action="store_true",
                   help="--calibrate: time each launch alone after a 1 GiB read instead of back to back")
    p.add_argument("--sweep-sizes", default="2,4,8,16,32,64,128,256,512,1024")
    p.add_argument("--sweep-reps", type=int, default=20)
    p.add_argument("--sweep-dtypes", default="bf16,f32")
    p.add_argument("--sweep-rows", default=",".join(SWEEP_ROWS),
                   help="rows of the per-role sweep; the _shifted rows put every input at an odd "
                        "element offset (the realigning reduction kernels)")
    p.add_argument("--library", default=None,
                   help="run this build of the relay library instead of pack_rr_helper_amd/librr.so (for A/B "
                        "comparisons of build options); the counter traffic of profiles/traffic.json is then "
                        "not attached")
    p.add_argument("--flush", choices=("read", "write", "none"), default="read",
                   help="--calibrate-alone: how a launch's inputs are pushed out of the caches before it is timed")
    p.add_argument("--sweep-out", default=None)
    p.add_argument("--role-fit", action="store_true",
                   help="time every launch of the step alone at --fit-sizes messages (1x to 8x a 64 MiB "
                        "message's bytes) and fit t = t0 + bytes/BW per role")
    p.add_argument("--fit-sizes", default="16,32,64,128,256,512")
    p.add_argument("--fit-reps", type=int, default=10)
    p.add_argument("--fit-log", default=None,
                   help="--role-fit: write the launch log (role, message, bytes of every relay launch in "
                        "issue order) here, to match a rocprofv3 kernel trace of the same run")
    p.add_argument("--fit-min-mib", type=float, default=0.0,
                   help="with --fit-trace: fit only the messages of at least this many MiB")
    p.add_argument("--fit-trace", default=None,
                   help="with --fit-log: fit per role from this rocprofv3 kernel_trace.csv instead of "
                        "running anything on the GPU; prints the table")
    return p.parse_args()


# --------------------------------------------------------------------------
# workload
# --------------------------------------------------------------------------

def host_inputs(M, dtype="bf16", rows=("ar2", "rs2", "ar4", "rs4", "a2a")):
    """Seeded host inputs of the rows at message M (pack_rr_helper_amd.synth):
    bf16 bit patterns (uint16) or float32 values; the all-to-all rows carry raw
    bits, and ``a2a_ragged`` has segmentCount = 5 mod 8 (the sweep's
    realigning shape)."""
    from pack_rr_helper_amd import synth
    f32 = dtype == "f32"
    n = M // (4 if f32 else 2)
    fp = (lambda v: v) if f32 else synth.as_bf16_bits
    bits = synth.bits32 if f32 else synth.bits16
    make = {
        "ar2": lambda: [fp(synth.normal(n, 1, a)) for a in range(2)],
        "rs2": lambda: [fp(synth.normal(n, 1, 10 + a)) for a in range(2)],
        "ar4": lambda: [fp(synth.uniform(n, -2, 2, 3, a)) for a in range(4)],
        "rs4": lambda: [fp(synth.normal(n, 2, s)) for s in range(4)],
        "a2a": lambda: [bits(n, 4, s) for s in range(4)],
        "a2a_ragged": lambda: [bits(4 * (n // 4 - 3), 5, s) for s in range(4)],
    }
    return {r: make[r]() for r in rows}


def device_inputs(M, seed, dtype="bf16"):
    """Seeded inputs of every row at message M drawn on the device, for timing
    only (the kernels' work does not depend on the values): N(0,1) rounded to
    the dtype, raw 16- or 32-bit patterns for the all-to-all."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    f32 = dtype == "f32"
    n = M // (4 if f32 else 2)
    tdt = torch.float32 if f32 else torch.bfloat16
    normal = lambda: torch.randn(n, device="cuda", generator=g).to(tdt)
    if f32:
        bits = lambda: torch.randint(-2 ** 31, 2 ** 31 - 1, (n,), dtype=torch.int32, device="cuda",
                                     generator=g).view(torch.float32)
    else:
        bits = lambda: torch.randint(-32768, 32768, (n,), dtype=torch.int16, device="cuda", generator=g)
    return {"ar2": [normal() for _ in range(2)], "rs2": [normal() for _ in range(2)],
            "ar4": [normal() for _ in range(4)], "rs4": [normal() for _ in range(4)],
            "a2a": [bits() for _ in range(4)]}


def build_rows(inp, rows=("ar2", "rs2", "ar4", "rs4", "a2a"), mode="share", dtype="bf16"):
    """The rows' workloads on device copies of `inp` (host arrays from
    host_inputs of the same dtype, or device tensors, which are cloned so that
    every call owns its buffers)."""
    import numpy as np
    import torch
    import pack_rr_helper_amd as rr
    from pack_rr_helper_amd import synth
    from pack_rr_helper_amd import workloads as W
    dt = rr.F32 if dtype == "f32" else rr.BF16

    def dev(arrs, bits=False):
        out = []
        for a in arrs:
            if isinstance(a, torch.Tensor):
                out.append(a.clone())
            elif bits:  # raw patterns: 16-bit words as int16, 32-bit words as float32
                out.append(synth.to_device(a.view(np.float32), rr.F32) if a.itemsize == 4 else
                           synth.to_device(a, None))
            else:
                out.append(synth.to_device(a, dt))
        return out

    out = {}
    if "ar2" in rows:
        out["ar2"] = W.AR2(dev(inp["ar2"]), dt, rr.AVG, mode=mode)
    if "rs2" in rows:
        out["rs2"] = W.RS2(dev(inp["rs2"]), dt, rr.AVG, mode=mode)
    if "ar4" in rows:
        out["ar4"] = W.AR4(dev(inp["ar4"]), dt, rr.AVG, mode=mode)
    if "rs4" in rows:
        out["rs4"] = W.RS4(dev(inp["rs4"]), dt, rr.SUM, mode=mode)
    if "a2a" in rows:
        out["a2a"] = W.A2A(dev(inp["a2a"], bits=True), dt, mode=mode)
    return out


# --------------------------------------------------------------------------
# CPU baseline: the oracle beside the GPU, on one thread and on the host's cores
# --------------------------------------------------------------------------

def host_threads():
    """Threads for the oracle's multi-thread figure: the CPUs this process may
    run on, at most 16 (one GPU's share of an 8-GPU host's cores)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def oracle_prep(inp, dt):
    """Read-only oracle inputs derived from the rows' inputs, built once and
    untimed: each A=4 reduce-scatter helper's scratch of twelve (owner, source)
    chunks, stand-ins for the reduced chunks an owner receives, and each
    all-to-all helper slice's packed buffers (the unpack's input)."""
    import numpy as np
    import oracle as orc
    prep = {}
    if "rs4" in inp:
        x = inp["rs4"]
        R = x[0].size // 4
        c = orc.geometry(4, 4, 0, 500, R, orc.REDUCE_SCATTER, dt)["chunk"]
        prep["rs4_scratch"] = [np.concatenate([x[s][o * R + h * c:o * R + (h + 1) * c]
                                               for o in range(4) for s in range(4) if s != o])
                               for h in range(4)]
        prep["rs4_reds"] = [np.ascontiguousarray(x[0][:c]) for _ in range(4)]
    es = orc.esize(dt)
    for row in ("a2a", "a2a_ragged"):
        if row in inp:
            x = inp[row]
            seg = x[0].size // 4
            c = orc.geometry(4, 4, 5, 0, seg, orc.ALLTOALL, dt)["chunk"]
            prep[row + "_packed"] = [orc.a2a_pack(es, 4, seg, c, h, x) for h in range(4)]
    return prep


def oracle_jobs(inp, prep, dt, variant="share", phase=True):
    """The GPU step's jobs through the oracle, as (role, algorithmic bytes,
    callable) in launch order: one GPU's share (3 A=2 helper jobs, one job in
    every other role) or, for the other variants, every job of the group.
    The A=4 allreduce's helper and active jobs carry the role of their shared
    launch, "ar4_phase", unless ``phase`` is False or every job is its own
    launch.
    Outputs are private to the returned list; inputs are only read.  Every
    callable binds its arguments when it is made."""
    import functools
    import numpy as np
    import oracle as orc
    P = functools.partial
    share = variant == "share"
    n_ar2, n_a2, n_a4 = (3, 1, 1) if share else (6, 2, 4)
    AVG, SUM = orc.AVG, orc.SUM
    es = orc.esize(dt)
    jobs = []
    if "ar2" in inp:
        x = inp["ar2"]
        count = x[0].size
        g = orc.geometry(2, 6, 8, 0, count, orc.ALLREDUCE, dt)
        c = g["chunk"]
        for k in range(n_ar2):
            jobs.append(("ar2_helper", 3 * c * es,
                         P(orc.ar2_helper, dt, AVG, x[0][k * c:(k + 1) * c], x[1][k * c:(k + 1) * c])))
        out = np.zeros_like(x[0])
        for a in range(n_a2):
            jobs.append(("ar2_active", 3 * g["direct_len"] * es,
                         P(orc.ar_active, dt, AVG, 2, 6, 8, 0, count, a, x, out)))
    if "rs2" in inp:
        x = inp["rs2"]
        R = x[0].size // 2
        for o in range(1 if share else 2):
            jobs.append(("rs2_owner", 3 * R * es,
                         P(orc.rs2_active, dt, AVG, x[0][o * R:(o + 1) * R], x[1][o * R:(o + 1) * R])))
    if "ar4" in inp:
        x = inp["ar4"]
        count = x[0].size
        g = orc.geometry(4, 4, 0, 500, count, orc.ALLREDUCE, dt)
        c = g["chunk"]
        # one launch for both roles of the phase, except with one launch per job
        roles = ("ar4_helper", "ar4_active") if variant == "job" or not phase else ("ar4_phase", "ar4_phase")
        for h in range(n_a4):
            jobs.append((roles[0], 5 * c * es, P(orc.ar4_helper, dt, AVG, [v[h * c:(h + 1) * c] for v in x])))
        out = np.zeros_like(x[0])
        for a in range(n_a4):
            n = g["dslice"] if a < 3 else g["direct_len"] - 3 * g["dslice"]
            jobs.append((roles[1], 5 * n * es, P(orc.ar_active, dt, AVG, 4, 4, 0, 500, count, a, x, out)))
    if "rs4" in inp:
        x = inp["rs4"]
        R = x[0].size // 4
        c = orc.geometry(4, 4, 0, 500, R, orc.REDUCE_SCATTER, dt)["chunk"]
        for h in range(n_a4):
            jobs.append(("rs4_pass1", 16 * c * es, P(orc.rs4_pass1, dt, 4, c, prep["rs4_scratch"][h])))
        for o in range(n_a4):
            blk = [v[o * R:(o + 1) * R] for v in x]
            jobs.append(("rs4_pass2", (3 * 4 * c + 5 * (R - 4 * c)) * es,
                         P(orc.rs4_pass2, dt, SUM, 4, 4, 500, R, o, blk, prep["rs4_reds"])))
    for row, tag in (("a2a", ""), ("a2a_ragged", "_ragged")):
        if row not in inp:
            continue
        x = inp[row]
        seg = x[0].size // 4
        c = orc.geometry(4, 4, 5, 0, seg, orc.ALLTOALL, dt)["chunk"]
        outs = [np.zeros_like(v) for v in x]
        for h in range(n_a4):
            jobs.append(("a2a_pack" + tag, 24 * c * es, P(orc.a2a_pack, es, 4, seg, c, h, x)))
            jobs.append(("a2a_unpack" + tag, 24 * c * es,
                         P(orc.a2a_unpack, es, 4, seg, c, h, prep[row + "_packed"][h], outs)))
    return jobs


def oracle_one_thread(jobs, budget_s, max_reps=100):
    """Runs the job list in order until `budget_s` seconds of job time (at
    least once); returns (seconds, bytes, passes)."""
    t, b, reps = 0.0, 0, 0
    while (t < budget_s and reps < max_reps) or reps == 0:
        for _, nb, fn in jobs:
            t0 = time.perf_counter()
            fn()
            t += time.perf_counter() - t0
            b += nb
        reps += 1
    return t, b, reps


def oracle_threads(make_jobs, threads, budget_s):
    """`threads` host threads, each running its own job list (make_jobs())
    over and over until `budget_s` seconds of wall time have passed (every
    thread completes at least one pass).  The oracle's C routines run without
    the interpreter lock, so the threads compute in parallel.  Returns (wall
    seconds from the common start to the last thread's end, bytes, passes)."""
    import threading
    lists = [make_jobs() for _ in range(threads)]
    done, passes, ends = [0] * threads, [0] * threads, [0.0] * threads
    gate = threading.Barrier(threads + 1)
    deadline = [0.0]

    def work(i):
        gate.wait()
        while True:
            for _, nb, fn in lists[i]:
                fn()
                done[i] += nb
            passes[i] += 1
            if time.perf_counter() >= deadline[0]:
                break
        ends[i] = time.perf_counter()

    ts = [threading.Thread(target=work, args=(i,)) for i in range(threads)]
    for t in ts:
        t.start()
    deadline[0] = time.perf_counter() + budget_s
    gate.wait()
    start = time.perf_counter()
    for t in ts:
        t.join()
    return max(ends) - start, sum(done), sum(passes)


def cpu_baseline(inp, dt, variant, budget_s=(10.0, 8.0), label=""):
    """The bench line's cpu_baseline object: the oracle on the step's jobs,
    on `host_threads()` threads (the value) and on one thread."""
    prep = oracle_prep(inp, dt)
    t1, b1, r1 = oracle_one_thread(oracle_jobs(inp, prep, dt, variant), budget_s[0])
    T = host_threads()
    tT, bT, rT = oracle_threads(lambda: oracle_jobs(inp, prep, dt, variant), T, budget_s[1])
    return {
        "value": round(bT / tT / 1e9, 3), "unit": "GB/s", "cores": T, "kind": "oracle",
        "sample": (f"{label}{variant} variant, one step = {b1 // r1} algorithmic bytes: {rT} step(s) over "
                   f"{T} threads in {tT:.1f} s wall (each thread its own outputs, same inputs); "
                   f"host {cpu_model()}"),
        "single_thread": {"value": round(b1 / t1 / 1e9, 3), "cores": 1,
                          "sample": f"{r1} step(s), {t1:.1f} s of oracle time"},
    }


def oracle_role_rates(M, dt_name, variant, budget_s=0.3):
    """The oracle's GB/s per role at message M, on one thread and on
    host_threads() threads, over the jobs the GPU launch of that role covers
    (same shapes, host inputs from the same recipe).  Roles are named as the
    sweep names them (the A=4 allreduce both as its shared launch and as
    separate roles)."""
    dt = F32_CODE if dt_name == "f32" else BF16_CODE
    rows = ("ar2", "rs2", "ar4", "rs4", "a2a", "a2a_ragged")
    inp = host_inputs(M, dt_name, rows)
    T, cpu = host_threads(), cpu_model()
    rates = {}
    for row in rows:
        sub = {row: inp[row]}
        prep = oracle_prep(sub, dt)
        for role, phase in sorted({(j[0], ph) for ph in (True, False)
                                   for j in oracle_jobs(sub, prep, dt, variant, ph)}):
            if role in rates:
                continue
            def make(role=role, sub=sub, prep=prep, phase=phase):
                return [j for j in oracle_jobs(sub, prep, dt, variant, phase) if j[0] == role]
            t1, b1, _ = oracle_one_thread(make(), budget_s)
            tT, bT, _ = oracle_threads(make, T, budget_s)
            rates[role] = {"threads": T, "gbs": round(bT / tT / 1e9, 3), "gbs_1t": round(b1 / t1 / 1e9, 3),
                           "sample_mib": M / MIB, "cpu": cpu}
    return rates


# --------------------------------------------------------------------------
# traffic from the committed rocprofv3 counter summary
# --------------------------------------------------------------------------

def code_digest(texts):
    """Digest of C/C++ sources with comments and white space removed."""
    h = hashlib.sha256()
    for text in texts:
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def kernel_source_digest():
    """Digest of the kernel code the counters were taken on: the kernel source
    and its tiling header, so that only a change to the code itself (not to
    its comments) invalidates the stored traffic."""
    texts = []
    for f in ("rr_kernels.hip", "rr_internal.h"):
        with open(os.path.join(ROOT, "pack_rr_helper_amd", "csrc", f)) as fh:
            texts.append(fh.read())
    return code_digest(texts)


TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
# --library: another build of the relay library is running (its counters are
# not the stored ones)
CUSTOM_LIBRARY = None


def workload_name(message_mib, dtype="bf16", ragged_a2a=False):
    """The benchmark step's workload, as its JSON line and its counter entries name it."""
    return (f"relay hot path, {message_mib:g} MiB per-rank {dtype} message: A=2 allreduce (H=6) + A=2 "
            "reduce-scatter + A=4 allreduce (H=4, 500 permille) + A=4 reduce-scatter + A=4 all-to-all "
            "pack/unpack" + (" (segmentCount = 5 mod 8)" if ragged_a2a else "") + ", one GPU")


def traffic_for(kernel, message_mib, variant, algo_bytes_per_launch, launches_per_step, dtype="bf16",
                path=TRAFFIC_JSON, workload=None):
    """HBM bytes per launch of `kernel` (counter-measured, scaled by a plain
    copy of known size) from profiles/traffic.json, or None if absent, taken
    on another workload or launch sequence (other message, variant, dtype or
    workload, other launches per step, or other algorithmic bytes per launch),
    or taken on other kernel sources.  workload: the step's workload_name
    (default: the plain step's)."""
    if CUSTOM_LIBRARY or not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("kernel_source_digest") != kernel_source_digest():
        return None
    workload = workload or workload_name(message_mib, dtype)
    for e in t.get("entries", []):
        if e.get("message_mib") != message_mib or e.get("variant") != variant or e.get("dtype") != dtype \
                or e.get("workload", workload) != workload:
            continue
        k = e.get("kernels", {}).get(kernel)
        if k and k.get("algorithmic_bytes_per_launch") == algo_bytes_per_launch \
                and k.get("launches_per_step") == launches_per_step:
            return k.get("hbm_bytes_per_launch")
    return None


def counter_rows(path, counter):
    """(kernel name, value) per dispatch of a rocprofv3 --pmc CSV, in dispatch order."""
    import csv
    with open(path) as fh:
        rows = [r for r in csv.DictReader(fh) if r["Counter_Name"] == counter]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return [(r["Kernel_Name"], float(r["Counter_Value"])) for r in rows]


def kernel_family(name):
    """The roofline family of a relay kernel symbol: reduce<bf16>, reduce<f32> or copy."""
    m = RELAY_KERNEL.search(name)
    if not m:
        return None
    if m.group(1) == "copy":
        return "copy"
    return "reduce<bf16>" if "<true" in name else "reduce<f32>"


SWEEP_ORDER = ["ar2_active", "ar2_helper", "rs2_owner", "ar4_active", "ar4_helper", "ar4_phase", "rs4_pass1",
               "rs4_pass2", "a2a_pack", "a2a_unpack", "a2a_pack_ragged", "a2a_unpack_ragged", "rs2_owner_shifted",
               "ar4_active_shifted", "ar4_helper_shifted", "torch_copy_calibration"]


def sweep_summary(args):
    """Markdown tables of a --sweep JSONL: per dtype, GB/s and % of peak
    (median), GB/s (best), relay / fastest plain-stream stand-in (and the
    pattern that was fastest), and the CPU oracle's rates."""
    recs = [json.loads(l) for l in open(args.sweep_summary)]
    sizes = sorted({r["message_mib"] for r in recs})

    def table(vals, cols, fmt, roles, unit="MiB"):
        out = ["| role | " + " | ".join(f"{c:g} {unit}" for c in cols) + " |", "|---|" + "---:|" * len(cols)]
        for role in roles:
            cells = ["" if vals.get((role, c)) is None else fmt(vals[(role, c)]) for c in cols]
            if any(cells):
                out.append(f"| {role} | " + " | ".join(cells) + " |")
        return out

    out = []
    for dt in ("bf16", "f32"):
        g = {(r["row"], r["message_mib"]): r for r in recs if r["dtype"] in (dt, "u8")}
        if not any(r["dtype"] == dt for r in recs):
            continue
        for title, key, fmt in (("GB/s, median", "gbs_median", lambda v: f"{v:.0f}"),
                                ("percent of 8 TB/s, median", "pct_peak_median", lambda v: f"{v:.1f}"),
                                ("GB/s, best of the reps", "gbs_best", lambda v: f"{v:.0f}")):
            out += [f"## {dt}: {title}", ""] + table({k: r[key] for k, r in g.items()}, sizes, fmt, SWEEP_ORDER) + [""]
        st = {k: r["stand_in"] for k, r in g.items() if r.get("stand_in")}
        out += [f"## {dt}: relay launch / fastest plain-stream stand-in of the same read/write mix and bytes (median)",
                ""] + table({k: v["relay_over_stand_in"] for k, v in st.items()}, sizes, lambda v: f"{v:.2f}",
                            SWEEP_ORDER) + [""]
        out += [f"## {dt}: fastest stand-in pattern", ""] + table({k: v.get("pattern", "relay") for k, v in st.items()},
                                                                  sizes, str, SWEEP_ORDER) + [""]
        # write-back stores timed alone end with written lines still in the
        # caches; the non-temporal and write-through patterns have no such
        # deferral
        nt = {}
        for k, v in st.items():
            pats = {p: g for p, g in v.get("patterns", {}).items() if not p.endswith("_wb")}
            if pats:
                nt[k] = g_row[k] / max(pats.values()) if (g_row := {kk: r["gbs_median"] for kk, r in g.items()}) else None
        out += [f"## {dt}: relay launch / fastest stand-in without write-back stores (median)", ""] + table(
            nt, sizes, lambda v: f"{v:.2f}", SWEEP_ORDER) + [""]
        orc = {k: r for k, r in g.items() if r.get("oracle")}
        if orc:
            samples = sorted({r["oracle"]["sample_mib"] for r in orc.values()})
            thr = next(iter(orc.values()))["oracle"]["threads"]
            ofmt = lambda v: f"{v:.2f}" if v < 100 else f"{v:.1f}"
            out += [f"## {dt}: CPU oracle GB/s on {thr} threads (by sample message)", ""] + table(
                {(k[0], r["oracle"]["sample_mib"]): r["oracle"]["gbs"] for k, r in orc.items()}, samples, ofmt,
                SWEEP_ORDER) + [""]
            out += [f"## {dt}: CPU oracle GB/s on one thread (by sample message)", ""] + table(
                {(k[0], r["oracle"]["sample_mib"]): r["oracle"]["gbs_1t"] for k, r in orc.items()}, samples, ofmt,
                SWEEP_ORDER) + [""]
            out += [f"## {dt}: GPU / oracle ({thr} threads), median", ""] + table(
                {k: r["oracle"]["gpu_over_oracle"] for k, r in orc.items()}, sizes, lambda v: f"{v:.0f}",
                SWEEP_ORDER) + [""]
    print("\n".join(out).rstrip())


def trace_summary(args):
    """Per kernel family, the call-weighted average duration of every relay
    dispatch in a rocprofv3 kernel trace of a bench.py run, and the run's last
    step launch by launch (its launch order from the run's JSON line), as
    markdown."""
    import csv
    with open(args.traffic_bench) as fh:
        run = json.loads(fh.read().strip().splitlines()[-1])
    cfg = run["config"]
    order, algo = cfg["launch_order"], cfg["rows_bytes_per_launch"]
    with open(args.trace_summary) as fh:
        rows = sorted(csv.DictReader(fh), key=lambda r: int(r["Dispatch_Id"]))
    relay = [r for r in rows if RELAY_KERNEL.search(r["Kernel_Name"])]
    fam = {}
    for r in relay:
        f = fam.setdefault(kernel_family(r["Kernel_Name"]), [0, 0.0])
        f[0] += 1
        f[1] += (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
    print("| family | relay dispatches | avg us |")
    print("|---|---:|---:|")
    for k, (n, us) in fam.items():
        print(f"| `{k}` | {n} | {us / n:.3f} |")
    rl = run["roofline"]
    print(f"\nbench.py's roofline kernel in the same run: `{rl['kernel']}`, {rl['avg_launch_us']} us per launch "
          f"(timing-only event intervals of {rl['avg_event_interval_us']} us less {rl['event_cost_us_per_launch']} us)\n")
    last = relay[-len(order):]
    print("| launch | kernel | workgroups | duration us | algorithmic MB | GB/s | % of 8 TB/s |")
    print("|---|---|---:|---:|---:|---:|---:|")
    tot_us = tot_b = 0.0
    for row, r in zip(order, last):
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
        wg = (int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])) // int(r["Workgroup_Size_X"])
        name = re.sub(r"^void rr::\(anonymous namespace\)::", "", r["Kernel_Name"]).split("(")[0]
        b = algo[row]
        tot_us += us
        tot_b += b
        print(f"| {row} | `{name}` | {wg} | {us:.2f} | {b / 1e6:.1f} | {b / us / 1e3:.0f} | {100 * b / us / 1e3 / PEAK_GBS:.1f} |")
    print(f"| **step (kernels only)** | | | {tot_us:.2f} | {tot_b / 1e6:.1f} | {tot_b / tot_us / 1e3:.0f} | "
          f"{100 * tot_b / tot_us / 1e3 / PEAK_GBS:.1f} |")


def traffic_from(args):
    """HBM bytes per launch of one step from two rocprofv3 --pmc passes
    (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) of a bench.py run with
    --calibrate-copy-mib C: the counters are scaled so that the run's plain
    C MiB device copy reads as C MiB fetched and C MiB written; the last
    (warmup + 2 x steps) steps of relay dispatches are the timed ones, and
    each launch of the step is averaged over them.  Records the entry in
    profiles/traffic.json (replacing one of the same message, variant and
    dtype) and prints a markdown table."""
    fetch_csv, write_csv = args.traffic_from.split(",")
    with open(args.traffic_bench) as fh:
        run = json.loads(fh.read().strip().splitlines()[-1])
    cfg = run["config"]
    order = cfg["launch_order"]
    L = len(order)
    nsteps = run["warmup"] + 2 * run["steps"]
    out = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = counter_rows(path, counter)
        relay_at = [i for i, (n, _) in enumerate(rows) if RELAY_KERNEL.search(n)]
        timed = relay_at[-nsteps * L:]
        if len(timed) != nsteps * L:
            raise SystemExit(f"{path}: {len(relay_at)} relay dispatches, fewer than {nsteps} steps of {L}")
        copies = [v for n, v in rows[:timed[0]] if "copyBuffer" in n][-3:]
        expect_kib = args.calibrate_copy_mib * 1024.0
        scale = expect_kib / statistics.median(copies)
        per = []
        for j in range(L):
            vals = [rows[timed[s * L + j]] for s in range(nsteps)]
            if len({n for n, _ in vals}) != 1:
                raise SystemExit(f"launch {j} of the step runs different kernels across steps")
            per.append((vals[0][0], statistics.mean(v for _, v in vals)))
        out[counter] = (scale, per)
    fscale, fper = out["FETCH_SIZE"]
    wscale, wper = out["WRITE_SIZE"]
    algo = cfg["rows_bytes_per_launch"]
    launches, fam = [], {}
    for j, row in enumerate(order):
        name = fper[j][0]
        hbm = (fper[j][1] * fscale + wper[j][1] * wscale) * 1024.0
        launches.append({"row": row, "kernel": re.sub(r"^void rr::\(anonymous namespace\)::", "", name).split("(")[0],
                         "fetch_kib": round(fper[j][1], 1), "write_kib": round(wper[j][1], 1),
                         "hbm_bytes": round(hbm), "algorithmic_bytes": algo[row],
                         "ratio": round(hbm / algo[row], 4)})
        f = fam.setdefault(kernel_family(name), [0.0, 0, 0])
        f[0] += hbm
        f[1] += algo[row]
        f[2] += 1
    entry = {"message_mib": run["config"]["message_bytes"] / MIB, "variant": cfg["variant"], "dtype": run["dtype"],
             "workload": cfg["workload"],
             "fetch_scale": fscale, "write_scale": wscale,
             "kernels": {k: {"hbm_bytes_per_launch": round(v[0] / v[2]), "algorithmic_bytes_per_launch": v[1] // v[2],
                             "launches_per_step": v[2]} for k, v in fam.items()},
             "launches": launches}
    t = {"kernel_source_digest": kernel_source_digest(), "entries": []}
    if os.path.exists(TRAFFIC_JSON):
        with open(TRAFFIC_JSON) as fh:
            old = json.load(fh)
        if old.get("kernel_source_digest") == t["kernel_source_digest"]:
            t["entries"] = [e for e in old.get("entries", []) if e.get("workload") != entry["workload"] or
                            (e["message_mib"], e["variant"], e["dtype"]) !=
                            (entry["message_mib"], entry["variant"], entry["dtype"])]
    t["entries"].append(entry)
    t["entries"].sort(key=lambda e: (e["dtype"], e["variant"], e["message_mib"]))
    with open(TRAFFIC_JSON, "w") as fh:
        json.dump(t, fh, indent=1)
        fh.write("\n")
    print(f"scale: fetch x{fscale:.4f}, write x{wscale:.4f} (plain {args.calibrate_copy_mib:g} MiB copy)\n")
    print("| launch | kernel | FETCH KiB | WRITE KiB | HBM bytes (scaled) | algorithmic bytes | ratio |")
    print("|---|---|---:|---:|---:|---:|---:|")
    for l in launches:
        print(f"| {l['row']} | `{l['kernel']}` | {l['fetch_kib']} | {l['write_kib']} | {l['hbm_bytes']} | "
              f"{l['algorithmic_bytes']} | {l['ratio']:.4f} |")
    print("\n| kernel | launches | HBM bytes/launch | algorithmic bytes/launch | ratio |")
    print("|---|---:|---:|---:|---:|")
    for k, v in entry["kernels"].items():
        print(f"| `{k}` | {v['launches_per_step']} | {v['hbm_bytes_per_launch']} | {v['algorithmic_bytes_per_launch']} | "
              f"{v['hbm_bytes_per_launch'] / v['algorithmic_bytes_per_launch']:.4f} |")


# --------------------------------------------------------------------------
# main benchmark
# --------------------------------------------------------------------------

def hip_runtime():
    """The HIP runtime library this process already uses (torch's), for
    fence-free timing events; loading the same file returns the same handle."""
    import ctypes
    path = "libamdhip64.so"
    with open("/proc/self/maps") as fh:
        for line in fh:
            if "libamdhip64" in line:
                path = line.split()[-1]
                break
    L = ctypes.CDLL(path)
    L.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    L.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return L


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # hip_runtime_api.h: timing-only events


def time_variant(inp, mode, steps, warmup, stream, buffer_sets, dtype="bf16"):
    """Timed region 1 alone (K whole steps, nothing between launches, the
    buffer sets used in turn) for the rows built in another variant: step
    bytes, launches and ms per step."""
    import torch
    sets = [build_rows(inp, mode=mode, dtype=dtype) for _ in range(buffer_sets)]
    set_calls = [[c for wl in wls.values() for c in wl.calls(stream)] for wls in sets]
    ms = time_steps(lambda i: [c[3] for c in set_calls[i % buffer_sets]], steps, warmup, stream)
    b, n = sum(c[2] for c in set_calls[0]), len(set_calls[0])
    del sets, set_calls
    torch.cuda.empty_cache()
    gbs = b / (ms * 1e-3) / 1e9
    return {"value": round(gbs, 1), "unit": "GB/s", "pct_of_peak": round(100.0 * gbs / PEAK_GBS, 2),
            "ms_per_step": round(ms, 5), "launches_per_step": n, "algorithmic_bytes_per_step": b,
            "variant_means": VARIANTS[mode]}


def time_launches(step_fns, calls, steps, warmup, stream):
    """The step timed twice: region 1 runs K steps with nothing between the
    launches (ms per step); region 2 runs K more with one timing-only HIP event
    (no system-scope fence) between consecutive launches on the kernels'
    stream, so launch i lasts from event i to event i+1.  An event between two
    launches delays the second one, so an interval is a launch plus the
    events' own cost; that cost per launch is region 2's step time less region
    1's, spread over the step's launches, and is subtracted from every
    interval.  step_fns(i) gives step i's launches; calls the (row, kernel,
    bytes, fn) of one step."""
    import ctypes
    import torch
    for i in range(warmup):
        for fn in step_fns(i):
            fn()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    for i in range(steps):
        for fn in step_fns(i):
            fn()
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / steps

    hip = hip_runtime()
    sp = ctypes.c_void_p(stream.cuda_stream)
    evs = []
    for _ in range(steps * len(calls) + 1):
        e = ctypes.c_void_p()
        if hip.hipEventCreateWithFlags(ctypes.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        evs.append(e)
    i = 0
    hip.hipEventRecord(evs[0], sp)
    for step in range(steps):
        for fn in step_fns(step):
            fn()
            i += 1
            hip.hipEventRecord(evs[i], sp)
    torch.cuda.synchronize()
    per_row, per_kernel = {}, {}
    f = ctypes.c_float()
    i = 0
    for _ in range(steps):
        for row, kern, b, _ in calls:
            hip.hipEventElapsedTime(ctypes.byref(f), evs[i], evs[i + 1])
            i += 1
            for key, table in ((row, per_row), (kern, per_kernel)):
                r = table.setdefault(key, [0.0, 0, 0])
                r[0] += f.value
                r[1] += b
                r[2] += 1
    for e in evs:
        hip.hipEventDestroy(e)
    events_ms_step = sum(r[0] for r in per_row.values()) / steps
    event_cost_ms = max(0.0, events_ms_step - ms_step) / len(calls)
    return {"ms_step": ms_step, "wall_s": wall, "per_row": per_row, "per_kernel": per_kernel,
            "event_cost_ms": event_cost_ms}


def launch_ms(t, ms, n):
    """Average launch duration (ms) of n launches whose event intervals sum to ms."""
    return ms / n - t["event_cost_ms"]


def roofline_of(t, steps, message_mib, variant, dtype, workload=None):
    """The roofline block for the kernel family with the largest share of the
    step's time: algorithmic bytes per launch / average launch duration."""
    per_kernel = t["per_kernel"]
    dom = max(per_kernel, key=lambda k: per_kernel[k][0])
    d_ms, d_b, d_n = per_kernel[dom]
    dur = launch_ms(t, d_ms, d_n)
    achieved = (d_b / d_n) / (dur * 1e-3) / 1e9
    return {
        "kernel": dom,
        "kernel_symbols": KERNEL_FORMS.get(dom, dom),
        "timing": ("timing-only HIP events between consecutive launches on the kernels' stream "
                   "(second timed region), less the events' own cost per launch: (second region's "
                   "step time - event-free first region's) / launches per step"),
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / PEAK_GBS, 4),
        "traffic": traffic_for(dom, message_mib, variant, d_b // d_n, d_n // steps, dtype, workload=workload),
        "algorithmic_bytes_per_launch": d_b // d_n,
        "avg_launch_us": round(1e3 * dur, 3),
        "avg_event_interval_us": round(1e3 * d_ms / d_n, 3),
        "event_cost_us_per_launch": round(1e3 * t["event_cost_ms"], 3),
        "launches": d_n,
    }


def rows_of(t):
    per_row = t["per_row"]
    return {
        "rows_gbs": {row: round(b / n / (launch_ms(t, ms, n) * 1e-3) / 1e9, 1) for row, (ms, b, n) in per_row.items()},
        "rows_us_per_launch": {row: round(1e3 * launch_ms(t, ms, n), 2) for row, (ms, b, n) in per_row.items()},
        "rows_bytes_per_launch": {row: b // n for row, (ms, b, n) in per_row.items()},
    }


def size_block(mib, variant, steps, warmup, stream, dtype):
    """The step at another message size, inputs drawn on the device (the
    kernels' work does not depend on the values): three buffer sets in turn
    while a step moves under 2 GB, one above (a step then streams many times
    the 256 MB Infinity Cache); fewer steps for steps over 4 GB."""
    import torch
    M = int(mib * MIB)
    inp = device_inputs(M, 3000 + int(mib * 16), dtype)
    first = build_rows(inp, mode=variant, dtype=dtype)
    calls = [c for wl in first.values() for c in wl.calls(stream)]
    step_bytes = sum(c[2] for c in calls)
    nsets = 3 if step_bytes < 2e9 else 1
    sets = [first] + [build_rows(inp, mode=variant, dtype=dtype) for _ in range(nsets - 1)]
    del inp
    set_calls = [calls] + [[c for wl in wls.values() for c in wl.calls(stream)] for wls in sets[1:]]
    k = steps if step_bytes < 4e9 else max(10, steps // 5)
    t = time_launches(lambda i: [c[3] for c in set_calls[i % nsets]], calls, k, warmup, stream)
    value = step_bytes / (t["ms_step"] * 1e-3) / 1e9
    out = {"message_mib": mib, "variant": variant, "value": round(value, 1), "unit": "GB/s",
           "pct_of_peak": round(100.0 * value / PEAK_GBS, 2), "ms_per_step": round(t["ms_step"], 5),
           "steps": k, "warmup": warmup, "buffer_sets": nsets, "launches_per_step": len(calls),
           "algorithmic_bytes_per_step": step_bytes, "inputs": "drawn on the device (seeded), timing only",
           **rows_of(t), "roofline": roofline_of(t, k, mib, variant, dtype)}
    del sets, set_calls, calls, first
    torch.cuda.empty_cache()
    return out


def step_bench(args):
    import torch
    import pack_rr_helper_amd as rr
    rr.load()
    torch.cuda.set_device(0)
    M = int(args.message_mib * MIB)
    print(f"[bench] generating inputs, M={args.message_mib} MiB", file=sys.stderr, flush=True)
    inp = device_inputs(M, 1000 + int(args.message_mib * 16), args.dtype) if args.device_inputs \
        else host_inputs(M, args.dtype)
    if args.ragged_a2a:
        # segmentCount = 5 mod 8: sources and destinations of the helper
        # slice's chunk moves disagree modulo 16 bytes (the realigning copy)
        if args.device_inputs:
            inp["a2a"] = [x[:4 * (x.numel() // 4 - 3)].clone() for x in inp["a2a"]]
        else:
            inp["a2a"] = host_inputs(M, args.dtype, rows=("a2a_ragged",))["a2a_ragged"]
    # --buffer-sets N: N independent copies of every buffer, used by
    # consecutive steps in turn, so that no step finds its data in a cache
    # left warm by the previous one
    sets = [build_rows(inp, mode=args.variant, dtype=args.dtype) for _ in range(args.buffer_sets)]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    set_calls = [[c for wl in wls.values() for c in wl.calls(stream)] for wls in sets]
    calls = set_calls[0]  # rows, kernels and bytes are the same in every set
    step_bytes = sum(b for _, _, b, _ in calls)

    def step_fns(i):
        return [fn for _, _, _, fn in set_calls[i % len(set_calls)]]

    if args.calibrate_copy_mib:
        # a plain device copy of known size, for scaling the HBM byte counters
        n = int(args.calibrate_copy_mib * MIB)
        a = torch.ones(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    print(f"[bench] warmup {args.warmup} steps, then 2 x {args.steps} timed steps, {len(calls)} launches per step",
          file=sys.stderr, flush=True)
    t = time_launches(step_fns, calls, args.steps, args.warmup, stream)
    ms_step = t["ms_step"]
    print(f"[bench] timed {args.steps} steps: {ms_step:.4f} ms/step (wall {t['wall_s']:.3f} s)", file=sys.stderr,
          flush=True)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "pct_of_peak": round(100.0 * value / PEAK_GBS, 2),
        "config": {
            "workload": workload_name(args.message_mib, args.dtype, args.ragged_a2a),
            "variant": args.variant,
            "variant_means": VARIANTS[args.variant],
            "message_bytes": M,
            "launches_per_step": len(calls),
            "algorithmic_bytes_per_step": step_bytes,
            "buffer_sets": args.buffer_sets,
            "inputs": ("drawn on the device (seeded), timing only" if args.device_inputs else
                       "seeded host arrays (pack_rr_helper_amd.synth), uploaded before timing"),
            "timed_region_1": "K steps, no events between launches (value, ms_per_step)",
            **rows_of(t),
            "launch_order": [row for row, _, _, _ in calls],
            **({"library": CUSTOM_LIBRARY} if CUSTOM_LIBRARY else {}),
        },
        "roofline": roofline_of(t, args.steps, args.message_mib, args.variant, args.dtype,
                                workload_name(args.message_mib, args.dtype, args.ragged_a2a)),
        "cpu_baseline": None,
    }
    if not args.no_other_variants:
        # the same inputs and K steps with each role's launch covering the
        # jobs of the other variants (first timed region only)
        result["other_variants"] = {}
        for other in VARIANTS:
            if other != args.variant:
                print(f"[bench] timing the {other} variant", file=sys.stderr, flush=True)
                result["other_variants"][other] = time_variant(inp, other, args.steps, args.warmup, stream,
                                                               args.buffer_sets, args.dtype)
    if not args.no_other_variants:
        # the same launch sequence as plain stream kernels of each launch's
        # read/write mix and bytes (bench_calib.hip), timed like timed region 1
        print("[bench] timing the plain-stream stand-in steps", file=sys.stderr, flush=True)
        result["stand_in_step"] = {
            "what": ("the same launch sequence with every launch replaced by a plain stream kernel "
                     "(bench_calib.hip) of its read/write mix and bytes, in each of the calibration's access "
                     "patterns, with the fastest pattern per launch, and with the library's own store "
                     "policy per launch, timed like timed region 1; relay_over_stand_in compares with the "
                     "fastest of them"),
            "unit": "GB/s",
            **stand_in_ceiling(calls, args.buffer_sets, stream, args.steps, args.warmup, value, args.ragged_a2a)}
    if args.sizes:
        # the same step at the larger messages of the configurations (the A=4
        # allreduce's 256 MiB, the all-to-all's 1 GiB), one GPU's share and
        # the whole group, each with its own roofline block
        del sets, set_calls, calls
        torch.cuda.empty_cache()
        result["sizes"] = []
        for mib in [float(v) for v in args.sizes.split(",")]:
            for variant in ("share", "group"):
                print(f"[bench] {mib:g} MiB message, {variant} variant", file=sys.stderr, flush=True)
                result["sizes"].append(size_block(mib, variant, args.steps, args.warmup, stream, args.dtype))
    if not args.no_cpu_baseline and not args.device_inputs:
        print(f"[bench] timing the CPU oracle on the step's jobs: one thread, then {host_threads()} threads",
              file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(inp, F32_CODE if args.dtype == "f32" else BF16_CODE, args.variant,
                                              label=f"{args.message_mib:g} MiB message, every row, ")
    print(json.dumps(result), flush=True)


# --------------------------------------------------------------------------
# sweep: per-row GB/s at 2 MiB .. 1 GiB
# --------------------------------------------------------------------------

def cache_evictor(torch, mode):
    """A function that pushes a launch's inputs out of the L2 caches and the
    256 MB Infinity Cache before a timed rep: "read" sums a 1 GiB buffer (the
    caches end up holding clean lines), "write" overwrites it (they end up
    holding dirty lines that the timed launch then writes back), "none"
    leaves the caches as the previous rep left them."""
    buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    if mode == "read":
        words = buf.view(torch.int32)
        return lambda: torch.sum(words, dtype=torch.int64)
    if mode == "write":
        return buf.zero_
    return lambda: None


def mode_of(args):
    """The sweep times one launch per role: the job variant sweeps as share."""
    return args.variant if args.variant != "job" else "share"


def sweep(args):
    """Per-role GB/s over message sizes and dtypes: one launch of each role
    (covering the jobs --variant selects), timed back to back over buffer
    sets that rotate through at least 1 GiB (b2b_timer), median and best of
    the trials.  Beside each row: plain streams of the launch's read/write mix
    and bytes in every calibration pattern, timed alike, and the CPU oracle on
    the same jobs."""
    import zlib
    import torch
    import pack_rr_helper_amd as rr
    from pack_rr_helper_amd import workloads as W
    rr.load()
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    times_of = b2b_timer()

    def record(mib, dt_name, role, kernel, b, ts, nsets):
        return {"message_mib": mib, "dtype": dt_name, "variant": mode_of(args), "timing": "back to back",
                "buffer_sets": nsets, "row": role, "kernel": kernel, "bytes_per_launch": b,
                "trials": len(ts), "us_min": round(min(ts) * 1e6, 2),
                "us_median": round(statistics.median(ts) * 1e6, 2),
                "gbs_best": round(b / min(ts) / 1e9, 1),
                "gbs_median": round(b / statistics.median(ts) / 1e9, 1),
                "pct_peak_median": round(100 * b / statistics.median(ts) / 1e9 / PEAK_GBS, 1)}

    out = open(args.sweep_out, "w") if args.sweep_out else sys.stdout
    gen = torch.Generator(device="cuda")
    oracle_cache = {}
    dtypes = {"bf16": (rr.BF16, torch.bfloat16, torch.int16), "f32": (rr.F32, torch.float32, torch.int32)}
    for mib in [float(v) for v in args.sweep_sizes.split(",")]:
        M = int(mib * MIB)
        for dt_name in args.sweep_dtypes.split(","):
            dt, tdt, bits_dt = dtypes[dt_name]
            n = M // W.ESIZE[dt]
            orates = {}
            if not args.no_cpu_baseline:
                # the oracle beside every row, on a sample of at most 64 MiB (its
                # rate does not depend on the message size past the host caches)
                sample = min(M, 64 * MIB)
                key = (dt_name, sample)
                if key not in oracle_cache:
                    print(f"[sweep] timing the CPU oracle per role, {dt_name}, {sample / MIB:g} MiB",
                          file=sys.stderr, flush=True)
                    oracle_cache[key] = oracle_role_rates(sample, dt_name, mode_of(args))
                orates = oracle_cache[key]
            for row in args.sweep_rows.split(","):
                gen.manual_seed(zlib.crc32(f"{row}/{dt_name}/{M}".encode()))
                base = row.split("_")[0]
                ranks = 2 if base in ("ar2", "rs2") else 4
                mode = mode_of(args)

                def make_xs():
                    if row.startswith("a2a"):
                        # ragged: segmentCount = 5 mod 8, so odd destinations' chunks sit
                        # at byte offsets that disagree with the packed buffer modulo 16
                        nr = n if row == "a2a" else 4 * (n // 4 - 3)
                        lim = 1 << (8 * W.ESIZE[dt] - 1)
                        return [torch.randint(-lim, lim - 1, (nr,), dtype=bits_dt, device="cuda", generator=gen)
                                for _ in range(ranks)]
                    if row.endswith("_shifted"):
                        # rank r's input starts 2r + 1 elements into its buffer: every
                        # input sits at another offset modulo 16 bytes
                        return [torch.randn(n + 16, device="cuda", generator=gen).to(tdt)[2 * r + 1:2 * r + 1 + n]
                                for r in range(ranks)]
                    return [torch.randn(n, device="cuda", generator=gen).to(tdt) for _ in range(ranks)]

                def make_wl(xs):
                    return {"ar2": lambda: W.AR2(xs, dt, rr.AVG, mode=mode),
                            "rs2": lambda: W.RS2(xs, dt, rr.AVG, mode=mode),
                            "ar4": lambda: W.AR4(xs, dt, rr.AVG, mode=mode, phase=row == "ar4_phase"),
                            "rs4": lambda: W.RS4(xs, dt, rr.SUM, mode=mode),
                            "a2a": lambda: W.A2A(xs, dt, mode=mode)}[base]()

                wls = [make_wl(make_xs())]
                calls0 = wls[0].calls(stream)
                nsets = rotation_sets(sum(c[2] for c in calls0))
                wls += [make_wl(make_xs()) for _ in range(nsets - 1)]
                set_calls = [wl.calls(stream) for wl in wls]
                suffix = "" if row == "ar4_phase" else row[len(base):]
                for role in sorted({c[0] for c in calls0}):
                    idx = next(i for i, c in enumerate(calls0) if c[0] == role)
                    role_call = calls0[idx]
                    name = role + suffix
                    rec = record(mib, dt_name, name, role_call[1], role_call[2],
                                 times_of([sc[idx][3] for sc in set_calls]), nsets)
                    # plain streams of this launch's read/write mix and bytes in every
                    # access pattern of the calibration, timed alike; the fastest is
                    # the ceiling the row is compared with
                    pats, k = {}, rotation_sets(role_call[2])
                    for pi, pname in enumerate(CALIB_PATTERNS):
                        st_sets, st_launch, st_bytes = stand_in_step([role_call], k, stream, pi)
                        pats[pname] = round(st_bytes / statistics.median(times_of([fs[0] for fs in st_sets])) / 1e9, 1)
                        del st_sets
                    top = max(pats, key=pats.get)
                    rec["stand_in"] = {"reads": st_launch[0][1], "writes": st_launch[0][2], "bytes": st_bytes,
                                       "gbs_median": pats[top], "pattern": top, "patterns": pats,
                                       "relay_over_stand_in": round(rec["gbs_median"] / pats[top], 3),
                                       "relay_over_relay_pattern": round(rec["gbs_median"] / pats["relay"], 3)}
                    # a realigned view changes where the data sits, not the oracle's work
                    oname = name if name in orates else role
                    if oname in orates:
                        o = dict(orates[oname])
                        o["gpu_over_oracle"] = round(rec["gbs_median"] / o["gbs"], 1)
                        rec["oracle"] = o
                    print(json.dumps(rec), file=out, flush=True)
                del wls, set_calls, calls0
                torch.cuda.empty_cache()
        # calibration: the runtime's own device-to-device copy of M bytes
        k = rotation_sets(2 * M)
        pairs = [(torch.empty(M, dtype=torch.uint8, device="cuda"), torch.empty(M, dtype=torch.uint8, device="cuda"))
                 for _ in range(k)]
        rec = record(mib, "u8", "torch_copy_calibration", "hipMemcpyAsync D2D", 2 * M,
                     times_of([(lambda a=a, bb=bb: bb.copy_(a)) for a, bb in pairs]), k)
        print(json.dumps(rec), file=out, flush=True)
        del pairs
        torch.cuda.empty_cache()


# --------------------------------------------------------------------------
# calibration: what plain streams of each read/write mix reach on this GPU
# --------------------------------------------------------------------------

CALIB_MIXES = [(1, 0), (2, 0), (4, 0), (0, 1), (1, 1), (2, 1), (3, 1), (4, 1), (2, 2)]
# bench_calib.hip's access patterns, by index: the relay reductions' own (16
# KiB tiles, one per workgroup, non-temporal), smaller tiles, several tiles per
# workgroup with the next tile's loads before the current stores, a persistent
# double-buffered grid, write-back stores, and agent-scope (write-through)
# stores with 16 and 8 KiB tiles (the relay copies' stores)
CALIB_PATTERNS = ["relay", "tile8k", "tile4k", "multi2", "multi4", "persistent", "persist_wb", "relay_wb",
                  "relay_wt", "tile8k_wt"]


def calibrate(args):
    """R reads + W writes per element (bench_calib.hip) in every access
    pattern of CALIB_PATTERNS, each timed back to back over buffer sets that
    rotate through at least 1 GiB (b2b_timer: no cache clearing, no event per
    launch), median and best of the trials per pattern, then one line per
    (size, mix) naming the fastest pattern by median: the ceiling for that
    mix.  --calibrate-alone times each launch alone after a 1 GiB read
    instead (the method of the per-role sweep before), which lets written
    data still sit in the Infinity Cache when a kernel ends."""
    import ctypes
    import functools
    import torch
    lib = _calib_lib()
    torch.cuda.set_device(0)
    vp = ctypes.c_void_p
    stream = torch.cuda.current_stream()
    sp = vp(stream.cuda_stream)
    if args.calibrate_alone:
        alone = alone_timer(cache_evictor(torch, args.flush), reps=args.sweep_reps, warm=3)
        times_of = lambda fns: alone(fns[0])
    else:
        times_of = b2b_timer()
    sink = torch.zeros(16, dtype=torch.uint8, device="cuda")
    out = open(args.calibrate_out, "w") if args.calibrate_out else sys.stdout
    for mib in [int(v) for v in args.calibrate_sizes.split(",")]:
        vectors = (mib * MIB // 16) // 1024 * 1024
        for R, W in CALIB_MIXES:
            b = (R + W) * vectors * 16
            nsets = 1 if args.calibrate_alone else rotation_sets(b)
            sets = []
            for _ in range(nsets):
                bufs = [torch.ones(vectors * 16, dtype=torch.uint8, device="cuda") for _ in range(R + W)]
                ins = (vp * 4)(*([x.data_ptr() for x in bufs[:R]] + [0] * (4 - R)))
                outs = (vp * 4)(*([x.data_ptr() for x in bufs[R:]] + [0] * (4 - W)))
                sets.append((bufs, ins, outs))
            best = None
            for pi, pname in enumerate(CALIB_PATTERNS):
                def launch(ins, outs, pi=pi):
                    rc = lib.calib_stream_pattern(pi, R, W, ins, outs, vp(sink.data_ptr()), vectors, sp)
                    if rc != 0:
                        raise RuntimeError(f"calib_stream_pattern({pi}, {R}, {W}) failed: {rc}")
                ts = times_of([functools.partial(launch, ins, outs) for _, ins, outs in sets])
                rec = {"mib_per_stream": mib, "reads": R, "writes": W, "pattern": pname,
                       "timing": "alone" if args.calibrate_alone else "back to back", "buffer_sets": nsets,
                       "bytes": b, "trials": len(ts),
                       "gbs_best": round(b / min(ts) / 1e9, 1),
                       "gbs_median": round(b / statistics.median(ts) / 1e9, 1),
                       "pct_peak_median": round(100 * b / statistics.median(ts) / 1e9 / PEAK_GBS, 1)}
                print(json.dumps(rec), file=out, flush=True)
                if best is None or rec["gbs_median"] > best["gbs_median"]:
                    best = rec
            print(json.dumps({"mib_per_stream": mib, "reads": R, "writes": W, "ceiling": True,
                              "best_pattern": best["pattern"], "gbs_median": best["gbs_median"],
                              "pct_peak_median": best["pct_peak_median"]}), file=out, flush=True)
            del sets
            torch.cuda.empty_cache()


# Read and write streams per element of each launch of the step, for its
# plain-stream stand-in: a K-input reduction reads K and writes 1; the
# reduce-scatter owner pass mixes 4+1 and 2+1 segments (24 reads to 8 writes
# per chunk), taken as 3+1; a copy reads 1 and writes 1.
STEP_MIX = {"ar2_helper": (2, 1), "ar2_active": (2, 1), "rs2_owner": (2, 1), "ar4_helper": (4, 1),
            "ar4_active": (4, 1), "ar4_phase": (4, 1), "rs4_pass1": (3, 1), "rs4_pass2": (3, 1), "a2a_pack": (1, 1),
            "a2a_unpack": (1, 1)}


def _calib_lib():
    import ctypes
    path = os.path.join(ROOT, "bench_calib.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    lib.calib_stream.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(vp), ctypes.POINTER(vp), vp,
                                 ctypes.c_int64, vp]
    lib.calib_stream_pattern.argtypes = [ctypes.c_int] + lib.calib_stream.argtypes
    lib.calib_fixed.argtypes = [ctypes.c_int, ctypes.c_int64, vp, vp, vp]
    if lib.calib_patterns() != len(CALIB_PATTERNS):
        raise RuntimeError(f"{path} has {lib.calib_patterns()} patterns; rebuild it")
    return lib


def time_steps(step_fns, steps, warmup, stream, host=False):
    """ms per step of K steps back to back (nothing between the launches),
    after the warm-up steps; step_fns(i) gives step i's launches.  host=True
    also returns the host's issue time per step in us (the loop that enqueues
    the K steps, before the final synchronisation)."""
    import torch
    for i in range(warmup):
        for fn in step_fns(i):
            fn()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    h0 = time.perf_counter()
    for i in range(steps):
        for fn in step_fns(i):
            fn()
    h1 = time.perf_counter()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    return (ms, (h1 - h0) * 1e6 / steps) if host else ms


def stand_in_step(calls, nsets, stream, pattern=0):
    """Plain-stream stand-ins for a step's launches (row, kernel, bytes, fn):
    per buffer set, one bench_calib.hip launch per relay launch with the row's
    read/write mix and bytes, in access pattern `pattern` (an index into
    CALIB_PATTERNS, or one per launch).  Returns (per-set launch lists,
    launches as (row, reads, writes, vectors per stream, relay bytes),
    stand-in bytes)."""
    import ctypes
    import functools
    import torch
    lib = _calib_lib()
    vp = ctypes.c_void_p
    sp = vp(stream.cuda_stream)
    sink = torch.zeros(16, dtype=torch.uint8, device="cuda")
    launches = []
    for row, _, b, _ in calls:
        R, W = STEP_MIX[row]
        launches.append((row, R, W, max(1024, round(b / (16 * (R + W)) / 1024) * 1024), b))
    pats = list(pattern) if isinstance(pattern, (list, tuple)) else [pattern] * len(launches)
    sets = []
    for _ in range(nsets):
        fns = []
        for (row, R, W, vectors, _), pat in zip(launches, pats):
            bufs = [torch.empty(vectors * 16, dtype=torch.uint8, device="cuda") for _ in range(R + W)]
            ins = (vp * 4)(*([x.data_ptr() for x in bufs[:R]] + [0] * (4 - R)))
            outs = (vp * 4)(*([x.data_ptr() for x in bufs[R:]] + [0] * (4 - W)))
            fn = functools.partial(lib.calib_stream_pattern, pat, R, W, ins, outs, vp(sink.data_ptr()), vectors, sp)
            fn.keep = (bufs, ins, outs, sink)
            if fn() != 0:
                raise RuntimeError(f"calib_stream_pattern({pat}, {R}, {W}, {vectors}) failed")
            fns.append(fn)
        sets.append(fns)
    return sets, launches, sum((R + W) * v * 16 for _, R, W, v, _ in launches)


def alone_timer(evict, reps, warm=2):
    """A function timing one launch function alone: `reps` times after `warm`
    warm-ups, each after evict() (clearing the caches of its inputs), with a
    fence-free HIP event pair; returns the durations in seconds."""
    import ctypes
    import torch
    hip = hip_runtime()
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    evs = []
    for _ in range(2):
        e = ctypes.c_void_p()
        if hip.hipEventCreateWithFlags(ctypes.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        evs.append(e)
    f = ctypes.c_float()

    def times_of(fn):
        ts = []
        for rep in range(reps + warm):
            evict()
            hip.hipEventRecord(evs[0], sp)
            fn()
            hip.hipEventRecord(evs[1], sp)
            torch.cuda.synchronize()
            hip.hipEventElapsedTime(ctypes.byref(f), evs[0], evs[1])
            if rep >= warm:
                ts.append(f.value * 1e-3)
        return ts
    times_of.events = evs  # kept alive with the function
    return times_of


# Launch sequences timed back to back rotate over buffer sets that together
# hold at least this much (four times the 256 MB Infinity Cache), so that no
# launch finds its inputs, or room for its outputs, left in a cache by the
# launches before it.
ROTATE_BYTES = 1 << 30
MAX_SETS = 256


def rotation_sets(bytes_per_set):
    """Buffer sets for a back-to-back sequence: enough to rotate through
    ROTATE_BYTES, at least 2, at most MAX_SETS."""
    return max(2, min(MAX_SETS, -(-ROTATE_BYTES // max(1, int(bytes_per_set)))))


def b2b_timer(trials=5, min_launches=30):
    """A function timing launches back to back: given one launch function per
    buffer set, it issues max(min_launches, 2 x sets) launches cycling through
    the sets, with one fence-free HIP event pair around them, `trials` times
    after one warm-up pass; returns the seconds per launch of each trial.  No
    per-launch event and no cache clearing: the steady state of a stream of
    launches, as in the benchmark step."""
    import ctypes
    import torch
    hip = hip_runtime()
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    evs = []
    for _ in range(2):
        e = ctypes.c_void_p()
        if hip.hipEventCreateWithFlags(ctypes.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        evs.append(e)
    f = ctypes.c_float()

    def times_of(fns):
        n = max(min_launches, 2 * len(fns))
        for fn in fns:
            fn()
        ts = []
        for _ in range(trials):
            torch.cuda.synchronize()
            hip.hipEventRecord(evs[0], sp)
            for i in range(n):
                fns[i % len(fns)]()
            hip.hipEventRecord(evs[1], sp)
            torch.cuda.synchronize()
            hip.hipEventElapsedTime(ctypes.byref(f), evs[0], evs[1])
            ts.append(f.value * 1e-3 / n)
        return ts
    times_of.events = evs
    return times_of


# the library's copy sizes: calls that move at least COPY_AGENT_MAX_BYTES
# (RR_COPY_AGENT_MAX_BYTES) store non-temporally, those of at least
# COPY_LONG_BYTES (RR_COPY_LONG_BYTES) also take 4 KiB tiles when aligned
COPY_AGENT_MAX_BYTES = 256 << 20
COPY_LONG_BYTES = 512 << 20


def library_patterns(calls, ragged=False):
    """Per launch, the calibration pattern with the relay kernels' own tiles
    and store policy: the reductions 16 KiB tiles, non-temporal stores; the
    copies 8 KiB tiles with agent-scope stores, non-temporal ones from
    COPY_AGENT_MAX_BYTES moved, and from the long-call size 4 KiB tiles (8 KiB
    for a ragged all-to-all)."""
    pats = []
    for row, _, b, _ in calls:
        if row.startswith("a2a"):
            moved = b // 2
            if moved >= COPY_LONG_BYTES:
                name = "tile8k" if ragged else "tile4k"
            else:
                name = "tile8k" if moved >= COPY_AGENT_MAX_BYTES else "tile8k_wt"
        else:
            name = "relay"
        pats.append(CALIB_PATTERNS.index(name))
    return pats


def stand_in_ceiling(calls, nsets, stream, steps, warmup, value, ragged=False):
    """The step's launch sequence replaced by plain streams of each launch's
    read/write mix and bytes, in every access pattern of bench_calib.hip
    (the same pattern for every launch), once with each launch in the
    pattern that ran its mix and bytes fastest (each launch's patterns timed
    back to back over rotating buffer sets), and once with each launch in the
    relay kernels' own tiles and store policy (library_patterns); each step
    timed like timed region 1.  The fastest of these is the ceiling the relay
    step is compared with."""
    import torch
    out = {"patterns": {}}
    for pi, name in enumerate(CALIB_PATTERNS):
        st_sets, _, st_bytes = stand_in_step(calls, nsets, stream, pi)
        ms = time_steps(lambda i: st_sets[i % nsets], steps, warmup, stream)
        gbs = st_bytes / (ms * 1e-3) / 1e9
        out["patterns"][name] = {"value": round(gbs, 1), "pct_of_peak": round(100.0 * gbs / PEAK_GBS, 2),
                                 "ms_per_step": round(ms, 5)}
        del st_sets
        torch.cuda.empty_cache()
    times_of = b2b_timer()
    best = []
    for c in calls:
        med = {}
        k = rotation_sets(c[2])
        for pi in range(len(CALIB_PATTERNS)):
            st_sets, _, _ = stand_in_step([c], k, stream, pi)
            med[pi] = statistics.median(times_of([fs[0] for fs in st_sets]))
            del st_sets
        best.append(min(med, key=med.get))
    torch.cuda.empty_cache()
    st_sets, _, st_bytes = stand_in_step(calls, nsets, stream, best)
    ms = time_steps(lambda i: st_sets[i % nsets], steps, warmup, stream)
    gbs = st_bytes / (ms * 1e-3) / 1e9
    out["best_per_launch"] = {"value": round(gbs, 1), "pct_of_peak": round(100.0 * gbs / PEAK_GBS, 2),
                              "ms_per_step": round(ms, 5),
                              "patterns": {c[0]: CALIB_PATTERNS[b] for c, b in zip(calls, best)}}
    del st_sets
    torch.cuda.empty_cache()
    lib_pats = library_patterns(calls, ragged)
    st_sets, _, st_bytes = stand_in_step(calls, nsets, stream, lib_pats)
    ms = time_steps(lambda i: st_sets[i % nsets], steps, warmup, stream)
    lib_gbs = st_bytes / (ms * 1e-3) / 1e9
    out["library_policy"] = {"value": round(lib_gbs, 1), "pct_of_peak": round(100.0 * lib_gbs / PEAK_GBS, 2),
                             "ms_per_step": round(ms, 5),
                             "patterns": {c[0]: CALIB_PATTERNS[b] for c, b in zip(calls, lib_pats)}}
    del st_sets
    torch.cuda.empty_cache()
    cands = [(v["value"], k) for k, v in out["patterns"].items()] + [(gbs, "best_per_launch"),
                                                                      (lib_gbs, "library_policy")]
    ceil, which = max(cands)
    out["ceiling"] = {"value": round(ceil, 1), "pct_of_peak": round(100.0 * ceil / PEAK_GBS, 2), "from": which}
    out["relay_over_stand_in"] = round(value / ceil, 4)
    out["relay_over_relay_pattern"] = round(value / out["patterns"]["relay"]["value"], 4)
    return out


def calibrate_step(args):
    """The benchmark step beside a stand-in step of plain streams: every
    launch replaced by one bench_calib.hip stream kernel with the same
    read/write mix and the same bytes (to within 16 KiB per stream), timed
    the same way (K steps back to back, the buffer sets in turn), twice in
    alternation.  What the stand-in reaches is what this launch sequence can
    reach on this GPU with the relay kernels' access pattern."""
    import torch
    import pack_rr_helper_amd as rr
    rr.load()
    torch.cuda.set_device(0)
    inp = host_inputs(int(args.message_mib * MIB), args.dtype)
    stream = torch.cuda.current_stream()
    nsets = args.buffer_sets
    sets = [build_rows(inp, mode=args.variant, dtype=args.dtype) for _ in range(nsets)]
    set_calls = [[c for wl in wls.values() for c in wl.calls(stream)] for wls in sets]
    relay_bytes = sum(c[2] for c in set_calls[0])
    stream_sets, launches, stream_bytes = stand_in_step(set_calls[0], nsets, stream)
    relay_ms, stream_ms = [], []
    for _ in range(2):
        relay_ms.append(time_steps(lambda i: [c[3] for c in set_calls[i % nsets]], args.steps, args.warmup, stream))
        stream_ms.append(time_steps(lambda i: stream_sets[i % nsets], args.steps, args.warmup, stream))
    rm, sm = min(relay_ms), min(stream_ms)
    rg, sg = relay_bytes / (rm * 1e-3) / 1e9, stream_bytes / (sm * 1e-3) / 1e9
    print(json.dumps({
        "calibrate_step": True, "message_mib": args.message_mib, "variant": args.variant,
        "buffer_sets": nsets, "steps": args.steps,
        "relay": {"ms_per_step": [round(v, 5) for v in relay_ms], "bytes_per_step": relay_bytes,
                  "gbs": round(rg, 1), "pct_of_peak": round(100 * rg / PEAK_GBS, 2)},
        "streams": {"ms_per_step": [round(v, 5) for v in stream_ms], "bytes_per_step": stream_bytes,
                    "gbs": round(sg, 1), "pct_of_peak": round(100 * sg / PEAK_GBS, 2)},
        "relay_over_streams": round(rg / sg, 4),
        "launches": [{"row": row, "reads": R, "writes": W, "relay_bytes": b, "stream_bytes": (R + W) * v * 16}
                     for row, R, W, v, b in launches],
    }), flush=True)


def graphs_of(step_lists, capture_stream):
    """One HIP graph per list of launches (prepared on capture_stream), each
    run once eagerly first."""
    import torch
    with torch.cuda.stream(capture_stream):
        for fns in step_lists:
            for fn in fns:
                fn()
    torch.cuda.synchronize()
    graphs = []
    for fns in step_lists:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=capture_stream):
            for fn in fns:
                fn()
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def step_sweep(args):
    """The step (one GPU's share and the whole group) and its plain-stream
    stand-in at each message size: K steps back to back, three buffer sets in
    turn while a step moves under 2 GB (one set above: a step then streams far
    more than the 256 MB Infinity Cache holds), issued from Python as one
    prepared call (plan) per launch, as one plan per step (a single C call),
    and replayed from HIP graphs; the host's issue time per step is recorded
    beside the GPU's time per step.  Inputs are drawn on the device (timing
    only).  One JSON line per (size, variant)."""
    import torch
    import pack_rr_helper_amd as rr
    rr.load()
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    out = open(args.sweep_out, "w") if args.sweep_out else sys.stdout
    for mib in [float(v) for v in args.sweep_sizes.split(",")]:
        M = int(mib * MIB)
        inp = device_inputs(M, 1000 + int(mib * 16))
        for variant in ("share", "group"):
            first = build_rows(inp, mode=variant)
            calls0 = [c for wl in first.values() for c in wl.calls(stream)]
            step_bytes = sum(c[2] for c in calls0)
            nsets = 3 if step_bytes < 2e9 else 1
            sets = [first] + [build_rows(inp, mode=variant) for _ in range(nsets - 1)]
            set_calls = [calls0] + [[c for wl in wls.values() for c in wl.calls(stream)] for wls in sets[1:]]
            steps = max(args.steps, 50)
            relay_ms, relay_host = time_steps(lambda i: [c[3] for c in set_calls[i % nsets]], steps, args.warmup,
                                              stream, host=True)
            # one plan per step: every call's recorded launches appended into one
            # plan, issued with a single C call
            step_plans = []
            for sc in set_calls:
                p = rr.Plan(sum(c[3].launches for c in sc))
                with p:
                    pass
                step_plans.append(p.extend(*[c[3] for c in sc]))
            plan_ms, plan_host = time_steps(lambda i: [step_plans[i % nsets]], steps, args.warmup, stream, host=True)
            st_sets, _, st_bytes = stand_in_step(calls0, nsets, stream)
            st_ms = time_steps(lambda i: st_sets[i % nsets], steps, args.warmup, stream)
            # the same steps replayed from HIP graphs (one per buffer set): no
            # host work per launch, so small messages show the GPU's own rate
            cs = torch.cuda.Stream()
            cs.wait_stream(stream)
            relay_cs = [[c[3] for wl in wls.values() for c in wl.calls(cs)] for wls in sets]
            st_cs = stand_in_step(calls0, nsets, cs)[0]  # holds the stand-in buffers the graphs write
            g_relay, g_st = graphs_of(relay_cs, cs), graphs_of(st_cs, cs)
            relay_g_ms = time_steps(lambda i: [g_relay[i % nsets].replay], steps, args.warmup, stream)
            st_g_ms = time_steps(lambda i: [g_st[i % nsets].replay], steps, args.warmup, stream)
            rg, sg = step_bytes / (relay_ms * 1e-3) / 1e9, st_bytes / (st_ms * 1e-3) / 1e9
            rgg, sgg = step_bytes / (relay_g_ms * 1e-3) / 1e9, st_bytes / (st_g_ms * 1e-3) / 1e9
            print(json.dumps({"message_mib": mib, "variant": variant, "buffer_sets": nsets, "steps": steps,
                              "launches": len(calls0), "bytes_per_step": step_bytes,
                              "relay_ms_per_step": round(relay_ms, 5), "relay_gbs": round(rg, 1),
                              "relay_pct_of_peak": round(100 * rg / PEAK_GBS, 2),
                              "relay_host_us_per_step": round(relay_host, 2),
                              "step_plan_ms_per_step": round(plan_ms, 5),
                              "step_plan_gbs": round(step_bytes / (plan_ms * 1e-3) / 1e9, 1),
                              "step_plan_pct_of_peak": round(100 * step_bytes / (plan_ms * 1e-3) / 1e9 / PEAK_GBS, 2),
                              "step_plan_host_us_per_step": round(plan_host, 2),
                              "stand_in_gbs": round(sg, 1), "stand_in_pct_of_peak": round(100 * sg / PEAK_GBS, 2),
                              "relay_over_stand_in": round(rg / sg, 4),
                              "graph_relay_gbs": round(rgg, 1), "graph_relay_pct_of_peak": round(100 * rgg / PEAK_GBS, 2),
                              "graph_stand_in_gbs": round(sgg, 1),
                              "graph_relay_over_stand_in": round(rgg / sgg, 4)}), file=out, flush=True)
            torch.cuda.synchronize()
            del g_relay, g_st          # the graphs go before the buffers they write
            del first, sets, set_calls, calls0, st_sets, relay_cs, st_cs, step_plans
            torch.cuda.empty_cache()
        del inp
        torch.cuda.empty_cache()


# --------------------------------------------------------------------------
# per-role fixed cost and asymptotic bandwidth: t = t0 + bytes / BW
# --------------------------------------------------------------------------

RELAY_KERNEL = re.compile(r"rr::\(anonymous namespace\)::(reduce|copy)\w*kernel")
FIXED_KERNEL = re.compile(r"(empty_kernel|touch_kernel)")  # bench_calib.hip's fixed-cost kernels
EVICT_KERNEL = re.compile(r"at::native::.*reduce_kernel")  # cache_evictor("read"): torch.sum


def linear_fit(xs, ys):
    """Least squares y = a + b*x; returns (a, b, r^2)."""
    n = len(xs)
    mx, my = sum(xs) / n, sum(ys) / n
    sxx = sum((x - mx) ** 2 for x in xs)
    sxy = sum((x - mx) * (y - my) for x, y in zip(xs, ys))
    b = sxy / sxx
    a = my - b * mx
    ss = sum((y - my) ** 2 for y in ys)
    res = sum((y - a - b * x) ** 2 for x, y in zip(xs, ys))
    return a, b, (1.0 - res / ss) if ss > 0 else 1.0


def fit_table(samples, ref_mib=64.0):
    """samples: {role: {message_mib: (bytes, [seconds...])}} -> rows of the
    fit over every size, with the decomposition at ref_mib: the launch's
    fraction of peak = (BW / peak) x (streaming time / (t0 + streaming time))."""
    rows = []
    for role, by in samples.items():
        sizes = sorted(by)
        xs = [by[m][0] for m in sizes]
        ys = [statistics.median(by[m][1]) for m in sizes]
        t0, inv_bw, r2 = linear_fit(xs, ys)
        bw = 1.0 / inv_bw / 1e9 if inv_bw > 0 else float("inf")
        row = {"role": role, "t0_us": round(t0 * 1e6, 3), "bw_gbs": round(bw, 1),
               "bw_pct_of_peak": round(100 * bw / PEAK_GBS, 2), "r2": round(r2, 5),
               "sizes_mib": sizes, "median_us": [round(y * 1e6, 3) for y in ys],
               "bytes": xs, "pct_of_peak": [round(100 * x / y / 1e9 / PEAK_GBS, 2) for x, y in zip(xs, ys)]}
        if ref_mib in by:
            b, y = by[ref_mib][0], statistics.median(by[ref_mib][1])
            stream_t = b * inv_bw
            row["at_ref"] = {"message_mib": ref_mib, "bytes": b, "measured_us": round(y * 1e6, 3),
                             "fit_us": round((t0 + stream_t) * 1e6, 3), "streaming_us": round(stream_t * 1e6, 3),
                             "pct_of_peak": round(100 * b / y / 1e9 / PEAK_GBS, 2),
                             "streaming_share": round(stream_t / (t0 + stream_t), 4)}
        rows.append(row)
    return rows


def role_fit(args):
    """Every launch of the step (one GPU's share, --variant) alone, at each
    --fit-sizes message, --fit-reps times after 2 warm-ups, each rep after a
    1 GiB read that clears the caches of its inputs, timed with a fence-free
    HIP event pair (which adds about 1.2 us to a launch).  Also a one-tile
    reduction launch (the smallest launch the library makes) for the fixed
    cost of a kernel.  Prints the event-timed fit; --fit-log records every
    relay launch in issue order so that a rocprofv3 kernel trace of this run
    can be fitted on kernel durations alone (--fit-trace)."""
    import ctypes
    import torch
    import pack_rr_helper_amd as rr
    rr.load()
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    hip = hip_runtime()
    evs = []
    for _ in range(2):
        e = ctypes.c_void_p()
        if hip.hipEventCreateWithFlags(ctypes.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        evs.append(e)
    f = ctypes.c_float()
    evict = cache_evictor(torch, "read")
    log, samples = [], {}

    def run(role, mib, b, fn):
        for rep in range(args.fit_reps + 2):
            evict()
            hip.hipEventRecord(evs[0], sp)
            fn()
            hip.hipEventRecord(evs[1], sp)
            torch.cuda.synchronize()
            hip.hipEventElapsedTime(ctypes.byref(f), evs[0], evs[1])
            log.append({"role": role, "message_mib": mib, "bytes": b, "warmup": rep < 2})
            if rep >= 2:
                samples.setdefault(role, {}).setdefault(mib, (b, []))[1].append(f.value * 1e-3)

    # the smallest launch: one tile of a two-input bf16 reduction (A=2 helper,
    # count = 8 chunks of 128 elements)
    tiny = [torch.randn(1024, device="cuda").to(torch.bfloat16) for _ in range(2)]
    tiny_out = torch.empty(128, dtype=torch.bfloat16, device="cuda")
    relay = rr.Relay(2, 6, 8, 0, 1024)
    tiny_fn = rr.rr_helper_reduce(relay, rr.ALLREDUCE, rr.BF16, rr.SUM, 0, [t[:128] for t in tiny], tiny_out,
                                  prepare=True)
    run("one_tile", 0.0, 3 * 128 * 2, tiny_fn)
    # a launch's fixed cost apart from the relay kernels: workgroups that touch
    # no memory, or load or store one 16-byte vector per lane (bench_calib.hip)
    lib = _calib_lib()
    buf = torch.empty(2048 * 4096, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(16, dtype=torch.uint8, device="cuda")
    for kind, name in ((0, "empty"), (1, "load_only"), (2, "store_only")):
        for blocks in (1, 2048):
            def fixed(kind=kind, blocks=blocks):
                if lib.calib_fixed(kind, blocks, ctypes.c_void_p(buf.data_ptr()), ctypes.c_void_p(sink.data_ptr()),
                                   sp) != 0:
                    raise RuntimeError("calib_fixed failed")
            run(f"{name}_{blocks}wg", 0.0, 0 if kind == 0 else blocks * 4096, fixed)
    print(f"[fit] one-tile launch: {statistics.median(samples['one_tile'][0.0][1]) * 1e6:.2f} us (event pair)",
          file=sys.stderr, flush=True)
    for mib in [float(v) for v in args.fit_sizes.split(",")]:
        M = int(mib * MIB)
        inp = device_inputs(M, 2000 + int(mib * 16))
        wls = build_rows(inp, mode=mode_of(args))
        del inp
        calls = [c for wl in wls.values() for c in wl.calls(stream)]
        for row, _, b, fn in calls:
            run(row, mib, b, fn)
        print(f"[fit] {mib:g} MiB: " + ", ".join(
            f"{row} {statistics.median(samples[row][mib][1]) * 1e6:.2f} us" for row, _, _, _ in calls),
            file=sys.stderr, flush=True)
        del wls, calls
        torch.cuda.empty_cache()
    for e in evs:
        hip.hipEventDestroy(e)
    if args.fit_log:
        with open(args.fit_log, "w") as fh:
            json.dump({"variant": mode_of(args), "launches": log}, fh)
    by_role = {r: v for r, v in samples.items() if r != "one_tile" and not r.endswith("wg")}
    print(json.dumps({"role_fit": True, "timing": "fence-free HIP event pair per launch (adds ~1.2 us)",
                      "variant": mode_of(args), "reps": args.fit_reps,
                      "one_tile_us": round(statistics.median(samples["one_tile"][0.0][1]) * 1e6, 3),
                      "roles": fit_table(by_role)}), flush=True)


def fit_from_trace(args):
    """Fit t = t0 + bytes/BW per role on the kernel durations of a rocprofv3
    kernel trace (End - Start of each dispatch) of a --role-fit run, matched
    launch by launch with that run's --fit-log; prints a markdown table."""
    import csv
    with open(args.fit_log) as fh:
        log = json.load(fh)
    with open(args.fit_trace) as fh:
        rows = sorted(csv.DictReader(fh), key=lambda r: int(r["Dispatch_Id"]))
    # every timed launch directly follows the cache-clearing read (a torch sum);
    # relay launches made while a workload stages its inputs do not
    relay = [r for prev, r in zip(rows, rows[1:])
             if (RELAY_KERNEL.search(r["Kernel_Name"]) or FIXED_KERNEL.search(r["Kernel_Name"]))
             and EVICT_KERNEL.search(prev["Kernel_Name"])]
    launches = log["launches"]
    if len(relay) != len(launches):
        raise SystemExit(f"trace holds {len(relay)} timed relay dispatches, the log {len(launches)} launches")
    samples, kernels = {}, {}
    for r, l in zip(relay, launches):
        if l["warmup"]:
            continue
        t = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
        samples.setdefault(l["role"], {}).setdefault(l["message_mib"], (l["bytes"], []))[1].append(t)
        kernels.setdefault(l["role"], set()).add(re.sub(r"^void rr::\(anonymous namespace\)::", "",
                                                        r["Kernel_Name"]).split("(")[0])
    tiny = samples.pop("one_tile", {})
    fixed = {r: statistics.median(samples.pop(r)[0.0][1]) * 1e6 for r in list(samples) if r.endswith("wg")}
    if getattr(args, "fit_min_mib", 0):
        samples = {r: {m: v for m, v in by.items() if m >= args.fit_min_mib} for r, by in samples.items()}
    fit = fit_table(samples)
    if args.sweep_out:
        with open(args.sweep_out, "w") as fh:
            json.dump({"variant": log["variant"], "one_tile_us": round(statistics.median(tiny[0.0][1]) * 1e6, 3)
                       if tiny else None, "fixed_us": {k: round(v, 3) for k, v in fixed.items()}, "roles": fit}, fh)
    print(f"one-tile reduction launch (kernel duration, median): "
          f"{statistics.median(tiny[0.0][1]) * 1e6:.2f} us\n" if tiny else "")
    if fixed:
        print("| fixed-cost kernel | kernel us (median) |")
        print("|---|---:|")
        for name, us in fixed.items():
            print(f"| {name} | {us:.2f} |")
        print()
    print("| role | kernel | t0 us | BW GB/s | BW % of peak | r^2 | " +
          " | ".join(f"{m:g} MiB us (% peak)" for m in fit[0]["sizes_mib"]) + " |")
    print("|---|---|---:|---:|---:|---:|" + "---:|" * len(fit[0]["sizes_mib"]))
    for row in fit:
        print(f"| {row['role']} | {', '.join(sorted(kernels[row['role']]))} | {row['t0_us']:.2f} | "
              f"{row['bw_gbs']:.0f} | {row['bw_pct_of_peak']:.1f} | {row['r2']:.4f} | " +
              " | ".join(f"{u:.2f} ({p:.1f})" for u, p in zip(row["median_us"], row["pct_of_peak"])) + " |")
    print()
    print("| role at 64 MiB | bytes | measured us | t0 us | bytes/BW us | % of peak | = BW % of peak | x streaming share |")
    print("|---|---:|---:|---:|---:|---:|---:|---:|")
    for row in fit:
        a = row.get("at_ref")
        if a:
            print(f"| {row['role']} | {a['bytes']} | {a['measured_us']:.2f} | {row['t0_us']:.2f} | "
                  f"{a['streaming_us']:.2f} | {a['pct_of_peak']:.1f} | {row['bw_pct_of_peak']:.1f} | "
                  f"{a['streaming_share']:.3f} |")


def main():
    args = parse()
    if args.library:
        global CUSTOM_LIBRARY
        import pack_rr_helper_amd
        pack_rr_helper_amd.library_path = os.path.abspath(args.library)
        rel = os.path.relpath(pack_rr_helper_amd.library_path, ROOT)
        CUSTOM_LIBRARY = pack_rr_helper_amd.library_path if rel.startswith("..") else rel
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (--gpus {args.gpus} "
              "requested). The relay's local kernels shard per rank; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.sweep_summary:
        sweep_summary(args)
    elif args.trace_summary:
        trace_summary(args)
    elif args.traffic_from:
        traffic_from(args)
    elif args.fit_trace:
        fit_from_trace(args)
    elif args.role_fit:
        role_fit(args)
    elif args.step_sweep:
        step_sweep(args)
    elif args.sweep:
        sweep(args)
    elif args.calibrate_step:
        calibrate_step(args)
    elif args.calibrate:
        calibrate(args)
    else:
        step_bench(args)


if __name__ == "__main__":
    main()
