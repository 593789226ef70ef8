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
    got = bench.traffic_for(kernel, t["message_mib"], t["variant"])
    if t["kernel_source_digest"] == bench.kernel_source_digest():
        assert got == t["kernels"][kernel]["hbm_bytes_per_launch"]
    else:
        assert got is None          # counters taken on other kernel code
    other = "group" if t["variant"] != "group" else "share"
    assert bench.traffic_for(kernel, t["message_mib"], other) is None
    assert bench.traffic_for(kernel, t["message_mib"] * 2, t["variant"]) is None
    assert bench.traffic_for("no such kernel", t["message_mib"], t["variant"]) is None


def test_more_than_one_gpu_is_refused():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                          capture_output=True, text=True, timeout=120)
    assert proc.returncode == 2
    assert "one GPU" in proc.stderr and proc.stdout == ""
