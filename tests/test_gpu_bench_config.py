"""Parity in the exact launch configuration bench.py times: the seeded inputs
and launches of one benchmark step at the 64 MiB message, for one GPU's share
(the default) and for the whole-group variant, in bf16 and (one GPU's share)
in fp32 as ``--dtype f32`` runs it, every output the step writes against the
CPU oracle, bit for bit.  Outputs hold a sentinel before the step runs
(tests/benchrows.py), so every compared byte was written by the step."""
import numpy as np
import pytest
import torch

import bench
from pack_rr_helper_amd import synth
from tests.benchrows import poison_outputs

pytestmark = pytest.mark.gpu
F32, BF16, SUM, AVG = 0, 1, 0, 1


def same(got, ref, what):
    got, ref = np.ascontiguousarray(got), np.ascontiguousarray(ref)
    assert got.dtype == ref.dtype and got.shape == ref.shape, what
    bad = np.flatnonzero(got.view(np.uint8) != ref.view(np.uint8))
    assert bad.size == 0, f"{what}: {bad.size} bytes differ, first at byte {bad[:1]}"


@pytest.mark.parametrize("variant,dtype", [("share", "bf16"), ("group", "bf16"), ("share", "f32")])
def test_benchmark_step_matches_the_oracle(orc, variant, dtype):
    print(f"[gpu-case] bench step 64 MiB, {variant}, {dtype}", flush=True)
    M = 64 << 20
    DT = F32 if dtype == "f32" else BF16
    inp = bench.host_inputs(M, dtype)
    wls = bench.build_rows(inp, mode=variant, dtype=dtype)
    calls = [c for w in wls.values() for c in w.calls()]
    assert len(calls) == 8   # the A=4 allreduce's helper and active slices share one launch
    share = variant == "share"
    poison_outputs(wls, share)
    for w in wls.values():
        w.run()
    torch.cuda.synchronize()
    # A=2 allreduce: helper reductions, then the actives' direct regions
    x = inp["ar2"]
    ar2 = wls["ar2"]
    c = ar2.g["chunk"]
    for k in range(3 if share else 6):
        same(synth.to_host(ar2.red[k])[:c], orc.ar2_helper(DT, AVG, x[0][k * c:(k + 1) * c], x[1][k * c:(k + 1) * c]),
             f"ar2 helper {k}")
    lo = ar2.g["direct_off"]
    for a in range(1 if share else 2):
        ref = orc.ar_active(DT, AVG, 2, 6, 8, 0, x[0].size, a, x, np.zeros_like(x[0]))
        same(synth.to_host(ar2.out[a])[lo:], ref[lo:], f"ar2 active {a}")
    # A=2 reduce-scatter owners
    x = inp["rs2"]
    R = x[0].size // 2
    same(synth.to_host(wls["rs2"].out[0]), orc.rs2_active(DT, AVG, x[0][:R], x[1][:R]), "rs2 owner 0")
    if not share:
        same(synth.to_host(wls["rs2"].out[1]), orc.rs2_active(DT, AVG, x[0][R:], x[1][R:]), "rs2 owner 1")
    # A=4 allreduce: helper slices and active direct slices
    x = inp["ar4"]
    ar4 = wls["ar4"]
    c, g = ar4.g["chunk"], ar4.g
    for h in range(1 if share else 4):
        same(synth.to_host(ar4.red[h])[:c], orc.ar4_helper(DT, AVG, [v[h * c:(h + 1) * c] for v in x]), f"ar4 helper {h}")
    for a in range(1 if share else 4):
        ref = orc.ar_active(DT, AVG, 4, 4, 0, 500, x[0].size, a, x, np.zeros_like(x[0]))
        lo = g["direct_off"] + a * g["dslice"]
        hi = lo + g["dslice"] if a < 3 else x[0].size
        same(synth.to_host(ar4.out[a])[lo:hi], ref[lo:hi], f"ar4 active {a}")
    # A=4 reduce-scatter: helper pass 1 and owner pass 2
    x = inp["rs4"]
    rs4 = wls["rs4"]
    R, c = x[0].size // 4, rs4.g["chunk"]
    for h in range(1 if share else 4):
        hs = np.concatenate([x[s][o * R + h * c:o * R + (h + 1) * c] for o in range(4) for s in range(4) if s != o])
        same(synth.to_host(rs4.scratch[h])[12 * c:16 * c], orc.rs4_pass1(DT, 4, c, hs), f"rs4 pass1 helper {h}")
    ref = orc.rs4_group(DT, SUM, 4, 500, R, x)
    for o in range(1 if share else 4):
        same(synth.to_host(rs4.out[o]), ref[o], f"rs4 owner {o}")
    # A=4 all-to-all: pack and unpack of the helper slices the step covers
    x = inp["a2a"]
    a2a = wls["a2a"]
    c, seg = a2a.g["chunk"], a2a.seg
    es = x[0].itemsize
    expect = [np.zeros(4 * seg, x[0].dtype) for _ in range(4)]
    for h in range(1 if share else 4):
        packed = orc.a2a_pack(es, 4, seg, c, h, x)
        for d in range(4):
            got = synth.to_host(a2a.packed[h][d])[:3 * c]
            assert np.array_equal(got.view(np.uint8), packed[d].view(np.uint8)), f"a2a pack helper {h} dest {d}"
        orc.a2a_unpack(es, 4, seg, c, h, packed, expect)
    for d in range(4):
        got = synth.to_host(a2a.out[d])
        assert np.array_equal(got.view(np.uint8), expect[d].view(np.uint8)), f"a2a unpack dest {d}"
