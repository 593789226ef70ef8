"""Parity in the exact launch configuration bench.py times: the seeded inputs
and batched launches of one benchmark step at the 64 MiB message, every
row's outputs against the CPU oracle."""
import numpy as np
import pytest
import torch

import bench
import pack_rr_helper_amd as rr
from pack_rr_helper_amd import synth

pytestmark = pytest.mark.gpu
BF16, SUM, AVG = 1, 0, 1


def ords(b):
    b = b.astype(np.int32)
    return np.where(b & 0x8000, 0x8000 - (b & 0x7FFF) - 1, b + 0x8000)


def same(got, ref, what):
    d = np.abs(ords(got) - ords(ref))
    assert d.max() <= 1, what
    assert int(np.sum(d == 0)) == d.size, f"{what}: not bit-exact"


def test_benchmark_step_matches_the_oracle(orc):
    print("[gpu-case] bench step 64 MiB", flush=True)
    M = 64 << 20
    inp = bench.host_inputs(M)
    wls = bench.build_rows(inp)
    for w in wls.values():
        w.run()
    torch.cuda.synchronize()
    # A=2 allreduce: helpers, then actives over the direct region
    x = inp["ar2"]
    ar2 = wls["ar2"]
    c = ar2.g["chunk"]
    for k in range(6):
        same(synth.to_host(ar2.red[k])[:c], orc.ar2_helper(BF16, AVG, x[0][k * c:(k + 1) * c], x[1][k * c:(k + 1) * c]),
             f"ar2 helper {k}")
    lo = ar2.g["direct_off"]
    for a in range(2):
        ref = orc.ar_active(BF16, AVG, 2, 6, 8, 0, x[0].size, a, x, np.zeros_like(x[0]))
        same(synth.to_host(ar2.out[a])[lo:], ref[lo:], f"ar2 active {a}")
    # A=2 reduce-scatter owners
    x = inp["rs2"]
    R = x[0].size // 2
    same(synth.to_host(wls["rs2"].out[0]), orc.rs2_active(BF16, AVG, x[0][:R], x[1][:R]), "rs2 owner 0")
    same(synth.to_host(wls["rs2"].out[1]), orc.rs2_active(BF16, AVG, x[0][R:], x[1][R:]), "rs2 owner 1")
    # A=4 allreduce: helpers and active slices
    x = inp["ar4"]
    ar4 = wls["ar4"]
    c, g = ar4.g["chunk"], ar4.g
    for h in range(4):
        same(synth.to_host(ar4.red[h])[:c], orc.ar4_helper(BF16, AVG, [v[h * c:(h + 1) * c] for v in x]), f"ar4 helper {h}")
    for a in range(4):
        ref = orc.ar_active(BF16, AVG, 4, 4, 0, 500, x[0].size, a, x, np.zeros_like(x[0]))
        lo = g["direct_off"] + a * g["dslice"]
        hi = lo + g["dslice"] if a < 3 else x[0].size
        same(synth.to_host(ar4.out[a])[lo:hi], ref[lo:hi], f"ar4 active {a}")
    # A=4 reduce-scatter: the whole group
    x = inp["rs4"]
    ref = orc.rs4_group(BF16, SUM, 4, 500, x[0].size // 4, x)
    for o in range(4):
        same(synth.to_host(wls["rs4"].out[o]), ref[o], f"rs4 owner {o}")
    # A=4 all-to-all: pack and unpack of every helper slice
    x = inp["a2a"]
    a2a = wls["a2a"]
    c, seg = a2a.g["chunk"], a2a.seg
    expect = [np.zeros(4 * seg, np.uint16) for _ in range(4)]
    for h in range(4):
        packed = orc.a2a_pack(2, 4, seg, c, h, x)
        for d in range(4):
            assert np.array_equal(synth.to_host(a2a.packed[h][d])[:3 * c].view(np.uint8), packed[d])
        orc.a2a_unpack(2, 4, seg, c, h, packed, expect)
    for d in range(4):
        assert np.array_equal(synth.to_host(a2a.out[d]), expect[d])
