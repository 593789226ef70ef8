"""Parity in the exact launch configuration bench.py times: the seeded inputs
and launches of one benchmark step at the 64 MiB message, for one GPU's share
(the default) and for the whole-group variant, every output the step writes
against the CPU oracle."""
import numpy as np
import pytest
import torch

import bench
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


@pytest.mark.parametrize("variant", ["share", "group"])
def test_benchmark_step_matches_the_oracle(orc, variant):
    print(f"[gpu-case] bench step 64 MiB, {variant}", flush=True)
    M = 64 << 20
    inp = bench.host_inputs(M)
    wls = bench.build_rows(inp, mode=variant)
    calls = [c for w in wls.values() for c in w.calls()]
    assert len(calls) == 9
    for w in wls.values():
        w.run()
    torch.cuda.synchronize()
    share = variant == "share"
    # A=2 allreduce: helper reductions, then the actives' direct regions
    x = inp["ar2"]
    ar2 = wls["ar2"]
    c = ar2.g["chunk"]
    for k in range(3 if share else 6):
        same(synth.to_host(ar2.red[k])[:c], orc.ar2_helper(BF16, AVG, x[0][k * c:(k + 1) * c], x[1][k * c:(k + 1) * c]),
             f"ar2 helper {k}")
    lo = ar2.g["direct_off"]
    for a in range(1 if share else 2):
        ref = orc.ar_active(BF16, AVG, 2, 6, 8, 0, x[0].size, a, x, np.zeros_like(x[0]))
        same(synth.to_host(ar2.out[a])[lo:], ref[lo:], f"ar2 active {a}")
    # A=2 reduce-scatter owners
    x = inp["rs2"]
    R = x[0].size // 2
    same(synth.to_host(wls["rs2"].out[0]), orc.rs2_active(BF16, AVG, x[0][:R], x[1][:R]), "rs2 owner 0")
    if not share:
        same(synth.to_host(wls["rs2"].out[1]), orc.rs2_active(BF16, AVG, x[0][R:], x[1][R:]), "rs2 owner 1")
    # A=4 allreduce: helper slices and active direct slices
    x = inp["ar4"]
    ar4 = wls["ar4"]
    c, g = ar4.g["chunk"], ar4.g
    for h in range(1 if share else 4):
        same(synth.to_host(ar4.red[h])[:c], orc.ar4_helper(BF16, AVG, [v[h * c:(h + 1) * c] for v in x]), f"ar4 helper {h}")
    for a in range(1 if share else 4):
        ref = orc.ar_active(BF16, AVG, 4, 4, 0, 500, x[0].size, a, x, np.zeros_like(x[0]))
        lo = g["direct_off"] + a * g["dslice"]
        hi = lo + g["dslice"] if a < 3 else x[0].size
        same(synth.to_host(ar4.out[a])[lo:hi], ref[lo:hi], f"ar4 active {a}")
    # A=4 reduce-scatter: helper pass 1 and owner pass 2
    x = inp["rs4"]
    rs4 = wls["rs4"]
    R, c = x[0].size // 4, rs4.g["chunk"]
    for h in range(1 if share else 4):
        hs = np.concatenate([x[s][o * R + h * c:o * R + (h + 1) * c] for o in range(4) for s in range(4) if s != o])
        same(synth.to_host(rs4.scratch[h])[12 * c:16 * c], orc.rs4_pass1(BF16, 4, c, hs), f"rs4 pass1 helper {h}")
    ref = orc.rs4_group(BF16, SUM, 4, 500, R, x)
    for o in range(1 if share else 4):
        same(synth.to_host(rs4.out[o]), ref[o], f"rs4 owner {o}")
    # A=4 all-to-all: pack and unpack of the helper slices the step covers
    x = inp["a2a"]
    a2a = wls["a2a"]
    c, seg = a2a.g["chunk"], a2a.seg
    expect = [np.zeros(4 * seg, np.uint16) for _ in range(4)]
    for h in range(1 if share else 4):
        packed = orc.a2a_pack(2, 4, seg, c, h, x)
        for d in range(4):
            assert np.array_equal(synth.to_host(a2a.packed[h][d])[:3 * c].view(np.uint8), packed[d])
        orc.a2a_unpack(2, 4, seg, c, h, packed, expect)
    for d in range(4):
        assert np.array_equal(synth.to_host(a2a.out[d]), expect[d])
