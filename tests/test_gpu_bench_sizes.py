"""Parity at the benchmark's larger message sizes, 256 MiB and 1 GiB per rank
in bf16, in the launch configuration bench.py times for them: inputs drawn on
the device with the benchmark's seeds, the rows built and issued as its timed
step issues them, for one GPU's share and for the whole group.  Every output
holds a sentinel before the step runs (tests/benchrows.py).

The outputs are too large for the oracle to recompute whole inside a test, so
each output region the step writes is sampled in windows of 4096 elements
(its first and last, and windows across 16 KiB tile boundaries at seeded
offsets), read back by slicing, and compared bit for bit with the oracle:

* steps that are element-wise by definition -- the helpers' folds, the A=2
  reduce-scatter owner, the A=4 reduce-scatter pass 1 (output chunk o,
  element i folds the scratch's (o, j) chunks at element i) -- are evaluated
  by the oracle on the same windows of their inputs;
* steps whose layout follows the full geometry -- the actives' direct
  regions, the A=4 reduce-scatter pass 2, all-to-all pack and unpack -- are
  evaluated by the oracle at full size on host inputs that hold the device's
  values at the windows the compared outputs read and zero elsewhere.  A
  window whose expected bytes are all zero is taken as a sampling mistake
  and fails, except where the step must leave the output untouched.

Pass 2 takes as inputs the reduced chunks the device's pass 1 wrote, as the
owner receives them; pass 1 itself is checked on its own windows.
"""
import numpy as np
import pytest
import torch

import bench
from pack_rr_helper_amd import synth
from tests.benchrows import poison_outputs

pytestmark = pytest.mark.gpu
BF16, SUM, AVG = 1, 0, 1
WIN = 4096     # elements per window
TILE = 8192    # bf16 elements in a 16 KiB tile


def say(*a):
    print("[gpu-case]", *a, flush=True)


def spots(lo, hi, seed, n=6):
    """Windows [a, b) inside [lo, hi): the first and the last WIN elements and
    n more centred on tile boundaries counted from lo, at seeded tiles."""
    if hi - lo <= 2 * WIN:
        return [(lo, hi)] if hi > lo else []
    rng = np.random.default_rng(seed)
    starts = {lo, hi - WIN}
    tiles = (hi - lo) // TILE
    if tiles > 1:
        for t in rng.integers(1, tiles, size=n):
            s = lo + int(t) * TILE - WIN // 2
            if lo <= s and s + WIN <= hi:
                starts.add(s)
    return sorted((s, s + WIN) for s in starts)


def win(t, a, b):
    return synth.to_host(t[a:b])


def sparse(t, ws, base=0, n=None):
    """Host copy of t[base:base + n] holding the device's values at the
    windows ws (relative to base) and zero elsewhere."""
    n = t.numel() - base if n is None else n
    h = np.zeros(n, np.uint16)
    for a, b in ws:
        h[a:b] = win(t, base + a, base + b)
    return h


def same(got, ref, what, nonzero=True):
    got, ref = got.view(np.uint16), ref.view(np.uint16)
    assert got.shape == ref.shape, what
    if nonzero:
        assert np.any(ref != 0), f"{what}: expected window is all zero (sampling mistake)"
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, f"{what}: {bad.size} of {got.size} elements differ, first at {bad[:1]}"


@pytest.fixture(scope="module", autouse=True)
def device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import pack_rr_helper_amd as rr
    rr.load()
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mib,variant", [(256, "share"), (256, "group"), (1024, "share"), (1024, "group")])
def test_benchmark_step_at_large_messages(orc, mib, variant):
    say(f"bench step {mib} MiB, {variant}, bf16: building rows")
    M = mib << 20
    share = variant == "share"
    inp = bench.device_inputs(M, 3000 + mib * 16, "bf16")   # the seed the benchmark's size block uses
    wls = bench.build_rows(inp, mode=variant, dtype="bf16")
    del inp
    assert len([c for w in wls.values() for c in w.calls()]) == 8
    poison_outputs(wls, share)
    say(f"bench step {mib} MiB, {variant}: running the step")
    for w in wls.values():
        w.run()
    torch.cuda.synchronize()
    say(f"bench step {mib} MiB, {variant}: comparing windows")
    seed = mib + (0 if share else 1)

    # A=2 allreduce: helper folds (element-wise), then the actives' direct regions
    ar2 = wls["ar2"]
    x, c, n = ar2.x, ar2.g["chunk"], ar2.count
    for k in range(3 if share else 6):
        for a, b in spots(0, c, seed + k):
            ref = orc.ar2_helper(BF16, AVG, win(x[0], k * c + a, k * c + b), win(x[1], k * c + a, k * c + b))
            same(win(ar2.red[k], a, b), ref, f"ar2 helper {k} [{a}, {b})")
    lo = ar2.g["direct_off"]
    ws = spots(lo, n, seed + 10)
    xs = [sparse(v, ws) for v in x]
    for act in range(1 if share else 2):
        ref = orc.ar_active(BF16, AVG, 2, 6, 8, 0, n, act, xs, np.zeros(n, np.uint16))
        for a, b in ws:
            same(win(ar2.out[act], a, b), ref[a:b], f"ar2 active {act} [{a}, {b})")
    del xs

    # A=2 reduce-scatter owners (element-wise over the owner's block)
    rs2 = wls["rs2"]
    R = rs2.R
    for o in range(1 if share else 2):
        for a, b in spots(0, R, seed + 20 + o):
            ref = orc.rs2_active(BF16, AVG, win(rs2.x[0], o * R + a, o * R + b), win(rs2.x[1], o * R + a, o * R + b))
            same(win(rs2.out[o], a, b), ref, f"rs2 owner {o} [{a}, {b})")

    # A=4 allreduce: helper slices (element-wise) and the actives' direct slices
    ar4 = wls["ar4"]
    x, g, n = ar4.x, ar4.g, ar4.count
    c = g["chunk"]
    for h in range(1 if share else 4):
        for a, b in spots(0, c, seed + 30 + h):
            ref = orc.ar4_helper(BF16, AVG, [win(v, h * c + a, h * c + b) for v in x])
            same(win(ar4.red[h], a, b), ref, f"ar4 helper {h} [{a}, {b})")
    for act in range(1 if share else 4):
        lo = g["direct_off"] + act * g["dslice"]
        hi = lo + g["dslice"] if act < 3 else n
        ws = spots(lo, hi, seed + 40 + act)
        xs = [sparse(v, ws) for v in x]
        ref = orc.ar_active(BF16, AVG, 4, 4, 0, 500, n, act, xs, np.zeros(n, np.uint16))
        for a, b in ws:
            same(win(ar4.out[act], a, b), ref[a:b], f"ar4 active {act} [{a}, {b})")
        del xs, ref

    # A=4 reduce-scatter: pass 1 per helper (element-wise per chunk), pass 2 per owner
    rs4 = wls["rs4"]
    R, c = rs4.R, rs4.g["chunk"]
    for h in range(1 if share else 4):
        sc = rs4.scratch[h]
        for a, b in spots(0, c, seed + 50 + h):
            hs = np.concatenate([win(sc, q * c + a, q * c + b) for q in range(12)])
            got = np.concatenate([win(sc, (12 + o) * c + a, (12 + o) * c + b) for o in range(4)])
            same(got, orc.rs4_pass1(BF16, 4, b - a, hs), f"rs4 pass1 helper {h} [{a}, {b})")
    for o in range(1 if share else 4):
        ws = sorted(set(spots(0, R, seed + 60 + o)) | set(spots(0, 4 * c, seed + 64 + o, n=4))
                    | set(spots(4 * c, R, seed + 68 + o, n=2)))
        blk = [sparse(v, ws, base=o * R, n=R) for v in rs4.x]
        red = [synth.to_host(rs4.reduced(h, o)) for h in range(4)]
        ref = orc.rs4_pass2(BF16, SUM, 4, 4, 500, R, o, blk, red)
        for a, b in ws:
            same(win(rs4.out[o], a, b), ref[a:b], f"rs4 owner {o} [{a}, {b})")
        del blk, red, ref

    # A=4 all-to-all: the step's helper slices, packed per destination, then
    # scattered back; the rest of every output stays zero
    a2a = wls["a2a"]
    seg, c = a2a.seg, a2a.g["chunk"]
    helpers = range(1 if share else 4)
    cw = {h: spots(0, c, seed + 70 + h, n=3) for h in helpers}
    src_ws = [[] for _ in range(4)]          # per source: windows its chunks are read at
    for h in helpers:
        for d in range(4):
            for s in range(4):
                if s != d:
                    src_ws[s] += [(d * seg + h * c + a, d * seg + h * c + b) for a, b in cw[h]]
    src = [sparse(a2a.src[s], sorted(set(src_ws[s]))) for s in range(4)]
    expect = [np.zeros(4 * seg, np.uint16) for _ in range(4)]
    for h in helpers:
        packed = orc.a2a_pack(2, 4, seg, c, h, src)
        for d in range(4):
            pk = packed[d].view(np.uint16)
            for j in range(3):
                for a, b in cw[h]:
                    same(win(a2a.packed[h][d], j * c + a, j * c + b), pk[j * c + a:j * c + b],
                         f"a2a pack helper {h} dest {d} chunk {j} [{a}, {b})")
        orc.a2a_unpack(2, 4, seg, c, h, packed, expect)
        del packed
    for d in range(4):
        for s in range(4):
            base = s * seg
            if s != d:
                for h in helpers:
                    for a, b in cw[h]:
                        lo_, hi_ = base + h * c + a, base + h * c + b
                        same(win(a2a.out[d], lo_, hi_), expect[d][lo_:hi_], f"a2a unpack dest {d} src {s} h {h}")
            # outside the step's slices: untouched (zero)
            first_free = base + (len(helpers) * c if s != d else 0)
            for a, b in spots(first_free, base + seg, seed + 80 + 4 * d + s, n=2):
                same(win(a2a.out[d], a, b), expect[d][a:b], f"a2a unpack dest {d} outside [{a}, {b})",
                     nonzero=False)
    del src, expect, wls
    torch.cuda.empty_cache()
    say(f"bench step {mib} MiB, {variant}: bit-exact on every window")
