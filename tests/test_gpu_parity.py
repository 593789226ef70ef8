"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle
on the same seeded bytes.

Tolerances (written here, checked per element):
* pack/unpack: bit-exact;
* fp32 reductions: |gpu - ref| <= 1e-6 * max(|ref|, sum_i |x_i|);
* bf16 reductions: at most 1 unit in the last place (monotone bit order).
Both sides add in fp32 in the same order and round once (round-to-nearest-
even), so the expected outcome is bit-exact; the tests also count and assert
the exactly-equal elements, so a silent drift shows up.  NaN results compare
as NaN (their payload is unspecified).

Full-size cases use the workload classes bench.py times (same entry points,
same arguments).
"""
import numpy as np
import pytest
import torch

import pack_rr_helper_amd as rr
from pack_rr_helper_amd import synth
from pack_rr_helper_amd import workloads as W

pytestmark = pytest.mark.gpu

F32, BF16 = 0, 1
SUM, AVG = 0, 1
AR, RS, A2A = 0, 1, 2


@pytest.fixture(scope="module", autouse=True)
def device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rr.load()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def say(*a):
    print("[gpu-case]", *a, flush=True)


def dev(a, dt=BF16):
    return synth.to_device(a, dt)


def host(t):
    torch.cuda.synchronize()
    return synth.to_host(t)


def ords(b):
    b = b.astype(np.int32)
    return np.where(b & 0x8000, 0x8000 - (b & 0x7FFF) - 1, b + 0x8000)


def check_bf16(got, ref, what):
    assert got.shape == ref.shape, what
    gnan = ((got & 0x7F80) == 0x7F80) & (got & 0x7F != 0)
    rnan = ((ref & 0x7F80) == 0x7F80) & (ref & 0x7F != 0)
    assert np.array_equal(gnan, rnan), f"{what}: NaN positions differ"
    d = np.abs(ords(got[~gnan]) - ords(ref[~rnan]))
    assert d.size == 0 or d.max() <= 1, f"{what}: {int(d.max())} ulp at {int(np.argmax(d))}"
    exact = int(np.sum(d == 0))
    say(what, f"{exact}/{d.size} bit-exact")
    assert exact == d.size, f"{what}: {d.size - exact} elements within 1 ulp but not bit-exact"


def check_f32(got, ref, inputs, what):
    absum = sum(np.abs(x.astype(np.float64)) for x in inputs)
    tol = 1e-6 * np.maximum(np.abs(ref.astype(np.float64)), absum)
    assert np.all(np.abs(got.astype(np.float64) - ref) <= tol), what
    exact = int(np.sum(got.view(np.uint32) == ref.view(np.uint32)))
    say(what, f"{exact}/{got.size} bit-exact")
    assert exact == got.size


# --------------------------------------------------------------------------
# A=2 allreduce helper, fp32, count 2^20, U[-1,1) seed 0, every k
# --------------------------------------------------------------------------

@pytest.mark.parametrize("op", [SUM, AVG])
@pytest.mark.parametrize("in_place", [False, True])
def test_ar2_helper_fp32_every_k(orc, op, in_place):
    count, H, nc = 2 ** 20, 6, 8
    say("ar2 helper fp32", count, op, in_place)
    xs = [synth.uniform(count, -1, 1, 0, a) for a in range(2)]
    dx = [dev(x, F32) for x in xs]
    relay = rr.Relay(2, H, nc, 0, count)
    c = rr.rr_geometry(relay, AR, F32)["chunk"]
    assert c == 131072
    for k in range(H):
        sl = slice(k * c, (k + 1) * c)
        slots = [dx[0][sl].clone(), dx[1][sl].clone()]
        out = slots[0] if in_place else torch.empty(c, dtype=torch.float32, device="cuda")
        rr.rr_helper_reduce(relay, AR, F32, op, k, slots, out)
        ref = orc.ar2_helper(F32, op, xs[0][sl].copy(), xs[1][sl].copy())
        check_f32(host(out), ref, [xs[0][sl], xs[1][sl]], f"k={k}")


# --------------------------------------------------------------------------
# A=2 allreduce group and reduce-scatter, bf16, count 2^25, N(0,1) seed 1
# --------------------------------------------------------------------------

@pytest.mark.parametrize("count", [2 ** 25, 8 * 128 * 37 + 1001, 1000])
def test_ar2_group_bf16(orc, count):
    say("ar2 group bf16", count)
    xs = [synth.as_bf16_bits(synth.normal(count, 1, a)) for a in range(2)]
    wl = W.AR2([dev(x) for x in xs], BF16, AVG)
    wl.run()
    c = wl.g["chunk"]
    for k in range(6):
        if c:
            ref = orc.ar2_helper(BF16, AVG, xs[0][k * c:(k + 1) * c].copy(), xs[1][k * c:(k + 1) * c].copy())
            check_bf16(host(wl.red[k])[:c], ref, f"helper k={k}")
    wl.deliver_returns()
    o0, o1 = orc.ar2_group(BF16, AVG, 6, 8, count, xs[0], xs[1])
    check_bf16(host(wl.out[0]), o0, "active 0 output")
    check_bf16(host(wl.out[1]), o1, "active 1 output")


@pytest.mark.parametrize("R,in_place", [(2 ** 24, False), (2 ** 24, True), (8 * 128 * 9 + 77, False)])
def test_rs2_passthrough_and_owner_bf16(orc, R, in_place):
    say("rs2 bf16", R, in_place)
    xs = [synth.as_bf16_bits(synth.normal(2 * R, 1, a)) for a in range(2)]
    dx = [dev(x) for x in xs]
    relay = rr.Relay(2, 6, 8, 0, R)
    g = rr.rr_geometry(relay, RS, BF16)
    c = g["chunk"]
    # passthrough: the helpers forward slot 0 (a0's block 1) to a1 and slot 1
    # (a1's block 0) to a0 unsummed; the direct exchange completes the blocks
    recv = [torch.empty(R, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    for k in range(6):
        sl = slice(k * c, (k + 1) * c)
        slot0, slot1 = dx[0][R:][sl].clone(), dx[1][:R][sl].clone()
        recv[1][sl].copy_(slot0)
        recv[0][sl].copy_(slot1)
    recv[1][6 * c:].copy_(dx[0][R + 6 * c:])
    recv[0][6 * c:].copy_(dx[1][6 * c:R])
    assert np.array_equal(host(recv[0]), xs[1][:R]) and np.array_equal(host(recv[1]), xs[0][R:])
    with pytest.raises(rr.RRError, match="passthrough"):
        rr.rr_helper_reduce(relay, RS, BF16, AVG, 0, [slot0, slot1], slot0)
    own = [dx[0][:R].clone(), dx[1][R:].clone()]
    outs = own if in_place else [torch.empty(R, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    rr.rr_active_add_scale(relay, RS, BF16, AVG, 0, [own[0], recv[0]], outs[0])
    rr.rr_active_add_scale(relay, RS, BF16, AVG, 1, [recv[1], own[1]], outs[1])
    p0, p1 = orc.rs2_group(BF16, AVG, 6, 8, R, xs[0], xs[1])
    check_bf16(host(outs[0]), p0, "owner 0")
    check_bf16(host(outs[1]), p1, "owner 1")
    # the timed workload reads the peer block in place of the delivered copy
    wl = W.RS2(dx, BF16, AVG)
    wl.run()
    check_bf16(host(wl.out[0]), p0, "workload owner 0")
    check_bf16(host(wl.out[1]), p1, "workload owner 1")


# --------------------------------------------------------------------------
# A=4 reduce-scatter, recvCount 2^22, N(0,1) seed 2
# --------------------------------------------------------------------------

@pytest.mark.parametrize("R", [2 ** 22, 8 * 128 * 11 + 24, 3000])
@pytest.mark.parametrize("op", [SUM, AVG])
def test_rs4_two_passes(orc, R, op):
    say("rs4", R, op)
    A, H = 4, 4
    xs = [synth.as_bf16_bits(synth.normal(A * R, 2, s)) for s in range(A)]
    wl = W.RS4([dev(x) for x in xs], BF16, op)
    c = wl.g["chunk"]
    wl.run()
    for h in range(H):
        if not c:
            break
        # the helper scratch as the scatter fills it, built on the host
        hs = np.concatenate([xs[s][o * R + h * c:o * R + (h + 1) * c]
                             for o in range(A) for s in range(A) if s != o])
        ref = orc.rs4_pass1(BF16, A, c, hs)
        got = host(wl.scratch[h])
        assert np.array_equal(got[:A * (A - 1) * c], hs), "staging"
        check_bf16(got[A * (A - 1) * c:A * A * c], ref, f"pass1 helper {h}")
    outs = orc.rs4_group(BF16, op, H, 500, R, xs)
    for o in range(A):
        check_bf16(host(wl.out[o]), outs[o], f"pass2 owner {o}")


def test_rs4_pass2_in_place(orc):
    A, H, R = 4, 4, 8 * 128 * 5 + 8
    say("rs4 in-place", R)
    blk = [synth.as_bf16_bits(synth.normal(R, 5, s)) for s in range(A)]
    relay = rr.Relay(A, H, 0, 500, R)
    c = rr.rr_geometry(relay, RS, BF16)["chunk"]
    reds = [synth.as_bf16_bits(synth.normal(c, 6, h)) for h in range(H)]
    db, dr = [dev(b) for b in blk], [dev(r) for r in reds]
    rr.rr_rs_multi_reduce(relay, BF16, AVG, 2, 1, db + dr, db[1])
    check_bf16(host(db[1]), orc.rs4_pass2(BF16, AVG, A, H, 500, R, 1, blk, reds), "owner 1 in place")


# --------------------------------------------------------------------------
# A=4 allreduce, count 2^27, U[-2,2) seed 3, 500 permille, 2 MiB floor
# --------------------------------------------------------------------------

@pytest.mark.parametrize("count", [2 ** 27, 2 ** 20, 2 ** 20 - 8, 2 ** 21 + 4 * 128 + 36])
def test_ar4_group(orc, count):
    say("ar4", count)
    xs = [synth.as_bf16_bits(synth.uniform(count, -2, 2, 3, a)) for a in range(4)]
    wl = W.AR4([dev(x) for x in xs], BF16, AVG)
    assert wl.g["pure_direct"] == (count * 2 < 2 * 2 ** 20)
    wl.run()
    c = wl.g["chunk"]
    for h in range(4):
        if c:
            ref = orc.ar4_helper(BF16, AVG, [x[h * c:(h + 1) * c].copy() for x in xs])
            check_bf16(host(wl.red[h])[:c], ref, f"helper {h}")
    wl.deliver()
    outs = orc.ar4_group(BF16, AVG, 4, 500, count, xs)
    for a in range(4):
        check_bf16(host(wl.out[a]), outs[a], f"active {a}")


# --------------------------------------------------------------------------
# A=4 all-to-all pack/unpack, random bits seed 4, 13.5 MiB .. 1 GiB
# --------------------------------------------------------------------------

@pytest.mark.parametrize("M", [1 << 30, int(13.5 * 2 ** 20), 64 * 2 ** 20, 4 * (5 * 128 * 7 + 3) * 2])
def test_a2a_pack_unpack(orc, M):
    A, H, nc = 4, 4, 5
    seg = M // (A * 2)
    say("a2a", M, seg)
    src = [synth.bits16(A * seg, 4, s) for s in range(A)]
    wl = W.A2A([dev(s, None) for s in src], BF16)
    c = wl.g["chunk"]
    wl.run()
    for h in range(H):
        ref = orc.a2a_pack(2, A, seg, c, h, src)
        for d in range(A):
            got = host(wl.packed[h][d])[:(A - 1) * c]
            assert np.array_equal(got.view(np.uint8), ref[d]), f"pack h={h} d={d}"
        del ref
    expect = [np.zeros(A * seg, np.uint16) for _ in range(A)]
    for h in range(H):
        orc.a2a_unpack(2, A, seg, c, h, orc.a2a_pack(2, A, seg, c, h, src), expect)
    for d in range(A):
        assert np.array_equal(host(wl.out[d]), expect[d]), f"unpack d={d}"
    say("a2a bit-exact", M)


# --------------------------------------------------------------------------
# edge cases
# --------------------------------------------------------------------------

def test_misaligned_views_are_realigned(orc):
    say("misaligned")
    count = 8 * 128 * 20 + 13
    xs = [synth.as_bf16_bits(synth.normal(count, 7, a)) for a in range(2)]
    big = [dev(np.concatenate([np.zeros(lead, np.uint16), x, np.zeros(8, np.uint16)]))
           for lead, x in zip((1, 3), xs)]
    views = [big[0][1:1 + count], big[1][3:3 + count]]
    relay = rr.Relay(2, 6, 8, 0, count)
    out = torch.zeros(count + 5, dtype=torch.bfloat16, device="cuda")[5:]
    for a in range(2):
        rr.rr_active_add_scale(relay, AR, BF16, SUM, a, views, out)
        ref = orc.ar_active(BF16, SUM, 2, 6, 8, 0, count, a, xs, np.zeros(count, np.uint16))
        g = rr.rr_geometry(relay, AR, BF16)
        check_bf16(host(out)[g["direct_off"]:], ref[g["direct_off"]:], f"misaligned active {a}")
    # odd segmentCount: source chunks sit at 2-byte offsets from the packed buffers
    A, seg = 4, 5 * 128 * 9 + 5
    src = [synth.bits16(A * seg, 8, s) for s in range(A)]
    wl = W.A2A([dev(s, None) for s in src], BF16)
    wl.run()
    c = wl.g["chunk"]
    for h in range(4):
        ref = orc.a2a_pack(2, A, seg, c, h, src)
        for d in range(A):
            assert np.array_equal(host(wl.packed[h][d])[:(A - 1) * c].view(np.uint8), ref[d])
    expect = [np.zeros(A * seg, np.uint16) for _ in range(A)]
    for h in range(4):
        orc.a2a_unpack(2, A, seg, c, h, orc.a2a_pack(2, A, seg, c, h, src), expect)
    for d in range(A):
        assert np.array_equal(host(wl.out[d]), expect[d])


def _view(host_arr, lead, dt):
    """host_arr placed `lead` elements into a device buffer with 16 guard
    elements on each side; returns (view, whole buffer)."""
    npdt = np.float32 if dt == F32 else np.uint16
    big = np.full(host_arr.size + lead + 32, npdt(0x7FA5) if dt == BF16 else npdt(-3.5), npdt)
    big[16 + lead:16 + lead + host_arr.size] = host_arr
    t = dev(big, dt)
    return t[16 + lead:16 + lead + host_arr.size], t


def _guards_ok(whole, view_lead, n, dt):
    b = host(whole)
    g = np.float32(-3.5) if dt == F32 else np.uint16(0x7FA5)
    return bool(np.all(b[:16 + view_lead] == g) and np.all(b[16 + view_lead + n:] == g))


def test_long_realigned_single_segment_reductions(orc):
    """A realigning reduction of one segment runs in the single-segment form;
    from 4096 tiles (32 MiB of bf16 output) the launch also reserves LDS to
    run fewer workgroups per CU.  The 2-input A=2 reduce-scatter owner and the
    4-input A=4 allreduce helper past that size, inputs and output at
    different element offsets, bit for bit, guards untouched."""
    say("long realigned single-segment reductions")
    vals = lambda n, seed, r: synth.as_bf16_bits(synth.normal(n, seed, r))
    R = (1 << 24) + 8 * 128 * 3 + 77
    relay = rr.Relay(2, 6, 8, 0, R)
    b0, b1 = vals(R, 24, 0), vals(R, 24, 1)
    v0, _ = _view(b0, 5, BF16)
    v1, _ = _view(b1, 2, BF16)
    ov, ow = _view(np.zeros(R, np.uint16), 7, BF16)
    rr.rr_active_add_scale(relay, RS, BF16, AVG, 1, [v0, v1], ov)
    assert np.array_equal(host(ov), orc.rs2_active(BF16, AVG, b0, b1)), "owner"
    assert _guards_ok(ow, 7, R, BF16)
    # the helper reads only its chunk of each input: those chunks are drawn alone
    count = (1 << 27) + 8 * 128 * 3 + 40
    relay = rr.Relay(4, 4, 0, 500, count)
    c = rr.rr_geometry(relay, AR, BF16)["chunk"]
    assert c > 4096 * 4096
    chunks = [vals(c, 26, a) for a in range(4)]
    slots = [_view(x, lead, BF16)[0] for x, lead in zip(chunks, (3, 0, 6, 1))]
    ov, ow = _view(np.zeros(c, np.uint16), 2, BF16)
    rr.rr_helper_reduce(relay, AR, BF16, AVG, 1, slots, ov)
    assert np.array_equal(host(ov), orc.ar4_helper(BF16, AVG, chunks)), "4-input helper"
    assert _guards_ok(ow, 2, c, BF16)


@pytest.mark.parametrize("dt", [BF16, F32])
def test_realigned_reductions_every_input_shift(orc, dt):
    """Reductions whose inputs each start at a different element offset from
    a 16-byte boundary (and from the output): the 4-input A=4 helper, the
    3-input reduce-scatter pass 1 and the 2-input reduce-scatter owner, over
    many realigning tiles and a ragged last one, bit for bit against the
    oracle, with the guard elements around every output untouched."""
    say("realigned reductions", dt)
    es = 4 if dt == F32 else 2
    vals = lambda n, seed, r: synth.normal(n, seed, r) if dt == F32 else synth.as_bf16_bits(synth.normal(n, seed, r))
    # 4 inputs: A=4 allreduce helper 2, chunk of 32+ tiles
    count = (1 << 20) + 8 * 128 * 3
    relay = rr.Relay(4, 4, 0, 500, count)
    c = rr.rr_geometry(relay, AR, dt)["chunk"]
    xs = [vals(count, 20, a) for a in range(4)]
    slots = [_view(x[2 * c:3 * c].copy(), lead, dt)[0] for x, lead in zip(xs, (0, 1, 3, 6))]
    ov, ow = _view(np.zeros(c, xs[0].dtype), 5, dt)
    rr.rr_helper_reduce(relay, AR, dt, AVG, 2, slots, ov)
    ref = orc.ar4_helper(dt, AVG, [x[2 * c:3 * c] for x in xs])
    assert np.array_equal(host(ov).view(np.uint8), ref.view(np.uint8)), "4-input helper"
    assert _guards_ok(ow, 5, c, dt)
    # 3 inputs: reduce-scatter pass 1 over a scratch view at one offset, output at another
    R = 8 * 4096 * 9 + 8 * 128 + 40
    relay = rr.Relay(4, 4, 0, 500, R)
    c = rr.rr_geometry(relay, RS, dt)["chunk"]
    scratch = vals(12 * c, 21, 0)
    sv, _ = _view(scratch, 1, dt)
    ov, ow = _view(np.zeros(4 * c, scratch.dtype), 6, dt)
    rr.rr_rs_multi_reduce(relay, dt, SUM, 1, 0, [sv], ov)
    assert np.array_equal(host(ov).view(np.uint8), orc.rs4_pass1(dt, 4, c, scratch).view(np.uint8)), "pass 1"
    assert _guards_ok(ow, 6, 4 * c, dt)
    # 2 inputs: A=2 reduce-scatter owner, inputs and output at three offsets
    R = 4096 * 7 + 77
    relay = rr.Relay(2, 6, 8, 0, R)
    b0, b1 = vals(R, 22, 0), vals(R, 22, 1)
    v0, _ = _view(b0, 1, dt)
    v1, _ = _view(b1, 6, dt)
    ov, ow = _view(np.zeros(R, b0.dtype), 3, dt)
    rr.rr_active_add_scale(relay, RS, dt, AVG, 0, [v0, v1], ov)
    assert np.array_equal(host(ov).view(np.uint8), orc.rs2_active(dt, AVG, b0, b1).view(np.uint8)), "owner"
    assert _guards_ok(ow, 3, R, dt)


def test_special_values_subnormals_and_infinities(orc):
    say("special values")
    n = 8 * 128 * 8
    rng = np.random.default_rng(9)
    a = rng.integers(0, 1 << 16, n, dtype=np.uint16)
    b = rng.integers(0, 1 << 16, n, dtype=np.uint16)
    a[:512] = rng.integers(0, 0x80, 512)            # positive subnormals
    b[:512] = rng.integers(0x8000, 0x8080, 512)     # negative subnormals
    a[512:520] = 0x7F80                             # +inf
    b[512:520] = 0xFF80                             # -inf -> NaN
    relay = rr.Relay(2, 6, 8, 0, n)
    c = rr.rr_geometry(relay, AR, BF16)["chunk"]
    for op in (SUM, AVG):
        out = torch.empty(c, dtype=torch.bfloat16, device="cuda")
        rr.rr_helper_reduce(relay, AR, BF16, op, 0, [dev(a[:c]), dev(b[:c])], out)
        check_bf16(host(out), orc.ar2_helper(BF16, op, a[:c].copy(), b[:c].copy()), f"special op={op}")


def _special_classes(n, seed, rank, dt):
    """Inputs mixing, element by element, raw random patterns, subnormals, the
    smallest normals (which AVG scales into the subnormal range), the largest
    finite binade (sums overflow to infinity), signed zeros, infinities and
    NaNs: float32 values, or bf16 bit patterns."""
    rng = synth.rng(seed, rank)
    if dt == F32:
        mbits, sbit, u = 23, 31, synth.bits32(n, seed, 100 + rank)
        specials = [0x0, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0xFFA00001, 0x00000001,
                    0x807FFFFF, 0x00800000]
    else:
        mbits, sbit, u = 7, 15, synth.bits16(n, seed, 100 + rank).astype(np.uint32)
        specials = [0x0, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0xFFA1, 0x0001, 0x807F, 0x0080]
    sign = rng.integers(0, 2, n, dtype=np.uint32) << sbit
    mant = rng.integers(0, 1 << mbits, n, dtype=np.uint32)
    cls = rng.integers(0, 6, n)
    u = np.where(cls == 1, sign | mant, u)                                  # subnormal (or zero)
    u = np.where(cls == 2, sign | (np.uint32(1) << mbits) | mant, u)         # smallest binade
    u = np.where(cls == 3, sign | (np.uint32(254) << mbits) | mant, u)       # largest binade
    u = np.where(cls == 4, np.array(specials, np.uint32)[rng.integers(0, len(specials), n)], u)
    return u.astype(np.uint32).view(np.float32) if dt == F32 else u.astype(np.uint16)


def check_bits(got, ref, dt, what):
    """Bit-exact, except that NaN results are compared by position only."""
    if dt == BF16:
        return check_bf16(got, ref, what)
    gu, ru = got.view(np.uint32), ref.view(np.uint32)
    gnan = ((gu & 0x7F800000) == 0x7F800000) & ((gu & 0x7FFFFF) != 0)
    rnan = ((ru & 0x7F800000) == 0x7F800000) & ((ru & 0x7FFFFF) != 0)
    assert np.array_equal(gnan, rnan), f"{what}: NaN positions differ"
    bad = np.flatnonzero((gu != ru) & ~rnan)
    sub = int(np.sum(((ru & 0x7F800000) == 0) & ((ru & 0x7FFFFF) != 0)))
    say(what, f"{got.size - bad.size}/{got.size} bit-exact, {sub} subnormal results, {int(rnan.sum())} NaN")
    assert bad.size == 0, f"{what}: {bad.size} differ, first got {gu[bad[0]]:#010x} oracle {ru[bad[0]]:#010x}"


@pytest.mark.parametrize("dt", [F32, BF16])
@pytest.mark.parametrize("op", [SUM, AVG])
def test_folds_on_subnormals_infinities_and_nans(orc, dt, op):
    """Sums keep subnormal inputs and results (no flush to zero), overflow to
    infinity, and give NaN where the oracle does: the two-, four- and
    three-input folds, fp32 and bf16."""
    say("special values", dt, op)
    c = 1 << 17
    xs = [_special_classes(c, 11, r, dt) for r in range(4)]
    tdt = torch.float32 if dt == F32 else torch.bfloat16
    # A=2 allreduce helper: two slots
    out = torch.empty(c, dtype=tdt, device="cuda")
    rr.rr_helper_reduce(rr.Relay(2, 6, 8, 0, 8 * c), AR, dt, op, 0, [dev(xs[0], dt), dev(xs[1], dt)], out)
    check_bits(host(out), orc.ar2_helper(dt, op, xs[0], xs[1]), dt, "two-input fold")
    # A=4 allreduce helper: four position slices (oChunk = count/8 at 500 permille)
    relay4 = rr.Relay(4, 4, 0, 500, 8 * c)
    assert rr.rr_geometry(relay4, AR, dt)["chunk"] == c
    rr.rr_helper_reduce(relay4, AR, dt, op, 0, [dev(x, dt) for x in xs], out)
    check_bits(host(out), orc.ar4_helper(dt, op, xs), dt, "four-input fold")
    # A=4 reduce-scatter pass 1: three-input partial sums per owner (no scale)
    R = 8 * (c // 4)
    rs = rr.Relay(4, 4, 0, 500, R)
    cc = rr.rr_geometry(rs, RS, dt)["chunk"]
    scratch = np.concatenate([_special_classes(12 * cc, 12, 0, dt), np.zeros(2 * R - 12 * cc, xs[0].dtype)])
    ds = dev(scratch, dt)
    rr.rr_rs_multi_reduce(rs, dt, op, 1, 0, [ds], ds[12 * cc:16 * cc])
    check_bits(host(ds)[12 * cc:16 * cc], orc.rs4_pass1(dt, 4, cc, scratch), dt, "three-input fold")


def test_empty_and_zero_chunk_calls_are_no_ops(orc):
    say("empty")
    x = torch.full((64,), 3.0, dtype=torch.bfloat16, device="cuda")
    relay = rr.Relay(2, 6, 8, 0, 0)
    rr.rr_active_add_scale(relay, AR, BF16, SUM, 0, [x, x], x)
    rr.rr_helper_reduce(rr.Relay(2, 6, 8, 0, 1000), AR, BF16, SUM, 0, [x, x], x)
    torch.cuda.synchronize()
    assert torch.all(x == 3.0)


def test_partial_overlap_is_rejected_on_device_tensors():
    say("alias")
    x = torch.zeros(2 ** 16, dtype=torch.bfloat16, device="cuda")
    relay = rr.Relay(2, 6, 8, 0, 2 ** 14)
    c = rr.rr_geometry(relay, AR, BF16)["chunk"]
    with pytest.raises(rr.RRError, match="RR_EALIAS"):
        rr.rr_helper_reduce(relay, AR, BF16, SUM, 0, [x[:c], x[c:2 * c]], x[8:8 + c])
    with pytest.raises(rr.RRError, match="dtype"):   # bf16 tensors passed as fp32 buffers
        rr.rr_helper_reduce(relay, AR, F32, SUM, 0, [x[:c], x[c:2 * c]], x[:c])


# --------------------------------------------------------------------------
# fused multi-group calls: heterogeneous groups, zero-chunk groups skipped
# --------------------------------------------------------------------------

def test_many_calls_over_heterogeneous_groups(orc):
    """One GPU helping three A=2 groups of different sizes (one of them too
    small to relay) and running the active epilogue of an A=2 and an A=4
    group, each role as one batched call."""
    say("many heterogeneous")
    counts = [2 ** 22 + 8 * 128 * 3 + 11, 8 * 128 * 40, 700]
    xs = [[synth.as_bf16_bits(synth.normal(n, 60 + g, a)) for a in range(2)] for g, n in enumerate(counts)]
    dx = [[dev(x) for x in pair] for pair in xs]
    jobs, outs = [], []
    for g, n in enumerate(counts):
        relay = rr.Relay(2, 6, 8, 0, n)
        c = rr.rr_geometry(relay, AR, BF16)["chunk"]
        h = (2 * g + 1) % 6
        o = torch.zeros(max(c, 1), dtype=torch.bfloat16, device="cuda")
        jobs.append((relay, h, [dx[g][0][h * c:(h + 1) * c], dx[g][1][h * c:(h + 1) * c]], o))
        outs.append((o, c, h))
    rr.rr_helper_reduce_many(AR, BF16, AVG, jobs)
    for g, (o, c, h) in enumerate(outs):
        if c:
            ref = orc.ar2_helper(BF16, AVG, xs[g][0][h * c:(h + 1) * c].copy(), xs[g][1][h * c:(h + 1) * c].copy())
            check_bf16(host(o)[:c], ref, f"group {g} helper {h}")
        else:
            assert torch.all(o == 0)
    n4 = 2 ** 21 + 4 * 128 * 5 + 6
    x4 = [synth.as_bf16_bits(synth.uniform(n4, -2, 2, 61, a)) for a in range(4)]
    d4 = [dev(x) for x in x4]
    o2 = [torch.zeros(counts[0], dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    o4 = [torch.zeros(n4, dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    ajobs = [(rr.Relay(2, 6, 8, 0, counts[0]), a, dx[0], o2[a]) for a in range(2)] + \
            [(rr.Relay(4, 4, 0, 500, n4), a, d4, o4[a]) for a in range(4)]
    rr.rr_active_add_scale_many(AR, BF16, AVG, ajobs)
    for a in range(2):
        ref = orc.ar_active(BF16, AVG, 2, 6, 8, 0, counts[0], a, xs[0], np.zeros(counts[0], np.uint16))
        check_bf16(host(o2[a]), ref, f"A=2 active {a}")
    for a in range(4):
        ref = orc.ar_active(BF16, AVG, 4, 4, 0, 500, n4, a, x4, np.zeros(n4, np.uint16))
        check_bf16(host(o4[a]), ref, f"A=4 active {a}")


def test_phase_call_runs_a4_helper_and_active_slices(orc):
    """One rank's phase of the fused A=4 allreduce as one call: its helper
    slices of the other group and its own direct slices, at a count whose
    direct slices start off a 16-byte boundary (those take the realigning
    launch), plus an A=2 helper job of a third group; every output equal to
    the oracle's, and the call equal to the two per-role calls."""
    say("phase call A=4 allreduce")
    n = 2 ** 21 + 4 * 128 * 5 + 7
    xs = [synth.as_bf16_bits(synth.uniform(n, -2, 2, 62, a)) for a in range(4)]
    ys = [synth.as_bf16_bits(synth.uniform(n, -2, 2, 63, a)) for a in range(4)]
    n2 = 8 * 128 * 40 + 3
    zs = [synth.as_bf16_bits(synth.normal(n2, 64, a)) for a in range(2)]
    dx, dy, dz = [dev(x) for x in xs], [dev(y) for y in ys], [dev(z) for z in zs]
    r4, r2 = rr.Relay(4, 4, 0, 500, n), rr.Relay(2, 6, 8, 0, n2)
    c, c2 = rr.rr_geometry(r4, AR, BF16)["chunk"], rr.rr_geometry(r2, AR, BF16)["chunk"]
    assert c > 0 and c2 > 0

    def run(fused):
        red = [torch.zeros(c, dtype=torch.bfloat16, device="cuda") for _ in range(4)]
        red2 = torch.zeros(c2, dtype=torch.bfloat16, device="cuda")
        outs = [torch.zeros(n, dtype=torch.bfloat16, device="cuda") for _ in range(4)]
        hj = [(r4, h, [y[h * c:(h + 1) * c] for y in dy], red[h]) for h in range(4)] + \
             [(r2, 5, [z[5 * c2:6 * c2] for z in dz], red2)]
        aj = [(r4, a, dx, outs[a]) for a in range(4)]
        if fused:
            rr.rr_phase_reduce_many(AR, BF16, AVG, hj, aj)
        else:
            rr.rr_helper_reduce_many(AR, BF16, AVG, hj)
            rr.rr_active_add_scale_many(AR, BF16, AVG, aj)
        return [host(t) for t in red + [red2] + outs]

    got, apart = run(True), run(False)
    for h in range(4):
        check_bf16(got[h], orc.ar4_helper(BF16, AVG, [y[h * c:(h + 1) * c].copy() for y in ys]), f"helper {h}")
    check_bf16(got[4], orc.ar2_helper(BF16, AVG, zs[0][5 * c2:6 * c2].copy(), zs[1][5 * c2:6 * c2].copy()),
               "A=2 helper 5")
    for a in range(4):
        check_bf16(got[5 + a], orc.ar_active(BF16, AVG, 4, 4, 0, 500, n, a, xs, np.zeros(n, np.uint16)),
                   f"active {a}")
    for i, (g, p) in enumerate(zip(got, apart)):
        assert np.array_equal(g, p), f"output {i}: the phase call differs from the per-role calls"
    # an active writing what a helper reads is rejected before any launch
    out = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(rr.RRError, match="RR_EALIAS"):
        rr.rr_phase_reduce_many(AR, BF16, AVG, [(r4, 0, [out[4 * c:5 * c]] + [y[:c] for y in dy[1:]], dy[0][:1].new_zeros(c))],
                                [(r4, 0, dx, out)])


def test_workload_modes_agree(orc):
    """One call per job, one call over the whole group's jobs and one call
    over one GPU's share write the same bytes where they overlap, each checked
    against the oracle (one GPU's share of the A=4 reduce-scatter: helper 0's
    pass 1 and owner 0's pass 2)."""
    say("workload modes")
    M = 8 * 2 ** 20
    xs = [synth.as_bf16_bits(synth.normal(M // 2, 2, s)) for s in range(4)]
    ref = orc.rs4_group(BF16, SUM, 4, 500, M // 8, xs)
    for mode, ncalls, owners in (("job", 8, 4), ("group", 2, 4), ("share", 2, 1)):
        wl = W.RS4([dev(x) for x in xs], BF16, SUM, mode=mode)
        assert len(wl.calls()) == ncalls
        wl.run()
        for o in range(owners):
            check_bf16(host(wl.out[o]), ref[o], f"mode={mode} owner {o}")
    with pytest.raises(ValueError):
        W.RS4([dev(x) for x in xs], BF16, SUM, mode="batched")


# --------------------------------------------------------------------------
# maximum sizes and fp32 coverage
# --------------------------------------------------------------------------

def _pattern(n, mult, device="cuda", step=1 << 26):
    """bf16 small integers ((i*mult) % 61 - 30), built on the device in pieces."""
    out = torch.empty(n, dtype=torch.bfloat16, device=device)
    for lo in range(0, n, step):
        hi = min(n, lo + step)
        i = torch.arange(lo, hi, dtype=torch.int64, device=device)
        out[lo:hi] = ((i * mult) % 61 - 30).to(torch.bfloat16)
    return out


def _pattern_host(idx, mult):
    return synth.as_bf16_bits((((idx.astype(np.int64) * mult) % 61) - 30).astype(np.float32))


def test_reduction_beyond_2_31_elements(orc):
    """A reduce-scatter owner epilogue over recvCount > 2^31 elements (over
    4 GiB per input): 64-bit offsets and tile counts across one launch.
    Outputs are read back as windows by slicing (contiguous device-to-host
    copies); torch's advanced indexing into a tensor of more than 2^31
    elements faulted on this software stack, so it is not used here.  The
    output sits between two guard bands of eight 16 KiB tiles each inside one
    sentinel-filled allocation, and both bands are read back (by slicing)
    after the launch: nothing may be written before or past the output."""
    R = 2 ** 31 + 8 * 128 * 3 + 5
    G = 65536
    say("beyond 2^31", R)
    a, b = _pattern(R, 3), _pattern(R, 7)
    whole = torch.empty(R + 2 * G, dtype=torch.int16, device="cuda")
    whole.fill_(SENTINEL)
    out = whole[G:G + R].view(torch.bfloat16)
    rr.rr_active_add_scale(rr.Relay(2, 6, 8, 0, R), RS, BF16, AVG, 0, [a, b], out)
    torch.cuda.synchronize()
    assert np.all(synth.to_host(whole[:G]) == SENTINEL), "write before the output"
    assert np.all(synth.to_host(whole[G + R:]) == SENTINEL), "write past the output"
    rng = np.random.default_rng(5)
    starts = [0, 2 ** 31 - 4096, R - 4096] + sorted(int(v) for v in rng.integers(0, R - 2048, 32))
    for lo in starts:
        hi = min(R, lo + (8192 if lo == 2 ** 31 - 4096 else 4096 if lo in (0, R - 4096) else 2048))
        got = synth.to_host(out[lo:hi])
        idx = np.arange(lo, hi, dtype=np.int64)
        ref = orc.rs2_active(BF16, AVG, _pattern_host(idx, 3), _pattern_host(idx, 7))
        check_bf16(got, ref, f"window [{lo}, {hi}) past 2^31")
    del a, b, out, whole
    torch.cuda.empty_cache()


def _bits_pattern(n, s, step=1 << 26):
    """Raw 16-bit words that identify (source s, position i), built on the
    device in pieces: ((i * 40503 + (i >> 16) * 97 + s * 7919) mod 2^16)."""
    out = torch.empty(n, dtype=torch.int16, device="cuda")
    for lo in range(0, n, step):
        hi = min(n, lo + step)
        i = torch.arange(lo, hi, dtype=torch.int64, device="cuda")
        out[lo:hi] = ((i * 40503 + (i >> 16) * 97 + s * 7919) % 65536 - 32768).to(torch.int16)
    return out


def _bits_pattern_host(idx, s):
    return (((idx * 40503 + (idx >> 16) * 97 + s * 7919) % 65536 + 32768) % 65536).astype(np.uint16)


def test_all_to_all_beyond_4_GiB_offsets(orc):
    """Pack and unpack of helper slice 3 with segmentCount = 2^30 + 5 bf16
    elements: 8 GiB per source and output buffer, the chunks of destinations 2
    and 3 wholly past byte offset 4 GiB of their sources, 9 of the 12 moves
    realigned.  Sampled windows of every packed chunk
    and of every scattered slice equal the all-to-all transpose (unpack of
    pack gives out_d[s*seg + p] = src_s[d*seg + p] on slice positions), and
    the words just outside each slice keep their sentinel.  About 70 GB of
    device memory."""
    A, H, nc, h = 4, 4, 5, 3
    seg = 2 ** 30 + 5
    c = orc.geometry(A, H, nc, 0, seg, A2A, BF16)["chunk"]
    say("all-to-all beyond 4 GiB offsets", seg, c)
    relay = rr.Relay(A, H, nc, 0, seg)
    src = [_bits_pattern(A * seg, s) for s in range(A)]
    packed = [torch.empty((A - 1) * c, dtype=torch.int16, device="cuda") for _ in range(A)]
    rr.rr_a2a_pack(relay, BF16, h, src, packed)
    out = [torch.full((A * seg,), 0x2222, dtype=torch.int16, device="cuda") for _ in range(A)]
    rr.rr_a2a_unpack(relay, BF16, h, packed, out)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    for d in range(A):
        for j, s in enumerate(x for x in range(A) if x != d):
            at = d * seg + h * c            # the chunk's first element in source s
            dst = s * seg + h * c           # its first element in output d
            starts = [0, c - 2048] + [int(v) for v in rng.integers(0, c - 2048, 6)]
            for lo in starts:
                hi = lo + 2048
                ref = _bits_pattern_host(np.arange(at + lo, at + hi, dtype=np.int64), s)
                got = synth.to_host(packed[d][j * c + lo:j * c + hi])
                assert np.array_equal(got, ref), f"packed d={d} j={j} [{lo}, {hi})"
                got = synth.to_host(out[d][dst + lo:dst + hi])
                assert np.array_equal(got, ref), f"unpacked d={d} s={s} [{lo}, {hi})"
            edge = np.concatenate([synth.to_host(out[d][dst - 8:dst]), synth.to_host(out[d][dst + c:dst + c + 8])])
            assert np.all(edge == 0x2222), f"unpack wrote outside slice d={d} s={s}"
    del src, packed, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("R", [8 * 128 * 6 + 40, 2 ** 20 + 8])
def test_fp32_a4_reduce_scatter_and_allreduce(orc, R):
    say("fp32 A=4", R)
    xs = [synth.normal(4 * R, 80, s) for s in range(4)]
    wl = W.RS4([dev(x, F32) for x in xs], F32, AVG)
    wl.run()
    ref = orc.rs4_group(F32, AVG, 4, 500, R, xs)
    for o in range(4):
        check_f32(host(wl.out[o]), ref[o], [x[o * R:(o + 1) * R] for x in xs], f"fp32 RS owner {o}")
    count = 4 * R
    ar = W.AR4([dev(x, F32) for x in xs], F32, AVG)
    ar.run()
    ar.deliver()
    ref = orc.ar4_group(F32, AVG, 4, 500, count, xs)
    for a in range(4):
        check_f32(host(ar.out[a]), ref[a], xs, f"fp32 AR active {a}")


def test_fp32_all_to_all_bits(orc):
    say("fp32 a2a")
    A, seg = 4, 5 * 128 * 7 + 3
    src = [synth.rng(81, s).integers(0, 2 ** 32, A * seg, dtype=np.uint32) for s in range(A)]
    wl = W.A2A([torch.from_numpy(s.view(np.int32)).cuda() for s in src], F32)
    wl.run()
    torch.cuda.synchronize()
    c = wl.g["chunk"]
    expect = [np.zeros(A * seg, np.uint32) for _ in range(A)]
    for h in range(4):
        orc.a2a_unpack(4, A, seg, c, h, orc.a2a_pack(4, A, seg, c, h, src), expect)
    for d in range(A):
        assert np.array_equal(wl.out[d].cpu().numpy().view(np.uint32), expect[d])


def _ragged_a2a_case(orc, es, seg, seed):
    """Pack and unpack of every helper slice for a segmentCount off the 16-byte
    grid, compared bit for bit with the oracle; returns the chunk size."""
    A = 4
    npdt, sdt = (np.uint16, np.int16) if es == 2 else (np.uint32, np.int32)
    src = [synth.rng(seed, s).integers(0, 1 << (8 * es), A * seg, dtype=npdt) for s in range(A)]
    wl = W.A2A([torch.from_numpy(s.view(sdt)).cuda() for s in src], BF16 if es == 2 else F32)
    c = wl.g["chunk"]
    wl.run()
    torch.cuda.synchronize()
    expect = [np.zeros(A * seg, npdt) for _ in range(A)]
    for h in range(4):
        ref = orc.a2a_pack(es, A, seg, c, h, src)
        for d in range(A):
            got = wl.packed[h][d].cpu().numpy()[:(A - 1) * c].view(np.uint8)
            assert np.array_equal(got, ref[d]), ("pack", es, seg, h, d)
        orc.a2a_unpack(es, A, seg, c, h, ref, expect)
    for d in range(A):
        assert np.array_equal(wl.out[d].cpu().numpy().view(npdt), expect[d]), ("unpack", es, seg, d)
    return c


@pytest.mark.parametrize("es,seg", [(2, 5 * 128 * 400 + r) for r in (1, 3, 5, 7)]
                         + [(4, 5 * 128 * 300 + r) for r in (1, 2, 3)])
def test_ragged_all_to_all_spans_full_realign_tiles(orc, es, seg):
    """Every shift residue of the source against the packed buffer, with chunks
    long enough for several full realigning tiles (each lane's neighbour
    exchange and the wave-end lanes' own loads) and a partial tail tile."""
    say("ragged a2a", es, seg)
    c = _ragged_a2a_case(orc, es, seg, 120 + seg % 8)
    assert c * es // 16 > 4 * 1024   # more than four realigning tiles of 1024 vectors or fewer


def test_ragged_all_to_all_at_64MiB(orc):
    """The 64 MiB per-rank message with segmentCount = 5 (mod 8): 9 of every
    helper's 12 chunk moves are realigned."""
    seg = (64 << 20) // 2 // 4 - 3
    say("ragged a2a 64 MiB", seg)
    _ragged_a2a_case(orc, 2, seg, 131)


@pytest.mark.parametrize("mode", ["group", "share"])
def test_step_captured_in_a_hip_graph_replays_like_eager(mode):
    """The library enqueues kernels only (no allocation, no memset), so a whole
    step can be captured in a HIP graph, in every launch form (one GPU's share
    runs its single-segment launches with arguments preloaded into registers,
    the whole group mostly uniform grids).  Each replay -- with eager work and
    synchronisations between replays -- must write what the eager step wrote."""
    say("graph replay", mode)
    M = 8 * 2 ** 20
    n = M // 2
    xs2 = [dev(synth.as_bf16_bits(synth.normal(n, 90, a))) for a in range(2)]
    xs4 = [dev(synth.as_bf16_bits(synth.normal(n, 91, a))) for a in range(4)]
    xa4 = [dev(synth.as_bf16_bits(synth.normal(n, 93, a))) for a in range(4)]
    src = [dev(synth.bits16(n, 92, a), None) for a in range(4)]
    rows = [W.AR2(xs2, BF16, AVG, mode=mode), W.AR4(xa4, BF16, AVG, mode=mode),
            W.RS4(xs4, BF16, SUM, mode=mode), W.A2A(src, BF16, mode=mode)]
    outs = lambda: [o for w in rows for o in w.out]
    main = torch.cuda.current_stream()
    for o in outs():
        o.zero_()                          # parts no kernel writes stay zero throughout
    for w in rows:
        w.run(main)
    torch.cuda.synchronize()
    eager = [synth.to_host(o).copy() for o in outs()]
    cs = torch.cuda.Stream()
    cs.wait_stream(main)
    with torch.cuda.stream(cs):
        for w in rows:
            w.run(cs)                      # prepare and warm on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        for w in rows:
            w.run(cs)
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs():
            o.zero_()                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, o in enumerate(outs()):
            assert np.array_equal(synth.to_host(o), eager[i]), f"replay {rep} output {i}"


GUARD = 4096
SENTINEL = 0x7FA5


def _guarded(n, lead):
    """A bf16 buffer of n elements at offset GUARD+lead inside a sentinel-filled
    allocation; returns (whole buffer, view)."""
    big = torch.full((n + 2 * GUARD + 8,), 0, dtype=torch.int16, device="cuda")
    big.fill_(SENTINEL)
    v = big[GUARD + lead:GUARD + lead + n]
    return big, v.view(torch.bfloat16)


def _guards_intact(big, n, lead):
    h = synth.to_host(big)
    assert np.all(h[:GUARD + lead] == SENTINEL), "write before the output"
    assert np.all(h[GUARD + lead + n:] == SENTINEL), "write past the output"


@pytest.mark.parametrize("lead", [0, 1, 3, 7])
def test_every_entry_point_writes_only_its_output(orc, lead):
    say("canaries", lead)
    # helper reduce (A=4) and active epilogue (A=2)
    count = 2 ** 20 + 4 * 128 * 7 + 6
    xs = [synth.as_bf16_bits(synth.normal(count, 95, a)) for a in range(4)]
    dx = [dev(x) for x in xs]
    r4 = rr.Relay(4, 4, 0, 500, count)
    c = rr.rr_geometry(r4, AR, BF16)["chunk"]
    big, out = _guarded(c, lead)
    rr.rr_helper_reduce(r4, AR, BF16, AVG, 2, [x[2 * c:3 * c] for x in dx], out)
    _guards_intact(big, c, lead)
    check_bf16(synth.to_host(out), orc.ar4_helper(BF16, AVG, [x[2 * c:3 * c].copy() for x in xs]), "guarded helper")
    r2 = rr.Relay(2, 6, 8, 0, count)
    g2 = rr.rr_geometry(r2, AR, BF16)
    big, out = _guarded(count, lead)
    rr.rr_active_add_scale(r2, AR, BF16, SUM, 1, dx[:2], out)
    _guards_intact(big, count, lead)
    ref = orc.ar_active(BF16, SUM, 2, 6, 8, 0, count, 1, xs[:2], np.full(count, SENTINEL, np.uint16))
    got = synth.to_host(out)
    assert np.all(got[:g2["direct_off"]] == SENTINEL)
    check_bf16(got[g2["direct_off"]:], ref[g2["direct_off"]:], "guarded active")
    # reduce-scatter pass 2 (A=4)
    R = 8 * 128 * 9 + 40
    blk = [synth.as_bf16_bits(synth.normal(R, 96, s)) for s in range(4)]
    rs = rr.Relay(4, 4, 0, 500, R)
    cr = rr.rr_geometry(rs, RS, BF16)["chunk"]
    reds = [synth.as_bf16_bits(synth.normal(cr, 97, h)) for h in range(4)]
    big, out = _guarded(R, lead)
    rr.rr_rs_multi_reduce(rs, BF16, AVG, 2, 3, [dev(b) for b in blk] + [dev(r) for r in reds], out)
    _guards_intact(big, R, lead)
    check_bf16(synth.to_host(out), orc.rs4_pass2(BF16, AVG, 4, 4, 500, R, 3, blk, reds), "guarded pass 2")
    # all-to-all pack and unpack
    A, seg = 4, 5 * 128 * 5 + 3
    ra = rr.Relay(A, 4, 5, 0, seg)
    ca = rr.rr_geometry(ra, A2A, BF16)["chunk"]
    src = [synth.bits16(A * seg, 98, s) for s in range(A)]
    dsts = [_guarded((A - 1) * ca, lead) for _ in range(A)]
    rr.rr_a2a_pack(ra, BF16, 1, [dev(s, None) for s in src], [d[1] for d in dsts])
    ref = orc.a2a_pack(2, A, seg, ca, 1, src)
    for (big, v), r in zip(dsts, ref):
        _guards_intact(big, (A - 1) * ca, lead)
        assert np.array_equal(synth.to_host(v).view(np.uint8), r)
    outs = [_guarded(A * seg, lead) for _ in range(A)]
    for _, v in outs:
        v.view(torch.int16).fill_(0)
    rr.rr_a2a_unpack(ra, BF16, 1, [d[1] for d in dsts], [o[1] for o in outs])
    expect = [np.zeros(A * seg, np.uint16) for _ in range(A)]
    orc.a2a_unpack(2, A, seg, ca, 1, ref, expect)
    for (big, v), e in zip(outs, expect):
        _guards_intact(big, A * seg, lead)
        assert np.array_equal(synth.to_host(v), e)


@pytest.mark.parametrize("njobs", [1, 8, 9, 40, 41])
@pytest.mark.parametrize("equal", [True, False])
def test_batches_at_the_segment_table_sizes(orc, njobs, equal):
    """A launch passes an 8- or 40-entry reduction table (a 16- or 64-entry
    copy table) by the size of its batch, and a call of more segments
    continues in a further launch: A=2 helper jobs of equal counts (uniform
    grid) or of different counts (tile table) at and across those sizes, bit
    for bit against the oracle."""
    say("segment table sizes", njobs, equal)
    rng = np.random.default_rng(njobs * 2 + int(equal))
    jobs, refs = [], []
    for j in range(njobs):
        count = 8 * 128 * (6 if equal else int(rng.integers(3, 12)))
        c = orc.geometry(2, 6, 8, 0, count, AR, BF16)["chunk"]
        x = [synth.as_bf16_bits(synth.normal(count, 300 + j, a)) for a in range(2)]
        h = j % 6
        out = torch.zeros(c, dtype=torch.bfloat16, device="cuda")
        jobs.append((rr.Relay(2, 6, 8, 0, count), h, [dev(v[h * c:(h + 1) * c].copy()) for v in x], out))
        refs.append(orc.ar2_helper(BF16, AVG, x[0][h * c:(h + 1) * c].copy(), x[1][h * c:(h + 1) * c].copy()))
    rr.rr_helper_reduce_many(AR, BF16, AVG, jobs)
    for j, ref in enumerate(refs):
        assert np.array_equal(host(jobs[j][3]), ref), f"job {j}"


@pytest.mark.parametrize("nslices,ragged", [(1, False), (2, False), (1, True), (2, True)])
def test_copy_batches_at_the_segment_table_sizes(orc, nslices, ragged):
    """All-to-all packs of one or two helper slices (12 or 24 chunk moves, in
    the 16- and the 64-entry copy table), aligned and with segmentCount = 5
    mod 8 (aligned and realigned moves in one mixed-mode launch)."""
    say("copy table sizes", nslices, ragged)
    A, H, nc = 4, 4, 5
    seg = 5 * 128 * 6 + (5 if ragged else 0)
    c = orc.geometry(A, H, nc, 0, seg, A2A, BF16)["chunk"]
    src = [synth.bits16(A * seg, 310, s) for s in range(A)]
    sdev = [dev(s, None) for s in src]
    relay = rr.Relay(A, H, nc, 0, seg)
    packed = [[torch.zeros((A - 1) * c, dtype=torch.int16, device="cuda") for _ in range(A)] for _ in range(nslices)]
    rr.rr_a2a_pack_many(BF16, [(relay, h, sdev, packed[h]) for h in range(nslices)])
    for h in range(nslices):
        ref = orc.a2a_pack(2, A, seg, c, h, src)
        for d in range(A):
            assert np.array_equal(host(packed[h][d]).view(np.uint8), ref[d]), f"slice {h} dest {d}"


def test_copy_batches_of_unequal_moves_fill_the_table(orc):
    """Six all-to-all pack jobs over groups of different segmentCounts (some 5
    mod 8): 72 chunk moves of unequal tile counts, so the first launch runs a
    full 64-entry tile table in the mixed-mode copy kernel and the rest
    continues in a second launch; every job bit for bit against the oracle."""
    say("copy table of unequal moves")
    A, H, nc = 4, 4, 5
    jobs, refs = [], []
    for j in range(6):
        seg = 5 * 128 * (40 + 24 * j) + (5 if j % 2 else 0)   # chunks of 2-9 copy tiles
        c = orc.geometry(A, H, nc, 0, seg, A2A, BF16)["chunk"]
        src = [synth.bits16(A * seg, 320 + j, s) for s in range(A)]
        dst = [torch.zeros((A - 1) * c, dtype=torch.int16, device="cuda") for _ in range(A)]
        h = j % H
        jobs.append((rr.Relay(A, H, nc, 0, seg), h, [dev(x, None) for x in src], dst))
        refs.append(orc.a2a_pack(2, A, seg, c, h, src))
    fn = rr.rr_a2a_pack_many(BF16, jobs, prepare=True)
    assert fn.launches == 2
    fn()
    for j, (job, ref) in enumerate(zip(jobs, refs)):
        for d in range(A):
            assert np.array_equal(host(job[3][d]).view(np.uint8), ref[d]), f"job {j} dest {d}"


# --------------------------------------------------------------------------
# plans: validated once, launched many times
# --------------------------------------------------------------------------

def test_plan_records_calls_and_launches_them_later(orc):
    """Three calls recorded into one rr.Plan (an A=2 reduce-scatter owner, a
    batched A=2 allreduce helper call over three groups, an all-to-all pack)
    enqueue nothing while they are recorded; the launched plan writes the
    oracle's bytes, and launched again after the inputs change in place it
    writes the new result."""
    R = 2 ** 20 + 8 * 128 * 3 + 5
    count = 2 ** 20
    c = count // 8
    seg = 5 * 128 * 4096 + 3
    say("plan", R, count, seg)
    xs = [dev(synth.as_bf16_bits(synth.normal(R, 80, a))) for a in range(2)]
    ss = [dev(synth.as_bf16_bits(synth.normal(count, 81, a))) for a in range(2)]
    src_h = [synth.bits16(4 * seg, 82, s) for s in range(4)]
    src = [synth.to_device(h, None) for h in src_h]
    ac = orc.geometry(4, 4, 5, 0, seg, A2A, BF16)["chunk"]
    out = torch.zeros(R, dtype=torch.bfloat16, device="cuda")
    hout = [torch.zeros(c, dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    dst = [torch.zeros(3 * ac, dtype=torch.int16, device="cuda") for _ in range(4)]
    relay2, relay4 = rr.Relay(2, 6, 8, 0, count), rr.Relay(4, 4, 5, 0, seg)
    plan = rr.Plan(16)
    with plan:
        rr.rr_active_add_scale(rr.Relay(2, 6, 8, 0, R), RS, BF16, AVG, 0, xs, out)
        rr.rr_helper_reduce_many(AR, BF16, SUM, [(relay2, h, [s[h * c:(h + 1) * c] for s in ss], hout[h])
                                                 for h in range(3)])
        rr.rr_a2a_pack(relay4, BF16, 1, src, dst)
    assert plan.launches == 3
    torch.cuda.synchronize()
    assert not out.any() and not any(h.any() for h in hout) and not any(d.any() for d in dst)

    def check(tag):
        xh, sh = [host(x) for x in xs], [host(s) for s in ss]
        check_bf16(host(out), orc.rs2_active(BF16, AVG, xh[0], xh[1]), f"plan {tag}: reduce-scatter owner")
        for h in range(3):
            ref = orc.ar2_helper(BF16, SUM, sh[0][h * c:(h + 1) * c].copy(), sh[1][h * c:(h + 1) * c].copy())
            check_bf16(host(hout[h]), ref, f"plan {tag}: helper {h}")
        ref = orc.a2a_pack(2, 4, seg, ac, 1, [host(s) for s in src])
        for d in range(4):
            assert np.array_equal(host(dst[d]).view(np.uint8), ref[d]), f"plan {tag}: pack destination {d}"

    plan()
    check("first launch")
    for t in xs + ss + src:
        t.copy_(torch.roll(t, 11))
    plan.launch(torch.cuda.current_stream())
    check("after new inputs")


def test_plan_of_a_call_that_spans_several_launches(orc):
    """A batched A=2 allreduce helper call of 50 jobs, every tenth job's slots
    and output at odd element offsets (the realigning kernels), so the 45
    aligned jobs exceed one launch's 40 reduction segments: prepared with
    prepare=True, the plan holds every launch of the call (two aligned, one
    realigning), and launched it writes the oracle's bytes for every job."""
    count = 8 * 128 * 24
    c = count // 8
    relay = rr.Relay(2, 6, 8, 0, count)
    say("plan, 50 jobs", count)
    jobs, refs = [], []
    for j in range(50):
        lead = 1 + (j % 7) if j % 10 == 0 else 0
        xs = [synth.as_bf16_bits(synth.normal(c + 8, 90 + j, a)) for a in range(2)]
        dx = [dev(x) for x in xs]
        out = torch.zeros(c + 8, dtype=torch.bfloat16, device="cuda")
        jobs.append((relay, j % 6, [x[lead:lead + c] for x in dx], out[lead:lead + c]))
        refs.append((out, lead, orc.ar2_helper(BF16, AVG, xs[0][lead:lead + c].copy(), xs[1][lead:lead + c].copy())))
    fn = rr.rr_helper_reduce_many(AR, BF16, AVG, jobs, prepare=True)
    assert fn.launches == 3      # two aligned launches (45 > 40 segments) and a realigning one
    torch.cuda.synchronize()
    assert not any(o.any() for o, _, _ in refs)
    fn()
    for j, (out, lead, ref) in enumerate(refs):
        got = host(out)
        check_bf16(got[lead:lead + c], ref, f"plan job {j}")
        assert not got[:lead].any() and not got[lead + c:].any(), f"plan job {j} wrote outside its output"
