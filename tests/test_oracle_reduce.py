"""Pins of the oracle's reductions, each against something other than the
oracle's own formulas:

* small integers: every sum is exact in bf16 and fp32, so the result must be
  the integer sum (times an exact power-of-two scale) whatever the order --
  this pins layout, indexing, operand choice and the scale placement;
* exact rational brute force (oracle/brute.py) on tiny random shapes: the
  same fp32 fold, rounded from first principles instead of by hardware;
* the plain collective definitions: the A=2 and A=4 allreduce and the A=2
  reduce-scatter compose to the plain result (exact sum, one rounding) within one bf16 ulp
  ("reduce-at-helper" equivalence, PR summary section 2), and the A=4
  reduce-scatter stays within the rounding-error bound of its two roundings;
* a planted mistake: summing the A=2 reduce-scatter slots at the helper (which
  the pull request deliberately does not do) fails the plain definition.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import brute
from pack_rr_helper_amd import synth

F32, BF16 = 0, 1
SUM, AVG = 0, 1


def ords(bits):
    """bf16 bit patterns -> integers that are monotone in the value."""
    b = bits.astype(np.int32)
    return np.where(b & 0x8000, 0x8000 - (b & 0x7FFF) - 1, b + 0x8000)


def bf16_vals(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def int_inputs(n, ranks, seed, lim=16, dt=BF16):
    xs = [synth.small_ints(n, lim, seed, r) for r in range(ranks)]
    return xs if dt == F32 else [synth.as_bf16_bits(x) for x in xs]


def as_float(a, dt):
    return a.astype(np.float64) if dt == F32 else bf16_vals(a)


# --------------------------------------------------------------------------
# small-integer exactness
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dt", [F32, BF16])
@pytest.mark.parametrize("op", [SUM, AVG])
def test_ar2_helper_small_ints(orc, dt, op):
    s0, s1 = int_inputs(3000, 2, 11, dt=dt)
    out = orc.ar2_helper(dt, op, s0, s1)
    exp = (as_float(s0, dt) + as_float(s1, dt)) * (0.5 if op == AVG else 1.0)
    assert np.array_equal(as_float(out, dt), exp)


@pytest.mark.parametrize("op", [SUM, AVG])
def test_ar4_helper_small_ints(orc, op):
    xs = int_inputs(2500, 4, 12)
    out = orc.ar4_helper(BF16, op, xs)
    exp = sum(bf16_vals(x) for x in xs) * (0.25 if op == AVG else 1.0)
    assert np.array_equal(bf16_vals(out), exp)


@pytest.mark.parametrize("A,H,nc,pm,count", [
    (2, 6, 8, 0, 8 * 128 * 3 + 77),   # relay + dirA + ragged dirB
    (2, 6, 8, 0, 500),                # zero chunk: pure direct
    (4, 4, 0, 500, 2 ** 20 + 12),     # A=4 over the 2 MiB floor, ragged slices
    (4, 4, 0, 500, 1000),             # A=4 under the floor
])
def test_ar_active_writes_exactly_its_region(orc, A, H, nc, pm, count):
    xs = int_inputs(count, A, 13)
    g = orc.geometry(A, H, nc, pm, count, 0, BF16)
    for a in range(A):
        canary = np.full(count, 0x7FA5, np.uint16)
        out = orc.ar_active(BF16, AVG, A, H, nc, pm, count, a, xs, canary.copy())
        if A == 2:
            lo, hi = g["direct_off"], count
        else:
            lo = g["direct_off"] + a * g["dslice"]
            hi = lo + g["dslice"] if a < A - 1 else count
        exp = sum(bf16_vals(x[lo:hi]) for x in xs) / A
        assert np.array_equal(bf16_vals(out[lo:hi]), exp)
        assert np.all(out[:lo] == 0x7FA5) and np.all(out[hi:] == 0x7FA5)


def test_rs4_passes_small_ints(orc):
    A, H, R = 4, 4, 8 * 128 * 2 + 40
    g = orc.geometry(A, H, 0, 500, R, 1, BF16)
    c = g["chunk"]
    assert c == 256
    scratch = np.concatenate(int_inputs(A * (A - 1) * c, 1, 14))
    red = orc.rs4_pass1(BF16, A, c, scratch)
    for o in range(A):
        parts = [bf16_vals(scratch[(o * 3 + j) * c:(o * 3 + j + 1) * c]) for j in range(3)]
        assert np.array_equal(bf16_vals(red[o * c:(o + 1) * c]), sum(parts))
    blk = int_inputs(R, A, 15)
    reds = int_inputs(c, H, 16)
    for o in range(A):
        out = orc.rs4_pass2(BF16, AVG, A, H, 500, R, o, blk, reds)
        for h in range(H):
            sl = slice(h * c, (h + 1) * c)
            assert np.array_equal(bf16_vals(out[sl]), (bf16_vals(blk[o][sl]) + bf16_vals(reds[h])) / 4)
        d = slice(H * c, R)
        assert np.array_equal(bf16_vals(out[d]), sum(bf16_vals(b[d]) for b in blk) / 4)


# --------------------------------------------------------------------------
# exact rational brute force on tiny shapes
# --------------------------------------------------------------------------

def _normal_bits(n, ranks, seed):
    return [synth.as_bf16_bits(synth.normal(n, seed, r) * np.float32(2.0 ** (r - 1))) for r in range(ranks)]


@pytest.mark.parametrize("op", [SUM, AVG])
def test_helpers_against_brute_force(orc, op):
    x2 = _normal_bits(300, 2, 21)
    got = orc.ar2_helper(BF16, op, x2[0], x2[1])
    assert list(got) == brute.reduce_bits(x2, 16, Fraction(1, 2) if op == AVG else 1)
    x4 = _normal_bits(300, 4, 22)
    got = orc.ar4_helper(BF16, op, x4)
    assert list(got) == brute.reduce_bits(x4, 16, Fraction(1, 4) if op == AVG else 1)


def test_fp32_helper_against_brute_force(orc):
    rng = np.random.default_rng(23)
    s = [(rng.standard_normal(300) * 10.0 ** rng.integers(-3, 4, 300)).astype(np.float32) for _ in range(2)]
    got = orc.ar2_helper(F32, AVG, s[0], s[1]).view(np.uint32)
    exp = brute.reduce_bits([a.view(np.uint32) for a in s], 32, Fraction(1, 2))
    assert list(got) == exp


def test_rs_passes_against_brute_force(orc):
    A, H, R = 4, 4, 8 * 128 + 8
    c = 128
    scratch = np.concatenate(_normal_bits(12 * c, 1, 24))
    red = orc.rs4_pass1(BF16, A, c, scratch)
    for o in range(A):
        ins = [scratch[(o * 3 + j) * c:(o * 3 + j + 1) * c] for j in range(3)]
        assert list(red[o * c:(o + 1) * c]) == brute.reduce_bits(ins, 16, 1)
    blk = _normal_bits(R, A, 25)
    reds = _normal_bits(c, H, 26)
    out = orc.rs4_pass2(BF16, SUM, A, H, 500, R, 2, blk, reds)
    assert list(out[:c]) == brute.reduce_bits([blk[2][:c], reds[0]], 16, 1)
    assert list(out[3 * c:4 * c]) == brute.reduce_bits([blk[2][3 * c:4 * c], reds[3]], 16, 1)
    assert list(out[4 * c:]) == brute.reduce_bits([b[4 * c:] for b in blk], 16, 1)
    b0, b1 = _normal_bits(200, 2, 27)
    assert list(orc.rs2_active(BF16, AVG, b0, b1)) == brute.reduce_bits([b0, b1], 16, Fraction(1, 2))


# --------------------------------------------------------------------------
# plain collective definitions
# --------------------------------------------------------------------------

def test_ar2_group_is_the_plain_allreduce(orc):
    """Reduce-at-helper: the helper's sum of the two slots is already the
    allreduced chunk, so the composed group equals the plain 2-rank AVG."""
    count = 8 * 128 * 5 + 333
    x0, x1 = _normal_bits(count, 2, 31)
    o0, o1 = orc.ar2_group(BF16, AVG, 6, 8, count, x0, x1)
    plain = orc.plain_sum(BF16, AVG, [x0, x1], 0, count)
    assert np.array_equal(o0, o1)
    assert np.max(np.abs(ords(o0) - ords(plain))) <= 1
    # integer inputs: every order is exact, so the two agree bit for bit
    i0, i1 = int_inputs(count, 2, 32)
    o0, _ = orc.ar2_group(BF16, AVG, 6, 8, count, i0, i1)
    assert np.array_equal(o0, orc.plain_sum(BF16, AVG, [i0, i1], 0, count))


@pytest.mark.parametrize("count", [2 ** 20 + 4 * 128 + 7, 3000])
def test_ar4_group_is_the_plain_allreduce(orc, count):
    xs = _normal_bits(count, 4, 33)
    outs = orc.ar4_group(BF16, AVG, 4, 500, count, xs)
    plain = orc.plain_sum(BF16, AVG, xs, 0, count)
    for o in outs:
        assert np.array_equal(o, outs[0])
        assert np.max(np.abs(ords(o) - ords(plain))) <= 1
    xi = int_inputs(count, 4, 34)
    assert np.array_equal(orc.ar4_group(BF16, AVG, 4, 500, count, xi)[3],
                          orc.plain_sum(BF16, AVG, xi, 0, count))


def _rs2_plain(orc, x0, x1, R):
    return [orc.plain_sum(BF16, AVG, [x0, x1], o * R, R) for o in range(2)]


@pytest.mark.parametrize("R", [8 * 128 * 4 + 19, 600])
def test_rs2_group_is_the_plain_reduce_scatter(orc, R):
    x0, x1 = _normal_bits(2 * R, 2, 35)
    o0, o1 = orc.rs2_group(BF16, AVG, 6, 8, R, x0, x1)
    p0, p1 = _rs2_plain(orc, x0, x1, R)
    assert np.max(np.abs(ords(o0) - ords(p0))) <= 1
    assert np.max(np.abs(ords(o1) - ords(p1))) <= 1
    i0, i1 = int_inputs(2 * R, 2, 36)
    o0, o1 = orc.rs2_group(BF16, AVG, 6, 8, R, i0, i1)
    p0, p1 = _rs2_plain(orc, i0, i1, R)
    assert np.array_equal(o0, p0) and np.array_equal(o1, p1)


def test_summing_reduce_scatter_slots_at_the_helper_is_wrong(orc):
    """Planted mistake: a helper that sums slot 0 (a0's block 1) and slot 1
    (a1's block 0) and returns the sum to both owners.  The plain definition
    catches it, which is why the pull request keeps those helpers passthrough."""
    R = 8 * 128 * 2
    c = 128
    x0, x1 = int_inputs(2 * R, 2, 37)
    out0 = orc.rs2_active(BF16, AVG, x0[:R], x1[:R])        # correct reference pieces
    wrong0 = out0.copy()
    for k in range(6):
        sl = slice(k * c, (k + 1) * c)
        mixed = orc.ar2_helper(BF16, SUM, x0[R:][sl].copy(), x1[:R][sl].copy())
        wrong0[sl] = orc.rs2_active(BF16, AVG, x0[:R][sl].copy(), mixed)
    p0, _ = _rs2_plain(orc, x0, x1, R)
    assert np.array_equal(out0, p0)
    assert not np.array_equal(wrong0, p0)


def test_rs4_group_within_two_rounding_bound(orc):
    """The A=4 reduce-scatter helper rounds its partial sum to bf16, so an
    offload element is not the plain sum.  Following its steps, with
    u = 2^-8 (bf16 has 8 significant bits), e = 2^-24 (fp32) and
    g_k = k*e/(1-k*e):
      s = fp32 fold of the 3 non-owner values   |s - p|  <= g_2 * sum|x_{s!=o}|
      r = RNE_bf16(s)                           |r - s|  <= u * |s|
      t = fp32(x_o + r)                         |t - (x_o + r)| <= e * |x_o + r|
      out = RNE_bf16(t)                         |out - t| <= u * |t| <= u/(1-u) * |out|
    and a direct element is one fp32 fold of 4 values and one rounding."""
    A, H = 4, 4
    R = 8 * 128 * 3 + 24
    xs = _normal_bits(A * R, A, 38)
    outs = orc.rs4_group(BF16, SUM, H, 500, R, xs)
    u, e = 2.0 ** -8, 2.0 ** -24
    g2, g3 = 2 * e / (1 - 2 * e), 3 * e / (1 - 3 * e)
    c = orc.geometry(A, H, 0, 500, R, 1, BF16)["chunk"]
    for o in range(A):
        vals = [bf16_vals(x[o * R:(o + 1) * R]) for x in xs]
        exact = sum(vals)
        got = bf16_vals(outs[o])
        abs_other = sum(np.abs(v) for i, v in enumerate(vals) if i != o)
        S = np.abs(exact - vals[o]) + g2 * abs_other          # bound on |s|
        off = (u / (1 - u) * np.abs(got) + e * (np.abs(vals[o]) + (1 + u) * S)
               + u * S + g2 * abs_other)
        direct = u / (1 - u) * np.abs(got) + g3 * sum(np.abs(v) for v in vals)
        bound = np.where(np.arange(R) < H * c, off, direct)
        assert np.all(np.abs(got - exact) <= bound * (1 + 1e-9))
        # the extra rounding is visible: not every offload element is the plain sum
        if o == 0:
            plain = bf16_vals(orc.plain_sum(BF16, SUM, xs, 0, R))
            assert np.any(got[:H * c] != plain[:H * c])
            assert np.max(np.abs(ords(outs[0][H * c:]) - ords(orc.plain_sum(BF16, SUM, xs, 0, R)[H * c:]))) <= 1
    xi = int_inputs(A * R, A, 39)
    outs = orc.rs4_group(BF16, SUM, H, 500, R, xi)
    for o in range(A):
        assert np.array_equal(outs[o], orc.plain_sum(BF16, SUM, xi, o * R, R))


# --------------------------------------------------------------------------
# the plain definition itself: exact sum, one rounding
# --------------------------------------------------------------------------

def _brute_plain(bit_lists, fmt_bits, d):
    """Expected plain_sum bits from first principles: decode every input
    exactly, sum the rationals, divide by d, round once (brute force), and
    give a rounded-away or exact zero the sign IEEE 754 gives it."""
    fmt = brute.BINARY32 if fmt_bits == 32 else brute.BFLOAT16
    sign_bit = 1 << (fmt_bits - 1)
    out = []
    for elems in zip(*bit_lists):
        vals = [brute.decode(b, fmt_bits) for b in elems]
        exact = sum(vals, Fraction(0)) / d
        r = brute.round_nearest_even(exact, fmt)
        bits = brute.encode(r, fmt_bits)
        if r == 0:
            if exact != 0:
                bits = sign_bit if exact < 0 else 0
            else:
                bits = sign_bit if all(int(b) == sign_bit for b in elems) else 0
        out.append(bits)
    return out


def _wide_bits(rng, n, fmt_bits, spread):
    """n random finite bit patterns.  spread=None: biased exponents uniform over
    the whole range (subnormals included); otherwise within `spread` binades
    of a random centre, so that the terms overlap and rounding is decided by
    bits far below the leading one."""
    man_bits = 23 if fmt_bits == 32 else 7
    if spread is None:
        e = rng.integers(0, 255, n)
    else:
        centre = rng.integers(1, 255)
        e = np.clip(centre + rng.integers(-spread, spread + 1, n), 0, 254)
    m = rng.integers(0, 1 << man_bits, n)
    s = rng.integers(0, 2, n)
    bits = (s << (fmt_bits - 1)) | (e << man_bits) | m
    return bits.astype(np.uint32 if fmt_bits == 32 else np.uint16)


def _plain_bits(orc, dt, op, cols):
    if dt == F32:
        xs = [np.ascontiguousarray(c).view(np.float32) for c in cols]
        return orc.plain_sum(dt, op, xs, 0, len(cols[0])).view(np.uint32)
    return orc.plain_sum(dt, op, [np.ascontiguousarray(c) for c in cols], 0, len(cols[0]))


def test_plain_sum_cases_double_rounding_gets_wrong(orc):
    """1 + 2^-8 + 2^-80 lies above the bf16 midpoint 1 + 2^-8, so the sum rounds
    up to 0x3F81; an fp64 accumulator loses the 2^-80 term and rounds the
    midpoint to even (0x3F80).  The same for binary32 with 1 + 2^-24 + 2^-100."""
    got = _plain_bits(orc, BF16, SUM, [np.array([0x3F80], np.uint16), np.array([0x3B80], np.uint16),
                                       np.array([0x1780], np.uint16)])
    assert int(got[0]) == 0x3F81
    assert _brute_plain([[0x3F80], [0x3B80], [0x1780]], 16, 1) == [0x3F81]
    cols = [np.array([v], np.float32).view(np.uint32) for v in (1.0, 2.0 ** -24, 2.0 ** -100)]
    got = _plain_bits(orc, F32, SUM, cols)
    assert int(got[0]) == 0x3F800001
    assert _brute_plain([[int(c[0])] for c in cols], 32, 1) == [0x3F800001]


@pytest.mark.parametrize("dt", [F32, BF16])
@pytest.mark.parametrize("A,op", [(2, SUM), (2, AVG), (3, SUM), (3, AVG), (4, SUM), (4, AVG)])
def test_plain_sum_against_brute_force_wide_exponents(orc, dt, A, op):
    """Random finite inputs with exponent spreads from a few binades to the
    whole binary32 range, subnormals, overflow to infinity and (AVG with
    A = 3) a quotient that is not a dyadic rational: every output is the
    correctly rounded value."""
    fmt_bits = 32 if dt == F32 else 16
    rng = np.random.default_rng(1000 + 10 * A + op + 100 * dt)
    cols = [[] for _ in range(A)]
    for spread in (None, 4, 12, 30, 60, 100):
        for c in cols:
            c.append(_wide_bits(rng, 250, fmt_bits, spread))
    cols = [np.concatenate(c) for c in cols]
    # cancellation: x, -x and a small remainder
    k = 200
    x = _wide_bits(rng, k, fmt_bits, 20)
    sign = np.array(1 << (fmt_bits - 1), x.dtype)
    small = _wide_bits(rng, k, fmt_bits, None)
    extra = [x, x ^ sign] + [small] * (A - 2)
    cols = [np.concatenate([c, e]) for c, e in zip(cols, extra)]
    got = _plain_bits(orc, dt, op, cols)
    exp = _brute_plain([list(map(int, c)) for c in cols], fmt_bits, A if op == AVG else 1)
    bad = [i for i in range(len(exp)) if int(got[i]) != exp[i]]
    assert not bad, [(i, [hex(int(c[i])) for c in cols], hex(int(got[i])), hex(exp[i])) for i in bad[:5]]


@pytest.mark.parametrize("dt", [F32, BF16])
def test_plain_sum_special_values(orc, dt):
    """NaN in, or +inf with -inf: the default quiet NaN; an infinity alone: that
    infinity; an exact zero: -0 only when every input is -0; a finite sum
    beyond the largest finite value: infinity of its sign."""
    if dt == F32:
        Q, PINF, NINF, NZ, MAX = 0x7FC00000, 0x7F800000, 0xFF800000, 0x80000000, 0x7F7FFFFF
        one, mone, snan = 0x3F800000, 0xBF800000, 0x7F800001
        typ = np.uint32
    else:
        Q, PINF, NINF, NZ, MAX = 0x7FC0, 0x7F80, 0xFF80, 0x8000, 0x7F7F
        one, mone, snan = 0x3F80, 0xBF80, 0x7F81
        typ = np.uint16
    cases = [
        ((snan, one), Q), ((one, Q), Q), ((PINF, NINF), Q), ((PINF, one), PINF), ((NINF, MAX), NINF),
        ((NZ, NZ), NZ), ((NZ, 0), 0), ((one, mone), 0), ((MAX, MAX), PINF), ((MAX | NZ, MAX | NZ), NINF),
        ((MAX, MAX | NZ), 0),
    ]
    cols = [np.array([c[0][j] for c in cases], typ) for j in range(2)]
    got = _plain_bits(orc, dt, SUM, cols)
    assert [int(g) for g in got] == [e for _, e in cases]
