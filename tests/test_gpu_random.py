"""GPU parity on seeded random geometries: random A, H, numChunks, permille,
counts, dtypes, ops and element offsets of every input and output, issued
as batched calls so that the library picks each launch form (one aligned
segment, equal segments on a uniform grid, the tile table) on irregular
shapes.  Every output is compared with the CPU oracle bit for bit (both
sides add in fp32 in the same order and round once), and the elements
around every output must keep their sentinel values."""
import numpy as np
import pytest
import torch

import pack_rr_helper_amd as rr
from pack_rr_helper_amd import synth

pytestmark = pytest.mark.gpu

F32, BF16 = 0, 1
AR, RS = 0, 1
PAD = 64                       # guard elements on each side of a view
SENTINEL = {F32: np.float32(-7.25), BF16: np.uint16(0x7FA5)}


@pytest.fixture(scope="module", autouse=True)
def device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rr.load()
    yield
    torch.cuda.synchronize()


def npdt(dt):
    return np.float32 if dt == F32 else np.uint16


def values(n, seed, rank, dt):
    x = synth.normal(n, seed, rank)
    return x if dt == F32 else synth.as_bf16_bits(x)


class View:
    """n elements at element offset `lead` inside a sentinel-filled device
    buffer with PAD guard elements on both sides."""

    def __init__(self, host, dt, lead):
        self.n, self.lead, self.dt = host.size, lead, dt
        big = np.full(host.size + lead + 2 * PAD, SENTINEL[dt], npdt(dt))
        big[PAD + lead:PAD + lead + host.size] = host
        self.big = synth.to_device(big, dt)
        self.t = self.big[PAD + lead:PAD + lead + host.size]

    def host(self):
        torch.cuda.synchronize()
        return synth.to_host(self.big)[PAD + self.lead:PAD + self.lead + self.n]

    def guards_intact(self):
        torch.cuda.synchronize()
        b = synth.to_host(self.big)
        s = SENTINEL[self.dt]
        return bool(np.all(b[:PAD + self.lead] == s) and np.all(b[PAD + self.lead + self.n:] == s))


def same_bits(got, ref, what):
    assert np.array_equal(got.view(np.uint8), np.ascontiguousarray(ref).view(np.uint8)), what


@pytest.mark.parametrize("seed", range(192))
def test_random_allreduce_batches(orc, seed):
    rng = np.random.default_rng(5000 + seed)
    A = int(rng.choice([2, 4]))
    H = int(rng.integers(1, 7)) if A == 2 else int(rng.integers(1, 5))
    dt = int(rng.choice([F32, BF16]))
    op = int(rng.choice([0, 1]))
    es = 4 if dt == F32 else 2
    nc = H + 2 + int(rng.integers(0, 3)) if A == 2 else 0
    pm = int(rng.choice([250, 500, 780, 1000])) if A == 4 else 0
    count = int(rng.integers(1, (3 << 20) // es)) if A == 4 else int(rng.integers(1, 400000))
    g = orc.geometry(A, H, nc, pm, count, AR, dt)
    print(f"[gpu-case] random allreduce seed={seed} A={A} H={H} dt={dt} op={op} count={count}", flush=True)
    relay = rr.Relay(A, H, nc, pm, count)
    xs = [values(count, 6000 + seed, r, dt) for r in range(A)]
    ins = [View(x, dt, int(rng.choice([0, int(rng.integers(0, 8))]))) for x in xs]
    outs = [View(np.full(count, SENTINEL[dt], npdt(dt)), dt, int(rng.integers(0, 8))) for _ in range(A)]
    rr.rr_active_add_scale_many(AR, dt, op, [(relay, a, [v.t for v in ins], outs[a].t) for a in range(A)])
    for a in range(A):
        ref = orc.ar_active(dt, op, A, H, nc, pm, count, a, xs, np.full(count, SENTINEL[dt], npdt(dt)))
        same_bits(outs[a].host(), ref, f"active {a}")
        assert outs[a].guards_intact(), f"active {a} wrote outside its output"
    c = g["chunk"]
    if c:
        hout = [View(np.zeros(c, npdt(dt)), dt, int(rng.integers(0, 8))) for _ in range(H)]
        jobs = [(relay, h, [v.t[h * c:(h + 1) * c] for v in ins], hout[h].t) for h in range(H)]
        rr.rr_helper_reduce_many(AR, dt, op, jobs)
        for h in range(H):
            sl = [x[h * c:(h + 1) * c].copy() for x in xs]
            ref = orc.ar2_helper(dt, op, *sl) if A == 2 else orc.ar4_helper(dt, op, sl)
            same_bits(hout[h].host(), ref, f"helper {h}")
            assert hout[h].guards_intact(), f"helper {h} wrote outside its output"


@pytest.mark.parametrize("seed", range(96))
def test_random_four_active_reduce_scatter(orc, seed):
    rng = np.random.default_rng(7000 + seed)
    A, H = 4, int(rng.integers(1, 5))
    dt = int(rng.choice([F32, BF16]))
    op = int(rng.choice([0, 1]))
    R = int(rng.integers(1, 300000))
    # the helper holds A*(A-1) input and A reduced chunks within 2*recvCount:
    # 16 * R * permille / (1000 * H) <= 2 R, i.e. permille <= 125 * H
    pm = int(rng.integers(1, 5 * H + 1)) * 25
    g = orc.geometry(A, H, 0, pm, R, RS, dt)
    c = g["chunk"]
    print(f"[gpu-case] random rs4 seed={seed} H={H} permille={pm} dt={dt} op={op} R={R} chunk={c}", flush=True)
    relay = rr.Relay(A, H, 0, pm, R)
    xs = [values(A * R, 8000 + seed, s, dt) for s in range(A)]
    blocks = [[View(xs[s][o * R:(o + 1) * R].copy(), dt, int(rng.integers(0, 8))) for s in range(A)]
              for o in range(A)]
    scratch = []
    if c:
        for h in range(H):
            hs = np.concatenate([xs[s][o * R + h * c:o * R + (h + 1) * c]
                                 for o in range(A) for s in range(A) if s != o])
            full = np.zeros(2 * R, npdt(dt))
            full[:hs.size] = hs
            scratch.append(View(full, dt, int(rng.integers(0, 8))))
        rr.rr_rs_multi_reduce_many(dt, op, [(relay, 1, h, [scratch[h].t], scratch[h].t[A * (A - 1) * c:])
                                            for h in range(H)])
    outs = [View(np.zeros(R, npdt(dt)), dt, int(rng.integers(0, 8))) for _ in range(A)]
    jobs = []
    for o in range(A):
        reds = [scratch[h].t[A * (A - 1) * c + o * c:A * (A - 1) * c + (o + 1) * c] if c else blocks[o][0].t
                for h in range(H)]
        jobs.append((relay, 2, o, [v.t for v in blocks[o]] + reds, outs[o].t))
    rr.rr_rs_multi_reduce_many(dt, op, jobs)
    ref = orc.rs4_group(dt, op, H, pm, R, xs)
    for o in range(A):
        same_bits(outs[o].host(), ref[o], f"owner {o}")
        assert outs[o].guards_intact(), f"owner {o} wrote outside its output"


@pytest.mark.parametrize("seed", range(96))
def test_random_all_to_all(orc, seed):
    rng = np.random.default_rng(9000 + seed)
    A, H = 4, int(rng.integers(1, 5))
    dt = int(rng.choice([F32, BF16]))
    es = 4 if dt == F32 else 2
    nc = H + 1 + int(rng.integers(0, 3))
    seg = int(rng.integers(1, 200000))
    c = orc.geometry(A, H, nc, 0, seg, 2, dt)["chunk"]
    print(f"[gpu-case] random a2a seed={seed} H={H} dt={dt} seg={seg} chunk={c}", flush=True)
    relay = rr.Relay(A, H, nc, 0, seg)
    raw = np.uint32 if es == 4 else np.uint16
    src = [synth.rng(9500 + seed, s).integers(0, 1 << (8 * es), A * seg, dtype=raw) for s in range(A)]
    dev_view = lambda a, lead: View(a.view(np.float32) if es == 4 else a, dt, lead)
    sv = [dev_view(s, int(rng.integers(0, 8))) for s in src]
    if not c:
        return
    packed = [[dev_view(np.zeros((A - 1) * c, raw), int(rng.integers(0, 8))) for _ in range(A)] for _ in range(H)]
    rr.rr_a2a_pack_many(dt, [(relay, h, [v.t for v in sv], [p.t for p in packed[h]]) for h in range(H)])
    outs = [dev_view(np.zeros(A * seg, raw), int(rng.integers(0, 8))) for _ in range(A)]
    rr.rr_a2a_unpack_many(dt, [(relay, h, [p.t for p in packed[h]], [o.t for o in outs]) for h in range(H)])
    expect = [np.zeros(A * seg, raw) for _ in range(A)]
    for h in range(H):
        ref = orc.a2a_pack(es, A, seg, c, h, src)
        for d in range(A):
            same_bits(packed[h][d].host(), ref[d], f"pack helper {h} dest {d}")
            assert packed[h][d].guards_intact()
        orc.a2a_unpack(es, A, seg, c, h, ref, expect)
    for d in range(A):
        same_bits(outs[d].host(), expect[d], f"unpack dest {d}")
        assert outs[d].guards_intact()
