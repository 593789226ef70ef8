"""One-GPU synthesis of the relay hot path: every rank's and every helper's
buffers of one sparse group live in this GPU's HBM, and each role's local
kernel is launched through the C ABI exactly as that rank would launch it.

Point-to-point hops are not local work and are not launched here; a buffer a
rank would receive is represented by the bytes it would receive:

* a helper's slots are views of the active ranks' buffers (the scatter would
  copy exactly those bytes into the helper's scratch);
* the A=2 reduce-scatter peer block is the other active's block (the
  passthrough forwards and the direct exchange deliver it unchanged);
* the A=4 reduce-scatter helper scratch is filled once, untimed, with the
  (owner, source) chunks the scatter would deliver, owner-major;
* the all-to-all pack reads the source ranks' inputs directly, and unpack
  reads the per-destination buffers pack wrote.

Message size M is the per-active-rank input in bytes (the pull request's sweep
axis), bf16 unless stated.  Workload classes expose ``calls(stream)``: one
entry per kernel launch, ``(row, kernel, algorithmic_bytes, fn)`` with ``fn()``
issuing exactly that launch; ``run(stream)`` issues them all, and the buffers
the parity tests compare are attributes.  Algorithmic bytes count every input
element read once and every output element written once.
"""
import torch

from . import (ALLREDUCE, AVG, BF16, F32, REDUCE_SCATTER, SUM, Relay, rr_a2a_pack, rr_a2a_unpack,
               rr_active_add_scale, rr_geometry, rr_helper_reduce, rr_rs_multi_reduce)

TORCH = {F32: torch.float32, BF16: torch.bfloat16}
ESIZE = {F32: 4, BF16: 2}


COPY = "copy_kernel"


def reduce_kernel(dtype):
    return "reduce_kernel<bf16>" if dtype == BF16 else "reduce_kernel<f32>"


class _Row:
    def run(self, stream=None):
        for _, _, _, fn in self.calls(stream):
            fn()

    def bytes_per_step(self):
        return sum(b for _, _, b, _ in self.calls())


class AR2(_Row):
    """A=2 allreduce: reduce-at-helper (summary section 2) over the H relay
    chunks and the active epilogue over the direct region (section 1)."""

    def __init__(self, xs, dtype, op=AVG, H=6, numChunks=8, helpers=True, actives=True):
        self.dtype, self.op = dtype, op
        self.count = xs[0].numel()
        self.relay = Relay(2, H, numChunks, 0, self.count)
        g = rr_geometry(self.relay, ALLREDUCE, dtype)
        self.g, c, es = g, g["chunk"], ESIZE[dtype]
        self.x = xs
        self.red = [torch.empty(max(c, 1), dtype=TORCH[dtype], device=xs[0].device) for _ in range(H)]
        self.out = [torch.empty_like(xs[0]) for _ in range(2)]
        self.do_helpers, self.do_actives = helpers, actives
        self.es = es

    def calls(self, stream=None):
        c, es, out = self.g["chunk"], self.es, []
        if self.do_helpers and c:
            for k in range(self.relay.H):
                sl = slice(k * c, (k + 1) * c)
                out.append(("ar2_helper", reduce_kernel(self.dtype), 3 * c * es,
                            lambda sl=sl, k=k: rr_helper_reduce(
                                self.relay, ALLREDUCE, self.dtype, self.op, k,
                                [self.x[0][sl], self.x[1][sl]], self.red[k], stream)))
        if self.do_actives and self.g["direct_len"]:
            for a in range(2):
                out.append(("ar2_active", reduce_kernel(self.dtype), 3 * self.g["direct_len"] * es,
                            lambda a=a: rr_active_add_scale(
                                self.relay, ALLREDUCE, self.dtype, self.op, a, self.x,
                                self.out[a], stream)))
        return out

    def deliver_returns(self):
        """The helpers' return hop (a copy per active), for whole-group checks."""
        c = self.g["chunk"]
        for k in range(self.relay.H):
            for a in range(2):
                self.out[a][k * c:(k + 1) * c].copy_(self.red[k][:c])


class RS2(_Row):
    """A=2 reduce-scatter owner epilogue: the fused add + scale of the relayed
    and direct chunks over the whole recvCount block (reduce-scatter core
    commit, phases 3 and 5).  xs[a] holds 2 blocks of R."""

    def __init__(self, xs, dtype, op=AVG, H=6, numChunks=8, in_place=False):
        self.dtype, self.op = dtype, op
        self.R = xs[0].numel() // 2
        self.relay = Relay(2, H, numChunks, 0, self.R)
        self.x = xs
        R = self.R
        if in_place:
            self.own = [xs[0][:R].clone(), xs[1][R:].clone()]
            self.out = self.own
        else:
            self.own = [xs[0][:R], xs[1][R:]]
            self.out = [torch.empty(R, dtype=TORCH[dtype], device=xs[0].device) for _ in range(2)]
        # the peer block as delivered: the other active's contribution, unsummed
        self.peer = [xs[1][:R], xs[0][R:]]

    def calls(self, stream=None):
        out = []
        for o in range(2 if self.R else 0):
            ins = [self.own[0], self.peer[0]] if o == 0 else [self.peer[1], self.own[1]]
            out.append(("rs2_owner", reduce_kernel(self.dtype), 3 * self.R * ESIZE[self.dtype],
                        lambda o=o, ins=ins: rr_active_add_scale(
                            self.relay, REDUCE_SCATTER, self.dtype, self.op, o, ins, self.out[o],
                            stream)))
        return out


class AR4(_Row):
    """A=4 allreduce at an offload fraction (summary section 4): the H helpers
    reduce their position slices 4->1, the A actives reduce their direct
    slices."""

    def __init__(self, xs, dtype, op=AVG, H=4, permille=500):
        self.dtype, self.op = dtype, op
        self.count = xs[0].numel()
        self.relay = Relay(4, H, 0, permille, self.count)
        g = rr_geometry(self.relay, ALLREDUCE, dtype)
        self.g, c, es = g, g["chunk"], ESIZE[dtype]
        self.x = xs
        self.red = [torch.empty(max(c, 1), dtype=TORCH[dtype], device=xs[0].device) for _ in range(H)]
        self.out = [torch.empty_like(xs[0]) for _ in range(4)]
        self.es = es

    def calls(self, stream=None):
        c, g, es, out = self.g["chunk"], self.g, self.es, []
        for h in range(self.relay.H if c else 0):
            sl = slice(h * c, (h + 1) * c)
            out.append(("ar4_helper", reduce_kernel(self.dtype), 5 * c * es,
                        lambda sl=sl, h=h: rr_helper_reduce(
                            self.relay, ALLREDUCE, self.dtype, self.op, h,
                            [x[sl] for x in self.x], self.red[h], stream)))
        for a in range(4):
            n = g["dslice"] if a < 3 else g["direct_len"] - 3 * g["dslice"]
            if n:
                out.append(("ar4_active", reduce_kernel(self.dtype), 5 * n * es,
                            lambda a=a: rr_active_add_scale(
                                self.relay, ALLREDUCE, self.dtype, self.op, a, self.x,
                                self.out[a], stream)))
        return out

    def deliver(self):
        """Broadcast of the helpers' chunks and the all-gather of the direct
        slices (copies), for whole-group checks."""
        c, g = self.g["chunk"], self.g
        for h in range(self.relay.H):
            for a in range(4):
                self.out[a][h * c:(h + 1) * c].copy_(self.red[h][:c])
        for a in range(4):
            lo = g["direct_off"] + a * g["dslice"]
            hi = lo + g["dslice"] if a < 3 else self.count
            for b in range(4):
                if b != a:
                    self.out[b][lo:hi].copy_(self.out[a][lo:hi])


class RS4(_Row):
    """A=4 reduce-scatter, flat reduce-at-helper (summary section 6): pass 1 at
    each helper over its (owner, source) scratch, pass 2 at each owner.
    xs[s] holds A blocks of R."""

    def __init__(self, xs, dtype, op=SUM, H=4, permille=500):
        A = 4
        self.dtype, self.op = dtype, op
        self.R = R = xs[0].numel() // A
        self.relay = Relay(A, H, 0, permille, R)
        g = rr_geometry(self.relay, REDUCE_SCATTER, dtype)
        self.g, c, es = g, g["chunk"], ESIZE[dtype]
        self.x = xs
        dev = xs[0].device
        # helper scratch, 2R each: A*(A-1) chunks owner-major, then A reduced chunks
        self.scratch = [torch.empty(2 * R, dtype=TORCH[dtype], device=dev) for _ in range(H)]
        for h in range(H):
            for o in range(A):
                for j, s in enumerate(s for s in range(A) if s != o):
                    dst = (o * (A - 1) + j) * c
                    self.scratch[h][dst:dst + c].copy_(xs[s][o * R + h * c:o * R + (h + 1) * c])
        self.out = [torch.empty(R, dtype=TORCH[dtype], device=dev) for _ in range(A)]
        self.es = es

    def reduced(self, h, o):
        c, A = self.g["chunk"], 4
        base = A * (A - 1) * c
        return self.scratch[h][base + o * c:base + (o + 1) * c]

    def calls(self, stream=None):
        A, c, R, H, es, out = 4, self.g["chunk"], self.R, self.relay.H, self.es, []
        for h in range(H if c else 0):
            out.append(("rs4_pass1", reduce_kernel(self.dtype), (A * (A - 1) + A) * c * es,
                        lambda h=h: rr_rs_multi_reduce(
                            self.relay, self.dtype, self.op, 1, h, [self.scratch[h]],
                            self.scratch[h][A * (A - 1) * c:], stream)))
        for o in range(A if R else 0):
            blocks = [x[o * R:(o + 1) * R] for x in self.x]
            reds = [self.reduced(h, o) if c else blocks[0] for h in range(H)]
            out.append(("rs4_pass2", reduce_kernel(self.dtype), (3 * H * c + (A + 1) * (R - H * c)) * es,
                        lambda o=o, ins=blocks + reds: rr_rs_multi_reduce(
                            self.relay, self.dtype, self.op, 2, o, ins, self.out[o], stream)))
        return out


class A2A(_Row):
    """A=4 all-to-all helper coalescing (reverted all-to-all paragraph): one
    pack and one unpack per helper slice.  src[s] holds A segments of seg."""

    def __init__(self, src, dtype=BF16, H=4, numChunks=5):
        A = 4
        self.dtype = dtype
        self.seg = seg = src[0].numel() // A
        self.relay = Relay(A, H, numChunks, 0, seg)
        g = rr_geometry(self.relay, 2, dtype)
        self.g, c, es = g, g["chunk"], ESIZE[dtype]
        self.src = src
        dev = src[0].device
        self.packed = [[torch.empty(max((A - 1) * c, 1), dtype=src[0].dtype, device=dev) for _ in range(A)]
                       for _ in range(H)]
        self.out = [torch.zeros_like(s) for s in src]
        self.es = es

    def calls(self, stream=None):
        A, c, es, out = 4, self.g["chunk"], self.es, []
        kern = COPY if (self.seg * es) % 16 == 0 else "copy_kernel+copy_shifted_kernel"
        for h in range(self.relay.H if c else 0):
            out.append(("a2a_pack", kern, 2 * A * (A - 1) * c * es,
                        lambda h=h: rr_a2a_pack(self.relay, self.dtype, h, self.src, self.packed[h],
                                                stream)))
        for h in range(self.relay.H if c else 0):
            out.append(("a2a_unpack", kern, 2 * A * (A - 1) * c * es,
                        lambda h=h: rr_a2a_unpack(self.relay, self.dtype, h, self.packed[h],
                                                  self.out, stream)))
        return out


def message_shapes(M, es=2):
    """Element counts for a per-active-rank input of M bytes."""
    return {
        "ar2_count": M // es,
        "rs2_recv": M // (2 * es),
        "ar4_count": M // es,
        "rs4_recv": M // (4 * es),
        "a2a_seg": M // (4 * es),
    }
