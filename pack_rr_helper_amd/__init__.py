"""Python binding of librr.so, the gfx950 C-ABI library for the per-GPU hot path
of the link-balanced sharded relay collectives (torchrec pull request #4570,
"Link-balance the sharded relay schedules").

The functions carry the C entry points' names and only marshal arguments:
torch device tensors become device pointers, ``stream`` defaults to torch's
current stream, and every step runs in the library's HIP kernels.  The binding
checks what the C ABI cannot see -- that every tensor lives on the GPU, is
contiguous, has the buffer dtype and is large enough -- and raises
``ValueError`` for a rejected argument and ``RuntimeError`` for a HIP failure
or a missing library.  There is no CPU fallback.

Every entry point also accepts ``prepare=True``: the checks, the ctypes
marshalling and the library's own validation and segment tables then run
once, recorded into a plan (rr_plan_* in rr.h), and a zero-argument callable
is returned that only re-issues the recorded launches (on the stream chosen at
preparation; the tensors are kept alive by the callable).  ``Plan`` records
several calls into one plan that is launched with a single C call.  The
``*_many`` forms take lists of per-group jobs and enqueue them together,
typically as one kernel launch.

Pointer/layout semantics of each call are documented in include/rr.h.
"""
import ctypes
import os
import threading
from dataclasses import dataclass

import torch

__all__ = [
    "Relay", "RRError", "F32", "BF16", "SUM", "AVG", "ALLREDUCE", "REDUCE_SCATTER", "ALLTOALL",
    "library_path", "load", "rr_abi_version", "rr_geometry", "rr_passthrough_helper_size",
    "rr_helper_reduce", "rr_active_add_scale", "rr_rs_multi_reduce", "rr_a2a_pack",
    "rr_a2a_unpack", "rr_helper_reduce_many", "rr_active_add_scale_many",
    "rr_rs_multi_reduce_many", "rr_a2a_pack_many", "rr_a2a_unpack_many", "rr_phase_reduce_many",
    "Plan",
]

F32, BF16 = 0, 1
SUM, AVG = 0, 1
ALLREDUCE, REDUCE_SCATTER, ALLTOALL = 0, 1, 2
RR_OK, RR_EINVAL, RR_EALIAS, RR_EUNSUPPORTED, RR_EHIP = 0, 1, 2, 3, 4
_STATUS = {1: "RR_EINVAL", 2: "RR_EALIAS", 3: "RR_EUNSUPPORTED", 4: "RR_EHIP"}

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "librr.so")


class RRError(ValueError):
    """A call the library rejected; ``status`` is the rr_status code."""

    def __init__(self, status, msg):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class _Relay(ctypes.Structure):
    _fields_ = [("A", ctypes.c_int32), ("H", ctypes.c_int32), ("numChunks", ctypes.c_int32),
                ("permille", ctypes.c_int32), ("count", ctypes.c_int64)]


class _Geom(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "chunk", "relay_total", "direct_off", "direct_len", "dirA_off", "dirA_len",
        "dirB_off", "dirB_len", "dslice", "helper_elems")] + [
        ("pure_direct", ctypes.c_int32), ("reserved", ctypes.c_int32)]


@dataclass(frozen=True)
class Relay:
    """One group's relay parameters in the pull request's terms (see rr.h)."""
    A: int
    H: int
    numChunks: int = 0
    permille: int = 500
    count: int = 0

    def _c(self):
        return _Relay(self.A, self.H, self.numChunks, self.permille, self.count)


class _HelperJob(ctypes.Structure):
    _fields_ = [("relay", _Relay), ("helper", ctypes.c_int32), ("nSlots", ctypes.c_int32),
                ("slots", ctypes.c_void_p * 4), ("out", ctypes.c_void_p)]


class _ActiveJob(ctypes.Structure):
    _fields_ = [("relay", _Relay), ("activeIdx", ctypes.c_int32), ("nIn", ctypes.c_int32),
                ("inp", ctypes.c_void_p * 4), ("out", ctypes.c_void_p)]


class _RsJob(ctypes.Structure):
    _fields_ = [("relay", _Relay), ("pass_", ctypes.c_int32), ("idx", ctypes.c_int32),
                ("nIn", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("inp", ctypes.POINTER(ctypes.c_void_p)), ("out", ctypes.c_void_p)]


class _A2AJob(ctypes.Structure):
    _fields_ = [("relay", _Relay), ("helper", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("inp", ctypes.POINTER(ctypes.c_void_p)), ("out", ctypes.POINTER(ctypes.c_void_p))]


_lib = None


def load():
    """Load librr.so (built by pack_rr_helper_amd/build.py); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise RuntimeError(
            f"{library_path} is missing: build it with `python -m pack_rr_helper_amd.build` "
            "(the relay hot path has no CPU fallback)")
    L = ctypes.CDLL(library_path)
    vp, i32, i64, pp = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.POINTER(ctypes.c_void_p)
    rp = ctypes.POINTER(_Relay)
    ci = ctypes.c_int
    for name, res, args in [
        ("rr_abi_version", ci, []),
        ("rr_last_error", ctypes.c_char_p, []),
        ("rr_geometry", ci, [rp, ci, ci, ctypes.POINTER(_Geom)]),
        ("rr_passthrough_helper_size", i64, [i64, i32, i32]),
        ("rr_helper_reduce", ci, [rp, ci, ci, ci, ci, pp, ci, vp, vp]),
        ("rr_active_add_scale", ci, [rp, ci, ci, ci, ci, pp, ci, vp, vp]),
        ("rr_rs_multi_reduce", ci, [rp, ci, ci, ci, ci, pp, ci, vp, vp]),
        ("rr_a2a_pack", ci, [rp, ci, ci, pp, pp, vp]),
        ("rr_a2a_unpack", ci, [rp, ci, ci, pp, pp, vp]),
        ("rr_helper_reduce_many", ci, [ci, ci, ci, ctypes.POINTER(_HelperJob), ci, vp]),
        ("rr_active_add_scale_many", ci, [ci, ci, ci, ctypes.POINTER(_ActiveJob), ci, vp]),
        ("rr_rs_multi_reduce_many", ci, [ci, ci, ctypes.POINTER(_RsJob), ci, vp]),
        ("rr_a2a_pack_many", ci, [ci, ctypes.POINTER(_A2AJob), ci, vp]),
        ("rr_a2a_unpack_many", ci, [ci, ctypes.POINTER(_A2AJob), ci, vp]),
        ("rr_phase_reduce_many", ci, [ci, ci, ci, ctypes.POINTER(_HelperJob), ci,
                                      ctypes.POINTER(_ActiveJob), ci, vp]),
        ("rr_plan_bytes", ctypes.c_size_t, [i32]),
        ("rr_plan_begin", ci, [vp, ctypes.c_size_t]),
        ("rr_plan_end", ci, [ctypes.POINTER(i32)]),
        ("rr_plan_append", ci, [vp, ctypes.c_size_t, vp]),
        ("rr_plan_launch", ci, [vp, vp]),
    ]:
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    _lib = L
    return L


def _raise(st):
    if st == RR_OK:
        return
    msg = load().rr_last_error().decode(errors="replace")
    if st == RR_EHIP:
        raise RuntimeError(f"RR_EHIP: {msg}")
    raise RRError(st, msg)


# --------------------------------------------------------------------------
# marshalling
# --------------------------------------------------------------------------

_TORCH_DT = {F32: (torch.float32,), BF16: (torch.bfloat16,)}
_BITS_DT = {4: (torch.float32, torch.int32, torch.uint32),
            2: (torch.bfloat16, torch.float16, torch.int16, torch.uint16)}


def _esize(dtype):
    if dtype not in (F32, BF16):
        raise RRError(RR_EINVAL, f"unknown dtype {dtype}")
    return 4 if dtype == F32 else 2


def _dev(t, what, dtype, min_elems, bits=False):
    """Device pointer of tensor t after the checks the C ABI cannot make."""
    if not isinstance(t, torch.Tensor):
        raise RRError(RR_EINVAL, f"{what} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise RRError(RR_EINVAL, f"{what} is on {t.device}, the kernels need device memory")
    ok_dt = _BITS_DT[_esize(dtype)] if bits else _TORCH_DT[dtype]
    if t.dtype not in ok_dt:
        raise RRError(RR_EINVAL, f"{what} has dtype {t.dtype}, expected one of {ok_dt}")
    if not t.is_contiguous():
        raise RRError(RR_EINVAL, f"{what} must be contiguous")
    if t.numel() < min_elems:
        raise RRError(RR_EINVAL, f"{what} holds {t.numel()} elements, needs {min_elems}")
    return t.data_ptr()


def _ptrs(ts, what, dtype, min_elems, bits=False):
    if isinstance(ts, torch.Tensor):
        ts = [ts]
    ts = list(ts)
    arr = (ctypes.c_void_p * max(len(ts), 1))()
    for i, t in enumerate(ts):
        arr[i] = _dev(t, f"{what}[{i}]", dtype, min_elems[i] if isinstance(min_elems, list) else min_elems,
                      bits)
    return arr, len(ts)


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


# --------------------------------------------------------------------------
# entry points
# --------------------------------------------------------------------------

def rr_abi_version():
    """ABI version compiled into librr.so (RR_ABI_VERSION)."""
    return load().rr_abi_version()


def rr_geometry(relay, coll, dtype):
    """The group's geometry as a dict (see rr_geom in rr.h)."""
    g = _Geom()
    r = relay._c()
    _raise(load().rr_geometry(ctypes.byref(r), coll, dtype, ctypes.byref(g)))
    return {n: getattr(g, n) for n, _ in _Geom._fields_ if n != "reserved"}


def rr_passthrough_helper_size(count_g, A, num_chunks):
    """Elements of a passthrough helper buffer: min(count_g, A * align_down(count_g / num_chunks, 128))."""
    v = load().rr_passthrough_helper_size(count_g, A, num_chunks)
    if v < 0:
        raise RRError(RR_EINVAL, "count_g < 0, A < 1 or num_chunks < 1")
    return v


_tls = threading.local()
PLAN_MAX_LAUNCHES = 4096  # RR_PLAN_MAX_LAUNCHES


class Plan:
    """Relay calls validated once and re-issued together with one C call.

    ``with Plan(n) as p:`` records every entry point called on this thread in
    the block (each validates as usual; nothing is enqueued), then ``p()`` or
    ``p.launch(stream)`` enqueues all recorded kernel launches in order, with
    no checks: the tensors the recorded calls named are kept alive by the plan
    and must keep their contents' meaning (same buffers, same sizes).  ``n``
    bounds the launches the plan holds (rr_plan_bytes); the plan's memory is a
    host buffer owned by this object."""

    def __init__(self, max_launches=64):
        nbytes = load().rr_plan_bytes(max_launches)
        if nbytes == 0:
            raise RRError(RR_EINVAL, f"a plan holds 1..{PLAN_MAX_LAUNCHES} launches, not {max_launches}")
        self._buf = (ctypes.c_uint64 * ((nbytes + 7) // 8))()  # 8-byte aligned host memory
        self._bytes = nbytes
        self._keep = []
        self.launches = None
        self.stream = None

    def __enter__(self):
        if getattr(_tls, "plan", None) is not None:
            raise RRError(RR_EINVAL, "this thread is already recording a plan")
        _raise(load().rr_plan_begin(self._buf, self._bytes))
        _tls.plan = self
        return self

    def __exit__(self, et, ev, tb):
        _tls.plan = None
        n = ctypes.c_int32()
        st = load().rr_plan_end(ctypes.byref(n))
        self.launches = n.value
        if et is None:
            _raise(st)
        return False

    def extend(self, *others):
        """Append the launches of finished plans (or prepared calls) to this
        finished plan, so that one launch issues them all in order."""
        for o in others:
            _raise(load().rr_plan_append(self._buf, self._bytes, o._buf))
            self._keep.append(o._keep)
            self.launches += o.launches
        return self

    def launch(self, stream=None):
        """Enqueue the recorded launches on `stream` (default: the stream
        chosen at preparation, else torch's current stream)."""
        s = _stream(stream) if stream is not None or self.stream is None else self.stream
        _raise(load().rr_plan_launch(self._buf, s))

    __call__ = launch


def _issue(fn, args, keep, prepare):
    """Call the C entry point now (recording it if a Plan is being recorded on
    this thread), or record it alone into a plan and return a callable that
    re-issues its launches on the stream of the call (its last argument)."""
    plan = getattr(_tls, "plan", None)
    if plan is not None:
        if prepare:
            raise RRError(RR_EINVAL, "prepare=True inside a Plan recording")
        _raise(fn(*args))
        plan._keep.append(keep)
        return None
    if not prepare:
        _raise(fn(*args))
        return None
    # recorded once to count its launches, then into a plan of that size
    scratch = getattr(_tls, "scratch", None)
    if scratch is None:
        scratch = _tls.scratch = Plan(PLAN_MAX_LAUNCHES)
    with scratch:
        _raise(fn(*args))
    p = Plan(max(scratch.launches, 1))
    with p:
        _raise(fn(*args))
    p.stream = args[-1]
    p._keep.append(keep)
    return p


def _helper_need(relay, coll, dtype):
    return rr_geometry(relay, coll, dtype)["chunk"] if coll == ALLREDUCE else 0


def rr_helper_reduce(relay, coll, dtype, op, helper, slots, out, stream=None, prepare=False):
    """Allreduce reduce-at-helper: out = scale * (slots[0] + ... + slots[A-1]) over
    the group's chunk (A=2: the two actives' copies of chunk `helper`; A=4: the
    four actives' position slices).  `out` may be slots[0] exactly.  A zero
    chunk is a no-op."""
    n = _helper_need(relay, coll, dtype)
    arr, k = _ptrs(slots, "slots", dtype, n)
    o = _dev(out, "out", dtype, n)
    r = relay._c()
    return _issue(load().rr_helper_reduce,
                  (ctypes.byref(r), coll, dtype, op, helper, arr, k, ctypes.c_void_p(o), _stream(stream)),
                  (r, arr, slots, out), prepare)


def rr_active_add_scale(relay, coll, dtype, op, active_idx, inputs, out, stream=None, prepare=False):
    """Active epilogue: out = scale * sum of the A inputs over this active's
    direct region (allreduce) or over the whole block (A=2 reduce-scatter
    owner).  Inputs are full buffers of relay.count elements, one per active in
    rank order; `out` may equal one of them exactly."""
    arr, k = _ptrs(inputs, "in", dtype, relay.count)
    o = _dev(out, "out", dtype, relay.count)
    r = relay._c()
    return _issue(load().rr_active_add_scale,
                  (ctypes.byref(r), coll, dtype, op, active_idx, arr, k, ctypes.c_void_p(o), _stream(stream)),
                  (r, arr, inputs, out), prepare)


def _rs_need(relay, dtype, pass_, n_inputs):
    g = rr_geometry(relay, REDUCE_SCATTER, dtype)
    A, c, R = relay.A, g["chunk"], relay.count
    if pass_ == 1:
        return [A * (A - 1) * c] * n_inputs, A * c
    return [R if i < A else c for i in range(n_inputs)], R


def rr_rs_multi_reduce(relay, dtype, op, pass_, idx, inputs, out, stream=None, prepare=False):
    """A=4 reduce-scatter passes.  pass_=1 (helper idx): inputs = [scratch]
    holding the A*(A-1) (owner, source) chunks; out receives the A reduced
    chunks.  pass_=2 (owner idx): inputs = the A blocks then the H reduced
    chunks; out receives the owner's recvCount elements."""
    inputs = list(inputs) if not isinstance(inputs, torch.Tensor) else [inputs]
    need, out_need = _rs_need(relay, dtype, pass_, len(inputs))
    arr, k = _ptrs(inputs, "in", dtype, need)
    o = _dev(out, "out", dtype, out_need)
    r = relay._c()
    return _issue(load().rr_rs_multi_reduce,
                  (ctypes.byref(r), dtype, op, pass_, idx, arr, k, ctypes.c_void_p(o), _stream(stream)),
                  (r, arr, inputs, out), prepare)


def _a2a_sizes(relay, dtype):
    g = rr_geometry(relay, ALLTOALL, dtype)
    return relay.A * relay.count, (relay.A - 1) * g["chunk"]


def _a2a_arrays(relay, dtype, ins, outs, unpack):
    full, packed = _a2a_sizes(relay, dtype)
    if len(ins) != relay.A or len(outs) != relay.A:
        raise RRError(RR_EINVAL, f"all-to-all takes A={relay.A} input and A output buffers")
    names = ("recv", "out") if unpack else ("src", "dst")
    a, _ = _ptrs(ins, names[0], dtype, packed if unpack else full, bits=True)
    b, _ = _ptrs(outs, names[1], dtype, full if unpack else packed, bits=True)
    return a, b


def rr_a2a_pack(relay, dtype, helper, src, dst, stream=None, prepare=False):
    """All-to-all gather for helper slice `helper`: dst[d] receives, in
    ascending source order skipping d, each source's chunk of segment d.
    Out-of-place only; raw bits are copied."""
    s, d = _a2a_arrays(relay, dtype, src, dst, False)
    r = relay._c()
    return _issue(load().rr_a2a_pack, (ctypes.byref(r), dtype, helper, s, d, _stream(stream)),
                  (r, s, d, src, dst), prepare)


def rr_a2a_unpack(relay, dtype, helper, recv, out, stream=None, prepare=False):
    """The inverse scatter: out[d] receives each source's chunk from recv[d] at
    the helper slice of that source's segment.  Out-of-place only."""
    s, d = _a2a_arrays(relay, dtype, recv, out, True)
    r = relay._c()
    return _issue(load().rr_a2a_unpack, (ctypes.byref(r), dtype, helper, s, d, _stream(stream)),
                  (r, s, d, recv, out), prepare)


# --------------------------------------------------------------------------
# batched forms: jobs are tuples in the single-job argument order
# --------------------------------------------------------------------------

def _helper_jobs(coll, dtype, jobs, first=0):
    arr = (_HelperJob * max(len(jobs), 1))()
    for j, (relay, helper, slots, out) in enumerate(jobs):
        n = _helper_need(relay, coll, dtype)
        p, k = _ptrs(slots, f"job {first + j} slots", dtype, n)
        arr[j].relay, arr[j].helper, arr[j].nSlots = relay._c(), helper, k
        for i in range(min(k, 4)):
            arr[j].slots[i] = p[i]
        arr[j].out = _dev(out, f"job {first + j} out", dtype, n)
    return arr


def _active_jobs(dtype, jobs, first=0):
    arr = (_ActiveJob * max(len(jobs), 1))()
    for j, (relay, idx, inputs, out) in enumerate(jobs):
        p, k = _ptrs(inputs, f"job {first + j} in", dtype, relay.count)
        arr[j].relay, arr[j].activeIdx, arr[j].nIn = relay._c(), idx, k
        for i in range(min(k, 4)):
            arr[j].inp[i] = p[i]
        arr[j].out = _dev(out, f"job {first + j} out", dtype, relay.count)
    return arr


def rr_helper_reduce_many(coll, dtype, op, jobs, stream=None, prepare=False):
    """jobs: [(relay, helper, slots, out), ...]"""
    arr = _helper_jobs(coll, dtype, jobs)
    return _issue(load().rr_helper_reduce_many, (coll, dtype, op, arr, len(jobs), _stream(stream)),
                  (arr, jobs), prepare)


def rr_active_add_scale_many(coll, dtype, op, jobs, stream=None, prepare=False):
    """jobs: [(relay, active_idx, inputs, out), ...]"""
    arr = _active_jobs(dtype, jobs)
    return _issue(load().rr_active_add_scale_many, (coll, dtype, op, arr, len(jobs), _stream(stream)),
                  (arr, jobs), prepare)


def rr_phase_reduce_many(coll, dtype, op, helper_jobs, active_jobs, stream=None, prepare=False):
    """The helper and active reductions of one phase in one call:
    helper_jobs as rr_helper_reduce_many's jobs, active_jobs as
    rr_active_add_scale_many's (numbered after the helper jobs in messages)."""
    h = _helper_jobs(coll, dtype, helper_jobs)
    a = _active_jobs(dtype, active_jobs, first=len(helper_jobs))
    return _issue(load().rr_phase_reduce_many,
                  (coll, dtype, op, h, len(helper_jobs), a, len(active_jobs), _stream(stream)),
                  (h, a, helper_jobs, active_jobs), prepare)


def rr_rs_multi_reduce_many(dtype, op, jobs, stream=None, prepare=False):
    """jobs: [(relay, pass_, idx, inputs, out), ...]"""
    arr = (_RsJob * max(len(jobs), 1))()
    keep = [arr, jobs]
    for j, (relay, pass_, idx, inputs, out) in enumerate(jobs):
        inputs = list(inputs)
        need, out_need = _rs_need(relay, dtype, pass_, len(inputs))
        p, k = _ptrs(inputs, f"job {j} in", dtype, need)
        keep.append(p)
        arr[j].relay, arr[j].pass_, arr[j].idx, arr[j].nIn = relay._c(), pass_, idx, k
        arr[j].inp = ctypes.cast(p, ctypes.POINTER(ctypes.c_void_p))
        arr[j].out = _dev(out, f"job {j} out", dtype, out_need)
    return _issue(load().rr_rs_multi_reduce_many, (dtype, op, arr, len(jobs), _stream(stream)),
                  keep, prepare)


def _a2a_many(fn, dtype, jobs, unpack, stream, prepare):
    arr = (_A2AJob * max(len(jobs), 1))()
    keep = [arr, jobs]
    for j, (relay, helper, ins, outs) in enumerate(jobs):
        a, b = _a2a_arrays(relay, dtype, list(ins), list(outs), unpack)
        keep += [a, b]
        arr[j].relay, arr[j].helper = relay._c(), helper
        arr[j].inp = ctypes.cast(a, ctypes.POINTER(ctypes.c_void_p))
        arr[j].out = ctypes.cast(b, ctypes.POINTER(ctypes.c_void_p))
    return _issue(fn, (dtype, arr, len(jobs), _stream(stream)), keep, prepare)


def rr_a2a_pack_many(dtype, jobs, stream=None, prepare=False):
    """jobs: [(relay, helper, src, dst), ...]"""
    return _a2a_many(load().rr_a2a_pack_many, dtype, jobs, False, stream, prepare)


def rr_a2a_unpack_many(dtype, jobs, stream=None, prepare=False):
    """jobs: [(relay, helper, recv, out), ...]"""
    return _a2a_many(load().rr_a2a_unpack_many, dtype, jobs, True, stream, prepare)
