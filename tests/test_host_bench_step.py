"""The benchmark step's launches at full size, replayed on the CPU.

bench.build_rows builds the rows on meta tensors (shapes and dtypes, no
memory), and the binding is pointed at the host replay library: the
product's C-ABI layer linked with a lane-by-lane replay of the kernels' index
arithmetic (tests/hostsim).  Every tensor storage gets a made-up device
address range, 2 MiB aligned with a 2 MiB gap after it, registered with the
replay; in check-only mode the replay checks every access of every launch
against those ranges without performing it.  So the launch configuration
bench.py times at 64 MiB, 256 MiB and 1 GiB per rank, one GPU's share and the
whole group, and one GPU's share at 64 MiB with the ragged all-to-all of
--ragged-a2a, is shown on the CPU to stay inside its buffers (and every body
vector to be stored exactly once), with the launch count, launch forms, copy
tiling and copy store policy that the kernel traces of those runs record.
"""
import ctypes

import pytest
import torch

import bench
import pack_rr_helper_amd as rr
from tests.hostsim import LIB, Sim

MIB = 1 << 20
GAP = 2 * MIB


class FakeHBM:
    """Made-up device addresses for meta tensors, one range per storage."""

    def __init__(self, sim):
        self.sim = sim
        self.next = 0x7E00_0000_0000
        self.ranges = {}

    def addr(self, t):
        st = t.untyped_storage()
        key = st._cdata
        if key not in self.ranges:
            nbytes = st.nbytes()
            self.ranges[key] = (self.next, st)   # the storage stays alive with its address
            self.sim.L.sim_register(ctypes.c_void_p(self.next), nbytes, 1)
            self.next += -(-nbytes // GAP) * GAP + GAP
        return self.ranges[key][0] + t.storage_offset() * t.element_size()

    def dev(self, t, what, dtype, min_elems, bits=False):
        """The binding's tensor checks, with a made-up address for the pointer."""
        assert t.device.type == "meta", what
        ok = rr._BITS_DT[rr._esize(dtype)] if bits else rr._TORCH_DT[dtype]
        assert t.dtype in ok and t.is_contiguous() and t.numel() >= min_elems, what
        return self.addr(t)


@pytest.fixture
def fake_gpu(monkeypatch):
    sim = Sim()
    sim.reset()
    sim.L.sim_set_check_only(1)
    hbm = FakeHBM(sim)
    monkeypatch.setattr(rr, "library_path", LIB)
    monkeypatch.setattr(rr, "_lib", None)
    monkeypatch.setattr(rr, "_dev", hbm.dev)
    monkeypatch.setattr(rr, "_stream", lambda stream: ctypes.c_void_p(0))
    try:
        yield sim
    finally:
        sim.L.sim_set_check_only(0)
        sim.reset()


def meta_inputs(M):
    n = M // 2
    val = lambda: torch.empty(n, dtype=torch.bfloat16, device="meta")
    bits = lambda: torch.empty(n, dtype=torch.int16, device="meta")
    return {"ar2": [val() for _ in range(2)], "rs2": [val() for _ in range(2)],
            "ar4": [val() for _ in range(4)], "rs4": [val() for _ in range(4)],
            "a2a": [bits() for _ in range(4)]}


def ragged(inp):
    """The all-to-all rows with segmentCount = 5 (mod 8), as bench.py --ragged-a2a
    builds them: chunk moves whose source and destination disagree modulo 16 bytes."""
    n = inp["a2a"][0].numel()
    inp["a2a"] = [torch.empty(4 * (n // 4 - 3), dtype=torch.int16, device="meta") for _ in range(4)]
    return inp


def counters(sim):
    L = sim.L
    return {"launches": L.sim_launches(),
            "red": [L.sim_form_launches(0, f) for f in range(3)],
            "copy": [L.sim_form_launches(1, f) for f in range(3)],
            "long": L.sim_copy_launches(1), "nt": L.sim_nt_copy_launches(1),
            "shifted": L.sim_shifted_copy_launches()}


@pytest.mark.parametrize("mib,ragged_a2a,variant", [
    (64, False, "share"), (64, False, "group"), (256, False, "share"), (256, False, "group"),
    (1024, False, "share"), (1024, False, "group"), (64, True, "share")],
    ids=["64MiB-share", "64MiB-group", "256MiB-share", "256MiB-group", "1GiB-share", "1GiB-group",
         "64MiB-ragged-share"])
def test_benchmark_step_launches_stay_inside_their_buffers(fake_gpu, mib, ragged_a2a, variant):
    sim = fake_gpu
    inp = meta_inputs(mib * MIB)
    wls = bench.build_rows(ragged(inp) if ragged_a2a else inp, mode=variant, dtype="bf16")
    calls = [c for w in wls.values() for c in w.calls()]
    assert [c[0] for c in calls] == ["ar2_helper", "ar2_active", "rs2_owner", "ar4_phase", "rs4_pass1",
                                     "rs4_pass2", "a2a_pack", "a2a_unpack"]
    sim.check()   # the untimed staging launches made while the rows were built
    before = counters(sim)
    for w in wls.values():
        w.run()
    sim.check()
    after = counters(sim)
    d = {k: ([a - b for a, b in zip(after[k], before[k])] if isinstance(after[k], list) else after[k] - before[k])
         for k in after}
    assert d["launches"] == 8
    # reductions: single-segment form for the one-job owner and active epilogues
    # of one GPU's share, the uniform grid for everything else, never the table
    share = variant == "share"
    assert d["red"] == ([0, 4, 2] if share else [0, 6, 0])
    assert d["copy"] == [0, 2, 0]
    moved = [b // 2 for row, _, b, _ in calls if row.startswith("a2a")]
    long_call = moved[0] >= bench.COPY_LONG_BYTES
    nt = long_call or moved[0] >= bench.COPY_AGENT_MAX_BYTES
    assert d["long"] == (2 if long_call else 0)
    assert d["nt"] == (2 if nt else 0)
    assert d["shifted"] == (2 if ragged_a2a else 0)   # ragged: both copies in the realigning kernels
