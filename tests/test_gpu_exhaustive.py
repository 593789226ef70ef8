"""Every ordered pair of bf16 bit patterns through the two-input reduction
(the A=2 allreduce helper: scale * (slot0 + slot1), fp32 sum, one
round-to-nearest-even), against the CPU oracle.  Both sides add the same two
exact binary32 widenings in the same order and round once, so every result
that is not a NaN must match bit for bit (zeros, subnormals, infinities and
both roundings of every tie included); where the oracle gives a NaN the GPU
must too (NaN payloads are not compared: the binary32 add does not fix which
operand's payload survives).

Each op runs all 2^32 pairs, in 16 launches of 2^28 (the pairs whose first
pattern is congruent to the slice index modulo 16), the oracle on the host's
cores beside it: about 7 s per op on an MI355X host.  Once on 16-byte aligned
buffers (the direct kernels) and once on views at element offsets 1, 2 and 3
(the realigning kernels; the first few elements go through the element-wise
edge code)."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import pack_rr_helper_amd as rr
from pack_rr_helper_amd import synth

pytestmark = pytest.mark.gpu
AR, BF16, SUM, AVG = 0, 1, 0, 1
PARTS = 16
N = (1 << 32) // PARTS


def oracle_threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_slice(orc, op, a, b):
    T = oracle_threads()
    bounds = np.linspace(0, a.size, T + 1).astype(np.int64)
    with ThreadPoolExecutor(T) as ex:  # the oracle's C routine runs outside the interpreter lock
        parts = list(ex.map(lambda t: orc.ar2_helper(BF16, op, a[bounds[t]:bounds[t + 1]],
                                                     b[bounds[t]:bounds[t + 1]]), range(T)))
    return np.concatenate(parts)


def is_nan(x):
    return ((x & 0x7F80) == 0x7F80) & ((x & 0x7F) != 0)


def placed(x, lead):
    """x on the device, starting `lead` elements into a larger buffer."""
    big = torch.empty(N + 8, dtype=torch.bfloat16, device="cuda")
    big[lead:lead + N].copy_(synth.to_device(x, BF16))
    return big[lead:lead + N]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("op", [SUM, AVG])
@pytest.mark.parametrize("leads", [(0, 0, 0), (1, 2, 3)])
def test_every_bf16_pair(orc, op, leads):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    relay = rr.Relay(2, 6, 8, 0, 8 * N)  # chunk = count / 8 = N
    assert rr.rr_geometry(relay, AR, BF16)["chunk"] == N
    out_buf = torch.empty(N + 8, dtype=torch.bfloat16, device="cuda")
    out = out_buf[leads[2]:leads[2] + N]
    checked = 0
    for part in range(PARTS):
        print(f"[gpu-case] bf16 pairs op={op} leads={leads} slice {part}/{PARTS}", flush=True)
        a, b = synth.pattern_pairs(part, PARTS)
        da, db = placed(a, leads[0]), placed(b, leads[1])
        rr.rr_helper_reduce(relay, AR, BF16, op, 0, [da, db], out)
        ref = oracle_slice(orc, op, a, b)
        got = synth.to_host(out)
        del da, db
        diff = np.flatnonzero(got != ref)
        if diff.size:
            nan_ref = is_nan(ref[diff])
            assert np.array_equal(nan_ref, is_nan(got[diff])), (
                f"slice {part}: {int(np.sum(nan_ref != is_nan(got[diff])))} NaN results differ")
            wrong = diff[~nan_ref]
            assert wrong.size == 0, (
                f"slice {part}: {wrong.size} results differ, first a={a[wrong[0]]:#06x} "
                f"b={b[wrong[0]]:#06x} got={got[wrong[0]]:#06x} oracle={ref[wrong[0]]:#06x}")
        checked += a.size
    print(f"[gpu-case] bf16 pairs op={op} leads={leads}: {checked} pairs bit-exact (NaN by position)",
          flush=True)
