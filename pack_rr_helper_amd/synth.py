"""Seeded synthetic inputs for the relay hot path.

This module holds the input recipe only -- no relay arithmetic -- and is the
one piece shared by the tests (which feed the same bytes to the CPU oracle and
to the GPU) and the benchmark.  Every rank r of a workload draws from its own
stream ``numpy.random.default_rng([seed, r])`` (PCG64):

* ``uniform(n, lo, hi)``: float32 ``rng.random`` scaled by (hi - lo) and
  shifted by lo; for the power-of-two widths used here (2 and 4) both steps are
  exact, so every value is a representable float32 in [lo, hi).
* ``normal(n)``: float32 ``rng.standard_normal``.
* ``bits16(n)``, ``bits32(n)``: uniform raw 16- and 32-bit patterns (NaN, Inf
  and subnormal encodings included).
* ``as_bf16_bits``: a float32 array rounded to bf16 with torch's CPU
  conversion (round-to-nearest-even), returned as raw uint16 bit patterns.
* ``pattern_pairs(part, parts)``: not random -- one of ``parts`` equal slices
  of the 2^32 ordered pairs of 16-bit patterns: the pairs whose first pattern
  is congruent to ``part`` modulo ``parts`` (so every slice spans every sign
  and exponent).
"""
import numpy as np
import torch


def rng(seed, rank):
    return np.random.default_rng([int(seed), int(rank)])


def uniform(n, lo, hi, seed, rank):
    r = rng(seed, rank).random(n, dtype=np.float32)
    return (r * np.float32(hi - lo) + np.float32(lo)).astype(np.float32)


def normal(n, seed, rank):
    return rng(seed, rank).standard_normal(n, dtype=np.float32)


def bits16(n, seed, rank):
    return rng(seed, rank).integers(0, 1 << 16, size=n, dtype=np.uint16)


def bits32(n, seed, rank):
    return rng(seed, rank).integers(0, 1 << 32, size=n, dtype=np.uint32)


def pattern_pairs(part, parts):
    """Slice `part` (0 <= part < parts, parts a power of two <= 65536) of the
    2^32 ordered pairs of 16-bit patterns: uint16 arrays (a, b) holding every
    pair whose first pattern a is congruent to part modulo parts, a ascending,
    then b from 0 to 65535."""
    a = np.repeat(np.arange(part, 1 << 16, parts, dtype=np.uint16), 1 << 16)
    b = np.tile(np.arange(1 << 16, dtype=np.uint16), (1 << 16) // parts)
    return a, b


def small_ints(n, lim, seed, rank):
    """Integers in [-lim, lim] as float32: every sum of a few of them is exact
    in bf16 and fp32, so any summation order gives the same bits."""
    return rng(seed, rank).integers(-lim, lim + 1, size=n).astype(np.float32)


def as_bf16_bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def to_device(a, dtype_code, device="cuda"):
    """Host array -> device tensor with the same bytes: float32 stays float32,
    uint16 bit patterns become a torch.bfloat16 tensor (dtype_code 1) or an
    int16 tensor holding raw bits (dtype_code None)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return torch.from_numpy(a).to(device)
    t = torch.from_numpy(a.view(np.int16)).to(device)
    return t.view(torch.bfloat16) if dtype_code == 1 else t


def to_host(t):
    """Device tensor -> host numpy array with the same bytes (bf16 and int16
    come back as uint16 bit patterns)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)
