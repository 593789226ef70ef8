"""Pins of the oracle's bf16 codec against library routines and the exact
rational rounding of oracle/brute.py (IEEE 754 round-to-nearest-even)."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import brute


def _torch_bf16_bits(x):
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_to_f32_all_patterns(orc):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = orc.bf16_to_f32(bits).view(np.uint32)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy().view(np.uint32)
    assert np.array_equal(ours, ref)


def test_bf16_roundtrip_of_representable_values(orc):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = orc.bf16_to_f32(bits)
    back = orc.f32_to_bf16(f)
    finite = ~np.isnan(f)
    assert np.array_equal(back[finite], bits[finite])


def test_f32_to_bf16_matches_torch_rne_on_random_patterns(orc):
    rng = np.random.default_rng(1234)
    u = rng.integers(0, 1 << 32, size=1 << 21, dtype=np.uint64).astype(np.uint32)
    # exact ties (low half 0x8000) with odd and even kept halves, and their neighbours
    hi = rng.integers(0, 1 << 16, size=4096, dtype=np.uint32)
    ties = np.concatenate([(hi << 16) | 0x8000, (hi << 16) | 0x7FFF, (hi << 16) | 0x8001])
    u = np.concatenate([u, ties.astype(np.uint32)])
    x = u.view(np.float32)
    ours = orc.f32_to_bf16(x)
    ref = _torch_bf16_bits(x)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    # NaN stays NaN (payload unspecified by the contract), sign kept, quiet bit set
    on = ours[nan]
    assert np.all((on & 0x7F80) == 0x7F80) and np.all(on & 0x007F)
    assert np.all((on >> 15) == (u[nan] >> 31))
    assert np.all(on & 0x0040)


def test_f32_to_bf16_ties_and_overflow_against_exact_rounding(orc):
    cases = [0x3F808000, 0x3F818000, 0x3F80_7FFF, 0x7F7F_FFFF, 0x7F7F_8000, 0x7F7F_7FFF,
             0x0000_8000, 0x0001_8000, 0x0000_0001, 0x8080_8000, 0xC2F7_8000, 0x0080_0000]
    for c in cases:
        x = np.array([c], np.uint32).view(np.float32)
        ours = int(orc.f32_to_bf16(x)[0])
        exact = brute.decode(c, 32)
        r = brute.round_nearest_even(exact, brute.BFLOAT16)
        assert ours == brute.encode(r, 16), hex(c)


@pytest.mark.parametrize("bits", [0x0001, 0x007F, 0x0080, 0x3F80, 0xBF80, 0x7F7F, 0x8001, 0x4049])
def test_brute_decode_agrees_with_torch(bits):
    f = np.array([bits], np.uint16).view(np.int16)
    ref = torch.from_numpy(f).view(torch.bfloat16).double().item()
    assert brute.decode(bits, 16) == Fraction(ref)
