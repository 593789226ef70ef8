"""Pins of the oracle's geometry: the helper-size constants the pull request's
tests assert by hand, the zero-chunk direct fallback, the relay floor, and the
helper-buffer contracts (PR summary sections 1, 4, 6 and the commit stack)."""
import json
import os

import pytest

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "printed_values.json")))
AR, RS, A2A = 0, 1, 2
F32, BF16 = 0, 1


def test_passthrough_helper_size_printed_constants(orc):
    g = GOLD["passthrough_helper_size"]
    for c in g["cases"]:
        assert orc.passthrough_helper_size(c["count_g"], c["A"], c["num_chunks"]) == c["expected"]
    # per-rank total: a rank is a helper for the three other 2-active groups
    size = orc.passthrough_helper_size(12002982488, 2, 7)
    assert 3 * size == g["per_rank_total_three_helper_groups"]


def test_passthrough_helper_size_alignment_boundary(orc):
    # Reading: "the exact alignment boundary" is count_g = num_chunks * 128 * 1000
    # for A = 2, num_chunks = 7, the smallest count_g whose chunk is 1000 whole
    # 128-element chunks; one element less drops a whole 128-element chunk.
    assert orc.passthrough_helper_size(7 * 128 * 1000, 2, 7) == GOLD["passthrough_helper_size"][
        "alignment_boundary_expected"]
    assert orc.passthrough_helper_size(7 * 128 * 1000 - 1, 2, 7) == 2 * 128 * 999


@pytest.mark.parametrize("count_g,A,nc", [(10**9 + 7, 2, 7), (123456789, 4, 5), (4096, 2, 8)])
def test_passthrough_slots_are_whole_128_chunks(orc, count_g, A, nc):
    size = orc.passthrough_helper_size(count_g, A, nc)
    assert size < count_g
    assert size % A == 0 and (size // A) % 128 == 0
    assert (size // A) <= count_g / nc < (size // A) + 128


def test_passthrough_min_clamp_and_tiny_fallback(orc):
    # min() binds only when A >= num_chunks
    assert orc.passthrough_helper_size(1000, 8, 2) == 1000
    # below one aligned chunk the size is zero (direct fallback reads no helper buffer)
    assert orc.passthrough_helper_size(7 * 128 - 1, 2, 7) == 0


def test_relay_floor_1792_elements_before_the_pr(orc):
    f = GOLD["relay_element_floor"]
    A, H, nc = f["A"], f["H"], f["num_chunks"]
    assert f["elements"] == A * nc * 128
    # The pre-PR schedule (numChunks = H+1) is not a valid A=2 schedule any more,
    # so the floor is read off the chunk formula it used: input elements = A * recvCount.
    for elements in range(f["elements"] - 4, f["elements"] + 5, 2):
        recv = elements // A
        chunk = (recv // nc) // 128 * 128
        assert (chunk > 0) == (elements >= f["elements"])
    # and with the pull request's numChunks = H+2 the oracle's floor moves to 2*8*128
    g0 = orc.geometry(2, H, H + 2, 0, 8 * 128 - 1, RS, BF16)
    g1 = orc.geometry(2, H, H + 2, 0, 8 * 128, RS, BF16)
    assert g0["chunk"] == 0 and g1["chunk"] == 128


@pytest.mark.parametrize("coll", [AR, RS, A2A])
@pytest.mark.parametrize("count", [0, 1, 7, 1023, 8 * 128 - 1])
def test_zero_chunk_direct_fallback(orc, coll, count):
    g = orc.geometry(2, 6, 8, 0, count, coll, BF16)
    assert g["chunk"] == 0 and g["pure_direct"] == 1 and g["relay_total"] == 0
    assert g["dirA_off"] == 0 and g["dirA_len"] == count // 2
    assert g["dirB_off"] == count // 2 and g["dirB_len"] == count - count // 2
    assert g["helper_elems"] == 0


def test_a2_two_group_geometry(orc):
    count = 2 ** 20 + 777
    g = orc.geometry(2, 6, 8, 0, count, AR, F32)
    c = g["chunk"]
    assert c % 128 == 0 and c <= count / 8 < c + 128
    assert g["relay_total"] == 6 * c
    assert (g["dirA_off"], g["dirA_len"]) == (6 * c, c)
    assert g["dirB_off"] == 7 * c and g["dirA_len"] + g["dirB_len"] == count - 6 * c
    assert g["helper_elems"] == 2 * c


def test_a2_rejects_three_group_chunking(orc):
    assert orc.geometry(2, 6, 7, 0, 2 ** 20, AR, BF16) is None
    assert orc.geometry(3, 5, 8, 0, 2 ** 20, AR, BF16) is None
    assert orc.geometry(2, 0, 8, 0, 2 ** 20, AR, BF16) is None


def test_a4_allreduce_two_mib_floor(orc):
    below = orc.geometry(4, 4, 0, 500, 2 ** 20 - 1, AR, BF16)   # 2 MiB - 2 bytes
    at = orc.geometry(4, 4, 0, 500, 2 ** 20, AR, BF16)          # exactly 2 MiB
    assert below["pure_direct"] == 1 and below["dslice"] == (2 ** 20 - 1) // 4
    assert at["pure_direct"] == 0 and at["chunk"] == 2 ** 20 // 8
    f = orc.geometry(4, 4, 0, 500, 2 ** 19 - 1, AR, F32)        # fp32: 4-byte elements
    assert f["pure_direct"] == 1


def test_a4_allreduce_balanced_split_and_scratch_cover(orc):
    g = orc.geometry(4, 4, 0, 500, 2 ** 27, AR, BF16)
    assert g["chunk"] == 2 ** 24 and g["relay_total"] == 2 ** 26
    assert g["direct_len"] == 2 ** 26 and g["dslice"] == 2 ** 24
    # a 2*total_g helper buffer holds the (A+1) offload chunks at every permille
    for count in (2 ** 20, 3 * 2 ** 20 + 5, 2 ** 27):
        for p in (1, 250, 500, 780, 999, 1000):
            gg = orc.geometry(4, 4, 0, p, count, AR, BF16)
            assert 5 * gg["chunk"] <= gg["helper_elems"] == 2 * count


def test_a4_reduce_scatter_helper_contract(orc):
    c = GOLD["rs4_helper_contract"]
    A, H = c["A"], c["H"]
    R = 2 ** 22
    g = orc.geometry(A, H, 0, 500, R, RS, BF16)
    assert g["chunk"] == R // 8
    assert A * (A - 1) == c["input_chunks"]
    assert A * (A - 1) * g["chunk"] * 2 == 3 * R              # 1.5 x recvCount
    assert g["helper_elems"] == c["buffer_ratio"] * R
    assert (A * (A - 1) + A) * g["chunk"] <= g["helper_elems"]  # reduced chunks fit too
    # an offload fraction whose chunks would overflow the contract is rejected
    assert orc.geometry(A, H, 0, 501, R, RS, BF16) is None


def test_a4_all_to_all_chunk(orc):
    g = orc.geometry(4, 4, 5, 0, 2 ** 27, A2A, BF16)
    assert g["chunk"] == 26843520
    assert g["helper_elems"] == 12 * 26843520
    assert g["direct_off"] == 4 * 26843520
