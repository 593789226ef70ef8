"""Pins of the oracle's all-to-all gather/scatter (the reverted all-to-all
paragraph of the PR summary): the composed group is the plain all-to-all
transpose, unpack inverts pack, every (destination, source, slice) chunk moves
exactly once, and nothing outside the helper slices is written."""
import numpy as np
import pytest

from pack_rr_helper_amd import synth

A2A, BF16, F32 = 2, 1, 0


@pytest.mark.parametrize("A,H,nc,seg", [(4, 4, 5, 5 * 128 * 3 + 41), (4, 4, 5, 600),
                                        (2, 6, 8, 8 * 128 * 2 + 3), (4, 4, 5, 5 * 128)])
def test_group_is_the_plain_all_to_all(orc, A, H, nc, seg):
    src = [synth.bits16(A * seg, 4, r) for r in range(A)]
    out = orc.a2a_group(2, A, H, nc, seg, src)
    for d in range(A):
        assert np.array_equal(out[d], orc.plain_all_to_all(2, A, seg, d, src))


def test_pack_moves_every_chunk_once_and_unpack_inverts_it(orc):
    A, H, nc, seg, es = 4, 4, 5, 5 * 128 * 2 + 7, 4
    c = orc.geometry(A, H, nc, 0, seg, A2A, F32)["chunk"]
    assert c == 256
    # element id = (source, destination segment, position): every value distinct
    src = [((s * A + np.arange(A * seg) // seg) * seg + np.arange(A * seg) % seg).astype(np.uint32)
           for s in range(A)]
    seen = set()
    out = [np.full(A * seg, 0xFFFFFFFF, np.uint32) for _ in range(A)]
    for h in range(H):
        dst = orc.a2a_pack(es, A, seg, c, h, src)
        for d in range(A):
            ids = dst[d].view(np.uint32)
            assert ids.size == (A - 1) * c
            srcs = ids // (A * seg)
            assert np.array_equal(np.unique(srcs), np.array([s for s in range(A) if s != d]))
            assert np.all((ids // seg) % A == d)                      # all destined for d
            pos = ids % seg
            for j, s in enumerate(s for s in range(A) if s != d):     # ascending sources
                assert np.array_equal(pos[j * c:(j + 1) * c], np.arange(h * c, (h + 1) * c))
                assert np.all(srcs[j * c:(j + 1) * c] == s)
            seen.update(ids.tolist())
        orc.a2a_unpack(es, A, seg, c, h, dst, out)
    assert len(seen) == A * (A - 1) * H * c                           # a bijection
    for d in range(A):
        for s in range(A):
            seg_out = out[d][s * seg:(s + 1) * seg]
            if s == d:
                assert np.all(seg_out == 0xFFFFFFFF)                  # own segment untouched
                continue
            relay = slice(0, H * c)
            assert np.array_equal(seg_out[relay], src[s][d * seg:(d + 1) * seg][relay])
            assert np.all(seg_out[H * c:] == 0xFFFFFFFF)              # direct region untouched


def test_pack_preserves_nan_payloads(orc):
    A, H, nc, seg = 4, 4, 5, 5 * 128
    src = [np.full(A * seg, 0x7F81 + s, np.uint16) for s in range(A)]   # signalling NaNs
    src[2][:] = 0xFFC3                                                  # negative quiet NaN
    dst = orc.a2a_pack(2, A, seg, 128, 1, src)
    for d in range(A):
        v = dst[d].view(np.uint16)
        expect = np.concatenate([src[s][:128] for s in range(A) if s != d])
        assert np.array_equal(v, expect)
