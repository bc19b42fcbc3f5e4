"""Pins of the oracle's bank packer/decoder (CPU only).

The pins come from outside the packer: a hand-derived worked example
(tests/golden/layout_worked_example.txt), the pages' tile geometry and
byte accounting, the 3-byte/4-byte identity the pages state, and
structural properties of the placement (a bijection with per-lane
contiguity).
"""

import os

import numpy as np
import pytest

from awq_int4_mixture_amd import inputs
from oracle import layout as OL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "layout_worked_example.txt")


def worked_example_weights():
    """The weight pattern stated in the golden file header (H=64, I=32)."""
    H, I = 64, 32
    k = np.arange(H)[:, None]
    i = np.arange(I)[None, :]
    q_gate = ((k + 2 * i) % 16).astype(np.uint8)
    q_up = np.broadcast_to((15 - (k % 16)), (H, I)).astype(np.uint8)
    ii = np.arange(I)[:, None]
    n = np.arange(H)[None, :]
    q_down = ((ii + n) % 16).astype(np.uint8)
    g = np.arange(H // 32)[:, None]
    s_gate = np.full((H // 32, I), 1.0, np.float16)
    s_up = np.full((H // 32, I), 0.5, np.float16)
    s_down = np.full((I // 32, H), 2.0, np.float16)
    z_gate = (16 * g + i).astype(np.uint8)
    z_up = (100 + i + g).astype(np.uint8)
    z_down = np.broadcast_to(n, (I // 32, H)).astype(np.uint8)
    return inputs.ExpertWeights(q_gate, q_up, q_down, s_gate, s_up, s_down, z_gate, z_up, z_down)


def golden_entries():
    out = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            parts = line.split()
            out.append((int(parts[0]), int(parts[1]), bytes(int(b, 16) for b in parts[2:])))
    return out


@pytest.mark.parametrize("rb", [3, 4])
def test_worked_example_bytes(rb):
    d = OL.Dims(1, 64, 32, rb)
    L = OL.layout(d)
    assert (L.w13_off, L.w13_meta_off, L.w2_off, L.w2_meta_off, L.expert_bytes) == (0, 2048, 2560, 3584, 3840)
    blk = OL.pack_expert(d, worked_example_weights())
    entries = [e for e in golden_entries() if e[0] == rb]
    assert len(entries) >= 6
    for _, off, want in entries:
        assert bytes(blk[off:off + len(want)]) == want, off


@pytest.mark.parametrize("rb", [3, 4])
@pytest.mark.parametrize("H,I,wide", [(64, 32, False), (256, 32, False), (96, 64, False), (96, 64, True)])
def test_round_trip(rb, H, I, wide):
    d = OL.Dims(3, H, I, rb)
    if wide:   # zeros 0..255, scales of both signs: +-0, subnormal, near 65504
        bi = inputs.bank_inputs(11, 3, H, I, draw=inputs.expert_weights_wide, big_w13_groups=(0,),
                                big_w2_groups=(1,))
    else:
        bi = inputs.bank_inputs(11, 3, H, I, zero_hi=256)
    bank = OL.pack_bank(d, bi)
    for e in range(3):
        w = bi.expert(e)
        dec = OL.decode_expert(d, bank, e)
        assert dec.pad_ok
        np.testing.assert_array_equal(dec.q13, OL.interleave_w13(w.q_gate, w.q_up))
        np.testing.assert_array_equal(dec.s13.view(np.uint16), OL.interleave_w13(w.s_gate, w.s_up).view(np.uint16))
        np.testing.assert_array_equal(dec.z13, OL.interleave_w13(w.z_gate, w.z_up))
        np.testing.assert_array_equal(dec.q2, w.q_down)
        np.testing.assert_array_equal(dec.s2.view(np.uint16), w.s_down.view(np.uint16))
        np.testing.assert_array_equal(dec.z2, w.z_down)


def test_three_and_four_byte_decode_identically():
    """PR #522 (Default switch): the two layouts decode to identical weights."""
    bi = inputs.bank_inputs(5, 2, 128, 64, zero_hi=256)
    b3 = OL.pack_bank(OL.Dims(2, 128, 64, 3), bi)
    b4 = OL.pack_bank(OL.Dims(2, 128, 64, 4), bi)
    for e in range(2):
        d3 = OL.decode_expert(OL.Dims(2, 128, 64, 3), b3, e)
        d4 = OL.decode_expert(OL.Dims(2, 128, 64, 4), b4, e)
        for f in ("q13", "z13", "q2", "z2"):
            np.testing.assert_array_equal(getattr(d3, f), getattr(d4, f))
        for f in ("s13", "s2"):
            np.testing.assert_array_equal(getattr(d3, f).view(np.uint16), getattr(d4, f).view(np.uint16))
        # weight sections are byte-identical; only the record sections differ
        L3 = OL.layout(OL.Dims(2, 128, 64, 3))
        L4 = OL.layout(OL.Dims(2, 128, 64, 4))
        blk3 = b3[e * L3.expert_bytes:(e + 1) * L3.expert_bytes]
        blk4 = b4[e * L4.expert_bytes:(e + 1) * L4.expert_bytes]
        np.testing.assert_array_equal(blk3[L3.w13_off:L3.w13_off + L3.w13_units],
                                      blk4[L4.w13_off:L4.w13_off + L4.w13_units])


def test_compact_record_is_low_24_bits_of_padded_record():
    bi = inputs.bank_inputs(6, 1, 64, 32, zero_hi=256)
    b3 = OL.pack_bank(OL.Dims(1, 64, 32, 3), bi)
    b4 = OL.pack_bank(OL.Dims(1, 64, 32, 4), bi)
    L3 = OL.layout(OL.Dims(1, 64, 32, 3))
    L4 = OL.layout(OL.Dims(1, 64, 32, 4))
    r3 = b3[L3.w13_meta_off:L3.w13_meta_off + L3.w13_meta].reshape(-1, 3)
    r4 = b4[L4.w13_meta_off:L4.w13_meta_off + L4.w13_meta].reshape(-1, 4)
    np.testing.assert_array_equal(r3, r4[:, :3])
    assert not r4[:, 3].any()


def test_tile_geometry_of_compact_records():
    """PR #522 (Purpose): a 96-byte tile = 24 aligned dwords = 32 records; the
    last record starts at byte 93 and ends inside the tile."""
    H, RB = 2560, 3
    starts = []
    for t in range(8):          # 8 lanes x 4 records
        for j in range(4):
            starts.append((4 * t + j) * RB)
    assert len(starts) == 32 and max(starts) == 93 and max(starts) + RB == 96 == 24 * 4
    # Each lane's four records form one 12-byte run that starts on a dword boundary.
    for g in range(H // 32):
        for quad in range(4):
            offs = [OL.w13_record_offset(H, RB, g, 4 * quad + j) for j in range(4)]
            assert offs == list(range(offs[0], offs[0] + 12, 3)) and offs[0] % 4 == 0


def test_byte_accounting_matches_pages():
    """PR #522 addendum (Layout-level capacity): 3-byte banks save 943,718,400 bytes
    per rank across 48 layers at E512 / hidden 2560 / local intermediate 160."""
    L3 = OL.layout(OL.Dims(512, 2560, 160, 3))
    L4 = OL.layout(OL.Dims(512, 2560, 160, 4))
    assert 48 * (L4.total_bytes - L3.total_bytes) == 943_718_400
    # no padding at this shape: every byte is a unit or a record
    for L in (L3, L4):
        assert L.expert_bytes == L.w13_units + L.w13_meta + L.w2_units + L.w2_meta


@pytest.mark.parametrize("H,I,rb", [(2560, 160, 3), (2560, 160, 4), (256, 32, 3), (8192, 2048, 3), (96, 64, 4)])
def test_placement_is_a_bijection_with_coalesced_lanes(H, I, rb):
    L = OL.layout(OL.Dims(1, H, I, rb))
    for (unit_off, rec_off, G, N) in (
        (lambda g, n: OL.w13_unit_offset(H, g, n), lambda g, n: OL.w13_record_offset(H, rb, g, n), H // 32, 2 * I),
        (lambda g, n: OL.w2_unit_offset(I, g, n), lambda g, n: OL.w2_record_offset(I, rb, g, n), I // 32, H),
    ):
        g = np.arange(G)[:, None]
        n = np.arange(N)[None, :]
        uo = np.broadcast_to(unit_off(g, n), (G, N)).ravel()
        ro = np.broadcast_to(rec_off(g, n), (G, N)).ravel()
        assert np.array_equal(np.sort(uo), np.arange(G * N) * 16)
        assert np.array_equal(np.sort(ro), np.arange(G * N) * rb)
        # within a tile, load j of lanes t = 0..4G-1 reads one contiguous range,
        # and the four records of lane t are one run starting on a dword boundary
        lanes = 4 * G
        for nt in (0, N // 16 - 1):
            for j in range(4):
                offs = [unit_off(t // 4, 16 * nt + 4 * (t % 4) + j) for t in range(lanes)]
                assert offs == list(range(offs[0], offs[0] + 16 * lanes, 16))
                assert offs[0] == nt * 256 * G + j * 16 * lanes
            for t in range(lanes):
                r = [rec_off(t // 4, 16 * nt + 4 * (t % 4) + j) for j in range(4)]
                assert r == list(range(r[0], r[0] + 4 * rb, rb)) and r[0] % 4 == 0
    assert L.total_bytes == L.expert_bytes
