"""Pins for the test-side decoder of the library's MMQ layout (CPU only).

The decoder checks every GPU-packed group buffer against the oracle's verbatim copy, so it is
pinned here against hand-derived positions from the layout's statement in
include/moe_prefill.h, and against being a bijection (no byte or nibble lost or doubled)."""
import numpy as np
import pytest

import mmq_layout as ml


@pytest.mark.parametrize("wtype", [ml.Q8_0, ml.Q4_1])
@pytest.mark.parametrize("H,F", [(128, 128), (256, 128), (384, 256)])
def test_decoder_is_a_bijection(wtype, H, F):
    """Random packed bytes decode to a buffer of the same size holding the same bytes (Q8_0) or
    the same nibbles (Q4_1, whose nibbles move between bytes), and distinct inputs stay
    distinct."""
    rng = np.random.default_rng(H + F + wtype)
    eb = ml.expert_bytes(H, F, wtype)
    packed = rng.integers(0, 256, eb, dtype=np.uint8)
    raw = ml.decode_expert(packed, wtype, H, F)
    assert raw.size == eb
    if wtype == ml.Q8_0:
        assert np.array_equal(np.sort(raw), np.sort(packed))
    else:
        nib = lambda a: np.sort(np.concatenate([a & 15, a >> 4]))
        assert np.array_equal(nib(raw), nib(packed))
    # a one-nibble change in the packed buffer changes exactly one nibble of the raw one
    p2 = packed.copy()
    k = int(rng.integers(eb))
    p2[k] ^= 0x01
    diff = ml.decode_expert(p2, wtype, H, F) ^ raw
    assert np.count_nonzero(diff) == 1 and int(diff.max()) in (0x01, 0x10)


def test_q8_0_hand_positions():
    """Q8_0, H = 256 (8 blocks a row), F = 128: gate row 70 (tile 1, row 6), block 5 (stage 1,
    block 1 of the stage).  Its 136-byte group sits at ((1*2 + 1)*64 + 6)*136 = 26928: d at
    +2*1, q at +8 + 32*1.  Decoded, raw block 70*8 + 5 = 565 starts at 565*34 = 19210."""
    H, F = 256, 128
    packed = np.zeros(ml.expert_bytes(H, F, ml.Q8_0), np.uint8)
    packed[26930:26932] = [0x34, 0x12]
    packed[26968:27000] = np.arange(1, 33, dtype=np.uint8)
    raw = ml.decode_expert(packed, ml.Q8_0, H, F)
    assert list(raw[19210:19212]) == [0x34, 0x12]
    assert np.array_equal(raw[19212:19244], np.arange(1, 33, dtype=np.uint8))
    assert np.count_nonzero(raw) == 34
    # the up matrix starts F*(H/32)*34 = 34816 bytes in, raw and packed alike: its row 0,
    # block 0 is the first group of its region
    packed[:] = 0
    packed[34816] = 0x77
    raw = ml.decode_expert(packed, ml.Q8_0, H, F)
    assert raw[34816] == 0x77 and np.count_nonzero(raw) == 1
    # the down matrix (H rows of F/32 = 4 blocks): row 129 = tile 2, row 1, stage 0 ->
    # group at 2*34816 + ((2*1 + 0)*64 + 1)*136; block 3's q[0] at +8 + 96; raw block
    # 129*4 + 3 = 519 of the down region, q[0] at 2*34816 + 519*34 + 2
    packed[:] = 0
    packed[2 * 34816 + 129 * 136 + 104] = 0x99
    raw = ml.decode_expert(packed, ml.Q8_0, H, F)
    assert raw[2 * 34816 + 519 * 34 + 2] == 0x99 and np.count_nonzero(raw) == 1


def test_q4_1_hand_positions():
    """Q4_1, the same row 70 and block 5: the 80-byte group at 198*80 = 15840, block 1's (d, m)
    at +4, its packed bytes at +16 + 16.  Packed byte 8*1 + 3 (half 1, i = 3) = 0xA5 holds
    element 16 + 3 = 19 (low nibble 5) and element 16 + 8 + 3 = 27 (high nibble 10).  In the raw
    block (565 * 20 = 11300; qs at +4, qs[j] = element j | element j+16 << 4) element 19 is
    qs[3]'s high nibble and element 27 is qs[11]'s."""
    H, F = 256, 128
    packed = np.zeros(ml.expert_bytes(H, F, ml.Q4_1), np.uint8)
    packed[15844:15848] = [1, 2, 3, 4]
    packed[15840 + 32 + 8 + 3] = 0xA5
    raw = ml.decode_expert(packed, ml.Q4_1, H, F)
    assert list(raw[11300:11304]) == [1, 2, 3, 4]
    assert raw[11304 + 3] == 0x50 and raw[11304 + 11] == 0xA0
    assert np.count_nonzero(raw) == 6
    # half 0, i = 0: elements 0 (low) and 8 (high) -> qs[0] low nibble, qs[8] low nibble
    packed[:] = 0
    packed[15840 + 32] = 0x3C
    raw = ml.decode_expert(packed, ml.Q4_1, H, F)
    assert raw[11304 + 0] == 0x0C and raw[11304 + 8] == 0x03 and np.count_nonzero(raw) == 2


def test_check_positions_flags_a_misplaced_expert():
    """The group-buffer check accepts the right encoding and fails on a wrong position and on a
    stray byte outside the positions.  (Q8_0 moves whole bytes, so decoding the byte indices
    0..eb-1 gives the permutation that encodes a raw expert.)"""
    rng = np.random.default_rng(3)
    H, F, wt = 128, 128, ml.Q8_0
    eb = ml.expert_bytes(H, F, wt)
    stride = (eb + 255) // 256 * 256
    perm = ml.decode_expert(np.arange(eb, dtype=np.int64), wt, H, F)   # raw[i] = packed[perm[i]]
    assert np.array_equal(np.sort(perm), np.arange(eb))
    raw = rng.integers(0, 256, eb, dtype=np.uint8)
    packed = np.empty(eb, np.uint8)
    packed[perm] = raw
    assert np.array_equal(ml.decode_expert(packed, wt, H, F), raw)
    buf = np.full(4 * stride, 0xEE, np.uint8)
    buf[stride:stride + eb] = packed
    ml.check_positions(buf, wt, H, F, [raw], 1, stride, fill=0xEE)
    with pytest.raises(AssertionError):
        ml.check_positions(buf, wt, H, F, [raw], 2, stride)
    buf[3 * stride + 5] = 0
    with pytest.raises(AssertionError):
        ml.check_positions(buf, wt, H, F, [raw], 1, stride, fill=0xEE)
