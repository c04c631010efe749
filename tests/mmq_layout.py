"""Decoder of the HIP library's MMQ layout of an expert, for checking what its gathers write
(tests only).

The pages gather an expert's bytes unchanged ("the same bytes land in the same places"); the
library's gather instead writes each expert in the layout its matmul stages (declared in
include/moe_prefill.h, "MMQ layout of an expert").  That layout is the library's private
choice, so the oracle does not know it: a GPU-packed buffer is checked by decoding it back to
the raw expert here and comparing that, byte for byte, with the oracle's verbatim copy
(orc_gather).  The layout, as the header states it: every matrix (gate, up, down in that order,
same sizes as raw) of n_rows rows and nblk blocks per row is stored as tiles of 64 rows by 4
blocks; for tile j, stage t and row i < 64 (matrix row 64j+i) the row's blocks 4t..4t+3 take
G = 4 * block bytes at byte ((j * nblk/4 + t) * 64 + i) * G, headers first:
  Q4_1 (G = 80):  the 4 blocks' (d, m), then each block's 16 packed bytes in two halves, byte
                  8h + i holding element 16h + i in its low nibble and 16h + 8 + i in its high
  Q8_0 (G = 136): the 4 blocks' d, then their q[32]
A raw Q4_1 block is (d, m, qs[16]) with qs[j] = element j | element j+16 << 4; a raw Q8_0 block
is (d, q[32]).  The decoder moves bytes and nibbles only, so it is a bijection between equally
sized buffers: decode(packed) == raw holds exactly when packed is raw's encoding.
"""
from __future__ import annotations

import numpy as np

Q8_0, Q4_1, Q8_0_D4 = 0, 1, 2


def _bb(wtype: int) -> int:
    return 20 if wtype == Q4_1 else 34


def decode_matrix(packed, wtype: int, n_rows: int, nblk: int) -> np.ndarray:
    """One matrix in the MMQ layout -> its raw blocks, [n_rows * nblk, block bytes] uint8."""
    G = 4 * _bb(wtype)
    packed = np.asarray(packed)
    if wtype == Q4_1 or packed.dtype != np.int64:   # Q8_0 also decodes int64 byte indices
        packed = packed.astype(np.uint8, copy=False)
    g = packed.reshape(n_rows // 64, nblk // 4, 64, G)
    g = g.transpose(0, 2, 1, 3).reshape(n_rows * nblk // 4, G)      # row-major 4-block groups
    if wtype == Q4_1:
        hdr = g[:, 0:16].reshape(-1, 4, 4)                          # (group, block, d|m bytes)
        half = g[:, 16:80].reshape(-1, 4, 2, 8)                     # (group, block, h, i)
        elem = np.empty(half.shape[:2] + (32,), np.uint8)           # the block's 32 elements
        for h in range(2):
            elem[:, :, 16 * h:16 * h + 8] = half[:, :, h, :] & 15
            elem[:, :, 16 * h + 8:16 * h + 16] = half[:, :, h, :] >> 4
        qs = elem[:, :, 0:16] | (elem[:, :, 16:32] << 4)
        raw = np.concatenate([hdr, qs], axis=2)                     # (group, block, 20)
    else:
        d = g[:, 0:8].reshape(-1, 4, 2)
        q = g[:, 8:136].reshape(-1, 4, 32)
        raw = np.concatenate([d, q], axis=2)                        # (group, block, 34)
    return raw.reshape(n_rows * nblk, _bb(wtype))


def decode_expert(packed, wtype: int, H: int, F: int) -> np.ndarray:
    """One expert in the MMQ layout -> the raw expert's bytes (gate | up | down)."""
    packed = np.asarray(packed).reshape(-1)
    bb = _bb(wtype)
    gu = F * (H // 32) * bb
    dn = H * (F // 32) * bb
    assert packed.size == 2 * gu + dn, (packed.size, 2 * gu + dn)
    parts = [decode_matrix(packed[0:gu], wtype, F, H // 32),
             decode_matrix(packed[gu:2 * gu], wtype, F, H // 32),
             decode_matrix(packed[2 * gu:], wtype, H, F // 32)]
    return np.concatenate([p.reshape(-1) for p in parts])


def expert_bytes(H: int, F: int, wtype: int) -> int:
    return (2 * F * (H // 32) + H * (F // 32)) * _bb(wtype)


def check_positions(buf, wtype: int, H: int, F: int, raw_experts, first_pos: int,
                    pos_stride: int, fill=None) -> None:
    """Positions first_pos.. of a group buffer hold the raw experts `raw_experts` (a list of
    byte arrays) in the MMQ layout; with `fill`, every other byte of the buffer still holds it."""
    buf = np.asarray(buf, np.uint8).reshape(-1)
    eb = expert_bytes(H, F, wtype)
    touched = np.zeros(buf.size, bool)
    for j, raw in enumerate(raw_experts):
        p = (first_pos + j) * pos_stride
        got = decode_expert(buf[p:p + eb], wtype, H, F)
        assert np.array_equal(got, np.asarray(raw, np.uint8).reshape(-1)), (j, first_pos)
        touched[p:p + eb] = True
    if fill is not None:
        assert np.all(buf[~touched] == fill), "bytes outside the positions changed"
