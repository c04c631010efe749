"""Pins for the oracle's gather (a3) and block dots (a4/a6) (CPU only)."""
import numpy as np
import pytest

import npref
from quantized_expert_grouped_amd import synth


def test_gather_is_per_expert_copy(orc):
    """Byte for byte the per-expert copies, for batches of 1..16 starting at every position
    (the group-gather page's test: batches of 1-16, starts mid-group, odd sizes)."""
    rng = np.random.default_rng(2)
    E, eb = 20, 1000 + 7                          # odd expert size
    stride = 1024 + 16
    pool = rng.integers(0, 256, E * 1100, dtype=np.uint8)
    off = rng.permutation(E).astype(np.int64) * 1100 + 3   # misaligned slots
    for n in range(1, 17):
        for first in (0, 16 - n, (16 - n) // 2):
            experts = rng.choice(E, n, replace=False).astype(np.int32)
            buf = np.full(16 * stride, 0xAB, np.uint8)
            orc.gather(pool, off, experts, eb, buf, first, stride)
            want = np.full(16 * stride, 0xAB, np.uint8)
            for j, e in enumerate(experts):
                p = (first + j) * stride
                want[p:p + eb] = pool[off[e]:off[e] + eb]
            assert np.array_equal(buf, want), (n, first)


def _decode_mmq_matrix(packed, wtype, n_rows, nblk):
    """Blocks (d, m, q) in raw block order, read from one MMQ-layout matrix by the layout's
    description: tile j of 64 rows, stage t of 4 blocks, row i -> one 4-block group at
    ((j * nblk/4 + t) * 64 + i) * G; Q4_1 G = 80: 4 x (d, m) then 4 x 16 packed bytes, byte
    8h + i holding element 16h + i (low nibble) and 16h + 8 + i (high); Q8_0 G = 136: 4 x d
    then 4 x q[32]."""
    G = 136 if wtype == synth.Q8_0 else 80
    g = np.asarray(packed, np.uint8).reshape(n_rows // 64, nblk // 4, 64, G)
    g = g.transpose(0, 2, 1, 3).reshape(n_rows * nblk // 4, G)   # row-major groups
    if wtype == synth.Q8_0:
        d = g[:, 0:8].copy().view("<u2").reshape(-1)
        q = g[:, 8:136].reshape(-1, 32).view(np.int8).astype(np.int64)
        return d, None, q
    hdr = g[:, 0:16].copy().view("<u2").reshape(-1, 4, 2)
    qs = g[:, 16:80].reshape(-1, 2, 8).astype(np.int64)        # (block, half, byte)
    q = np.concatenate([qs & 15, qs >> 4], 2).reshape(-1, 32)   # half h: 16h..16h+7, 16h+8..
    return hdr[:, :, 0].reshape(-1), hdr[:, :, 1].reshape(-1), q


def _decode_mmq(packed, wtype, H, F):
    bb = 34 if wtype == synth.Q8_0 else 20
    gu = F * (H // 32) * bb
    parts = [_decode_mmq_matrix(packed[0:gu], wtype, F, H // 32),
             _decode_mmq_matrix(packed[gu:2 * gu], wtype, F, H // 32),
             _decode_mmq_matrix(packed[2 * gu:], wtype, H, F // 32)]
    d = np.concatenate([p[0] for p in parts])
    q = np.concatenate([p[2] for p in parts])
    m = None if wtype == synth.Q8_0 else np.concatenate([p[1] for p in parts])
    return d, m, q


def _decode_raw(raw, wtype):
    bb = 34 if wtype == synth.Q8_0 else 20
    b = np.asarray(raw, np.uint8).reshape(-1, bb)
    d = b[:, 0:2].copy().view("<u2").reshape(-1)
    if wtype == synth.Q8_0:
        return d, None, b[:, 2:34].view(np.int8).astype(np.int64)
    qs = b[:, 4:20].astype(np.int64)
    return d, b[:, 2:4].copy().view("<u2").reshape(-1), np.concatenate([qs & 15, qs >> 4], 1)


@pytest.mark.parametrize("wtype", [synth.Q8_0, synth.Q4_1])
@pytest.mark.parametrize("H,F", [(128, 128), (256, 128), (384, 256)])
def test_mmq_pack_keeps_every_block(orc, wtype, H, F):
    """The MMQ layout holds every block's scale, min and quantised values of the raw expert, and
    nothing else (it has the raw expert's size)."""
    rng = np.random.default_rng(60 + wtype + H + F)
    eb = orc.expert_bytes(H, F, wtype)
    nblocks = eb // (34 if wtype == synth.Q8_0 else 20)
    raw = synth.random_blocks(rng, nblocks, wtype).reshape(-1)
    packed = orc.mmq_pack(wtype, raw, H, F)
    assert packed.size == orc.mmq_expert_bytes(H, F, wtype) == eb
    d1, m1, q1 = _decode_mmq(packed, wtype, H, F)
    d0, m0, q0 = _decode_raw(raw, wtype)
    assert np.array_equal(d1, d0) and np.array_equal(q1, q0)
    if wtype == synth.Q4_1:
        assert np.array_equal(m1, m0)
    # the dequantised weights of all three matrices are unchanged
    gu = F * (H // 32)
    rows = np.concatenate([np.zeros(1, int), np.cumsum([gu, gu, H * (F // 32)])])
    for a, b, (n_rows, k_in) in zip(rows[:-1], rows[1:], [(F, H), (F, H), (H, F)]):
        bb = 34 if wtype == synth.Q8_0 else 20
        w0 = npref.dequant_matrix(raw[a * bb:b * bb], n_rows, k_in, wtype)
        dd = npref.f16_val(d1[a:b]).reshape(n_rows, k_in // 32)
        w1 = q1[a:b].reshape(n_rows, k_in // 32, 32) * dd[..., None]
        if m1 is not None:
            w1 = w1 + npref.f16_val(m1[a:b]).reshape(n_rows, k_in // 32)[..., None]
        assert np.array_equal(w0, w1.reshape(n_rows, k_in))


@pytest.mark.parametrize("wtype", [synth.Q8_0, synth.Q4_1])
def test_gather_mmq_positions(orc, wtype):
    """Each expert lands packed at its position; batches start mid-group; other bytes untouched."""
    rng = np.random.default_rng(70 + wtype)
    H, F, E = 256, 128, 6
    eb = orc.expert_bytes(H, F, wtype)
    pb = orc.mmq_expert_bytes(H, F, wtype)
    stride = (pb + 255) // 256 * 256
    pool = synth.random_blocks(rng, E * eb // (34 if wtype == synth.Q8_0 else 20), wtype).reshape(-1)
    off = rng.permutation(E).astype(np.int64) * eb
    for n, first in ((1, 0), (3, 5), (6, 10)):
        experts = rng.choice(E, n, replace=False).astype(np.int32)
        buf = np.full(16 * stride, 0xCD, np.uint8)
        orc.gather_mmq(pool, off, experts, wtype, H, F, buf, first, stride)
        want = np.full(16 * stride, 0xCD, np.uint8)
        for j, e in enumerate(experts):
            p = (first + j) * stride
            want[p:p + pb] = orc.mmq_pack(wtype, pool[off[e]:off[e] + eb], H, F)
        assert np.array_equal(buf, want), (n, first)


def _block(wtype, rng, nb):
    return synth.random_blocks(rng, nb, wtype)


@pytest.mark.parametrize("wtype", [synth.Q8_0, synth.Q4_1])
def test_block_idot_against_unpacked_integers(orc, wtype):
    rng = np.random.default_rng(4 + wtype)
    blocks = _block(wtype, rng, 500)
    xq = rng.integers(-127, 128, (500, 32)).astype(np.int8)
    xq[0] = 127
    xq[1] = -127
    q, _, _ = npref.unpack_matrix(blocks.reshape(-1), 500, 32, wtype)
    for i in range(500):
        assert orc.block_idot(wtype, blocks[i], xq[i]) == int(q[i] @ xq[i].astype(np.int64))
    # extreme: |I| <= 32 * 127 * 127
    if wtype == synth.Q8_0:
        b = synth.pack_q8_0(np.full((1, 32), -127, np.int8), np.array([1.0], np.float16))[0]
        assert orc.block_idot(wtype, b, np.full(32, 127, np.int8)) == -32 * 127 * 127


@pytest.mark.parametrize("wtype", [synth.Q8_0, synth.Q4_1, synth.Q8_0_D4])
def test_row_dot_against_dequantised_fp64(orc, wtype):
    """sum_b y_b equals the fp64 dot of the dequantised weight row and activation row:
    exactly (to fp64 summation) for Q8_0; for Q4_1 up to the term m_w * (s16 - d16*sum q_x),
    the rounding of the stored s, whose size the test computes."""
    rng = np.random.default_rng(40 + wtype)
    k_in = 512
    nb = k_in // 32
    x = rng.standard_normal((6, k_in)).astype(np.float32)
    x[2] = 0
    xq8 = orc.q8_1_rows(x, orc.act_layout(wtype))
    xh = npref.dequant_act(xq8, k_in, wtype)
    qx, dx, sx = npref.q8_1_decode(xq8, k_in)
    for _ in range(30):
        wrow = _block(wtype, rng, nb).reshape(-1)
        wdq = npref.dequant_matrix(wrow, 1, k_in, wtype)[0]
        _, _, m = npref.unpack_matrix(wrow, 1, k_in, wtype)
        for r in range(6):
            got = orc.row_dot(wtype, wrow, xq8[r], k_in)
            want = float(wdq @ xh[r])
            scale = float(np.abs(wdq * xh[r]).sum()) + 1e-300
            bound = 1e-13 * scale
            if wtype == synth.Q4_1:
                S = qx[r].reshape(nb, 32).sum(axis=1)
                bound += float(np.sum(np.abs(m[0]) * np.abs(sx[r] - dx[r] * S)))
            assert abs(got - want) <= bound, (r, got, want, bound)
        assert orc.row_dot(wtype, wrow, xq8[2], k_in) == 0.0


@pytest.mark.parametrize("wtype", [synth.Q8_0, synth.Q4_1])
def test_block_dots_matrix(orc, wtype):
    rng = np.random.default_rng(8)
    n_out, k_in, rows = 5, 256, 4
    wmat = _block(wtype, rng, n_out * k_in // 32).reshape(-1)
    x = rng.standard_normal((rows, k_in)).astype(np.float32)
    act = orc.q8_1_rows(x)
    got = orc.block_dots(wtype, wmat, n_out, k_in, act)
    q, _, _ = npref.unpack_matrix(wmat, n_out, k_in, wtype)
    qx, _, _ = npref.q8_1_decode(act, k_in)
    want = np.einsum("nbj,rbj->rnb", q.reshape(n_out, -1, 32), qx.reshape(rows, -1, 32))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("wtype", [synth.Q8_0, synth.Q4_1, synth.Q8_0_D4])
def test_mmq_rows_matrix_form(orc, wtype):
    """The products of many rows against numpy's matrix form (d*q dequantised, plus m @ s)."""
    rng = np.random.default_rng(18 + wtype)
    n_out, k_in = 9, 384
    wmat = _block(wtype, rng, n_out * k_in // 32).reshape(-1)
    act = orc.q8_1_rows(rng.standard_normal((5, k_in)).astype(np.float32), orc.act_layout(wtype))
    got = orc.mmq_rows(wtype, wmat, n_out, k_in, act)
    parts = npref.matrix_parts(wmat, n_out, k_in, wtype)
    for r in range(5):
        want = npref.qproduct(parts, act[r], k_in, wtype)
        assert np.allclose(got[r], want, rtol=1e-12, atol=1e-12)
