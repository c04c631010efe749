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
def test_matrix_rows_matrix_form(orc, wtype):
    """The products of many rows against numpy's matrix form (d*q dequantised, plus m @ s)."""
    rng = np.random.default_rng(18 + wtype)
    n_out, k_in = 9, 384
    wmat = _block(wtype, rng, n_out * k_in // 32).reshape(-1)
    act = orc.q8_1_rows(rng.standard_normal((5, k_in)).astype(np.float32), orc.act_layout(wtype))
    got = orc.matrix_rows(wtype, wmat, n_out, k_in, act)
    parts = npref.matrix_parts(wmat, n_out, k_in, wtype)
    for r in range(5):
        want = npref.qproduct(parts, act[r], k_in, wtype)
        assert np.allclose(got[r], want, rtol=1e-12, atol=1e-12)
