"""Pins for the oracle's number and byte formats (CPU only)."""
import numpy as np
import pytest

import npref
from quantized_expert_grouped_amd import synth


def _all_f16_values():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return bits, bits.view(np.float16)


def test_f16_to_f64_every_code(orc):
    bits, vals = _all_f16_values()
    for b, v in zip(bits[::1], vals[::1]):
        got = orc.f16_to_f64(int(b))
        want = float(v)
        if np.isnan(want):
            assert np.isnan(got)
        else:
            assert got == want and np.signbit(got) == np.signbit(want), hex(int(b))


def _check_f32_to_f16(orc, xs):
    xs = np.asarray(xs, np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        want = xs.astype(np.float16).view(np.uint16)
    for x, w in zip(xs, want):
        got = orc.f32_to_f16(float(x))
        if np.isnan(x):
            assert (got & 0x7c00) == 0x7c00 and (got & 0x3ff) != 0
        else:
            assert got == int(w), (float(x), hex(got), hex(int(w)))


def test_f32_to_f16_every_boundary_and_midpoint(orc):
    """Every finite fp16 value, the midpoints between neighbours (ties to even) and the fp32
    neighbours of those midpoints, against numpy's IEEE conversion."""
    _, vals = _all_f16_values()
    finite = vals[np.isfinite(vals)].astype(np.float64)
    finite = np.unique(finite)
    pos = finite[finite >= 0]
    mids = (pos[:-1] + pos[1:]) / 2.0                    # exact in fp32 (12 significant bits)
    mids32 = mids.astype(np.float32)
    assert np.all(mids32.astype(np.float64) == mids)
    up = np.nextafter(mids32, np.float32(np.inf))
    dn = np.nextafter(mids32, np.float32(0))
    xs = np.concatenate([pos.astype(np.float32), mids32, up, dn])
    xs = np.concatenate([xs, -xs])
    _check_f32_to_f16(orc, xs)


def test_f32_to_f16_overflow_and_specials(orc):
    xs = [65504.0, 65519.99, 65520.0, 70000.0, 1e30, np.inf, -np.inf, 0.0, -0.0,
          2.0 ** -24, 2.0 ** -25, np.nextafter(np.float32(2.0 ** -25), np.float32(1)),
          2.0 ** -26, 1e-10, 6.1e-5, 2.0 ** -14, np.nextafter(np.float32(2.0 ** -14), np.float32(0))]
    _check_f32_to_f16(orc, xs)
    assert orc.f32_to_f16(float("nan")) & 0x7c00 == 0x7c00


def test_f32_to_f16_random(orc):
    rng = np.random.default_rng(7)
    xs = (rng.standard_normal(20000) * np.exp2(rng.integers(-30, 17, 20000))).astype(np.float32)
    _check_f32_to_f16(orc, xs)


def test_sizes_closed_form(orc):
    assert orc.block_bytes(orc.Q8_0) == 34 and orc.block_bytes(orc.Q4_1) == 20
    # expert = gate + up (F x H) + down (H x F), 32 weights per block
    assert orc.expert_bytes(2048, 512, orc.Q8_0) == 3 * 2048 * 512 // 32 * 34 == 3342336
    assert orc.expert_bytes(2048, 512, orc.Q4_1) == 3 * 2048 * 512 // 32 * 20 == 1966080
    assert orc.q8_1_row_bytes(2048) == 2304 and orc.q8_1_row_bytes(512) == 576
    assert synth.expert_bytes(2048, 512, synth.Q8_0) == orc.expert_bytes(2048, 512, orc.Q8_0)


def test_q4_1_nibble_layout_round_trip():
    """Byte j of a Q4_1 block's 16 packed bytes: element j low, element j+16 high."""
    q = np.arange(32, dtype=np.uint8)[None, :] % 16
    q[0, 16:] = 15 - q[0, 16:]
    d = np.array([0.5], np.float16)
    m = np.array([-0.25], np.float16)
    blk = synth.pack_q4_1(q, d, m)[0]
    assert blk[0:2].view("<f2")[0] == np.float16(0.5)
    assert blk[2:4].view("<f2")[0] == np.float16(-0.25)
    for j in range(16):
        assert blk[4 + j] == (q[0, j] | (q[0, j + 16] << 4))
    qq, dd, mm = npref.unpack_matrix(blk, 1, 32, npref.Q4_1)
    assert np.array_equal(qq[0], q[0].astype(np.int64))
    assert dd[0, 0] == 0.5 and mm[0, 0] == -0.25


def test_q8_0_layout_round_trip():
    q = (np.arange(32, dtype=np.int64) * 9 - 127).clip(-127, 127).astype(np.int8)[None, :]
    d = np.array([2.0 ** -7], np.float16)
    blk = synth.pack_q8_0(q, d)[0]
    assert blk.size == 34
    assert blk[0:2].view("<f2")[0] == np.float16(2.0 ** -7)
    assert np.array_equal(blk[2:].view(np.int8), q[0])


@pytest.mark.parametrize("wtype", [synth.Q8_0, synth.Q4_1])
def test_generated_pool_ranges(wtype):
    c = synth.make_case(T=3, H=256, F=128, E=4, K=2, wtype=wtype, seed=5)
    for e in range(c.E):
        q, d, m = npref.unpack_matrix(c.expert(e), 3 * 128 * 256 // 256, 256, wtype)
        assert d.min() >= 0.00099 and d.max() <= 0.01001
        if wtype == synth.Q8_0:
            assert q.min() >= -127 and q.max() <= 127
        else:
            assert q.min() >= 0 and q.max() <= 15
            assert m.min() >= -0.05001 and m.max() <= 0.0
    offs = np.sort(c.expert_off)
    assert np.all(np.diff(offs) == c.expert_stride) and c.expert_stride % 256 == 0
