"""Pins for the oracle's q8_1 quantiser and its two forms (CPU only).

The pages fix the invariant (the scatter form writes the same bytes as the per-row gather
form, for T = 1, 2, 7, 600, 2099 with 10 of 512 experts and one all-zero token); the
mathematics fixes the closed forms and bounds below; an independent numpy quantiser fixes
every byte.
"""
import numpy as np
import pytest

import npref


def test_closed_form_power_of_two_scale(orc):
    """amax = 127 * 2^k makes d = 2^k exactly, so q_j = v_j / 2^k with halves rounded away
    from zero (not to even)."""
    for k in (-12, -3, 0, 5):
        s = 2.0 ** k
        qv = np.array([127, -126, 2.5, -2.5, 0.5, -0.5, 1.5, -1.5, 3.49, -3.51, 0, 64, -64.5]
                      + [1.0] * 19, np.float64)
        v = (qv * s).astype(np.float32)
        q, d16, s16 = orc.q8_1_block(v)
        want = np.sign(qv) * np.floor(np.abs(qv) + 0.5)
        assert np.array_equal(q.astype(np.float64), want)
        assert q[2] == 3 and q[3] == -3 and q[4] == 1 and q[5] == -1 and q[6] == 2
        assert orc.f16_to_f64(d16) == s
        S = int(want.sum())
        assert s16 == int(np.float16(np.float32(s) * np.float32(S)).view(np.uint16))


def test_zero_block(orc):
    q, d16, s16 = orc.q8_1_block(np.zeros(32, np.float32))
    assert not q.any() and d16 == 0 and s16 == 0
    q, d16, s16 = orc.q8_1_block(-np.zeros(32, np.float32))
    assert not q.any() and d16 == 0 and s16 == 0


def test_max_element_maps_to_127_and_error_bound(orc):
    rng = np.random.default_rng(11)
    for _ in range(2000):
        v = (rng.standard_normal(32) * np.exp2(rng.integers(-20, 20))).astype(np.float32)
        q, d16, s16 = orc.q8_1_block(v)
        j = int(np.argmax(np.abs(v)))
        assert abs(int(q[j])) == 127 and np.sign(q[j]) == np.sign(v[j])
        amax = float(np.max(np.abs(v)))
        d = float(np.float32(amax) / np.float32(127))
        # |d q - v| <= d/2 up to the rounding of v/d
        err = np.abs(d * q.astype(np.float64) - v.astype(np.float64))
        assert np.all(err <= d * (0.5 + 2.0 ** -20))
        # the stored scale is the fp16 of d; the dequantised error grows by 127 |d16 - d|
        d16v = orc.f16_to_f64(d16)
        # relative half-ulp for normal fp16, absolute half the subnormal spacing below 2^-14
        assert abs(d16v - d) <= max(d * 2.0 ** -11, 2.0 ** -25)
        err16 = np.abs(d16v * q.astype(np.float64) - v.astype(np.float64))
        assert np.all(err16 <= 0.5 * d * (1 + 2.0 ** -20) + 127 * abs(d16v - d))
        assert orc.f16_to_f64(s16) == float(np.float16(np.float32(d) * np.float32(int(q.sum()))))


def test_block_against_numpy_quantiser(orc):
    rng = np.random.default_rng(12)
    v = rng.standard_normal((3000, 32)).astype(np.float32)
    v[::7] *= np.float32(1e-6)
    v[1::9] = np.round(v[1::9] * 8) / 8          # many exact halves after scaling
    v[5] = 0
    qn, dn, sn = npref.q8_1_blocks(v)
    for i in range(v.shape[0]):
        q, d16, s16 = orc.q8_1_block(v[i])
        assert np.array_equal(q, qn[i]) and d16 == dn[i] and s16 == sn[i], i


@pytest.mark.parametrize("n", [128, 256, 2048])
def test_row_layout_against_numpy(orc, n):
    rng = np.random.default_rng(n)
    v = rng.standard_normal((9, n)).astype(np.float32)
    v[3] = 0
    got = orc.q8_1_rows(v)
    assert got.shape == (9, n // 128 * 144)
    assert np.array_equal(got, npref.q8_1_rows(v))


def test_golden_rows(orc):
    """Fixed rows whose bytes were derived by hand (tests/golden/q8_1_rows.txt)."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "q8_1_rows.txt")
    cases = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            vals_s, hexbytes = line.split("|")
            vals = np.array([float(t) for t in vals_s.split()], np.float32)
            cases.append((vals, bytes.fromhex(hexbytes.strip())))
    assert cases
    for vals, want in cases:
        got = orc.q8_1_rows(vals[None, :])[0].tobytes()
        assert got == want


@pytest.mark.parametrize("T", [1, 2, 7, 600, 2099])
def test_scatter_equals_gather(orc, T):
    """The invariant the quantize-once-and-scatter page checks: scatter writes exactly the
    bytes of the per-row gather, over the whole output buffer (10 of 512 experts, one
    all-zero token)."""
    rng = np.random.default_rng(100 + T)
    H, K, E = 256, 10, 512
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[T // 2] = 0
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx, _ = orc.route_topk(logits, K)
    m = orc.build_maps(idx, E)
    g = orc.quantize_gather(x, K, m["src"])
    s = orc.quantize_scatter(x, K, m["slot"])
    assert np.array_equal(g, s)
    # and both are the numpy quantiser's rows placed through src
    want = npref.q8_1_rows(x)[m["src"] // K]
    assert np.array_equal(g, want)
    z = m["slot"][(T // 2) * K:(T // 2) * K + K]
    assert not g[z].any()


@pytest.mark.parametrize("n", [128, 2048])
def test_d4_rows_against_numpy(orc, n):
    """D4 (the layout the quantize-once page names for Q8_0): per 128 values the 4 blocks' fp32
    d = amax/127, then the q of DS4.  Against numpy's float32 arithmetic, plus the links to the
    pinned DS4 form: the same q bytes, and fp16 of the D4 d is DS4's d16."""
    rng = np.random.default_rng(n + 5)
    v = (rng.standard_normal((5, n)) * 3).astype(np.float32)
    v[1, :32] = 0                       # an all-zero block: zero header, zero q
    v[2, 32:64] = np.float32(1e-30)     # a tiny block: d far below fp16's range
    v[3, 64] = np.float32(-1e7)         # d above fp16's largest finite value (DS4: d16 = inf)
    got = orc.q8_1_rows(v, orc.D4)
    assert np.array_equal(got, npref.q8_1_rows_d4(v))
    ds4 = orc.q8_1_rows(v)
    g = got.reshape(5, n // 128, 144)
    h = ds4.reshape(5, n // 128, 144)
    assert np.array_equal(g[:, :, 16:], h[:, :, 16:])
    d = g[:, :, :16].copy().view("<f4").reshape(5, n // 32)
    amax = np.abs(v.reshape(5, n // 32, 32)).max(axis=-1)
    assert np.array_equal(d, (amax / np.float32(127)).astype(np.float32))
    assert d[1, 0] == 0 and not g[1, 0, 16:48].any()
    d16 = h[:, :, :16].copy().view("<u2").reshape(5, n // 32, 2)[..., 0]
    assert np.array_equal(d.astype(np.float16).view(np.uint16), d16)


@pytest.mark.parametrize("T", [1, 2, 7, 600, 2099])
def test_scatter_equals_gather_d4(orc, T):
    """The page's scatter-equals-gather check for the D4 layout (10 of 512 experts, one
    all-zero token), and both are numpy's D4 rows placed through src."""
    rng = np.random.default_rng(200 + T)
    H, K, E = 256, 10, 512
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[T // 2] = 0
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx, _ = orc.route_topk(logits, K)
    m = orc.build_maps(idx, E)
    g = orc.quantize_gather(x, K, m["src"], orc.D4)
    s = orc.quantize_scatter(x, K, m["slot"], orc.D4)
    assert np.array_equal(g, s)
    assert np.array_equal(g, npref.q8_1_rows_d4(x)[m["src"] // K])
    z = m["slot"][(T // 2) * K:(T // 2) * K + K]
    assert not g[z].any()
