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
