"""Pins for the oracle's expert chain (a4..a6), combine (a7) and whole layer (CPU only)."""
import numpy as np
import pytest

import npref
from quantized_expert_grouped_amd import synth


def _rel_err(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - b)) / max(np.max(np.abs(b)), 1e-300))


@pytest.mark.parametrize("wtype", [synth.Q8_0, synth.Q4_1, synth.Q8_0_D4])
def test_dense_special_case(orc, wtype):
    """E = 1, K = 1, w = 1 reduces the layer to one quantised FFN, which numpy.matmul on the
    dequantised weights and activations computes independently (gate = first F rows)."""
    c = synth.make_case(T=9, H=256, F=128, E=1, K=1, wtype=wtype, seed=21, zero_tokens=(4,))
    idx = np.zeros((c.T, 1), np.int32)
    w = np.ones((c.T, 1), np.float32)
    out, dbg = orc.prefill_layer(c.x, idx, w, wtype, c.pool, c.expert_off, c.F, c.E, debug=True)
    ref = npref.layer(c.x, idx, w, c.pool, c.expert_off, c.expert_bytes, c.H, c.F, wtype)
    assert _rel_err(out, ref) <= 1e-6
    assert not out[4].any()                               # an all-zero token gives a zero row
    # K = 1, w = 1: the output is Dm rounded to fp32
    assert np.array_equal(out, dbg["Dm"].astype(np.float32))
    # the requantised h is the numpy quantiser's bytes of the oracle's own fp32 h
    assert np.array_equal(dbg["hq8"], npref.q8_1_rows_for(dbg["h"], wtype))
    assert np.array_equal(dbg["q8x"], npref.q8_1_rows_for(c.x, wtype))


def test_swapped_gate_up_is_detected(orc):
    """The dense check distinguishes gate from up: exchanging them changes the output."""
    c = synth.make_case(T=4, H=256, F=128, E=1, K=1, wtype=synth.Q8_0, seed=22)
    idx = np.zeros((c.T, 1), np.int32)
    w = np.ones((c.T, 1), np.float32)
    out = orc.prefill_layer(c.x, idx, w, c.wtype, c.pool, c.expert_off, c.F, c.E)
    sw = c.pool.copy()
    gu = c.F * (c.H // 32) * 34
    o = int(c.expert_off[0])
    sw[o:o + gu], sw[o + gu:o + 2 * gu] = c.pool[o + gu:o + 2 * gu], c.pool[o:o + gu]
    ref_sw = npref.layer(c.x, idx, w, sw, c.expert_off, c.expert_bytes, c.H, c.F, c.wtype)
    assert _rel_err(out, ref_sw) > 1e-2


@pytest.mark.parametrize("wtype", [synth.Q8_0, synth.Q4_1, synth.Q8_0_D4])
def test_tiny_layer_against_numpy(orc, wtype):
    """The five-config 'tiny' shape (T=7, H=256, F=128, E=16, K=2, token 3 zero) through
    the whole layer against the numpy dense chain per route."""
    c = synth.make_case(T=7, H=256, F=128, E=16, K=2, wtype=wtype, seed=1001, zero_tokens=(3,))
    idx, w = orc.route_topk(c.logits, c.K)
    out = orc.prefill_layer(c.x, idx, w, wtype, c.pool, c.expert_off, c.F, c.E)
    ref = npref.layer(c.x, idx, w, c.pool, c.expert_off, c.expert_bytes, c.H, c.F, wtype)
    assert _rel_err(out, ref) <= 1e-6
    assert not out[3].any()
    # loose sanity against the unquantised fp64 MoE (q8_1 activations cost ~1%)
    ref_fp = npref.layer_unquantized(c.x, idx, w, c.pool, c.expert_off, c.expert_bytes, c.H, c.F,
                                     wtype)
    assert _rel_err(out, ref_fp) < 0.05


def test_combine_closed_forms(orc):
    rng = np.random.default_rng(5)
    T, K, H = 6, 3, 8
    R = T * K
    Dm = rng.standard_normal((R, H))
    slot = rng.permutation(R).astype(np.int32)
    w = rng.uniform(0, 1, (T, K)).astype(np.float32)
    out = orc.combine(Dm, slot, w)
    for t in range(T):
        acc = np.zeros(H)
        for k in range(K):
            acc = acc + float(w[t, k]) * Dm[slot[t * K + k]]
        assert np.allclose(out[t], acc, rtol=1e-7, atol=0)
    # K = 1 and w = 1: the row itself
    out1 = orc.combine(Dm[:T], np.arange(T, dtype=np.int32), np.ones((T, 1), np.float32))
    assert np.array_equal(out1, Dm[:T].astype(np.float32))
    # the combine reads row slot[t*K+k] (not row t*K+k): permuting rows permutes nothing else
    perm = rng.permutation(R)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(R)
    out2 = orc.combine(Dm[perm], inv[slot].astype(np.int32), w)
    assert np.array_equal(out, out2)


@pytest.mark.parametrize("wtype", [synth.Q8_0, synth.Q4_1, synth.Q8_0_D4])
def test_token_out_equals_layer_rows(orc, wtype):
    c = synth.make_case(T=11, H=256, F=128, E=8, K=3, wtype=wtype, seed=31)
    idx, w = orc.route_topk(c.logits, c.K)
    out = orc.prefill_layer(c.x, idx, w, wtype, c.pool, c.expert_off, c.F, c.E)
    for t in (0, 5, 10):
        row = orc.token_out(c.x[t], idx[t], w[t], wtype, c.pool, c.expert_off, c.F)
        assert np.array_equal(row, out[t])


def test_layer_token_permutation_equivariance(orc):
    c = synth.make_case(T=10, H=256, F=128, E=8, K=3, wtype=synth.Q4_1, seed=32)
    idx, w = orc.route_topk(c.logits, c.K)
    out = orc.prefill_layer(c.x, idx, w, c.wtype, c.pool, c.expert_off, c.F, c.E)
    p = np.random.default_rng(0).permutation(c.T)
    out_p = orc.prefill_layer(c.x[p], idx[p], w[p], c.wtype, c.pool, c.expert_off, c.F, c.E)
    assert np.array_equal(out_p, out[p])


def test_layer_rejects_bad_shapes(orc):
    c = synth.make_case(T=2, H=256, F=128, E=4, K=2, wtype=synth.Q8_0, seed=1)
    idx = np.zeros((2, 5), np.int32)
    with pytest.raises(ValueError):
        orc.prefill_layer(c.x, idx, np.ones((2, 5), np.float32), c.wtype, c.pool, c.expert_off,
                          c.F, c.E)


def test_d4_and_ds4_differ_only_by_the_activation_scales(orc):
    """The same Q8_0 experts with D4 and with DS4 activations: the q bytes of x agree, the
    outputs differ by about fp16's relative precision (DS4 rounds d to fp16, D4 keeps fp32)."""
    a = synth.make_case(T=20, H=256, F=128, E=6, K=2, wtype=synth.Q8_0, seed=51)
    b = synth.make_case(T=20, H=256, F=128, E=6, K=2, wtype=synth.Q8_0_D4, seed=51)
    assert np.array_equal(a.pool, b.pool)
    idx, w = orc.route_topk(a.logits, a.K)
    oa, da = orc.prefill_layer(a.x, idx, w, a.wtype, a.pool, a.expert_off, a.F, a.E, debug=True)
    ob, db = orc.prefill_layer(b.x, idx, w, b.wtype, b.pool, b.expert_off, b.F, b.E, debug=True)
    G = a.H // 128
    qa = da["q8x"].reshape(-1, G, 144)[:, :, 16:]
    qb = db["q8x"].reshape(-1, G, 144)[:, :, 16:]
    assert np.array_equal(qa, qb)
    err = _rel_err(ob, oa.astype(np.float64))
    assert 0 < err < 4e-3
