"""Pins for the oracle's routing (a0) and token->row maps (a1) (CPU only)."""
import math

import numpy as np
import pytest

import npref


@pytest.mark.parametrize("T,E,K", [(7, 16, 2), (50, 512, 10), (33, 64, 8)])
def test_route_against_stable_sort(orc, T, E, K):
    rng = np.random.default_rng(T * E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[3, 5:20] = logits[3, 4]                 # ties: lower id first
    idx, w = orc.route_topk(logits, K)
    ridx, rw = npref.route(logits, K)
    assert np.array_equal(idx, ridx)
    assert np.allclose(w, rw, rtol=1e-6, atol=0)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)


def test_route_weight_closed_forms(orc):
    # chosen logits 0, -ln2, -ln4 -> weights 4/7, 2/7, 1/7 (the rest far below)
    E = 8
    l = np.full((1, E), -50.0, np.float32)
    l[0, 6], l[0, 2], l[0, 4] = 0.0, -math.log(2), -math.log(4)
    idx, w = orc.route_topk(l, 3)
    assert list(idx[0]) == [6, 2, 4]
    assert np.allclose(w[0], [4 / 7, 2 / 7, 1 / 7], rtol=1e-6)
    # all equal -> the K lowest ids, equal weights
    idx, w = orc.route_topk(np.zeros((2, 12), np.float32), 4)
    assert np.array_equal(idx, [[0, 1, 2, 3]] * 2) and np.allclose(w, 0.25)
    # -0.0 and +0.0 compare equal: the lower id wins
    l = np.zeros((1, 4), np.float32)
    l[0, 0] = -0.0
    l[0, 3] = 1.0
    idx, _ = orc.route_topk(l, 2)
    assert list(idx[0]) == [3, 0]
    # K = 1 -> weight exactly 1
    idx, w = orc.route_topk(np.random.default_rng(1).standard_normal((5, 9)).astype(np.float32), 1)
    assert np.all(w == 1.0)


def test_route_shift_invariance(orc):
    rng = np.random.default_rng(3)
    l = rng.standard_normal((20, 64)).astype(np.float32)
    i1, w1 = orc.route_topk(l, 6)
    i2, w2 = orc.route_topk((l * 1).astype(np.float32) + np.float32(0.0), 6)
    assert np.array_equal(i1, i2) and np.array_equal(w1, w2)
    # a full-softmax-then-renormalise reading gives the same weights
    z = l.astype(np.float64)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(p, i1.astype(np.int64), axis=1)
    assert np.allclose(w1, sel / sel.sum(axis=1, keepdims=True), rtol=1e-6)


@pytest.mark.parametrize("T,K,E,ring", [(7, 2, 16, 0), (7, 2, 16, 5), (300, 10, 512, 77),
                                        (64, 4, 32, 31)])
def test_maps_against_brute_force(orc, T, K, E, ring):
    rng = np.random.default_rng(T + E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    if E == 32:
        logits[:, :20] -= 100          # 12 of 32 experts receive every row, 20 receive none
    idx, _ = orc.route_topk(logits, K)
    m = orc.build_maps(idx, E, ring)
    ref = npref.maps(idx, E, ring)
    for key in ("counts", "offsets", "src", "slot", "order"):
        assert np.array_equal(m[key], ref[key]), key
    assert m["n_active"] == len(ref["order"])


def test_maps_invariants(orc):
    rng = np.random.default_rng(9)
    T, K, E = 257, 10, 512
    idx, _ = orc.route_topk(rng.standard_normal((T, E)).astype(np.float32), K)
    m = orc.build_maps(idx, E, 100)
    R = T * K
    src, slot = m["src"], m["slot"]
    assert np.array_equal(np.sort(src), np.arange(R))        # a permutation
    assert np.array_equal(slot[src], np.arange(R))           # slot is src's inverse
    assert np.array_equal(src[slot], np.arange(R))
    assert m["counts"].sum() == R and m["offsets"][-1] == R
    flat = idx.reshape(-1)
    for e in range(E):
        seg = src[m["offsets"][e]:m["offsets"][e + 1]]
        assert np.all(flat[seg] == e)                       # only its own rows
        assert np.all(np.diff(seg) > 0)                     # ascending t*K+k (stable)
    # ring order: starts at the first active expert at or after ring_start, wraps once
    o = m["order"]
    pos = (o - 100) % E
    assert np.all(np.diff(pos) > 0)
    assert set(o.tolist()) == set(np.nonzero(m["counts"])[0].tolist())
