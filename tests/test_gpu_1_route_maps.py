"""GPU parity: routing (a0) and the token->row maps (a1) against the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

from gpu_util import dev, empty, gpu_maps, host, note
from quantized_expert_grouped_amd import abi

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,E,K,zipf", [(7, 16, 2, None), (2048, 512, 10, None),
                                        (3001, 512, 10, 1.2), (64, 2048, 64, None),
                                        (100, 64, 1, None), (33, 10, 10, None)])
def test_route_topk(orc, T, E, K, zipf):
    note(f"route T={T} E={E} K={K} zipf={zipf}")
    rng = np.random.default_rng(T * 7 + E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    if zipf:
        logits += (-zipf * np.log(np.arange(1, E + 1)))[rng.permutation(E)].astype(np.float32)
    logits[0, :] = 0.5                      # a token whose logits all tie
    logits[min(1, T - 1), 3:9] = logits[min(1, T - 1), 2]
    idx = empty((T, K), torch.int32)
    w = empty((T, K), torch.float32)
    abi.route_topk(dev(logits), K, idx, w)
    gi, gw = host(idx), host(w)
    oi, ow = orc.route_topk(logits, K)
    assert np.array_equal(gi, oi)
    assert np.max(np.abs(gw.astype(np.float64) - ow) / ow) <= 1e-6


def test_route_topk_signed_zeros_and_extremes(orc):
    """Logits the order-preserving integer keys must rank as floats compare: -0.0 and +0.0 equal
    (the lower id first), negative values only, subnormals, values near the float range's ends,
    and a zero of either sign at the K-th place."""
    E, K = 64, 8
    L = np.full((6, E), -1.0, np.float32)
    for i, z in ((5, -0.0), (3, 0.0), (10, -0.0), (2, -0.0), (40, 0.0)):
        L[0, i] = z                                   # five zeros, mixed signs: ids 2, 3, 5, 10, 40
    L[1] = -np.logspace(-30, 30, E).astype(np.float32)[np.random.default_rng(1).permutation(E)]
    L[2, :] = np.float32(0.0)
    L[2, ::3] = np.float32(1e-40)                     # subnormal positives
    L[2, 1::3] = np.float32(-1e-40)                   # subnormal negatives
    L[2, 7] = np.float32(-0.0)
    L[3, :] = np.float32(-3e38)
    L[3, [9, 4, 60, 33]] = np.float32(3e38)           # ties at the top of the range
    L[4] = np.random.default_rng(4).standard_normal(E).astype(np.float32)
    L[5, :] = np.float32(-2.0)
    L[5, :7] = np.float32(1.0)
    L[5, 20] = np.float32(-0.0)                       # the 8th pick: a zero among the -2s
    L[5, 12] = np.float32(0.0)
    note("route signed zeros and extremes")
    idx = empty((6, K), torch.int32)
    w = empty((6, K), torch.float32)
    abi.route_topk(dev(L), K, idx, w)
    gi, gw = host(idx), host(w)
    oi, ow = orc.route_topk(L, K)
    assert np.array_equal(gi, oi)
    assert gi[0, :5].tolist() == [2, 3, 5, 10, 40]
    assert gi[5, 7] == 12
    # token 3's last four weights underflow to exactly 0 on both sides
    assert np.all(np.abs(gw.astype(np.float64) - ow) <= 1e-6 * np.abs(ow))


@pytest.mark.parametrize("T,K,E,ring", [(7, 2, 16, 0), (7, 2, 16, 9), (1, 1, 1, 0),
                                        (1000, 10, 512, 123), (8192, 10, 512, 5),
                                        (4099, 3, 2048, 2047), (513, 8, 64, 17)])
def test_build_maps_bit_exact(orc, T, K, E, ring):
    note(f"maps T={T} K={K} E={E} ring={ring}")
    rng = np.random.default_rng(T + K + E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    if E == 64:
        logits[:, :40] -= 50.0            # 40 experts receive no rows
    idx, _ = orc.route_topk(logits, K)
    got, _ = gpu_maps(idx, E, ring)
    want = orc.build_maps(idx, E, ring)
    for key in ("counts", "offsets", "src", "slot", "order"):
        assert np.array_equal(got[key], want[key]), key
    assert got["n_active"] == want["n_active"]
    assert got["n_invalid"] == 0


def test_build_maps_single_expert_skew(orc):
    """Every row on one expert (the extreme of a skewed routing): one expert holds all rows."""
    T, K, E = 5000, 1, 32
    idx = np.full((T, K), 7, np.int32)
    got, _ = gpu_maps(idx, E, 3)
    want = orc.build_maps(idx, E, 3)
    for key in ("counts", "offsets", "src", "slot", "order"):
        assert np.array_equal(got[key], want[key]), key
    assert got["n_active"] == 1


def test_build_maps_zipf_config(orc):
    T, E, K = 30118, 512, 10
    rng = np.random.default_rng(1005)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits += (-1.2 * np.log(np.arange(1, E + 1)))[rng.permutation(E)].astype(np.float32)
    idx, _ = orc.route_topk(logits, K)
    note("maps zipf T=30118")
    got, _ = gpu_maps(idx, E, 300)
    want = orc.build_maps(idx, E, 300)
    for key in ("counts", "offsets", "src", "slot", "order"):
        assert np.array_equal(got[key], want[key]), key
    assert want["n_active"] < E          # some experts receive no rows


@pytest.mark.parametrize("T,K,E,ring", [(7, 2, 16, 3), (1000, 10, 512, 123), (4099, 3, 2048, 2047)])
def test_build_maps_out_of_range_ids(orc, T, K, E, ring):
    """Ids outside [0, E) (a caller error): they are counted in the scratch's status word, take
    the rows after every real expert's in index order with src = -1, get slot = -1, and leave
    the real experts' maps as the oracle gives them with those ids taken as one more expert E
    (sorting after the rest)."""
    rng = np.random.default_rng(T + E + 1)
    idx, _ = orc.route_topk(rng.standard_normal((T, E)).astype(np.float32), K)
    flat = idx.reshape(-1).copy()
    bad_at = np.unique(np.concatenate([[0, len(flat) - 1],
                                       rng.choice(len(flat), max(1, len(flat) // 50))]))
    bad_vals = np.array([-1, E, E + 7, 2 ** 31 - 1, -(2 ** 31)], np.int64)
    flat[bad_at] = bad_vals[np.arange(len(bad_at)) % len(bad_vals)].astype(np.int32)
    bad = flat.reshape(T, K)
    note(f"maps with {len(bad_at)} out-of-range ids T={T} K={K} E={E}")
    got, _ = gpu_maps(bad, E, ring)
    assert got["n_invalid"] == len(bad_at)
    virt = flat.copy()
    virt[bad_at] = E                                   # the oracle's view: one more expert
    want = orc.build_maps(virt.reshape(T, K), E + 1, 0)
    rv = int(want["offsets"][E])                       # rows of the real experts
    assert np.array_equal(got["counts"], want["counts"][:E])
    assert np.array_equal(got["offsets"], want["offsets"][:E + 1])
    assert np.array_equal(got["src"][:rv], want["src"][:rv])
    assert np.all(got["src"][rv:] == -1) and len(got["src"]) - rv == len(bad_at)
    good = np.ones(len(flat), bool)
    good[bad_at] = False
    assert np.array_equal(got["slot"][good], want["slot"][good])
    assert np.all(got["slot"][~good] == -1)
    order = [(ring + j) % E for j in range(E) if want["counts"][(ring + j) % E] > 0]
    assert np.array_equal(got["order"], np.array(order, np.int32))
    # both quantiser forms skip those routes: their rows keep the buffer's old bytes
    x = rng.standard_normal((T, 256)).astype(np.float32)
    rb = abi.q8_1_row_bytes(256)
    for mode in (0, abi.QUANT_PER_ROW):
        q8 = torch.full((T * K, rb), 0xAB, dtype=torch.uint8, device="cuda")
        note(f"quantize mode={mode} with out-of-range routes")
        abi.quantize_scatter_q8_1(dev(x), K, dev(got["slot"]), dev(got["src"]), mode, q8)
        g = host(q8)
        assert np.all(g[rv:] == 0xAB)
        rows = orc.q8_1_rows(x)
        for i in np.flatnonzero(good)[::max(1, int(good.sum()) // 200)]:
            assert np.array_equal(g[got["slot"][i]], rows[i // K])
    # a later call with every id in range clears the count
    got2, _ = gpu_maps(idx, E, ring)
    assert got2["n_invalid"] == 0
