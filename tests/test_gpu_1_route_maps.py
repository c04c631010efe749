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
