"""moe_build_maps_noalloc, the map build for callers that cannot allocate, against the workspace
form moe_build_maps on the same routes, bit for bit (integer work), through the C ABI: calls in a
row on one GPU (the static scratch keeps the previous call's contents; the second call is
smaller), ids out of range, the largest size it accepts, and the sizes it refuses."""
import numpy as np
import pytest
import torch

from gpu_util import dev, empty, gpu_maps, host, note
from quantized_expert_grouped_amd import abi

pytestmark = pytest.mark.gpu

KEYS = ("counts", "offsets", "src", "slot", "order")


def noalloc_maps(idx, E, ring, with_flag=True):
    T, K = idx.shape
    R = T * K
    out = dict(counts=empty(E, torch.int32), offsets=empty(E + 1, torch.int32),
               src=empty(R, torch.int32), slot=empty(R, torch.int32),
               order=empty(E, torch.int32), n_active=empty(1, torch.int32))
    flag = torch.full((1,), -7, dtype=torch.int32, device="cuda") if with_flag else None
    note(f"maps_noalloc T={T} K={K} E={E} ring={ring}")
    abi.build_maps_noalloc(dev(idx.astype(np.int32)), E, ring, out["counts"], out["offsets"],
                           out["src"], out["slot"], out["order"], out["n_active"], flag)
    res = {k: host(v) for k, v in out.items()}
    res["n_active"] = int(res["n_active"][0])
    res["order"] = res["order"][:res["n_active"]]
    res["n_invalid"] = int(host(flag)[0]) if with_flag else None
    return res


def _routes(rng, T, K, E):
    return rng.integers(0, E, size=(T, K), dtype=np.int64).astype(np.int32)


def _same(got, want):
    for k in KEYS:
        assert np.array_equal(got[k], want[k]), k
    assert got["n_active"] == want["n_active"]


def test_noalloc_equals_workspace_form_on_calls_in_a_row(orc):
    rng = np.random.default_rng(77)
    cases = [(8192, 10, 512, 5, 0), (1000, 3, 2048, 2047, 9), (7, 2, 16, 3, 0), (513, 8, 64, 17, 0)]
    for T, K, E, ring, n_bad in cases:            # each call smaller than the first
        idx = _routes(rng, T, K, E)
        if n_bad:
            flat = idx.reshape(-1)
            flat[rng.choice(flat.size, n_bad, replace=False)] = np.array([-1, E, E + 3])[
                np.arange(n_bad) % 3]
        got = noalloc_maps(idx, E, ring)
        want, _ = gpu_maps(idx, E, ring)
        _same(got, want)
        assert got["n_invalid"] == want["n_invalid"] == n_bad
        if n_bad == 0:
            o = orc.build_maps(idx, E, ring)
            for k in KEYS:
                assert np.array_equal(got[k], o[k]), k


def test_noalloc_largest_size_then_smaller_without_flag(orc):
    """T*K = 2^19 routes over 2048 experts (the whole array in use), then a small call with no
    status pointer: both equal the workspace form."""
    rng = np.random.default_rng(5)
    idx = _routes(rng, 32768, 16, 2048)
    got = noalloc_maps(idx, 2048, 100)
    want, _ = gpu_maps(idx, 2048, 100)
    _same(got, want)
    assert got["n_invalid"] == 0
    idx2 = _routes(rng, 300, 4, 40)
    got2 = noalloc_maps(idx2, 40, 7, with_flag=False)
    want2, _ = gpu_maps(idx2, 40, 7)
    _same(got2, want2)


def test_noalloc_refuses_sizes_beyond_its_array():
    """Refused on the host before anything is enqueued (the outputs are sized for the call all
    the same, so that nothing could be written out of bounds even if a check were missing)."""
    def outs(T, K, E):
        R = T * K
        return [empty(E, torch.int32), empty(E + 1, torch.int32), empty(R, torch.int32),
                empty(R, torch.int32), empty(E, torch.int32), empty(1, torch.int32)]
    T = (1 << 19) // 16 + 1                                          # T*K = 2^19 + 16
    big = torch.zeros((T, 16), dtype=torch.int32, device="cuda")
    assert abi.raw_build_maps_noalloc(big, 512, 0, *outs(T, 16, 512)) == -2
    small = torch.zeros((4, 2), dtype=torch.int32, device="cuda")
    assert abi.raw_build_maps_noalloc(small, 2049, 0, *outs(4, 2, 2049)) == -2   # E > MOE_MAX_E
    assert abi.raw_build_maps_noalloc(small, 16, 16, *outs(4, 2, 16)) == -1      # bad ring_start
