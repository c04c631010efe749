"""GPU parity at the named workloads' full sizes, in the launch configuration the benchmark times.

The oracle cannot run whole layers of this size in seconds, so it checks what it can compute
one by one: routing, maps and quantised rows in full or on samples, and the output rows of
sampled tokens (each one depends only on its own x row and K routes)."""
import numpy as np
import pytest
import torch

from gpu_util import dev, host, note, rel_err
from quantized_expert_grouped_amd import abi, synth
from quantized_expert_grouped_amd.layer import MoePrefillLayer

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.mark.parametrize("name", ["tiny", "t2k", "t8k", "t32k", "t30k_zipf", "t30k_z092", "t2k_d4"])
def test_full_size_workload(orc, name):
    if name.endswith("_d4"):                 # the same Q8_0 experts with D4 activations
        c = synth.config_case(name[:-3])
        c.wtype = synth.Q8_0_D4
    else:
        c = synth.config_case(name)
    layer = MoePrefillLayer(c.pool, c.expert_off, c.H, c.F, c.E, c.wtype, c.T, c.K,
                            group_size=16, ring_start=c.ring_start)
    x, logits = dev(c.x), dev(c.logits)
    note(f"full-size {name} T={c.T} wtype={c.wtype}")
    idx_d, w_d = layer.route(logits)
    out = host(layer.forward(x, idx_d, w_d))
    idx, w = host(idx_d), host(w_d)
    rng = np.random.default_rng(c.T)
    # routing: exact ids, weights within 1e-6 of the fp64 softmax, on sampled tokens
    ts = np.unique(np.concatenate([rng.choice(c.T, min(c.T, 256), replace=False),
                                   np.array(c.zero_tokens, dtype=np.int64)]))
    oi, ow = orc.route_topk(c.logits[ts], c.K)
    assert np.array_equal(idx[ts], oi)
    assert np.max(np.abs(w[ts] - ow) / ow) <= 1e-6
    # maps from the GPU's routing, whole
    m = orc.build_maps(idx, c.E, c.ring_start)
    R, H = c.R, c.H
    ws = layer.ws

    def region(which, nbytes):
        o = abi.workspace_offset(which, c.T, c.H, c.F, c.E, c.K, c.wtype, 16)
        return host(ws[o:o + nbytes])

    assert np.array_equal(region(abi.WS_SRC, 4 * R).view(np.int32), m["src"])
    assert np.array_equal(region(abi.WS_SLOT, 4 * R).view(np.int32), m["slot"])
    n = int(region(abi.WS_NACTIVE, 4).view(np.int32)[0])
    assert n == m["n_active"]
    assert np.array_equal(region(abi.WS_ORDER, 4 * c.E).view(np.int32)[:n], m["order"])
    # quantised rows of sampled tokens, at every one of their K rows
    xrb = abi.q8_1_row_bytes(H)
    o = abi.workspace_offset(abi.WS_Q8X, c.T, c.H, c.F, c.E, c.K, c.wtype, 16)
    q8 = ws[o:o + R * xrb].view(R, xrb)
    rows = orc.q8_1_rows(c.x[ts], orc.act_layout(c.wtype))
    for j, t in enumerate(ts):
        got_rows = host(q8[torch.as_tensor(m["slot"][t * c.K:(t + 1) * c.K].astype(np.int64),
                                           device="cuda")])
        assert np.array_equal(got_rows, np.repeat(rows[j:j + 1], c.K, axis=0)), t
    # a sampled expert's gathered bytes
    stride = abi.workspace_offset(abi.WS_GROUP_STRIDE, c.T, c.H, c.F, c.E, c.K, c.wtype, 16)
    og = abi.workspace_offset(abi.WS_GROUPS, c.T, c.H, c.F, c.E, c.K, c.wtype, 16)
    for i in sorted({0, n // 2, n - 1}):
        got_e = host(ws[og + i * stride:og + i * stride + c.expert_bytes])
        assert np.array_equal(got_e, orc.mmq_pack(c.wtype, c.expert(int(m["order"][i])), c.H, c.F))
    # output rows of sampled tokens against the oracle (the GPU's routing as its input)
    ts_out = ts[:24] if len(ts) > 24 else ts
    ts_out = np.unique(np.concatenate([ts_out, np.array(c.zero_tokens, dtype=np.int64)]))
    want = np.stack([orc.token_out(c.x[t], idx[t], w[t], c.wtype, c.pool, c.expert_off, c.F)
                     for t in ts_out])
    assert rel_err(out[ts_out], want) <= 1e-3
    for t in c.zero_tokens:
        assert not out[t].any()
    assert np.isfinite(out).all()


@pytest.mark.parametrize("wtype", [synth.Q4_1, synth.Q8_0])
def test_large_expert_shape(orc, wtype):
    """H = 7168, F = 2048 (56 and 16 stages of 128 values, 2048-row down tiles): the layer's rows
    of sampled tokens against the oracle."""
    c = synth.make_case("large", T=96, H=7168, F=2048, E=12, K=4, wtype=wtype, seed=71 + wtype,
                        zero_tokens=(5,))
    layer = MoePrefillLayer(c.pool, c.expert_off, c.H, c.F, c.E, c.wtype, c.T, c.K,
                            group_size=16, ring_start=c.ring_start)
    note(f"large shape H=7168 F=2048 wtype={wtype}")
    idx, w = orc.route_topk(c.logits, c.K)
    out = host(layer.forward(dev(c.x), dev(idx), dev(w)))
    ts = [0, 5, 37, 95]
    want = np.stack([orc.token_out(c.x[t], idx[t], w[t], c.wtype, c.pool, c.expert_off, c.F)
                     for t in ts])
    assert rel_err(out[ts], want) <= 1e-3
    assert not out[5].any()
