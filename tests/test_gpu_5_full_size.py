"""GPU parity at the named workloads' full sizes, in the launch configuration the benchmark times
(routing from the logits on the GPU, then the layer).

The oracle routes the same logits itself; its ids must equal the GPU's everywhere and its
weights agree within 1e-6.  Where the whole oracle layer runs in seconds (T = 2048 and 8192,
20,480 and 81,920 routed rows) the whole output is compared, and every group position's bytes
are decoded and compared with the oracle's copy of its expert.  At T = 32768 and 30118 the oracle
checks what it can compute one by one: the maps whole, the q8_1 rows and the output rows of
sampled tokens (each output row depends only on its own x row and K routes), and sampled group
positions."""
import numpy as np
import pytest
import torch

import mmq_layout
from gpu_util import dev, host, note, rel_err
from quantized_expert_grouped_amd import abi, synth
from quantized_expert_grouped_amd.layer import MoePrefillLayer

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

WHOLE = {"tiny", "t2k", "t8k", "t2k_d4"}     # whole output and every group position


def oracle_case(name):
    if name.endswith("_d4"):                 # the same Q8_0 experts with D4 activations
        c = synth.config_case(name[:-3])
        c.wtype = synth.Q8_0_D4
        c.name = name
        return c
    return synth.config_case(name)


def oracle_layer(orc, oracle_cache, c):
    """The oracle's routing and whole layer for a workload (cached for the session)."""
    if c.name not in oracle_cache:
        idx, w = orc.route_topk(c.logits, c.K)
        out = orc.prefill_layer(c.x, idx, w, c.wtype, c.pool, c.expert_off, c.F, c.E)
        oracle_cache[c.name] = (idx, w, out)
    return oracle_cache[c.name]


@pytest.mark.parametrize("name", ["tiny", "t2k", "t8k", "t32k", "t30k_zipf", "t30k_z092", "t2k_d4"])
def test_full_size_workload(orc, oracle_cache, name):
    c = oracle_case(name)
    whole = name in WHOLE
    layer = MoePrefillLayer(c.pool, c.expert_off, c.H, c.F, c.E, c.wtype, c.T, c.K,
                            group_size=16, ring_start=c.ring_start)
    x, logits = dev(c.x), dev(c.logits)
    note(f"full-size {name} T={c.T} wtype={c.wtype}")
    idx_d, w_d = layer.route(logits)
    out = host(layer.forward(x, idx_d, w_d))
    idx, w = host(idx_d), host(w_d)
    # routing, every token: the oracle's ids exactly, its weights within 1e-6
    if whole:
        oi, ow, want = oracle_layer(orc, oracle_cache, c)
    else:
        oi, ow = orc.route_topk(c.logits, c.K)
    assert np.array_equal(idx, oi)
    assert np.max(np.abs(w - ow) / ow) <= 1e-6
    # maps, whole, from the oracle's routing
    m = orc.build_maps(oi, c.E, c.ring_start)
    R, H = c.R, c.H
    ws = layer.ws

    def off(which):
        return abi.workspace_offset(which, c.T, c.H, c.F, c.E, c.K, c.wtype, 16)

    def region(which, nbytes):
        return host(ws[off(which):off(which) + nbytes])

    assert np.array_equal(region(abi.WS_COUNTS, 4 * c.E).view(np.int32), m["counts"])
    assert np.array_equal(region(abi.WS_SRC, 4 * R).view(np.int32), m["src"])
    assert np.array_equal(region(abi.WS_SLOT, 4 * R).view(np.int32), m["slot"])
    n = int(region(abi.WS_NACTIVE, 4).view(np.int32)[0])
    assert n == m["n_active"]
    assert np.array_equal(region(abi.WS_ORDER, 4 * c.E).view(np.int32)[:n], m["order"])
    # quantised rows of sampled tokens (the zero tokens included), at every one of their K rows
    rng = np.random.default_rng(c.T)
    ts = np.unique(np.concatenate([rng.choice(c.T, min(c.T, 256), replace=False),
                                   np.array(c.zero_tokens, dtype=np.int64)]))
    xrb = abi.q8_1_row_bytes(H)
    q8 = ws[off(abi.WS_Q8X):off(abi.WS_Q8X) + R * xrb].view(R, xrb)
    rows = orc.q8_1_rows(c.x[ts], orc.act_layout(c.wtype))
    for j, t in enumerate(ts):
        got_rows = host(q8[torch.as_tensor(m["slot"][t * c.K:(t + 1) * c.K].astype(np.int64),
                                           device="cuda")])
        assert np.array_equal(got_rows, np.repeat(rows[j:j + 1], c.K, axis=0)), t
    # group positions, decoded, against the oracle's copy of their experts: all of them where
    # the whole layer is compared, else the first, middle and last few
    stride = off(abi.WS_GROUP_STRIDE)
    og = off(abi.WS_GROUPS)
    eb = c.expert_bytes
    pos = range(n) if whole else sorted({0, 1, n // 3, n // 2, n - 2, n - 1} & set(range(n)))
    for i0 in range(0, len(pos), 64):
        chunk = list(pos)[i0:i0 + 64]
        raw = np.zeros(len(chunk) * eb, np.uint8)
        orc.gather(c.pool, c.expert_off, m["order"][chunk], eb, raw, 0, eb)
        for j, i in enumerate(chunk):
            got_e = host(ws[og + i * stride:og + i * stride + eb])
            mmq_layout.check_positions(got_e, c.wtype, c.H, c.F, [raw[j * eb:(j + 1) * eb]], 0, 0)
    # the output
    if whole:
        assert rel_err(out, want) <= 1e-3
    else:
        ts_out = np.unique(np.concatenate([ts[:32], np.array(c.zero_tokens, dtype=np.int64)]))
        want = np.stack([orc.token_out(c.x[t], oi[t], ow[t], c.wtype, c.pool, c.expert_off, c.F)
                         for t in ts_out])
        assert rel_err(out[ts_out], want) <= 1e-3
    for t in c.zero_tokens:
        assert not out[t].any()
    assert np.isfinite(out).all()


@pytest.mark.parametrize("wtype", [synth.Q4_1, synth.Q8_0])
def test_large_expert_shape(orc, wtype):
    """H = 7168, F = 2048 (56 and 16 stages of 128 values, 2048-row down tiles): the whole
    output against the oracle."""
    c = synth.make_case("large", T=96, H=7168, F=2048, E=12, K=4, wtype=wtype, seed=71 + wtype,
                        zero_tokens=(5,))
    layer = MoePrefillLayer(c.pool, c.expert_off, c.H, c.F, c.E, c.wtype, c.T, c.K,
                            group_size=16, ring_start=c.ring_start)
    note(f"large shape H=7168 F=2048 wtype={wtype}")
    idx, w = orc.route_topk(c.logits, c.K)
    out = host(layer.forward(dev(c.x), dev(idx), dev(w)))
    want = orc.prefill_layer(c.x, idx, w, c.wtype, c.pool, c.expert_off, c.F, c.E)
    assert rel_err(out, want) <= 1e-3
    assert not out[5].any()
