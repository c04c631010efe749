"""GPU parity: the whole layer (moe_prefill_layer) against the oracle, with its intermediate
buffers, the invariances the pages state, and edge cases."""
import zlib

import numpy as np
import pytest
import torch

import mmq_layout
from gpu_util import dev, host, note, rel_err
from quantized_expert_grouped_amd import abi, synth
from quantized_expert_grouped_amd.layer import MoePrefillLayer

pytestmark = pytest.mark.gpu

TOL = 1e-3   # max |gpu - oracle| <= 1e-3 * max |oracle|


def _layer(c, **kw):
    return MoePrefillLayer(c.pool, c.expert_off, c.H, c.F, c.E, c.wtype, c.T, c.K,
                           group_size=kw.get("group_size", 16),
                           ring_start=kw.get("ring_start", c.ring_start))


def _run(layer, c, idx, w, **kw):
    note(f"layer {c.name} T={c.T} H={c.H} F={c.F} E={c.E} K={c.K} wtype={c.wtype} {kw}")
    out = layer.forward(dev(c.x), dev(idx), dev(w), **kw)
    return host(out)


CASES = [
    # name, T, H, F, E, K, wtype, zipf
    ("tiny", 7, 256, 128, 16, 2, synth.Q8_0, None),
    ("tiny_q4_1", 7, 256, 128, 16, 2, synth.Q4_1, None),
    ("ragged", 301, 512, 256, 24, 4, synth.Q8_0, None),
    ("ragged_q4_1", 301, 512, 256, 24, 4, synth.Q4_1, None),
    ("skew", 403, 256, 384, 32, 3, synth.Q4_1, 1.2),
    ("wide", 64, 1024, 128, 8, 8, synth.Q8_0, None),
    ("ragged_d4", 301, 512, 256, 24, 4, synth.Q8_0_D4, None),
    ("three_stages", 150, 384, 384, 12, 3, synth.Q4_1, None),
    ("three_stages_q8_0", 150, 384, 384, 12, 3, synth.Q8_0, None),
    # H = 640: five 128-column n-tiles, a down workgroup's sweep of four and one of one
    ("five_ntiles", 211, 640, 256, 14, 3, synth.Q4_1, None),
    ("five_ntiles_q8_0", 211, 640, 256, 14, 3, synth.Q8_0, 1.2),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_layer_against_oracle(orc, case):
    name, T, H, F, E, K, wtype, zipf = case
    c = synth.make_case(name, T=T, H=H, F=F, E=E, K=K, wtype=wtype, seed=zlib.crc32(name.encode()) % 10000,
                        zero_tokens=(T // 3,), zipf=zipf)
    idx, w = orc.route_topk(c.logits, K)
    want, dbg = orc.prefill_layer(c.x, idx, w, wtype, c.pool, c.expert_off, F, E, debug=True)
    layer = _layer(c)
    got = _run(layer, c, idx, w)
    assert rel_err(got, want) <= TOL
    assert not got[T // 3].any()                      # an all-zero token: an exact zero row
    # intermediate results in the workspace
    R = T * K
    m = orc.build_maps(idx, E, c.ring_start)
    ws = host(layer.ws)

    def region(which, nbytes):
        o = abi.workspace_offset(which, T, H, F, E, K, wtype, 16)
        return ws[o:o + nbytes]

    assert np.array_equal(region(abi.WS_COUNTS, 4 * E).view(np.int32), m["counts"])
    assert np.array_equal(region(abi.WS_OFFSETS, 4 * (E + 1)).view(np.int32), m["offsets"])
    assert np.array_equal(region(abi.WS_SRC, 4 * R).view(np.int32), m["src"])
    assert np.array_equal(region(abi.WS_SLOT, 4 * R).view(np.int32), m["slot"])
    n = int(region(abi.WS_NACTIVE, 4).view(np.int32)[0])
    assert n == m["n_active"]
    assert np.array_equal(region(abi.WS_ORDER, 4 * E).view(np.int32)[:n], m["order"])
    xrb = abi.q8_1_row_bytes(H)
    assert np.array_equal(region(abi.WS_Q8X, R * xrb).reshape(R, xrb), dbg["q8x"])
    stride = abi.workspace_offset(abi.WS_GROUP_STRIDE, T, H, F, E, K, wtype, 16)
    groups = region(abi.WS_GROUPS, n * stride).reshape(n, stride)
    raw = np.zeros(n * c.expert_bytes, np.uint8)      # the oracle's copy of each position
    orc.gather(c.pool, c.expert_off, m["order"], c.expert_bytes, raw, 0, c.expert_bytes)
    mmq_layout.check_positions(groups, c.wtype, c.H, c.F,
                               [raw[i * c.expert_bytes:(i + 1) * c.expert_bytes]
                                for i in range(n)], 0, stride)
    Dm = region(abi.WS_DM, R * H * 4).view(np.float32).reshape(R, H)
    assert rel_err(Dm, dbg["Dm"]) <= TOL


def test_layer_bit_identical_over_group_size_and_ring_start(orc):
    """Every byte reaches the same place whatever the grouping and wherever the ring walk
    starts: the output is bitwise identical."""
    c = synth.make_case("inv", T=257, H=256, F=256, E=40, K=5, wtype=synth.Q4_1, seed=5,
                        zipf=0.9)
    idx, w = orc.route_topk(c.logits, c.K)
    layer = _layer(c, group_size=16, ring_start=0)
    ref = _run(layer, c, idx, w, group_size=16, ring_start=0)
    for gs, rs in [(1, 0), (5, 7), (16, 39), (3, 20), (16, 1)]:
        got = _run(layer, c, idx, w, group_size=gs, ring_start=rs)
        assert np.array_equal(got, ref), (gs, rs)


def test_layer_token_permutation_equivariance(orc):
    c = synth.make_case("perm", T=200, H=256, F=128, E=16, K=3, wtype=synth.Q8_0, seed=6)
    idx, w = orc.route_topk(c.logits, c.K)
    layer = _layer(c)
    ref = _run(layer, c, idx, w)
    p = np.random.default_rng(1).permutation(c.T)
    c2 = synth.make_case("perm", T=200, H=256, F=128, E=16, K=3, wtype=synth.Q8_0, seed=6)
    c2.x = c.x[p].copy()
    got = _run(layer, c2, idx[p].copy(), w[p].copy())
    assert np.array_equal(got, ref[p])


@pytest.mark.parametrize("edge", ["T1", "K_eq_E", "E1", "one_expert_takes_all", "half_empty",
                                  "max_E_and_K"])
def test_layer_edge_cases(orc, edge):
    T, H, F, E, K, wtype = 50, 256, 128, 8, 2, synth.Q8_0
    if edge == "T1":
        T = 1
    if edge == "max_E_and_K":                 # E = 2048 and K = 64, the largest the ABI takes
        T, H, E, K = 40, 128, 2048, 64
    if edge == "K_eq_E":
        E, K = 6, 6
    if edge == "E1":
        E, K = 1, 1
    c = synth.make_case(edge, T=T, H=H, F=F, E=E, K=K, wtype=wtype, seed=len(edge))
    if edge == "one_expert_takes_all":
        c.logits[:, 5] += 100.0
        K = 1
        c.K = 1
    if edge == "half_empty":
        c.logits[:, :4] -= 100.0
    idx, w = orc.route_topk(c.logits, c.K)
    want = orc.prefill_layer(c.x, idx, w, wtype, c.pool, c.expert_off, F, E)
    layer = _layer(c, ring_start=0)
    got = _run(layer, c, idx, w, ring_start=0)
    assert rel_err(got, want) <= TOL


# Rows per expert that put an expert's last 64-row tile in every case the MMQ launches treat
# apart: each count of live 8-row groups in the first and the second 32-row tile, whole tiles,
# and one row past them; the last four experts receive no rows.
TILE_ROWS = [1, 7, 8, 9, 16, 17, 24, 25, 31, 32, 33, 40, 41, 48, 49, 56, 57, 63, 64, 65, 96, 127,
             128, 129, 0, 0, 0, 0]


@pytest.mark.parametrize("wtype", [synth.Q4_1, synth.Q8_0])
def test_layer_tile_row_counts(orc, wtype):
    """Experts with exactly the row counts above (one expert per token, K = 1), so that every
    partial-tile form of both MMQ launches runs: output and the down projection's rows against
    the oracle."""
    counts = np.array(TILE_ROWS)
    E, T, H, F = len(counts), int(counts.sum()), 256, 256
    c = synth.make_case("tile_rows", T=T, H=H, F=F, E=E, K=1, wtype=wtype, seed=77 + wtype)
    rng = np.random.default_rng(5 + wtype)
    idx = rng.permutation(np.repeat(np.arange(E, dtype=np.int32), counts)).reshape(T, 1)
    w = np.ones((T, 1), np.float32)
    want, dbg = orc.prefill_layer(c.x, idx, w, wtype, c.pool, c.expert_off, F, E, debug=True)
    layer = _layer(c)
    got = _run(layer, c, idx, w)
    assert rel_err(got, want) <= TOL
    ws = host(layer.ws)
    o = abi.workspace_offset(abi.WS_DM, T, H, F, E, 1, wtype, 16)
    Dm = ws[o:o + T * H * 4].view(np.float32).reshape(T, H)
    m = orc.build_maps(idx, E, c.ring_start)
    assert np.array_equal(np.bincount(idx[:, 0], minlength=E), m["counts"])
    for e in range(E):                       # every expert's rows, each within the bound
        r0, r1 = m["offsets"][e], m["offsets"][e + 1]
        if r1 > r0:
            assert rel_err(Dm[r0:r1], dbg["Dm"][r0:r1]) <= TOL, (e, r1 - r0)


def test_layer_step_with_gpu_routing(orc):
    """Routing and the layer in one pass on the GPU (the benchmark's step)."""
    c = synth.make_case("step", T=300, H=512, F=256, E=32, K=4, wtype=synth.Q4_1, seed=8)
    layer = _layer(c)
    note("layer step with routing")
    out = host(layer.step(dev(c.x), dev(c.logits)))
    idx, w = orc.route_topk(c.logits, c.K)
    want = orc.prefill_layer(c.x, idx, w, c.wtype, c.pool, c.expert_off, c.F, c.E)
    assert rel_err(out, want) <= TOL


def test_layer_repeat_is_deterministic(orc):
    c = synth.make_case("rep", T=128, H=256, F=128, E=16, K=4, wtype=synth.Q4_1, seed=9)
    idx, w = orc.route_topk(c.logits, c.K)
    layer = _layer(c)
    a = _run(layer, c, idx, w)
    b = _run(layer, c, idx, w)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("case", [CASES[0], CASES[3], CASES[4], CASES[6]],
                         ids=["tiny", "ragged_q4_1", "skew", "ragged_d4"])
def test_layer_packed_pool_equals_gathered_layer(orc, case):
    """Experts kept in the MMQ layout and read in place (no gather): the packed pool decodes to
    the raw pool, the same bytes reach the matmul, so the output is the gathered layer's bit for
    bit, and within the layer's tolerance of the oracle."""
    name, T, H, F, E, K, wtype, zipf = case
    c = synth.make_case(name, T=T, H=H, F=F, E=E, K=K, wtype=wtype,
                        seed=zlib.crc32(name.encode()) % 10000, zero_tokens=(T // 3,), zipf=zipf)
    idx, w = orc.route_topk(c.logits, K)
    want = orc.prefill_layer(c.x, idx, w, wtype, c.pool, c.expert_off, F, E)
    layer = _layer(c)
    ref = _run(layer, c, idx, w)
    packed = layer.pack_pool()
    # every expert of the packed pool decodes to its raw bytes
    ph = host(packed)
    for e in range(E):
        o = int(c.expert_off[e])
        mmq_layout.check_positions(ph[o:o + c.expert_bytes], wtype, H, F, [c.expert(e)], 0, 0)
    note(f"packed layer {name}")
    for rs in (c.ring_start, 0):
        got = host(layer.forward_packed(dev(c.x), dev(idx), dev(w), ring_start=rs))
        assert np.array_equal(got, ref), rs
        assert rel_err(got, want) <= TOL


def test_layer_step_in_a_hip_graph(orc):
    """Routing + the layer captured in one HIP graph: every replay, with eager work and
    synchronisations between the replays, equals the eager step bit for bit."""
    c = synth.make_case("graph", T=257, H=256, F=128, E=24, K=4, wtype=synth.Q4_1, seed=12,
                        zipf=0.9)
    layer = _layer(c)
    x, logits = dev(c.x), dev(c.logits)
    note("layer step eager, then captured in a graph")
    want = host(layer.step(x, logits))
    out = torch.empty((c.T, c.H), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.step(x, logits, out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.step(x, logits, out)
    for r in range(4):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        got = host(out)
        assert np.array_equal(got, want), r
        # eager work between the replays
        host(layer.step(x, logits))
    idx, w = orc.route_topk(c.logits, c.K)
    assert rel_err(want, orc.prefill_layer(c.x, idx, w, c.wtype, c.pool, c.expert_off, c.F,
                                           c.E)) <= TOL


def test_layer_calls_on_two_streams_overlap(orc):
    """Two layers (own pools and workspaces, different shapes and weight types) stepped on two
    streams at once, three rounds with no synchronisation inside a round: every result equals
    that layer's eager step on the default stream bit for bit (the library keeps no state a
    call could share with another)."""
    ca = synth.make_case("streamA", T=900, H=512, F=256, E=32, K=4, wtype=synth.Q4_1, seed=31)
    cb = synth.make_case("streamB", T=700, H=384, F=384, E=20, K=3, wtype=synth.Q8_0, seed=32,
                         zipf=1.1)
    la, lb = _layer(ca), _layer(cb)
    xa, ga, xb, gb = dev(ca.x), dev(ca.logits), dev(cb.x), dev(cb.logits)
    note("two layers eager, then overlapped on two streams")
    want_a, want_b = host(la.step(xa, ga)), host(lb.step(xb, gb))
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for r in range(3):
        oa = torch.empty((ca.T, ca.H), dtype=torch.float32, device="cuda")
        ob = torch.empty((cb.T, cb.H), dtype=torch.float32, device="cuda")
        sa.wait_stream(torch.cuda.current_stream())
        sb.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(sa):
            la.step(xa, ga, oa)
        with torch.cuda.stream(sb):
            lb.step(xb, gb, ob)
        outs.append((oa, ob))
    torch.cuda.synchronize()
    for r, (oa, ob) in enumerate(outs):
        assert np.array_equal(host(oa), want_a), r
        assert np.array_equal(host(ob), want_b), r
    ia, wa = orc.route_topk(ca.logits, ca.K)
    assert rel_err(want_a, orc.prefill_layer(ca.x, ia, wa, ca.wtype, ca.pool, ca.expert_off,
                                             ca.F, ca.E)) <= TOL
    ib, wb = orc.route_topk(cb.logits, cb.K)
    assert rel_err(want_b, orc.prefill_layer(cb.x, ib, wb, cb.wtype, cb.pool, cb.expert_off,
                                             cb.F, cb.E)) <= TOL


def test_layer_out_of_range_ids_contribute_nothing(orc):
    """Routes naming no real expert (ids -1, E, E + 7): the layer counts them in its workspace's
    status word, every other token's row equals the oracle's for the original routing, and a
    token with such a route equals the oracle with that route's weight set to 0."""
    c = synth.make_case("badids", T=301, H=512, F=256, E=24, K=4, wtype=synth.Q4_1, seed=17,
                        zero_tokens=(9,))
    idx, w = orc.route_topk(c.logits, c.K)
    rng = np.random.default_rng(4)
    bad_t = rng.choice(c.T, 20, replace=False)
    bad = idx.copy()
    bad_k = rng.integers(0, c.K, len(bad_t))
    bad[bad_t, bad_k] = np.array([-1, c.E, c.E + 7])[np.arange(len(bad_t)) % 3]
    bad[bad_t[0], :] = -1                               # one token with no real expert at all
    layer = _layer(c)
    got = _run(layer, c, bad, w)
    n_bad = int(np.sum((bad < 0) | (bad >= c.E)))
    assert int(host(layer.ws_view(abi.WS_STATUS, c.T, 4)).view(np.int32)[0]) == n_bad
    want = orc.prefill_layer(c.x, idx, w, c.wtype, c.pool, c.expert_off, c.F, c.E)
    ok = np.ones(c.T, bool)
    ok[bad_t] = False
    assert rel_err(got[ok], want[ok]) <= TOL
    fixed_i, fixed_w = bad.copy(), w.copy()
    inval = (bad < 0) | (bad >= c.E)
    fixed_i[inval], fixed_w[inval] = 0, 0.0
    want2 = orc.prefill_layer(c.x, fixed_i, fixed_w, c.wtype, c.pool, c.expert_off, c.F, c.E)
    assert rel_err(got, want2) <= TOL
    assert not got[bad_t[0]].any()                      # no real route: an exact zero row
    # the next call with every id in range clears the count and is unaffected
    got3 = _run(layer, c, idx, w)
    assert int(host(layer.ws_view(abi.WS_STATUS, c.T, 4)).view(np.int32)[0]) == 0
    assert rel_err(got3, want) <= TOL


def test_packed_layer_flags_a_misaligned_expert(orc):
    """A packed pool whose expert sits at an offset that is not a multiple of 16 (a caller
    error, refused by pack_pool): the layer skips that expert's tiles, sets the second status
    word, and every token not routed to it equals the oracle."""
    c = synth.make_case("misal", T=200, H=256, F=128, E=12, K=2, wtype=synth.Q4_1, seed=23)
    idx, w = orc.route_topk(c.logits, c.K)
    layer = _layer(c)
    layer.pack_pool()
    bad_e = int(idx[0, 0])
    off = c.expert_off.copy()
    shifted = torch.zeros(layer.pool.numel() + c.expert_bytes + 64, dtype=torch.uint8,
                          device="cuda")
    shifted[:layer.packed.numel()] = layer.packed
    o = int(off[bad_e])
    tail = layer.pool.numel() + 8                      # the expert's packed bytes, moved to +8
    shifted[tail:tail + c.expert_bytes] = layer.packed[o:o + c.expert_bytes]
    off[bad_e] = tail
    layer.packed = shifted
    layer.expert_off = dev(off)
    note("packed layer with one expert at a misaligned offset")
    got = host(layer.forward_packed(dev(c.x), dev(idx), dev(w)))
    st = host(layer.ws_view(abi.WS_STATUS, c.T, 8)).view(np.int32)
    assert st[0] == 0 and st[1] > 0
    want = orc.prefill_layer(c.x, idx, w, c.wtype, c.pool, c.expert_off, c.F, c.E)
    ok = ~np.any(idx == bad_e, axis=1)
    assert ok.sum() > 0 and rel_err(got[ok], want[ok]) <= TOL
    with pytest.raises(ValueError):
        layer.expert_off = dev(off)
        layer.pack_pool()
