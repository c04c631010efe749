"""GPU parity of the streamed walk (moe_prefill_layer_streamed): experts copied from a pinned host
arena through a ring of device slots reach the group buffer as the same bytes and give the same
output as the resident layer (bit for bit, the page's "same output" claim for its walk), and
the oracle's output within the layer's tolerance."""
import zlib

import numpy as np
import pytest
import torch

from gpu_util import dev, host, note, rel_err
from quantized_expert_grouped_amd import abi, synth
from quantized_expert_grouped_amd.layer import MoePrefillLayer

pytestmark = pytest.mark.gpu

TOL = 1e-3


class Streamed:
    """A resident layer (the reference path) and a walk over the same experts."""

    def __init__(self, c, n_slots):
        self.c = c
        self.layer = MoePrefillLayer(c.pool, c.expert_off, c.H, c.F, c.E, c.wtype, c.T, c.K,
                                     group_size=16, ring_start=c.ring_start)
        self.arena = torch.from_numpy(c.pool).pin_memory()
        self.stride = abi.workspace_offset(abi.WS_GROUP_STRIDE, c.T, c.H, c.F, c.E, c.K,
                                           c.wtype, 16)
        self.ring = torch.empty(n_slots * self.stride, dtype=torch.uint8, device="cuda")
        self.walk = abi.Walk(self.ring, n_slots, self.stride)
        self.ws = torch.empty_like(self.layer.ws)

    def resident_ptrs(self, mask):
        base = self.layer.pool.data_ptr()
        return [base + int(self.c.expert_off[e]) if mask[e] else 0 for e in range(self.c.E)]

    def run(self, x, idx, w, mask, group_size, ring_start, flags):
        c = self.c
        note(f"streamed {c.name} T={x.shape[0]} E={c.E} wtype={c.wtype} slots={self.walk.n_slots} "
             f"G={group_size} ring_start={ring_start} flags={flags} resident={int(np.sum(mask))}")
        out = torch.empty((x.shape[0], c.H), dtype=torch.float32, device="cuda")
        abi.prefill_layer_streamed(self.walk, dev(x), dev(idx), dev(w), c.wtype, self.arena,
                                   c.expert_off, self.resident_ptrs(mask), c.F, c.E, group_size,
                                   ring_start, flags, self.ws, out)
        return host(out)

    def reference(self, x, idx, w, group_size, ring_start):
        note(f"resident layer {self.c.name} G={group_size} ring_start={ring_start}")
        return host(self.layer.forward(dev(x), dev(idx), dev(w), group_size=group_size,
                                       ring_start=ring_start))

    def groups(self, ws, T, n):
        c = self.c
        o = abi.workspace_offset(abi.WS_GROUPS, T, c.H, c.F, c.E, c.K, c.wtype, 16)
        return host(ws[o:o + n * self.stride])


CASES = [
    # name, T, H, F, E, K, wtype, zipf
    ("tiny", 7, 256, 128, 16, 2, synth.Q8_0, None),
    ("ragged_q4_1", 301, 512, 256, 24, 4, synth.Q4_1, None),
    ("skew", 403, 256, 384, 48, 3, synth.Q4_1, 1.5),
    ("d4", 120, 256, 128, 20, 3, synth.Q8_0_D4, 0.8),
]

# n_slots, group_size, flags, resident pattern
WALKS = [
    (96, 16, 0, "none"),
    (1, 16, 0, "half"),
    (5, 3, 0, "none"),
    (16, 16, abi.WALK_GATHER_ONE, "none"),
    (3, 7, abi.WALK_NO_SKIP_FLUSH, "third"),
    (2, 16, 0, "all"),
    (96, 16, abi.WALK_MMQ_PER_GROUP, "half"),
]


def _mask(kind, E):
    if kind == "none":
        return np.zeros(E, bool)
    if kind == "all":
        return np.ones(E, bool)
    if kind == "half":
        return np.arange(E) % 2 == 0
    return np.arange(E) % 3 == 1


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_streamed_walk_equals_resident_layer(orc, case):
    name, T, H, F, E, K, wtype, zipf = case
    c = synth.make_case(name, T=T, H=H, F=F, E=E, K=K, wtype=wtype,
                        seed=zlib.crc32(name.encode()) % 10000, zipf=zipf)
    idx, w = orc.route_topk(c.logits, K)
    want = orc.prefill_layer(c.x, idx, w, wtype, c.pool, c.expert_off, F, E)
    m = orc.build_maps(idx, E, c.ring_start)
    n = int(m["n_active"])
    for n_slots, G, flags, res in WALKS:
        s = Streamed(c, n_slots)
        ref = s.reference(c.x, idx, w, G, c.ring_start)
        ref_groups = s.groups(s.layer.ws, T, n)
        mask = _mask(res, E)
        got = s.run(c.x, idx, w, mask, G, c.ring_start, flags)
        assert np.array_equal(got, ref), (n_slots, G, flags, res)
        assert np.array_equal(s.groups(s.ws, T, n), ref_groups), (n_slots, G, flags, res)
        assert rel_err(got, want) <= TOL
        st = s.walk.stats()
        routed = np.flatnonzero(m["counts"] > 0)
        assert st["copies"] == int(np.sum(~mask[routed]))
        assert st["bytes"] == st["copies"] * c.expert_bytes
        assert st["waits"] <= st["batches"] and st["routing_syncs"] == 1
        groups = (n + G - 1) // G
        if flags & abi.WALK_MMQ_PER_GROUP:
            assert st["mmq_launches"] == 2 * groups
        else:  # consecutive groups' MMQs merge unless a batch between them waits for copies
            assert 2 <= st["mmq_launches"] <= 2 * groups
            if res == "all":
                assert st["mmq_launches"] == 2
        if flags & abi.WALK_GATHER_ONE:
            assert st["batches"] == n
        s.walk.close()


def test_streamed_walk_carries_the_ring_across_calls(orc):
    """Three layers in a row through one 4-slot ring with different routings: every refill waits
    for the previous call's readers, and each call equals the resident layer."""
    c = synth.make_case("calls", T=180, H=256, F=256, E=20, K=3, wtype=synth.Q8_0, seed=31,
                        zipf=0.8)
    s = Streamed(c, 4)
    rng = np.random.default_rng(3)
    mask = _mask("third", c.E)
    for call in range(3):
        x = rng.standard_normal((c.T, c.H), dtype=np.float32)
        logits = rng.standard_normal((c.T, c.E), dtype=np.float32)
        idx, w = orc.route_topk(logits, c.K)
        rs = int(rng.integers(c.E))
        ref = s.reference(x, idx, w, 16, rs)
        got = s.run(x, idx, w, mask, 6, rs, 0)
        assert np.array_equal(got, ref), call
    assert s.walk.stats()["routing_syncs"] == 3
    st = s.walk.stats()
    assert 0 <= st["copy_waits"] <= st["copies"]
    s.walk.close()


def test_streamed_walk_full_size_t8k(orc, oracle_cache):
    """T = 8192, H = 2048, F = 512, E = 512, K = 10, Q4_1, every expert streamed through a
    96-slot ring: equal to the resident layer bit for bit, and the whole output within the
    layer's tolerance of the oracle's."""
    c = synth.config_case("t8k")
    s = Streamed(c, 96)
    if c.name not in oracle_cache:
        i0, w0 = orc.route_topk(c.logits, c.K)
        oracle_cache[c.name] = (i0, w0, orc.prefill_layer(c.x, i0, w0, c.wtype, c.pool,
                                                          c.expert_off, c.F, c.E))
    idx, w, want = oracle_cache[c.name]
    ref = s.reference(c.x, idx, w, 16, c.ring_start)
    got = s.run(c.x, idx, w, np.zeros(c.E, bool), 16, c.ring_start, 0)
    assert np.array_equal(got, ref)
    assert rel_err(got, want) <= TOL
    st = s.walk.stats()
    assert st["copies"] == int(np.sum(orc.build_maps(idx, c.E, c.ring_start)["counts"] > 0))
    s.walk.close()


def test_streamed_walk_merges_contiguous_copies(orc):
    """An arena laid out by expert id, slot_stride apart: a batch's consecutive experts go out as
    one transfer when their slots follow each other; the bytes and the output are unchanged."""
    c = synth.make_case("merge", T=300, H=256, F=256, E=40, K=4, wtype=synth.Q4_1, seed=41,
                        zipf=0.7)
    idx, w = orc.route_topk(c.logits, c.K)
    for n_slots, G in [(96, 16), (5, 3), (7, 16), (1, 4)]:
        s = Streamed(c, n_slots)
        by_id = np.zeros(c.E * s.stride, np.uint8)
        for e in range(c.E):
            by_id[e * s.stride:e * s.stride + c.expert_bytes] = c.expert(e)
        s.arena = torch.from_numpy(by_id).pin_memory()
        s.c = synth.Case(**{**c.__dict__, "expert_off": np.arange(c.E, dtype=np.int64) * s.stride})
        ref = s.reference(c.x, idx, w, G, c.ring_start)
        got = s.run(c.x, idx, w, np.zeros(c.E, bool), G, c.ring_start, 0)
        assert np.array_equal(got, ref), (n_slots, G)
        st = s.walk.stats()
        if n_slots == 1:
            assert st["transfers"] == st["copies"]
        else:
            assert st["transfers"] < st["copies"], (n_slots, G, st)
        s.walk.close()


def test_streamed_host_validation():
    c = synth.make_case("val", T=16, H=256, F=128, E=8, K=2, wtype=synth.Q8_0, seed=2)
    s = Streamed(c, 2)
    idx = np.zeros((c.T, c.K), np.int32)
    idx[:, 1] = 1
    w = np.full((c.T, c.K), 0.5, np.float32)
    out = torch.empty((c.T, c.H), dtype=torch.float32, device="cuda")
    args = lambda **kw: dict(dict(walk=s.walk, x=dev(c.x), topk_idx=dev(idx), topk_w=dev(w),
                                  wtype=c.wtype, host_arena=s.arena, host_off=c.expert_off,
                                  resident=[0] * c.E, F=c.F, E=c.E, group_size=16, ring_start=0,
                                  flags=0, ws=s.ws, out=out), **kw)
    small = c.expert_off.max() + c.expert_bytes - 1          # the last expert does not fit
    assert abi.raw_prefill_layer_streamed(**args(arena_bytes=int(small))) == -1
    assert abi.raw_prefill_layer_streamed(**args(host_arena=None)) == -1
    assert abi.raw_prefill_layer_streamed(**args(flags=8)) == -1       # an unknown flag bit
    assert abi.raw_prefill_layer_streamed(**args(group_size=17)) == -1
    assert s.walk.stats()["routing_syncs"] == 0              # nothing was enqueued
    s.walk.close()


SHARE_CASES = [
    # name, T, H, F, E, K, wtype, zipf
    ("share_q8_0", 96, 256, 128, 40, 4, synth.Q8_0, 0.7),
    ("share_q4_1", 150, 512, 256, 48, 3, synth.Q4_1, None),
    ("share_d4", 64, 256, 128, 24, 2, synth.Q8_0_D4, 1.1),
]


@pytest.mark.parametrize("case", SHARE_CASES, ids=[c[0] for c in SHARE_CASES])
def test_streamed_walk_cpu_share(orc, case):
    """The CPU share ("#1282 prefill: STRATA_PREFILL_CPU_SHARE=auto hands a small chunk's
    least-routed experts to the idle CPU pool", "What it does"): the host takes the least-routed
    streamed experts (at most max_tokens tokens each, fewest first), the GPU neither copies nor
    gathers them, the combine weights their rows.  The output is within the layer's tolerance of
    the oracle; a token none of whose routes went to the host equals the resident layer bit for
    bit (its rows are the GPU's)."""
    name, T, H, F, E, K, wtype, zipf = case
    c = synth.make_case(name, T=T, H=H, F=F, E=E, K=K, wtype=wtype,
                        seed=zlib.crc32(name.encode()) % 10000, zipf=zipf, zero_tokens=(5,))
    idx, w = orc.route_topk(c.logits, K)
    want = orc.prefill_layer(c.x, idx, w, wtype, c.pool, c.expert_off, F, E)
    m = orc.build_maps(idx, E, c.ring_start)
    for share, max_tok, n_slots, res in [(0.5, 0, 8, "none"), (1.0, 6, 3, "third"),
                                         (-1.0, 0, 96, "none")]:
        s = Streamed(c, n_slots)
        s.walk.cpu_share(share, max_tok, 4, T, H, T * K)
        ref = s.reference(c.x, idx, w, 16, c.ring_start)
        mask = _mask(res, E)
        prev = None
        for call in range(2 if share < 0 else 1):
            st0 = s.walk.stats()
            got = s.run(c.x, idx, w, mask, 16, c.ring_start, 0)
            last = s.walk.stats()       # share_ppm and the two rates describe the last call
            st = {k: v - st0[k] for k, v in last.items()}
            assert rel_err(got, want) <= TOL, (share, call)
            assert not got[5].any()
            streamed_routed = [e for e in range(E) if m["counts"][e] > 0 and not mask[e]]
            counts = m["counts"]
            order = sorted(streamed_routed, key=lambda e: (counts[e], e))
            eligible = [e for e in order if max_tok == 0 or counts[e] <= max_tok]
            # the host takes share x the streamed experts (the share this call used: fixed, or
            # 0.25 on an automatic walk's first call and g / (c + g) after), least-routed first
            used = last["share_ppm"] / 1e6
            if share > 0:
                assert used == share
            elif call == 0:
                assert used == 0.25
            n_host = min(len(eligible), int(used * len(streamed_routed) + 0.5))
            assert st["host_experts"] == n_host, (share, call, st)
            if share > 0 or call == 0:
                assert n_host > 0
            assert st["copies"] == len(streamed_routed) - n_host
            assert st["host_rows"] == int(sum(counts[e] for e in eligible[:n_host]))
            # tokens not routed to any of the host's experts are the GPU's alone
            host = set(eligible[:n_host])
            clean = ~np.isin(idx, list(host)).any(axis=1)
            assert clean.sum() > 0
            assert np.array_equal(got[clean], ref[clean]), (share, call)
            if share < 0 and call == 1:  # the share came from the rates measured by call 0:
                g = last["gpu_ns_per_expert"]          # the GPU's (its events, read now)
                c = prev["host_ns_per_expert"]         # and the host's (timed in call 0)
                assert g > 0 and c > 0
                assert abs(used - g / (g + c)) < 1e-5
            prev = last
        s.walk.close()


def test_streamed_walk_cpu_share_rejects_shapes_outside_its_buffers(orc):
    c = synth.make_case("share_val", T=40, H=256, F=128, E=12, K=2, wtype=synth.Q8_0, seed=9)
    s = Streamed(c, 4)
    s.walk.cpu_share(0.5, 0, 2, 20, 256, 40)       # T above the share's capacity
    idx, w = orc.route_topk(c.logits, c.K)
    out = torch.empty((c.T, c.H), dtype=torch.float32, device="cuda")
    rc = abi.raw_prefill_layer_streamed(s.walk, dev(c.x), dev(idx), dev(w), c.wtype, s.arena,
                                        c.expert_off, [0] * c.E, c.F, c.E, 16, 0, 0, s.ws, out)
    assert rc == -1
    s.walk.cpu_share(0.0, 0, 0, 0, 0, 0)           # off: the call runs on the GPU alone
    assert abi.raw_prefill_layer_streamed(s.walk, dev(c.x), dev(idx), dev(w), c.wtype, s.arena,
                                          c.expert_off, [0] * c.E, c.F, c.E, 16, 0, 0, s.ws,
                                          out) == 0
    s.walk.close()
