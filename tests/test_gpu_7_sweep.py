"""A seeded sweep of the whole layer over mixed shapes, weight types, group sizes and ring
starts: each case against the oracle (the layer's tolerance), its maps and q8_1 rows bit for
bit, and its output bit for bit against the same layer at group size 16 (the pages' claim that
the grouping does not change the output).  Expert row counts land on every residue of the
MMQ's 64-row tiles and 8-row groups, and H and F on odd and even stage counts."""
import numpy as np
import pytest

from gpu_util import dev, host, note, rel_err
from quantized_expert_grouped_amd import abi, synth
from quantized_expert_grouped_amd.layer import MoePrefillLayer

pytestmark = pytest.mark.gpu

TOL = 1e-3


def _cases(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        wtype = [synth.Q8_0, synth.Q4_1, synth.Q8_0_D4][i % 3]
        H = int(rng.choice([128, 256, 384, 640]))
        F = int(rng.choice([128, 256, 384]))
        E = int(rng.integers(1, 70))
        K = int(rng.integers(1, min(E, 12) + 1))
        T = int(rng.integers(1, 400))
        G = int(rng.integers(1, 17))
        zipf = [None, 0.8, 1.5][i % 3 if E > 2 else 0]
        out.append((f"sweep{i}", T, H, F, E, K, wtype, G, zipf, int(rng.integers(10000))))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_layer_sweep(orc, case):
    name, T, H, F, E, K, wtype, G, zipf, seed = case
    c = synth.make_case(name, T=T, H=H, F=F, E=E, K=K, wtype=wtype, seed=seed, zipf=zipf)
    note(f"sweep {name} T={T} H={H} F={F} E={E} K={K} wtype={wtype} G={G} "
         f"ring_start={c.ring_start} zipf={zipf}")
    idx, w = orc.route_topk(c.logits, K)
    want = orc.prefill_layer(c.x, idx, w, wtype, c.pool, c.expert_off, F, E)
    layer = MoePrefillLayer(c.pool, c.expert_off, H, F, E, wtype, T, K, group_size=G,
                            ring_start=c.ring_start)
    got = host(layer.forward(dev(c.x), dev(idx), dev(w)))
    assert rel_err(got, want) <= TOL
    m = orc.build_maps(idx, E, c.ring_start)
    R = T * K
    ws = host(layer.ws)

    def region(which, nbytes):
        o = abi.workspace_offset(which, T, H, F, E, K, wtype, G)
        return ws[o:o + nbytes]

    assert np.array_equal(region(abi.WS_SLOT, 4 * R).view(np.int32), m["slot"])
    xrb = abi.q8_1_row_bytes(H)
    want_q8 = orc.q8_1_rows(c.x, orc.act_layout(wtype))
    q8 = region(abi.WS_Q8X, R * xrb).reshape(R, xrb)
    assert np.array_equal(q8[m["slot"]], np.repeat(want_q8, K, axis=0))
    # the same routing through groups of 16 and ring start 0: the same bytes out
    ref = host(layer.forward(dev(c.x), dev(idx), dev(w), group_size=16, ring_start=0))
    assert np.array_equal(got, ref)
