"""GPU parity: q8_1 quantise-scatter (a2) and the group gather (a3), byte for byte."""
import numpy as np
import pytest
import torch

import mmq_layout
from gpu_util import dev, empty, gpu_quantize, host, note
from quantized_expert_grouped_amd import abi, synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,H,K,E", [(1, 256, 10, 512), (2, 256, 10, 512), (7, 256, 2, 16),
                                     (600, 2048, 10, 512), (2099, 1152, 10, 512),
                                     (97, 128, 64, 64), (300, 3200, 3, 8)])
def test_quantize_both_modes_bit_exact(orc, T, H, K, E):
    """The page's identity (scatter == per-row gather, T = 1, 2, 7, 600, 2099, 10 of 512
    experts, one all-zero token) and both equal to the oracle's bytes."""
    note(f"quantize T={T} H={H} K={K}")
    rng = np.random.default_rng(T * H + K)
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[T // 2] = 0.0
    if T > 3:
        x[1] *= np.float32(1e-30)          # tiny values: fp16 subnormal / zero scales
        x[2, :64] = np.round(x[2, :64] * 4) / 4
    idx, _ = orc.route_topk(rng.standard_normal((T, E)).astype(np.float32), K)
    m = orc.build_maps(idx, E)
    want = orc.quantize_scatter(x, K, m["slot"])
    g0 = gpu_quantize(x, K, m["slot"], m["src"], 0)
    g1 = gpu_quantize(x, K, m["slot"], m["src"], 1)
    assert np.array_equal(g0, want)
    assert np.array_equal(g1, want)


@pytest.mark.parametrize("T,H,K,E", [(1, 256, 10, 512), (7, 256, 2, 16), (600, 2048, 10, 512),
                                     (2099, 1152, 10, 512)])
def test_quantize_d4_both_modes_bit_exact(orc, T, H, K, E):
    """The same identity for the D4 layout (fp32 d per block, the layout the page names for
    Q8_0), both forms against the oracle's bytes."""
    note(f"quantize D4 T={T} H={H} K={K}")
    rng = np.random.default_rng(T * H + K + 1)
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[T // 2] = 0.0
    if T > 3:
        x[1] *= np.float32(1e-30)
        x[2, :64] = np.round(x[2, :64] * 4) / 4
    idx, _ = orc.route_topk(rng.standard_normal((T, E)).astype(np.float32), K)
    m = orc.build_maps(idx, E)
    want = orc.quantize_scatter(x, K, m["slot"], orc.D4)
    g0 = gpu_quantize(x, K, m["slot"], m["src"], abi.QUANT_D4)
    g1 = gpu_quantize(x, K, m["slot"], m["src"], abi.QUANT_D4 | abi.QUANT_PER_ROW)
    assert np.array_equal(g0, want)
    assert np.array_equal(g1, want)


def test_quantize_full_t32k_sampled(orc):
    """T = 32768, H = 2048, K = 10 (input larger than the on-chip cache): the whole buffer in both
    modes is compared byte for byte with the oracle on 512 sampled tokens' rows, and the two modes
    with each other everywhere."""
    T, H, K, E = 32768, 2048, 10, 512
    rng = np.random.default_rng(1004)
    x = rng.standard_normal((T, H)).astype(np.float32)
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    m = orc.build_maps(idx, E)
    note("quantize T=32768 both modes")
    g0 = gpu_quantize(x, K, m["slot"], m["src"], 0)
    g1 = gpu_quantize(x, K, m["slot"], m["src"], 1)
    assert np.array_equal(g0, g1)
    ts = rng.choice(T, 512, replace=False)
    rows = orc.q8_1_rows(x[ts])
    for j, t in enumerate(ts):
        for k in range(K):
            assert np.array_equal(g0[m["slot"][t * K + k]], rows[j])


@pytest.mark.parametrize("eb,stride,misalign", [(104448, 104448, 0), (3342336, 3342336, 0),
                                                (1000 + 7, 1024, 0), (4096, 4352, 3),
                                                (1966080, 1966080 + 256, 0)])
def test_gather_group_bytes(eb, stride, misalign):
    """Batches of 1..16 experts at every start position, byte for byte the per-expert copies;
    odd sizes and misaligned sources take the fallback and land the same bytes."""
    rng = np.random.default_rng(eb % 1000 + misalign)
    E = 20
    slot = ((eb + 255) // 256) * 256 + 64
    pool = rng.integers(0, 256, E * slot + 64, dtype=np.uint8)
    d_pool = dev(pool)
    base = d_pool.data_ptr()
    off = rng.permutation(E) * slot + misalign
    buf = torch.empty(16 * stride, dtype=torch.uint8, device="cuda")
    cases = [(n, f) for n in (1, 2, 5, 15, 16) for f in sorted({0, (16 - n) // 2, 16 - n})]
    if eb > 10 ** 6:
        cases = [(16, 0), (7, 9), (1, 15)]
    for n, first in cases:
        note(f"gather eb={eb} n={n} first={first} misalign={misalign}")
        experts = rng.choice(E, n, replace=False)
        buf.fill_(0xAB)
        abi.gather_group([base + int(off[e]) for e in experts], eb, buf, first, stride)
        got = host(buf)
        want = np.full(16 * stride, 0xAB, np.uint8)
        for j, e in enumerate(experts):
            want[(first + j) * stride:(first + j) * stride + eb] = pool[off[e]:off[e] + eb]
        assert np.array_equal(got, want), (n, first)


def test_gather_batch_equals_per_expert_launches():
    """One launch for a group equals sixteen one-expert launches, byte for byte."""
    c = synth.make_case(T=4, H=256, F=128, E=16, K=2, wtype=synth.Q4_1, seed=77)
    d_pool = dev(c.pool)
    ptrs = [d_pool.data_ptr() + int(o) for o in c.expert_off]
    a = torch.zeros(16 * c.expert_stride, dtype=torch.uint8, device="cuda")
    b = torch.zeros_like(a)
    note("gather batch vs per expert")
    abi.gather_group(ptrs, c.expert_bytes, a, 0, c.expert_stride)
    for j in range(16):
        abi.gather_group([ptrs[j]], c.expert_bytes, b, j, c.expert_stride)
    assert torch.equal(a, b)


@pytest.mark.parametrize("wtype,H,F,misalign", [(synth.Q4_1, 256, 128, 0), (synth.Q8_0, 256, 128, 0),
                                                (synth.Q8_0, 256, 128, 8), (synth.Q4_1, 256, 128, 8),
                                                (synth.Q4_1, 384, 256, 3), (synth.Q8_0, 2048, 512, 0),
                                                (synth.Q4_1, 2048, 512, 0)])
def test_gather_group_mmq_bytes(orc, wtype, H, F, misalign):
    """The MMQ-layout gather, decoded, against the oracle's verbatim copy of the raw experts,
    byte for byte: batches of 1..16 at several start positions, every byte outside the
    positions untouched; sources 8-byte (Q4_1) or 1-byte aligned take the byte-wise path."""
    rng = np.random.default_rng(H + F + misalign + 10 * wtype)
    eb = abi.expert_bytes(H, F, wtype)
    E = 18
    slot = ((eb + 255) // 256) * 256 + 64
    pool = rng.integers(0, 256, E * slot + 64, dtype=np.uint8)
    d_pool = dev(pool)
    base = d_pool.data_ptr()
    off = (rng.permutation(E) * slot + misalign).astype(np.int64)
    stride = ((eb + 255) // 256) * 256
    buf = torch.empty(16 * stride, dtype=torch.uint8, device="cuda")
    cases = [(1, 0), (3, 13), (16, 0), (7, 4)] if eb < 10 ** 6 else [(16, 0), (2, 14)]
    for n, first in cases:
        note(f"gather_mmq wtype={wtype} H={H} F={F} n={n} first={first} misalign={misalign}")
        experts = rng.choice(E, n, replace=False).astype(np.int32)
        buf.fill_(0xAB)
        abi.gather_group_mmq([base + int(off[e]) for e in experts], wtype, H, F, buf, first, stride)
        got = host(buf)
        raw = np.zeros(n * eb, np.uint8)
        orc.gather(pool, off, experts, eb, raw, 0, eb)
        mmq_layout.check_positions(got, wtype, H, F, [raw[j * eb:(j + 1) * eb] for j in range(n)],
                                   first, stride, fill=0xAB)


def test_gather_mmq_batch_equals_per_expert_launches():
    """One MMQ-layout launch for a group equals sixteen one-expert launches, byte for byte."""
    c = synth.make_case(T=4, H=256, F=128, E=16, K=2, wtype=synth.Q8_0, seed=78)
    d_pool = dev(c.pool)
    ptrs = [d_pool.data_ptr() + int(o) for o in c.expert_off]
    a = torch.zeros(16 * c.expert_stride, dtype=torch.uint8, device="cuda")
    b = torch.zeros_like(a)
    note("gather_mmq batch vs per expert")
    abi.gather_group_mmq(ptrs, c.wtype, c.H, c.F, a, 0, c.expert_stride)
    for j in range(16):
        abi.gather_group_mmq([ptrs[j]], c.wtype, c.H, c.F, b, j, c.expert_stride)
    assert torch.equal(a, b)
