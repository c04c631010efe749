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


def _near_half_integer_rows(T: int, H: int, seed: int) -> np.ndarray:
    """Rows whose blocks put v / d on, or within a few ulps of, a half-integer (d = amax / 127 is
    known in advance: each block holds its amax).  Block kinds: d a power of two (exact ties);
    (j + 0.5) d moved by 0..4096 ulps; and, on every third token, values 1e-4..3e-4 away from a
    half-integer (close, yet outside the band where the reciprocal product is not trusted), so
    that whole wavefronts take the fast rounding near its edge."""
    rng = np.random.default_rng(seed)
    nb = H // 32
    x = np.empty((T, nb, 32), np.float32)
    ulps = np.array([0, 1, -1, 2, -2, 3, -3, 4, -4, 6, -6, 8, -8, 16, -16, 64, -64, 256, -256,
                     1024, -1024, 4096, -4096], np.int32)
    for t in range(T):
        for b in range(nb):
            tie = t % 3 != 2 and (t * nb + b) % 8 == 0
            am = np.float32(127.0 * 2.0 ** int(rng.integers(-20, 4)) if tie
                            else rng.uniform(0.01, 100.0))
            d = am / np.float32(127.0)
            j = rng.integers(-127, 127, 31).astype(np.float64)
            if t % 3 == 2:
                delta = rng.uniform(1e-4, 3e-4, 31) * rng.choice([-1.0, 1.0], 31)
                v = ((j + 0.5 + delta) * np.float64(d)).astype(np.float32)
            else:
                v = (j + 0.5).astype(np.float32) * d
                if not tie:
                    v = (v.view(np.int32) + ulps[rng.integers(0, len(ulps), 31)]).view(np.float32)
            x[t, b, 0] = am if rng.integers(0, 2) else -am
            x[t, b, 1:] = v
            x[t, b] = x[t, b, rng.permutation(32)]
    return x.reshape(T, H)


def test_quantize_near_half_integer_quotients(orc):
    """q = roundf(v / d) where v / d sits on or next to a half-integer (a reciprocal product alone
    rounds thousands of these values the other way), exact ties (away from zero), and scales
    near the bottom of the float range (d = 2^-125, the smallest taken through the reciprocal;
    d = 2^-126 and subnormal d, which are not): both forms and both layouts against the
    oracle's bytes."""
    T, H, K, E = 48, 1024, 2, 16
    x = _near_half_integer_rows(T, H, seed=77)
    x[4, :32] *= np.float32(2.0 ** -125) * np.float32(127.0) / np.max(np.abs(x[4, :32]))
    x[4, 32:64] *= np.float32(2.0 ** -126) * np.float32(127.0) / np.max(np.abs(x[4, 32:64]))
    x[4, 64:96] *= np.float32(1e-37) / np.max(np.abs(x[4, 64:96]))     # d subnormal
    x[4, 96:128] *= np.float32(3e-39) / np.max(np.abs(x[4, 96:128]))   # amax subnormal
    rng = np.random.default_rng(78)
    idx, _ = orc.route_topk(rng.standard_normal((T, E)).astype(np.float32), K)
    m = orc.build_maps(idx, E)
    for layout, flag in ((orc.DS4, 0), (orc.D4, abi.QUANT_D4)):
        want = orc.quantize_scatter(x, K, m["slot"], layout)
        for form in (0, abi.QUANT_PER_ROW):
            note(f"quantize near half-integers layout={layout} form={form}")
            assert np.array_equal(gpu_quantize(x, K, m["slot"], m["src"], flag | form), want)


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
