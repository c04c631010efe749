"""GPU parity: the grouped MMQ (a4..a6) through moe_mmq_grouped against the oracle.

Block dots are compared bit for bit; fp32 products within the rounding bound of an fp32
accumulation over the blocks; the SwiGLU epilogue's q8_1 bytes bit for bit against the oracle's
quantiser applied to the kernel's own h, and that h against the oracle's fp64 h."""
import numpy as np
import pytest
import torch

import npref
from gpu_util import dev, empty, gpu_group_buffer, host, note
from quantized_expert_grouped_amd import abi, synth

pytestmark = pytest.mark.gpu


def _setup(orc, wtype, T, H, F, E, K, seed, skew=None):
    c = synth.make_case(T=T, H=H, F=F, E=E, K=K, wtype=wtype, seed=seed, zero_tokens=(1,),
                        zipf=skew)
    idx, _ = orc.route_topk(c.logits, K)
    m = orc.build_maps(idx, E)
    q8x = orc.quantize_scatter(c.x, K, m["slot"], orc.act_layout(wtype))
    # group buffer: positions 0..n-1 hold experts in a shuffled order, in the MMQ layout, as the
    # library's gather writes it (checked against the oracle's copy of the raw experts)
    experts = np.random.default_rng(seed).permutation(E)[:min(E, 16)].astype(np.int32)
    gbuf = gpu_group_buffer(orc, c, experts)
    return c, m, q8x, experts, gbuf


def _abs_term_bound(wtype, wmat, n_out, k_in, act, dots):
    """Sum over blocks of |y_b| per (row, n): scales the fp32 accumulation's rounding error."""
    _, d, mm = npref.unpack_matrix(wmat, n_out, k_in, wtype)
    _, dx, sx = (npref.q8_1_decode_d4 if wtype == synth.Q8_0_D4 else npref.q8_1_decode)(act, k_in)
    t = np.abs(dots.astype(np.float64)) * dx[:, None, :] * d[None, :, :]
    if mm is not None:
        t = t + np.abs(mm[None, :, :] * sx[:, None, :])
    return t.sum(axis=2)


def _d4_scale_bound(wtype, wmat, n_out, k_in, act, dots):
    """D4 only: what the kernel's scale arithmetic moves sum_b y_b, beyond the fp32 accumulation.

    Two terms per block, each at most |I_b| * |dw_b| * max(2^-22 dx_b, 2^-25):
      - representation: dx enters as hi + lo = fp16(dx) + fp16(dx - fp16(dx)); the remainder is
        at most 2^-11 dx and lo rounds it to 2^-11 of itself, or to half fp16's smallest
        subnormal (2^-25), so |dx - (hi + lo)| <= max(2^-22 dx, 2^-25);
      - the MFMA's sum of the two exact fp32 products hi*dw + lo*dw: one rounding, at most
        2^-24 |(hi + lo) dw| <= 2^-23 dx |dw|, within the same max.
    Hence the factor 2."""
    if wtype != synth.Q8_0_D4:
        return 0.0
    _, d, _ = npref.unpack_matrix(wmat, n_out, k_in, wtype)
    _, dx, _ = npref.q8_1_decode_d4(act, k_in)
    e = np.maximum(dx * 2.0 ** -22, 2.0 ** -25)
    return 2 * (np.abs(dots.astype(np.float64)) * e[:, None, :] * np.abs(d)[None, :, :]).sum(axis=2)


@pytest.mark.parametrize("wtype", [synth.Q8_0, synth.Q4_1, synth.Q8_0_D4])
@pytest.mark.parametrize("shape", [(150, 512, 256, 12, 3, None), (700, 256, 128, 16, 2, 1.5),
                                   (90, 384, 384, 10, 3, None)])      # three stages each
def test_mmq_block_dots_bit_exact(orc, wtype, shape):
    T, H, F, E, K, skew = shape
    c, m, q8x, experts, gbuf = _setup(orc, wtype, T, H, F, E, K, seed=T + wtype, skew=skew)
    R = T * K
    out = torch.zeros((R, 2 * F, H // 32), dtype=torch.int32, device="cuda")
    note(f"mmq i32 wtype={wtype} shape={shape}")
    abi.mmq_grouped(wtype, gbuf, c.expert_stride, 0, 2 * F, H, experts, dev(m["offsets"]),
                    E, dev(q8x), abi.EPI_I32_BLOCKDOTS, out)
    got = host(out)
    gu = 2 * F * (H // 32) * synth.BLOCK_BYTES[wtype]
    for j, e in enumerate(experts):
        r0, r1 = m["offsets"][e], m["offsets"][e + 1]
        if r1 == r0:
            continue
        wmat = c.expert(e)[:gu]          # the raw matrices (the group buffer is repacked)
        want = orc.block_dots(wtype, wmat, 2 * F, H, q8x[r0:r1])
        assert np.array_equal(got[r0:r1], want), (j, e)
    # rows of experts outside the group stay untouched
    in_group = np.zeros(R, bool)
    for e in experts:
        in_group[m["offsets"][e]:m["offsets"][e + 1]] = True
    assert not got[~in_group].any()


@pytest.mark.parametrize("wtype", [synth.Q8_0, synth.Q4_1, synth.Q8_0_D4])
@pytest.mark.parametrize("shape", [(150, 512, 256, 12, 3, None), (1300, 256, 128, 4, 1, 3.0),
                                   (90, 384, 384, 10, 3, None)])
def test_mmq_down_f32(orc, wtype, shape):
    """The down projection's fp32 rows (n_out = H, k_in = F) on random q8_1 rows of h."""
    T, H, F, E, K, skew = shape
    c, m, _, experts, gbuf = _setup(orc, wtype, T, H, F, E, K, seed=3 * T + wtype, skew=skew)
    R = T * K
    rng = np.random.default_rng(5)
    hq8 = orc.q8_1_rows((rng.standard_normal((R, F)) * 0.3).astype(np.float32), orc.act_layout(wtype))
    mat_off = 2 * F * (H // 32) * synth.BLOCK_BYTES[wtype]
    out = torch.zeros((R, H), dtype=torch.float32, device="cuda")
    note(f"mmq f32 wtype={wtype} shape={shape}")
    abi.mmq_grouped(wtype, gbuf, c.expert_stride, mat_off, H, F, experts, dev(m["offsets"]),
                    E, dev(hq8), abi.EPI_F32, out)
    got = host(out)
    nb = F // 32
    for j, e in enumerate(experts):
        r0, r1 = m["offsets"][e], m["offsets"][e + 1]
        if r1 == r0:
            continue
        wmat = c.expert(e)[mat_off:mat_off + H * nb * synth.BLOCK_BYTES[wtype]]
        want = orc.matrix_rows(wtype, wmat, H, F, hq8[r0:r1])
        dots = orc.block_dots(wtype, wmat, H, F, hq8[r0:r1])
        bound = _abs_term_bound(wtype, wmat, H, F, hq8[r0:r1], dots) * (nb + 2) * 2.0 ** -23
        bound = bound + _d4_scale_bound(wtype, wmat, H, F, hq8[r0:r1], dots)
        assert np.all(np.abs(got[r0:r1] - want) <= bound + 1e-30), (j, e)


@pytest.mark.parametrize("wtype", [synth.Q8_0, synth.Q4_1, synth.Q8_0_D4])
def test_mmq_swiglu_q8_1(orc, wtype):
    T, H, F, E, K = 150, 512, 256, 12, 3
    c, m, q8x, experts, gbuf = _setup(orc, wtype, T, H, F, E, K, seed=11 + wtype)
    R = T * K
    hq = torch.zeros((R, abi.q8_1_row_bytes(F)), dtype=torch.uint8, device="cuda")
    dh = torch.zeros((R, F), dtype=torch.float32, device="cuda")
    note(f"mmq swiglu wtype={wtype}")
    abi.mmq_grouped(wtype, gbuf, c.expert_stride, 0, F, H, experts, dev(m["offsets"]), E,
                    dev(q8x), abi.EPI_SWIGLU_Q8_1, hq, dh)
    got_hq, got_h = host(hq), host(dh)
    gu_bytes = F * (H // 32) * synth.BLOCK_BYTES[wtype]
    checked = 0
    for j, e in enumerate(experts):
        r0, r1 = m["offsets"][e], m["offsets"][e + 1]
        if r1 == r0:
            continue
        g = orc.matrix_rows(wtype, c.expert(e)[:gu_bytes], F, H, q8x[r0:r1])
        u = orc.matrix_rows(wtype, c.expert(e)[gu_bytes:2 * gu_bytes], F, H, q8x[r0:r1])
        h = g / (1.0 + np.exp(-g)) * u
        # the kernel's h: fp32 accumulation of the same products
        assert np.max(np.abs(got_h[r0:r1] - h)) <= 1e-5 * max(np.max(np.abs(h)), 1e-30)
        # its q8_1 bytes are exactly the quantiser's bytes of that h
        assert np.array_equal(got_hq[r0:r1], orc.q8_1_rows(got_h[r0:r1], orc.act_layout(wtype)))
        checked += r1 - r0
    assert checked > 0


def test_mmq_group_position_independence(orc):
    """The same expert at another group position and another set of neighbours gives the same
    bytes (the products do not depend on the group)."""
    wtype, T, H, F, E, K = synth.Q4_1, 200, 256, 128, 10, 2
    c, m, q8x, experts, gbuf = _setup(orc, wtype, T, H, F, E, K, seed=99)
    R = T * K
    outs = []
    for perm_seed in (0, 1):
        perm = np.random.default_rng(perm_seed).permutation(len(experts))
        ex2 = experts[perm]
        gb2 = gpu_group_buffer(orc, c, ex2)
        out = torch.zeros((R, abi.q8_1_row_bytes(F)), dtype=torch.uint8, device="cuda")
        note(f"mmq position permutation {perm_seed}")
        abi.mmq_grouped(wtype, gb2, c.expert_stride, 0, F, H, ex2, dev(m["offsets"]), E,
                        dev(q8x), abi.EPI_SWIGLU_Q8_1, out)
        outs.append(host(out))
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("wtype", [synth.Q8_0, synth.Q4_1])
def test_mmq_down_subnormal_scales(orc, wtype):
    """Activation rows whose q8_1 scales are fp16 subnormals (|h| ~ 1e-3): the scale products
    must keep them (no flush to zero)."""
    T, H, F, E, K = 120, 256, 128, 4, 2
    c, m, _, experts, gbuf = _setup(orc, wtype, T, H, F, E, K, seed=41 + wtype)
    R = T * K
    rng = np.random.default_rng(6)
    h = (rng.standard_normal((R, F)) * 1e-3).astype(np.float32)   # d = amax/127 ~ 2e-5
    h[::3] *= np.float32(1e-2)
    hq8 = orc.q8_1_rows(h)
    _, dx, _ = npref.q8_1_decode(hq8, F)
    assert np.mean((dx > 0) & (dx < 2.0 ** -14)) > 0.5        # mostly subnormal scales
    mat_off = 2 * F * (H // 32) * synth.BLOCK_BYTES[wtype]
    out = torch.zeros((R, H), dtype=torch.float32, device="cuda")
    note(f"mmq f32 subnormal scales wtype={wtype}")
    abi.mmq_grouped(wtype, gbuf, c.expert_stride, mat_off, H, F, experts, dev(m["offsets"]),
                    E, dev(hq8), abi.EPI_F32, out)
    got = host(out)
    nb = F // 32
    for j, e in enumerate(experts):
        r0, r1 = m["offsets"][e], m["offsets"][e + 1]
        if r1 == r0:
            continue
        wmat = c.expert(e)[mat_off:mat_off + H * nb * synth.BLOCK_BYTES[wtype]]
        want = orc.matrix_rows(wtype, wmat, H, F, hq8[r0:r1])
        dots = orc.block_dots(wtype, wmat, H, F, hq8[r0:r1])
        bound = _abs_term_bound(wtype, wmat, H, F, hq8[r0:r1], dots) * (nb + 2) * 2.0 ** -23
        assert np.all(np.abs(got[r0:r1] - want) <= bound + 1e-38), (j, e)
        assert np.count_nonzero(got[r0:r1]) > 0.9 * got[r0:r1].size
