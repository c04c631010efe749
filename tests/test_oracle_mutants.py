"""The pins catch plausible mistakes: each mutant below plants one mistake in a temporary copy
of the oracle's C source, builds it with gcc, and must fail at least one pin (CPU only)."""
import importlib.util
import os
import subprocess

import numpy as np
import pytest

import test_oracle_formats as tf
import test_oracle_gather_dot as tg
import test_oracle_layer as tl
import test_oracle_q8_1 as tq
import test_oracle_route_maps as tr
from quantized_expert_grouped_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")
INIT = os.path.join(ROOT, "oracle", "__init__.py")

MUTANTS = {
    "gate_up_swapped": ("const uint8_t *up = expert + (size_t)F * gu_row;",
                        "const uint8_t *up = expert; gate = expert + (size_t)F * gu_row;"),
    "q4_1_min_term_dropped": ("if (wtype == ORC_Q4_1) y += orc_f16_to_f64(rd16(blk + 2)) * sx;",
                              "(void)sx;"),
    "round_half_even": ("float r = roundf(v[j] / d);", "float r = rintf(v[j] / d);"),
    "reciprocal_multiply": ("float r = roundf(v[j] / d);", "float r = roundf(v[j] * (127.0f / amax));"),
    "nibbles_swapped": ("I += (int32_t)(qs[j] & 15) * (int32_t)xq[j];\n            I += (int32_t)(qs[j] >> 4) * (int32_t)xq[j + 16];",
                        "I += (int32_t)(qs[j] >> 4) * (int32_t)xq[j];\n            I += (int32_t)(qs[j] & 15) * (int32_t)xq[j + 16];"),
    "silu_sign": ("h[f] = (float)(g / (1.0 + exp(-g)) * u);", "h[f] = (float)(g / (1.0 + exp(g)) * u);"),
    "combine_row_index": ("Dm[(size_t)slot[(size_t)t * K + k] * H + i];", "Dm[((size_t)t * K + k) * H + i];"),
    "s_from_fp16_d": ("*s16 = orc_f32_to_f16(d * (float)S);",
                      "*s16 = orc_f32_to_f16((float)orc_f16_to_f64(orc_f32_to_f16(d)) * (float)S);"),
    "route_tie_higher_id": ("if (best < 0 || l[e] > l[best]) best = e;", "if (best < 0 || l[e] >= l[best]) best = e;"),
    "maps_unstable": ("for (int i = 0; i < R; ++i) {\n        int e = idx[i];",
                      "for (int i = R - 1; i >= 0; --i) {\n        int e = idx[i];"),
    "ring_ignored": ("int e = (ring_start + j) % E;", "int e = j; (void)ring_start;"),
    "ds_header_swapped": ("wr16(grp + 4 * j, d16);\n            wr16(grp + 4 * j + 2, s16);",
                          "wr16(grp + 4 * j, s16);\n            wr16(grp + 4 * j + 2, d16);"),
    "f16_ties_away": ("double m = nearbyint(a * ldexp(1.0, 10 - E));", "double m = floor(a * ldexp(1.0, 10 - E) + 0.5);"),
    "weights_not_renormalised": ("for (int k = 0; k < K; ++k) w[(size_t)t * K + k] = (float)(ex[k] / sum);",
                                 "for (int k = 0; k < K; ++k) w[(size_t)t * K + k] = (float)(ex[k] / (sum + 1.0));"),
    "gather_position_ignores_first": ("memcpy(group_buf + (size_t)(first_pos + j) * pos_stride,",
                                      "memcpy(group_buf + (size_t)j * pos_stride,"),
    "down_at_up_offset": ("const uint8_t *down = expert + (size_t)2 * F * gu_row;",
                          "const uint8_t *down = expert + (size_t)F * gu_row;"),
    "scatter_first_row_only": ("        for (int k = 1; k < K; ++k)\n            memcpy(q8 + (size_t)slot[(size_t)t * K + k] * rb, row, rb);",
                               "        for (int k = 1; k < 1; ++k)\n            memcpy(q8 + (size_t)slot[(size_t)t * K + k] * rb, row, rb);"),
    "combine_unweighted": ("acc += (double)w[(size_t)t * K + k] * Dm[(size_t)slot[(size_t)t * K + k] * H + i];",
                           "acc += Dm[(size_t)slot[(size_t)t * K + k] * H + i];"),
    "silu_dropped": ("h[f] = (float)(g / (1.0 + exp(-g)) * u);", "h[f] = (float)(g * u);"),
    "d4_header_fp16": ("memcpy(grp + 4 * j, &d, 4);",
                       "{ float dr = (float)orc_f16_to_f64(orc_f32_to_f16(d)); memcpy(grp + 4 * j, &dr, 4); }"),
    "d4_q_from_fp16_d": ("for (int i = 0; i < 32; ++i) q[i] = amax == 0.0f ? 0 : (int8_t)(int)roundf(b[i] / d);",
                         "for (int i = 0; i < 32; ++i) q[i] = amax == 0.0f ? 0 : (int8_t)(int)roundf(b[i] / (float)orc_f16_to_f64(orc_f32_to_f16(d)));"),
    "d4_dx_read_as_fp16": ("            dx = (double)d32;", "            dx = orc_f16_to_f64(rd16(grp + 4 * (b % 4)));"),
    "d4_h_requantised_ds4": ("q8_1_row_layout(wtype == ORC_Q8_0_D4 ? ORC_D4 : ORC_DS4, h, F, hq8);",
                             "q8_1_row_layout(ORC_DS4, h, F, hq8);"),
}


def _pins(orc):
    """Every oracle pin, called with the given oracle module."""
    W = (synth.Q8_0, synth.Q4_1)
    yield lambda: tf.test_f32_to_f16_every_boundary_and_midpoint(orc)
    yield lambda: tq.test_closed_form_power_of_two_scale(orc)
    yield lambda: tq.test_block_against_numpy_quantiser(orc)
    yield lambda: tq.test_golden_rows(orc)
    yield lambda: tq.test_row_layout_against_numpy(orc, 256)
    yield lambda: tq.test_scatter_equals_gather(orc, 7)
    yield lambda: tq.test_d4_rows_against_numpy(orc, 128)
    yield lambda: tq.test_scatter_equals_gather_d4(orc, 7)
    yield lambda: tr.test_route_against_stable_sort(orc, 7, 16, 2)
    yield lambda: tr.test_route_weight_closed_forms(orc)
    yield lambda: tr.test_maps_against_brute_force(orc, 64, 4, 32, 31)
    yield lambda: tg.test_gather_is_per_expert_copy(orc)
    for w in W:
        yield lambda w=w: tg.test_block_idot_against_unpacked_integers(orc, w)
        yield lambda w=w: tg.test_row_dot_against_dequantised_fp64(orc, w)
        yield lambda w=w: tl.test_dense_special_case(orc, w)
        yield lambda w=w: tl.test_tiny_layer_against_numpy(orc, w)
    yield lambda: tl.test_combine_closed_forms(orc)
    yield lambda: tg.test_row_dot_against_dequantised_fp64(orc, synth.Q8_0_D4)
    yield lambda: tl.test_dense_special_case(orc, synth.Q8_0_D4)


def _build_variant(tmp_path, name, before, after):
    src = open(SRC).read()
    assert src.count(before) == 1, f"mutation site for {name} not found exactly once"
    d = tmp_path / name
    d.mkdir()
    (d / "moe_oracle.c").write_text(src.replace(before, after))
    (d / "moe_oracle.h").write_text(open(os.path.join(ROOT, "oracle", "moe_oracle.h")).read())
    so = d / "liboracle.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    str(d / "moe_oracle.c"), "-o", str(so), "-lm"], check=True)
    spec = importlib.util.spec_from_file_location(f"oracle_mutant_{name}", INIT)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod._SRC = str(d / "moe_oracle.c")
    mod._LIB = str(so)
    mod._lib = None
    os.utime(so)
    return mod


def test_unmutated_copy_passes_every_pin(tmp_path):
    mod = _build_variant(tmp_path, "none", "#include <math.h>", "#include <math.h>")
    for pin in _pins(mod):
        pin()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    before, after = MUTANTS[name]
    mod = _build_variant(tmp_path, name, before, after)
    for pin in _pins(mod):
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            return
    pytest.fail(f"no pin caught the planted mistake '{name}'")
