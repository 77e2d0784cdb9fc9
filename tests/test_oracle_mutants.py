"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a private copy of ``oracle/dc1d_oracle.c``
(a dropped term, a wrong sign or index, a transposed operand, a wrong
rounding), builds it on the CPU into a temporary directory, points the
oracle front end at that build, and runs the pins of
``test_oracle_pins.py``: at least one must fail.  The real oracle is never
modified.  CPU only.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
import test_oracle_backward as bwd
import test_oracle_packed as pk
import test_oracle_2d as o2
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "dc1d_oracle.c")

MUTANTS = {
    "lerp weights swapped": ("double v = (1.0 - f) * x_ext(row, L_in, i0) + f * x_ext(row, L_in, i0 + 1);",
                             "double v = f * x_ext(row, L_in, i0) + (1.0 - f) * x_ext(row, L_in, i0 + 1);"),
    "right neighbour dropped": ("double v = (1.0 - f) * x_ext(row, L_in, i0) + f * x_ext(row, L_in, i0 + 1);",
                                "double v = (1.0 - f) * x_ext(row, L_in, i0);"),
    "left edge off by one": ("return (i >= 0 && i < L) ? row[i] : 0.0;",
                             "return (i >= 1 && i < L) ? row[i] : 0.0;"),
    "padding sign": ("sample(row, L_in, l * s - p + k * d, offsets[oi], mask ? mask + oi : NULL);\n                }",
                     "sample(row, L_in, l * s + p + k * d, offsets[oi], mask ? mask + oi : NULL);\n                }"),
    "dilation ignored": ("sample(row, L_in, l * s - p + k * d, offsets[oi], mask ? mask + oi : NULL);\n                }",
                         "sample(row, L_in, l * s - p + k, offsets[oi], mask ? mask + oi : NULL);\n                }"),
    "stride ignored": ("sample(row, L_in, l * s - p + k * d, offsets[oi], mask ? mask + oi : NULL);\n                }",
                       "sample(row, L_in, l - p + k * d, offsets[oi], mask ? mask + oi : NULL);\n                }"),
    "truncate instead of floor": ("double fl = floor(o);", "double fl = trunc(o);"),
    "offset group interleaved": ("            const int64_t g = ci / cpo;\n            const double *row",
                                 "            const int64_t g = ci % G;\n            const double *row"),
    "mask ignored": ("return m ? v * (*m) : v;", "return v;"),
    "bias dropped": ("out[(b * C_out + co) * L_out + l] = acc + (bias ? bias[co] : 0.0);",
                     "out[(b * C_out + co) * L_out + l] = acc;"),
    "weight transposed": ("acc += weight[(co * cpg + cl) * K + k] *\n",
                          "acc += weight[(cl * C_out + co) * K + k] *\n"),
    "conv group ignored": ("S[((b * C_in + grp * cpg + cl) * K + k) * L_out + l];",
                           "S[((b * C_in + cl) * K + k) * L_out + l];"),
    "tap order reversed": ("acc += weight[(co * cpg + cl) * K + k] *\n",
                           "acc += weight[(co * cpg + cl) * K + (K - 1 - k)] *\n"),
    "output length off by one": ("return num / s + 1;", "return (num + 1) / s + 1;"),
    # the backward
    "bwd left weight dropped": ("grow[i0] += ds * m * (1.0 - f);", "grow[i0] += ds * m;"),
    "bwd mask missing in gx": ("grow[i0 + 1] += ds * m * f;", "grow[i0 + 1] += ds * f;"),
    "bwd offset derivative sign": ("ao += ds * m * (x1 - x0);", "ao += ds * m * (x0 - x1);"),
    "bwd mask gradient scaled by mask": ("am += ds * ((1.0 - f) * x0 + f * x1);",
                                         "am += ds * m * ((1.0 - f) * x0 + f * x1);"),
    "bwd conv group ignored in dS": ("const int64_t co = grp * opg + oc;", "const int64_t co = oc;"),
    "bwd weight gradient without mask": (
        "acc += dout[(b * C_out + co) * L_out + l] *\n"
        "                                   sample(row, L_in, l * s - p + k * d, offsets[oi], mask ? mask + oi : NULL);",
        "acc += dout[(b * C_out + co) * L_out + l] *\n"
        "                                   sample(row, L_in, l * s - p + k * d, offsets[oi], NULL);"),
    "bwd bias over the first batch only": ("            for (int64_t b = 0; b < B; ++b)\n                for (int64_t l = 0; l < L_out; ++l)\n                    acc += dout",
                                           "            for (int64_t b = 0; b < 1; ++b)\n                for (int64_t l = 0; l < L_out; ++l)\n                    acc += dout"),
    # the packed layer's generator
    "gen head channels k-major": ("const int64_t g = gk / K, k = gk % K;", "const int64_t g = gk % G, k = gk / G;"),
    "gen trunk dilation ignored": ("acc += tw[c * K + k] * x_ext(row, L_in, l * s - p + k * d);",
                                   "acc += tw[c * K + k] * x_ext(row, L_in, l * s - p + k);"),
    "gen trunk bias dropped": ("t[c * L_out + l] = tb ? acc + tb[c] : acc;", "t[c * L_out + l] = acc;"),
    "gen sigmoid sign": ("mask_out[o] = 1.0 / (1.0 + exp(-z));", "mask_out[o] = 1.0 / (1.0 + exp(z));"),
    "gen mask from the offset head": ("zm += mw[gk * C_in + c] * t[c * L_out + l];",
                                      "zm += ow[gk * C_in + c] * t[c * L_out + l];"),
    "gen offset bias dropped": ("offsets_out[o] = ob ? zo + ob[gk] : zo;", "offsets_out[o] = zo;"),
    # 2D
    "2d row and column offsets swapped": (
        "split_position(oh * sh - ph + i * dh, oy[q], &r0, &fy);\n"
        "                            split_position(ow * sw - pw + j * dw, ox[q], &c0, &fx);",
        "split_position(oh * sh - ph + i * dh, ox[q], &r0, &fy);\n"
        "                            split_position(ow * sw - pw + j * dw, oy[q], &c0, &fx);"),
    "2d taps column-major": ("const int64_t tap = (g * kh + i) * kw + j;", "const int64_t tap = (g * kw + j) * kh + i;"),
    "2d corner transposed": ("(1.0 - fy) * fx * x_ext2(plane, H, W, r0, c0 + 1)",
                             "(1.0 - fy) * fx * x_ext2(plane, H, W, r0 + 1, c0)"),
    "2d mask per group only": ("mask + (b * G * T + tap) * HWo", "mask + (b * G * T + g) * HWo"),
    "2d row stride ignored": ("split_position(oh * sh - ph + i * dh, oy[q], &r0, &fy);",
                              "split_position(oh - ph + i * dh, oy[q], &r0, &fy);"),
}

PIN_CALLS = [
    ("zero offsets = conv1d (grouped, strided)", lambda: pins.test_zero_offsets_equal_conv1d(pins.ZERO_OFFSET_CASES[5])),
    ("zero offsets = conv1d (offset groups)", lambda: pins.test_zero_offsets_equal_conv1d(pins.ZERO_OFFSET_CASES[4])),
    ("integer shift", lambda: pins.test_integer_offset_is_shift((1, 6, 6, 31, 4, 2, 3, 1, 3, 3), -3)),
    ("torchvision demo", pins.test_torchvision_issue_demo),
    ("fractional = spread conv1d", lambda: pins.test_constant_fractional_offset_equals_spread_conv1d(-2, 0.625, 2, 3, 2)),
    ("affine ramp", pins.test_affine_ramp_closed_form),
    ("hat brute force", lambda: pins.test_oracle_equals_hat_brute_force((2, 2, 3, 2, 4))),
    ("mask invariants", pins.test_mask_invariants),
    ("grouped = block diagonal", pins.test_grouped_equals_block_diagonal_dense),
    ("offset group blocks", pins.test_offset_group_channel_blocks),
    ("positions exact", pins.test_positions_exact_at_large_base),
    ("positions edges", pins.test_positions_edges),
    ("output length", pins.test_output_length_closed_form_vs_count),
    ("operator examples", pins.test_conv1d_operator_examples_shapes_and_params),
    ("backward = finite differences", lambda: bwd.test_backward_equals_finite_differences(bwd.SHAPES[1])),
    ("backward = hat-form autograd", lambda: bwd.test_backward_matches_hat_form_autograd(bwd.SHAPES[3])),
    ("backward = conv1d autograd", lambda: bwd.test_zero_offsets_match_conv1d_autograd(bwd.SHAPES[1])),
    ("generator = conv1d composition", lambda: pk.test_generator_equals_conv1d_composition(pk.SHAPES[0])),
    ("generator: zero mask head halves", pk.test_zero_mask_projection_halves_the_output),
    ("generator: bias-only head", pk.test_bias_only_offset_head_places_each_channel),
    ("2d torchvision demo", o2.test_torchvision_issue_demo_2d),
    ("2d zero offsets = conv2d", lambda: o2.test_zero_offsets_equal_conv2d(o2.SHAPES[1])),
    ("2d integer shift", lambda: o2.test_integer_group_shift_is_shifted_conv2d(o2.SHAPES[1])),
    ("2d one row = 1d", lambda: o2.test_one_line_reduces_to_the_1d_oracle("column")),
    ("2d one column = 1d", lambda: o2.test_one_line_reduces_to_the_1d_oracle("row")),
    ("2d bilinear field", o2.test_bilinear_field_is_reproduced),
    ("2d hat brute force", lambda: o2.test_equals_product_of_hats_brute_force(o2.SHAPES[1])),
    ("2d mask invariants", o2.test_mask_invariants),
]


@pytest.fixture(scope="module")
def workdir():
    with tempfile.TemporaryDirectory(prefix="dc1d_mutants_") as d:
        yield d


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, workdir):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation site not found: %s" % name
    mutated = src.replace(old, new)
    cpath = os.path.join(workdir, "m_%d.c" % abs(hash(name)))
    sopath = cpath[:-2] + ".so"
    open(cpath, "w").write(mutated)
    subprocess.check_call(["gcc", *oracle.CFLAGS, "-o", sopath, cpath, "-lm"])
    saved = oracle._default
    oracle._default = oracle.load_variant(sopath)
    caught = []
    try:
        for label, call in PIN_CALLS:
            try:
                call()
            except (AssertionError, ValueError):
                caught.append(label)
    finally:
        oracle._default = saved
    assert caught, "no pin caught the planted mistake %r" % name
