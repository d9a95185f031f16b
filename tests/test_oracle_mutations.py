"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch every one of them.  Each mutant is the oracle source with one textual
change, compiled with the oracle's own flags; a mutant survives if all the
selected pin checks pass on it."""
import numpy as np
import pytest

import test_oracle_pins as pins

MUTATIONS = [
    ("fma operands transposed", "rintf(fmaf(w, scale, zero))", "rintf(fmaf(zero, scale, w))"),
    ("zero init sign", "zero = -(mn * scale);", "zero = mn * scale;"),
    ("W_r sign of zero", "float wr = (q[i] - zero) / scale;", "float wr = (q[i] + zero) / scale;"),
    ("W_r multiplies by scale", "float wr = (q[i] - zero) / scale;", "float wr = (q[i] - zero) * scale;"),
    ("residual sign", "float x = w[i] - wr;", "float x = wr - w[i];"),
    ("W_e added instead of subtracted", "(sum_w - sum_e)", "(sum_w + sum_e)"),
    ("W_e dropped from the mean", "te[i] = (double)e[i];", "te[i] = 0.0;"),
    ("tree sum skips its last level", "for (int st = 1; st < gs; st *= 2)", "for (int st = 1; st < gs / 2; st *= 2)"),
    ("mean over gs-1", "zero = (float)(num / (double)gs);", "zero = (float)(num / (double)(gs - 1));"),
    ("exponent p instead of p-1", "float pm1 = p - 1.0f;", "float pm1 = p;"),
    ("beta divides", "float v = a - pw / beta;", "float v = a - pw * beta;"),
    ("beta updated before use", "        for (int i = 0; i < gs; ++i) {\n            float wr",
     "        beta = beta * kappa;\n        for (int i = 0; i < gs; ++i) {\n            float wr"),
    ("ties away from zero", "float q = rintf(fmaf(w, scale, zero));", "float q = roundf(fmaf(w, scale, zero));"),
    ("no upper clamp", "    if (q > qmax)\n        q = qmax;\n", ""),
    ("final codes from the init zero", "        codes[i] = (uint8_t)quantize_one(w[i], scale, zero, qmax);",
     "        codes[i] = (uint8_t)quantize_one(w[i], scale, tr_zero ? tr_zero[0] : -(mn * scale), qmax);"),
    ("pack MSB first", "word |= ((uint32_t)codes[r * cols + col] & mask) << (j * nbits);",
     "word |= ((uint32_t)codes[r * cols + col] & mask) << ((C - 1 - j) * nbits);"),
    ("fp16 subnormal widening off by 2", "mag = ldexpf((float)man, -24);", "mag = ldexpf((float)man, -23);"),
]


def _checks(o):
    """The pin checks run on a mutant (a selection of the pin tests)."""
    return [
        lambda: pins.test_f16_to_f32_all_patterns(o),
        lambda: pins.test_iters0_is_minmax_rtn(o, 4),
        lambda: pins.test_iters0_is_minmax_rtn(o, 2),
        lambda: pins.test_rtn_ties_go_to_even(o, 4),
        lambda: pins.test_constant_group(o),
        lambda: pins.test_p1_is_soft_threshold(o),
        lambda: pins.test_shrink_matches_fp64_formula(o),
        lambda: pins.test_zero_update_is_quadratic_argmin(o, 10.0),
        lambda: pins.test_zero_update_is_quadratic_argmin(o, 1000.0),
        lambda: pins.test_codes_follow_current_zero(o),
        lambda: pins.test_residual_and_beta_schedule(o),
        lambda: pins.test_grid_weights_are_a_fixed_point(o, 4, 64),
        lambda: pins.test_grid_weights_are_a_fixed_point(o, 2, 16),
        lambda: pins.test_codes_in_range_and_axis_layout(o, 2),
        lambda: pins.test_alternation_descends_when_we_zero(o, 2, 16),
        lambda: pins.test_pack_hand_derived_words(o),
        lambda: pins.test_clamp_engaged(o, 3, 64, 1.0, 0.1, 1.5, "up", 2),
        lambda: pins.test_clamp_engaged(o, 2, 16, 0.7, 0.1, 1.5, "lo", 23),
    ]


def test_every_mutation_is_caught(oracle_mod, tmp_path):
    src = oracle_mod.source()
    survivors = []
    for i, (name, old, new) in enumerate(MUTATIONS):
        assert src.count(old) >= 1, f"mutation '{name}' does not apply"
        path = oracle_mod.build_variant(src.replace(old, new), str(tmp_path / f"mut{i}.so"))
        o = oracle_mod.Oracle(path)
        caught = False
        for check in _checks(o):
            try:
                check()
            except (AssertionError, ValueError, IndexError, OverflowError):
                caught = True
                break
        if not caught:
            survivors.append(name)
    assert not survivors, f"mutations not caught by any pin: {survivors}"


def test_unmutated_oracle_passes_the_selection(oracle_mod):
    for check in _checks(oracle_mod):
        check()
