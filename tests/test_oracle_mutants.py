"""Planted mistakes: the pins must catch a plausible bug anywhere in the oracle.

Each case patches the oracle's C source in a temporary directory (the committed
source is never touched), builds it with the same flags, and runs the pin tests
against the mutant. A mutant that passes every pin is a hole in the pins.
"""

import pathlib

import pytest

import oracle
import test_oracle_act as act_pins
import test_oracle_conv as conv_pins
import test_oracle_decode_bf16_state as bf16_state_pins
import test_oracle_formats as format_pins
import test_oracle_rounding as round_pins

SRC = oracle.SOURCE.read_text()

MUTANTS = {
    "taps reversed": [("fmaf(w[0 * ws1], hist[0], acc)", "fmaf(w[0 * ws1], cur, acc)"),
                      ("fmaf(w[3 * ws1], cur, acc)", "fmaf(w[3 * ws1], hist[0], acc)")],
    "bias dropped": [("float acc = bias_c ? *bias_c : 0.0f;", "float acc = 0.0f;")],
    "taps newest first": [("fmaf(w[0 * ws1], hist[0], acc);\n  acc = fmaf(w[1 * ws1], hist[1], acc);\n"
                           "  acc = fmaf(w[2 * ws1], hist[2], acc);\n  acc = fmaf(w[3 * ws1], cur, acc);",
                           "fmaf(w[3 * ws1], cur, acc);\n  acc = fmaf(w[2 * ws1], hist[2], acc);\n"
                           "  acc = fmaf(w[1 * ws1], hist[1], acc);\n  acc = fmaf(w[0 * ws1], hist[0], acc);")],
    "bias added last": [("float acc = bias_c ? *bias_c : 0.0f;", "float acc = 0.0f;"),
                        ("acc = fmaf(w[3 * ws1], cur, acc);\n  return acc;",
                         "acc = fmaf(w[3 * ws1], cur, acc);\n  return bias_c ? acc + *bias_c : acc;")],
    "unfused multiply-add": [("acc = fmaf(w[1 * ws1], hist[1], acc);",
                              "acc = w[1 * ws1] * hist[1] + acc;")],
    "silu sign": [("oracle_crexpf(-a)", "oracle_crexpf(a)")],
    "silu via reciprocal": [("return a / d;", "return a * (1.0f / d);")],
    "state written newest first": [("k * cs_stride2] = hist[k];", "k * cs_stride2] = hist[2 - k];")],
    "state never read": [("int init = live && has_initial_state && has_initial_state[s];",
                          "int init = 0;")],
    "null block ignored": [("int live = !(has_null_block && line == null_block_id) && line >= 0",
                            "int live = 1 && line >= 0")],
    "weight strides taken as contiguous": [("const float* w = weight + c * w_stride0;",
                                            "const float* w = weight + c * 4;"),
                                           ("conv_acc(w, w_stride1, b, hist, cur)",
                                            "conv_acc(w, 1, b, hist, cur)")],
    "cache index stride ignored": [("int64_t line = cache_indices[s * ci_stride];",
                                    "int64_t line = cache_indices[s];")],
    "missing initial-state array read as all set": [
        ("int init = live && has_initial_state && has_initial_state[s];",
         "int init = live && (!has_initial_state || has_initial_state[s]);")],
    "window shift wrong": [("hist[0] = hist[1];\n        hist[1] = hist[2];",
                            "hist[1] = hist[2];\n        hist[0] = hist[1];")],
    "planes transposed": [("int64_t o = (plane * num_tokens + t) * part_dim + col;",
                           "int64_t o = (t * (dim / part_dim) + plane) * part_dim + col;")],
    "ties away from even": [("(dropped == 0x8000u && (kept & 1u))", "(dropped == 0x8000u)")],
    "bf16 truncates": [("if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1;",
                        "(void)dropped;")],
    "f16 truncates": [("uint32_t m = (uint32_t)rintf(ldexpf(a, 10 - e));",
                       "uint32_t m = (uint32_t)truncf(ldexpf(a, 10 - e));")],
    "f16 subnormal quantum": [("rintf(a * 0x1p24f)", "rintf(a * 0x1p23f)")],
    "f16 overflow at the largest number": [("if (a >= 65520.0f)", "if (a > 65504.0f)")],
    "f16 ties away from zero": [("uint32_t m = (uint32_t)rintf(ldexpf(a, 10 - e));",
                                 "uint32_t m = (uint32_t)roundf(ldexpf(a, 10 - e));")],
    "f16 widen keeps signalling NaN": [("sign | 0x7FC00000u | (frac << 13)",
                                        "sign | 0x7F800000u | (frac << 13)")],
    "f16 widen exponent bias": [("(int)expo - 25", "(int)expo - 24")],
    "f32 output NaN payload kept": [("isnan(y) ? 0x7FC00000u : bits_of(y)", "bits_of(y)")],
    "f16 read as bf16": [("return fmt == ORACLE_F16 ? oracle_f16_to_f32(h) : oracle_bf16_to_f32(h);",
                          "return oracle_bf16_to_f32(h);")],
    "bf16 state: token word rounded through FP32": [
        ("2 * cs_stride2] = xw;", "2 * cs_stride2] = oracle_f32_to_bf16(oracle_bf16_to_f32(xw));")],
    "bf16 state: part stride ignored": [("weight + plane * w_part_stride + col * w_stride0",
                                         "weight + c * w_stride0")],
    "bf16 state: oldest entry kept": [("0 * cs_stride2] = words[1];", "0 * cs_stride2] = words[0];")],
    "bf16 state: null block ignored": [
        ("&& !(has_null_block && line == null_block_id);", ";")],
    "bf16 state: width and channel strides swapped": [
        ("col * w_stride0;\n      float acc = conv_acc(w, w_stride1,",
         "col * w_stride1;\n      float acc = conv_acc(w, w_stride0,")],
    "exp one ulp high": [("    return (float)q;\n  }\n  return (float)e;",
                          "    return (float)q;\n  }\n  return nextafterf((float)e, INFINITY);")],
}

PINS = [
    *[(f"brute force {s}", lambda lib, s=s: conv_pins.test_brute_force_exact(lib, s)) for s in range(6)],
    *[(f"unit tap {t}", lambda lib, t=t: conv_pins.test_unit_taps_shift_the_input(lib, t)) for t in range(4)],
    ("near midpoints", conv_pins.test_brute_force_near_bf16_midpoints),
    ("bias first", conv_pins.test_bias_enters_first),
    ("oldest first", conv_pins.test_taps_enter_oldest_first),
    ("ones", lambda lib: conv_pins.test_all_ones_taps_sum_integers(lib, False)),
    ("plane layout", conv_pins.test_plane_layout),
    ("state last three", lambda lib: conv_pins.test_state_is_last_three_inputs(lib, True)),
    ("null block", conv_pins.test_null_block_runs_from_zero_and_leaves_its_line),
    *[(f"weight strides {l}", lambda lib, l=l: conv_pins.test_weight_strides_against_brute_force(lib, l))
      for l in ("transposed", "padded")],
    ("cache index stride", conv_pins.test_cache_index_stride_against_brute_force),
    ("no initial-state array", conv_pins.test_no_initial_state_array_means_none_set),
    ("out-of-range line", lambda lib: conv_pins.test_out_of_range_line_acts_as_null_block(lib, 3)),
    ("torch conv1d silu", lambda lib: conv_pins.test_against_torch_conv1d_float64(lib, 0, True)),
    ("silu random", act_pins.test_silu_random_against_exact),
    ("silu near midpoints", act_pins.test_silu_near_bf16_midpoints),
    ("bf16 closed forms", lambda lib: [round_pins.test_bf16_round_closed_forms(lib, u)
                                       for u in (0x3F808000, 0x3F818000, 0x00018000)]),
    ("f16 binades", format_pins.test_f16_round_every_binade_critical_bits),
    ("f16 widen", format_pins.test_f16_widen_every_pattern),
    ("f32 word", format_pins.test_f32_word_reading),
    *[(f"brute force {f} {s}", lambda lib, f=f, s=s: format_pins.test_brute_force_exact(lib, f, s))
      for f in ("f16", "f32") for s in range(3)],
    ("bf16 state brute force", lambda lib: bf16_state_pins.test_brute_force_exact(lib, 0)),
    ("bf16 state width-major taps", bf16_state_pins.test_width_major_taps_land_on_their_channels),
    ("bf16 state NaN words", bf16_state_pins.test_nan_words_keep_their_payloads),
    ("bf16 state null block", lambda lib: bf16_state_pins.test_null_block_and_lines_outside(lib, -1)),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path: pathlib.Path):
    src = SRC
    for old, new in MUTANTS[name]:
        assert src.count(old) == 1, f"patch for {name!r} no longer matches the oracle source"
        src = src.replace(old, new)
    mutant_src = tmp_path / "kdaconv_oracle.c"
    mutant_src.write_text(src)
    so = tmp_path / "libmutant.so"
    import subprocess

    subprocess.run(["gcc", *oracle._CFLAGS, "-o", str(so), str(mutant_src), "-lquadmath", "-lm"],
                   check=True)
    lib = oracle.load(so)
    caught = []
    for pin_name, pin in PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            caught.append(pin_name)
    assert caught, f"no pin catches the planted mistake {name!r}"
