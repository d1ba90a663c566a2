"""Planted mistakes in the oracle must be caught by its pins.

Each case copies ``oracle/q4_oracle.c``, changes one expression to a
plausible bug (swapped nibbles, wrong offset, wrong scale index, a dropped
term, a flipped sign, the wrong input row, a wrong exponent bias, a wrong
pack shift; in the quantizer a wrong divisor, rounding mode, code offset or
absmax, and in the binary16 encoder a wrong rounding, bias or subnormal
quantum), compiles the copy on the CPU and checks that at least one pin
fails for it.  The real oracle passing every pin is ``test_oracle.py``.
"""
import os
import shutil
import subprocess

import pytest

import oracle
from tests import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "q4_oracle.c")

MUTANTS = {
    "nibble_order": ("k / 2];\n    return (k % 2 == 0) ? (byte & 0x0F) : (byte >> 4);",
                     "k / 2];\n    return (k % 2 == 0) ? (byte >> 4) : (byte & 0x0F);"),
    "tiled_nibble_order": ("return 4 * (r / 2) + 16 * (r % 2);", "return 4 * (r % 4) + 16 * (r / 4);"),
    "tiled_lane_order": ("16 * (16 * g + c)", "16 * (4 * c + g)"),
    "tiled_word_endian": ("((uint32_t)wq[4 * w + 3] << 24)", "((uint32_t)wq[4 * w + 3] << 16)"),
    "tiled_scale_order": ("* 64 + 4 * c + i", "* 64 + 16 * i + c"),
    # quads per tile rounded down instead of up: tiles overlap when K is not
    # a multiple of 128 (every index stays inside the buffers, so the
    # mutant's packer cannot write past them and corrupt the test process)
    "tiled_quad_stride": ("(t * quads_of(K) + q) * 1024", "(t * (K / 128) + q) * 1024"),
    "offset_7": ("(double)(q - 8)", "(double)(q - 7)"),
    "scale_index": (": scales[n * (K / 32) + k / 32]", ": scales[n * (K / 32) + (k / 32 + 1) % (K / 32)]"),
    "scale_per_16": (": scales[n * (K / 32) + k / 32]", ": scales[n * (K / 32) + (k / 16) % (K / 32)]"),
    "dropped_last_term": ("for (int64_t k = 0; k < K; ++k) {\n        const double t",
                          "for (int64_t k = 0; k < K - 1; ++k) {\n        const double t"),
    "flipped_sign": ("acc += t;", "acc -= t;"),
    "wrong_row": ("one_output(xd + m * K,", "one_output(xd + ((m + 1) % M) * K,"),
    "f16_bias": ("expo - 25)", "expo - 24)"),
    "f16_subnormal": ("ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    "bf16_bias": ("expo - 134)", "expo - 133)"),
    "pack_shift": ("wq[n * (K / 2) + j] = (uint8_t)(lo | (hi << 4));",
                   "wq[n * (K / 2) + j] = (uint8_t)(lo | (hi << 3));"),
    "tiled_pack_shift": ("(uint8_t)(code << (bit % 8));", "(uint8_t)(code << (bit % 4));"),
    "abs_dropped": ("mag += fabs(t);", "mag += t;"),
    "quant_divisor": ("q4o_f64_to_f16(absmax / 7.0);", "q4o_f64_to_f16(absmax / 8.0);"),
    "quant_round_away": ("double q = nearbyint(w_value(w, kind, base + k) / d);",
                         "double q = round(w_value(w, kind, base + k) / d);"),
    "quant_offset": ("code = (int)q + 8;", "code = (int)q + 7;"),
    "quant_upper_clamp": ("if (q > 7.0)\n                        q = 7.0;", "if (q > 8.0)\n                        q = 8.0;"),
    "quant_zero_block": ("int code = 8;", "int code = 0;"),
    "quant_signed_absmax": ("const double a = fabs(w_value(w, kind, base + k));",
                            "const double a = w_value(w, kind, base + k);"),
    "f16_encode_round_away": ("double n = nearbyint(ldexp(a, 10 - E));", "double n = round(ldexp(a, 10 - E));"),
    "f16_encode_subnormal": ("nearbyint(ldexp(a, 24));", "nearbyint(ldexp(a, 23));"),
    "f16_encode_bias": ("(uint16_t)((E + 15) << 10)", "(uint16_t)((E + 16) << 10)"),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor for %s not unique in the oracle" % name
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib_path = str(tmp_path / "libmutant.so")
    oracle.compile_library(str(mutated), lib_path)
    lib = oracle.load_library(lib_path)
    failures = []
    for pin_name, pin in oracle_pins.ALL_PINS.items():
        try:
            pin(lib)
        except AssertionError as e:
            failures.append(pin_name)
    assert failures, "planted mistake %r passed every pin" % name
