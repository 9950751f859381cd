"""The oracle's pins are sensitive: plausible mistakes planted in a copy of the
oracle source (a wrong shift, a swapped nibble, a dropped overwrite, a wrong
tie-break, ...) each make at least one pin fail.

Each mutation is a textual edit of ``oracle/splitzip_oracle.c`` compiled into a
temporary library; the real oracle is never modified.
"""
import os
import subprocess

import pytest

import oracle as O
import test_oracle_pins as P
import test_oracle_variants as PV

SRC = os.path.join(os.path.dirname(O.__file__), "splitzip_oracle.c")

MUTATIONS = {
    "bf16_exponent_shift": ("return (x >> 7) & 0xFFu;", "return (x >> 8) & 0xFFu;"),
    "bf16_sign_bit": ("unsigned sign = (x >> 15) & 1u;", "unsigned sign = (x >> 14) & 1u;"),
    "bf16_mantissa_mask": ("unsigned mant = x & 0x7Fu;", "unsigned mant = x & 0x3Fu;"),
    "e5m2_exponent_shift": ("return (b >> 2) & 0x1Fu;", "return (b >> 3) & 0x1Fu;"),
    "e5m2_triple_shift": ("g |= (uint64_t)s << (3 * j);", "g |= (uint64_t)s << (3 * (7 - j));"),
    "nibble_order_swapped": ("nib[i / 2] = (uint8_t)(nib[i / 2] | nibble);\n      else\n        nib[i / 2] = (uint8_t)(nib[i / 2] | (nibble << 4));",
                             "nib[i / 2] = (uint8_t)(nib[i / 2] | (nibble << 4));\n      else\n        nib[i / 2] = (uint8_t)(nib[i / 2] | nibble);"),
    "escape_nibble_not_zero": ("nibble = 0; /* R4 */", "nibble = 15; /* R4 */"),
    "escape_position_off_by_one": ("uint64_t pos = i - first;  /* R5 */", "uint64_t pos = i - first + 1;  /* R5 */"),
    "escape_record_fields_transposed": ("put_u16(esc + 3 * E, pos); /* R6 */\n        esc[3 * E + 2] = (uint8_t)e;",
                                        "put_u16(esc + 3 * E + 1, pos); /* R6 */\n        esc[3 * E] = (uint8_t)e;"),
    "escape_overwrite_dropped": ("      put_element(dtype, out, i, v, s);\n    }\n  }\n  return SZO_OK;",
                                 "      (void)v; (void)s;\n    }\n  }\n  return SZO_OK;"),
    "calibrate_ties_to_higher": ("if (best < 0 || hist[v] > hist[best]) best = (int)v;",
                                 "if (best < 0 || hist[v] >= hist[best]) best = (int)v;"),
    "calibrate_skips_last_value": ("for (unsigned v = 0; v < V; ++v) {\n      if (chosen[v]) continue;",
                                   "for (unsigned v = 0; v + 1 < V; ++v) {\n      if (chosen[v]) continue;"),
    "chunk_codebook_index": ("return (c * SZO_CHUNK) / seg;", "return c / seg;"),
    "offsets_inclusive": ("    put_u64(off + 8 * c, E);\n    for (uint64_t i = first; i < last; ++i) {\n      unsigned e = get_exponent(dtype, in, i);",
                          "    for (uint64_t i = first; i < last; ++i) {\n      unsigned e = get_exponent(dtype, in, i);"),
    "no_section_alignment": ("return (x + 255ull) / 256ull * 256ull;", "return x;"),
    "total_bytes_field": ("put_u64(out + 24, L.P + 3 * E);", "put_u64(out + 24, L.P + 2 * E);"),
    # ablation variants
    "sentinel_code_14": ("written = 15; /* V2 */", "written = 14; /* V2 */"),
    "top8_uses_seven_codes": ("return v == SZO_V_SENTINEL ? 15u : 8u;", "return v == SZO_V_SENTINEL ? 15u : 7u;"),
    "top8_code_order_reversed": ("g |= (uint64_t)code << (3 * j);", "g |= (uint64_t)code << (3 * (7 - j));"),
    "sentinel_values_from_stream_start": ("    uint64_t r = get_u64(off + 8 * c);\n    for (uint64_t i = first; i < last; ++i) {\n      unsigned code",
                                          "    uint64_t r = 0;\n    for (uint64_t i = first; i < last; ++i) {\n      unsigned code"),
    "variant_byte_missing": ("out[48] = (uint8_t)v; /* V1 */", "(void)v; /* V1 */"),
}

PINS = [
    P.test_hand_worked_bf16_stream,
    P.test_hand_worked_e5m2_stream,
    lambda: P.test_bf16_all_patterns_roundtrip("calibrated"),
    lambda: P.test_bf16_all_patterns_roundtrip("excludes_0_255"),
    lambda: P.test_e5m2_all_patterns_roundtrip("includes_0_31"),
    lambda: P.test_escapes_and_codes_match_definition(O.BF16),
    lambda: P.test_escapes_and_codes_match_definition(O.E5M2),
    lambda: [P.test_calibrate_matches_bruteforce(s) for s in range(6)],
    P.test_calibrate_extreme_exponents,
    P.test_bf16_split_matches_float_semantics,
    P.test_explainer_position50_golden,
    P.test_error_paths,
    lambda: PV.test_exhaustive_round_trip(O.SENTINEL),
    lambda: PV.test_exhaustive_round_trip(O.TOP8),
    lambda: PV.test_escape_sets_and_order_against_numpy(O.SENTINEL),
    lambda: PV.test_escape_sets_and_order_against_numpy(O.TOP8),
    PV.test_hand_worked_sentinel_stream,
    PV.test_hand_worked_top8_stream,
]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique/present: {name}"
    mutated = tmp_path / "mut.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-w", "-shared", "-fPIC", "-o", str(lib), str(mutated)])
    O.use_library(str(lib))
    caught = []
    try:
        for pin in PINS:
            try:
                pin()
            except (AssertionError, ValueError):
                caught.append(getattr(pin, "__name__", "lambda"))
                break
    finally:
        O.use_library(None)
    assert caught, f"no pin caught the planted mistake '{name}'"


def test_unmutated_oracle_passes_all_pins():
    for pin in PINS:
        pin()
