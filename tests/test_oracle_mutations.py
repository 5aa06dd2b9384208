"""Plant plausible mistakes in a copy of the oracle (on the CPU only) and check
that the pins catch every one: a dropped term, a wrong sign, a wrong index or
bound, a swapped tie rule, a transposed nibble. The original must pass the
same checks."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from tests import test_oracle_formats as F
from tests import test_oracle_method as M
from tests import test_oracle_rotation as RO
from tests import test_oracle_sweep as SW
from tests import test_oracle_tiles as TI
from tests import test_oracle_two_level as T

SRC = os.path.join(os.path.dirname(oracle.__file__), "lq_oracle.c")
HDR = os.path.join(os.path.dirname(oracle.__file__), "lq_oracle.h")

# (name, text to find, replacement, pins expected to catch it)
MUTATIONS = [
    ("hadamard sign", "v[i + h] = a - b;", "v[i + h] = b - a;",
     [lambda o: M.test_hadamard_butterfly(o)]),
    ("tie to odd", "return (fmod(n, 2.0) == 0.0) ? lo : hi;", "return (fmod(n, 2.0) == 0.0) ? hi : lo;",
     [lambda o: F.test_every_midpoint_brute_force(o, "e4m3")]),
    ("scale off by one", "float t = amax / (float)qmax;", "float t = amax / (float)(qmax + 1.0);",
     [lambda o: M.test_symmetric_matches_bruteforce(o, "int8", "f32", "block", 32)]),
    ("ue8m0 bound", "while (ldexp(qmax, e) < absmax) e++;", "while (ldexp(qmax, e) <= absmax) e++;",
     [lambda o: F.test_ue8m0_exponent_brute_force(o)]),
    ("zero point dropped", "if (!d->symmetric) q += (double)sc->zp;", "if (!d->symmetric) q += 0.0;",
     [lambda o: M.test_asymmetric_matches_bruteforce(o, "int4", "f16", "block", 64, "rne")]),
    ("subnormal spacing", "int k = kmin;\n  if (a >= ldexp(1.0, kmin))", "int k = kmin - 1;\n  if (a >= ldexp(1.0, kmin))",
     [lambda o: F.test_random_values_brute_force(o, "e5m2")]),
    ("error term dropped", "e2 += diff * diff;", "e2 += diff * diff * 0.5;",
     [lambda o: M.test_symmetric_matches_bruteforce(o, "e4m3", "ue8m0", "block", 32)]),
    ("nibble order", "if ((e & 1) == 0) *b = (uint8_t)((*b & 0xF0u) | (code & 0xFu));",
     "if ((e & 1) == 1) *b = (uint8_t)((*b & 0xF0u) | (code & 0xFu));",
     [lambda o: M.test_page_int4_group_example(o)]),
    ("ieee-style e4m3", "/* ORK_E4M3 */ {4, 3, 7, 0, 1},", "/* ORK_E4M3 */ {4, 3, 7, 1, 0},",
     [lambda o: F.test_printed_ranges(o)]),
    ("int8 symmetric range", "*qmin = d->symmetric ? -127.0 : -128.0;", "*qmin = -128.0;",
     [lambda o: M.test_clamp_ranges_with_given_scales(o, "int8", True, -127, 127)]),
    ("dequant uses unstored scale", "sc->s = (float)or_fp_decode(ORK_FP16, sc->sbits);", "sc->s = t;",
     [lambda o: M.test_symmetric_matches_bruteforce(o, "int4", "f16", "block", 16)]),
    ("integer taken before the clip", "    if (q < qmin) q = qmin;\n    if (q > qmax) q = qmax;\n    int qi = (int)q;",
     "    int qi = (int)q;\n    if (qi < (int)qmin) qi = (int)qmin;\n    if (qi > (int)qmax) qi = (int)qmax;",
     [lambda o: M.test_clamp_ranges_with_given_scales(o, "int8", True, -127, 127)]),
    ("rotation scale", "float or_rotation_scale(int n) { return (float)(1.0 / sqrt((double)n)); }",
     "float or_rotation_scale(int n) { return (float)(2.0 / sqrt((double)n)); }",
     [lambda o: M.test_hadamard_butterfly(o)]),
    ("tensor scale without the E4M3 maximum", "const float denom = 448.0f * (float)elem_qmax(d);",
     "const float denom = (float)elem_qmax(d);",
     [lambda o: T.test_largest_block_takes_the_largest_e4m3_scale(o, "e2m1")]),
    ("tensor scale divides the dequant", "if (d->two_level) xh = xh * S;", "if (d->two_level) xh = xh / S;",
     [lambda o: T.test_two_level_matches_bruteforce(o, "int4", 16, "bf16")]),
    ("normalization skipped", "nrm[j] = d->two_level ? row[j] / S : row[j];", "nrm[j] = row[j];",
     [lambda o: T.test_power_of_two_input_scaling(o, "e2m1")]),
    ("error against the normalized values", "double diff = (double)xo[j] - (double)xh;",
     "double diff = (double)v[j] - (double)xh;",
     [lambda o: T.test_two_level_matches_bruteforce(o, "e4m3", 32, "f32")]),
    ("zero tensor scale kept", "return S == 0.0f ? 1.0f : S;", "return S;",
     [lambda o: T.test_zero_tensor_and_storage(o)]),
    ("tile statistic of one row", "r < nrows && r < (b + 1) * d->tile_rows; r++)",
     "r < nrows && r < b * d->tile_rows + 1; r++)",
     [lambda o: TI.test_tiles_match_bruteforce(o, "int8", "f32", 3, 32)]),
    ("signs after the butterflies",
     "  for (int i = 0; i < n; i++)\n    if (sign_bit(signs, col0 + i)) v[i] = -v[i];\n  butterflies(v, n);\n  const float c",
     "  butterflies(v, n);\n  for (int i = 0; i < n; i++)\n    if (sign_bit(signs, col0 + i)) v[i] = -v[i];\n  const float c",
     [lambda o: RO.test_rotation_matches_signed_hadamard_matrix(o, 64)]),
    ("sign column offset ignored", "static int sign_bit(const uint32_t* signs, int64_t col) {\n  return signs ? (int)((signs[col >> 5]",
     "static int sign_bit(const uint32_t* signs, int64_t col) {\n  col &= 31;\n  return signs ? (int)((signs[col >> 5]",
     [lambda o: RO.test_rotation_matches_signed_hadamard_matrix(o, 32)]),
    ("tally pair takes the wrong float format", "static const int fp_slot[3] = {OR_E4M3, OR_E5M2, OR_E2M1};",
     "static const int fp_slot[3] = {OR_E5M2, OR_E4M3, OR_E2M1};",
     [lambda o: SW.test_tally_pairs_and_slots(o)]),
    ("tally table transposed", "const double qi = qsnr[t * 25 + int_slot[p] * 5 + g];",
     "const double qi = qsnr[t * 25 + g * 5 + int_slot[p]];",
     [lambda o: SW.test_tally_pairs_and_slots(o)]),
    ("tally winner swapped", "return d > 0.0 ? OR_WIN_INT : OR_WIN_FP;", "return d > 0.0 ? OR_WIN_FP : OR_WIN_INT;",
     [lambda o: SW.test_tally_infinities_and_nan(o)]),
    ("tally margin ignored", "if (a > tie_db + margin_db) return", "if (a >= tie_db) return",
     [lambda o: SW.test_tally_band_edges(o)]),
    ("tally infinities unequal", "const double d = (q_int == q_fp) ? 0.0 : q_int - q_fp;",
     "const double d = q_int - q_fp;",
     [lambda o: SW.test_tally_infinities_and_nan(o)]),
    ("fp6 code bits in the wrong order", "c |= (uint32_t)((codes[bit >> 3] >> (bit & 7)) & 1u) << k;",
     "c |= (uint32_t)((codes[bit >> 3] >> (bit & 7)) & 1u) << (5 - k);",
     [lambda o: SW.test_fp6_dequant_bit_by_bit(o, "e2m3", "ue8m0")]),
    ("tile column ignored", "sc = tsc[(r / d->tile_rows) * groups_per_row + g];",
     "sc = tsc[(r / d->tile_rows) * groups_per_row];",
     [lambda o: TI.test_tiles_match_bruteforce(o, "e4m3", "f32", 2, 16)]),
]


def _build_mutant(tmp_path, find, repl):
    src = open(SRC).read()
    assert src.count(find) == 1, f"mutation anchor not unique/found: {find!r}"
    d = tmp_path / "m"
    d.mkdir(exist_ok=True)
    shutil.copy(HDR, d / "lq_oracle.h")
    (d / "lq_oracle.c").write_text(src.replace(find, repl))
    so = d / f"mut_{abs(hash(find)) % 10**8}.so"
    subprocess.run(["gcc", *oracle.GCC_FLAGS, str(d / "lq_oracle.c"), "-o", str(so), "-lm"], check=True)
    return str(so)


def _passes(checks):
    for chk in checks:
        try:
            chk(oracle)
        except AssertionError:
            return False
    return True


@pytest.mark.parametrize("name,find,repl,checks", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, name, find, repl, checks):
    assert _passes(checks), f"pins fail on the unmodified oracle ({name})"
    so = _build_mutant(tmp_path, find, repl)
    with oracle.swap_library(so):
        caught = not _passes(checks)
    assert caught, f"planted mistake '{name}' was not caught"
    assert np.isfinite(oracle.fp_max("e4m3"))  # original library restored
