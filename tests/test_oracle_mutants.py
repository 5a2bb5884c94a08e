"""The pins must catch plausible mistakes: each case plants one mistake in a copy of the
oracle's C source (on the CPU, in a temporary directory), builds it, and runs the pin
tests against that build; at least one pin has to fail."""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kvfp4_oracle.c")
PIN_TESTS = [os.path.join(ROOT, "tests", f) for f in
             ("test_oracle_formats.py", "test_oracle_quant.py", "test_oracle_attend.py",
              "test_oracle_paged.py", "test_oracle_rtn.py", "test_oracle_f32_fake.py")]

MUTANTS = {
    "e2m1 ties to odd": ("(d == bestd && (c % 2) == 0)", "(d == bestd && (c % 2) == 1)"),
    "e2m1 grid entry": ("{0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0}", "{0.0, 0.5, 1.0, 1.5, 2.0, 2.5, 4.0, 6.0}"),
    "e2m1 drops sign": ("return (code & 8) ? -mag : mag;", "return mag;"),
    "e4m3 exponent bias": ("return ldexp(1.0 + m / 8.0, e - 7);", "return ldexp(1.0 + m / 8.0, e - 8);"),
    "e4m3 subnormal step": ("return ldexp((double)m, -9);", "return ldexp((double)m, -10);"),
    "e4m3 ties to odd": ("(d == bestd && (b % 2) == 0)", "(d == bestd && (b % 2) == 1)"),
    "bf16 ties up": ("else pick = ((lo >> 16) & 1u) ? hi : lo;", "else pick = hi;"),
    "static_6 divisor": ("make_candidate(xb, m, 6.0f, s_enc, s_dec, &c6);\n        pick = &c6;",
                         "make_candidate(xb, m, 5.0f, s_enc, s_dec, &c6);\n        pick = &c6;"),
    "global scale uses 240": ("float s_enc = (A > 0.0f) ? (E2M1_MAX * E4M3_MAX) / A : 0.0f;",
                              "float s_enc = (A > 0.0f) ? (E2M1_MAX * 240.0f) / A : 0.0f;"),
    "nibbles swapped": ("(uint8_t)((pick->code[2 * j] & 15) | ((pick->code[2 * j + 1] & 15) << 4))",
                        "(uint8_t)((pick->code[2 * j + 1] & 15) | ((pick->code[2 * j] & 15) << 4))"),
    "mse tie prefers 4": ("pick = (err4 < err6) ? &c4 : &c6;", "pick = (err4 <= err6) ? &c4 : &c6;"),
    "mse error not squared": ("e_lo = fmaf(d, d, e_lo);", "e_lo = fmaf(fabsf(d), 1.0f, e_lo);"),
    "reciprocal perturbed": ("float inv = (S > 0.0f) ? 1.0f / S : 0.0f;",
                             "float inv = (S > 0.0f) ? 1.0f / (S * 1.0001f) : 0.0f;"),
    "dequant drops global scale": ("float S = (float)kvfp4_oracle_e4m3_value(scales[r * nb + i / 16]) * s_dec;",
                                   "float S = (float)kvfp4_oracle_e4m3_value(scales[r * nb + i / 16]) * s_dec * 2.0f;"),
    "dequant product order": ("return (float)kvfp4_oracle_e2m1_value(c) * S;",
                              "return (float)((float)kvfp4_oracle_e2m1_value(c) * (float)kvfp4_oracle_e4m3_value(scales[r * nb + i / 16])) * s_dec; (void)S;"),
    "fake quant ignores the rule": ("if (!rc) rc = kvfp4_oracle_quantize(x, rows, d, rows_per_group, rule, codes, scales, group_amax);",
                                    "if (!rc) rc = kvfp4_oracle_quantize(x, rows, d, rows_per_group, 0, codes, scales, group_amax);"),
    "paged f32 uses block index as page": ("int rc = kvfp4_oracle_dequantize_rows_f32(codes + pg * rows_per_page * (d / 2),",
                                           "pg = b; int rc = kvfp4_oracle_dequantize_rows_f32(codes + pg * rows_per_page * (d / 2),"),
    "group amax from first row": ("for (int64_t i = 0; i < n; ++i) {\n    float v = fabsf", "for (int64_t i = 0; i < (n < 16 ? n : 16); ++i) {\n    float v = fabsf"),
    "attention scale ignored": ("s *= scale;", "s *= 1.0;"),
    "paged uses block index as page": ("int rc = kvfp4_oracle_dequantize_rows(codes + pg * rows_per_page * (d / 2),",
                                       "pg = b; int rc = kvfp4_oracle_dequantize_rows(codes + pg * rows_per_page * (d / 2),"),
    "rtn truncates": ("? 0.0f : rintf(xb[i] * inv);", "? 0.0f : truncf(xb[i] * inv);"),
    "zero element times inf": ("float y = (xb[i] == 0.0f) ? xb[i] : xb[i] * inv;",
                               "float y = xb[i] * inv;"),
    "rtn qmax off by one": ("const int qmax = (1 << (bits - 1)) - 1;\n  const int per_byte = 8 / bits;\n  const int nb = d / 16;\n  for (int64_t r = 0; r < rows; ++r) {\n    for (int b = 0;",
                            "const int qmax = (1 << (bits - 1));\n  const int per_byte = 8 / bits;\n  const int nb = d / 16;\n  for (int64_t r = 0; r < rows; ++r) {\n    for (int b = 0;"),
    "rtn scale kept in fp32": ("uint16_t sh = kvfp4_oracle_float_to_bf16(m / (float)qmax);\n      float sv = kvfp4_oracle_bf16_to_float(sh);",
                               "uint16_t sh = kvfp4_oracle_float_to_bf16(m / (float)qmax);\n      float sv = m / (float)qmax;"),
    "rtn dequant drops sign": ("int q = (raw >= (1 << (bits - 1))) ? raw - (1 << bits) : raw;", "int q = raw;"),
    "attention output rounded through binary32": (
        "kvfp4_oracle_double_to_bf16(o / den);", "kvfp4_oracle_float_to_bf16((float)(o / den));"),
    "double to bf16 ties up": ("if (above < below || (above == below && fmod(k, 2.0) != 0.0)) k += 1.0;",
                               "if (above <= below) k += 1.0;"),
    "attention keys off by one": ("const uint16_t* kr = k + (j * heads + h) * d;",
                                  "const uint16_t* kr = k + (((j + 1) % tk) * heads + h) * d;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site not found: {name}"
    mutated = src.replace(old, new, 1)
    with tempfile.TemporaryDirectory() as td:
        c = os.path.join(td, "mut.c")
        so = os.path.join(td, "libmut.so")
        open(c, "w").write(mutated)
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                        "-o", so, c, "-lm"], check=True, capture_output=True)
        env = dict(os.environ, KVFP4_ORACLE_LIB=so)
        # the E4M3 brute force (~30 s) is left out here: the E4M3 mutants are caught by the
        # midpoint sweeps, and it would otherwise run once per mutant
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            "-k", "not every_binary32", *PIN_TESTS], cwd=ROOT, env=env,
                           capture_output=True, text=True, timeout=600)
        assert r.returncode != 0, f"no pin failed for planted mistake: {name}\n{r.stdout[-2000:]}"
