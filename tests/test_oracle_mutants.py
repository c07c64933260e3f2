"""Mutation check of the oracle pins: each case plants one plausible mistake in
a copy of the oracle source (a wrong comparison, exponent, clamp, constant,
index or nibble order), builds it, and runs the pin suite against it.  Every
mutant must make the pins fail; a surviving mutant means a gap in the pins."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mxfp4_oracle.c")

MUTANTS = {
    "tie_rule_floor": ("(rule == OR_FLOOR) ? (mag > kMids[i])", "(rule == OR_FLOOR) ? (mag >= kMids[i])"),
    "tie_rule_amct": (": (mag >= kMids[i])", ": (mag > kMids[i])"),
    "floor_exponent": ("int k = (e - 1) - 2;", "int k = (e - 1) - 1;"),
    "floor_clamp": ("return k < -127 ? -127 : k;", "return k < -126 ? -126 : k;"),
    "amct_clamp": ("kMinScaleRaw = 0x1p-30f", "kMinScaleRaw = 0x1p-31f"),
    "amct_round": ("return (int)rintf(l);", "return (int)floorf(l);"),
    # the exact nearest integer to log2 r (no binary32 rounding of the log)
    "amct_exact_log2": ("float l = (float)log2l((long double)r);\n  return (int)rintf(l);",
                        "return (int)lround(log2((double)r));"),
    # torch.round sends halves to even, C's roundf away from zero
    "amct_round_half_away": ("return (int)rintf(l);", "return (int)roundf(l);"),
    # AMCT sign from the exact quotient instead of the binary32 one
    "amct_sign_exact_quotient": ("q_in = (double)((float)v / (float)scale);", "q_in = v / scale;"),
    "codebook_value": ("{0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0}", "{0.0, 0.5, 1.0, 1.5, 2.0, 2.5, 4.0, 6.0}"),
    "midpoint_value": ("{0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0}", "{0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 4.5}"),
    "mask_strictness": ("(fabs(v) > kE2M1Max * scale)", "(fabs(v) >= kE2M1Max * scale)"),
    "clip_limit": ("static const double kE2M1Max = 6.0;", "static const double kE2M1Max = 4.0;"),
    "sign_of_negative_zero_code": ("double q = sgn * kCodes[code];", "double q = (sgn < 0 && code == 0) ? 0.0 : sgn * kCodes[code];"),
    # a short tail block that runs on into the next row (a flattened view)
    "row_tail_crosses_rows": ("int n = (int)((cols - c0) < block ? (cols - c0) : block);\n      for (int j = 0; j < n; ++j) idx[j] = r * cols + c0 + j;",
                              "int n = (int)((cols - c0) < block ? (cols - c0) : block);\n      if (n < block && r + 1 < rows) n += 1;\n      for (int j = 0; j < n; ++j) idx[j] = r * cols + c0 + j;"),
    "column_index": ("for (int j = 0; j < n; ++j) idx[j] = (r0 + j) * cols + c;\n      int k = qdq_block(dtype, rule, sf, x, idx, n, y, clip, NULL);\n      if (e8m0) e8m0[b * cols + c]",
                     "for (int j = 0; j < n; ++j) idx[j] = (r0 + j) * cols + (cols - 1 - c);\n      int k = qdq_block(dtype, rule, sf, x, idx, n, y, clip, NULL);\n      if (e8m0) e8m0[b * cols + c]"),
    "group_restart": ("for (int64_t r0 = start; r0 < end; r0 += block, ++brow) {",
                      "for (int64_t r0 = start; r0 < end; r0 = (r0 / block + 1) * block, ++brow) {"),
    "ste_negative_zero": ("if (clip && clip[i]) g = 0.0;", "if (clip && clip[i]) g = -0.0;"),
    "nibble_order": ("codes[r * half + t] = (uint8_t)(lo | (hi << 4));", "codes[r * half + t] = (uint8_t)(hi | (lo << 4));"),
    "kmajor_nibble_order": ("codes_t[c * ldk + (t * block + o) / 2] = (uint8_t)(lo | (hi << 4));",
                            "codes_t[c * ldk + (t * block + o) / 2] = (uint8_t)(hi | (lo << 4));"),
    "kmajor_scale_layout": ("scales_t[c * k_blocks + t] = ", "scales_t[t * cols + c] = "),
    "kmajor_pad_code": ("uint8_t lo = o < n ? nib[idx[o]] : 0;", "uint8_t lo = o < n ? nib[idx[o]] : 8;"),
    "kmajor_leading_dim": ("int64_t ldk = k_blocks * block / 2;", "int64_t ldk = nbt * block / 2;"),
    "mxfp8_ties_away": ("double q = rint(a / quantum) * quantum;", "double q = round(a / quantum) * quantum;"),
    "mxfp8_emax": ("*mb = 3; *bias = 7; *maxn = 448.0; *emax = 8;", "*mb = 3; *bias = 7; *maxn = 448.0; *emax = 7;"),
    "mxfp8_e4m3_max_480": ("*mb = 3; *bias = 7; *maxn = 448.0;", "*mb = 3; *bias = 7; *maxn = 480.0;"),
    "mxfp8_zero_sign": ("codes[j] = (uint8_t)(m | (signbit(v) ? 0x80 : 0));", "codes[j] = (uint8_t)(m | (v < 0 && m ? 0x80 : 0));"),
    "mxfp8_kmajor_pad_code": ("q_t[c * ldq + t * 32 + o] = o < bl[t] ? codes[o] : 0;", "q_t[c * ldq + t * 32 + o] = o < bl[t] ? codes[o] : 0x80;"),
    "mxfp8_kmajor_group_restart": ("for (int64_t r0 = start; r0 < end; r0 += 32) {\n      bs[nbt] = r0;", "for (int64_t r0 = start; r0 < end; r0 = (r0 / 32 + 1) * 32) {\n      bs[nbt] = r0;"),
    "mxfp8_kmajor_scale_layout": ("scales_t[c * k_blocks + t] = mx8_block(", "scales_t[t * cols + c] = mx8_block("),
    "mxfp8_kmajor_leading_dim": ("const int64_t ldq = k_blocks * 32;", "const int64_t ldq = nbt * 32;"),
    "mxfp8_block128_max_of_first_32": ("const int n = (int)((cols - c0) < block ? (cols - c0) : block);\n      for (int j = 0; j < n; ++j) idx[j] = r * cols + c0 + j;\n      scales[r * nb + b] = mx8_block(",
                                       "const int n = (int)((cols - c0) < 32 ? (cols - c0) : 32);\n      for (int j = 0; j < n; ++j) idx[j] = r * cols + c0 + j;\n      scales[r * nb + b] = mx8_block("),
    "mxfp8_decode_block": ("v *= ldexp(1.0, (int)scales[r * nb + c / block] - 127);", "v *= ldexp(1.0, (int)scales[r * nb + c / 32] - 127);"),
    "mxfp8_subnormal_quantum": ("const int emin = 1 - bias; /* exponent of the smallest normal */", "const int emin = -bias;"),
    "gmm_group_weight": ("const double *w = right + (int64_t)g * K * N;", "const double *w = right + (int64_t)(g > 0 ? g - 1 : 0) * K * N;"),
    "gmm_list_type": ("const int64_t end = list_type == 1 ? start + group_list[g] : group_list[g];",
                      "const int64_t end = list_type == 1 ? group_list[g] : group_list[g];"),
    "gmm_reduction_range": ("for (int64_t k = start; k < end; ++k)", "for (int64_t k = 0; k < end; ++k)"),
    "gmm_transposed_right": ("acc += (long double)left[m * K + k] * (long double)w[k * N + n];",
                             "acc += (long double)left[m * K + k] * (long double)w[(n * K + k) % (K * N)];"),
    "gmm_double_sum": ("long double acc = 0.0L;\n          for (int64_t k = 0; k < K; ++k)", "double acc = 0.0;\n          for (int64_t k = 0; k < K; ++k)"),
    "gmm_group_out_stride": ("double *o = out + (int64_t)g * M * N;", "double *o = out + (int64_t)g * M;"),
    "e8m0_bias": ("if (e8m0) e8m0[r * nb + b] = (uint8_t)(k + 127);", "if (e8m0) e8m0[r * nb + b] = (uint8_t)(k + 128);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_kill_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutated = src.replace(old, new, 1)
    csrc = tmp_path / "m.c"
    csrc.write_text(mutated)
    lib = tmp_path / "libm.so"
    sys.path.insert(0, ROOT)
    from oracle import build as B
    subprocess.run(["gcc", *B.CFLAGS, str(csrc), "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, MXFP4_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
