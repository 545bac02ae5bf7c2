"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (on the CPU,
never in the HIP path), builds it to a temporary library, and runs the pin
suite against it in a subprocess: the suite must fail.  The unmodified source
must pass the same run.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "fp8q_oracle.c")
PINS = ["tests/test_oracle_codec.py", "tests/test_oracle_quantize.py", "tests/test_oracle_mx8.py",
        "tests/test_oracle_next.py"]

MUTANTS = {
    "e4m3_max_480": ("return fmt == ORACLE_E4M3 ? 448.0 : 57344.0;",
                     "return fmt == ORACLE_E4M3 ? 480.0 : 57344.0;"),
    "e4m3_bias_8": ("static int fmt_bias(int fmt) { return fmt == ORACLE_E4M3 ? 7 : 15; }",
                    "static int fmt_bias(int fmt) { return fmt == ORACLE_E4M3 ? 8 : 15; }"),
    "round_half_up": ("m = nearbyint(a / quantum);", "m = floor(a / quantum + 0.5);"),
    "subnormal_decode_off_by_one": ("v = ldexp((double)M, 1 - bias - mbits);",
                                    "v = ldexp((double)M, -bias - mbits);"),
    "signed_zero_lost": ("const uint8_t sign = signbit(y) ? 0x80 : 0x00;",
                         "const uint8_t sign = y < 0 ? 0x80 : 0x00;"),
    "scale_by_reciprocal": ("s = amax / fmax;                 /* IEEE fp32 divide */",
                            "s = amax * (1.0f / fmax);"),
    "no_scale_floor": ("    if (s < smin)\n        s = smin;\n    *scale = s;",
                       "    *scale = s;"),
    "quotient_not_rounded_to_fp32": (
        "float qf = elem(x, i) / s;   /* fp32 quotient, rounded once */\n"
        "        q[i] = oracle_fp8_encode((double)qf, fmt);",
        "double qf = (double)elem(x, i) / (double)s;\n"
        "        q[i] = oracle_fp8_encode(qf, fmt);"),
    "nonfinite_only_nan": ("        float v = elem(x, i);\n        if (!isfinite(v)) {",
                           "        float v = elem(x, i);\n        if (isnan(v)) {"),
    "reduce_scale_index": ("float d = oracle_fp8_decode(q[p][i], fmt) * scales[p][i / ORACLE_BLOCK];",
                           "float d = oracle_fp8_decode(q[p][i], fmt) * scales[p][i / 64];"),
    "reduce_first_scale_index": ("float acc = oracle_fp8_decode(q[0][i], fmt) * scales[0][i / ORACLE_BLOCK];",
                                 "float acc = oracle_fp8_decode(q[0][i], fmt) * scales[0][i % ORACLE_BLOCK];"),
    "requantize_to_input_format": ("quantize_block_any(acc, elem_f32, len, fmt_out, q_out + lo, s_out + b);",
                                   "quantize_block_any(acc, elem_f32, len, fmt_in, q_out + lo, s_out + b);"),
    "requantize_through_bf16": ("static float elem_f32(const void *p, size_t i) { return ((const float *)p)[i]; }",
                                "static float elem_f32(const void *p, size_t i) { return oracle_bf16_to_f32(oracle_f32_to_bf16(((const float *)p)[i])); }"),
    "tensorwise_first_block_only": ("    quantize_block_any(x, elem_bf16, n, fmt, q, scale);\n}",
                                    "    quantize_block_any(x, elem_bf16, n < 128 ? n : 128, fmt, q, scale);\n    { size_t i; for (i = 128; i < n; ++i) q[i] = oracle_fp8_encode((double)(elem_bf16(x, i) / *scale), fmt); }\n}"),
    "mx_dequant_exponent_off": ("    return ldexpf(1.0f, (int)code - 127);", "    return ldexpf(1.0f, (int)code - 126);"),
    "mx_dequant_row_stride": ("oracle_e8m0_decode(e8m0[r * (K / ORACLE_MX_BLOCK) + c / ORACLE_MX_BLOCK]);",
                              "oracle_e8m0_decode(e8m0[r + c / ORACLE_MX_BLOCK]);"),
    "mx_reduce_drops_peer": ("            for (p = 1; p < k; ++p) {\n                float d = mx_value",
                             "            for (p = 2; p < k; ++p) {\n                float d = mx_value"),
    "reduce_drops_last_peer": ("    for (p = 1; p < k; ++p) {\n        float d = oracle_fp8_decode",
                               "    for (p = 1; p + 1 < k; ++p) {\n        float d = oracle_fp8_decode"),
    "reduce_in_double": ("            acc = acc + d;", "            acc = (float)((double)acc + (double)d + 0x1p-60);"),
    "dequant_scale_index": ("float d = oracle_fp8_decode(q[i], fmt) * scales[i / ORACLE_BLOCK];",
                            "float d = oracle_fp8_decode(q[i], fmt) * scales[i / 128 / 2];"),
    "bf16_round_half_up": ("b += 0x7FFFu + lsb;", "b += 0x8000u + 0 * lsb;"),
    "mx_exponent_off_by_one": ("X = (ex - 1) - 8;", "X = ex - 8;"),
    "mx_clamp_wrong": ("if (X < -127) X = -127;", "if (X < -126) X = -126;"),
    "mx_divides_wrong_way": ("double v = ldexp((double)oracle_bf16_to_f32(w[i]), -X);",
                             "double v = ldexp((double)oracle_bf16_to_f32(w[i]), X);"),
}


def _run_pins(lib_path, tmp_path):
    env = dict(os.environ)
    if lib_path:
        env["FP8Q_ORACLE_LIB"] = lib_path
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PINS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode


def _build(src_text, tmp_path, name):
    c = tmp_path / (name + ".c")
    so = tmp_path / (name + ".so")
    c.write_text(src_text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                    "-shared", "-o", str(so), str(c), "-lm"], check=True)
    return str(so)


def _check_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    if text.count(old) != 1:
        return name + ": anchor not found exactly once"
    so = _build(text.replace(old, new), tmp_path, name)
    return None if _run_pins(so, tmp_path) != 0 else name + ": not caught"


@pytest.mark.slow
def test_unmodified_oracle_passes(tmp_path):
    so = _build(open(SRC).read(), tmp_path, "clean")
    assert _run_pins(so, tmp_path) == 0


@pytest.mark.slow
def test_every_mutant_is_caught(tmp_path):
    # the pin runs are separate processes; run them side by side
    workers = max(1, min(8, os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        problems = list(ex.map(lambda m: _check_mutant(m, tmp_path), sorted(MUTANTS)))
    problems = [p for p in problems if p]
    assert not problems, problems
