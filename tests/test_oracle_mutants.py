"""The oracle's pins must catch plausible mistakes.

Each case copies the oracle source, plants one mistake by text replacement,
builds the mutant with gcc in a temporary directory and runs the pin suite
against it in a subprocess (SKINNY_ORACLE_LIB).  The suite must fail.  The
mistakes are planted in the oracle, on the CPU only.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "skinny_oracle.c")

MUTANTS = {
    "dropped_first_k": ("for (long k = 0; k < K; ++k)\n                acc += oracle_decode_bf16",
                        "for (long k = 1; k < K; ++k)\n                acc += oracle_decode_bf16"),
    "transposed_W_index": ("* oracle_decode_bf16(w[n * K + k]);",
                           "* oracle_decode_bf16(w[k * N + n]);"),
    "bias_sign": ("            if (bias)\n                acc += oracle_decode_bf16(bias[n]);\n            emit(acc, m * N + n, out16, out32);\n        }\n    }\n}\n\n/* FP8 e4m3 with one fp32",
                  "            if (bias)\n                acc -= oracle_decode_bf16(bias[n]);\n            emit(acc, m * N + n, out16, out32);\n        }\n    }\n}\n\n/* FP8 e4m3 with one fp32"),
    "bias_index": ("acc += oracle_decode_bf16(bias[n]);\n            emit(acc, m * N + n, out16, out32);\n        }\n    }\n}\n\n/* FP8 e4m3 with one fp32",
                   "acc += oracle_decode_bf16(bias[0]);\n            emit(acc, m * N + n, out16, out32);\n        }\n    }\n}\n\n/* FP8 e4m3 with one fp32"),
    "round_half_away": ("double r = nearbyint(q);", "double r = floor(q + 0.5);"),
    "fp32_intermediate": ("out16[idx] = oracle_round_bf16(acc);",
                          "out16[idx] = oracle_round_bf16((double)(float)acc);"),
    "overflow_to_max": ("return (uint16_t)(sign | 0x7F80);\n    /* res is exactly",
                        "return (uint16_t)(sign | 0x7F7F);\n    /* res is exactly"),
    "e4m3_bias": ("v = ldexp(8.0 + (double)m, e - 10);", "v = ldexp(8.0 + (double)m, e - 11);"),
    "mx_scale_index": ("oracle_decode_e8m0(xe[m * KB + b])", "oracle_decode_e8m0(xe[m * KB])"),
    "fp8_double_scale": ("double acc = dot * scale;", "double acc = dot * scale * (double)sw;"),
    # FP8 bias placement: before the per-tensor scale product, dropped, and
    # (MX) dropped or folded into the first block before its scales
    "fp8_bias_before_scale": ("double acc = dot * scale;\n            if (bias)\n                acc += oracle_decode_bf16(bias[n]);",
                              "double acc = dot;\n            if (bias)\n                acc += oracle_decode_bf16(bias[n]);\n            acc *= scale;"),
    "fp8_bias_dropped": ("double acc = dot * scale;\n            if (bias)\n                acc += oracle_decode_bf16(bias[n]);",
                         "double acc = dot * scale;\n            (void)bias;"),
    "mx_bias_dropped": ("* block;\n            }\n            if (bias)\n                acc += oracle_decode_bf16(bias[n]);",
                        "* block;\n            }\n            (void)bias;"),
    "mx_bias_in_first_block": (
        "double block = 0.0;\n"
        "                for (long k = b * 32; k < b * 32 + 32; ++k)\n"
        "                    block += oracle_decode_e4m3(xq[m * K + k]) * oracle_decode_e4m3(wq[n * K + k]);\n"
        "                acc += oracle_decode_e8m0(xe[m * KB + b]) * oracle_decode_e8m0(we[n * KB + b]) * block;\n"
        "            }\n"
        "            if (bias)\n"
        "                acc += oracle_decode_bf16(bias[n]);",
        "double block = (b == 0 && bias) ? oracle_decode_bf16(bias[n]) : 0.0;\n"
        "                for (long k = b * 32; k < b * 32 + 32; ++k)\n"
        "                    block += oracle_decode_e4m3(xq[m * K + k]) * oracle_decode_e4m3(wq[n * K + k]);\n"
        "                acc += oracle_decode_e8m0(xe[m * KB + b]) * oracle_decode_e8m0(we[n * KB + b]) * block;\n"
        "            }"),
    "subnormal_quantum": ("e = -126;", "e = -125;"),
    "quant_divides": ("float v = (float)oracle_decode_bf16(x[i]) * inv;",
                      "float v = (float)oracle_decode_bf16(x[i]) / s;"),
    "quant_no_clamp": ("v = v < -448.0f ? -448.0f : (v > 448.0f ? 448.0f : v);", "(void)0;"),
    "e4m3_round_half_up": ("double r = nearbyint(ldexp(a, -q_exp));",
                           "double r = floor(ldexp(a, -q_exp) + 0.5);"),
    "e4m3_subnormal_edge": ("if (e < -6)\n        e = -6;                /* subnormal range */",
                            "if (e < -7)\n        e = -7;                /* subnormal range */"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "mutant.c")
        so = os.path.join(d, "libmutant.so")
        open(c, "w").write(src.replace(old, new))
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o", so, c, "-lm"],
                       check=True)
        env = dict(os.environ, SKINNY_ORACLE_LIB=so)
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
        assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"
