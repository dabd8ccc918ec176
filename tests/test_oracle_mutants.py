"""Plant plausible mistakes in copies of the CPU oracle and check that the pin
suite catches every one of them.  The mutants are built from the oracle's own
source by text replacement into a temporary directory; the oracle itself is
never modified.  Each mutant stays inside its buffers (no wild indices)."""
import os
import tempfile

import pytest

import oracle
import oracle_pins
import oracle_pins_fmt

MUTANTS = [
    ("sign of the code offset", "(double)(q - 8) * s", "(double)(8 - q) * s"),
    ("code offset off by one", "(double)(q - 8) * s", "(double)(q - 7) * s"),
    ("scale dropped", "(double)(q - 8) * s", "(double)(q - 8)"),
    ("nibble order swapped", "(k % 2 == 0) ? (byte & 0x0F) : (byte >> 4)",
     "(k % 2 == 0) ? (byte >> 4) : (byte & 0x0F)"),
    ("group of 128 instead of 64", "scales[n * (K / 64) + k / 64]", "scales[n * (K / 64) + k / 128]"),
    ("groups reversed", "scales[n * (K / 64) + k / 64]", "scales[n * (K / 64) + (K / 64 - 1 - k / 64)]"),
    ("code row stride lost", "codes[n * (K / 2) + k / 2]", "codes[k / 2]"),
    ("activations read k-major", "s += w[k] * q4o_bf16_to_double(xt[k]);",
     "s += w[k] * q4o_bf16_to_double(x[k * T + t]);"),
    ("output written n-major", "y[t * N + n] = q4o_double_to_bf16(s);",
     "y[n * T + t] = q4o_double_to_bf16(s);"),
    ("rounded through binary32", "y[t * N + n] = q4o_double_to_bf16(s);",
     "y[t * N + n] = q4o_double_to_bf16((double)(float)s);"),
    ("ties away from zero", "(frac == 0.5 && fmod(whole, 2.0) != 0.0)", "(frac == 0.5)"),
    ("truncation instead of rounding",
     "if (frac > 0.5 || (frac == 0.5 && fmod(whole, 2.0) != 0.0))", "if (0)"),
    ("fp16 subnormal scale", "ldexp((double)m, -24)", "ldexp((double)m, -25)"),
    ("fp16 exponent bias", "ldexp((double)(m + 1024), e - 25)", "ldexp((double)(m + 1024), e - 24)"),
    ("bf16 hidden bit", "ldexp((double)(m + 128), e - 134)", "ldexp((double)(m + 127), e - 134)"),
    ("binary32 accumulation", "double s = 0.0;\n                const uint16_t *xt",
     "float s = 0.0f;\n                const uint16_t *xt"),
    ("no bf16 subnormals", "int qexp = (e < -126) ? -133 : e - 7;", "int qexp = e - 7;"),
    ("residual dropped", "s += q4o_bf16_to_double(r[t * N + n]);", "s += 0.0;"),
    ("residual read n-major", "s += q4o_bf16_to_double(r[t * N + n]);",
     "s += q4o_bf16_to_double(r[(n * T + t) % (N * T)]);"),
    ("residual added after a first rounding", "s += q4o_bf16_to_double(r[t * N + n]);",
     "s = q4o_bf16_to_double(q4o_double_to_bf16(s)) + q4o_bf16_to_double(r[t * N + n]);"),
    ("swiglu gate sign", "g[i] / (1.0 + exp(-g[i]))", "g[i] / (1.0 + exp(g[i]))"),
    ("swiglu sigmoid without the g factor", "g[i] / (1.0 + exp(-g[i]))", "1.0 / (1.0 + exp(-g[i]))"),
    ("swiglu gate and up swapped", "g[i] / (1.0 + exp(-g[i]));\n        y[i] = q4o_double_to_bf16(silu * u[i]);",
     "u[i] / (1.0 + exp(-u[i]));\n        y[i] = q4o_double_to_bf16(silu * g[i]);"),
    ("swiglu gate rounded to binary32 first", "y[i] = q4o_double_to_bf16(silu * u[i]);",
     "y[i] = q4o_double_to_bf16((double)(float)silu * (double)(float)u[i]);"),
    ("residual subtracted", "s += q4o_bf16_to_double(r[t * N + n]);", "s -= q4o_bf16_to_double(r[t * N + n]);"),
    ("Q5 code offset 15", "(double)(q - 16) * q4o_fp16_to_double", "(double)(q - 15) * q4o_fp16_to_double"),
    ("Q5 high bits read from the top", "(hi[n * (K / 8) + k / 8] >> (k % 8)) & 1", "(hi[n * (K / 8) + k / 8] >> (7 - k % 8)) & 1"),
    ("Q5 high plane stride", "(hi[n * (K / 8) + k / 8] >> (k % 8)) & 1", "(hi[n * (K / 16) + k / 8] >> (k % 8)) & 1"),
    ("Q5 high bit weighted 8", "int q = low_nibble(lo, K, n, k) | (h << 4);\n        return (double)(q - 16)",
     "int q = low_nibble(lo, K, n, k) | (h << 3);\n        return (double)(q - 16)"),
    ("Q6 pairs packed as nibbles", "(hi[n * (K / 4) + k / 4] >> (2 * (k % 4))) & 3", "(hi[n * (K / 4) + k / 4] >> (k % 4)) & 3"),
    ("Q6 code offset 16", "(double)(q - 32) * q4o_fp16_to_double", "(double)(q - 16) * q4o_fp16_to_double"),
    ("W8 codes unsigned", "int c = (int)(int8_t)lo[n * K + k];", "int c = (int)lo[n * K + k];"),
    ("W8 groups of 64", "s16[n * (K / 32) + k / 32]", "s16[n * (K / 32) + k / 64]"),
    ("NVFP4 groups of 32", "s8[n * (K / 16) + k / 16]", "s8[n * (K / 16) + k / 32]"),
    ("E2M1 subnormal as 1", "(e == 0) ? 0.5 * m", "(e == 0) ? 1.0 * m"),
    ("E4M3 exponent bias 6", "ldexp((double)(m + 8), e - 10)", "ldexp((double)(m + 8), e - 9)"),
    ("E4M3 subnormal scale", "ldexp((double)m, -9);           /* subnormal", "ldexp((double)m, -10);           /* subnormal"),
    ("BF16 weight row stride", "return q4o_bf16_to_double(w[n * K + k]);", "return q4o_bf16_to_double(w[(n * K + k) / 2 * 2]);"),
    ("Q5 byte count 40", "return n * (k / 64) * 42;", "return n * (k / 64) * 40;"),
    ("sampled format path reads the wrong token", "fmt_weight(fmt, lo, hi, sc, K, ns[i], k) * q4o_bf16_to_double(x[ts[i] * K + k]);",
     "fmt_weight(fmt, lo, hi, sc, K, ns[i], k) * q4o_bf16_to_double(x[k]);"),
    ("sampled path reads k-major",
     "acc += weight_value(codes, scales, K, n, k) * q4o_bf16_to_double(x[t * K + k]);",
     "acc += weight_value(codes, scales, K, n, k) * q4o_bf16_to_double(x[(k * 7 + t) % K]);"),
]


def _catches(o):
    """Name of the first pin that fails on oracle `o` (None if every pin passes)."""
    for pin in oracle_pins.ALL_PINS + oracle_pins_fmt.ALL_PINS:
        try:
            pin(o)
        except AssertionError:
            return pin.__name__
    return None


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    src = open(oracle.SOURCE).read()
    assert src.count(old) >= 1, "mutation point missing from the oracle source: %r" % old
    mutated = src.replace(old, new)
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "mutant.c")
        with open(path, "w") as f:
            f.write(mutated)
        lib = oracle.compile_source(path, os.path.join(d, "libmutant.so"))
        caught = _catches(oracle.Oracle(lib))
    assert caught, "no pin caught the mutant: %s" % name
