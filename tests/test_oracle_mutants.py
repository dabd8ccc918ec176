"""Plant plausible mistakes in copies of the CPU oracle and check that the pin
suite catches every one of them.  The mutants are built from the oracle's own
source by text replacement into a temporary directory; the oracle itself is
never modified.  Each mutant stays inside its buffers (no wild indices)."""
import os
import tempfile

import pytest

import oracle
import oracle_pins

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
    ("sampled path reads k-major",
     "acc += weight_value(codes, scales, K, n, k) * q4o_bf16_to_double(x[t * K + k]);",
     "acc += weight_value(codes, scales, K, n, k) * q4o_bf16_to_double(x[(k * 7 + t) % K]);"),
]


def _catches(o):
    failures = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(o)
        except AssertionError:
            failures.append(pin.__name__)
    return failures


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
