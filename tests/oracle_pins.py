"""Pins for the CPU oracle: checks against facts that do not come from the
oracle itself.  Each ``pin_*`` takes an ``oracle.Oracle`` so the same checks can
be run on deliberately broken copies of the oracle (see
``test_oracle_mutants.py``) to show that they catch plausible mistakes.

Where each fact comes from:

* hand-worked examples (``tests/golden/worked_examples.json``), derived on
  paper from the op's definition: ``(q-8)*scale`` per 64-weight group, low
  nibble = even k, token-major X/Y, one round-to-nearest-even to bf16;
* library routines: numpy's float16 decode, torch's bfloat16 decode and its
  binary32 -> bfloat16 rounding, numpy's binary64 matrix product, Python's
  exact rationals (``fractions.Fraction``);
* the pages' closed form for weight bytes ("linear-benchmark.md" section 4:
  34 bytes per 64-weight group; "q4-linear.md": 16,711,680 bytes for
  6144x5120; "linear-benchmark.md" section 9: 11,141,120 bytes for 4096x5120);
* invariants of a linear map: exact scaling by powers of two, locality of rows,
  columns and groups, independence of tokens, zero weights give zero.
"""
from __future__ import annotations

import json
import os
import struct
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_examples.json")


# --------------------------------------------------------------------------
# independent helpers (library-based or exact rational)
# --------------------------------------------------------------------------
def torch_bf16_decode(bits) -> np.ndarray:
    import torch
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16)).view(np.int16)
    return torch.from_numpy(b.copy()).view(torch.bfloat16).to(torch.float64).numpy()


def torch_f32_to_bf16_bits(v) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(v, dtype=np.float32)))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def frac_to_bf16_bits(v: Fraction) -> int:
    """Exact rational -> bf16 bits, round to nearest even, by exact arithmetic;
    the final (exactly representable) value is encoded through binary32 with
    the struct module."""
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    qexp = max(e - 7, -133)
    q = Fraction(2) ** qexp
    r = a / q
    whole = r.numerator // r.denominator
    rem = r - whole
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and whole % 2 == 1):
        whole += 1
    value = whole * q
    if value >= Fraction(2) ** 128:
        return sign | 0x7F80
    f32 = struct.unpack("<I", struct.pack("<f", float(value)))[0]
    assert Fraction(struct.unpack("<f", struct.pack("<I", f32))[0]) == value
    return sign | (f32 >> 16)


def fp16_exact(bits: int) -> Fraction:
    return Fraction(float(np.array([bits], dtype=np.uint16).view(np.float16)[0]))


def bf16_exact(bits: int) -> Fraction:
    return Fraction(float(torch_bf16_decode([bits])[0]))


# --------------------------------------------------------------------------
# golden examples
# --------------------------------------------------------------------------
def load_examples():
    with open(GOLDEN) as f:
        return json.load(f)["examples"]


def _h(s) -> int:
    return int(s, 16) if isinstance(s, str) else int(s)


def materialize(ex):
    n, k, t = ex["n"], ex["k"], ex["t"]
    codes = np.full((n, k // 2), _h(ex["codes"]["fill"]), dtype=np.uint8)
    for key, val in ex["codes"].get("set", {}).items():
        if ":" in key:
            r, j = key.split(":")
            codes[int(r), int(j)] = _h(val)
        else:
            codes[:, int(key)] = _h(val)
    scales = np.array([_h(s) for s in ex["scales"]], dtype=np.uint16).reshape(n, k // 64)
    xs = ex["x"]
    if isinstance(xs, list):
        x = np.array([_h(v) for v in xs], dtype=np.uint16)
    elif "alternate" in xs:
        a, b = (_h(v) for v in xs["alternate"])
        x = np.array([a if i % 2 == 0 else b for i in range(k * t)], dtype=np.uint16)
    else:
        x = np.full(k * t, _h(xs["fill"]), dtype=np.uint16)
        for key, val in xs.get("set", {}).items():
            x[int(key)] = _h(val)
        for lo, hi, val in xs.get("range_fill", []):
            x[lo:hi] = _h(val)
    y = np.array([_h(v) for v in ex["y"]], dtype=np.uint16)
    return x.reshape(t, k), codes, scales, y


def pin_worked_examples(o):
    for ex in load_examples():
        x, codes, scales, want = materialize(ex)
        got = o.linear(x, codes, scales, ex["n"], ex["k"], ex["t"]).reshape(-1)
        assert np.array_equal(got, want), "%s: got %s want %s" % (
            ex["name"], [hex(v) for v in got], [hex(v) for v in want])


GOLDEN_ADD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_examples_add.json")


def load_add_examples():
    with open(GOLDEN_ADD) as f:
        return json.load(f)["examples"]


def materialize_add(ex):
    x, codes, scales, y = materialize(ex)
    r = np.array([_h(v) for v in ex["r"]], dtype=np.uint16).reshape(ex["t"], ex["n"])
    return x, codes, scales, r, y


def pin_add_worked_examples(o):
    for ex in load_add_examples():
        x, codes, scales, r, want = materialize_add(ex)
        got = o.linear_add(x, codes, scales, r, ex["n"], ex["k"], ex["t"]).reshape(-1)
        assert np.array_equal(got, want), "%s: got %s want %s" % (
            ex["name"], [hex(v) for v in got], [hex(v) for v in want])


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------
def pin_fp16_decode(o):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    lib = bits.view(np.float16).astype(np.float64)
    got = np.array([o.fp16_to_double(int(b)) for b in bits])
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], lib[~nan])


def pin_bf16_decode(o):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    lib = torch_bf16_decode(bits)
    got = np.array([o.bf16_to_double(int(b)) for b in bits])
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], lib[~nan])


def _rounding_cases(seed=7, count=4000):
    r = np.random.default_rng(seed)
    cases = []
    # random magnitudes over the whole bf16 range and a bit beyond
    exps = r.integers(-140, 130, size=count)
    mant = r.uniform(1.0, 2.0, size=count)
    sgn = r.choice([-1.0, 1.0], size=count)
    cases += list(sgn * np.ldexp(mant, exps))
    # exact midpoints between neighbouring bf16 values, and just off them
    for _ in range(count // 2):
        e = int(r.integers(-133, 120))
        m = int(r.integers(128, 256))
        q = 2.0 ** (e - 7) if e >= -126 else 2.0 ** -133
        mid = (m + 0.5) * q if e >= -126 else (int(r.integers(0, 128)) + 0.5) * q
        cases += [mid, -mid, mid * (1 + 2.0 ** -40), mid * (1 - 2.0 ** -40)]
    # overflow boundary and the smallest magnitudes
    big = (2.0 - 2.0 ** -8) * 2.0 ** 127
    cases += [big, -big, big * (1 - 2.0 ** -30), big * (1 + 2.0 ** -30), 2.0 ** 128, 1e300,
              2.0 ** -134, 2.0 ** -134 * (1 + 2.0 ** -20), 2.0 ** -135, 5e-324, 0.0, -0.0]
    return [float(c) for c in cases]


def pin_rounding_nearest_even(o):
    for v in _rounding_cases():
        b = o.double_to_bf16(v)
        fv = Fraction(v)
        mag = b & 0x7FFF
        if mag == 0x7F80:   # Inf: |v| must be at or beyond the overflow midpoint
            assert abs(fv) >= Fraction(2) ** 127 * (2 - Fraction(1, 256)), v
            assert (b >> 15) == (1 if v < 0 else 0)
            continue
        assert mag < 0x7F80, (v, hex(b))
        val = bf16_exact(b)
        if v != 0:
            assert (b >> 15) == (1 if v < 0 else 0) or val == 0, (v, hex(b))
        d = abs(fv - val)
        # neighbours along the magnitude axis
        neigh = []
        if mag > 0:
            neigh.append(bf16_exact((b & 0x8000) | (mag - 1)))
        else:
            neigh.append(-bf16_exact(1) if v < 0 else bf16_exact(1))
            neigh.append(bf16_exact(1) if v < 0 else -bf16_exact(1))
        if mag + 1 < 0x7F80:
            neigh.append(bf16_exact((b & 0x8000) | (mag + 1)))
        for nv in neigh:
            dn = abs(fv - nv)
            assert d <= dn, (v, hex(b))
            if d == dn and nv != val:
                assert mag % 2 == 0, ("tie not to even", v, hex(b))


def pin_rounding_vs_torch(o):
    """For binary32-representable values, torch's binary32 -> bfloat16
    conversion is a single correct rounding; the oracle must agree."""
    r = np.random.default_rng(11)
    v32 = np.concatenate([
        r.standard_normal(20000).astype(np.float32),
        (r.standard_normal(5000) * 1e30).astype(np.float32),
        (r.standard_normal(5000) * 1e-36).astype(np.float32),
        # 1 + m * 2^-8 scaled by powers of two: odd m are exact bf16 midpoints
        np.ldexp(1.0 + r.integers(0, 256, 4000) * 2.0 ** -8,
                 r.integers(-120, 120, 4000)).astype(np.float32),
    ])
    want = torch_f32_to_bf16_bits(v32)
    got = np.array([o.double_to_bf16(float(v)) for v in v32], dtype=np.uint16)
    assert np.array_equal(got, want)


def pin_weight_bytes(o):
    # pages' printed closed forms
    assert o.weight_bytes(6144, 5120) == 16_711_680
    assert o.weight_bytes(4096, 5120) == 11_141_120
    # the same formula at the workload shapes: groups * 34
    for n, k in [(512, 1024), (14336, 5120), (34816, 5120), (5120, 17408)]:
        assert o.weight_bytes(n, k) == n * k // 64 * 34
    # the storage planes of the generated inputs add up to it
    from weight_only_bit_q4_amd import inputs
    c = inputs.gen_codes(512, 1024, 1)
    s = inputs.gen_scales(512, 1024, 1)
    assert c.nbytes + s.nbytes == o.weight_bytes(512, 1024) == 278_528


# --------------------------------------------------------------------------
# special cases that reduce to library routines
# --------------------------------------------------------------------------
def _int_weights(codes, n, k):
    lo = (codes & 0x0F).astype(np.int64)
    hi = (codes >> 4).astype(np.int64)
    q = np.empty((n, k), dtype=np.int64)
    q[:, 0::2] = lo
    q[:, 1::2] = hi
    return q - 8


def pin_unit_scales_integer_x(o):
    """Scales 1.0 and small-integer activations: every output is a small
    integer, computed here by numpy's integer product and rounded by torch."""
    r = np.random.default_rng(3)
    n, k, t = 24, 192, 5
    codes = r.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    scales = np.full((n, k // 64), 0x3C00, dtype=np.uint16)
    xi = r.integers(-3, 4, size=(t, k)).astype(np.int64)
    x = torch_f32_to_bf16_bits(xi.astype(np.float32))
    ref = (_int_weights(codes, n, k) @ xi.T).T          # [t, n] integers
    want = torch_f32_to_bf16_bits(ref.astype(np.float32))
    got = o.linear(x, codes, scales, n, k, t)
    assert np.array_equal(got, want)


def pin_unit_scales_matmul(o):
    """Scales 1.0: W is an integer matrix; numpy's binary64 product is exact
    here (a few dozen significant bits at most), so rounding it with the
    separately pinned bf16 rounding must match the oracle bit for bit."""
    from weight_only_bit_q4_amd import inputs
    n, k, t = 48, 512, 6
    codes = inputs.gen_codes(n, k, 5)
    x = inputs.gen_x(k, t, 5)
    scales = np.full((n, k // 64), 0x3C00, dtype=np.uint16)
    xf = torch_bf16_decode(x.reshape(-1)).reshape(t, k)
    ref = xf @ _int_weights(codes, n, k).astype(np.float64).T   # [t, n]
    want = np.array([[o.double_to_bf16(v) for v in row] for row in ref], dtype=np.uint16)
    got = o.linear(x, codes, scales, n, k, t)
    assert np.array_equal(got, want)


def _exact_sums(x, codes, scales, n, k, t):
    """The exact rational sums W . X, [t][n] lists of Fractions."""
    q = _int_weights(codes, n, k)
    sc = [[fp16_exact(int(scales[i, g])) for g in range(k // 64)] for i in range(n)]
    xs = [[bf16_exact(int(x[j, kk])) for kk in range(k)] for j in range(t)]
    out = [[Fraction(0)] * n for _ in range(t)]
    for j in range(t):
        for i in range(n):
            acc = Fraction(0)
            for kk in range(k):
                if q[i, kk]:
                    acc += int(q[i, kk]) * sc[i][kk // 64] * xs[j][kk]
            out[j][i] = acc
    return out


def _exact_linear(x, codes, scales, n, k, t):
    sums = _exact_sums(x, codes, scales, n, k, t)
    out = np.zeros((t, n), dtype=np.uint16)
    for j in range(t):
        for i in range(n):
            out[j, i] = frac_to_bf16_bits(sums[j][i])
    return out


def pin_add_exact_bruteforce(o, trials=6):
    """LinearAdd against exact rationals: the exact sum plus the exact residual,
    rounded once (round to nearest, ties to even)."""
    r = np.random.default_rng(29)
    for trial in range(trials):
        n = int(r.integers(1, 5))
        k = 64 * int(r.integers(1, 3))
        t = int(r.integers(1, 4))
        codes = r.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
        sv = r.choice([-1, 1], size=(n, k // 64)) * np.ldexp(r.uniform(1, 2, (n, k // 64)),
                                                             r.integers(-12, 4, (n, k // 64)))
        scales = sv.astype(np.float16).view(np.uint16)
        xv = (r.standard_normal((t, k)) * np.ldexp(1.0, r.integers(-6, 6, (t, k)))).astype(np.float32)
        x = torch_f32_to_bf16_bits(xv)
        res = torch_f32_to_bf16_bits((r.standard_normal((t, n)) * 4.0).astype(np.float32))
        q = _int_weights(codes, n, k)
        sc = [[fp16_exact(int(scales[i, g])) for g in range(k // 64)] for i in range(n)]
        want = np.zeros((t, n), dtype=np.uint16)
        for j in range(t):
            for i in range(n):
                acc = bf16_exact(int(res[j, i]))
                for kk in range(k):
                    if q[i, kk]:
                        acc += int(q[i, kk]) * sc[i][kk // 64] * bf16_exact(int(x[j, kk]))
                want[j, i] = frac_to_bf16_bits(acc)
        got = o.linear_add(x, codes, scales, res, n, k, t)
        assert np.array_equal(got, want), "trial %d (n=%d k=%d t=%d)" % (trial, n, k, t)


def pin_add_all_code8_passes_residual(o):
    """All-eight codes make every weight 0, so the result is the residual itself,
    bit for bit (any finite bf16 residual, across the binades)."""
    n, k, t = 24, 192, 3
    x, codes, scales = _problem(n, k, t, 31)
    codes[:] = 0x88
    r = np.random.default_rng(31)
    res = torch_f32_to_bf16_bits((r.standard_normal((t, n)) * np.ldexp(1.0, r.integers(-60, 60, (t, n))))
                                 .astype(np.float32))
    got = o.linear_add(x, codes, scales, res, n, k, t)
    assert np.array_equal(got, res)


def pin_add_zero_residual_and_shift(o):
    """R = 0 leaves the plain Linear result; an R that is a multiple of the
    result's own bf16 spacing and keeps its binade shifts it exactly."""
    n, k, t = 16, 256, 2
    x, codes, scales = _problem(n, k, t, 37)
    plain = o.linear(x, codes, scales, n, k, t)
    zero = np.zeros((t, n), dtype=np.uint16)
    assert np.array_equal(o.linear_add(x, codes, scales, zero, n, k, t), plain)
    # weights in {-1, 0, 1} (nibbles 7, 8, 9), unit scales and activations:
    # the sum is an integer s with |s| <= 128, so s and s + 1 are bf16 values
    # and R = 1 shifts the result exactly
    k2 = 128
    r = np.random.default_rng(37)
    nib = r.integers(7, 10, size=(n, k2))
    codes2 = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    scales2 = np.full((n, k2 // 64), 0x3C00, dtype=np.uint16)  # 1.0
    x2 = np.full((t, k2), 0x3F80, dtype=np.uint16)              # 1.0
    s = (nib - 8).sum(axis=1)
    ones = np.full((t, n), 0x3F80, dtype=np.uint16)
    got = o.linear_add(x2, codes2, scales2, ones, n, k2, t)
    from oracle import bf16_bits_to_f64
    assert np.array_equal(bf16_bits_to_f64(got), np.tile((s + 1).astype(np.float64), (t, 1)))


def pin_exact_bruteforce(o, trials=6):
    """Exact rational sums with an exact round-to-nearest-even, on tiny shapes
    with wide-range scales (including subnormal and negative FP16) and
    activations spread over many binades."""
    r = np.random.default_rng(17)
    for trial in range(trials):
        n = int(r.integers(1, 6))
        k = 64 * int(r.integers(1, 4))
        t = int(r.integers(1, 4))
        codes = r.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
        sv = r.choice([-1, 1], size=(n, k // 64)) * np.ldexp(r.uniform(1, 2, (n, k // 64)),
                                                             r.integers(-26, 6, (n, k // 64)))
        scales = sv.astype(np.float16).view(np.uint16)
        xv = (r.standard_normal((t, k)) * np.ldexp(1.0, r.integers(-20, 20, (t, k)))).astype(np.float32)
        x = torch_f32_to_bf16_bits(xv)
        want = _exact_linear(x, codes, scales, n, k, t)
        got = o.linear(x, codes, scales, n, k, t)
        assert np.array_equal(got, want), "trial %d (n=%d k=%d t=%d)" % (trial, n, k, t)


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------
def _problem(n, k, t, seed):
    from weight_only_bit_q4_amd import inputs
    return inputs.gen_x(k, t, seed), inputs.gen_codes(n, k, seed), inputs.gen_scales(n, k, seed)


def pin_all_code8_zero(o):
    x, codes, scales = _problem(16, 256, 3, 21)
    codes[:] = 0x88
    y = o.linear(x, codes, scales, 16, 256, 3)
    assert np.all((y & 0x7FFF) == 0)


def pin_pow2_scale_invariance(o):
    from oracle import bf16_bits_to_f64
    n, k, t = 32, 256, 4
    x, codes, scales = _problem(n, k, t, 23)
    y0 = bf16_bits_to_f64(o.linear(x, codes, scales, n, k, t))
    for j in (-3, 2, 5):
        sj = (scales.astype(np.int32) + (j << 10)).astype(np.uint16)   # exponent field += j
        yj = bf16_bits_to_f64(o.linear(x, codes, sj, n, k, t))
        assert np.array_equal(yj, y0 * 2.0 ** j), j


def pin_locality(o):
    n, k, t = 8, 256, 3
    x, codes, scales = _problem(n, k, t, 29)
    y0 = o.linear(x, codes, scales, n, k, t)

    def only_changes(y1, rows=None, toks=None):
        diff = y1 != y0
        assert diff.any()
        mask = np.zeros_like(diff)
        if rows is not None:
            mask[:, rows] = True
        if toks is not None:
            mask[toks, :] = True
        assert not (diff & ~mask).any()

    s = scales.copy()
    s[5, 2] = 0x3C00                           # one group's scale of row 5
    only_changes(o.linear(x, codes, s, n, k, t), rows=5)
    c = codes.copy()
    c[2, 70] ^= 0x77                           # codes of row 2 (group 2)
    only_changes(o.linear(x, c, scales, n, k, t), rows=2)
    xx = x.copy()
    xx[1, 100] = 0x4120                        # token 1, k = 100
    only_changes(o.linear(xx, codes, scales, n, k, t), toks=1)
    # a group's scale only matters through that group's k-range
    xz = x.copy()
    xz[:, 128:192] = 0                         # zero the activations of group 2
    s = scales.copy()
    s[:, 2] = 0x5000
    assert np.array_equal(o.linear(xz, codes, s, n, k, t), o.linear(xz, codes, scales, n, k, t))


def pin_token_independence(o):
    n, k, t = 16, 320, 5
    x, codes, scales = _problem(n, k, t, 31)
    y = o.linear(x, codes, scales, n, k, t)
    for j in range(t):
        yj = o.linear(x[j:j + 1], codes, scales, n, k, 1)
        assert np.array_equal(yj[0], y[j])
    # a row slice of W gives the same rows of Y
    ys = o.linear(x, codes[4:11], scales[4:11], 7, k, t)
    assert np.array_equal(ys, y[:, 4:11])


def pin_group_permutation(o):
    """Permuting whole 64-groups of W's columns together with X's rows changes
    only the summation order: bf16 results agree except within a hair of a
    rounding midpoint."""
    from oracle import bf16_bits_to_f64
    n, k, t = 16, 512, 3
    x, codes, scales = _problem(n, k, t, 37)
    y0, a0 = o.linear(x, codes, scales, n, k, t, with_acc=True)
    perm = np.random.default_rng(1).permutation(k // 64)
    cp = codes.reshape(n, k // 64, 32)[:, perm].reshape(n, k // 2)
    sp = scales[:, perm]
    xp = x.reshape(t, k // 64, 64)[:, perm].reshape(t, k)
    y1, a1 = o.linear(xp, cp, sp, n, k, t, with_acc=True)
    assert np.allclose(a0, a1, rtol=1e-12, atol=0)
    assert np.array_equal(y0, y1)
    assert np.all(np.abs(bf16_bits_to_f64(y0) - a0) <= np.abs(a0) * 2.0 ** -8)


def pin_linear_at(o):
    n, k, t = 64, 512, 7
    x, codes, scales = _problem(n, k, t, 41)
    y = o.linear(x, codes, scales, n, k, t)
    r = np.random.default_rng(2)
    ns = r.integers(0, n, 300)
    ts = r.integers(0, t, 300)
    got = o.linear_at(x, codes, scales, n, k, t, ns, ts)
    assert np.array_equal(got, y[ts, ns])


# -- LinearSwiGLU: Y = bf16(silu(G) * U), G and U the sums of two weights -----
def pin_swiglu_zero_gate_or_up(o):
    """silu(0) = 0: an all-eight gate gives zeros signed like U; an all-eight
    up weight gives zeros of either sign."""
    n, k, t = 24, 256, 3
    x, cg, sg = _problem(n, k, t, 91)
    _, cu, su = _problem(n, k, t, 92)
    zero = np.full_like(cg, 0x88)
    _, u = o.linear(x, cu, su, n, k, t, with_acc=True)
    y = o.linear_swiglu(x, zero, sg, cu, su, n, k, t)
    assert np.array_equal(y, np.where(u < 0, 0x8000, 0x0000).astype(np.uint16))
    y = o.linear_swiglu(x, cg, sg, zero, su, n, k, t)
    assert np.all((y & 0x7FFF) == 0)


def pin_swiglu_saturated_gate(o):
    """For G >= 64, silu(G) = G (1 - e^-G) is G to far below bf16 resolution
    (e^-64 < 2^-92), so Y = bf16(G U) from the exact rationals, except where
    G U is itself a bf16 tie (skipped: the e^-G term decides those); for
    G <= -64, silu(G) < 64 e^-64 < 2^-86 and |Y| underflows to zero for the
    |U| < 2^10 used here."""
    n, k, t = 6, 128, 2
    r = np.random.default_rng(93)
    x = np.full((t, k), 0x3F80, dtype=np.uint16)              # X = 1
    sg = np.full((n, k // 64), 0x3C00, dtype=np.uint16)        # scale 1
    cg = np.full((n, k // 2), 0x99, dtype=np.uint8)            # G = K = 128
    cg[n // 2:] = 0x77                                         # G = -128
    _, cu, su = _problem(n, k, t, 94)
    su = (r.integers(0x2C00, 0x3400, size=su.shape)).astype(np.uint16)   # |s| in [2^-4, 2^-2)
    y = o.linear_swiglu(x, cg, sg, cu, su, n, k, t)
    G = _exact_sums(x, cg, sg, n, k, t)
    U = _exact_sums(x, cu, su, n, k, t)
    checked = 0
    for j in range(t):
        for i in range(n):
            assert abs(U[j][i]) < 2 ** 10
            if G[j][i] > 0:
                prod = G[j][i] * U[j][i]
                lo = bf16_exact(frac_to_bf16_bits(prod))
                if prod != lo and 2 * prod == lo + bf16_exact(frac_to_bf16_bits(2 * prod - lo)):
                    continue  # a tie
                assert int(y[j, i]) == frac_to_bf16_bits(prod), (i, j)
                checked += 1
            else:
                assert int(y[j, i]) & 0x7FFF == 0, (i, j)
    assert checked >= n * t // 2 - 1


def pin_swiglu_single_rounding(o):
    """Worked example: X = 1 at k = 0 and 64, 2^-6 at k = 128, zero elsewhere.
    Gate: code 0 at k = 0 with scale -16, all other codes 8, so G = 128 and
    silu(G) = 128 in binary64 (e^-128 < 2^-184).  Up: code 9 at k = 0, 64,
    128 with scales 1, 2^-8, 2^-24 (the fp16 subnormal 0x0001), so
    U = 1 + 2^-8 + 2^-30.  G U = 128.5 + 2^-23 lies just above the bf16
    midpoint between 128 and 129 (spacing 1 there): one rounding gives 129
    (0x4301); rounding U to binary32 first would leave the tie 128.5, which
    goes to the even 128 (0x4300).  A negative up weight mirrors it."""
    n, k, t = 2, 192, 1
    x = np.zeros((t, k), dtype=np.uint16)
    x[0, 0] = x[0, 64] = 0x3F80
    x[0, 128] = 0x3C80
    cg = np.full((n, k // 2), 0x88, dtype=np.uint8)
    cg[:, 0] = 0x80
    sg = np.array([[0xCC00, 0x3C00, 0x3C00]] * n, dtype=np.uint16)
    cu = np.full((n, k // 2), 0x88, dtype=np.uint8)
    cu[0, [0, 32, 64]] = 0x89
    cu[1, [0, 32, 64]] = 0x87
    su = np.array([[0x3C00, 0x1C00, 0x0001]] * n, dtype=np.uint16)
    y = o.linear_swiglu(x, cg, sg, cu, su, n, k, t)
    assert [int(v) for v in y.reshape(-1)] == [0x4301, 0xC301], [hex(int(v)) for v in y.reshape(-1)]


def pin_swiglu_bruteforce(o, trials=4):
    """Exact rational sums for G and U, the gate from the logistic function
    through its tanh form, sigma(g) = (1 + tanh(g / 2)) / 2, a second route
    to silu(g) = g sigma(g); the two agree to a few binary64 ulps, so the bf16
    results agree except where the value lies within that of a rounding
    boundary (at most one bf16 ulp apart, and rarely)."""
    import math
    total = off = 0
    for trial in range(trials):
        n, k, t = 5, 128, 2
        x, cg, sg = _problem(n, k, t, 100 + trial)
        _, cu, su = _problem(n, k, t, 200 + trial)
        y = o.linear_swiglu(x, cg, sg, cu, su, n, k, t)
        G = _exact_sums(x, cg, sg, n, k, t)
        U = _exact_sums(x, cu, su, n, k, t)
        for j in range(t):
            for i in range(n):
                g = float(G[j][i])
                v = Fraction(g * (1.0 + math.tanh(g / 2.0)) / 2.0) * U[j][i]
                want = frac_to_bf16_bits(v)
                got = int(y[j, i])
                total += 1
                if got != want:
                    off += 1
                    assert abs(bf16_exact(got) - bf16_exact(want)) <= abs(bf16_exact(want)) * Fraction(1, 128)
    assert off <= max(1, total // 50), (off, total)


ALL_PINS = [
    pin_worked_examples, pin_fp16_decode, pin_bf16_decode, pin_rounding_nearest_even,
    pin_rounding_vs_torch, pin_weight_bytes, pin_unit_scales_integer_x, pin_unit_scales_matmul,
    pin_exact_bruteforce, pin_all_code8_zero, pin_pow2_scale_invariance, pin_locality,
    pin_token_independence, pin_group_permutation, pin_linear_at,
    pin_add_worked_examples, pin_add_exact_bruteforce, pin_add_all_code8_passes_residual,
    pin_add_zero_residual_and_shift,
    pin_swiglu_zero_gate_or_up, pin_swiglu_saturated_gate, pin_swiglu_single_rounding, pin_swiglu_bruteforce,
]
