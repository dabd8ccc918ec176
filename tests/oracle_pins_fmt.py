"""Pins for the oracle's other weight formats (Q5G64_F16S, Q6G64_F16S,
W8G32_F16S, NVFP4, BF16_CTRL): checks against facts that do not come from
the oracle itself.  Like ``oracle_pins``, each ``pin_*`` takes an
``oracle.Oracle`` so that the mutant test can run them on broken copies.

Where each fact comes from:

* the pages' weight-format table ("linear-benchmark.md", section 4): bytes
  per group 42 (Q5, per 64), 50 (Q6, per 64), 34 (W8, per 32), 9 (NVFP4, per
  16) and 2 N K for BF16_CTRL;
* hand-worked examples (``tests/golden/worked_examples_fmt.json``), derived
  on paper from the readings stated in the oracle;
* library routines: torch's float8 E4M3 decode, numpy's float16 decode, the
  OCP E2M1 value table (0, 0.5, 1, 1.5, 2, 3, 4, 6), numpy's binary64
  product, exact rationals;
* relations between formats that share a weight matrix: W8 with codes
  q - 8 and each Q4 scale on both 32-halves is the Q4 weight; Q6 with high
  pair h + 1 is the Q5 weight with high bit h; Q5 with high bits 0 is the Q4
  weight minus 8 scales.  The Q4 oracle these lean on is pinned on its own.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

from oracle_pins import frac_to_bf16_bits, torch_bf16_decode, torch_f32_to_bf16_bits, _h

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_examples_fmt.json")
FMT = {"Q4": 0, "Q5": 1, "Q6": 2, "W8": 3, "NVFP4": 4, "BF16": 5}
E2M1_OCP = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # OCP microscaling spec, E2M1 magnitudes


def plane_sizes(fmt, n, k):
    """Bytes of the (code, high, scale) planes, from the readings."""
    return {0: (n * k // 2, 0, n * k // 32), 1: (n * k // 2, n * k // 8, n * k // 32),
            2: (n * k // 2, n * k // 4, n * k // 32), 3: (n * k, 0, n * k // 16),
            4: (n * k // 2, 0, n * k // 16), 5: (2 * n * k, 0, 0)}[fmt]


def load_examples():
    with open(GOLDEN) as f:
        return json.load(f)["examples"]


def materialize(ex):
    fmt = FMT[ex["fmt"]]
    n, k, t = ex["n"], ex["k"], ex["t"]
    lo_b, hi_b, sc_b = plane_sizes(fmt, n, k)
    if fmt == FMT["BF16"]:
        lo = np.full(n * k, _h(ex["lo"]["fill"]), dtype=np.uint16)
    else:
        lo = np.full(lo_b, _h(ex["lo"]["fill"]), dtype=np.uint8)
    for key, v in ex["lo"].get("set", {}).items():
        lo[int(key)] = _h(v)
    hi = None
    if hi_b:
        hi = np.full(hi_b, _h(ex["hi"]["fill"]), dtype=np.uint8)
        for key, v in ex["hi"].get("set", {}).items():
            hi[int(key)] = _h(v)
    sc = None
    if sc_b:
        dt = np.uint8 if fmt == FMT["NVFP4"] else np.uint16
        sc = np.array([_h(v) for v in ex["scales"]], dtype=dt)
    x = np.full(k * t, _h(ex["x"]["fill"]), dtype=np.uint16)
    for key, v in ex["x"].get("set", {}).items():
        x[int(key)] = _h(v)
    y = np.array([_h(v) for v in ex["y"]], dtype=np.uint16)
    return fmt, x.reshape(t, k), lo, hi, sc, y


def pin_fmt_worked_examples(o):
    for ex in load_examples():
        fmt, x, lo, hi, sc, want = materialize(ex)
        got = o.linear_fmt(fmt, x, lo, hi, sc, ex["n"], ex["k"], ex["t"]).reshape(-1)
        assert np.array_equal(got, want), "%s: got %s want %s" % (
            ex["name"], [hex(v) for v in got], [hex(v) for v in want])


def pin_fmt_weight_bytes(o):
    # the pages' table: bytes per group and group size
    table = {FMT["Q4"]: (34, 64), FMT["Q5"]: (42, 64), FMT["Q6"]: (50, 64), FMT["W8"]: (34, 32),
             FMT["NVFP4"]: (9, 16)}
    for n, k in [(6144, 5120), (4096, 5120), (14336, 5120), (34816, 5120), (5120, 17408), (512, 1024)]:
        for f, (b, g) in table.items():
            assert o.fmt_weight_bytes(f, n, k) == n * k // g * b
        assert o.fmt_weight_bytes(FMT["BF16"], n, k) == 2 * n * k
    assert o.fmt_weight_bytes(FMT["Q4"], 6144, 5120) == 16_711_680
    # the planes of each format add up to it
    for f in FMT.values():
        assert sum(plane_sizes(f, 512, 1024)) == o.fmt_weight_bytes(f, 512, 1024)


def pin_e4m3_decode(o):
    import torch
    allb = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(allb.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([o.e4m3_to_double(int(b)) for b in allb])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), [hex(int(b)) for b in allb[~same]][:8]
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def pin_e2m1_decode(o):
    for nib in range(16):
        mag = E2M1_OCP[nib & 7]
        want = -mag if nib & 8 else mag
        got = o.e2m1_to_double(nib)
        assert got == want and (np.signbit(got) == bool(nib & 8)), (nib, got, want)


def _q4_like(r, n, k):
    return r.integers(0, 256, size=(n, k // 2), dtype=np.uint8)


def pin_w8_is_q4_weight(o):
    """W8 with codes q - 8 (q the Q4 codes) and each Q4 scale repeated for
    both 32-halves of its group is the same weight matrix: identical outputs."""
    r = np.random.default_rng(41)
    for n, k, t in [(5, 128, 3), (17, 320, 2)]:
        codes = _q4_like(r, n, k)
        q = np.empty((n, k), dtype=np.int64)
        q[:, 0::2] = codes & 0xF
        q[:, 1::2] = codes >> 4
        w8 = (q - 8).astype(np.int8)
        sv = (r.choice([-1, 1], (n, k // 64)) * np.ldexp(r.uniform(1, 2, (n, k // 64)),
                                                         r.integers(-14, 8, (n, k // 64))))
        s = sv.astype(np.float16).view(np.uint16)
        s32 = np.repeat(s, 2, axis=1)
        x = torch_f32_to_bf16_bits(r.standard_normal((t, k)).astype(np.float32))
        a = o.linear(x, codes, s, n, k, t)
        b = o.linear_fmt(FMT["W8"], x, w8, None, s32, n, k, t)
        assert np.array_equal(a, b)
        assert np.array_equal(o.linear_fmt(FMT["Q4"], x, codes, None, s, n, k, t), a)


def _spread_bits(h, per):
    """(n, k) small integers -> packed plane, `per` bits each, k = (8/per) b + i in bits per*i of byte b."""
    n, k = h.shape
    m = 8 // per
    out = np.zeros((n, k // m), dtype=np.int64)
    for i in range(m):
        out |= h[:, i::m].astype(np.int64) << (per * i)
    return out.astype(np.uint8)


def pin_q6_q5_relation(o):
    """Q6 with high pair h + 1 is Q5 with high bit h (q - 32 = lo + 16 (h + 1)
    - 32 = lo + 16 h - 16); Q5 with high bits 0 is Q4 minus 8 scales."""
    r = np.random.default_rng(43)
    n, k, t = 9, 192, 4
    lo = _q4_like(r, n, k)
    h = r.integers(0, 2, size=(n, k))
    s = np.ldexp(r.uniform(1, 2, (n, k // 64)), r.integers(-10, 4, (n, k // 64))).astype(np.float16).view(np.uint16)
    x = torch_f32_to_bf16_bits(r.standard_normal((t, k)).astype(np.float32))
    a = o.linear_fmt(FMT["Q5"], x, lo, _spread_bits(h, 1), s, n, k, t)
    b = o.linear_fmt(FMT["Q6"], x, lo, _spread_bits(h + 1, 2), s, n, k, t)
    assert np.array_equal(a, b)
    # high bits 0, unit scales, small-integer activations: exact integers
    ones = np.full((n, k // 64), 0x3C00, dtype=np.uint16)
    xi = r.integers(-3, 4, size=(t, k))
    xb = torch_f32_to_bf16_bits(xi.astype(np.float32))
    _, acc5 = o.linear_fmt(FMT["Q5"], xb, lo, np.zeros(n * k // 8, np.uint8), ones, n, k, t, with_acc=True)
    _, acc4 = o.linear(xb, lo, ones, n, k, t, with_acc=True)
    assert np.array_equal(acc5, acc4 - 8.0 * xi.sum(axis=1)[:, None])


def pin_bf16_matmul(o):
    """BF16_CTRL with small-integer weights and activations: numpy's binary64
    product is exact, so after the (separately pinned) rounding it must match
    bit for bit; and a general case against exact rationals."""
    r = np.random.default_rng(47)
    n, k, t = 12, 256, 3
    wi = r.integers(-9, 10, size=(n, k))
    xi = r.integers(-5, 6, size=(t, k))
    w = torch_f32_to_bf16_bits(wi.astype(np.float32))
    x = torch_f32_to_bf16_bits(xi.astype(np.float32))
    ref = (xi @ wi.T).astype(np.float64)
    want = np.array([[o.double_to_bf16(v) for v in row] for row in ref], dtype=np.uint16)
    assert np.array_equal(o.linear_fmt(FMT["BF16"], x, w, None, None, n, k, t), want)


def _weights_exact(fmt, lo, hi, sc, n, k):
    """W as exact rationals from independent decoders (numpy float16, torch
    E4M3, the OCP E2M1 table) and the readings' bit layouts."""
    import torch
    W = [[None] * k for _ in range(n)]
    if fmt == FMT["BF16"]:
        vals = torch_bf16_decode(lo.reshape(-1)).reshape(n, k)
        return [[Fraction(float(vals[i, j])) for j in range(k)] for i in range(n)]
    nib = None
    if fmt != FMT["W8"]:
        lb = lo.reshape(n, k // 2)
        nib = np.empty((n, k), dtype=np.int64)
        nib[:, 0::2] = lb & 0xF
        nib[:, 1::2] = lb >> 4
    if fmt == FMT["NVFP4"]:
        sv = torch.from_numpy(sc.reshape(-1).copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        sv = sv.reshape(n, k // 16)
    else:
        sv = sc.reshape(-1).view(np.float16).astype(np.float64).reshape(n, -1)
    for i in range(n):
        for j in range(k):
            if fmt == FMT["Q5"]:
                q = int(nib[i, j]) | (((int(hi.reshape(n, -1)[i, j // 8]) >> (j % 8)) & 1) << 4)
                W[i][j] = (q - 16) * Fraction(float(sv[i, j // 64]))
            elif fmt == FMT["Q6"]:
                q = int(nib[i, j]) | (((int(hi.reshape(n, -1)[i, j // 4]) >> (2 * (j % 4))) & 3) << 4)
                W[i][j] = (q - 32) * Fraction(float(sv[i, j // 64]))
            elif fmt == FMT["W8"]:
                c = int(lo.reshape(n, k)[i, j].astype(np.int8))
                W[i][j] = c * Fraction(float(sv[i, j // 32]))
            elif fmt == FMT["NVFP4"]:
                v = int(nib[i, j])
                e = Fraction(E2M1_OCP[v & 7]) * (-1 if v & 8 else 1)
                W[i][j] = e * Fraction(float(sv[i, j // 16]))
    return W


def _random_planes(r, fmt, n, k):
    lo_b, hi_b, sc_b = plane_sizes(fmt, n, k)
    if fmt == FMT["BF16"]:
        w = (r.standard_normal(n * k) * np.ldexp(1.0, r.integers(-12, 12, n * k))).astype(np.float32)
        lo = torch_f32_to_bf16_bits(w)
    else:
        lo = r.integers(0, 256, size=lo_b, dtype=np.uint8)
    hi = r.integers(0, 256, size=hi_b, dtype=np.uint8) if hi_b else None
    if fmt == FMT["NVFP4"]:
        sc = r.integers(0, 0x7F, size=sc_b, dtype=np.uint8)      # finite E4M3, both signs
        sc |= (r.integers(0, 2, size=sc_b) << 7).astype(np.uint8)
    elif sc_b:
        sv = r.choice([-1, 1], sc_b // 2) * np.ldexp(r.uniform(1, 2, sc_b // 2), r.integers(-24, 8, sc_b // 2))
        sc = sv.astype(np.float16).view(np.uint16)
    else:
        sc = None
    return lo, hi, sc


def pin_fmt_bruteforce(o, trials=2):
    """Exact rational sums with an exact round-to-nearest-even, every format,
    tiny shapes, wide-range scales and activations."""
    r = np.random.default_rng(53)
    for fmt in (FMT["Q5"], FMT["Q6"], FMT["W8"], FMT["NVFP4"], FMT["BF16"]):
        for trial in range(trials):
            n, k, t = int(r.integers(1, 4)), 64 * int(r.integers(1, 3)), int(r.integers(1, 3))
            lo, hi, sc = _random_planes(r, fmt, n, k)
            xv = (r.standard_normal((t, k)) * np.ldexp(1.0, r.integers(-12, 12, (t, k)))).astype(np.float32)
            x = torch_f32_to_bf16_bits(xv)
            xs = torch_bf16_decode(x.reshape(-1)).reshape(t, k)
            W = _weights_exact(fmt, lo, hi, sc, n, k)
            want = np.array([[frac_to_bf16_bits(sum(W[i][j] * Fraction(float(xs[tt, j])) for j in range(k)))
                              for i in range(n)] for tt in range(t)], dtype=np.uint16)
            got = o.linear_fmt(fmt, x, lo, hi, sc, n, k, t)
            assert np.array_equal(got, want), "fmt %d trial %d (n=%d k=%d t=%d)" % (fmt, trial, n, k, t)


def pin_fmt_linear_at(o):
    r = np.random.default_rng(59)
    for fmt in (FMT["Q5"], FMT["Q6"], FMT["W8"], FMT["NVFP4"], FMT["BF16"]):
        n, k, t = 11, 192, 5
        lo, hi, sc = _random_planes(r, fmt, n, k)
        x = torch_f32_to_bf16_bits(r.standard_normal((t, k)).astype(np.float32))
        full = o.linear_fmt(fmt, x, lo, hi, sc, n, k, t)
        ns, ts = r.integers(0, n, 30), r.integers(0, t, 30)
        assert np.array_equal(o.linear_fmt_at(fmt, x, lo, hi, sc, n, k, t, ns, ts), full[ts, ns])


ALL_PINS = [pin_fmt_worked_examples, pin_fmt_weight_bytes, pin_e4m3_decode, pin_e2m1_decode, pin_w8_is_q4_weight,
            pin_q6_q5_relation, pin_bf16_matmul, pin_fmt_bruteforce, pin_fmt_linear_at]
