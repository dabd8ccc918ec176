"""Seeded synthetic inputs for the Q4_G64_FP16 Linear op.

This module only draws random numbers and packs them into the storage format;
it holds none of the op's arithmetic.  Both the GPU path's tests/benchmark and
the CPU oracle are fed from here.

Storage format (the Q4_G64_FP16 group of "linear-benchmark.md" section 4:
32 code bytes + one 2-byte FP16 scale per 64 weights):

* ``codes``  -- uint8 ``[N, K/2]`` row-major; byte ``j`` of row ``n`` holds the
  code of ``k = 2j`` in its low nibble and ``k = 2j+1`` in its high nibble;
* ``scales`` -- uint16 FP16 bit patterns ``[N, K/64]`` row-major; scale ``g``
  covers ``k`` in ``[64g, 64g+64)``;
* ``x``      -- uint16 BF16 bit patterns, token-major ``[T, K]`` (element
  ``(k, t)`` at ``t*K + k``); the output uses the same order, ``[T, N]``.

Value distributions follow the workload descriptions: codes uniform in 0..15,
scales drawn uniformly from ``[2^-7, 2^-5]`` then rounded to FP16, activations
drawn from N(0, 1) in binary32 then rounded to BF16.  Every stream is seeded
from ``numpy.random.PCG64`` through ``SeedSequence([seed, stream])``.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

STREAM_CODES = 0
STREAM_SCALES = 1
STREAM_X = 2

BASE_SEED = 20261202


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(stream)])))


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """binary32 -> bfloat16 bit patterns, round to nearest even (NaN kept quiet)."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(np.asarray(v, dtype=np.float32))
    if nan.any():
        out[nan] = 0x7FC0
    return out


def gen_codes(n: int, k: int, seed: int) -> np.ndarray:
    """uint8 [N, K/2]: two independent uniform 4-bit codes per byte."""
    r = _rng(seed, STREAM_CODES)
    return r.integers(0, 256, size=(n, k // 2), dtype=np.uint8)


def gen_scales(n: int, k: int, seed: int, lo: float = 2.0 ** -7, hi: float = 2.0 ** -5) -> np.ndarray:
    """uint16 FP16 bits [N, K/64], uniform in [lo, hi] before rounding to FP16."""
    r = _rng(seed, STREAM_SCALES)
    s = r.uniform(lo, hi, size=(n, k // 64))
    return s.astype(np.float16).view(np.uint16)


def gen_x(k: int, t: int, seed: int) -> np.ndarray:
    """uint16 BF16 bits [T, K] (token-major), N(0,1) drawn in binary32."""
    r = _rng(seed, STREAM_X)
    v = r.standard_normal(size=(t, k), dtype=np.float32)
    return f32_to_bf16_bits(v)


# The other weight formats (the weight-format table of "linear-benchmark.md"
# section 4), numbered as the library's Q4LIN_FMT_* values; the plane layouts
# are the ones stated in include/q4lin.h.
FMT_Q4, FMT_Q5, FMT_Q6, FMT_W8, FMT_NVFP4, FMT_BF16 = range(6)
FMT_NAMES = {FMT_Q4: "Q4G64_F16S", FMT_Q5: "Q5G64_F16S", FMT_Q6: "Q6G64_F16S", FMT_W8: "W8G32_F16S",
             FMT_NVFP4: "NVFP4", FMT_BF16: "BF16_CTRL"}


def gen_fmt_weight(fmt: int, n: int, k: int, seed: int):
    """(w, w_hi, scales) planes of an N x K weight in format ``fmt``, seeded:
    code bytes uniform (every code equally likely; W8 bytes uniform in
    -128..127), high planes uniform, fp16 scales uniform in [2^-7, 2^-5]
    (one per 64 weights, per 32 for W8), NVFP4 E4M3 scales uniform over the
    positive encodings with exponent field 4..9 (about 2^-3..2^2); BF16
    weights N(0, 1/16^2) rounded to bf16.  Planes that a format lacks are
    None."""
    r = _rng(seed, STREAM_CODES)
    if fmt == FMT_Q4:
        return gen_codes(n, k, seed), None, gen_scales(n, k, seed)
    if fmt in (FMT_Q5, FMT_Q6):
        lo = r.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
        hi = r.integers(0, 256, size=(n, k // (8 if fmt == FMT_Q5 else 4)), dtype=np.uint8)
        return lo, hi, gen_scales(n, k, seed)
    if fmt == FMT_W8:
        w = r.integers(0, 256, size=(n, k), dtype=np.uint8)
        s = _rng(seed, STREAM_SCALES).uniform(2.0 ** -7, 2.0 ** -5, size=(n, k // 32))
        return w, None, s.astype(np.float16).view(np.uint16)
    if fmt == FMT_NVFP4:
        w = r.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
        s = _rng(seed, STREAM_SCALES).integers(0x20, 0x50, size=(n, k // 16), dtype=np.uint8)
        return w, None, s
    if fmt == FMT_BF16:
        v = r.standard_normal(size=(n, k), dtype=np.float32) * np.float32(1.0 / 16)
        return f32_to_bf16_bits(v), None, None
    raise ValueError("unknown format %r" % (fmt,))


@dataclass(frozen=True)
class Problem:
    n: int
    k: int
    t: int
    seed: int


def gen_problem(n: int, k: int, t: int, seed: int):
    """(x [T,K] bf16 bits, codes [N,K/2] u8, scales [N,K/64] fp16 bits)."""
    return gen_x(k, t, seed), gen_codes(n, k, seed), gen_scales(n, k, seed)


# The workloads: shapes and token counts with the distributions above.
WORKLOADS = {
    "small_512x1024_t4": dict(shapes=[(512, 1024)], ts=[4]),
    "decode_6144x5120_t1": dict(shapes=[(6144, 5120)], ts=[1]),
    "sweep_6144x5120_t1_128": dict(shapes=[(6144, 5120)], ts=list(range(1, 129))),
    "prefill_6144x5120_t1024": dict(shapes=[(6144, 5120)], ts=[1024, 512, 384, 385, 640, 641]),
    "large_shapes_t1_t1024": dict(shapes=[(14336, 5120), (34816, 5120), (5120, 17408)], ts=[1, 1024]),
}


def workload_seed(name: str) -> int:
    return BASE_SEED + list(WORKLOADS).index(name)
