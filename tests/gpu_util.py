"""Helpers for the GPU parity tests: device transfer, one call of the op
through the C ABI, and the parity tolerance.

Tolerance (the accuracy bound stated for this operation): every output must
satisfy |y - y_o| <= 1e-2 * |y_o| + 1e-3 * rms(y_o), with y_o the oracle's
bf16 output and rms over the oracle output tensor.  Where only sampled
outputs are computed by the oracle, rms is taken over the sample (an unbiased
estimate of the full-tensor value for a uniform sample).  Bit-identical
values (including infinities) always pass.
"""
from __future__ import annotations

import sys

import numpy as np

import oracle
from oracle import bf16_bits_to_f64

REL = 1e-2
ABS_RMS = 1e-3


def torch():
    import torch as _t
    return _t


def dev(a: np.ndarray):
    """numpy (uint8 / uint16 bits) -> torch device tensor of the same bytes."""
    t = torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return t.from_numpy(a.view(np.int16).copy()).cuda()
    if a.dtype == np.uint8:
        return t.from_numpy(a.copy()).cuda()
    raise TypeError(a.dtype)


def host_bits(tensor) -> np.ndarray:
    return tensor.detach().cpu().contiguous().view(torch().int16).numpy().view(np.uint16)


def announce(msg: str):
    """Name the case on the real stderr before a GPU step (survives capture)."""
    sys.__stderr__.write("[gpu] %s\n" % msg)
    sys.__stderr__.flush()


def run_op(x, codes, scales, n, k, t, y=None, workspace=None, what=""):
    """Run the HIP op on numpy inputs; returns bf16 bits [t, n]."""
    import weight_only_bit_q4_amd as q4
    announce("%s q4lin_linear n=%d k=%d t=%d route=%d" % (what, n, k, t, q4.q4lin_route(n, k, t)))
    th = torch()
    xd = dev(np.asarray(x, dtype=np.uint16).reshape(t, k))
    cd = dev(np.asarray(codes, dtype=np.uint8).reshape(n, k // 2))
    sd = dev(np.asarray(scales, dtype=np.uint16).reshape(n, k // 64))
    yd = q4.linear(xd, cd, sd, y=y, workspace=workspace)
    th.cuda.synchronize()
    return host_bits(yd)


def tolerance_violations(y_gpu, y_ref, rms=None):
    """(number of violations, worst |err| / bound) for bf16 bit arrays."""
    yg = bf16_bits_to_f64(np.asarray(y_gpu).reshape(-1))
    yo = bf16_bits_to_f64(np.asarray(y_ref).reshape(-1))
    same = np.asarray(y_gpu).reshape(-1) == np.asarray(y_ref).reshape(-1)
    finite = np.isfinite(yo)
    if rms is None:
        rms = float(np.sqrt(np.mean(yo[finite] ** 2))) if finite.any() else 0.0
    bound = REL * np.abs(yo) + ABS_RMS * rms
    with np.errstate(invalid="ignore"):
        err = np.abs(yg - yo)
        bad = ~same & ~(err <= bound)
        ratio = np.where(same, 0.0, np.where(bound > 0, err / np.where(bound > 0, bound, 1), np.inf))
    worst = float(np.nanmax(ratio)) if ratio.size else 0.0
    return int(bad.sum()), worst


def assert_close(y_gpu, y_ref, rms=None, what=""):
    nbad, worst = tolerance_violations(y_gpu, y_ref, rms)
    assert nbad == 0, "%s: %d outputs outside tolerance (worst %.3g x bound)" % (what, nbad, worst)
    return worst


def sample_indices(n, t, count, seed, extra_n=(), extra_t=()):
    """Uniform random (n, t) samples plus every combination of the listed
    boundary rows/tokens that fall inside the shape."""
    r = np.random.default_rng(seed)
    ns = list(r.integers(0, n, count))
    ts = list(r.integers(0, t, count))
    en = sorted({v for v in extra_n if 0 <= v < n} | {0, n - 1})
    et = sorted({v for v in extra_t if 0 <= v < t} | {0, t - 1})
    for a in en:
        for b in et:
            ns.append(a)
            ts.append(b)
    return np.array(ns, dtype=np.int64), np.array(ts, dtype=np.int64)


def oracle_full(x, codes, scales, n, k, t):
    return oracle.linear(x, codes, scales, n, k, t)


def oracle_sampled(x, codes, scales, n, k, t, ns, ts):
    return oracle.linear_at(x, codes, scales, n, k, t, ns, ts)
