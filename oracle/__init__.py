"""CPU oracle for the Q4_G64_FP16 pure Linear op -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The library under
``weight_only_bit_q4_amd`` never imports it and shares no code with it.

The arithmetic lives in ``q4lin_oracle.c`` (plain C, binary64, one rounding to
bfloat16 at the end); this module only builds that file with gcc and marshals
numpy arrays to it.  What it computes, and where the pages define it, is stated
in the C file's header:

* "q4-linear.md", setup table: Q4_G64_FP16 weights (64 weights per FP16
  scale, row-split), ``W[N,K] x X[K,T] -> Y[N,T]``, BF16 in and out;
* "q4-linear.md", test paragraph: independent decode of codes and scales, an
  FP64 matrix product as the oracle;
* "linear-benchmark.md", section 4 table: 34 bytes per 64-weight group.

The other weight formats of the same op (Q5G64_F16S, Q6G64_F16S,
W8G32_F16S, NVFP4, BF16_CTRL; "linear-benchmark.md", sections 0 and 4) are
``linear_fmt`` / ``linear_fmt_at`` with the format's planes; their readings
(bit layouts and code meanings the pages leave open) are stated in the C
file.

Parity status: ``fp16_to_double``, ``bf16_to_double``, ``double_to_bf16``,
``weight_bytes``, ``linear`` and ``linear_at``, and ``e4m3_to_double``,
``e2m1_to_double``, ``fmt_weight_bytes``, ``linear_fmt`` and
``linear_fmt_at`` are each pinned by the CPU test-suite (hand-worked
examples, library special cases, invariants, relations between formats,
exact rational brute force); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "q4lin_oracle.c")
LIB_PATH = os.path.join(_HERE, "libq4lin_oracle.so")


def compile_source(src: str, out: str) -> str:
    """gcc -O2 with OpenMP and without fast-math; atomic replace of ``out``."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=gnu11",
           "-fno-fast-math", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile the C oracle next to its source."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    return compile_source(SOURCE, LIB_PATH)


def _ptr(a, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, lib_path: str):
        lib = ctypes.CDLL(lib_path)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        f64p = ctypes.POINTER(ctypes.c_double)
        i64p = ctypes.POINTER(ctypes.c_int64)
        i64 = ctypes.c_int64
        lib.q4o_fp16_to_double.argtypes = [ctypes.c_uint16]
        lib.q4o_fp16_to_double.restype = ctypes.c_double
        lib.q4o_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.q4o_bf16_to_double.restype = ctypes.c_double
        lib.q4o_double_to_bf16.argtypes = [ctypes.c_double]
        lib.q4o_double_to_bf16.restype = ctypes.c_uint16
        lib.q4o_weight_bytes.argtypes = [i64, i64]
        lib.q4o_weight_bytes.restype = i64
        lib.q4o_linear.argtypes = [u16p, u8p, u16p, u16p, f64p, i64, i64, i64, ctypes.c_int]
        lib.q4o_linear.restype = None
        lib.q4o_linear_add.argtypes = [u16p, u8p, u16p, u16p, u16p, i64, i64, i64, ctypes.c_int]
        lib.q4o_linear_add.restype = None
        lib.q4o_linear_at.argtypes = [u16p, u8p, u16p, i64, i64, i64, i64p, i64p, i64,
                                      u16p, f64p, ctypes.c_int]
        lib.q4o_linear_at.restype = None
        lib.q4o_swiglu.argtypes = [f64p, f64p, u16p, i64]
        lib.q4o_swiglu.restype = None
        lib.q4o_max_threads.argtypes = []
        lib.q4o_max_threads.restype = ctypes.c_int
        vp = ctypes.c_void_p
        lib.q4o_e4m3_to_double.argtypes = [ctypes.c_uint8]
        lib.q4o_e4m3_to_double.restype = ctypes.c_double
        lib.q4o_e2m1_to_double.argtypes = [ctypes.c_uint8]
        lib.q4o_e2m1_to_double.restype = ctypes.c_double
        lib.q4o_fmt_weight_bytes.argtypes = [ctypes.c_int, i64, i64]
        lib.q4o_fmt_weight_bytes.restype = i64
        lib.q4o_linear_fmt.argtypes = [ctypes.c_int, u16p, u8p, u8p, vp, u16p, f64p, i64, i64, i64, ctypes.c_int]
        lib.q4o_linear_fmt.restype = None
        lib.q4o_linear_fmt_at.argtypes = [ctypes.c_int, u16p, u8p, u8p, vp, i64, i64, i64, i64p, i64p, i64,
                                          u16p, ctypes.c_int]
        lib.q4o_linear_fmt_at.restype = None
        self.lib = lib
        self.path = lib_path

    # scalar helpers -------------------------------------------------------
    def fp16_to_double(self, bits: int) -> float:
        return self.lib.q4o_fp16_to_double(int(bits) & 0xFFFF)

    def bf16_to_double(self, bits: int) -> float:
        return self.lib.q4o_bf16_to_double(int(bits) & 0xFFFF)

    def double_to_bf16(self, v: float) -> int:
        return int(self.lib.q4o_double_to_bf16(float(v)))

    def weight_bytes(self, n: int, k: int) -> int:
        return int(self.lib.q4o_weight_bytes(int(n), int(k)))

    def max_threads(self) -> int:
        return int(self.lib.q4o_max_threads())

    def e4m3_to_double(self, bits: int) -> float:
        return self.lib.q4o_e4m3_to_double(int(bits) & 0xFF)

    def e2m1_to_double(self, nib: int) -> float:
        return self.lib.q4o_e2m1_to_double(int(nib) & 0xF)

    def fmt_weight_bytes(self, fmt: int, n: int, k: int) -> int:
        return int(self.lib.q4o_fmt_weight_bytes(int(fmt), int(n), int(k)))

    # other weight formats ---------------------------------------------------
    @staticmethod
    def _prep_fmt(fmt, x, lo, hi, sc, n, k, t):
        if k % 64 != 0 or k < 64:
            raise ValueError("K must be a positive multiple of 64")
        if fmt not in PLANES:
            raise ValueError("unknown format %r" % (fmt,))
        lo_b, hi_b, sc_b = (f(n, k) for f in PLANES[fmt])
        x = np.ascontiguousarray(x, dtype=np.uint16).reshape(-1)
        lo = np.ascontiguousarray(lo).reshape(-1).view(np.uint8)
        hi = np.zeros(1, np.uint8) if hi_b == 0 else np.ascontiguousarray(hi).reshape(-1).view(np.uint8)
        sc = np.zeros(1, np.uint8) if sc_b == 0 else np.ascontiguousarray(sc).reshape(-1).view(np.uint8)
        if x.size != k * t or lo.size != lo_b or (hi_b and hi.size != hi_b) or (sc_b and sc.size != sc_b):
            raise ValueError("plane sizes do not match the format and N, K, T")
        return x, lo, hi, sc

    def linear_fmt(self, fmt: int, x, lo, hi, sc, n: int, k: int, t: int, threads: int = 0,
                   with_acc: bool = False):
        """Y = bf16(W . X) for a weight in format ``fmt`` (FMT_*), given as
        its planes (numpy arrays of any dtype, read as bytes; ``hi`` and
        ``sc`` may be None where the format has none).  Returns bf16 bits
        ``[T, N]`` (and the binary64 sums with ``with_acc``)."""
        x, lo, hi, sc = self._prep_fmt(fmt, x, lo, hi, sc, n, k, t)
        y = np.zeros(t * n, dtype=np.uint16)
        acc = np.zeros(t * n, dtype=np.float64) if with_acc else None
        self.lib.q4o_linear_fmt(int(fmt), _ptr(x, ctypes.c_uint16), _ptr(lo, ctypes.c_uint8),
                                _ptr(hi, ctypes.c_uint8), sc.ctypes.data, _ptr(y, ctypes.c_uint16),
                                _ptr(acc, ctypes.c_double), n, k, t, int(threads))
        y = y.reshape(t, n)
        if with_acc:
            return y, acc.reshape(t, n)
        return y

    def linear_fmt_at(self, fmt: int, x, lo, hi, sc, n: int, k: int, t: int, ns, ts, threads: int = 0):
        """Selected elements ``Y[ns[i], ts[i]]`` of the format-``fmt`` product."""
        x, lo, hi, sc = self._prep_fmt(fmt, x, lo, hi, sc, n, k, t)
        ns = np.ascontiguousarray(ns, dtype=np.int64)
        ts = np.ascontiguousarray(ts, dtype=np.int64)
        if ns.shape != ts.shape or (ns.size and (ns.min() < 0 or ns.max() >= n or ts.min() < 0 or ts.max() >= t)):
            raise ValueError("bad sample indices")
        out = np.zeros(ns.size, dtype=np.uint16)
        self.lib.q4o_linear_fmt_at(int(fmt), _ptr(x, ctypes.c_uint16), _ptr(lo, ctypes.c_uint8),
                                   _ptr(hi, ctypes.c_uint8), sc.ctypes.data, n, k, t,
                                   _ptr(ns, ctypes.c_int64), _ptr(ts, ctypes.c_int64), ns.size,
                                   _ptr(out, ctypes.c_uint16), int(threads))
        return out

    # the product ------------------------------------------------------------
    @staticmethod
    def _prep(x, codes, scales, n, k, t):
        if k % 64 != 0 or k < 64:
            raise ValueError("K must be a positive multiple of 64")
        x = np.ascontiguousarray(x, dtype=np.uint16).reshape(-1)
        codes = np.ascontiguousarray(codes, dtype=np.uint8).reshape(-1)
        scales = np.ascontiguousarray(scales, dtype=np.uint16).reshape(-1)
        if codes.size != n * k // 2 or scales.size != n * (k // 64) or x.size != k * t:
            raise ValueError("array sizes do not match N, K, T")
        return x, codes, scales

    def linear(self, x, codes, scales, n: int, k: int, t: int,
               threads: int = 0, with_acc: bool = False):
        """Y = bf16(W . X).  ``x``: bf16 bits, token-major ``[T, K]``;
        ``codes``: uint8 ``[N, K/2]``; ``scales``: fp16 bits ``[N, K/64]``.
        Returns bf16 bits ``[T, N]`` (token-major) and, with ``with_acc``, the
        unrounded binary64 sums in the same shape."""
        x, codes, scales = self._prep(x, codes, scales, n, k, t)
        y = np.zeros(t * n, dtype=np.uint16)
        acc = np.zeros(t * n, dtype=np.float64) if with_acc else None
        self.lib.q4o_linear(_ptr(x, ctypes.c_uint16), _ptr(codes, ctypes.c_uint8),
                            _ptr(scales, ctypes.c_uint16), _ptr(y, ctypes.c_uint16),
                            _ptr(acc, ctypes.c_double), n, k, t, int(threads))
        y = y.reshape(t, n)
        if with_acc:
            return y, acc.reshape(t, n)
        return y

    def linear_add(self, x, codes, scales, r, n: int, k: int, t: int, threads: int = 0):
        """Y = bf16(W . X + R), rounded once.  ``r``: bf16 bits, token-major
        ``[T, N]`` like the result.  Returns bf16 bits ``[T, N]``."""
        x, codes, scales = self._prep(x, codes, scales, n, k, t)
        r = np.ascontiguousarray(r, dtype=np.uint16).reshape(-1)
        if r.size != t * n:
            raise ValueError("residual size does not match T x N")
        y = np.zeros(t * n, dtype=np.uint16)
        self.lib.q4o_linear_add(_ptr(x, ctypes.c_uint16), _ptr(codes, ctypes.c_uint8),
                                _ptr(scales, ctypes.c_uint16), _ptr(r, ctypes.c_uint16),
                                _ptr(y, ctypes.c_uint16), n, k, t, int(threads))
        return y.reshape(t, n)

    def swiglu(self, g, u):
        """bf16(silu(g) * u) element by element, g and u binary64 sums."""
        g = np.ascontiguousarray(g, dtype=np.float64).reshape(-1)
        u = np.ascontiguousarray(u, dtype=np.float64).reshape(-1)
        if g.size != u.size:
            raise ValueError("gate and up sizes differ")
        y = np.zeros(g.size, dtype=np.uint16)
        self.lib.q4o_swiglu(_ptr(g, ctypes.c_double), _ptr(u, ctypes.c_double), _ptr(y, ctypes.c_uint16), g.size)
        return y

    def linear_swiglu(self, x, codes_g, scales_g, codes_u, scales_u, n: int, k: int, t: int, threads: int = 0):
        """Y = bf16(silu(Wg . X) * (Wu . X)), both sums in binary64 and one
        rounding.  Returns bf16 bits ``[T, N]``."""
        _, g = self.linear(x, codes_g, scales_g, n, k, t, threads=threads, with_acc=True)
        _, u = self.linear(x, codes_u, scales_u, n, k, t, threads=threads, with_acc=True)
        return self.swiglu(g, u).reshape(t, n)

    def linear_at(self, x, codes, scales, n: int, k: int, t: int, ns, ts,
                  threads: int = 0, with_acc: bool = False):
        """Selected elements ``Y[ns[i], ts[i]]`` (bf16 bits), each summed alone."""
        x, codes, scales = self._prep(x, codes, scales, n, k, t)
        ns = np.ascontiguousarray(ns, dtype=np.int64)
        ts = np.ascontiguousarray(ts, dtype=np.int64)
        if ns.shape != ts.shape:
            raise ValueError("ns and ts differ in shape")
        if ns.size and (ns.min() < 0 or ns.max() >= n or ts.min() < 0 or ts.max() >= t):
            raise ValueError("sample index out of range")
        out = np.zeros(ns.size, dtype=np.uint16)
        acc = np.zeros(ns.size, dtype=np.float64) if with_acc else None
        self.lib.q4o_linear_at(_ptr(x, ctypes.c_uint16), _ptr(codes, ctypes.c_uint8),
                               _ptr(scales, ctypes.c_uint16), n, k, t,
                               _ptr(ns, ctypes.c_int64), _ptr(ts, ctypes.c_int64), ns.size,
                               _ptr(out, ctypes.c_uint16), _ptr(acc, ctypes.c_double),
                               int(threads))
        if with_acc:
            return out, acc
        return out


# Weight formats (the pages' "linear-benchmark.md" section 4 table) and the
# byte sizes of their planes (low/code plane, high plane, scale plane).
FMT_Q4, FMT_Q5, FMT_Q6, FMT_W8, FMT_NVFP4, FMT_BF16 = range(6)
PLANES = {
    FMT_Q4: (lambda n, k: n * k // 2, lambda n, k: 0, lambda n, k: n * (k // 64) * 2),
    FMT_Q5: (lambda n, k: n * k // 2, lambda n, k: n * k // 8, lambda n, k: n * (k // 64) * 2),
    FMT_Q6: (lambda n, k: n * k // 2, lambda n, k: n * k // 4, lambda n, k: n * (k // 64) * 2),
    FMT_W8: (lambda n, k: n * k, lambda n, k: 0, lambda n, k: n * (k // 32) * 2),
    FMT_NVFP4: (lambda n, k: n * k // 2, lambda n, k: 0, lambda n, k: n * (k // 16)),
    FMT_BF16: (lambda n, k: n * k * 2, lambda n, k: 0, lambda n, k: 0),
}

_lock = threading.Lock()
_default = None


def default() -> Oracle:
    """The oracle built from ``q4lin_oracle.c`` (compiled on first use if absent)."""
    global _default
    with _lock:
        if _default is None:
            if not os.path.exists(LIB_PATH):
                build(force=True)
            _default = Oracle(LIB_PATH)
        return _default


def fp16_to_double(bits):
    return default().fp16_to_double(bits)


def bf16_to_double(bits):
    return default().bf16_to_double(bits)


def double_to_bf16(v):
    return default().double_to_bf16(v)


def weight_bytes(n, k):
    return default().weight_bytes(n, k)


def linear(*args, **kw):
    return default().linear(*args, **kw)


def linear_add(*args, **kw):
    return default().linear_add(*args, **kw)


def swiglu(*args, **kw):
    return default().swiglu(*args, **kw)


def linear_swiglu(*args, **kw):
    return default().linear_swiglu(*args, **kw)


def linear_at(*args, **kw):
    return default().linear_at(*args, **kw)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns -> binary64 values (exact), for tolerance checks."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def linear_fmt(*args, **kw):
    return default().linear_fmt(*args, **kw)


def linear_fmt_at(*args, **kw):
    return default().linear_fmt_at(*args, **kw)
