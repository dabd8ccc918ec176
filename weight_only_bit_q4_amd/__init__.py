"""weight_only_bit_q4_amd -- the Q4_G64_FP16 weight-only Linear on MI355X.

Python binding of the C ABI declared in ``include/q4lin.h``.  The functions
carry the C names and only marshal arguments; every step of the op runs in the
HIP kernels of ``libq4lin.so``.  The library is loaded on the first call
(``load()``) and a missing library raises at once (build it with
``python -m weight_only_bit_q4_amd.build``); there is no fallback path.  The
seeded input generators in ``weight_only_bit_q4_amd.inputs`` import without
it.

``linear`` is a convenience over torch tensors (device memory and streams
only): it checks dtypes/shapes, allocates the output and workspace when the
caller does not pass them, and calls ``q4lin_linear`` on the current stream.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libq4lin.so")

Q4LIN_OK = 0
Q4LIN_E_NULL = 1
Q4LIN_E_SHAPE = 2
Q4LIN_E_ALIGN = 3
Q4LIN_E_WORKSPACE = 4
Q4LIN_E_LAUNCH = 5
Q4LIN_E_FORMAT = 6

Q4LIN_FMT_Q4G64_F16S = 0
Q4LIN_FMT_Q5G64_F16S = 1
Q4LIN_FMT_Q6G64_F16S = 2
Q4LIN_FMT_W8G32_F16S = 3
Q4LIN_FMT_NVFP4 = 4
Q4LIN_FMT_BF16 = 5

Q4LIN_ROUTE_NONE = 0
Q4LIN_ROUTE_GEMV = 1
Q4LIN_ROUTE_SKINNY = 2
Q4LIN_ROUTE_TILED = 3
Q4LIN_ROUTE_DECODE = 4
Q4LIN_ROUTE_MID = 5

EXPORTED = ("q4lin_workspace_bytes", "q4lin_linear", "q4lin_linear_add", "q4lin_linear_pair",
            "q4lin_pair_workspace_bytes", "q4lin_linear_swiglu", "q4lin_swiglu_workspace_bytes",
            "q4lin_status_string", "q4lin_route", "q4lin_version", "q4lin_linear_noalloc",
            "q4lin_noalloc_scratch_bytes", "q4lin_linear_fmt", "q4lin_fmt_weight_bytes",
            "q4lin_fmt_workspace_bytes")


class Q4LinError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__("q4lin: %s (status %d)" % (q4lin_status_string(status), status))


def _load() -> ctypes.CDLL:
    # Device memory and streams come from torch, which carries its own HIP
    # runtime; import it first so libq4lin.so binds to that runtime instead of
    # mapping a second one (pointers and streams are only valid in the runtime
    # that made them).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError("libq4lin.so is not built: run `python -m weight_only_bit_q4_amd.build` "
                          "(expected at %s)" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    i64 = ctypes.c_int64
    vp = ctypes.c_void_p
    lib.q4lin_workspace_bytes.argtypes = [i64, i64, i64]
    lib.q4lin_workspace_bytes.restype = i64
    lib.q4lin_linear.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, ctypes.c_size_t, vp]
    lib.q4lin_linear.restype = ctypes.c_int
    lib.q4lin_linear_add.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp, ctypes.c_size_t, vp]
    lib.q4lin_linear_add.restype = ctypes.c_int
    lib.q4lin_linear_pair.argtypes = [vp, vp, vp, vp, i64, vp, vp, vp, i64, i64, i64, vp, ctypes.c_size_t, vp]
    lib.q4lin_linear_pair.restype = ctypes.c_int
    lib.q4lin_pair_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.q4lin_pair_workspace_bytes.restype = i64
    lib.q4lin_linear_swiglu.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, vp, ctypes.c_size_t, vp]
    lib.q4lin_linear_swiglu.restype = ctypes.c_int
    lib.q4lin_swiglu_workspace_bytes.argtypes = [i64, i64, i64]
    lib.q4lin_swiglu_workspace_bytes.restype = i64
    lib.q4lin_status_string.argtypes = [ctypes.c_int]
    lib.q4lin_status_string.restype = ctypes.c_char_p
    lib.q4lin_route.argtypes = [i64, i64, i64]
    lib.q4lin_route.restype = ctypes.c_int
    lib.q4lin_version.argtypes = []
    lib.q4lin_version.restype = ctypes.c_int
    lib.q4lin_linear_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp]
    lib.q4lin_linear_noalloc.restype = ctypes.c_int
    lib.q4lin_noalloc_scratch_bytes.argtypes = []
    lib.q4lin_noalloc_scratch_bytes.restype = i64
    ci = ctypes.c_int
    lib.q4lin_linear_fmt.argtypes = [ci, vp, vp, vp, vp, vp, i64, i64, i64, vp, ctypes.c_size_t, vp]
    lib.q4lin_linear_fmt.restype = ci
    lib.q4lin_fmt_weight_bytes.argtypes = [ci, i64, i64]
    lib.q4lin_fmt_weight_bytes.restype = i64
    lib.q4lin_fmt_workspace_bytes.argtypes = [ci, i64, i64, i64]
    lib.q4lin_fmt_workspace_bytes.restype = i64
    return lib


_lib = None


def load() -> ctypes.CDLL:
    """Load libq4lin.so (once); raises ImportError when it is not built."""
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib


# -- the C ABI, same names ---------------------------------------------------
def q4lin_workspace_bytes(n: int, k: int, t: int) -> int:
    return int(load().q4lin_workspace_bytes(int(n), int(k), int(t)))


def q4lin_linear(x: int, codes: int, scales: int, y: int, n: int, k: int, t: int,
                 workspace: int, workspace_bytes: int, stream: int) -> int:
    """Raw call: device addresses as integers (0 for NULL); returns the status."""
    return int(load().q4lin_linear(x or None, codes or None, scales or None, y or None,
                                 int(n), int(k), int(t), workspace or None,
                                 int(workspace_bytes), stream or None))


def q4lin_linear_add(x: int, codes: int, scales: int, residual: int, y: int, n: int, k: int, t: int,
                     workspace: int, workspace_bytes: int, stream: int) -> int:
    """Raw call of the LinearAdd entry point (Y = W x X + R); returns the status."""
    return int(load().q4lin_linear_add(x or None, codes or None, scales or None, residual or None, y or None,
                                       int(n), int(k), int(t), workspace or None,
                                       int(workspace_bytes), stream or None))


def q4lin_linear_pair(x: int, codes1: int, scales1: int, y1: int, n1: int, codes2: int, scales2: int, y2: int,
                      n2: int, k: int, t: int, workspace: int, workspace_bytes: int, stream: int) -> int:
    """Raw call of the LinearPair entry point (Y1 = W1 x X, Y2 = W2 x X); returns the status."""
    return int(load().q4lin_linear_pair(x or None, codes1 or None, scales1 or None, y1 or None, int(n1),
                                        codes2 or None, scales2 or None, y2 or None, int(n2), int(k), int(t),
                                        workspace or None, int(workspace_bytes), stream or None))


def q4lin_pair_workspace_bytes(n1: int, n2: int, k: int, t: int) -> int:
    return int(load().q4lin_pair_workspace_bytes(int(n1), int(n2), int(k), int(t)))


def q4lin_linear_swiglu(x: int, codes_gate: int, scales_gate: int, codes_up: int, scales_up: int, y: int,
                        n: int, k: int, t: int, workspace: int, workspace_bytes: int, stream: int) -> int:
    """Raw call of the LinearSwiGLU entry point (Y = silu(Wg x X) * (Wu x X)); returns the status."""
    return int(load().q4lin_linear_swiglu(x or None, codes_gate or None, scales_gate or None, codes_up or None,
                                          scales_up or None, y or None, int(n), int(k), int(t),
                                          workspace or None, int(workspace_bytes), stream or None))


def q4lin_swiglu_workspace_bytes(n: int, k: int, t: int) -> int:
    return int(load().q4lin_swiglu_workspace_bytes(int(n), int(k), int(t)))


def q4lin_linear_noalloc(x: int, codes: int, scales: int, y: int, n: int, k: int, t: int, stream: int) -> int:
    """Raw call of the no-allocation entry point (scratch inside the library); returns the status."""
    return int(load().q4lin_linear_noalloc(x or None, codes or None, scales or None, y or None,
                                           int(n), int(k), int(t), stream or None))


def q4lin_noalloc_scratch_bytes() -> int:
    return int(load().q4lin_noalloc_scratch_bytes())


def q4lin_linear_fmt(fmt: int, x: int, w: int, w_hi: int, scales: int, y: int, n: int, k: int, t: int,
                     workspace: int, workspace_bytes: int, stream: int) -> int:
    """Raw call of the weight-format entry point (Q4LIN_FMT_*); returns the status."""
    return int(load().q4lin_linear_fmt(int(fmt), x or None, w or None, w_hi or None, scales or None, y or None,
                                       int(n), int(k), int(t), workspace or None, int(workspace_bytes),
                                       stream or None))


def q4lin_fmt_weight_bytes(fmt: int, n: int, k: int) -> int:
    return int(load().q4lin_fmt_weight_bytes(int(fmt), int(n), int(k)))


def q4lin_fmt_workspace_bytes(fmt: int, n: int, k: int, t: int) -> int:
    return int(load().q4lin_fmt_workspace_bytes(int(fmt), int(n), int(k), int(t)))


def q4lin_status_string(status: int) -> str:
    return load().q4lin_status_string(int(status)).decode()


def q4lin_route(n: int, k: int, t: int) -> int:
    return int(load().q4lin_route(int(n), int(k), int(t)))


def q4lin_version() -> int:
    return int(load().q4lin_version())


# -- torch convenience (marshalling only) -------------------------------------
def linear(x, codes, scales, y=None, workspace=None, stream=None, residual=None):
    """Y = W x X (or, with ``residual``, the LinearAdd Y = W x X + R) on torch
    device tensors.

    ``x``: uint16/int16/bfloat16 ``[T, K]`` (bf16 bits, token-major);
    ``codes``: uint8 ``[N, K/2]``; ``scales``: float16/int16/uint16 ``[N, K/64]``;
    ``y``: optional bfloat16/int16/uint16 ``[T, N]`` output; ``residual``:
    optional ``[T, N]`` bf16 bits (may be ``y`` itself).  Returns ``y``.
    """
    import torch

    t, k = x.shape
    n = codes.shape[0]
    if codes.shape[1] * 2 != k or tuple(scales.shape) != (n, k // 64):
        raise ValueError("shape mismatch: x %s codes %s scales %s" % (tuple(x.shape), tuple(codes.shape),
                                                                      tuple(scales.shape)))
    for name, ten, size in (("x", x, 2), ("codes", codes, 1), ("scales", scales, 2)):
        if not ten.is_contiguous() or ten.element_size() != size:
            raise ValueError("%s must be contiguous with %d-byte elements" % (name, size))
    if y is None:
        y = torch.empty((t, n), dtype=torch.bfloat16, device=x.device)
    if tuple(y.shape) != (t, n) or y.element_size() != 2 or not y.is_contiguous():
        raise ValueError("y must be a contiguous [T, N] tensor of 2-byte elements")
    need = q4lin_workspace_bytes(n, k, t)
    if need < 0:
        raise Q4LinError(-need)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else 0
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    if residual is None:
        st = q4lin_linear(x.data_ptr(), codes.data_ptr(), scales.data_ptr(), y.data_ptr(), n, k, t,
                          ws_ptr, ws_bytes, stream)
    else:
        if tuple(residual.shape) != (t, n) or residual.element_size() != 2 or not residual.is_contiguous():
            raise ValueError("residual must be a contiguous [T, N] tensor of 2-byte elements")
        st = q4lin_linear_add(x.data_ptr(), codes.data_ptr(), scales.data_ptr(), residual.data_ptr(),
                              y.data_ptr(), n, k, t, ws_ptr, ws_bytes, stream)
    if st != Q4LIN_OK:
        raise Q4LinError(st)
    return y


def linear_pair(x, codes1, scales1, codes2, scales2, y1=None, y2=None, workspace=None, stream=None):
    """LinearPair on torch device tensors: ``(W1 x X, W2 x X)`` for two weights
    of the same K over one ``x`` (layouts as in ``linear``).  Returns
    ``(y1, y2)``."""
    import torch

    t, k = x.shape
    n1, n2 = codes1.shape[0], codes2.shape[0]
    for i, (c, sc) in enumerate(((codes1, scales1), (codes2, scales2)), 1):
        n = c.shape[0]
        if c.shape[1] * 2 != k or tuple(sc.shape) != (n, k // 64):
            raise ValueError("shape mismatch: x %s codes%d %s scales%d %s" % (tuple(x.shape), i, tuple(c.shape),
                                                                           i, tuple(sc.shape)))
    for name, ten, size in (("x", x, 2), ("codes1", codes1, 1), ("scales1", scales1, 2), ("codes2", codes2, 1),
                            ("scales2", scales2, 2)):
        if not ten.is_contiguous() or ten.element_size() != size:
            raise ValueError("%s must be contiguous with %d-byte elements" % (name, size))
    outs = []
    for y, n in ((y1, n1), (y2, n2)):
        if y is None:
            y = torch.empty((t, n), dtype=torch.bfloat16, device=x.device)
        if tuple(y.shape) != (t, n) or y.element_size() != 2 or not y.is_contiguous():
            raise ValueError("outputs must be contiguous [T, N] tensors of 2-byte elements")
        outs.append(y)
    need = q4lin_pair_workspace_bytes(n1, n2, k, t)
    if need < 0:
        raise Q4LinError(-need)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else 0
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    st = q4lin_linear_pair(x.data_ptr(), codes1.data_ptr(), scales1.data_ptr(), outs[0].data_ptr(), n1,
                           codes2.data_ptr(), scales2.data_ptr(), outs[1].data_ptr(), n2, k, t,
                           ws_ptr, ws_bytes, stream)
    if st != Q4LIN_OK:
        raise Q4LinError(st)
    return outs[0], outs[1]


def linear_swiglu(x, codes_gate, scales_gate, codes_up, scales_up, y=None, workspace=None, stream=None):
    """LinearSwiGLU on torch device tensors: ``silu(Wg x X) * (Wu x X)``, both
    weights with ``linear``'s layouts and the same shape.  Returns ``y``."""
    import torch

    t, k = x.shape
    n = codes_gate.shape[0]
    for name, c, sc in (("gate", codes_gate, scales_gate), ("up", codes_up, scales_up)):
        if tuple(c.shape) != (n, k // 2) or tuple(sc.shape) != (n, k // 64):
            raise ValueError("shape mismatch: x %s %s codes %s scales %s" % (tuple(x.shape), name, tuple(c.shape),
                                                                          tuple(sc.shape)))
    for name, ten, size in (("x", x, 2), ("codes_gate", codes_gate, 1), ("scales_gate", scales_gate, 2),
                            ("codes_up", codes_up, 1), ("scales_up", scales_up, 2)):
        if not ten.is_contiguous() or ten.element_size() != size:
            raise ValueError("%s must be contiguous with %d-byte elements" % (name, size))
    if y is None:
        y = torch.empty((t, n), dtype=torch.bfloat16, device=x.device)
    if tuple(y.shape) != (t, n) or y.element_size() != 2 or not y.is_contiguous():
        raise ValueError("y must be a contiguous [T, N] tensor of 2-byte elements")
    need = q4lin_swiglu_workspace_bytes(n, k, t)
    if need < 0:
        raise Q4LinError(-need)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else 0
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    st = q4lin_linear_swiglu(x.data_ptr(), codes_gate.data_ptr(), scales_gate.data_ptr(), codes_up.data_ptr(),
                             scales_up.data_ptr(), y.data_ptr(), n, k, t, ws_ptr, ws_bytes, stream)
    if st != Q4LIN_OK:
        raise Q4LinError(st)
    return y


def linear_fmt(fmt, x, w, w_hi=None, scales=None, y=None, stream=None):
    """Y = W x X for a weight in format ``fmt`` (Q4LIN_FMT_*) on torch device
    tensors: ``x`` ``[T, K]`` bf16 bits; ``w``, ``w_hi``, ``scales`` the
    format's planes as laid out in ``include/q4lin.h`` (any dtype, read as
    bytes; ``w`` gives N as its first dimension).  Returns ``y`` ``[T, N]``."""
    import torch

    t, k = x.shape
    n = w.shape[0]
    if not x.is_contiguous() or x.element_size() != 2:
        raise ValueError("x must be contiguous with 2-byte elements")
    for name, ten in (("w", w), ("w_hi", w_hi), ("scales", scales)):
        if ten is not None and not ten.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    if y is None:
        y = torch.empty((t, n), dtype=torch.bfloat16, device=x.device)
    if tuple(y.shape) != (t, n) or y.element_size() != 2 or not y.is_contiguous():
        raise ValueError("y must be a contiguous [T, N] tensor of 2-byte elements")
    need = q4lin_fmt_workspace_bytes(fmt, n, k, t)
    if need < 0:
        raise Q4LinError(-need)
    ws = torch.empty(need, dtype=torch.uint8, device=x.device) if need > 0 else None
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    st = q4lin_linear_fmt(fmt, x.data_ptr(), w.data_ptr(), w_hi.data_ptr() if w_hi is not None else 0,
                          scales.data_ptr() if scales is not None else 0, y.data_ptr(), n, k, t,
                          ws.data_ptr() if ws is not None else 0, need, stream)
    if st != Q4LIN_OK:
        raise Q4LinError(st)
    return y
