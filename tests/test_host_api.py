"""The C-ABI library on the host: it loads, exports every symbol the header
declares, and rejects bad arguments before any HIP call (no GPU needed: every
call here returns from host-side validation)."""
import os
import re

import pytest

import weight_only_bit_q4_amd as q

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "q4lin.h")


def declared_functions():
    src = open(HEADER).read()
    return re.findall(r"Q4LIN_API\s+[\w\s\*]+?\b(q4lin_\w+)\s*\(", src)


def test_header_declares_the_binding_names():
    assert sorted(declared_functions()) == sorted(q.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = q.load()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for st in range(0, 7):
        assert q.q4lin_status_string(st)
    assert q.q4lin_status_string(99) == "unknown status"


@pytest.mark.parametrize("n,k,t", [(8, 0, 1), (8, 32, 1), (8, 96, 1), (8, 100, 1), (-1, 64, 1),
                                   (8, 64, -1), (1 << 25, 64, 1), (8, 64, (1 << 21) + 1),
                                   (8, (1 << 20) + 64, 1)])
def test_shape_rejected(n, k, t):
    assert q.q4lin_workspace_bytes(n, k, t) == -q.Q4LIN_E_SHAPE
    assert q.q4lin_route(n, k, t) == -q.Q4LIN_E_SHAPE
    st = q.q4lin_linear(0x1000, 0x1000, 0x1000, 0x1000, n, k, t, 0x1000, 1 << 30, 0)
    assert st == q.Q4LIN_E_SHAPE


@pytest.mark.parametrize("n,k,t", [
    (64, 1 << 20, 1024),        # float16 activation copy 2 GiB: past the tiled kernels' 32-bit offsets
    (1 << 24, 4096, 160),       # scale plane n * k / 32 = 2 GiB
])
def test_tiled_route_rejects_shapes_past_32bit_offsets(n, k, t):
    # the shapes pass the general limits and would take the many-token route
    assert q.q4lin_route(n, k, t) == q.Q4LIN_ROUTE_TILED
    assert q.q4lin_workspace_bytes(n, k, t) == -q.Q4LIN_E_SHAPE
    st = q.q4lin_linear(0x1000, 0x1000, 0x1000, 0x1000, n, k, t, 0x1000, 1 << 40, 0)
    assert st == q.Q4LIN_E_SHAPE
    # just inside both bounds the query answers with a size
    assert q.q4lin_workspace_bytes(64, 1 << 19, 1024) > 0


def test_empty_product_is_a_no_op():
    for n, t in [(0, 5), (6, 0), (0, 0)]:
        assert q.q4lin_route(n, 128, t) == q.Q4LIN_ROUTE_NONE
        assert q.q4lin_workspace_bytes(n, 128, t) == 0
        assert q.q4lin_linear(0, 0, 0, 0, n, 128, t, 0, 0, 0) == q.Q4LIN_OK


@pytest.mark.parametrize("which", range(4))
def test_null_pointer_rejected(which):
    ptrs = [0x1000, 0x1000, 0x1000, 0x1000]
    ptrs[which] = 0
    assert q.q4lin_linear(*ptrs, 64, 128, 1, 0, 0, 0) == q.Q4LIN_E_NULL


@pytest.mark.parametrize("which,addr", [(0, 0x1008), (1, 0x1004), (2, 0x1001), (3, 0x1001)])
def test_misaligned_pointer_rejected(which, addr):
    ptrs = [0x1000, 0x1000, 0x1000, 0x1000]
    ptrs[which] = addr
    assert q.q4lin_linear(*ptrs, 64, 128, 1, 0, 0, 0) == q.Q4LIN_E_ALIGN


def test_workspace_checks():
    n, k, t = 256, 512, 300
    need = q.q4lin_workspace_bytes(n, k, t)
    assert need > 0
    p = 0x10000
    assert q.q4lin_linear(p, p, p, p, n, k, t, p, need - 1, 0) == q.Q4LIN_E_WORKSPACE
    assert q.q4lin_linear(p, p, p, p, n, k, t, 0, need, 0) == q.Q4LIN_E_NULL
    assert q.q4lin_linear(p, p, p, p, n, k, t, p + 16, need, 0) == q.Q4LIN_E_ALIGN


def test_routes_and_workspace_sizes():
    # T = 1 is the single-token route, with no workspace
    assert q.q4lin_route(6144, 5120, 1) == q.Q4LIN_ROUTE_DECODE
    assert q.q4lin_workspace_bytes(6144, 5120, 1) == 0
    for t in (1, 2, 3, 4, 5, 16, 64, 128, 512, 1024):
        r = q.q4lin_route(6144, 5120, t)
        assert r in (q.Q4LIN_ROUTE_DECODE, q.Q4LIN_ROUTE_GEMV, q.Q4LIN_ROUTE_SKINNY, q.Q4LIN_ROUTE_TILED,
                     q.Q4LIN_ROUTE_MID)
        ws = q.q4lin_workspace_bytes(6144, 5120, t)
        if r == q.Q4LIN_ROUTE_TILED:
            # float16 activations padded to 32 tokens plus one int32 per token
            tp = (t + 31) // 32 * 32
            assert ws >= tp * 5120 * 2 + tp * 4
        elif r == q.Q4LIN_ROUTE_MID:
            # one pass of the weight formats' kernel: no workspace
            assert ws == 0
        else:
            assert ws == 0
    for t in (33, 64, 65, 128):
        assert q.q4lin_route(6144, 5120, t) == q.Q4LIN_ROUTE_MID
    assert q.q4lin_route(6144, 5120, 1024) == q.Q4LIN_ROUTE_TILED


# -- LinearAdd: same contract plus the residual --------------------------------
def test_linear_add_empty_product_is_a_no_op():
    for n, t in [(0, 5), (6, 0)]:
        assert q.q4lin_linear_add(0, 0, 0, 0, 0, n, 128, t, 0, 0, 0) == q.Q4LIN_OK


@pytest.mark.parametrize("which", range(5))
def test_linear_add_null_pointer_rejected(which):
    ptrs = [0x1000] * 5
    ptrs[which] = 0
    assert q.q4lin_linear_add(*ptrs, 64, 128, 1, 0, 0, 0) == q.Q4LIN_E_NULL


@pytest.mark.parametrize("which,addr", [(0, 0x1008), (1, 0x1004), (2, 0x1001), (3, 0x1001), (4, 0x1001)])
def test_linear_add_misaligned_pointer_rejected(which, addr):
    ptrs = [0x1000] * 5
    ptrs[which] = addr
    assert q.q4lin_linear_add(*ptrs, 64, 128, 1, 0, 0, 0) == q.Q4LIN_E_ALIGN


def test_linear_add_shape_and_workspace_checks():
    p = 0x10000
    assert q.q4lin_linear_add(p, p, p, p, p, 8, 96, 1, 0, 0, 0) == q.Q4LIN_E_SHAPE
    n, k, t = 256, 512, 300
    need = q.q4lin_workspace_bytes(n, k, t)
    assert q.q4lin_linear_add(p, p, p, p, p, n, k, t, p, need - 1, 0) == q.Q4LIN_E_WORKSPACE


# -- LinearPair: two weights over one X ----------------------------------------
def test_linear_pair_empty_and_one_plane():
    assert q.q4lin_linear_pair(0, 0, 0, 0, 0, 0, 0, 0, 0, 128, 5, 0, 0, 0) == q.Q4LIN_OK
    assert q.q4lin_linear_pair(0, 0, 0, 0, 6, 0, 0, 0, 7, 128, 0, 0, 0, 0) == q.Q4LIN_OK
    p = 0x10000
    # one plane empty: only the other weight's pointers are checked (a
    # misaligned output stops the call before any launch)
    assert q.q4lin_linear_pair(p, p, p, p + 1, 64, 0, 0, 0, 0, 128, 1, 0, 0, 0) == q.Q4LIN_E_ALIGN
    assert q.q4lin_linear_pair(p, 0, 0, 0, 0, p, p, p + 1, 64, 128, 1, 0, 0, 0) == q.Q4LIN_E_ALIGN
    assert q.q4lin_linear_pair(p, p, p, 0, 64, 0, 0, 0, 0, 128, 1, 0, 0, 0) == q.Q4LIN_E_NULL


@pytest.mark.parametrize("which", [0, 1, 2, 3, 5, 6, 7])
def test_linear_pair_null_pointer_rejected(which):
    args = [0x1000, 0x1000, 0x1000, 0x1000, 64, 0x1000, 0x1000, 0x1000, 64, 128, 1, 0, 0, 0]
    args[which] = 0
    assert q.q4lin_linear_pair(*args) == q.Q4LIN_E_NULL


@pytest.mark.parametrize("which,addr", [(0, 0x1008), (1, 0x1004), (2, 0x1001), (3, 0x1001), (5, 0x1004),
                                        (6, 0x1001), (7, 0x1001)])
def test_linear_pair_misaligned_pointer_rejected(which, addr):
    args = [0x1000, 0x1000, 0x1000, 0x1000, 64, 0x1000, 0x1000, 0x1000, 64, 128, 1, 0, 0, 0]
    args[which] = addr
    assert q.q4lin_linear_pair(*args) == q.Q4LIN_E_ALIGN


def test_linear_pair_shapes_and_workspace():
    p = 0x10000
    assert q.q4lin_linear_pair(p, p, p, p, 8, p, p, p, 8, 96, 1, 0, 0, 0) == q.Q4LIN_E_SHAPE
    assert q.q4lin_linear_pair(p, p, p, p, -1, p, p, p, 8, 128, 1, 0, 0, 0) == q.Q4LIN_E_SHAPE
    assert q.q4lin_pair_workspace_bytes(8, 8, 96, 1) == -q.Q4LIN_E_SHAPE
    # the fused one-to-128-token routes need none
    assert q.q4lin_pair_workspace_bytes(3072, 3072, 5120, 1) == 0
    assert q.q4lin_pair_workspace_bytes(1000, 700, 2048, 20) == 0
    assert q.q4lin_pair_workspace_bytes(3072, 3072, 5120, 64) == 0
    assert q.q4lin_pair_workspace_bytes(1000, 333, 2048, 128) == 0
    # many tokens: the activations once, then each weight's row exponents
    # (and partial sums under a K split)
    n1, n2, k, t = 768, 256, 1024, 200
    need = q.q4lin_pair_workspace_bytes(n1, n2, k, t)
    tp = (t + 31) // 32 * 32
    assert need >= tp * k * 2 + tp * 4 + (n1 + n2) * 4
    assert need < q.q4lin_workspace_bytes(n1, k, t) + q.q4lin_workspace_bytes(n2, k, t)
    assert q.q4lin_linear_pair(p, p, p, p, n1, p, p, p, n2, k, t, p, need - 1, 0) == q.Q4LIN_E_WORKSPACE
    assert q.q4lin_pair_workspace_bytes(0, 512, 1024, 300) == q.q4lin_workspace_bytes(512, 1024, 300)


# -- LinearSwiGLU: silu(gate sums) * (up sums) ---------------------------------
def test_linear_swiglu_checks():
    p = 0x10000
    assert q.q4lin_linear_swiglu(0, 0, 0, 0, 0, 0, 0, 128, 5, 0, 0, 0) == q.Q4LIN_OK
    assert q.q4lin_linear_swiglu(0, 0, 0, 0, 0, 0, 6, 128, 0, 0, 0, 0) == q.Q4LIN_OK
    assert q.q4lin_swiglu_workspace_bytes(0, 128, 5) == 0
    assert q.q4lin_linear_swiglu(p, p, p, p, p, p, 8, 96, 1, 0, 0, 0) == q.Q4LIN_E_SHAPE
    assert q.q4lin_swiglu_workspace_bytes(8, 96, 1) == -q.Q4LIN_E_SHAPE
    # one to four tokens on the single-token route: one pass, no workspace
    # (a null workspace is accepted)
    assert q.q4lin_swiglu_workspace_bytes(6144, 5120, 1) == 0
    assert q.q4lin_swiglu_workspace_bytes(2048, 1024, 4) == 0
    assert q.q4lin_linear_swiglu(p, p, p, p, p, p + 1, 6144, 5120, 1, 0, 0, 0) == q.Q4LIN_E_ALIGN
    # 5 to 128 tokens on the weight formats' kernel: one pass, no workspace
    for n, k, t in [(1000, 2048, 20), (768, 1024, 100), (3072, 5120, 5), (3072, 5120, 128)]:
        assert q.q4lin_swiglu_workspace_bytes(n, k, t) == 0
    # its scale table of both weights' rows does not fit for K = 2^20 beyond
    # 16 tokens: one medium-T launch per weight and the combine
    assert q.q4lin_swiglu_workspace_bytes(16, 1 << 20, 40) == 2 * ((16 * 40 * 4 + 255) // 256 * 256)
    # the many-token route with the 2N-row problem on 96 x 256 tiles and no K
    # split: one tiled launch applies the gate in its epilogue; the workspace
    # holds only the activation preparation (FP16 activations, token
    # exponents, both weights' row exponents)
    al = lambda v: (v + 255) // 256 * 256
    for n, k, t in [(1024, 1024, 300), (3072, 5120, 1024), (200, 1024, 300)]:
        tp = (t + 31) // 32 * 32
        assert q.q4lin_swiglu_workspace_bytes(n, k, t) == al(tp * k * 2) + al(tp * 4) + 2 * al(n * 4)
    # with a K split (3072 x 5120 at T = 512: 128 tiles, two K shares) the
    # sums stay in the workspace for the combine
    for n, k, t in [(128, 20480, 3), (3072, 5120, 512), (16, 1 << 20, 40), (1024, 1024, 300)]:
        need = q.q4lin_swiglu_workspace_bytes(n, k, t)
        if (n, k, t) != (1024, 1024, 300):
            assert need >= 2 * n * t * 4
        assert need % 256 == 0
        assert q.q4lin_linear_swiglu(p, p, p, p, p, p, n, k, t, p, need - 1, 0) == q.Q4LIN_E_WORKSPACE
        assert q.q4lin_linear_swiglu(p, p, p, p, p, p, n, k, t, 0, need, 0) == q.Q4LIN_E_NULL
        assert q.q4lin_linear_swiglu(p, p, p, p, p, p, n, k, t, p + 16, need, 0) == q.Q4LIN_E_ALIGN


@pytest.mark.parametrize("which", range(6))
def test_linear_swiglu_null_pointer_rejected(which):
    ptrs = [0x1000] * 6
    ptrs[which] = 0
    assert q.q4lin_linear_swiglu(*ptrs, 64, 128, 1, 0x1000, 1 << 20, 0) == q.Q4LIN_E_NULL


@pytest.mark.parametrize("which,addr", [(0, 0x1008), (1, 0x1004), (2, 0x1001), (3, 0x1004), (4, 0x1001),
                                        (5, 0x1001)])
def test_linear_swiglu_misaligned_pointer_rejected(which, addr):
    ptrs = [0x1000] * 6
    ptrs[which] = addr
    assert q.q4lin_linear_swiglu(*ptrs, 64, 128, 1, 0x1000, 1 << 20, 0) == q.Q4LIN_E_ALIGN


# -- the no-allocation entry point: host-side checks only ---------------------
def test_noalloc_scratch_size_and_rejections():
    cap = q.q4lin_noalloc_scratch_bytes()
    assert cap == 64 << 20
    p = 0x10000
    # empty product, shape, NULL and alignment errors as q4lin_linear
    assert q.q4lin_linear_noalloc(0, 0, 0, 0, 0, 128, 5, 0) == q.Q4LIN_OK
    assert q.q4lin_linear_noalloc(p, p, p, p, 8, 100, 1, 0) == q.Q4LIN_E_SHAPE
    assert q.q4lin_linear_noalloc(p, 0, p, p, 64, 128, 1, 0) == q.Q4LIN_E_NULL
    assert q.q4lin_linear_noalloc(p + 8, p, p, p, 64, 128, 1, 0) == q.Q4LIN_E_ALIGN
    # a many-token shape whose workspace exceeds the array: rejected before
    # anything touches a device
    n, k, t = 6144, 5120, 8192
    assert q.q4lin_workspace_bytes(n, k, t) > cap
    assert q.q4lin_linear_noalloc(p, p, p, p, n, k, t, 0) == q.Q4LIN_E_WORKSPACE
    # the benchmarked workloads fit
    for (n, k, t) in [(6144, 5120, 1024), (6144, 5120, 128), (14336, 5120, 1024), (34816, 5120, 1024),
                      (5120, 17408, 1024)]:
        assert 0 <= q.q4lin_workspace_bytes(n, k, t) <= cap, (n, k, t)


# -- the weight-format entry point: host-side checks only ---------------------
def test_fmt_weight_bytes_and_rejections():
    n, k = 6144, 5120
    assert q.q4lin_fmt_weight_bytes(q.Q4LIN_FMT_Q4G64_F16S, n, k) == 16_711_680
    assert q.q4lin_fmt_weight_bytes(q.Q4LIN_FMT_Q5G64_F16S, n, k) == n * k // 64 * 42
    assert q.q4lin_fmt_weight_bytes(q.Q4LIN_FMT_Q6G64_F16S, n, k) == n * k // 64 * 50
    assert q.q4lin_fmt_weight_bytes(q.Q4LIN_FMT_W8G32_F16S, n, k) == n * k // 32 * 34
    assert q.q4lin_fmt_weight_bytes(q.Q4LIN_FMT_NVFP4, n, k) == n * k // 16 * 9
    assert q.q4lin_fmt_weight_bytes(q.Q4LIN_FMT_BF16, n, k) == 2 * n * k
    assert q.q4lin_fmt_weight_bytes(9, n, k) == -q.Q4LIN_E_FORMAT
    assert q.q4lin_fmt_weight_bytes(1, n, 100) == -q.Q4LIN_E_SHAPE
    p = 0x10000
    assert q.q4lin_linear_fmt(9, p, p, p, p, p, 64, 128, 1, 0, 0, 0) == q.Q4LIN_E_FORMAT
    assert q.q4lin_status_string(q.Q4LIN_E_FORMAT) == "unknown weight format"
    for f in (1, 2, 3, 4, 5):
        assert q.q4lin_fmt_workspace_bytes(f, n, k, 1024) == 0
        assert q.q4lin_linear_fmt(f, 0, 0, 0, 0, 0, 0, 128, 4, 0, 0, 0) == q.Q4LIN_OK      # empty
        assert q.q4lin_linear_fmt(f, p, p, p, p, p, 64, 96, 1, 0, 0, 0) == q.Q4LIN_E_SHAPE
        assert q.q4lin_linear_fmt(f, 0, p, p, p, p, 64, 128, 1, 0, 0, 0) == q.Q4LIN_E_NULL
        assert q.q4lin_linear_fmt(f, p + 8, p, p, p, p, 64, 128, 1, 0, 0, 0) == q.Q4LIN_E_ALIGN
    # planes a format has are required; the ones it lacks may be NULL
    assert q.q4lin_linear_fmt(q.Q4LIN_FMT_Q5G64_F16S, p, p, 0, p, p, 64, 128, 1, 0, 0, 0) == q.Q4LIN_E_NULL
    assert q.q4lin_linear_fmt(q.Q4LIN_FMT_W8G32_F16S, p, p, p, 0, p, 64, 128, 1, 0, 0, 0) == q.Q4LIN_E_NULL
    assert q.q4lin_linear_fmt(q.Q4LIN_FMT_Q6G64_F16S, p, p, p + 2, p, p, 64, 128, 1, 0, 0, 0) == q.Q4LIN_E_ALIGN
    assert q.q4lin_linear_fmt(q.Q4LIN_FMT_Q6G64_F16S, p, p, p + 4, p, p, 64, 128, 1, 0, 0, 0) == q.Q4LIN_E_ALIGN
    assert q.q4lin_linear_fmt(q.Q4LIN_FMT_Q5G64_F16S, p, p, p + 2, p, p, 64, 128, 1, 0, 0, 0) == q.Q4LIN_E_ALIGN
    assert q.q4lin_linear_fmt(q.Q4LIN_FMT_NVFP4, p, p, p, p + 1, p, 64, 128, 1, 0, 0, 0) == q.Q4LIN_E_ALIGN
    # Q4 goes through q4lin_linear's checks and workspace
    assert q.q4lin_fmt_workspace_bytes(0, n, k, 1024) == q.q4lin_workspace_bytes(n, k, 1024)
    assert q.q4lin_linear_fmt(0, p, p, 0, p, p, n, k, 1024, p, 16, 0) == q.Q4LIN_E_WORKSPACE
