"""LinearSwiGLU (Y = bf16(silu(Wg x X) * (Wu x X))) on the GPU against the
oracle, through the C ABI (q4lin_linear_swiglu), on every way the two sums
are made (one pass with the gate applied in the final sum for one to four
tokens and for 5 to 128, both weights' sums in one launch, one launch per
weight on the wide-K routes, the many-token route with and without a K
split): seeded problems within the tolerance, the closed
forms (an all-eight gate gives zeros signed like U, an all-eight up weight
zeros), the single-rounding worked example, and sampled outputs at the
6144 x 5120 shape.  The tolerance is the plain op's, carried through the
gate to first order (swiglu_close)."""
import numpy as np
import pytest

import oracle
from gpu_util import announce, assert_close, dev, host_bits, torch
from weight_only_bit_q4_amd import inputs

pytestmark = pytest.mark.gpu


def run_swiglu(x, cg, sg, cu, su, n, k, t, what=""):
    import weight_only_bit_q4_amd as q4
    announce("%s q4lin_linear_swiglu n=%d k=%d t=%d route(2n)=%d route(n)=%d" % (
        what, n, k, t, q4.q4lin_route(2 * n, k, t), q4.q4lin_route(n, k, t)))
    th = torch()
    xd = dev(np.asarray(x, dtype=np.uint16).reshape(t, k))
    args = [dev(np.asarray(a, dtype=dt).reshape(n, -1)) for a, dt in
            ((cg, np.uint8), (sg, np.uint16), (cu, np.uint8), (su, np.uint16))]
    y = q4.linear_swiglu(xd, *args)
    th.cuda.synchronize()
    return host_bits(y)


def swiglu_close(got, g, u, what=""):
    """The plain op's tolerance carried through silu(G) U to first order: the
    output's own bound 1e-2 |y| + 1e-3 rms(y), plus what an error of
    1e-3 rms(G) in the gate sum and 1e-3 rms(U) in the up sum moves y by
    (|silu'(G) U| and |silu(G)| times them), since each sum is the plain op
    before its rounding and the GPU's sums are held to that bound."""
    g = np.asarray(g, dtype=np.float64).reshape(-1)
    u = np.asarray(u, dtype=np.float64).reshape(-1)
    want = oracle.swiglu(g, u)
    yo = oracle.bf16_bits_to_f64(want)
    yg = oracle.bf16_bits_to_f64(np.asarray(got, dtype=np.uint16).reshape(-1))
    sig = 1.0 / (1.0 + np.exp(-g))
    silu, dsilu = g * sig, sig * (1.0 + g * (1.0 - sig))
    rms = lambda v: float(np.sqrt(np.mean(v * v))) if v.size else 0.0
    bound = (1e-2 * np.abs(yo) + 1e-3 * rms(yo) + np.abs(dsilu * u) * 1e-3 * rms(g)
             + np.abs(silu) * 1e-3 * rms(u))
    err = np.abs(yg - yo)
    bad = ~(err <= bound)
    assert not bad.any(), "%s: %d outputs outside tolerance (worst %.3g x bound)" % (
        what, int(bad.sum()), float(np.max(err / np.maximum(bound, 1e-300))))


def _pair(n, k, t, seed):
    x, cg, sg = inputs.gen_problem(n, k, t, seed)
    _, cu, su = inputs.gen_problem(n, k, t, seed + 1)
    return x, cg, sg, cu, su


# From 129 tokens, where the 2N-row problem takes 96 x 256 tiles without a
# K split, one tiled launch applies the gate in its epilogue (tiles of 48
# rows of each weight; ragged rows and tokens, five groups); with a K split
# (3072 x 5120 at T = 512) the sums go through the workspace and the combine.
# 5 to 128 tokens run one launch of the weight formats' kernel, each
# workgroup on the same rows of both weights: 16 or 32 rows of each (two or
# four column tiles), few-token and many-token kernels, one and two token
# ranges, ragged row blocks; K = 2^20 beyond 16 tokens takes one medium-T
# launch per weight and the combine
@pytest.mark.parametrize("n,k,t", [(3072, 5120, 1), (1000, 2048, 1), (2048, 1024, 4), (1000, 2048, 20),
                                   (517, 1280, 9), (128, 20480, 3), (768, 1024, 100), (1024, 1024, 300),
                                   (97, 320, 40), (6144, 5120, 64), (6144, 256, 1024), (2560, 17408, 1),
                                   (3072, 5120, 5), (3072, 5120, 16), (6000, 1024, 12), (6000, 1024, 17),
                                   (6000, 640, 100), (1000, 2048, 128), (333, 640, 65), (4100, 640, 33),
                                   (16, 1 << 20, 40), (1, 640, 100), (5, 64, 17), (2, 128, 5), (1000, 64, 128),
                                   (257, 2048, 33), (3000, 320, 1000), (1001, 640, 700), (200, 1024, 300),
                                   (3072, 5120, 512), (4800, 192, 257)])
def test_swiglu_matches_oracle(n, k, t):
    x, cg, sg, cu, su = _pair(n, k, t, 101)
    got = run_swiglu(x, cg, sg, cu, su, n, k, t, what="seeded")
    _, g = oracle.linear(x, cg, sg, n, k, t, with_acc=True)
    _, u = oracle.linear(x, cu, su, n, k, t, with_acc=True)
    assert np.array_equal(oracle.swiglu(g, u).reshape(t, n), oracle.linear_swiglu(x, cg, sg, cu, su, n, k, t))
    swiglu_close(got, g, u, what="LinearSwiGLU %dx%d T=%d" % (n, k, t))


@pytest.mark.parametrize("n,k,t", [(512, 1024, 1), (1000, 2048, 20), (700, 1280, 70), (3000, 320, 1000)])
def test_swiglu_zero_gate_and_zero_up(n, k, t):
    x, cg, sg, cu, su = _pair(n, k, t, 103)
    eights = np.full_like(cg, 0x88)
    _, u = oracle.linear(x, cu, su, n, k, t, with_acc=True)
    import weight_only_bit_q4_amd as q4
    got = run_swiglu(x, eights, sg, cu, su, n, k, t, what="all-eight gate")
    assert np.all((got & 0x7FFF) == 0)
    if q4.q4lin_route(n, k, t) != q4.Q4LIN_ROUTE_TILED:
        # the sign of the zero follows U on the routes that sum in binary64;
        # the many-token route's zero sign is not asserted
        assert np.array_equal(got, np.where(u < 0, 0x8000, 0x0000).astype(np.uint16))
    got = run_swiglu(x, cg, sg, eights, su, n, k, t, what="all-eight up")
    assert np.all((got & 0x7FFF) == 0)


@pytest.mark.parametrize("replicate", [1, 4, 20, 40])
def test_swiglu_single_rounding_example(replicate):
    # the oracle pin's worked example (G = 128, U = 1 + 2^-8 + 2^-30): one
    # rounding from binary64 gives 129; the GPU's sums are binary32, which
    # may leave the tie at 128.5 (one bf16 ulp, within the tolerance)
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
    xr = np.tile(x, (replicate, 1))
    got = run_swiglu(xr, cg, sg, cu, su, n, k, t * replicate, what="single rounding")
    want = np.tile(np.array([[0x4301, 0xC301]], dtype=np.uint16), (replicate, 1))
    assert np.all(np.abs(got.astype(np.int32) - want.astype(np.int32)) <= 1)
    assert_close(got, want, what="single rounding")


def test_swiglu_prefill_6144x5120_t1024_sampled():
    import gpu_util
    n, k, t = 6144, 5120, 1024
    x, cg, sg, cu, su = _pair(n, k, t, 107)
    got = run_swiglu(x, cg, sg, cu, su, n, k, t, what="prefill sampled")
    ns, ts = gpu_util.sample_indices(n, t, 400, 109, extra_n=(0, n - 1), extra_t=(0, t - 1))
    _, g = oracle.linear_at(x, cg, sg, n, k, t, ns, ts, with_acc=True)
    _, u = oracle.linear_at(x, cu, su, n, k, t, ns, ts, with_acc=True)
    swiglu_close(got[ts, ns], g, u, what="LinearSwiGLU 6144x5120 T=1024 sampled")


@pytest.mark.parametrize("t", [1, 16, 64, 300])
def test_swiglu_graph_replay_with_changed_inputs(t):
    """One LinearSwiGLU call captured in a HIP graph (one pass with the gate in
    the final sum at 1, 16 and 64 tokens; the tiled sums and the combine pass
    at 300), the activations and both weights overwritten in place before each
    replay, eager work between replays: every replay matches the oracle."""
    import weight_only_bit_q4_amd as q4
    th = torch()
    n, k = 200, 1024
    x0, cg0, sg0, cu0, su0 = _pair(n, k, t, 800 + t)
    xd = dev(np.asarray(x0, dtype=np.uint16).reshape(t, k))
    planes = [dev(np.asarray(a, dtype=dt).reshape(n, -1)) for a, dt in
              ((cg0, np.uint8), (sg0, np.uint16), (cu0, np.uint8), (su0, np.uint16))]
    y = th.empty((t, n), dtype=th.bfloat16, device="cuda")
    need = q4.q4lin_swiglu_workspace_bytes(n, k, t)
    ws = th.empty(max(need, 1), dtype=th.uint8, device="cuda")
    wsv = ws[:need] if need else None
    q4.linear_swiglu(xd, *planes, y=y, workspace=wsv)   # warm-up outside capture
    th.cuda.synchronize()
    g = th.cuda.CUDAGraph()
    announce("swiglu graph capture n=%d k=%d t=%d" % (n, k, t))
    with th.cuda.graph(g):
        q4.linear_swiglu(xd, *planes, y=y, workspace=wsv)
    for rep in range(3):
        x, cg, sg, cu, su = _pair(n, k, t, 810 + 10 * rep + t)
        xd.copy_(dev(np.asarray(x, dtype=np.uint16).reshape(t, k)))
        for p, (a, dt) in zip(planes, ((cg, np.uint8), (sg, np.uint16), (cu, np.uint8), (su, np.uint16))):
            p.copy_(dev(np.asarray(a, dtype=dt).reshape(n, -1)))
        th.cuda.synchronize()
        g.replay()
        th.cuda.synchronize()
        _, gs = oracle.linear(x, cg, sg, n, k, t, with_acc=True)
        _, us = oracle.linear(x, cu, su, n, k, t, with_acc=True)
        swiglu_close(host_bits(y), gs, us, what="LinearSwiGLU replay %d T=%d" % (rep, t))
        junk = th.randn(1 << 20, device="cuda")
        junk.sum().item()
