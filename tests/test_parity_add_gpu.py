"""LinearAdd (Y = W x X + R, one rounding) on the GPU against the oracle,
through the C ABI (q4lin_linear_add), on every route: hand-worked examples
bit for bit, the all-eight closed form (Y = R exactly), seeded problems of
the workloads' distributions within the tolerance, and the in-place form
(residual = y)."""
import numpy as np
import pytest

import oracle
import oracle_pins
from gpu_util import announce, assert_close, dev, host_bits, torch
from weight_only_bit_q4_amd import inputs

pytestmark = pytest.mark.gpu


def run_add(x, codes, scales, res, n, k, t, in_place=False, what=""):
    import weight_only_bit_q4_amd as q4
    announce("%s q4lin_linear_add n=%d k=%d t=%d route=%d%s" % (what, n, k, t, q4.q4lin_route(n, k, t),
                                                               " in place" if in_place else ""))
    th = torch()
    xd = dev(np.asarray(x, dtype=np.uint16).reshape(t, k))
    cd = dev(np.asarray(codes, dtype=np.uint8).reshape(n, k // 2))
    sd = dev(np.asarray(scales, dtype=np.uint16).reshape(n, k // 64))
    rd = dev(np.asarray(res, dtype=np.uint16).reshape(t, n))
    if in_place:
        yd = q4.linear(xd, cd, sd, y=rd, residual=rd)
    else:
        yd = q4.linear(xd, cd, sd, residual=rd)
    th.cuda.synchronize()
    return host_bits(yd)


def _residual(t, n, seed, scale=1.0):
    r = np.random.default_rng(seed)
    return oracle_pins.torch_f32_to_bf16_bits((r.standard_normal((t, n)) * scale).astype(np.float32))


# replication factors that move the tiny examples onto every route:
# 1 token (single-token or few-token), 3 (few-token / small-T), 20 (small-T),
# 40 (many-token)
@pytest.mark.parametrize("replicate", [1, 3, 20, 40])
def test_add_worked_examples_bit_exact(replicate):
    for ex in oracle_pins.load_add_examples():
        x, codes, scales, r, want = oracle_pins.materialize_add(ex)
        n, k, t = ex["n"], ex["k"], ex["t"]
        xr = np.tile(x, (replicate, 1))
        rr = np.tile(r, (replicate, 1))
        got = run_add(xr, codes, scales, rr, n, k, t * replicate, what=ex["name"])
        want_r = np.tile(want.reshape(t, n), (replicate, 1))
        assert np.array_equal(got.reshape(-1), want_r.reshape(-1)), (
            ex["name"], [hex(v) for v in got.reshape(-1)[:8]], [hex(v) for v in want_r.reshape(-1)[:8]])


@pytest.mark.parametrize("n,k,t", [(6144, 5120, 1), (512, 1024, 4), (1000, 2048, 20), (700, 1280, 70),
                                   (1024, 1024, 300)])
def test_add_all_code8_returns_residual(n, k, t):
    x, codes, scales = inputs.gen_problem(n, k, t, 41)
    codes[:] = 0x88
    res = _residual(t, n, 43, scale=8.0)
    got = run_add(x, codes, scales, res, n, k, t, what="all-eight")
    assert np.array_equal(got, res.reshape(t, n))


@pytest.mark.parametrize("n,k,t", [(6144, 5120, 1), (512, 1024, 4), (1536, 5120, 9), (1000, 2048, 20),
                                   (2048, 1024, 64), (700, 1280, 70), (1024, 1024, 300), (97, 320, 40),
                                   (6144, 256, 1024), (6100, 320, 1000), (2600, 17408, 1)])
def test_add_matches_oracle(n, k, t):
    x, codes, scales = inputs.gen_problem(n, k, t, 47)
    # a residual of the size of the product, so both terms matter
    res = _residual(t, n, 53, scale=0.5)
    got = run_add(x, codes, scales, res, n, k, t, what="seeded")
    want = oracle.linear_add(x, codes, scales, res, n, k, t)
    assert_close(got, want, what="LinearAdd %dx%d T=%d" % (n, k, t))


@pytest.mark.parametrize("n,k,t", [(6144, 5120, 1), (1000, 2048, 20), (1024, 1024, 300), (6144, 256, 1024)])
def test_add_in_place(n, k, t):
    x, codes, scales = inputs.gen_problem(n, k, t, 59)
    res = _residual(t, n, 61, scale=0.5)
    got = run_add(x, codes, scales, res, n, k, t, in_place=True, what="in place")
    want = oracle.linear_add(x, codes, scales, res, n, k, t)
    assert_close(got, want, what="LinearAdd in place %dx%d T=%d" % (n, k, t))


def test_add_prefill_6144x5120_t1024_sampled():
    n, k, t = 6144, 5120, 1024
    x, codes, scales = inputs.gen_problem(n, k, t, inputs.workload_seed("prefill_6144x5120_t1024"))
    res = _residual(t, n, 67, scale=0.5)
    got = run_add(x, codes, scales, res, n, k, t, what="prefill sampled")
    r = np.random.default_rng(71)
    ns = np.concatenate([r.integers(0, n, 600), [0, n - 1]])
    ts = np.concatenate([r.integers(0, t, 600), [t - 1, 0]])
    _, acc = oracle.linear_at(x, codes, scales, n, k, t, ns, ts, with_acc=True)
    o = oracle.default()
    want = np.array([o.double_to_bf16(a + o.bf16_to_double(int(res[tt, nn]))) for a, nn, tt in zip(acc, ns, ts)],
                    dtype=np.uint16)
    assert_close(got[ts, ns], want, what="LinearAdd prefill sampled")
