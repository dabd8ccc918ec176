"""The other weight formats (Q5G64_F16S, Q6G64_F16S, W8G32_F16S, NVFP4 A16,
BF16_CTRL) on the GPU against the oracle, through the C ABI
(q4lin_linear_fmt): hand-worked examples bit for bit, seeded problems of the
workload's shape at T = 1 and 16 and ragged shapes element by element, the
offset codes' exact zeros, wide-range scales, inputs preserved and writes
confined to y."""
import numpy as np
import pytest

import oracle
import oracle_pins_fmt
from gpu_util import announce, assert_close, dev, host_bits, sample_indices, torch
from weight_only_bit_q4_amd import inputs

pytestmark = pytest.mark.gpu

FMTS = [inputs.FMT_Q5, inputs.FMT_Q6, inputs.FMT_W8, inputs.FMT_NVFP4, inputs.FMT_BF16]
FMT_IDS = [inputs.FMT_NAMES[f] for f in FMTS]
# examples whose exact sum needs more than binary32 (held to the tolerance)
FP32_INEXACT = {"BF16_single_rounding"}


def _bytes_dev(a):
    a = np.ascontiguousarray(a)
    return torch().from_numpy(a.reshape(-1).view(np.uint8).copy()).cuda()


def run_fmt(fmt, x, w, hi, sc, n, k, t, y=None, what=""):
    import weight_only_bit_q4_amd as q4
    th = torch()
    announce("%s q4lin_linear_fmt fmt=%d n=%d k=%d t=%d" % (what, fmt, n, k, t))
    xd = dev(np.asarray(x, dtype=np.uint16).reshape(t, k))
    wd = _bytes_dev(w).view(n, -1)
    hd = _bytes_dev(hi) if hi is not None else None
    sd = _bytes_dev(sc) if sc is not None else None
    yd = q4.linear_fmt(fmt, xd, wd, hd, sd, y=y)
    th.cuda.synchronize()
    return host_bits(yd)


@pytest.mark.parametrize("replicate", [1, 3, 20, 40], ids=["t1", "t3", "t20", "t40"])
def test_fmt_worked_examples(replicate):
    for ex in oracle_pins_fmt.load_examples():
        fmt, x, lo, hi, sc, want = oracle_pins_fmt.materialize(ex)
        n, k, t = ex["n"], ex["k"], ex["t"]
        xr = np.tile(x, (replicate, 1))
        got = run_fmt(fmt, xr, lo, hi, sc, n, k, t * replicate, what=ex["name"])
        want_r = np.tile(want.reshape(t, n), (replicate, 1))
        if ex["name"] in FP32_INEXACT:
            assert_close(got, want_r, what=ex["name"])
        else:
            assert np.array_equal(got.reshape(-1), want_r.reshape(-1)), (
                ex["name"], [hex(v) for v in got.reshape(-1)[:8]], [hex(v) for v in want_r.reshape(-1)[:8]])


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("t", [1, 16])
def test_fmt_6144x5120(fmt, t):
    n, k = 6144, 5120
    seed = inputs.workload_seed("decode_6144x5120_t1") + 100 * fmt
    w, hi, sc = inputs.gen_fmt_weight(fmt, n, k, seed)
    x = inputs.gen_x(k, t, seed)
    got = run_fmt(fmt, x, w, hi, sc, n, k, t, what="6144x5120")
    assert_close(got, oracle.linear_fmt(fmt, x, w, hi, sc, n, k, t), what="%s T=%d" % (inputs.FMT_NAMES[fmt], t))


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("n,k,t", [(1, 64, 1), (7, 64, 3), (97, 320, 5), (300, 1088, 17), (1000, 2048, 33),
                                   (4100, 704, 32), (20000, 256, 2), (4100, 8192, 3)])
def test_fmt_ragged(fmt, n, k, t):
    w, hi, sc = inputs.gen_fmt_weight(fmt, n, k, 300 + n + k + t)
    x = inputs.gen_x(k, t, 300 + t)
    got = run_fmt(fmt, x, w, hi, sc, n, k, t, what="ragged")
    assert_close(got, oracle.linear_fmt(fmt, x, w, hi, sc, n, k, t),
                 what="%s %dx%d T=%d" % (inputs.FMT_NAMES[fmt], n, k, t))


# One token, K up to 8192: the streaming GEMV, one instantiation per number
# of 16-byte pieces a lane takes along a row (Q5/Q6/NVFP4: 32 weights a piece,
# 1..4 pieces; W8: 16, 1..6 and 8; BF16_CTRL: 8, 2..16), each at the smallest and
# the largest K it serves, on an odd row count (the grid's last wave takes
# one real row); K = 8256 is past the GEMV (the matrix-core kernel at T = 1).
GEMV_KS = {
    inputs.FMT_Q5: [64, 2048, 2112, 4096, 4160, 6144, 6208, 8192, 8256],
    inputs.FMT_Q6: [64, 2048, 2112, 4096, 4160, 6144, 6208, 8192, 8256],
    inputs.FMT_NVFP4: [64, 2048, 2112, 4096, 4160, 6144, 6208, 8192, 8256],
    inputs.FMT_W8: [64, 1024, 1088, 2048, 2112, 3072, 3136, 4096, 4160, 5120, 5184, 6144, 6208, 8192, 8256],
    inputs.FMT_BF16: [64, 1024, 1088, 2048, 2112, 3072, 3136, 4096, 4160, 5120, 5184, 6144, 6208, 8192, 8256],
}


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_fmt_one_token_lane_shapes(fmt):
    n = 37
    for k in GEMV_KS[fmt]:
        w, hi, sc = inputs.gen_fmt_weight(fmt, n, k, 900 + k)
        x = inputs.gen_x(k, 1, 901 + k)
        got = run_fmt(fmt, x, w, hi, sc, n, k, 1, what="one token")
        assert_close(got, oracle.linear_fmt(fmt, x, w, hi, sc, n, k, 1),
                     what="%s %dx%d T=1" % (inputs.FMT_NAMES[fmt], n, k))


# (n, k, t): the many-token kernel's token tiles (2, 3, 4, 6, 8 per wave)
# with one to four column tiles, one or two token ranges per row block (two
# from 65 tokens up to 8192 rows; a ragged second range; a grid whose last
# row of eight has row blocks past N), a run of pairs longer than one chunk
# of codes (K = 16384), a single unit (K = 64), and T past 128
TOKEN_TILE_SHAPES = [(2048, 2048, 24), (2048, 2048, 40), (6144, 1024, 64), (6144, 1024, 80), (6144, 1024, 128),
                     (6144, 2048, 128), (2000, 1024, 77), (4096, 1024, 200), (4096, 1024, 60), (10240, 640, 48), (16384, 640, 64),
                     (16384, 640, 100), (500, 16384, 97), (300, 1088, 130), (100, 64, 33)]


@pytest.mark.parametrize("fmt", [inputs.FMT_Q4] + FMTS, ids=["Q4G64_F16S"] + FMT_IDS)
@pytest.mark.parametrize("n,k,t", TOKEN_TILE_SHAPES)
def test_fmt_token_tiles(fmt, n, k, t):
    w, hi, sc = inputs.gen_fmt_weight(fmt, n, k, 500 + n + t)
    x = inputs.gen_x(k, t, 501 + t)
    got = run_fmt(fmt, x, w, hi, sc, n, k, t, what="token tiles")
    assert_close(got, oracle.linear_fmt(fmt, x, w, hi, sc, n, k, t),
                 what="%s %dx%d T=%d" % (inputs.FMT_NAMES[fmt], n, k, t))


def test_fmt_long_k_scale_table():
    """K = 131072 in W8: a row's scales take 8 KiB, so a block holds 12 rows
    instead of 13 (the LDS scale table is capped); every output compared."""
    fmt, n, k, t = inputs.FMT_W8, 3100, 131072, 2
    w, hi, sc = inputs.gen_fmt_weight(fmt, n, k, 77)
    x = inputs.gen_x(k, t, 78)
    got = run_fmt(fmt, x, w, hi, sc, n, k, t, what="long K")
    assert_close(got, oracle.linear_fmt(fmt, x, w, hi, sc, n, k, t), what="W8 3100x131072 T=2")


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_fmt_prefill_t1024_sampled(fmt):
    """T = 1024 runs the kernel once per 128 tokens; sampled outputs and the
    token-run boundaries against the oracle."""
    n, k, t = 6144, 5120, 1024
    seed = inputs.workload_seed("prefill_6144x5120_t1024") + 100 * fmt
    w, hi, sc = inputs.gen_fmt_weight(fmt, n, k, seed)
    x = inputs.gen_x(k, t, seed)
    got = run_fmt(fmt, x, w, hi, sc, n, k, t, what="prefill")
    ns, ts = sample_indices(n, t, 1500, seed, (15, 16, 255, 256, n - 1), (31, 32, 33, 127, 128, 511, 512, 1023))
    ref = oracle.linear_fmt_at(fmt, x, w, hi, sc, n, k, t, ns, ts)
    assert_close(got[ts, ns], ref, what="%s T=1024 sampled" % inputs.FMT_NAMES[fmt])


@pytest.mark.parametrize("t", [1, 20])
def test_fmt_offset_codes_give_exact_zeros(t):
    n, k = 96, 640
    x = inputs.gen_x(k, t, 77)
    cases = {
        inputs.FMT_Q5: (np.zeros((n, k // 2), np.uint8), np.full((n, k // 8), 0xFF, np.uint8)),
        inputs.FMT_Q6: (np.zeros((n, k // 2), np.uint8), np.full((n, k // 4), 0xAA, np.uint8)),
        inputs.FMT_W8: (np.zeros((n, k), np.uint8), None),
        inputs.FMT_NVFP4: (np.full((n, k // 2), 0x88, np.uint8), None),   # E2M1 -0
    }
    for fmt, (w, hi) in cases.items():
        _, _, sc = inputs.gen_fmt_weight(fmt, n, k, 78)
        got = run_fmt(fmt, x, w, hi, sc, n, k, t, what="offset codes")
        assert np.all((got & 0x7FFF) == 0), inputs.FMT_NAMES[fmt]


@pytest.mark.parametrize("fmt", [inputs.FMT_Q5, inputs.FMT_Q6, inputs.FMT_W8], ids=["Q5", "Q6", "W8"])
def test_fmt_wide_range_scales(fmt):
    """fp16 scales over many binades (subnormal, negative, zero) and
    activations over many binades."""
    n, k, t = 64, 1024, 9
    r = np.random.default_rng(5 + fmt)
    w, hi, sc = inputs.gen_fmt_weight(fmt, n, k, 91)
    m = sc.size
    sv = r.choice([-1, 1], size=m) * np.ldexp(r.uniform(1, 2, m), r.integers(-24, 12, m))
    sv[r.random(m) < 0.05] = 0.0
    sc = sv.astype(np.float16).view(np.uint16).reshape(sc.shape)
    xv = (r.standard_normal((t, k)) * np.ldexp(1.0, r.integers(-20, 20, (t, k)))).astype(np.float32)
    x = inputs.f32_to_bf16_bits(xv)
    got = run_fmt(fmt, x, w, hi, sc, n, k, t, what="wide range")
    assert_close(got, oracle.linear_fmt(fmt, x, w, hi, sc, n, k, t), what="wide range %s" % inputs.FMT_NAMES[fmt])


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_fmt_inputs_preserved_and_output_guarded(fmt):
    import hashlib
    import weight_only_bit_q4_amd as q4
    th = torch()
    n, k, t = 400, 768, 20
    w, hi, sc = inputs.gen_fmt_weight(fmt, n, k, 4242)
    x = inputs.gen_x(k, t, 4242)
    xd, wd = dev(x), _bytes_dev(w)
    hd = _bytes_dev(hi) if hi is not None else None
    sd = _bytes_dev(sc) if sc is not None else None
    ins = [v for v in (xd, wd, hd, sd) if v is not None]

    def digest(v):
        return hashlib.sha256(v.cpu().contiguous().view(th.uint8).numpy().tobytes()).hexdigest()

    before = [digest(v) for v in ins]
    pad, canary = 4096, 0x5A5A
    buf = th.full((t * n + 2 * pad,), canary, dtype=th.int16, device="cuda")
    y = buf[pad:pad + t * n]
    announce("guard q4lin_linear_fmt fmt=%d n=%d k=%d t=%d" % (fmt, n, k, t))
    st = q4.q4lin_linear_fmt(fmt, xd.data_ptr(), wd.data_ptr(), hd.data_ptr() if hd is not None else 0,
                             sd.data_ptr() if sd is not None else 0, y.data_ptr(), n, k, t, 0, 0,
                             th.cuda.current_stream().cuda_stream)
    assert st == 0, q4.q4lin_status_string(st)
    th.cuda.synchronize()
    assert [digest(v) for v in ins] == before
    h = buf.cpu().numpy()
    assert np.all(h[:pad] == canary) and np.all(h[pad + t * n:] == canary)
    assert_close(host_bits(y).reshape(t, n), oracle.linear_fmt(fmt, x, w, hi, sc, n, k, t), what="guarded")


def test_fmt_q4_is_q4lin_linear():
    """Format 0 through q4lin_linear_fmt is q4lin_linear, bit for bit."""
    import weight_only_bit_q4_amd as q4
    n, k, t = 512, 1024, 70
    x, c, s = inputs.gen_problem(n, k, t, 12)
    a = run_fmt(inputs.FMT_Q4, x, c, None, s, n, k, t, what="fmt Q4")
    xd, cd, sd = dev(x), dev(c), dev(s)
    b = host_bits(q4.linear(xd, cd, sd))
    assert np.array_equal(a, b)


@pytest.mark.parametrize("fmt", [inputs.FMT_Q5, inputs.FMT_W8, inputs.FMT_NVFP4, inputs.FMT_BF16],
                         ids=["Q5", "W8", "NVFP4", "BF16_CTRL"])
@pytest.mark.parametrize("t", [1, 16, 40])
def test_fmt_graph_replay_with_changed_inputs(fmt, t):
    """One format call captured in a HIP graph (the one-token GEMV, the
    few-token and the many-token kernels); the activations and every weight
    plane are then overwritten in place before each replay, with unrelated
    eager work between replays: every replay matches the oracle for the
    inputs of that moment (no workspace, no state kept between calls)."""
    import weight_only_bit_q4_amd as q4
    th = torch()
    n, k = 300, 2048
    w0, h0, s0 = inputs.gen_fmt_weight(fmt, n, k, 700 + t)
    x0 = inputs.gen_x(k, t, 701 + t)
    xd = dev(np.asarray(x0, dtype=np.uint16).reshape(t, k))
    wd = _bytes_dev(w0).view(n, -1)
    hd = _bytes_dev(h0) if h0 is not None else None
    sd = _bytes_dev(s0) if s0 is not None else None
    y = th.empty((t, n), dtype=th.bfloat16, device="cuda")
    q4.linear_fmt(fmt, xd, wd, hd, sd, y=y)   # warm-up outside capture
    th.cuda.synchronize()
    g = th.cuda.CUDAGraph()
    announce("format graph capture fmt=%d n=%d k=%d t=%d" % (fmt, n, k, t))
    with th.cuda.graph(g):
        q4.linear_fmt(fmt, xd, wd, hd, sd, y=y)
    for rep in range(3):
        w, hi, sc = inputs.gen_fmt_weight(fmt, n, k, 710 + 10 * rep + t)
        x = inputs.gen_x(k, t, 711 + 10 * rep + t)
        xd.copy_(dev(np.asarray(x, dtype=np.uint16).reshape(t, k)))
        wd.copy_(_bytes_dev(w).view(n, -1))
        if hd is not None:
            hd.copy_(_bytes_dev(hi))
        if sd is not None:
            sd.copy_(_bytes_dev(sc))
        th.cuda.synchronize()
        g.replay()
        th.cuda.synchronize()
        assert_close(host_bits(y), oracle.linear_fmt(fmt, x, w, hi, sc, n, k, t),
                     what="%s replay %d T=%d" % (inputs.FMT_NAMES[fmt], rep, t))
        junk = th.randn(1 << 20, device="cuda")
        junk.sum().item()
