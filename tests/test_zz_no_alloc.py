"""The no-allocation entry point (q4lin_linear_noalloc) against q4lin_linear
through the C ABI: the same kernels, so the outputs must be bit-identical,
and both within the tolerance of the oracle.  Two calls in a row on the
shared scratch array, the second with a smaller problem, for each of the
routes that use scratch (the many-token route with and without a K split)
and one that does not (a single token)."""
import numpy as np
import pytest

from gpu_util import announce, assert_close, dev, host_bits, oracle_full, oracle_sampled, sample_indices, torch
from weight_only_bit_q4_amd import inputs

pytestmark = pytest.mark.gpu


def _both(x, c, s, n, k, t, what):
    import weight_only_bit_q4_amd as q4
    th = torch()
    xd, cd, sd = dev(x.reshape(t, k)), dev(c.reshape(n, k // 2)), dev(s.reshape(n, k // 64))
    need = q4.q4lin_workspace_bytes(n, k, t)
    assert 0 <= need <= q4.q4lin_noalloc_scratch_bytes()
    ws = th.empty(max(need, 1), dtype=th.uint8, device="cuda")
    y_ref = th.full((t, n), 0x7FC1, dtype=th.int16, device="cuda")
    y_na = th.full((t, n), 0x7FC1, dtype=th.int16, device="cuda")
    h = th.cuda.current_stream().cuda_stream
    announce("%s q4lin_linear n=%d k=%d t=%d route=%d" % (what, n, k, t, q4.q4lin_route(n, k, t)))
    st = q4.q4lin_linear(xd.data_ptr(), cd.data_ptr(), sd.data_ptr(), y_ref.data_ptr(), n, k, t,
                         ws.data_ptr(), need, h)
    assert st == 0, q4.q4lin_status_string(st)
    announce("%s q4lin_linear_noalloc n=%d k=%d t=%d" % (what, n, k, t))
    st = q4.q4lin_linear_noalloc(xd.data_ptr(), cd.data_ptr(), sd.data_ptr(), y_na.data_ptr(), n, k, t, h)
    assert st == 0, q4.q4lin_status_string(st)
    th.cuda.synchronize()
    return host_bits(y_ref), host_bits(y_na)


@pytest.mark.parametrize("first,second", [
    ((6144, 5120, 1024), (1000, 2048, 300)),   # many-token route, then a smaller one
    ((1000, 2048, 200), (700, 1728, 160)),     # K split over workgroups (partials in scratch)
    ((6144, 5120, 1), (512, 1024, 1)),         # single token: no scratch at all
], ids=["tiled", "k_split", "one_token"])
def test_noalloc_matches_linear_two_calls(first, second):
    for i, (n, k, t) in enumerate((first, second)):
        x, c, s = inputs.gen_problem(n, k, t, 8100 + 7 * i + n + t)
        y_ref, y_na = _both(x, c, s, n, k, t, "noalloc call %d" % (i + 1))
        assert np.array_equal(y_ref, y_na), "noalloc differs from q4lin_linear at %dx%d T=%d" % (n, k, t)
        if n * k * t <= (1 << 31):
            assert_close(y_na, oracle_full(x, c, s, n, k, t), what="noalloc %dx%d T=%d" % (n, k, t))
        else:
            ns, ts = sample_indices(n, t, 2000, 8200 + i, (95, 96, n - 1), (255, 256, t - 1))
            assert_close(y_na[ts, ns], oracle_sampled(x, c, s, n, k, t, ns, ts),
                         what="noalloc %dx%d T=%d sampled" % (n, k, t))
