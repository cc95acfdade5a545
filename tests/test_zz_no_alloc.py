"""The allocation-free prompt product pg_qgemm_noalloc (the split workspace
is the library's own device scratch) against pg_qgemm_ex with a
caller-allocated workspace of pg_qgemm_workspace_bytes: bitwise equal, on two
calls in a row with the second smaller, and within 1e-3 of the fp64 oracle on
sampled rows.  Shapes whose split would need more than the scratch are
refused before any launch."""
import numpy as np
import pytest

import qgemv_amd as q
from oracle import p8f
from qgemv_amd import synth
from tests.helpers import TOL, dev, host, rel_err_rows


def _case(n, k, m, seed):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, (n, k // 4), dtype=np.uint8)
    scales = synth.random_scale_bits(n, k, seed + 1)
    x = synth.bf16_activations_bits(m, k, seed=seed + 2)
    return codes, scales, x


@pytest.mark.gpu
def test_noalloc_equals_caller_workspace_two_calls():
    import torch
    for n, k, m, seed in ((2560, 4096, 512, 11), (640, 1024, 128, 12)):
        assert q.pg_qgemm_workspace_bytes(n, k, m) > 0          # the split (and the scratch) is used
        codes, scales, x = _case(n, k, m, seed)
        dc, ds, dx = dev(codes), dev(scales.view(np.int16)), dev(x.view(np.int16))
        y0 = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
        y1 = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
        q.pg_qgemm_noalloc(dc, ds, n, k, dx, m, y0)
        wsb = q.pg_qgemm_workspace_bytes(n, k, m)
        ws = torch.empty(wsb // 4, dtype=torch.float32, device="cuda")
        q.pg_qgemm_ex(dc, ds, n, k, dx, m, y1, ws, wsb)
        torch.cuda.synchronize()
        a, b = host(y0), host(y1)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (n, k, m)
        rows = np.random.default_rng(seed).choice(m, 8, replace=False)
        ref = p8f.gemm_ref(codes, scales, p8f.bf16_bits_to_float(x[rows]))
        assert np.max(rel_err_rows(a[rows], ref)) <= TOL


def test_noalloc_refuses_shapes_beyond_the_scratch():
    """Host-side check, no launch: 10240 x 8192 at m = 512 needs 40 MiB of
    split workspace, more than the 32 MiB scratch."""
    n, k, m = 10240, 8192, 512
    assert q.pg_qgemm_workspace_bytes(n, k, m) > 32 << 20
    p = 1 << 20                                    # aligned, never dereferenced: the call fails first
    with pytest.raises(q.PgError) as e:
        q.pg_qgemm_noalloc(p, p, n, k, p, m, p, 0)
    assert e.value.code == q._lib.PG_ERR_UNSUPPORTED and "scratch" in str(e.value)
