"""GPU parity of the fused stage pg_rot_qgemv (RMS normalisation + rotation +
product in one launch) against the oracle's fp64 chain of the same steps,
for both of its kernels: v_dot4 (batch 1, and any batch when forced,
activations quantised per 32 values) and the int8 matrix cores (batch 2..8,
per 128-block)."""
import numpy as np
import pytest

import qgemv_amd as q
from oracle import p8f
from qgemv_amd import synth
from qgemv_amd.stack import Stack
from tests.helpers import TOL, dev, encoded_qwen, host, oracle_chain, rel_err, rel_err_rows

pytestmark = pytest.mark.gpu


_KFLAGS = {"auto": 0, "vdot": q.PG_FLAG_KERNEL_VDOT, "mma": q.PG_FLAG_KERNEL_MMA}
_kflag = [0]


@pytest.fixture(params=["auto", "vdot", "mma"])
def kernel(request):
    """Which kernel pg_rot_qgemv runs: its own choice by batch (the
    register-rotation stage at batch 1 for k <= 4096, the matrix-core stage
    from batch 2), the v_dot4 stage with the matrix-core rotation at every
    batch (PG_FLAG_KERNEL_VDOT), or the matrix-core stage at every batch
    (PG_FLAG_KERNEL_MMA; it takes k <= 4096 only and leaves larger k to the
    library's choice)."""
    _kflag[0] = _KFLAGS[request.param]
    yield request.param
    _kflag[0] = 0


def _run(codes, scales, x, x_dt, ldx, k, sb, flags):
    import torch
    n = codes.shape[0]
    b = x.shape[0]
    y = torch.empty((b, n), dtype=torch.float32, device="cuda")
    q.pg_rot_qgemv(dev(codes), dev(scales), n, k, dev(x), x_dt, ldx, dev(sb), flags | _kflag[0], b, y)
    torch.cuda.synchronize()
    return host(y)


@pytest.mark.parametrize("name", ["q", "o", "gate", "down"])
def test_fp16_input_no_norm(name, kernel):
    codes, scales = encoded_qwen(name)
    k = codes.shape[1] * 4
    x = synth.activations_fp16(1, k)
    sb = synth.site_sign_bits(0, synth.SITE_OF[name], k)
    y = _run(codes, scales, x, q.PG_F16, k, k, sb, 0)
    ref = p8f.gemv_ref(codes, scales, p8f.rotate(x.astype(np.float64), sb))
    assert rel_err(y, ref) <= TOL


@pytest.mark.parametrize("batch", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("n,k,ldx", [(33, 128, 128), (100, 640, 700), (512, 2560, 6144), (64, 9728, 19456),
                                     (300, 4096, 4096), (40, 16384, 16384), (2000, 2560, 2560)])
def test_rmsnorm_strided_fp32_input(n, k, ldx, batch, kernel):
    rng = np.random.default_rng(n + k + batch)
    codes = rng.integers(0, 256, (n, k // 4), dtype=np.uint8)
    scales = synth.random_scale_bits(n, k, n)
    x = (rng.standard_normal((batch, ldx)) * 7.0).astype(np.float32)
    sb = rng.integers(0, 256, k // 8, dtype=np.uint8)
    ref = p8f.gemv_ref(codes, scales, p8f.rotate(p8f.rmsnorm16(x[:, :k].astype(np.float64)), sb))
    y = _run(codes, scales, x, q.PG_F32, ldx, k, sb, q.PG_FLAG_RMSNORM)
    assert np.max(rel_err_rows(y, ref)) <= TOL
    # repeated calls are bitwise identical
    y2 = _run(codes, scales, x, q.PG_F32, ldx, k, sb, q.PG_FLAG_RMSNORM)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("batch", [1, 5])
def test_fp16_input_rmsnorm_and_ragged_rows(batch, kernel):
    rng = np.random.default_rng(11 + batch)
    n, k = 1001, 1152
    codes = rng.integers(0, 256, (n, k // 4), dtype=np.uint8)
    scales = synth.random_scale_bits(n, k, 3)
    x = (rng.standard_normal((batch, k)) * 3.0).astype(np.float16)
    sb = rng.integers(0, 256, k // 8, dtype=np.uint8)
    ref = p8f.gemv_ref(codes, scales, p8f.rotate(p8f.rmsnorm16(x.astype(np.float64)), sb))
    y = _run(codes, scales, x, q.PG_F16, k, k, sb, q.PG_FLAG_RMSNORM)
    assert np.max(rel_err_rows(y, ref)) <= TOL


def test_zero_input_gives_zero_output(kernel):
    n, k = 96, 512
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, (n, k // 4), dtype=np.uint8)
    scales = synth.random_scale_bits(n, k, 5)
    sb = rng.integers(0, 256, k // 8, dtype=np.uint8)
    y = _run(codes, scales, np.zeros((2, k), np.float16), q.PG_F16, k, k, sb, 0)
    assert np.all(y == 0.0)
    y = _run(codes, scales, np.zeros((2, k), np.float32), q.PG_F32, k, k, sb, q.PG_FLAG_RMSNORM)
    assert np.all(y == 0.0)


@pytest.mark.parametrize("shapes_fn,layers", [(synth.qwen3_4b_shapes, 2), (synth.llama31_8b_shapes, 2)])
def test_fused_chain_matches_oracle(shapes_fn, layers):
    import torch
    shapes = shapes_fn()
    st = Stack(shapes, layers, fused=True)
    got = host(st.token()).copy()
    torch.cuda.synchronize()
    codes, scales, signs = zip(*[st.host_arrays(l) for l in range(layers)])
    ref = oracle_chain(list(codes), list(scales), list(signs), shapes, host(st.h0).astype(np.float64), layers)
    assert rel_err(got, ref) <= TOL
    d2 = host(st.token())
    assert np.array_equal(d2.view(np.uint32), got.view(np.uint32))


@pytest.mark.parametrize("batch", [1, 8])
def test_fused_graph_replays_match_eager(batch):
    import torch
    st = Stack(synth.qwen3_4b_shapes(), 3, batch=batch, fused=True)
    eager = host(st.token()).copy()
    st.capture()
    for i in range(4):
        st.out["down"].zero_()
        torch.cuda.synchronize()
        got = host(st.replay())
        assert np.array_equal(got.view(np.uint32), eager.view(np.uint32)), i
        assert np.array_equal(host(st.token()).view(np.uint32), eager.view(np.uint32))


def test_fused_and_split_paths_agree():
    shapes = synth.llama31_8b_shapes()
    a = host(Stack(shapes, 3, fused=True).token())
    b = host(Stack(shapes, 3, fused=False).token())
    assert rel_err(a, b) <= 1e-3
