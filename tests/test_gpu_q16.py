"""The PG_Q16 fast path: rotation to 16-bit fixed point, and qgemv on it
(both product kernels: v_dot4 per batch row, and the int8 matrix cores that
take batch 2..8 by default).

qgemv is checked against the oracle on host-packed activations (exact fp64
reference of the very values the kernel reads: the bar is fp32 accumulation,
1e-5) and end to end from fp16 activations through the rotation (bar 1e-3)."""
import numpy as np
import pytest

import qgemv_amd as q
from oracle import p8f
from qgemv_amd import synth
from tests import q16pack
from tests.helpers import TOL, dev, encoded_qwen, encoded_single, host, rel_err_rows

pytestmark = pytest.mark.gpu


_KFLAGS = {"auto": 0, "q16": q.PG_FLAG_KERNEL_VDOT, "mma": q.PG_FLAG_KERNEL_MMA}
_kflag = [0]


@pytest.fixture(params=["auto", "q16", "mma"])
def kernel(request):
    """Which PG_Q16 product kernel pg_qgemv_ex runs: its own choice by batch,
    or one selected by PG_FLAG_KERNEL_VDOT / PG_FLAG_KERNEL_MMA."""
    _kflag[0] = _KFLAGS[request.param]
    yield request.param
    _kflag[0] = 0


def _rotate_q16(x_np, in_dt, sb, rows, k, flags=0):
    import torch
    y = torch.zeros((rows, q16pack.row_bytes(k)), dtype=torch.uint8, device="cuda")
    q.pg_fwht_rotate(dev(x_np), in_dt, y, q.PG_Q16, dev(sb), rows, k, flags)
    torch.cuda.synchronize()
    return host(y)


def _qgemv_q16(codes, scales, buf, batch):
    import torch
    n, kg = codes.shape
    y = torch.empty((batch, n), dtype=torch.float32, device="cuda")
    q.pg_qgemv_ex(dev(codes), dev(scales), n, 4 * kg, dev(buf), q.PG_Q16, batch, _kflag[0], y)
    torch.cuda.synchronize()
    return host(y)


def test_row_bytes_matches_library():
    for k in (128, 256, 2560, 9728, 14336):
        assert q.lib().pg_q16_row_bytes(k) == q16pack.row_bytes(k)


@pytest.mark.parametrize("k", [128, 2560, 9728, 14336])
def test_rotation_to_q16_matches_oracle(k):
    rows = 2
    x = synth.activations_fp16(rows, k, seed=k)
    sb = synth.site_sign_bits(0, 2, k)
    buf = _rotate_q16(x, q.PG_F16, sb, rows, k)
    qv, sx, sums = q16pack.unpack(buf, k)
    ref = p8f.rotate(x.astype(np.float64), sb)
    refb = ref.reshape(rows, k // 128, 128)
    mx = np.abs(refb).max(axis=2)
    assert np.allclose(sx, mx / 32512, rtol=1e-5)
    assert np.all(np.abs(qv) <= 32512)
    err = np.abs(q16pack.dequant(qv, sx) - ref).reshape(rows, k // 128, 128)
    assert np.all(err <= 0.5001 * sx[..., None] + 1e-6 * mx[..., None])
    assert np.array_equal(sums, qv.reshape(rows, k // 64, 64).sum(axis=2))


@pytest.mark.parametrize("out_dt", ["q16", "f32"])
def test_rotate_ex_strided_rows_equal_contiguous(out_dt):
    """pg_fwht_rotate_ex over the first k columns of rows ldx apart gives
    exactly what pg_fwht_rotate gives on a contiguous copy of them."""
    import torch
    rows, k, ldx = 5, 2560, 6144
    rng = np.random.default_rng(8)
    xfull = torch.from_numpy(rng.standard_normal((rows, ldx)).astype(np.float32)).cuda()
    xc = xfull[:, :k].contiguous()
    sb = torch.from_numpy(rng.integers(0, 256, k // 8, dtype=np.uint8)).cuda()
    if out_dt == "q16":
        dt, ya, yb = q.PG_Q16, *(torch.zeros((rows, q16pack.row_bytes(k)), dtype=torch.uint8, device="cuda")
                                  for _ in range(2))
    else:
        dt, ya, yb = q.PG_F32, *(torch.zeros((rows, k), dtype=torch.float32, device="cuda") for _ in range(2))
    q.pg_fwht_rotate_ex(xfull, q.PG_F32, ldx, ya, dt, sb, rows, k, q.PG_FLAG_RMSNORM)
    q.pg_fwht_rotate(xc, q.PG_F32, yb, dt, sb, rows, k, q.PG_FLAG_RMSNORM)
    torch.cuda.synchronize()
    assert np.array_equal(host(ya).view(np.uint8), host(yb).view(np.uint8))


@pytest.mark.parametrize("batch", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("n,k", [(512, 2048), (45, 384), (33, 128), (1000, 2560), (300, 9728), (64, 14336)])
def test_qgemv_q16_exact_inputs(n, k, batch, kernel):
    rng = np.random.default_rng(n * 31 + k + batch)
    codes = rng.integers(0, 256, (n, k // 4), dtype=np.uint8)
    scales = synth.random_scale_bits(n, k, n + k)
    qv, sx = q16pack.random_q16(batch, k, seed=batch + k)
    buf = q16pack.pack(qv, sx)
    y = _qgemv_q16(codes, scales, buf, batch)
    ref = p8f.gemv_ref(codes, scales, q16pack.dequant(qv, sx))
    assert np.max(rel_err_rows(y, ref)) <= 1e-5


def test_qgemv_q16_one_hot_per_block(kernel):
    codes, scales = encoded_single()
    k = 2048
    w = p8f.decode_weights(codes, scales)
    qv = np.zeros((1, k), np.int32)
    sx = np.zeros((1, k // 128), np.float32)
    qv[0, 300] = 32512
    sx[0, 300 // 128] = 1.0 / 32512
    y = _qgemv_q16(codes, scales, q16pack.pack(qv, sx), 1)
    assert np.allclose(y[0], w[:, 300], rtol=1e-6, atol=0)


@pytest.mark.parametrize("name", ["q", "o", "down"])
def test_rotate_then_qgemv_end_to_end(name):
    codes, scales = encoded_qwen(name)
    n, kg = codes.shape
    k = 4 * kg
    x = synth.activations_fp16(1, k)
    sb = synth.site_sign_bits(0, synth.SITE_OF[name], k)
    buf = _rotate_q16(x, q.PG_F16, sb, 1, k)
    y = _qgemv_q16(codes, scales, buf, 1)
    ref = p8f.gemv_ref(codes, scales, p8f.rotate(x.astype(np.float64), sb))
    assert np.max(rel_err_rows(y, ref)) <= TOL


@pytest.mark.parametrize("shapes_fn", [synth.qwen3_4b_shapes, synth.llama31_8b_shapes])
def test_stack_shapes_q16_sampled_rows(shapes_fn, kernel):
    merged = synth.random_layer_merged(1, shapes_fn())
    rng = np.random.default_rng(3)
    for site, (codes, scales) in merged.items():
        n, kg = codes.shape
        k = 4 * kg
        for b in (1, 4, 8):
            qv, sx = q16pack.random_q16(b, k, seed=b)
            y = _qgemv_q16(codes, scales, q16pack.pack(qv, sx), b)
            rows = np.sort(rng.choice(n, 256, replace=False))
            ref = p8f.gemv_ref(codes[rows], scales[rows], q16pack.dequant(qv, sx))
            assert np.max(rel_err_rows(y[:, rows], ref)) <= 1e-5, site


@pytest.mark.parametrize("batch", [1, 8])
def test_qgemv_q16_deterministic(batch, kernel):
    codes, scales = encoded_qwen("gate")
    k = codes.shape[1] * 4
    qv, sx = q16pack.random_q16(batch, k, seed=5)
    buf = q16pack.pack(qv, sx)
    a = _qgemv_q16(codes, scales, buf, batch)
    b = _qgemv_q16(codes, scales, buf, batch)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
