"""GPU parity of pg_fwht_rotate against the oracle's explicit fp64 rotation
(the run-time activation side of the random Hadamard rotation, "Pingala-8"
landing page, section "How it works")."""
import numpy as np
import pytest

import qgemv_amd as q
from oracle import p8f
from qgemv_amd import synth
from tests.helpers import TOL, dev, host, rel_err_rows

pytestmark = pytest.mark.gpu

DT = {q.PG_F32: np.float32, q.PG_F16: np.float16, q.PG_BF16: np.uint16}


def _input(rows, k, dt, seed):
    f = np.random.default_rng(seed).standard_normal((rows, k), dtype=np.float32) * 3.0
    if dt == q.PG_F32:
        return f, f.astype(np.float64)
    if dt == q.PG_F16:
        h = f.astype(np.float16)
        return h, h.astype(np.float64)
    b = p8f.bf16_rne_bits(f)
    return b, p8f.bf16_bits_to_float(b)


def _run(x_np, in_dt, out_dt, sb, rows, k, flags):
    import torch
    torch_dt = {q.PG_F32: torch.float32, q.PG_F16: torch.float16, q.PG_BF16: torch.bfloat16}[out_dt]
    y = torch.empty((rows, k), dtype=torch_dt, device="cuda")
    q.pg_fwht_rotate(dev(x_np), in_dt, y, out_dt, dev(sb), rows, k, flags)
    torch.cuda.synchronize()
    if out_dt == q.PG_BF16:
        return p8f.bf16_bits_to_float(host(y.view(torch.int16)).view(np.uint16))
    return host(y).astype(np.float64)


@pytest.mark.parametrize("k", [128, 2048, 2560, 9728, 14336])
@pytest.mark.parametrize("in_dt,out_dt", [(q.PG_F16, q.PG_F32), (q.PG_F32, q.PG_F32), (q.PG_BF16, q.PG_BF16),
                                          (q.PG_F16, q.PG_F16)])
def test_rotation_matches_oracle(k, in_dt, out_dt):
    rows = 3
    x_np, x64 = _input(rows, k, in_dt, seed=k)
    sb = synth.site_sign_bits(0, 1, k)
    got = _run(x_np, in_dt, out_dt, sb, rows, k, 0)
    ref = p8f.rotate(x64, sb)
    if out_dt == q.PG_F32:
        assert np.max(rel_err_rows(got, ref)) <= 1e-6
    else:
        # equal to the rounded oracle value except where fp32 evaluation sits
        # next to a rounding boundary; there at most one unit in the last place
        ref_r = p8f.fp16_rne(ref) if out_dt == q.PG_F16 else p8f.bf16_bits_to_float(p8f.bf16_rne_bits(ref))
        mant = 10 if out_dt == q.PG_F16 else 7
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref_r), 1e-30))) - mant)
        # outputs that cancel to ~0 are only accurate to fp32's absolute
        # error, about 2^-24 * sqrt(128) * the row's scale
        absb = 1e-6 * np.sqrt(np.mean(ref ** 2, axis=1, keepdims=True))
        bad = got != ref_r
        assert np.all((np.abs(got - ref_r) <= np.maximum(ulp * 1.0001, absb))[bad])
        assert bad.mean() < 0.01


@pytest.mark.parametrize("k", [2560, 4096, 9728])
def test_rmsnorm_then_rotation(k):
    rows = 4
    x = (np.random.default_rng(9).standard_normal((rows, k)) * 40.0).astype(np.float32)
    sb = synth.site_sign_bits(1, 2, k)
    got = _run(x, q.PG_F32, q.PG_F32, sb, rows, k, q.PG_FLAG_RMSNORM)
    ref = p8f.rotate(p8f.rmsnorm16(x.astype(np.float64)), sb)
    # the fp16 rounding after the normalisation may differ by one unit on a
    # few elements (fp32 versus fp64 normalisation); bound from 2^-11 per
    # flipped element
    assert np.max(rel_err_rows(got, ref)) <= 1e-4


def test_many_rows_prompt_shape():
    rows, k = 512, 2560
    b = synth.bf16_activations_bits(rows, k)
    sb = synth.site_sign_bits(0, 0, k)
    got = _run(b, q.PG_BF16, q.PG_F32, sb, rows, k, 0)
    ref = p8f.rotate(p8f.bf16_bits_to_float(b), sb)
    assert np.max(rel_err_rows(got, ref)) <= 1e-6


@pytest.mark.parametrize("in_dt,pad", [("f32", 1), ("f16", 3), ("f32", 4)])
def test_rmsnorm_rows_any_stride(in_dt, pad):
    """Rows ldx = k + pad apart (pad 1 or 3: rows not 16-byte aligned, so the
    sums of squares take element loads; pad 4: 16-byte loads) against the
    oracle's normalisation and rotation, and against the same rows made
    contiguous (the 16-byte path)."""
    import torch
    rows, k = 4, 2560
    ldx = k + pad
    rng = np.random.default_rng(ldx)
    xs = rng.standard_normal((rows, ldx)).astype(np.float32)
    dt, npdt = (q.PG_F32, np.float32) if in_dt == "f32" else (q.PG_F16, np.float16)
    xs = xs.astype(npdt)
    sb = rng.integers(0, 256, k // 8, dtype=np.uint8)
    flat = torch.from_numpy(np.ascontiguousarray(xs).reshape(-1)).cuda()
    y = torch.zeros((rows, k), dtype=torch.float32, device="cuda")
    q.pg_fwht_rotate_ex(flat, dt, ldx, y, q.PG_F32, dev(sb), rows, k, q.PG_FLAG_RMSNORM)
    yc = torch.zeros((rows, k), dtype=torch.float32, device="cuda")
    q.pg_fwht_rotate(dev(np.ascontiguousarray(xs[:, :k])), dt, yc, q.PG_F32, dev(sb), rows, k, q.PG_FLAG_RMSNORM)
    torch.cuda.synchronize()
    got, gotc = host(y), host(yc)
    ref = np.stack([p8f.rotate(p8f.rmsnorm16(xs[r, :k].astype(np.float64)), sb) for r in range(rows)])
    assert np.max(rel_err_rows(got, ref)) <= TOL
    assert np.max(np.abs(got - gotc)) <= 1e-3 * np.max(np.abs(gotc))
