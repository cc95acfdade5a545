"""GPU parity of pg_qgemv against the oracle's fp64 product (the batch-1
generation path: one pass over the compressed weights per token, article
"8 open models...", section "What 2-bit keeps").  Bar: relative error
||y - y_ref|| / ||y_ref|| <= 1e-3 per output vector (fp32 accumulation
gives ~1e-6)."""
import numpy as np
import pytest

import qgemv_amd as q
from oracle import p8f
from qgemv_amd import synth
from tests.helpers import TOL, dev, encoded_qwen, encoded_single, host, rel_err_rows

pytestmark = pytest.mark.gpu


def _qgemv(codes, scales, x, x_dt):
    import torch
    n, kg = codes.shape
    k = 4 * kg
    b = x.shape[0]
    y = torch.empty((b, n), dtype=torch.float32, device="cuda")
    q.pg_qgemv(dev(codes), dev(scales), n, k, dev(x), x_dt, b, y)
    torch.cuda.synchronize()
    return host(y)


def _x(b, k, x_dt, seed=7):
    f = np.random.default_rng(seed).standard_normal((b, k), dtype=np.float32)
    return f if x_dt == q.PG_F32 else f.astype(np.float16)


@pytest.mark.parametrize("x_dt", [q.PG_F32, q.PG_F16])
@pytest.mark.parametrize("batch", [1, 2, 3, 4, 8])
def test_single_layer(batch, x_dt):
    codes, scales = encoded_single()
    x = _x(batch, 2048, x_dt)
    y = _qgemv(codes, scales, x, x_dt)
    ref = p8f.gemv_ref(codes, scales, x)
    assert np.max(rel_err_rows(y, ref)) <= TOL


@pytest.mark.parametrize("name", list(synth.MATS))
def test_qwen_layer_matrices_batch1(name):
    codes, scales = encoded_qwen(name)
    x = _x(1, codes.shape[1] * 4, q.PG_F16)
    y = _qgemv(codes, scales, x, q.PG_F16)
    ref = p8f.gemv_ref(codes, scales, x)
    assert np.max(rel_err_rows(y, ref)) <= TOL


@pytest.mark.parametrize("n,k", [(1, 128), (33, 256), (45, 384), (100, 1152), (7, 14336), (64, 9728)])
def test_ragged_shapes(n, k):
    rng = np.random.default_rng(n + k)
    codes = rng.integers(0, 256, (n, k // 4), dtype=np.uint8)
    scales = synth.random_scale_bits(n, k, n * 7 + 1)
    for b in (1, 4):
        x = _x(b, k, q.PG_F32, seed=b)
        y = _qgemv(codes, scales, x, q.PG_F32)
        assert np.max(rel_err_rows(y, p8f.gemv_ref(codes, scales, x))) <= TOL


def test_one_hot_returns_decoded_column():
    codes, scales = encoded_single()
    w = p8f.decode_weights(codes, scales)
    for col in (0, 1, 63, 64, 127, 128, 2047):
        x = np.zeros((1, 2048), np.float32)
        x[0, col] = 1.0
        y = _qgemv(codes, scales, x, q.PG_F32)
        assert np.array_equal(y[0].astype(np.float64), w[:, col])


def test_zero_input_and_determinism():
    codes, scales = encoded_qwen("o")
    k = codes.shape[1] * 4
    assert not _qgemv(codes, scales, np.zeros((1, k), np.float32), q.PG_F32).any()
    x = _x(4, k, q.PG_F16)
    a = _qgemv(codes, scales, x, q.PG_F16)
    b = _qgemv(codes, scales, x, q.PG_F16)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("shapes_fn,layer", [(synth.qwen3_4b_shapes, 0), (synth.llama31_8b_shapes, 3)])
def test_stack_shapes_sampled_rows(shapes_fn, layer):
    """Full-size merged launches of a random-code stack layer (as timed by the
    benchmark) checked on 256 sampled output rows per matrix."""
    shapes = shapes_fn()
    merged = synth.random_layer_merged(layer, shapes)
    rng = np.random.default_rng(layer)
    for site, (codes, scales) in merged.items():
        n, kg = codes.shape
        for b in (1, 4):
            x = _x(b, 4 * kg, q.PG_F16, seed=11 + b)
            y = _qgemv(codes, scales, x, q.PG_F16)
            rows = np.sort(rng.choice(n, 256, replace=False))
            ref = p8f.gemv_ref(codes[rows], scales[rows], x)
            assert np.max(rel_err_rows(y[:, rows], ref)) <= TOL, site
