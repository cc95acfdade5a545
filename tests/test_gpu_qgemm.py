"""GPU parity of pg_qgemm (the prompt path on the matrix cores) against the
oracle's fp64 product on the same bf16 activations.  Bar: relative error
<= 1e-3 per output row."""
import numpy as np
import pytest

import qgemv_amd as q
from oracle import p8f
from qgemv_amd import synth
from tests.helpers import TOL, dev, encoded_qwen, host, rel_err_rows

pytestmark = pytest.mark.gpu


def _qgemm(codes, scales, xb):
    import torch
    n, kg = codes.shape
    k = 4 * kg
    m = xb.shape[0]
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    q.pg_qgemm(dev(codes), dev(scales), n, k, dev(xb), m, y)
    torch.cuda.synchronize()
    return host(y)


@pytest.fixture(params=["auto", "1", "2"])
def kernel(request, monkeypatch):
    """Which product kernel pg_qgemm runs: its own choice by grid size, or
    one forced through PG_QGEMM_KERNEL (the 128x128 tile or the pipelined
    256x128 tile)."""
    if request.param == "auto":
        monkeypatch.delenv("PG_QGEMM_KERNEL", raising=False)
    else:
        monkeypatch.setenv("PG_QGEMM_KERNEL", request.param)
    return request.param


@pytest.mark.parametrize("m,n,k", [(128, 128, 128), (256, 384, 512), (77, 130, 640), (1, 5, 256), (300, 1024, 2560),
                                   (513, 257, 1152)])
def test_small_and_ragged(m, n, k, kernel):
    rng = np.random.default_rng(m * n + k)
    codes = rng.integers(0, 256, (n, k // 4), dtype=np.uint8)
    scales = synth.random_scale_bits(n, k, m + n)
    xb = synth.bf16_activations_bits(m, k, seed=m)
    y = _qgemm(codes, scales, xb)
    ref = p8f.gemm_ref(codes, scales, p8f.bf16_bits_to_float(xb))
    assert np.max(rel_err_rows(y, ref)) <= TOL


def test_encoded_matrix_m512(kernel):
    codes, scales = encoded_qwen("k")
    xb = synth.bf16_activations_bits(512, codes.shape[1] * 4)
    y = _qgemm(codes, scales, xb)
    ref = p8f.gemm_ref(codes, scales, p8f.bf16_bits_to_float(xb))
    assert np.max(rel_err_rows(y, ref)) <= TOL


@pytest.mark.parametrize("m", [512, 4096])
def test_prompt_shapes_sampled_rows(m):
    """Full-size Qwen3-4B-shaped launches (merged qkv and gate/up), checked on
    32 sampled activation rows against the oracle."""
    merged = synth.random_layer_merged(0, synth.qwen3_4b_shapes())
    rng = np.random.default_rng(m)
    for site, (codes, scales) in merged.items():
        k = codes.shape[1] * 4
        xb = synth.bf16_activations_bits(m, k, seed=m + k)
        y = _qgemm(codes, scales, xb)
        rows = np.sort(rng.choice(m, 32, replace=False))
        ref = p8f.gemm_ref(codes, scales, p8f.bf16_bits_to_float(xb[rows]))
        assert np.max(rel_err_rows(y[rows], ref)) <= TOL, site


def test_one_hot_column(kernel):
    codes, scales = encoded_qwen("v")
    n, kg = codes.shape
    k = 4 * kg
    w = p8f.decode_weights(codes, scales)
    xb = np.zeros((128, k), np.uint16)
    cols = [0, 5, 127, 128, 1000, 2559]
    for i, c in enumerate(cols):
        xb[i, c] = 0x3F80            # bf16 1.0
    y = _qgemm(codes, scales, xb)
    for i, c in enumerate(cols):
        assert np.array_equal(y[i].astype(np.float64), w[:, c])
    assert not y[len(cols):].any()
