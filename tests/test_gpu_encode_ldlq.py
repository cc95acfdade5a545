"""GPU LDLQ encoder (pg_encode_ldlq) against the host reference
(pg_encode_ref_ldlq): bit-identical codes and scales, on low-rank proxy
Hessians (inputs near a subspace, as real layer inputs) and the identity
(where it must equal pg_encode).  LDLQ: "Pingala-8" landing page, section
"How it works"."""
import numpy as np
import pytest

import qgemv_amd as q
from tests.helpers import dev, host

pytestmark = pytest.mark.gpu


def _lowrank_spd(k, r, seed, ridge=0.01):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((k, r))
    return a @ a.T / r + ridge * np.eye(k)


def _gpu(w, sb, h):
    import torch
    n, k = w.shape
    codes = torch.empty((n, k // 4), dtype=torch.uint8, device="cuda")
    scales = torch.empty((n, k // 128), dtype=torch.int16, device="cuda")
    q.pg_encode_ldlq(dev(w), n, k, dev(sb), np.ascontiguousarray(h), codes, scales)
    return host(codes), host(scales).view(np.uint16)


def _ref(w, sb, h):
    n, k = w.shape
    codes = np.zeros((n, k // 4), np.uint8)
    scales = np.zeros((n, k // 128), np.uint16)
    q.pg_encode_ref_ldlq(w, n, k, sb, np.ascontiguousarray(h), codes, scales, 0)
    return codes, scales


@pytest.mark.parametrize("n,k,r,seed", [(64, 512, 16, 1), (300, 1024, 48, 2), (40, 2560, 64, 3), (5, 128, 8, 4)])
def test_gpu_ldlq_bit_identical_to_reference(n, k, r, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    w.reshape(-1)[rng.choice(w.size, max(1, w.size // 1000), replace=False)] *= 20.0     # outliers
    sb = rng.integers(0, 256, k // 8, dtype=np.uint8)
    h = _lowrank_spd(k, r, seed + 50)
    cg, sg = _gpu(w, sb, h)
    cr, sr = _ref(w, sb, h)
    assert np.array_equal(sg, sr)
    assert np.array_equal(cg, cr)


def test_gpu_ldlq_identity_equals_pg_encode():
    import torch
    rng = np.random.default_rng(9)
    n, k = 96, 768
    w = rng.standard_normal((n, k)).astype(np.float32)
    sb = rng.integers(0, 256, k // 8, dtype=np.uint8)
    cg, sg = _gpu(w, sb, np.eye(k))
    codes = torch.empty((n, k // 4), dtype=torch.uint8, device="cuda")
    scales = torch.empty((n, k // 128), dtype=torch.int16, device="cuda")
    q.pg_encode(dev(w), n, k, dev(sb), codes, scales)
    torch.cuda.synchronize()
    assert np.array_equal(cg, host(codes)) and np.array_equal(sg, host(scales).view(np.uint16))


def test_gpu_ldlq_zero_rows():
    """All-zero rows: zero scales and zero codes in every block (the
    feedback of a zero error is zero)."""
    n, k = 8, 384
    w = np.zeros((n, k), np.float32)
    w[3] = 1.0
    sb = np.zeros(k // 8, np.uint8)
    h = _lowrank_spd(k, 8, 3)
    cg, sg = _gpu(w, sb, h)
    cr, sr = _ref(w, sb, h)
    assert np.array_equal(cg, cr) and np.array_equal(sg, sr)
    assert not np.any(sg[[0, 1, 2, 4, 5, 6, 7]]) and not np.any(cg[[0, 1, 2, 4, 5, 6, 7]])
