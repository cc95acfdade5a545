"""GPU encoder through a codebook table (pg_encode_table) against the host
reference (pg_encode_ref_table): bit-identical codes and scales on P8F v1's
trellis and the rate-2/3 one, with the formats' own tables and non-uniform
ones; sampled rows of a full Qwen3-4B-shaped matrix; and a round trip
through pg_rot_qgemv_table against the oracle.  The table-driven codebook
is the coset-trellis design space of the "Pingala-8" landing page, section
"Paper"."""
import numpy as np
import pytest

import qgemv_amd as q
from oracle import p8f
from qgemv_amd import synth
from tests.helpers import TOL, dev, host, rel_err_rows

pytestmark = pytest.mark.gpu


def _tables():
    return {"v1": q.pg_codebook_table(), "r23": q.pg_codebook_table_ex(q.PG_FLAG_RATE23),
            "gauss": synth.random_codebook_table(41, "gauss"), "uniform": synth.random_codebook_table(42, "uniform")}


def _gpu(w, sb, t, flags):
    import torch
    n, k = w.shape
    codes = torch.empty((n, k // 4), dtype=torch.uint8, device="cuda")
    scales = torch.empty((n, k // 128), dtype=torch.int16, device="cuda")
    q.pg_encode_table(dev(w), n, k, dev(sb), dev(t), flags, codes, scales)
    torch.cuda.synchronize()
    return host(codes), host(scales).view(np.uint16)


def _ref(w, sb, t, flags):
    n, k = w.shape
    codes = np.zeros((n, k // 4), np.uint8)
    scales = np.zeros((n, k // 128), np.uint16)
    q.pg_encode_ref_table(np.ascontiguousarray(w), n, k, sb, np.ascontiguousarray(t), flags, codes, scales, 0)
    return codes, scales


@pytest.mark.parametrize("tname,r23", [("v1", False), ("gauss", False), ("uniform", False), ("r23", True),
                                        ("gauss", True)])
@pytest.mark.parametrize("n,k", [(1, 128), (37, 640), (200, 2560)])
def test_gpu_table_encoder_bit_identical(n, k, tname, r23):
    rng = np.random.default_rng(n + k + r23)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    if n > 2:
        w[2] = 0.0
        w.reshape(-1)[rng.choice(w.size, max(1, w.size // 1000), replace=False)] *= 20.0
    sb = rng.integers(0, 256, k // 8, dtype=np.uint8)
    t = _tables()[tname]
    fl = q.PG_FLAG_RATE23 if r23 else 0
    cg, sg = _gpu(w, sb, t, fl)
    cr, sr = _ref(w, sb, t, fl)
    assert np.array_equal(sg, sr)
    assert np.array_equal(cg, cr)


def test_gpu_table_encoder_full_matrix_sampled_rows():
    """The Qwen3-4B q matrix (4096 x 2560, 0.02 N(0,1) with outliers) through
    a rounded-Gaussian table: 48 sampled rows against the host reference."""
    w = synth.qwen_layer_weights("q")
    n, k = w.shape
    sb = synth.site_sign_bits(0, 0, k)
    t = _tables()["gauss"]
    cg, sg = _gpu(w, sb, t, 0)
    rows = np.sort(np.random.default_rng(4).choice(n, 48, replace=False))
    cr, sr = _ref(np.ascontiguousarray(w[rows]), sb, t, 0)
    assert np.array_equal(cg[rows], cr) and np.array_equal(sg[rows], sr)


@pytest.mark.parametrize("r23", [False, True])
def test_round_trip_through_the_table_stage(r23):
    """Weights encoded on the GPU through a table, then multiplied through
    the same table by the fused stage: within the product tolerance of the
    oracle's product of those codes; sampled rows' codes and scales equal the
    oracle's encoder's."""
    import torch
    rng = np.random.default_rng(50 + r23)
    n, k = 640, 2560
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    sb = synth.site_sign_bits(3, 0, k)
    t = _tables()["r23" if r23 else "gauss"]
    fl = q.PG_FLAG_RATE23 if r23 else 0
    codes, scales = _gpu(w, sb, t, fl)
    x = synth.activations_fp16(1, k, seed=9)
    y = torch.empty((1, n), dtype=torch.float32, device="cuda")
    q.pg_rot_qgemv_table(dev(codes), dev(scales), n, k, dev(x), q.PG_F16, dev(sb), dev(t), fl, y)
    torch.cuda.synchronize()
    ref = p8f.gemv_table_ref(codes, scales, t, p8f.rotate(x.astype(np.float64), sb), rate23=r23)
    assert np.max(rel_err_rows(host(y), ref)) <= TOL
    # the GPU's codes are the oracle's optimum for these weights and table
    rows = np.arange(0, n, 40)
    c_or, s_or = p8f.encode_matrix_table(w[rows], sb, t, r23)
    assert np.array_equal(scales[rows], s_or) and np.array_equal(codes[rows], c_or)
