"""GPU parity of the carried-state variant (the trellis state runs on from
block to block along a row; oracle: p8f's carry functions, pinned in
test_oracle_carry.py): decode bit-exact, the fused stage within the product
tolerance, the GPU encoder at the oracle's optimum, and a chained stack."""
import numpy as np
import pytest

import qgemv_amd as q
from oracle import p8f
from qgemv_amd import synth
from qgemv_amd.stack import Stack
from tests.helpers import TOL, dev, host, oracle_chain, rel_err

pytestmark = pytest.mark.gpu
CARRY = q.PG_FLAG_CARRY_STATE


@pytest.mark.parametrize("n,k", [(5, 128), (33, 640), (64, 2560), (17, 9728)])
def test_decode_bit_exact(n, k):
    import torch
    rng = np.random.default_rng(n + k)
    codes = rng.integers(0, 256, (n, k // 4), dtype=np.uint8)
    scales = synth.random_scale_bits(n, k, n)
    w = torch.empty((n, k), dtype=torch.float32, device="cuda")
    q.pg_decode_ex(dev(codes), dev(scales), n, k, CARRY, w)
    torch.cuda.synchronize()
    want = p8f.decode_weights(codes, scales, carry=True).astype(np.float32)
    assert np.array_equal(host(w).view(np.uint32), want.view(np.uint32))
    q.pg_decode_ex(dev(codes), dev(scales), n, k, 0, w)
    torch.cuda.synchronize()
    assert np.array_equal(host(w).view(np.uint32), p8f.decode_weights(codes, scales).astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("batch", [1, 3])
@pytest.mark.parametrize("n,k", [(100, 640), (512, 2560), (64, 9728), (40, 16384), (2000, 2560)])
def test_fused_stage(n, k, batch):
    import torch
    rng = np.random.default_rng(n + k + batch)
    codes = rng.integers(0, 256, (n, k // 4), dtype=np.uint8)
    scales = synth.random_scale_bits(n, k, 3)
    sb = rng.integers(0, 256, k // 8, dtype=np.uint8)
    x = (rng.standard_normal((batch, k)) * 3.0).astype(np.float32)
    y = torch.empty((batch, n), dtype=torch.float32, device="cuda")
    q.pg_rot_qgemv(dev(codes), dev(scales), n, k, dev(x), q.PG_F32, k, dev(sb), q.PG_FLAG_RMSNORM | CARRY, batch, y)
    torch.cuda.synchronize()
    ref = p8f.gemv_ref(codes, scales, p8f.rotate(p8f.rmsnorm16(x.astype(np.float64)), sb), carry=True)
    assert rel_err(host(y), ref) <= TOL
    # the same codes read per block give a different product
    ref_v1 = p8f.gemv_ref(codes, scales, p8f.rotate(p8f.rmsnorm16(x.astype(np.float64)), sb))
    assert rel_err(ref_v1, ref) > 10 * TOL


def _gpu_encode_carry(w, sb):
    import torch
    n, k = w.shape
    codes = torch.empty((n, k // 4), dtype=torch.uint8, device="cuda")
    scales = torch.empty((n, k // 128), dtype=torch.int16, device="cuda")
    q.pg_encode_ex(dev(w), n, k, dev(sb), CARRY, codes, scales)
    torch.cuda.synchronize()
    return host(codes), host(scales).view(np.uint16)


@pytest.mark.parametrize("n,k", [(6, 256), (20, 1024), (8, 4096)])
def test_encoder_reaches_the_oracle_optimum(n, k):
    rng = np.random.default_rng(k + n)
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    w[0, 128:256] = 0.0 if k > 128 else w[0, 128:256]       # a zero-scale block inside a row
    sb = rng.integers(0, 256, k // 8, dtype=np.uint8)
    gc, gs = _gpu_encode_carry(w, sb)
    oc, os_ = p8f.encode_matrix_carry(w, sb)
    assert np.array_equal(gs, os_)
    wr = p8f.rotate(w.astype(np.float64), sb).reshape(n, k // 128, 128)
    differ = 0
    for r in range(n):
        if np.array_equal(gc[r], oc[r]):
            continue
        differ += 1
        dg = p8f.row_distortion_carry(wr[r], gc[r].reshape(-1, 32), gs[r])
        do = p8f.row_distortion_carry(wr[r], oc[r].reshape(-1, 32), os_[r])
        assert abs(dg - do) <= 1e-12 * do, r
    assert differ <= max(1, n // 10)
    if k > 128:
        assert not gc[0, 32:64].any()                        # the zero block is 32 zero bytes


def test_encode_ex_without_flags_is_pg_encode():
    import torch
    rng = np.random.default_rng(5)
    w = (0.02 * rng.standard_normal((9, 512))).astype(np.float32)
    sb = rng.integers(0, 256, 64, dtype=np.uint8)
    a = torch.empty((9, 128), dtype=torch.uint8, device="cuda")
    sa = torch.empty((9, 4), dtype=torch.int16, device="cuda")
    b = torch.empty_like(a)
    sbb = torch.empty_like(sa)
    q.pg_encode(dev(w), 9, 512, dev(sb), a, sa)
    q.pg_encode_ex(dev(w), 9, 512, dev(sb), 0, b, sbb)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(sa, sbb)


def test_chained_stack_matches_oracle():
    import torch
    shapes = synth.qwen3_4b_shapes()
    st = Stack(shapes, 2, fused=True, carry=True)
    got = host(st.token()).copy()
    torch.cuda.synchronize()
    codes, scales, signs = zip(*[st.host_arrays(l) for l in range(2)])
    ref = oracle_chain(list(codes), list(scales), list(signs), shapes, host(st.h0).astype(np.float64), 2, carry=True)
    assert rel_err(got, ref) <= TOL
