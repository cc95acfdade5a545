"""GPU parity of the table-driven codebook variant (pg_decode_table,
pg_rot_qgemv_table) against the oracle's table decode and fp64 products.
The variant is the codebook half of the small-state coset trellis of the
"Pingala-8" landing page, section "Paper": a group read in state s as byte c
takes the point T[s][c] of a caller-supplied int8 table.  Tables: P8F v1's
own (from the library's pg_codebook_table on the GPU side, the oracle's
codebook_table on the other), and seeded uniform-int8 and rounded-Gaussian
tables from the input generators.  Decode is bit-exact; products are within
the relative error bar of the fp64 oracle, and with v1's table bitwise equal
to pg_rot_qgemv's batch-1 stage."""
import numpy as np
import pytest

import qgemv_amd as q
from oracle import p8f
from qgemv_amd import synth
from qgemv_amd.stack import Stack
from tests.helpers import TOL, dev, host, oracle_chain, rel_err, rel_err_rows

pytestmark = pytest.mark.gpu


def _decode_table(codes, scales, k, table, flags=0):
    import torch
    n = codes.shape[0]
    w = torch.empty((n, k), dtype=torch.float32, device="cuda")
    q.pg_decode_table(dev(codes), dev(scales), n, k, dev(table), flags, w)
    torch.cuda.synchronize()
    return host(w)


def _stage_table(codes, scales, k, x, x_dt, sb, table, flags):
    import torch
    n = codes.shape[0]
    y = torch.empty((1, n), dtype=torch.float32, device="cuda")
    q.pg_rot_qgemv_table(dev(codes), dev(scales), n, k, dev(x), x_dt, dev(sb), dev(table), flags, y)
    torch.cuda.synchronize()
    return host(y)


def _stage_v1(codes, scales, k, x, x_dt, sb, flags):
    import torch
    n = codes.shape[0]
    y = torch.empty((1, n), dtype=torch.float32, device="cuda")
    q.pg_rot_qgemv(dev(codes), dev(scales), n, k, dev(x), x_dt, k, dev(sb), flags, 1, y)
    torch.cuda.synchronize()
    return host(y)


def _tables():
    return {"v1": (q.pg_codebook_table(), p8f.codebook_table()),
            "r23": (q.pg_codebook_table_ex(q.PG_FLAG_RATE23), p8f.codebook_table_r23()),
            "uniform": (synth.random_codebook_table(21, "uniform"),) * 2,
            "gauss": (synth.random_codebook_table(22, "gauss"),) * 2}


# table and trellis: each table read on P8F v1's trellis, the rate-2/3
# variant's own table on its trellis, and a random table on the rate-2/3
# trellis
_CASES = [("v1", False), ("uniform", False), ("gauss", False), ("r23", True), ("gauss", True)]


@pytest.mark.parametrize("tname,r23", _CASES)
@pytest.mark.parametrize("carry", [False, True])
@pytest.mark.parametrize("n,k", [(37, 640), (300, 4096), (3, 16384)])
def test_decode_table_bit_exact(n, k, carry, tname, r23):
    gpu_t, ora_t = _tables()[tname]
    rng = np.random.default_rng(n + k)
    codes = rng.integers(0, 256, (n, k // 4), dtype=np.uint8)
    scales = synth.random_scale_bits(n, k, n)
    fl = (q.PG_FLAG_CARRY_STATE if carry else 0) | (q.PG_FLAG_RATE23 if r23 else 0)
    got = _decode_table(codes, scales, k, gpu_t, fl)
    want = p8f.decode_weights_table(codes, scales, ora_t, carry, r23).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_decode_table_v1_equals_closed_form_decode():
    import torch
    n, k = 129, 1280
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 256, (n, k // 4), dtype=np.uint8)
    scales = synth.random_scale_bits(n, k, 4)
    got = _decode_table(codes, scales, k, q.pg_codebook_table())
    w = torch.empty((n, k), dtype=torch.float32, device="cuda")
    q.pg_decode(dev(codes), dev(scales), n, k, w)
    torch.cuda.synchronize()
    assert np.array_equal(got.view(np.uint32), host(w).view(np.uint32))


@pytest.mark.parametrize("n,k", [(33, 128), (100, 640), (512, 2560), (2000, 2560), (300, 4096)])
@pytest.mark.parametrize("x_dt", ["f16", "f32norm"])
def test_stage_with_v1_table_is_bitwise_the_closed_form_stage(n, k, x_dt):
    rng = np.random.default_rng(n * 7 + k)
    codes = rng.integers(0, 256, (n, k // 4), dtype=np.uint8)
    scales = synth.random_scale_bits(n, k, n + 1)
    sb = rng.integers(0, 256, k // 8, dtype=np.uint8)
    if x_dt == "f16":
        x, dt, fl = (rng.standard_normal((1, k))).astype(np.float16), q.PG_F16, 0
    else:
        x, dt, fl = (rng.standard_normal((1, k)) * 5.0).astype(np.float32), q.PG_F32, q.PG_FLAG_RMSNORM
    a = _stage_table(codes, scales, k, x, dt, sb, q.pg_codebook_table(), fl)
    b = _stage_v1(codes, scales, k, x, dt, sb, fl)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("tname,r23", _CASES)
@pytest.mark.parametrize("carry", [False, True])
@pytest.mark.parametrize("n,k", [(33, 128), (100, 640), (512, 2560), (64, 9728), (300, 4096), (40, 16384),
                                 (2000, 2560), (1001, 1152)])
def test_stage_table_matches_oracle(n, k, carry, tname, r23):
    gpu_t, ora_t = _tables()[tname]
    rng = np.random.default_rng(n + 3 * k + carry)
    codes = rng.integers(0, 256, (n, k // 4), dtype=np.uint8)
    scales = synth.random_scale_bits(n, k, n)
    x = (rng.standard_normal((1, k)) * 7.0).astype(np.float32)
    sb = rng.integers(0, 256, k // 8, dtype=np.uint8)
    fl = q.PG_FLAG_RMSNORM | (q.PG_FLAG_CARRY_STATE if carry else 0) | (q.PG_FLAG_RATE23 if r23 else 0)
    y = _stage_table(codes, scales, k, x, q.PG_F32, sb, gpu_t, fl)
    ref = p8f.gemv_table_ref(codes, scales, ora_t, p8f.rotate(p8f.rmsnorm16(x.astype(np.float64)), sb), carry, r23)
    assert np.max(rel_err_rows(y, ref)) <= TOL
    y2 = _stage_table(codes, scales, k, x, q.PG_F32, sb, gpu_t, fl)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("site,n,k", [("gu", 19456, 2560), ("down", 2560, 9728)])
def test_stage_table_full_size_sampled_rows(site, n, k):
    """Qwen3-4B launch-group shapes with a rounded-Gaussian table, fp16
    input without normalisation; 64 sampled rows against the oracle."""
    t = synth.random_codebook_table(23, "gauss")
    codes = synth.random_codes(n, k, 5)
    scales = synth.random_scale_bits(n, k, 6)
    x = synth.activations_fp16(1, k)
    sb = synth.site_sign_bits(0, synth.SITES.index(site), k)
    y = _stage_table(codes, scales, k, x, q.PG_F16, sb, t, 0)
    rows = np.random.default_rng(7).choice(n, 64, replace=False)
    ref = p8f.gemv_table_ref(codes[rows], scales[rows], t, p8f.rotate(x.astype(np.float64), sb))
    got = y[:, rows]
    assert np.max(np.abs(got - ref)) <= TOL * np.sqrt(np.mean(ref * ref)) * 4


def test_stage_table_zero_input():
    n, k = 96, 512
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, (n, k // 4), dtype=np.uint8)
    scales = synth.random_scale_bits(n, k, 5)
    sb = rng.integers(0, 256, k // 8, dtype=np.uint8)
    t = synth.random_codebook_table(1, "uniform")
    assert np.all(_stage_table(codes, scales, k, np.zeros((1, k), np.float16), q.PG_F16, sb, t, 0) == 0.0)
    assert np.all(_stage_table(codes, scales, k, np.zeros((1, k), np.float32), q.PG_F32, sb, t,
                               q.PG_FLAG_RMSNORM) == 0.0)


@pytest.mark.parametrize("shapes_fn,carry,r23", [(synth.qwen3_4b_shapes, False, False),
                                               (synth.llama31_8b_shapes, True, False),
                                               (synth.qwen3_4b_shapes, False, True)])
def test_table_stack_chain_matches_oracle(shapes_fn, carry, r23):
    """Two layers of the stack with every launch group through a table (down
    at k = 9728 / 14336 included): a rounded-Gaussian one on P8F v1's
    trellis, or the rate-2/3 variant's own on its trellis; against the
    oracle's chain with the same table; replays bitwise repeatable."""
    import torch
    if r23:
        t, t_or = q.pg_codebook_table_ex(q.PG_FLAG_RATE23), p8f.codebook_table_r23()
    else:
        t = t_or = synth.random_codebook_table(24, "gauss")
    shapes = shapes_fn()
    st = Stack(shapes, 2, fused=True, carry=carry, table=dev(t), rate23=r23)
    got = host(st.token()).copy()
    torch.cuda.synchronize()
    codes, scales, signs = zip(*[st.host_arrays(l) for l in range(2)])
    ref = oracle_chain(list(codes), list(scales), list(signs), shapes, host(st.h0).astype(np.float64), 2,
                       carry=carry, table=t_or, rate23=r23)
    assert rel_err(got, ref) <= TOL
    assert np.array_equal(host(st.token()).view(np.uint32), got.view(np.uint32))


def test_rate23_stage_and_decode_agree():
    """The rate-2/3 variant's own table: the fused stage's product equals the
    product of the GPU's decoded weights with the oracle's rotated input, to
    the stage's tolerance (two GPU paths through the same trellis)."""
    import torch
    n, k = 257, 1536
    rng = np.random.default_rng(31)
    codes = rng.integers(0, 256, (n, k // 4), dtype=np.uint8)
    scales = synth.random_scale_bits(n, k, 32)
    x = synth.activations_fp16(1, k, seed=33)
    sb = rng.integers(0, 256, k // 8, dtype=np.uint8)
    t = q.pg_codebook_table_ex(q.PG_FLAG_RATE23)
    y = _stage_table(codes, scales, k, x, q.PG_F16, sb, t, q.PG_FLAG_RATE23)
    w = _decode_table(codes, scales, k, t, q.PG_FLAG_RATE23).astype(np.float64)
    ref = w @ p8f.rotate(x.astype(np.float64), sb)[0]
    assert np.max(rel_err_rows(y, ref[None, :])) <= TOL
    torch.cuda.synchronize()
