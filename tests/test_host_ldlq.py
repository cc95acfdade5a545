"""The library's host LDLQ encoder (pg_encode_ref_ldlq, CPU) against the
oracle's block LDLQ: identical codes and scales, the identity Hessian
reducing to pg_encode_ref, and the argument checks on the Hessian.  LDLQ is
named on the "Pingala-8" landing page, section "How it works"."""
import numpy as np
import pytest

import qgemv_amd as q
from oracle import p8f


def _lowrank_spd(k, r, seed, ridge=0.01):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((k, r))
    return a @ a.T / r + ridge * np.eye(k)


def _encode_ref_ldlq(w, sb, h, threads=4):
    n, k = w.shape
    codes = np.zeros((n, k // 4), np.uint8)
    scales = np.zeros((n, k // 128), np.uint16)
    q.pg_encode_ref_ldlq(np.ascontiguousarray(w, dtype=np.float32), n, k, sb, np.ascontiguousarray(h), codes, scales,
                         threads)
    return codes, scales


@pytest.mark.parametrize("n,k,r,seed", [(7, 384, 12, 1), (20, 512, 48, 2), (3, 1280, 32, 3)])
def test_library_ldlq_equals_oracle(n, k, r, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    sb = rng.integers(0, 256, k // 8, dtype=np.uint8)
    h = _lowrank_spd(k, r, seed + 100)
    c_lib, s_lib = _encode_ref_ldlq(w, sb, h)
    c_or, s_or = p8f.encode_matrix_ldlq(w, sb, h)
    assert np.array_equal(s_lib, s_or)
    assert np.array_equal(c_lib, c_or)


def test_identity_hessian_gives_pg_encode_ref():
    rng = np.random.default_rng(4)
    n, k = 9, 640
    w = rng.standard_normal((n, k)).astype(np.float32)
    sb = rng.integers(0, 256, k // 8, dtype=np.uint8)
    c1, s1 = _encode_ref_ldlq(w, sb, np.eye(k))
    c0 = np.zeros((n, k // 4), np.uint8)
    s0 = np.zeros((n, k // 128), np.uint16)
    q.pg_encode_ref(w, n, k, sb, c0, s0, 2)
    assert np.array_equal(c1, c0) and np.array_equal(s1, s0)


def test_library_ldlq_lowers_the_proxy_loss():
    rng = np.random.default_rng(5)
    n, k = 12, 512
    w = rng.standard_normal((n, k)).astype(np.float32)
    sb = rng.integers(0, 256, k // 8, dtype=np.uint8)
    h = _lowrank_spd(k, 16, 6)
    c1, s1 = _encode_ref_ldlq(w, sb, h)
    c0 = np.zeros((n, k // 4), np.uint8)
    s0 = np.zeros((n, k // 128), np.uint16)
    q.pg_encode_ref(w, n, k, sb, c0, s0, 2)
    wr = p8f.rotate(w.astype(np.float64), sb)
    hr = p8f.rotate_hessian(h, sb)
    assert p8f.proxy_loss(wr, p8f.decode_weights(c1, s1), hr) < 0.5 * p8f.proxy_loss(wr, p8f.decode_weights(c0, s0), hr)


@pytest.mark.parametrize("bad", ["indefinite", "asymmetric", "nan"])
def test_hessian_checks(bad):
    k = 256
    h = _lowrank_spd(k, 8, 7)
    if bad == "indefinite":
        h[200:, 200:] -= 50 * np.eye(56)
    elif bad == "asymmetric":
        h[3, 250] += 1.0
    else:
        h[10, 10] = np.nan
    w = np.zeros((2, k), np.float32)
    with pytest.raises(q.PgError) as ei:
        _encode_ref_ldlq(w, np.zeros(k // 8, np.uint8), h)
    assert ei.value.code == q._lib.PG_ERR_INVALID_ARG


def test_k_beyond_the_feedback_matrix_limit():
    rc = q.lib().pg_encode_ref_ldlq(1 << 20, 2, 32768, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1)
    assert rc == q._lib.PG_ERR_UNSUPPORTED
    with pytest.raises(ValueError, match="hessian"):
        q.pg_encode_ref_ldlq(np.zeros((2, 256), np.float32), 2, 256, np.zeros(32, np.uint8), np.eye(128),
                             np.zeros((2, 64), np.uint8), np.zeros((2, 2), np.uint16))
