"""The library's host encoder through a codebook table (pg_encode_ref_table,
CPU) against the oracle's: identical codes and scales on P8F v1's trellis
and on the rate-2/3 one, with the formats' own tables and a non-uniform
one; on v1's own table it is pg_encode_ref.  The table-driven codebook is
the coset-trellis design space of the "Pingala-8" landing page, section
"Paper"."""
import numpy as np
import pytest

import qgemv_amd as q
from oracle import p8f
from qgemv_amd import synth


def _lib_encode(w, sb, table, flags):
    n, k = w.shape
    codes = np.zeros((n, k // 4), np.uint8)
    scales = np.zeros((n, k // 128), np.uint16)
    q.pg_encode_ref_table(w, n, k, sb, np.ascontiguousarray(table), flags, codes, scales, 4)
    return codes, scales


@pytest.mark.parametrize("tname,r23", [("v1", False), ("gauss", False), ("r23", True), ("gauss", True)])
def test_library_table_encoder_equals_oracle(tname, r23):
    rng = np.random.default_rng(17 + r23)
    n, k = 12, 384
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    w[3] = 0.0                                              # zero-scale blocks
    sb = rng.integers(0, 256, k // 8, dtype=np.uint8)
    lib_t = {"v1": q.pg_codebook_table(), "r23": q.pg_codebook_table_ex(q.PG_FLAG_RATE23),
             "gauss": synth.random_codebook_table(40, "gauss")}[tname]
    ora_t = {"v1": p8f.codebook_table(), "r23": p8f.codebook_table_r23(), "gauss": lib_t}[tname]
    c_lib, s_lib = _lib_encode(w, sb, lib_t, q.PG_FLAG_RATE23 if r23 else 0)
    c_or, s_or = p8f.encode_matrix_table(w, sb, ora_t, r23)
    assert np.array_equal(s_lib, s_or)
    assert np.array_equal(c_lib, c_or)


def test_v1_table_encoder_is_pg_encode_ref():
    rng = np.random.default_rng(19)
    n, k = 7, 640
    w = rng.standard_normal((n, k)).astype(np.float32)
    sb = rng.integers(0, 256, k // 8, dtype=np.uint8)
    c1, s1 = _lib_encode(w, sb, q.pg_codebook_table(), 0)
    c0 = np.zeros((n, k // 4), np.uint8)
    s0 = np.zeros((n, k // 128), np.uint16)
    q.pg_encode_ref(w, n, k, sb, c0, s0, 2)
    assert np.array_equal(c1, c0) and np.array_equal(s1, s0)


def test_table_encoder_argument_checks():
    w = np.zeros((2, 256), np.float32)
    with pytest.raises(q.PgError) as ei:
        q.pg_encode_ref_table(w, 2, 256, np.zeros(32, np.uint8), np.zeros((8, 256, 4), np.int8), q.PG_FLAG_CARRY_STATE,
                              np.zeros((2, 64), np.uint8), np.zeros((2, 2), np.uint16))
    assert ei.value.code == q._lib.PG_ERR_INVALID_ARG
    with pytest.raises(ValueError, match="table"):
        q.pg_encode_ref_table(w, 2, 256, np.zeros(32, np.uint8), np.zeros(100, np.int8), 0,
                              np.zeros((2, 64), np.uint8), np.zeros((2, 2), np.uint16))
