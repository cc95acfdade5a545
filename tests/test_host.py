"""CPU tests of libpingala's host side: the C ABI loads and exports every
declared symbol, argument validation fails before any launch, the decode
table equals the oracle's closed form, and the host reference encoder
reproduces the oracle's codes."""
import os
import re

import numpy as np
import pytest

import qgemv_amd as q
from oracle import p8f
from qgemv_amd import synth
from tests.helpers import assert_codes_equivalent

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    txt = open(os.path.join(ROOT, "include", "pingala.h")).read()
    return sorted(set(re.findall(r"\b(pg_[a-z_0-9]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    import ctypes
    lib = q.lib()
    declared = _declared_symbols()
    assert set(declared) == set(q.EXPORTS)
    for name in declared:
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr)


def test_version_and_footprint():
    assert q.pg_version() == (1 << 16) | 1
    assert q.pg_footprint_bytes(512, 2048) == 278528
    assert q.pg_footprint_bytes(0, 2048) == 0
    assert q.pg_footprint_bytes(4, 100) == 0


def test_codebook_table_matches_oracle():
    assert np.array_equal(q.pg_codebook_table(), p8f.codebook_table())


def test_codebook_tables_by_format_match_oracle():
    """pg_codebook_table_ex: 0 is P8F v1's table, PG_FLAG_RATE23 the rate-2/3
    variant's, each equal to the oracle's table of that format."""
    assert np.array_equal(q.pg_codebook_table_ex(0), p8f.codebook_table())
    assert np.array_equal(q.pg_codebook_table_ex(q.PG_FLAG_RATE23), p8f.codebook_table_r23())
    with pytest.raises(q.PgError) as ei:
        q.pg_codebook_table_ex(q.PG_FLAG_CARRY_STATE)
    assert ei.value.code == q._lib.PG_ERR_INVALID_ARG


@pytest.mark.parametrize("call", [
    lambda: q.pg_encode(1 << 20, 8, 200, 1 << 20, 1 << 20, 1 << 20, stream=0),                # k % 128
    lambda: q.pg_encode(1 << 20, 0, 256, 1 << 20, 1 << 20, 1 << 20, stream=0),                # n < 1
    lambda: q.pg_encode(None, 8, 256, 1 << 20, 1 << 20, 1 << 20, stream=0),                   # null w
    lambda: q.pg_encode(1 << 20, 8, 256, 1 << 20, (1 << 20) + 4, 1 << 20, stream=0),          # codes align
    lambda: q.pg_encode((1 << 20) + 2, 8, 256, 1 << 20, 1 << 20, 1 << 20, stream=0),          # w align
    lambda: q.pg_qgemv(1 << 20, 1 << 20, 0, 2048, 1 << 20, 0, 1, 1 << 20, stream=0),        # n < 1
    lambda: q.pg_qgemv(1 << 20, 1 << 20, 8, 100, 1 << 20, 0, 1, 1 << 20, stream=0),         # k % 128
    lambda: q.pg_qgemv(1 << 20, 1 << 20, 8, 256, 1 << 20, 0, 9, 1 << 20, stream=0),         # batch
    lambda: q.pg_qgemv(1 << 20, 1 << 20, 8, 256, 1 << 20, 2, 1, 1 << 20, stream=0),         # bf16 x
    lambda: q.pg_qgemv(None, 1 << 20, 8, 256, 1 << 20, 0, 1, 1 << 20, stream=0),            # null
    lambda: q.pg_qgemv((1 << 20) + 4, 1 << 20, 8, 256, 1 << 20, 0, 1, 1 << 20, stream=0),   # misaligned
    lambda: q.pg_qgemm(1 << 20, 1 << 20, 8, 256, 1 << 20, 0, 1 << 20, stream=0),            # m < 1
    lambda: q.pg_qgemm_ex(1 << 20, 1 << 20, 8, 256, 1 << 20, 4, 1 << 22, None, 64, stream=0),        # null ws
    lambda: q.pg_qgemm_ex(1 << 20, 1 << 20, 8, 256, 1 << 20, 4, 1 << 22, (1 << 24) + 8, 64, stream=0),  # ws align
    lambda: q.pg_qgemm_ex(1 << 20, 1 << 20, 8, 256, 1 << 21, 4, 1 << 22, (1 << 22) + 64, 256, stream=0),  # ws on y
    lambda: q.pg_qgemm_ex(1 << 20, 1 << 20, 8, 256, 1 << 21, 4, 1 << 22, (1 << 21) + 1024, 64, stream=0),  # on x
    lambda: q.pg_qgemm_ex(1 << 20, 1 << 23, 8, 256, 1 << 21, 4, 1 << 22, 1 << 23, 64, stream=0),      # on scales
    lambda: q.pg_qgemm_ex(1 << 20, 1 << 20, 8, 256, 1 << 21, 0, 1 << 22, 1 << 23, 64, stream=0),      # m < 1
    lambda: q.pg_decode(1 << 20, (1 << 20) + 1, 8, 256, 1 << 20, stream=0),                 # scales odd
    lambda: q.pg_fwht_rotate(1 << 20, 0, 1 << 20, 0, 1 << 20, 1, 256, 0, stream=0),         # overlap
    lambda: q.pg_fwht_rotate(1 << 20, 0, 1 << 22, 5, 1 << 20, 1, 256, 0, stream=0),         # dtype
    lambda: q.pg_fwht_rotate(1 << 20, 0, 1 << 22, 0, 1 << 20, 1, 256, 4, stream=0),         # flags
    lambda: q.pg_fwht_rotate_ex(1 << 20, 0, 128, 1 << 22, 0, 1 << 20, 1, 256, 0, stream=0),  # ldx < k
    lambda: q.pg_fwht_rotate_ex(1 << 20, 0, 4096, (1 << 20) + 4 * 4096 + 16, 0, 1 << 20, 2, 256, 0,
                                stream=0),                                                   # overlap, 2nd row
    lambda: q.pg_rot_qgemv(1 << 20, 1 << 20, 8, 256, 1 << 22, 0, 255, 1 << 20, 1, 1, 1 << 24, stream=0),  # ldx < k
    lambda: q.pg_rot_qgemv(1 << 20, 1 << 20, 8, 256, 1 << 22, 0, 256, 1 << 20, 16, 1, 1 << 24, stream=0),  # flags
    lambda: q.pg_rot_qgemv(1 << 20, 1 << 20, 8, 256, 1 << 22, 0, 256, 1 << 20, 13, 1, 1 << 24, stream=0),  # vdot+mma
    lambda: q.pg_qgemv_ex(1 << 20, 1 << 20, 8, 256, 1 << 20, 3, 2, 12, 1 << 24, stream=0),  # vdot+mma
    lambda: q.pg_qgemv_ex(1 << 20, 1 << 20, 8, 256, 1 << 20, 0, 2, 4, 1 << 24, stream=0),   # choice, fp32 x
    lambda: q.pg_qgemv_ex(1 << 20, 1 << 20, 8, 256, 1 << 20, 3, 2, 1, 1 << 24, stream=0),   # flags
    lambda: q.pg_qgemm_tune(1 << 20, 1 << 20, 8, 256, 1 << 21, 4, 1 << 22, None, 0, 9, 0, 0, stream=0),   # kernel
    lambda: q.pg_qgemm_tune(1 << 20, 1 << 20, 8, 256, 1 << 21, 4, 1 << 22, None, 0, 0, -1, 0, stream=0),  # splits
    lambda: q.pg_decode_ex(1 << 20, 1 << 20, 8, 256, 4, 1 << 24, stream=0),                  # flags
    lambda: q.pg_decode_ex(1 << 20, 1 << 20, 8, 200, 2, 1 << 24, stream=0),                  # k % 128
    lambda: q.pg_decode_ex(1 << 20, 1 << 20, 8, 256, 2, (1 << 24) + 4, stream=0),            # w align
    lambda: q.pg_encode_ex(1 << 20, 8, 256, 1 << 20, 4, 1 << 20, 1 << 20, stream=0),          # flags
    lambda: q.pg_encode_ex(1 << 20, 8, 200, 1 << 20, 2, 1 << 20, 1 << 20, stream=0),          # k % 128
    lambda: q.pg_encode_ex(None, 8, 256, 1 << 20, 2, 1 << 20, 1 << 20, stream=0),             # null w
    lambda: q.pg_rot_qgemv(1 << 20, 1 << 20, 8, 256, 1 << 22, 0, 256, 1 << 20, 1, 0, 1 << 24, stream=0),  # batch
    lambda: q.pg_rot_qgemv(1 << 20, 1 << 20, 8, 256, 1 << 22, 3, 256, 1 << 20, 1, 1, 1 << 24, stream=0),  # dtype
    lambda: q.pg_rot_qgemv(1 << 20, 1 << 20, 8, 256, 1 << 22, 0, 256, 1 << 20, 1, 2, 1 << 22, stream=0),  # overlap
    lambda: q.pg_rot_qgemv(1 << 20, 1 << 20, 8, 256, 1 << 22, 0, 258, 1 << 20, 1, 1, 1 << 24, stream=0),  # row align
    lambda: q.pg_rot_qgemv(1 << 20, 1 << 20, 8, 256, 1 << 22, 1, 260, 1 << 20, 1, 1, 1 << 24, stream=0),  # row align
    lambda: q.pg_rot_qgemv(1 << 20, 1 << 20, 8, 256, (1 << 22) + 8, 0, 256, 1 << 20, 1, 1, 1 << 24, stream=0),
    lambda: q.pg_rot_qgemv(1 << 20, 1 << 20, 8, 256, 1 << 22, 0, 256, (1 << 20) + 2, 1, 1, 1 << 24, stream=0),
    lambda: q.pg_decode_table(1 << 20, 1 << 20, 8, 256, 1 << 22, 1, 1 << 24, stream=0),             # flags
    lambda: q.pg_decode_table(1 << 20, 1 << 20, 8, 256, 1 << 22, 32, 1 << 24, stream=0),            # flags
    lambda: q.pg_decode_table(1 << 20, 1 << 20, 8, 256, (1 << 22) + 4, 0, 1 << 24, stream=0),       # table align
    lambda: q.pg_decode_table(1 << 20, 1 << 20, 8, 200, 1 << 22, 0, 1 << 24, stream=0),             # k
    lambda: q.pg_decode_table(1 << 20, 1 << 20, 8, 256, 0, 0, 1 << 24, stream=0),                   # null table
    lambda: q.pg_rot_qgemv_table(1 << 20, 1 << 20, 8, 256, 1 << 22, 0, 1 << 20, 1 << 18, 4, 1 << 24, stream=0),  # flags
    lambda: q.pg_rot_qgemv_table(1 << 20, 1 << 20, 8, 256, 1 << 22, 0, 1 << 20, 1 << 18, 32, 1 << 24, stream=0),
    lambda: q.pg_rot_qgemv_table(1 << 20, 1 << 20, 8, 256, 1 << 22, 2, 1 << 20, 1 << 18, 1, 1 << 24, stream=0),  # dtype
    lambda: q.pg_rot_qgemv_table(1 << 20, 1 << 20, 8, 256, 1 << 22, 0, 1 << 20, (1 << 18) + 8, 1, 1 << 24,
                                 stream=0),                                                            # table align
    lambda: q.pg_rot_qgemv_table(1 << 20, 1 << 20, 8, 256, 1 << 22, 0, 1 << 20, 1 << 18, 1, (1 << 22) + 64,
                                 stream=0),                                                            # x, y overlap
])
def test_invalid_arguments_fail_before_launch(call):
    # the pointers are never dereferenced: validation rejects the call first
    with pytest.raises(q.PgError) as ei:
        call()
    assert ei.value.code == q._lib.PG_ERR_INVALID_ARG
    assert q.pg_last_error() != ""


def test_rot_qgemv_row_stride_beyond_32_bits_is_unsupported():
    # the stage kernels take ldx in 32 bits; validation refuses larger strides
    # before any launch (the pointers are never dereferenced)
    with pytest.raises(q.PgError) as ei:
        q.pg_rot_qgemv(1 << 20, 1 << 20, 8, 256, 1 << 22, 0, 1 << 31, 1 << 20, 1, 1, 1 << 24, stream=0)
    assert ei.value.code == q._lib.PG_ERR_UNSUPPORTED
    assert "2^31" in q.pg_last_error()


def test_encode_ref_equals_oracle_on_single_layer():
    w = synth.single_layer_weights()
    sb = synth.site_sign_bits(0, 0, 2048)
    codes = np.zeros((512, 512), np.uint8)
    scales = np.zeros((512, 16), np.uint16)
    q.pg_encode_ref(w, 512, 2048, sb, codes, scales)
    oc, os_ = p8f.encode_matrix(w, sb)
    assert np.array_equal(scales, os_)
    assert_codes_equivalent(w, sb, codes, oc, scales)


def test_encode_ref_equals_oracle_on_qwen_rows():
    # 64 rows of each Qwen3-4B-shaped matrix (outliers included)
    for name in ("q", "o", "down"):
        w = synth.qwen_layer_weights(name)
        n, k = w.shape
        rows = np.random.default_rng(5).choice(n, 64, replace=False)
        ws = np.ascontiguousarray(w[rows])
        sb = synth.site_sign_bits(0, synth.SITE_OF[name], k)
        codes = np.zeros((64, k // 4), np.uint8)
        scales = np.zeros((64, k // 128), np.uint16)
        q.pg_encode_ref(ws, 64, k, sb, codes, scales, 4)
        oc, os_ = p8f.encode_matrix(ws, sb)
        assert np.array_equal(scales, os_), name
        assert_codes_equivalent(ws, sb, codes, oc, scales)


def test_encode_ref_zero_and_constant_rows():
    w = np.zeros((2, 256), np.float32)
    w[1, :] = 0.5
    sb = np.zeros(32, np.uint8)
    codes = np.full((2, 64), 7, np.uint8)
    scales = np.full((2, 2), 7, np.uint16)
    q.pg_encode_ref(w, 2, 256, sb, codes, scales, 1)
    oc, os_ = p8f.encode_matrix(w, sb)
    assert np.array_equal(scales, os_) and np.array_equal(codes, oc)
    assert not codes[0].any() and not scales[0].any()


def test_encode_ref_rejects_bad_arguments():
    w = np.zeros((2, 200), np.float32)
    with pytest.raises(q.PgError):
        q.pg_encode_ref(w, 2, 200, np.zeros(25, np.uint8), np.zeros((2, 50), np.uint8),
                        np.zeros((2, 2), np.uint16))


def test_rot_qgemv_rejects_k_beyond_its_register_staging():
    with pytest.raises(q.PgError) as ei:
        q.pg_rot_qgemv(1 << 20, 1 << 20, 8, 32768, 1 << 22, 0, 32768, 1 << 20, 1, 1, 1 << 28, stream=0)
    assert ei.value.code == q._lib.PG_ERR_UNSUPPORTED


def test_table_stage_rejects_k_beyond_its_rotation_rounds():
    with pytest.raises(q.PgError) as ei:
        q.pg_rot_qgemv_table(1 << 20, 1 << 20, 8, 32768, 1 << 22, 0, 1 << 20, 1 << 18, 1, 1 << 28, stream=0)
    assert ei.value.code == q._lib.PG_ERR_UNSUPPORTED


def test_table_stage_rejects_fp32_input_without_normalisation():
    with pytest.raises(q.PgError) as ei:
        q.pg_rot_qgemv_table(1 << 20, 1 << 20, 8, 256, 1 << 22, q.PG_F32, 1 << 20, 1 << 18, 0, 1 << 24, stream=0)
    assert ei.value.code == q._lib.PG_ERR_UNSUPPORTED


def test_rot_qgemv_rejects_fp32_input_without_normalisation():
    with pytest.raises(q.PgError) as ei:
        q.pg_rot_qgemv(1 << 20, 1 << 20, 8, 256, 1 << 22, q.PG_F32, 256, 1 << 20, 0, 1, 1 << 24, stream=0)
    assert ei.value.code == q._lib.PG_ERR_UNSUPPORTED


def test_carried_state_encoder_rejects_k_beyond_its_lds_survivors():
    with pytest.raises(q.PgError) as ei:
        q.pg_encode_ex(1 << 20, 8, 32768, 1 << 20, q.PG_FLAG_CARRY_STATE, 1 << 20, 1 << 20, stream=0)
    assert ei.value.code == q._lib.PG_ERR_UNSUPPORTED


def test_qgemm_workspace_bytes():
    """Whole 256 x 128 fp32 tile blocks, at most 7 per tile; none for a shape
    whose tiles fill the chip in whole rounds, none for invalid sizes."""
    tb = 256 * 128 * 4
    for n, k, m in [(2560, 4096, 512), (2560, 9728, 512), (5, 640, 1), (130, 1152, 77), (2560, 4096, 4096),
                    (19456, 2560, 512)]:
        b = q.pg_qgemm_workspace_bytes(n, k, m)
        tiles = -(-n // 128) * -(-m // 256)
        assert b > 0 and b % tb == 0 and b // tb <= min(7, k // 128 - 1) * tiles, (n, k, m, b)
    assert q.pg_qgemm_workspace_bytes(6144, 2560, 4096) == 0               # 768 tiles: three whole rounds
    assert q.pg_qgemm_workspace_bytes(8, 200, 4) == 0
    assert q.pg_qgemm_workspace_bytes(8, 256, 0) == 0
    assert q.pg_qgemm_workspace_bytes(0, 256, 4) == 0


class _FakeDeviceTensor:
    """Stands in for a GPU tensor in the binding's checks (no GPU here)."""

    def __init__(self, nbytes, contiguous=True):
        self._n, self._c, self.is_cuda = nbytes, contiguous, True

    def numel(self):
        return self._n

    def element_size(self):
        return 1

    def is_contiguous(self):
        return self._c

    def data_ptr(self):
        return 1 << 20


@pytest.mark.parametrize("bad,what", [
    (lambda t: q.pg_decode(t(256 * 64 - 1), t(256 * 4), 256, 256, t(256 * 256 * 4)), "codes"),
    (lambda t: q.pg_decode(t(256 * 64), t(256 * 4 - 2), 256, 256, t(256 * 256 * 4)), "scales"),
    (lambda t: q.pg_decode(t(256 * 64), t(256 * 4), 256, 256, t(256 * 256 * 4 - 4)), "w_rot"),
    (lambda t: q.pg_rot_qgemv(t(64 * 64), t(64 * 4), 64, 256, t((300 + 256) * 4 - 4), 0, 300, t(32), 1, 2, t(2 * 64 * 4)),
     "x"),
    (lambda t: q.pg_rot_qgemv(t(64 * 64), t(64 * 4), 64, 256, t(300 * 4 + 256 * 4), 0, 300, t(31), 1, 2,
                              t(2 * 64 * 4)), "sign_bits"),
    (lambda t: q.pg_qgemv(t(64 * 64), t(64 * 4), 64, 256, t(2 * q.pg_q16_row_bytes(256) - 1), 3, 2, t(2 * 64 * 4)),
     "x_rot"),
    (lambda t: q.pg_qgemm_ex(t(64 * 64), t(64 * 4), 64, 256, t(8 * 256 * 2), 8, t(8 * 64 * 4), t(100), 128),
     "workspace"),
    (lambda t: q.pg_fwht_rotate(t(4 * 256 * 2), 1, t(4 * 256 * 4 - 1), 0, t(32), 4, 256), "y"),
    (lambda t: q.pg_decode(t(256 * 64, contiguous=False), t(256 * 4), 256, 256, t(256 * 256 * 4)), "codes"),
    (lambda t: q.pg_decode_table(t(256 * 64), t(256 * 4), 256, 256, t(8191), 0, t(256 * 256 * 4)), "table"),
    (lambda t: q.pg_rot_qgemv_table(t(64 * 64), t(64 * 4), 64, 256, t(256 * 2 - 2), 1, t(32), t(8192), 1,
                                    t(64 * 4)), "x"),
    (lambda t: q.pg_rot_qgemv_table(t(64 * 64), t(64 * 4), 64, 256, t(256 * 2), 1, t(32), t(8192), 1, t(63 * 4)),
     "y"),
])
def test_binding_checks_device_buffers_before_the_call(bad, what):
    """Undersized, non-contiguous or host buffers raise ValueError in the
    binding, before the library is called (so no kernel can run past a
    caller's buffer)."""
    with pytest.raises(ValueError, match=what):
        bad(_FakeDeviceTensor)


def test_binding_refuses_host_tensors_for_device_arguments():
    import torch
    with pytest.raises(ValueError, match="not on the GPU"):
        q.pg_decode(torch.zeros(64, dtype=torch.uint8), 1 << 20, 1, 256, 1 << 20)
    with pytest.raises(ValueError, match="numpy"):
        q.pg_decode(np.zeros(64, np.uint8), 1 << 20, 1, 256, 1 << 20)
