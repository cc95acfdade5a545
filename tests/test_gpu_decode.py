"""GPU parity of pg_decode against the oracle: bit-exact (uint32 views,
signed zeros included), on the encoded single layer, on Qwen3-4B-shaped
matrices and on random blocks with edge-case scales."""
import numpy as np
import pytest

import qgemv_amd as q
from oracle import p8f
from tests.helpers import dev, encoded_qwen, encoded_single, host

pytestmark = pytest.mark.gpu


def _decode_gpu(codes, scales):
    import torch
    n, kg = codes.shape
    k = 4 * kg
    w = torch.empty((n, k), dtype=torch.float32, device="cuda")
    q.pg_decode(dev(codes), dev(scales), n, k, w)
    torch.cuda.synchronize()
    return host(w)


def _assert_bit_exact(codes, scales):
    got = _decode_gpu(codes, scales)
    want = p8f.decode_weights(codes, scales).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_decode_single_layer_bit_exact():
    codes, scales = encoded_single()
    _assert_bit_exact(codes, scales)


def test_decode_random_blocks_edge_scales():
    rng = np.random.default_rng(100)
    codes = rng.integers(0, 256, (37, 96), dtype=np.uint8)          # ragged n, 3 blocks per row
    scales = rng.integers(0, 0x7C00, (37, 3)).astype(np.uint16)     # finite fp16 incl. subnormals
    scales[0, 0] = 0x0000        # +0 scale: signed zeros from negative levels
    scales[1, 1] = 0x8000        # -0 scale
    scales[2, 2] = 0x0001        # smallest subnormal
    scales[3, 0] = 0x7BFF        # largest finite
    scales[4, 1] = 0xC000        # negative scale (-2): still exact
    _assert_bit_exact(codes, scales)


@pytest.mark.parametrize("name", ["k", "o", "down"])
def test_decode_qwen_matrices_bit_exact(name):
    codes, scales = encoded_qwen(name)
    _assert_bit_exact(codes, scales)


def test_decode_one_row_one_block():
    codes = np.array([[0x5A, 0x3C, 0x81, 0x07] + [0] * 28], dtype=np.uint8)
    scales = np.array([[np.float16(0.5).view(np.uint16)]], dtype=np.uint16)
    got = _decode_gpu(codes, scales)[0, :16]
    assert got.tolist() == [2.5, -3.5, 2.5, -3.5, 0.5, 2.5, -1.5, -3.5, -3.5, -3.5, -3.5, 2.5,
                            -1.5, -1.5, -3.5, -3.5]
