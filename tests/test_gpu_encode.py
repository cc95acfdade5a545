"""GPU trellis encoder pg_encode: bit-identical codes and scales to the host
reference encoder pg_encode_ref (same fp64 steps in the same order), and the
same optimum as the oracle's Viterbi search (codes equal except on blocks the
two searches tie, where both reach the same distortion)."""
import numpy as np
import pytest

import qgemv_amd as q
from oracle import p8f
from qgemv_amd import synth
from tests.helpers import assert_codes_equivalent, dev, host

pytestmark = pytest.mark.gpu


def _gpu_encode(w, sb):
    import torch
    n, k = w.shape
    codes = torch.empty((n, k // 4), dtype=torch.uint8, device="cuda")
    scales = torch.empty((n, k // 128), dtype=torch.int16, device="cuda")
    q.pg_encode(dev(w), n, k, dev(sb), codes, scales)
    torch.cuda.synchronize()
    return host(codes), host(scales).view(np.uint16)


def _host_encode(w, sb):
    n, k = w.shape
    codes = np.zeros((n, k // 4), np.uint8)
    scales = np.zeros((n, k // 128), np.uint16)
    q.pg_encode_ref(np.ascontiguousarray(w), n, k, sb, codes, scales, 0)
    return codes, scales


def _weights(n, k, seed):
    """0.02 N(0,1) with 0.1% of the entries x20 (the layer recipe), fp32."""
    rng = np.random.default_rng(seed)
    w = 0.02 * rng.standard_normal((n, k), dtype=np.float32)
    idx = rng.choice(n * k, max(1, n * k // 1000), replace=False)
    w.reshape(-1)[idx] *= 20
    return w


@pytest.mark.parametrize("n,k", [(1, 128), (7, 640), (64, 2560), (300, 256), (33, 4096)])
def test_equals_host_reference(n, k):
    w = _weights(n, k, n + k)
    sb = np.random.default_rng(k).integers(0, 256, k // 8, dtype=np.uint8)
    gc, gs = _gpu_encode(w, sb)
    hc, hs = _host_encode(w, sb)
    assert np.array_equal(gs, hs)
    assert np.array_equal(gc, hc)


def test_equivalent_to_oracle():
    w = _weights(48, 1024, 3)
    sb = synth.site_sign_bits(0, 1, 1024)
    gc, gs = _gpu_encode(w, sb)
    oc, os_ = p8f.encode_matrix(w, sb)
    assert np.array_equal(gs, os_)
    assert_codes_equivalent(w, sb, gc, oc, gs)


def test_special_blocks():
    """Zero rows (zero scale, every byte 0), constant rows, exact zeros inside
    a block (tied branch metrics), tiny weights (subnormal fp16 scale) and
    huge ones (scale clamped to 65504)."""
    k = 512
    rng = np.random.default_rng(11)
    w = np.zeros((6, k), np.float32)
    w[1, :] = 0.5
    w[2] = 0.02 * rng.standard_normal(k).astype(np.float32)
    w[2, ::3] = 0.0
    w[3] = 1e-5 * rng.standard_normal(k).astype(np.float32)
    w[4] = 1e6 * rng.standard_normal(k).astype(np.float32)
    w[5, 128:256] = 0.25                                   # one constant block among zero blocks
    sb = rng.integers(0, 256, k // 8, dtype=np.uint8)
    gc, gs = _gpu_encode(w, sb)
    hc, hs = _host_encode(w, sb)
    assert np.array_equal(gs, hs) and np.array_equal(gc, hc)
    assert not gc[0].any() and not gs[0].any()
    assert gs[4].max() == 0x7BFF                           # 65504
    assert (gs[3] < 0x0400).all() and gs[3].any()          # subnormal scales
    oc, os_ = p8f.encode_matrix(w, sb)
    assert np.array_equal(gs, os_)
    assert_codes_equivalent(w, sb, gc, oc, gs)


def test_full_matrix_sampled_rows():
    """A whole Qwen3-4B-shaped q matrix (4096 x 2560) on the GPU; 48 sampled
    rows against the host reference."""
    w = synth.qwen_layer_weights("q")
    n, k = w.shape
    sb = synth.site_sign_bits(0, synth.SITE_OF["q"], k)
    gc, gs = _gpu_encode(w, sb)
    rows = np.sort(np.random.default_rng(2).choice(n, 48, replace=False))
    hc, hs = _host_encode(np.ascontiguousarray(w[rows]), sb)
    assert np.array_equal(gs[rows], hs)
    assert np.array_equal(gc[rows], hc)


def test_decode_of_gpu_codes_is_the_oracle_decode():
    w = _weights(16, 768, 9)
    sb = np.random.default_rng(4).integers(0, 256, 96, dtype=np.uint8)
    gc, gs = _gpu_encode(w, sb)
    import torch
    out = torch.empty((16, 768), dtype=torch.float32, device="cuda")
    q.pg_decode(dev(gc), dev(gs.view(np.int16)), 16, 768, out)
    torch.cuda.synchronize()
    assert np.array_equal(host(out).astype(np.float64), p8f.decode_weights(gc, gs))
