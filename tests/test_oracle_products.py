"""Pins of the oracle's fp64 products and activation helpers (CPU only).

Batch-1 generation reads the weights once per token and forms y = W~ x~
(article "8 open models...", section "What 2-bit keeps").  Pinned to: a
one-hot input returning one decoded column exactly, zero input, linearity,
a pure-Python triple loop on a tiny case, and closed forms of the RMS
normalisation."""
import numpy as np

from oracle import p8f


def _tiny(seed=0, n=3, k=256, b=2):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, (n, k // 4), dtype=np.uint8)
    scales = np.random.default_rng(seed + 1).uniform(0.01, 2.0, (n, k // 128)).astype(np.float16).view(np.uint16)
    x = rng.standard_normal((b, k))
    return codes, scales, x


def test_one_hot_returns_decoded_column_exactly():
    codes, scales, _ = _tiny()
    w = p8f.decode_weights(codes, scales)
    for k in (0, 1, 127, 128, 255):
        e = np.zeros((1, 256))
        e[0, k] = 1.0
        assert np.array_equal(p8f.gemv_ref(codes, scales, e)[0], w[:, k])


def test_zero_input_and_linearity():
    codes, scales, x = _tiny(1)
    assert not p8f.gemv_ref(codes, scales, np.zeros((1, 256))).any()
    y1 = p8f.gemv_ref(codes, scales, x[:1])
    y2 = p8f.gemv_ref(codes, scales, x[1:])
    y12 = p8f.gemv_ref(codes, scales, 2.0 * x[:1] - 0.5 * x[1:])
    assert np.allclose(y12, 2.0 * y1 - 0.5 * y2, rtol=1e-13, atol=1e-13)


def test_triple_loop_on_tiny_case():
    codes, scales, x = _tiny(2, n=2, k=256, b=2)
    y = p8f.gemv_ref(codes, scales, x)
    for m in range(2):
        for n in range(2):
            acc = 0.0
            for blk in range(2):
                s = float(np.array([scales[n, blk]], dtype=np.uint16).view(np.float16)[0])
                lv = p8f.decode_block_levels(codes[n, 32 * blk:32 * blk + 32])
                part = 0.0
                for i in range(128):
                    part += lv[i] * x[m, 128 * blk + i]
                acc += s * part
            assert abs(acc - y[m, n]) <= 1e-12 * max(1.0, abs(acc))


def test_gemm_equals_gemv_per_row():
    codes, scales, x = _tiny(3, n=5, k=384, b=4)
    y = p8f.gemm_ref(codes, scales, x)
    for m in range(4):
        assert np.allclose(y[m], p8f.gemv_ref(codes, scales, x[m:m + 1])[0], rtol=0, atol=1e-12)


def test_rmsnorm16_closed_forms():
    v = np.full((1, 256), 3.0)
    out = p8f.rmsnorm16(v)
    assert np.all(out == np.float16(3.0 / np.sqrt(9.0 + 1e-6)))
    rng = np.random.default_rng(5)
    v = rng.standard_normal((2, 512)) * 40.0
    out = p8f.rmsnorm16(v)
    assert np.allclose(np.sqrt(np.mean(out ** 2, axis=1)), 1.0, atol=2e-3)
    assert np.array_equal(out, out.astype(np.float16).astype(np.float64))


def test_rmsnorm16_eps_hand_examples():
    """N1, N2: constant rows small enough that eps (1e-6) decides the fp16
    result (values derived by hand in the fixture)."""
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "viterbi_tie_example.json")) as f:
        cases = json.load(f)["rmsnorm"]
    for c in cases:
        out = p8f.rmsnorm16(np.full((1, c["length"]), c["value"]))
        assert np.all(out == c["out"]), (c["id"], out[0, 0])


def test_bf16_rounding_helper():
    vals = np.array([1.0, 1.00390625, 1.005859375, -2.5, 3.0e-3], dtype=np.float32)
    bits = p8f.bf16_rne_bits(vals)
    back = p8f.bf16_bits_to_float(bits)
    # bf16 keeps 8 significant bits; ties go to even
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == 1.0078125 and back[3] == -2.5
    # within half a bf16 ulp: 2^(floor(log2 x) - 8)
    x = float(vals[4])
    assert abs(back[4] - x) <= 2.0 ** (np.floor(np.log2(x)) - 8)
