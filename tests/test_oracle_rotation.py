"""Pins of the oracle's random-sign Hadamard rotation (CPU only).

The pages say a random Hadamard rotation spreads large weights before coding
("Pingala-8" landing page, section "How it works"); the activations get the
same rotation at run time so that W~ x~ = W x.  Pinned to: orthogonality,
norm preservation, an independent fast Walsh-Hadamard transform written here,
the closed form for unit vectors, and the product identity."""
import numpy as np

from oracle import p8f


def fwht_inplace(v):
    """Iterative butterflies (an algorithm independent of the oracle's
    explicit matrix), natural (Sylvester) order, unnormalised."""
    v = v.copy()
    h = 1
    n = v.shape[-1]
    while h < n:
        for i in range(0, n, 2 * h):
            a = v[..., i:i + h].copy()
            b = v[..., i + h:i + 2 * h].copy()
            v[..., i:i + h] = a + b
            v[..., i + h:i + 2 * h] = a - b
        h *= 2
    return v


def test_hadamard_is_orthogonal():
    h = p8f.sylvester_hadamard(128)
    assert np.array_equal(h @ h.T, 128 * np.eye(128))
    assert np.array_equal(h, h.T)
    rng = np.random.default_rng(1)
    r = p8f.rotation_block_matrix(np.where(rng.integers(0, 2, 128) == 1, -1.0, 1.0))
    assert np.max(np.abs(r @ r.T - np.eye(128))) <= 1e-15


def test_unit_vector_closed_form(golden):
    c = golden["hadamard_unit"]["value_2_pow_minus_3_5"]
    assert 2.0 ** -3.5 == c
    signs = np.zeros(16, dtype=np.uint8)                  # sigma = +1
    for j in (0, 1, 77, 127):
        x = np.zeros((1, 128))
        x[0, j] = 1.0
        y = p8f.rotate(x, signs)[0]
        want = np.array([(-1) ** bin(i & j).count("1") * c for i in range(128)])
        assert np.array_equal(y, want)


def test_rotation_equals_fwht_of_signed_input():
    rng = np.random.default_rng(2)
    k = 512
    sb = rng.integers(0, 256, k // 8, dtype=np.uint8)
    x = rng.standard_normal((3, k))
    sig = np.array([-1.0 if (sb[i >> 3] >> (i & 7)) & 1 else 1.0 for i in range(k)])
    want = np.concatenate([fwht_inplace((x * sig)[:, b * 128:(b + 1) * 128]) for b in range(k // 128)], axis=1)
    want *= 2.0 ** -3.5
    got = p8f.rotate(x, sb)
    assert np.max(np.abs(got - want)) <= 1e-13


def test_norm_preserved_and_inverse():
    rng = np.random.default_rng(3)
    k = 1024
    sb = rng.integers(0, 256, k // 8, dtype=np.uint8)
    x = rng.standard_normal((4, k))
    y = p8f.rotate(x, sb)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)
    # R^T R x = x, with R^T applied block by block from the explicit matrix
    sig = p8f.signs_from_bits(sb, k)
    back = np.empty_like(y)
    for b in range(k // 128):
        r = p8f.rotation_block_matrix(sig[b * 128:(b + 1) * 128])
        back[:, b * 128:(b + 1) * 128] = y[:, b * 128:(b + 1) * 128] @ r
    assert np.max(np.abs(back - x)) <= 1e-13


def test_sign_bit_packing():
    sb = np.array([0b00000101, 0b10000000], dtype=np.uint8)
    sig = p8f.signs_from_bits(sb, 16)
    assert sig.tolist() == [-1, 1, -1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, -1]


def test_rotation_convention_product_identity():
    # decoded W~hat times (R x) equals (W~hat R) times x, and coding error
    # is the same measured in either domain (Parseval)
    rng = np.random.default_rng(4)
    n, k = 16, 256
    sb = rng.integers(0, 256, k // 8, dtype=np.uint8)
    w = rng.standard_normal((n, k)).astype(np.float32)
    codes, scales = p8f.encode_matrix(w, sb)
    what_rot = p8f.decode_weights(codes, scales)          # rotated domain
    sig = p8f.signs_from_bits(sb, k)
    rfull = np.zeros((k, k))
    for b in range(k // 128):
        rfull[b * 128:(b + 1) * 128, b * 128:(b + 1) * 128] = p8f.rotation_block_matrix(sig[b * 128:(b + 1) * 128])
    x = rng.standard_normal(k)
    lhs = what_rot @ p8f.rotate(x[None], sb)[0]
    rhs = (what_rot @ rfull) @ x
    assert np.max(np.abs(lhs - rhs)) <= 1e-12 * np.max(np.abs(rhs))
    wt = p8f.rotate(w.astype(np.float64), sb)
    e_orig = np.linalg.norm(w - what_rot @ rfull)
    e_rot = np.linalg.norm(wt - what_rot)
    assert abs(e_orig - e_rot) <= 1e-12 * e_rot
