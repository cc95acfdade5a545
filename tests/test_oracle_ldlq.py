"""Pins of the oracle's LDLQ encoder with a proxy Hessian (CPU only).  The
"Pingala-8" landing page, section "How it works", names LDLQ as the
compressor's rounding: each coded unit's error is passed on through the
Hessian to the units not yet coded.  Here the unit is the 128-block of the
trellis.  Pinned to: the factorisation's definition (U D U^T = H, shapes of
U and D); H = I, diagonal and block-diagonal Hessians reducing to the plain
encoder; the loss identity that defines LDLQ's feedback (the proxy loss
equals the sum of the blocks' own D-weighted rounding errors); exhaustive
search over every byte string of tiny blocks with the feedback rule; the
rotated Hessian against explicit rotation matrices."""
import numpy as np
import pytest

from oracle import p8f


def _spd(k, seed, ridge=0.05):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((k, 2 * k))
    # correlated inputs: a random mixing plus a smooth neighbour coupling
    a[1:] += 0.8 * a[:-1]
    return a @ a.T / (2 * k) + ridge * np.eye(k)


@pytest.mark.parametrize("k,block", [(384, 128), (24, 8), (40, 4)])
def test_block_udu_definition(k, block):
    h = _spd(k, k)
    u, d = p8f.block_udu(h, block)
    assert np.allclose(u @ d @ u.T, h, rtol=0, atol=1e-11 * np.abs(h).max())
    nb = k // block
    for i in range(nb):
        for j in range(nb):
            ub = u[i * block:(i + 1) * block, j * block:(j + 1) * block]
            db = d[i * block:(i + 1) * block, j * block:(j + 1) * block]
            if i == j:
                assert np.array_equal(ub, np.eye(block))
                assert np.all(np.linalg.eigvalsh(db) > 0)
            else:
                assert not np.any(db)
                if i > j:
                    assert not np.any(ub)


def test_block_udu_refuses_an_indefinite_matrix():
    h = _spd(16, 1)
    h[12:, 12:] = -np.eye(4)
    with pytest.raises(np.linalg.LinAlgError):
        p8f.block_udu(h, 4)


def test_rotated_hessian_is_r_h_rt():
    rng = np.random.default_rng(3)
    k = 256
    sb = rng.integers(0, 256, k // 8, dtype=np.uint8)
    h = _spd(k, 4)
    sig = p8f.signs_from_bits(sb, k)
    r = np.zeros((k, k))
    for b in range(2):
        r[b * 128:(b + 1) * 128, b * 128:(b + 1) * 128] = p8f.rotation_block_matrix(sig[b * 128:(b + 1) * 128])
    assert np.allclose(p8f.rotate_hessian(h, sb), r @ h @ r.T, atol=1e-12)


@pytest.mark.parametrize("kind", ["identity", "diagonal", "block_diagonal"])
def test_hessians_without_cross_block_terms_give_the_plain_encoder(kind):
    """U = I when H~ has no cross-block terms: the feedback vanishes and the
    codes are the plain encoder's, bit for bit (a diagonal or block-diagonal
    H stays block-diagonal under the block rotation)."""
    rng = np.random.default_rng(5)
    n, k = 6, 512
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    sb = rng.integers(0, 256, k // 8, dtype=np.uint8)
    if kind == "identity":
        h = np.eye(k)
    elif kind == "diagonal":
        h = np.diag(rng.uniform(0.1, 3.0, k))
    else:
        h = np.zeros((k, k))
        for b in range(k // 128):
            h[b * 128:(b + 1) * 128, b * 128:(b + 1) * 128] = _spd(128, 10 + b)
    c1, s1 = p8f.encode_matrix_ldlq(w, sb, h)
    c0, s0 = p8f.encode_matrix(w, sb)
    assert np.array_equal(c1, c0) and np.array_equal(s1, s0)


@pytest.mark.parametrize("k,block,seed", [(384, 128, 1), (32, 8, 2)])
def test_proxy_loss_equals_sum_of_block_rounding_losses(k, block, seed):
    """With E = What - W~ and eta the blocks' own rounding errors,
    tr(E H~ E^T) = sum_j tr(eta_j D_j eta_j^T): the identity LDLQ's feedback
    is built for.  A wrong sign, a transposed factor or feedback from the
    wrong blocks breaks it."""
    rng = np.random.default_rng(seed)
    n = 5
    w = rng.standard_normal((n, k))
    h = _spd(k, seed + 20)
    codes, scales, eta = p8f.ldlq_encode_rotated(w, h, block)
    nb, g = k // block, block // 4
    what = np.zeros((n, k))
    for r in range(n):
        for j in range(nb):
            lv = p8f.decode_block_levels(codes[r, j * g:(j + 1) * g])
            what[r, j * block:(j + 1) * block] = p8f.fp16_bits_to_float(scales[r, j:j + 1])[0] * np.array(lv)
    _, d = p8f.block_udu(h, block)
    right = sum(float(np.sum((eta[:, j * block:(j + 1) * block] @ d[j * block:(j + 1) * block,
                                                                   j * block:(j + 1) * block])
                             * eta[:, j * block:(j + 1) * block])) for j in range(nb))
    left = p8f.proxy_loss(w, what, h)
    assert abs(left - right) <= 1e-9 * abs(left)


def test_exhaustive_search_with_the_feedback_rule_tiny_blocks():
    """Blocks of 2 groups (8 weights), three blocks per row, a synthetic SPD
    Hessian: block by block, the target from the feedback of the errors
    chosen so far (summed in increasing column order), its scale by the rule,
    then the best of all 65536 byte strings; the LDLQ encoder must pick the
    same strings."""
    rng = np.random.default_rng(11)
    n, k, block = 3, 24, 8
    w = rng.standard_normal((n, k))
    h = _spd(k, 12)
    codes, scales, _ = p8f.ldlq_encode_rotated(w, h, block)
    u, _ = p8f.block_udu(h, block)
    for r in range(n):
        err = np.zeros(k)
        for j in range(k // block):
            acc = np.zeros(block)
            for cp in range(j * block):
                acc = acc + err[cp] * u[cp, j * block:(j + 1) * block]
            t = w[r, j * block:(j + 1) * block] + acc
            sb = int(p8f.block_scale_bits(t[None, :])[0])
            assert sb == scales[r, j]
            dist, best = p8f.exhaustive_encode_bytes(t, sb)
            assert best == codes[r, 2 * j:2 * j + 2].tolist()
            lv = np.array(p8f.decode_block_levels(best), dtype=np.float64)
            err[j * block:(j + 1) * block] = w[r, j * block:(j + 1) * block] - \
                p8f.fp16_bits_to_float(np.array([sb], dtype=np.uint16))[0] * lv


def test_ldlq_lowers_the_proxy_loss_on_correlated_inputs():
    """Inputs that live near a 16-dimensional subspace (a low-rank Hessian
    plus a small ridge, the shape of real layer inputs): the feedback steers
    the errors out of that subspace and the proxy loss drops well below the
    plain encoder's (about 4x on this seed)."""
    rng = np.random.default_rng(13)
    n, k = 16, 512
    w = rng.standard_normal((n, k))
    a = rng.standard_normal((k, 16))
    h = a @ a.T / 16 + 0.01 * np.eye(k)
    c1, s1, _ = p8f.ldlq_encode_rotated(w, h)
    sb0 = p8f.block_scale_bits(w.reshape(-1, 128)).reshape(n, k // 128)
    c0 = p8f.viterbi_encode(w.reshape(-1, 128), sb0.reshape(-1)).reshape(n, k // 4)

    def what(c, s):
        return p8f.decode_weights(c, s)
    assert p8f.proxy_loss(w, what(c1, s1), h) < 0.5 * p8f.proxy_loss(w, what(c0, sb0), h)
