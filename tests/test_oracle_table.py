"""Pins of the oracle's table-driven codebook variant (CPU only): the code
byte of a group, read in trellis state s, names the 4-D point T[s][byte] of
a table of int8 levels.  The variant is one point of the small-state
coset-trellis design space named on the "Pingala-8" landing page, section
"Paper"; its trellis is the one of section "How it works" (format P8F v1).
Pinned to a worked example derived by hand (tests/golden/table_example.json),
to the closed-form v1 decode (on v1's own table), to byte- and
coordinate-permuted tables whose effect is known in closed form, to an
elementwise level map, and to the scalar walk that defines the decode."""
import json
import os

import numpy as np
import pytest

from oracle import p8f
from qgemv_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "table_example.json")


def _hand_table(ex):
    """The golden's table, built only from its stated rule on top of the v1
    table: T[s][c] = phi(v1(s, c ^ xor))."""
    v1 = p8f.codebook_table().astype(np.int64)
    phi = {int(a): b for a, b in ex["phi"].items()}
    t = np.empty((8, 256, 4), dtype=np.int8)
    for s in range(8):
        for c in range(256):
            t[s, c] = [phi[int(v)] for v in v1[s, c ^ ex["byte_xor"]]]
    return t


def _golden_codes(ex):
    codes = ex["codes_head"] + [ex["codes_tail_byte"]] * (32 - len(ex["codes_head"]))
    return np.array([codes], dtype=np.uint8)


def test_hand_example_levels():
    ex = json.load(open(GOLDEN))
    codes = _golden_codes(ex)
    want = ex["hand_levels_head"] + ex["hand_levels_tail_group"] * (32 - len(ex["codes_head"]))
    assert p8f.decode_levels_table(codes, _hand_table(ex))[0].tolist() == want
    assert p8f.decode_block_levels_table(codes[0], _hand_table(ex)) == want
    v1 = ex["v1_levels_head"] + ex["v1_levels_tail_group"] * (32 - len(ex["codes_head"]))
    assert p8f.decode_levels_table(codes, p8f.codebook_table())[0].tolist() == v1
    assert p8f.decode_levels(codes)[0].tolist() == v1


def test_hand_example_product():
    ex = json.load(open(GOLDEN))
    codes = _golden_codes(ex)
    scale = np.array([[np.float16(ex["scale"]).view(np.uint16)]], dtype=np.uint16)
    y = p8f.gemv_table_ref(codes, scale, _hand_table(ex), np.ones((1, 128)))
    assert y.shape == (1, 1) and y[0, 0] == ex["y_hand_ones"]


@pytest.mark.parametrize("carry", [False, True])
def test_v1_table_equals_closed_form(carry):
    """On v1's own table the table walk is the closed-form decode (which
    shares no code with it beyond the per-group rule that fills the table)."""
    rng = np.random.default_rng(71)
    codes = rng.integers(0, 256, (13, 96), dtype=np.uint8)
    t = p8f.codebook_table()
    assert np.array_equal(p8f.decode_levels_table(codes, t, carry), p8f.decode_levels(codes, carry))
    sc = synth.random_scale_bits(13, 384, 5)
    assert np.array_equal(p8f.decode_weights_table(codes, sc, t, carry), p8f.decode_weights(codes, sc, carry))
    x = rng.standard_normal((2, 384))
    assert np.allclose(p8f.gemv_table_ref(codes, sc, t, x, carry), p8f.gemv_ref(codes, sc, x, carry), rtol=1e-13,
                       atol=0)


@pytest.mark.parametrize("dist", ["uniform", "gauss"])
def test_vectorised_walk_equals_scalar_walk(dist):
    t = synth.random_codebook_table(3, dist)
    rng = np.random.default_rng(72)
    codes = rng.integers(0, 256, (7, 64), dtype=np.uint8)       # two blocks per row
    fast = p8f.decode_levels_table(codes, t)
    for r in range(7):
        want = p8f.decode_block_levels_table(codes[r, :32], t) + p8f.decode_block_levels_table(codes[r, 32:], t)
        assert fast[r].tolist() == want
    # with carry: one walk over the row
    fast_c = p8f.decode_levels_table(codes, t, carry=True)
    for r in range(7):
        assert fast_c[r].tolist() == p8f.decode_block_levels_table(codes[r], t)


def test_states_follow_the_scalar_trellis():
    rng = np.random.default_rng(73)
    codes = rng.integers(0, 256, (3, 64), dtype=np.uint8)
    st = p8f.trellis_states(codes)
    for r in range(3):
        for b in range(2):
            s = 0
            for j in range(32):
                assert st[r, 32 * b + j] == s
                s = p8f.next_state(s, int(codes[r, 32 * b + j]) & 1)


def _bitrev7(v):
    return int(f"{v:07b}"[::-1], 2)


def test_byte_permuted_table():
    """T'[s][c] = T_v1[s][pi(c)] for a permutation pi that keeps the branch
    bit: decoding c under T' is decoding pi(c) under v1 (same state path)."""
    pi = np.array([(c & 1) | (_bitrev7(c >> 1) << 1) for c in range(256)], dtype=np.uint8)
    assert sorted(pi.tolist()) == list(range(256)) and np.all((pi & 1) == np.arange(256) % 2)
    t = p8f.codebook_table()[:, pi, :]
    rng = np.random.default_rng(74)
    codes = rng.integers(0, 256, (9, 64), dtype=np.uint8)
    assert np.array_equal(p8f.decode_levels_table(codes, t), p8f.decode_levels(pi[codes]))


def test_coordinate_permuted_table_and_level_map():
    """Reversing the four coordinates of every point reverses each decoded
    group; an elementwise level map applies to every decoded level."""
    rng = np.random.default_rng(75)
    codes = rng.integers(0, 256, (5, 32), dtype=np.uint8)
    v1 = p8f.decode_levels(codes).reshape(5, 32, 4)
    t = p8f.codebook_table()
    rev = p8f.decode_levels_table(codes, t[:, :, ::-1]).reshape(5, 32, 4)
    assert np.array_equal(rev, v1[:, :, ::-1])
    lut = np.zeros(16, dtype=np.int8)
    lut[[0, 2, 4, 6, 8, 10, 12, 14]] = [-100, -41, -12, -2, 5, 17, 60, 127]   # level -7 + i -> lut[i]
    tm = lut[t.astype(np.int64) + 7]
    assert np.array_equal(p8f.decode_levels_table(codes, tm).reshape(5, 32, 4), lut[v1.astype(np.int64) + 7])


def test_table_product_brute_force():
    """Tiny product by plain loops over the scalar walk."""
    t = synth.random_codebook_table(9, "uniform")
    rng = np.random.default_rng(76)
    codes = rng.integers(0, 256, (3, 64), dtype=np.uint8)
    sc = synth.random_scale_bits(3, 256, 8)
    x = rng.standard_normal((2, 256))
    y = p8f.gemv_table_ref(codes, sc, t, x)
    for r in range(3):
        lv = p8f.decode_block_levels_table(codes[r, :32], t) + p8f.decode_block_levels_table(codes[r, 32:], t)
        s = [float(np.array([sc[r, j]], dtype=np.uint16).view(np.float16)[0]) for j in range(2)]
        for b in range(2):
            want = sum(s[i // 128] * lv[i] * x[b, i] for i in range(256))
            assert abs(y[b, r] - want) <= 1e-12 * max(1.0, abs(want))


def test_uniform_table_covers_int8_range():
    t = synth.random_codebook_table(1, "uniform")
    assert t.dtype == np.int8 and t.shape == (8, 256, 4)
    assert t.min() == -128 and t.max() == 127
    g = synth.random_codebook_table(1, "gauss")
    assert g.min() >= -127 and g.max() <= 127 and len(np.unique(g)) > 60


# ------------------------------------------------ encoder through a table
def _brute_min(w, sb, table, rate23):
    """Least distortion over all 65536 strings of a 2-group block."""
    sv = float(np.array([sb], dtype=np.uint16).view(np.float16)[0])
    t = np.asarray(table, dtype=np.float64)
    nxt = p8f.next_state_r23 if rate23 else p8f.next_state
    umask = 3 if rate23 else 1
    best = np.inf
    for c0 in range(256):
        d0 = w[:4] - sv * t[0, c0]
        s1 = nxt(0, c0 & umask)
        d1 = w[None, 4:] - sv * t[s1]                       # all second bytes at once
        tot = float(np.sum(d0 * d0)) + np.sum(d1 * d1, axis=1)
        best = min(best, float(np.min(tot)))
    return best


@pytest.mark.parametrize("rate23", [False, True])
@pytest.mark.parametrize("seed", range(3))
def test_table_encoder_equals_exhaustive_search(rate23, seed):
    rng = np.random.default_rng(200 + seed)
    t = synth.random_codebook_table(30 + seed, "gauss")
    w = rng.standard_normal(8) * 3.0
    sb = int(np.float16(0.21 + 0.05 * seed).view(np.uint16))
    codes = p8f.viterbi_encode_table(w[None, :], np.array([sb], np.uint16), t, rate23)
    got = p8f.block_distortion_table(w[None, :], codes, np.array([sb], np.uint16), t, rate23)[0]
    assert abs(got - _brute_min(w, sb, t, rate23)) <= 1e-9 * max(1.0, got)


def test_table_encoder_on_own_tables_is_the_plain_encoders():
    """P8F v1's table on its trellis gives viterbi_encode's codes, the
    rate-2/3 variant's table on its trellis viterbi_encode_r23's (same tie
    rules), including a zero-scale block."""
    rng = np.random.default_rng(210)
    w = rng.standard_normal((9, 128))
    w[4] = 0.0
    sb = p8f.block_scale_bits(w)
    assert np.array_equal(p8f.viterbi_encode_table(w, sb, p8f.codebook_table()), p8f.viterbi_encode(w, sb))
    assert np.array_equal(p8f.viterbi_encode_table(w, sb, p8f.codebook_table_r23(), True),
                          p8f.viterbi_encode_r23(w, sb))


def test_table_encoder_on_a_byte_permuted_table():
    """Permuting the bytes (branch bits kept) permutes the code book only:
    the least distortion is the same."""
    pi = np.array([(c & 1) | (_bitrev7(c >> 1) << 1) for c in range(256)], dtype=np.uint8)
    tp = p8f.codebook_table()[:, pi, :]
    rng = np.random.default_rng(211)
    w = rng.standard_normal((5, 128))
    sb = p8f.block_scale_bits(w)
    c0 = p8f.viterbi_encode(w, sb)
    cp = p8f.viterbi_encode_table(w, sb, tp)
    assert np.allclose(p8f.block_distortion_table(w, cp, sb, tp), p8f.block_distortion(w, c0, sb), rtol=1e-12)


def test_nonuniform_table_encoding_lowers_gaussian_mse():
    """Diagnostic (parity unpinned: the pages give no codebook values): on
    Gaussian weights a table whose eight levels follow the Gaussian's shape
    codes with less error than the uniform v1 levels at the same scale rule
    (scales from the usual rule, so both tables see the same scales)."""
    phi = {-7: -9, -5: -6, -3: -3, -1: -1, 1: 1, 3: 3, 5: 6, 7: 9}
    v1 = p8f.codebook_table()
    t = np.vectorize(lambda v: phi[int(v)])(v1).astype(np.int8)
    rng = np.random.default_rng(212)
    w = rng.standard_normal((24, 128))
    sb = p8f.block_scale_bits(w, c=0.29 * 7 / 9)
    e_t = np.mean(p8f.block_distortion_table(w, p8f.viterbi_encode_table(w, sb, t), sb, t))
    sb1 = p8f.block_scale_bits(w)
    e_1 = np.mean(p8f.block_distortion(w, p8f.viterbi_encode(w, sb1), sb1))
    assert 0 < e_t < e_1            # 12.56 against 13.58 on this seed


def test_table_encoder_tie_rules_on_the_hand_example():
    """The hand-derived tie example (tests/golden/viterbi_tie_example.json,
    T1: two paths of equal distortion, several equally near points) through
    P8F v1's table: the table encoder picks the codes derived by hand, so its
    predecessor, byte and end-state tie rules are viterbi_encode's."""
    ex = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "viterbi_tie_example.json")))["tie"]
    w = np.array([ex["w_rot"]], dtype=np.float64)
    sb = np.array([np.float16(ex["scale"]).view(np.uint16)], dtype=np.uint16)
    codes = p8f.viterbi_encode_table(w, sb, p8f.codebook_table())
    assert codes[0].tolist() == ex["codes"]
    # T2: equally near bytes within a coset, the smaller byte wins
    ex2 = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "viterbi_tie_example.json")))["tie_bytes"]
    w2 = np.array([ex2["w_rot"]], dtype=np.float64)
    sb2 = np.array([np.float16(ex2["scale"]).view(np.uint16)], dtype=np.uint16)
    assert p8f.viterbi_encode_table(w2, sb2, p8f.codebook_table())[0].tolist() == ex2["codes"]
    assert p8f.viterbi_encode(w2, sb2)[0].tolist() == ex2["codes"]
