"""Pins of the oracle's carried-state variant (CPU only): the trellis state
runs on from block to block along a row.  The variant is one point of the
small-state coset-trellis design space named on the "Pingala-8" landing
page, section "Paper"; its decoding rule per group is the one of section
"How it works" (format P8F v1).  Pinned to a worked example derived by hand
(tests/golden/carry_example.json), the scalar walk that defines the variant,
the v1 decode restarted from the carried state, and exhaustive search over
all branch paths of short rows."""
import json
import os

import numpy as np
import pytest

from oracle import p8f

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "carry_example.json")


def _rel(a, b):
    return abs(a - b) / max(abs(b), 1e-300)


def test_worked_example_e5():
    ex = json.load(open(GOLDEN))["carry"][0]
    codes = np.array([ex["codes_block0"] + ex["codes_block1"]], dtype=np.uint8)
    lv = p8f.decode_levels(codes, carry=True)[0]
    assert lv[128:144].reshape(4, 4).tolist() == ex["block1_first_groups"]
    assert p8f.decode_row_levels_carry(codes[0])[128:144] == sum(ex["block1_first_groups"], [])
    assert p8f.decode_levels(codes)[0][128:144].reshape(4, 4).tolist() == ex["block1_first_groups_v1"]


def test_vectorised_carry_decode_equals_scalar_walk():
    rng = np.random.default_rng(61)
    codes = rng.integers(0, 256, (9, 96), dtype=np.uint8)          # 3 blocks per row
    fast = p8f.decode_levels(codes, carry=True)
    for r in range(9):
        assert fast[r].tolist() == p8f.decode_row_levels_carry(codes[r])


def test_block_decodes_as_v1_from_the_carried_state():
    """Block b is the v1 walk started in the state the last three branch
    bits of block b - 1 give (newest bit at bit 0)."""
    rng = np.random.default_rng(62)
    codes = rng.integers(0, 256, (5, 128), dtype=np.uint8)         # 4 blocks per row
    lv = p8f.decode_levels(codes, carry=True)
    for r in range(5):
        for b in range(1, 4):
            prev = codes[r, 32 * b - 3:32 * b] & 1
            s = int(prev[2]) | (int(prev[1]) << 1) | (int(prev[0]) << 2)
            walk = []
            for byte in codes[r, 32 * b:32 * b + 32]:
                walk.extend(p8f.decode_group(int(byte), s))
                s = p8f.next_state(s, int(byte) & 1)
            assert lv[r, 128 * b:128 * b + 128].tolist() == walk


def test_one_block_rows_equal_v1():
    rng = np.random.default_rng(63)
    codes = rng.integers(0, 256, (6, 32), dtype=np.uint8)
    assert np.array_equal(p8f.decode_levels(codes, carry=True), p8f.decode_levels(codes))
    w = rng.standard_normal((6, 128))
    sb = p8f.block_scale_bits(w)
    for r in range(6):
        a = p8f.viterbi_encode_row_carry(w[r:r + 1], sb[r:r + 1])
        assert np.array_equal(a, p8f.viterbi_encode(w[r:r + 1], sb[r:r + 1]))


@pytest.mark.parametrize("nb,g", [(2, 3), (2, 5), (2, 6), (3, 4)])
def test_carry_viterbi_equals_exhaustive_path_search(nb, g):
    rng = np.random.default_rng(70 + 10 * nb + g)
    for _ in range(3):
        w = rng.standard_normal((nb, 4 * g)) * rng.uniform(0.3, 3.0, (nb, 1))
        sb = p8f.block_scale_bits(w)
        codes = p8f.viterbi_encode_row_carry(w, sb)
        dist = p8f.row_distortion_carry(w, codes, sb)
        assert _rel(dist, p8f.exhaustive_encode_paths_carry(w, sb)) <= 1e-12


def test_zero_scale_block_is_zero_bytes_and_resets_the_state():
    rng = np.random.default_rng(64)
    w = rng.standard_normal((3, 128))
    w[1] = 0.0
    sb = p8f.block_scale_bits(w)
    assert sb[1] == 0
    codes = p8f.viterbi_encode_row_carry(w, sb)
    assert not codes[1].any()
    # the state entering block 2 is 0, so block 2 decodes as in v1
    lv = p8f.decode_levels(codes.reshape(1, -1), carry=True)[0]
    assert lv[256:384].tolist() == p8f.decode_block_levels(codes[2])


def test_encode_matrix_carry_layout():
    rng = np.random.default_rng(65)
    w = rng.standard_normal((3, 256)).astype(np.float32)
    sb = rng.integers(0, 256, 32, dtype=np.uint8)
    codes, scales = p8f.encode_matrix_carry(w, sb)
    wr = p8f.rotate(w.astype(np.float64), sb).reshape(3, 2, 128)
    assert np.array_equal(scales, p8f.block_scale_bits(wr.reshape(-1, 128)).reshape(3, 2))
    for r in range(3):
        assert np.array_equal(codes[r].reshape(2, 32), p8f.viterbi_encode_row_carry(wr[r], scales[r]))
