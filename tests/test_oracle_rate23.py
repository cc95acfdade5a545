"""Pins of the oracle's rate-2/3 trellis variant (CPU only): two branch bits
per group, four branches per state, 8 cosets of 64 points of the same
512-point set as P8F v1, labelled along the set-partition chain value set /
D4 parity / RZ4 split.  The variant follows the "Pingala-8" landing page,
sections "Where the name comes from" (eight states over short patterns,
Ungerboeck-style labels) and "Paper" (small-state coset trellis).  Pinned to
a worked example derived by hand (tests/golden/rate23_example.json), to the
partition's closed-form structure, to Ungerboeck's labelling rules checked
by enumeration, to a path-validity check, and to exhaustive search: over
every byte string of 2-group blocks, and over every branch path (with the
nearest point of each coset by brute force) of blocks up to 6 groups."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import p8f

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rate23_example.json")


def test_hand_example():
    ex = json.load(open(GOLDEN))
    codes = ex["codes_head"] + [ex["codes_tail_byte"]] * (32 - len(ex["codes_head"]))
    want = ex["levels_head"] + ex["levels_tail_group"] * (32 - len(ex["codes_head"]))
    assert p8f.decode_block_levels_r23(codes) == want
    s, states = 0, []
    for c in codes[:8]:
        states.append(s)
        s = p8f.next_state_r23(s, c & 3)
    assert states == ex["states_head"]


def _all_points():
    return [tuple(v) for v in itertools.product((-7, -3, 1, 5), repeat=4)] + \
           [tuple(v) for v in itertools.product((-5, -1, 3, 7), repeat=4)]


def test_cosets_partition_the_512_points_into_8_of_64():
    pts = _all_points()
    assert len(set(pts)) == 512
    by = {}
    for p in pts:
        by.setdefault(p8f.coset_of_levels(p), []).append(p)
    assert sorted(by) == [(a, b, c) for a in range(2) for b in range(2) for c in range(2)]
    assert all(len(v) == 64 for v in by.values())


def _d2(a, b):
    return sum((x - y) ** 2 for x, y in zip(a, b))


def test_partition_chain_distances():
    """Minimum squared distance inside each level of the chain (levels in
    units of the scale): the whole set 16, a value set 16, a D4 coset 32, an
    RZ4 coset 32 (RZ4 has D4's minimum norm: the split keeps it)."""
    pts = _all_points()

    def mind(group):
        return min(_d2(a, b) for a, b in itertools.combinations(group, 2))
    assert mind(pts) == 16
    for key_len, want in ((1, 16), (2, 32), (3, 32)):
        by = {}
        for p in pts:
            by.setdefault(p8f.coset_of_levels(p)[:key_len], []).append(p)
        assert all(mind(v) == want for v in by.values()), key_len


def test_every_byte_decodes_into_its_branch_coset_bijectively():
    for s in range(8):
        seen = set()
        for c in range(256):
            lv = tuple(p8f.decode_group_r23(c, s))
            assert p8f.coset_of_levels(lv) == p8f.coset_r23(s, c & 3)
            seen.add(lv)
        # the 256 bytes name the 256 points of the state's value set
        assert len(seen) == 256 and {p8f.coset_of_levels(p)[0] for p in seen} == {s & 1}


def test_ungerboeck_labelling_rules():
    """Branches leaving a state and branches entering a state carry the four
    distinct cosets of one value set; no parallel branches."""
    for s in range(8):
        out = [p8f.coset_r23(s, u) for u in range(4)]
        assert len(set(out)) == 4 and len({z[0] for z in out}) == 1
        assert len({p8f.next_state_r23(s, u) for u in range(4)}) == 4
    for sn in range(8):
        inc = [(s, u) for s in range(8) for u in range(4) if p8f.next_state_r23(s, u) == sn]
        assert len(inc) == 4
        zs = [p8f.coset_r23(s, u) for s, u in inc]
        assert len(set(zs)) == 4 and len({z[0] for z in zs}) == 1


def test_decoded_paths_are_valid_and_corruption_is_caught():
    rng = np.random.default_rng(81)
    for _ in range(20):
        codes = rng.integers(0, 256, 32)
        lv = p8f.decode_block_levels_r23(codes)
        assert p8f.levels_trellis_valid_r23(lv)
    # the first group is read in state 0: value set A0 only, A1 is no branch of it
    lv = p8f.decode_block_levels_r23([0] * 32)
    bad = list(lv)
    bad[0:4] = [-5, -5, -5, -5]
    assert not p8f.levels_trellis_valid_r23(bad)
    # a point whose coset no branch of the current state carries
    lv = p8f.decode_block_levels_r23([1] + [0] * 31)       # state 1 after group 0: value set A1
    bad = list(lv)
    bad[4:8] = [-7, -7, -7, -7]
    assert not p8f.levels_trellis_valid_r23(bad)


def _scale_bits(v):
    return int(np.float16(v).view(np.uint16))


@pytest.mark.parametrize("seed", range(4))
def test_viterbi_equals_exhaustive_byte_search_two_groups(seed):
    rng = np.random.default_rng(90 + seed)
    w = rng.standard_normal(8)
    sb = _scale_bits(0.25 + 0.1 * seed)
    codes = p8f.viterbi_encode_r23(w[None, :], np.array([sb], dtype=np.uint16))
    got = p8f.block_distortion_r23(w[None, :], codes, np.array([sb], dtype=np.uint16))[0]
    assert abs(got - p8f.exhaustive_encode_r23(w, sb)) <= 1e-12


def _path_search(w, sb):
    """Every branch path of the block; per group the nearest point of the
    path's coset by brute force over all 256 bytes of the branch."""
    g = w.shape[0] // 4
    sv = float(np.array([sb], dtype=np.uint16).view(np.float16)[0])
    best = np.inf
    for path in itertools.product(range(4), repeat=g):
        s, tot = 0, 0.0
        for t, u in enumerate(path):
            dmin = min(_d2(w[4 * t:4 * t + 4], [sv * v for v in p8f.decode_group_r23((hi << 2) | u, s)])
                       for hi in range(64))
            tot += dmin
            s = p8f.next_state_r23(s, u)
        best = min(best, tot)
    return best


@pytest.mark.parametrize("g,seed", [(3, 1), (4, 2), (5, 3), (6, 4)])
def test_viterbi_equals_exhaustive_path_search(g, seed):
    rng = np.random.default_rng(100 + seed)
    w = rng.standard_normal(4 * g) * 1.3
    sb = _scale_bits(0.3)
    codes = p8f.viterbi_encode_r23(w[None, :], np.array([sb], dtype=np.uint16))
    got = p8f.block_distortion_r23(w[None, :], codes, np.array([sb], dtype=np.uint16))[0]
    assert abs(got - _path_search(w, sb)) <= 1e-9


def test_zero_scale_block_codes_zero_bytes():
    w = np.ones((1, 128))
    assert np.all(p8f.viterbi_encode_r23(w, np.array([0], dtype=np.uint16)) == 0)


def test_full_block_viterbi_beats_greedy():
    """On a real 128-weight block the Viterbi's distortion is no worse than
    the greedy path (nearest point group by group along its own states)."""
    rng = np.random.default_rng(7)
    w = rng.standard_normal((1, 128))
    sb = np.array([_scale_bits(0.29)], dtype=np.uint16)
    sv = float(sb.view(np.float16)[0])
    codes = p8f.viterbi_encode_r23(w, sb)
    vit = p8f.block_distortion_r23(w, codes, sb)[0]
    s, greedy = 0, []
    for t in range(32):
        best = min(range(256), key=lambda c: _d2(w[0, 4 * t:4 * t + 4], [sv * v for v in p8f.decode_group_r23(c, s)]))
        greedy.append(best)
        s = p8f.next_state_r23(s, best & 3)
    assert vit <= p8f.block_distortion_r23(w, np.array([greedy], dtype=np.uint8), sb)[0] + 1e-12
    assert p8f.levels_trellis_valid_r23(p8f.decode_block_levels_r23(codes[0]))


@pytest.mark.parametrize("carry", [False, True])
def test_table_decode_with_rate23_states_equals_the_scalar_walk(carry):
    """The rate-2/3 variant through the table decode: its own table with the
    rate-2/3 state rule equals the defining scalar walk (per block, or along
    the row with carried state); a random table follows the same states."""
    rng = np.random.default_rng(111)
    codes = rng.integers(0, 256, (6, 96), dtype=np.uint8)            # three blocks per row
    got = p8f.decode_levels_table(codes, p8f.codebook_table_r23(), carry=carry, rate23=True)
    for r in range(6):
        if carry:
            want = p8f.decode_block_levels_r23(codes[r])
        else:
            want = sum((p8f.decode_block_levels_r23(codes[r, 32 * b:32 * b + 32]) for b in range(3)), [])
        assert got[r].tolist() == want
    t = rng.integers(-128, 128, (8, 256, 4)).astype(np.int8)
    st = p8f.trellis_states(codes, carry, rate23=True)
    for r in range(2):
        s = 0
        for j in range(96):
            if j % 32 == 0 and not carry:
                s = 0
            assert st[r, j] == s
            s = p8f.next_state_r23(s, int(codes[r, j]) & 3)
    assert np.array_equal(p8f.decode_levels_table(codes, t, carry, True).reshape(6, 96, 4), t[st, codes])
