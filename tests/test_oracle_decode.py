"""Pins of the oracle's trellis decoder (CPU only).

Pinned to: hand-derived worked examples (tests/golden), the structural facts
the pages state (8 states, groups of 4, the carried state picks the value set
of the next group: "Pingala-8" landing page, sections "How it works" and
"Where the name comes from"; coset coding: the paper title), and properties
of the Ungerboeck set partition that any correct reading must have."""
import itertools

import numpy as np
import pytest

from oracle import p8f

pytestmark = pytest.mark.filterwarnings("ignore")

A0 = {-7, -3, 1, 5}
A1 = {-5, -1, 3, 7}


def test_worked_examples(golden):
    for ex in golden["decode"]:
        lv = p8f.decode_block_levels(ex["codes"])
        if "levels" in ex:
            assert lv == ex["levels"], ex["id"]
        else:
            got = [ex["scale"] * v for v in lv]
            assert got == ex["weights"], ex["id"]


def test_worked_examples_through_vectorised_decode(golden):
    e1 = golden["decode"][0]
    lv = p8f.decode_levels(np.array([e1["codes"]], dtype=np.uint8))
    assert lv.tolist()[0] == e1["levels"]
    e2 = golden["decode"][1]
    codes = np.zeros((1, 32), dtype=np.uint8)
    codes[0, :len(e2["codes"])] = e2["codes"]
    assert p8f.decode_levels(codes)[0, :32].tolist() == e2["levels"]


def test_every_state_maps_bytes_one_to_one_onto_its_value_set():
    t = p8f.codebook_table()
    for s in range(8):
        allowed = A1 if (s >> 1) & 1 else A0
        pts = {tuple(int(v) for v in t[s, b]) for b in range(256)}
        assert len(pts) == 256                       # injective, hence bijective
        assert all(set(p) <= allowed for p in pts)   # all four weights in A_z0


def test_branch_structure_of_the_8_state_trellis():
    # both branches leaving a state share the value set and differ in coset;
    # both branches entering a state share the value set and differ in coset
    for s in range(8):
        z0s = {p8f.z0_of_state(s)}
        z1s = {p8f.z1_of_branch(s, u) for u in (0, 1)}
        assert len(z0s) == 1 and z1s == {0, 1}
    for sn in range(8):
        u = sn & 1
        preds = [sn >> 1, (sn >> 1) | 4]
        assert all(p8f.next_state(p, u) == sn for p in preds)
        assert len({p8f.z0_of_state(p) for p in preds}) == 1
        assert {p8f.z1_of_branch(p, u) for p in preds} == {0, 1}
    # the four cosets (z0, z1) are used equally often over all (state, u)
    counts = {}
    for s in range(8):
        for u in (0, 1):
            key = (p8f.z0_of_state(s), p8f.z1_of_branch(s, u))
            counts[key] = counts.get(key, 0) + 1
    assert sorted(counts.values()) == [4, 4, 4, 4]


def test_cosets_partition_the_value_set_by_parity():
    # within a value set, the two branches from a state give disjoint
    # 128-point cosets whose union is A^4, split by the parity of sum(p_j)
    t = p8f.codebook_table()
    for s in range(8):
        c = [{tuple(int(v) for v in t[s, b]) for b in range(256) if (b & 1) == u} for u in (0, 1)]
        assert len(c[0]) == len(c[1]) == 128 and not (c[0] & c[1])
        z0 = p8f.z0_of_state(s)
        for u in (0, 1):
            z1 = p8f.z1_of_branch(s, u)
            for pt in c[u]:
                p = [(v + 7 - 2 * z0) // 4 for v in pt]
                assert sum(x % 2 for x in p) % 2 == z1
        # minimum squared distance inside a coset is 2 * 4^2 (a D4 coset),
        # against 4^2 between the two cosets
        pts = np.array(sorted(c[0]), dtype=np.int64)
        d = ((pts[:, None, :] - pts[None, :, :]) ** 2).sum(-1)
        assert d[d > 0].min() == 32


def test_state_resets_and_memory_is_three_groups():
    rng = np.random.default_rng(11)
    for _ in range(50):
        blk = rng.integers(0, 256, 32).tolist()
        base = p8f.decode_block_levels(blk)
        t = int(rng.integers(0, 32))
        flipped = list(blk)
        flipped[t] ^= 1                                  # one branch bit
        lv = p8f.decode_block_levels(flipped)
        changed = {i // 4 for i in range(128) if lv[i] != base[i]}
        assert changed <= set(range(t, min(32, t + 4)))
        assert t in changed


def test_vectorised_decode_equals_scalar_walk():
    rng = np.random.default_rng(12)
    codes = rng.integers(0, 256, (7, 96), dtype=np.uint8)        # 3 blocks per row
    fast = p8f.decode_levels(codes)
    for r in range(7):
        for b in range(3):
            slow = p8f.decode_block_levels(codes[r, 32 * b:32 * b + 32])
            assert fast[r, 128 * b:128 * b + 128].tolist() == slow


def test_random_byte_strings_decode_to_valid_trellis_paths():
    rng = np.random.default_rng(13)
    for _ in range(200):
        blk = rng.integers(0, 256, 32)
        assert p8f.levels_trellis_valid(p8f.decode_block_levels(blk))


def test_trellis_validity_checker_rejects_broken_paths():
    # a planted mistake: swap the value set of one group -> invalid
    lv = p8f.decode_block_levels([3, 200, 17, 99, 5, 250])
    bad = list(lv)
    bad[8:12] = [v + 2 if v < 7 else v - 2 for v in bad[8:12]]
    assert p8f.levels_trellis_valid(lv)
    assert not p8f.levels_trellis_valid(bad)


def test_decoded_weights_are_exact_in_fp32_and_signed_zero():
    rng = np.random.default_rng(14)
    codes = rng.integers(0, 256, (3, 64), dtype=np.uint8)
    scales = rng.integers(0, 0x7C00, (3, 2)).astype(np.uint16)    # finite fp16 incl. subnormals
    scales[0, 0] = 0                                               # s = 0 -> signed zeros
    w = p8f.decode_weights(codes, scales)
    assert np.array_equal(w.astype(np.float32).astype(np.float64), w)
    lv = p8f.decode_levels(codes)
    neg = lv[0, :128] < 0
    z = w[0, :128].astype(np.float32)
    assert np.all(np.signbit(z[neg])) and not np.any(np.signbit(z[~neg]))


def test_footprint_is_two_bits_plus_scales(golden):
    from qgemv_amd import synth
    fp = golden["footprint_bytes"]

    def nbytes(shapes, layers):
        return layers * sum(n * k // 4 + (n * k // 128) * 2 for n, k in shapes.values())

    assert 512 * 2048 // 4 + 512 * 2048 // 64 == fp["single_512x2048"]
    assert nbytes(synth.qwen3_4b_shapes(), 1) == fp["qwen_layer"]
    assert nbytes(synth.qwen3_4b_shapes(), 36) == fp["qwen_36_layers"]
    assert nbytes(synth.llama31_8b_shapes(), 32) == fp["llama_32_layers"]
    # the arrays the generators hand over have exactly that many bytes
    c, s = synth.random_matrix(0, "q", synth.qwen3_4b_shapes())
    assert c.nbytes + s.nbytes == 4096 * 2560 * 17 // 64
    # 2.125 bits per weight
    assert (c.nbytes + s.nbytes) * 8 / (4096 * 2560) == pytest.approx(2.125, abs=0)


def test_codebook_table_closed_form_levels():
    # every entry is 4 p + 2 z0 - 7 with p in 0..3 built from the stated bits
    t = p8f.codebook_table()
    for s, byte in itertools.product(range(8), range(256)):
        z0 = (s >> 1) & 1
        for j in range(4):
            e = (byte >> (4 + j)) & 1
            v = int(t[s, byte, j])
            assert (v - 2 * z0 + 7) % 4 == 0
            p = (v - 2 * z0 + 7) // 4
            assert p >> 1 == e
            if j < 3:
                assert p & 1 == (byte >> (1 + j)) & 1
