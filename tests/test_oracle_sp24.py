"""Pins for the oracle's 2:4 prune / check / compress / decompress: the pages' toy vectors and
mechanism figure, exhaustive brute force over every four-code group, and round trips."""
import itertools
import json
import os

import numpy as np

from oracle import quant, sp24

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _codes_of(values):
    """Quantise a short vector (zero-padded to a multiple of 16) into one row of codes."""
    v = np.zeros(((len(values) + 15) // 16) * 16, np.float32)
    v[:len(values)] = values
    return quant.quantize(v[None, :])[0]


def test_toy_vectors_per_group_not_global_fraction():
    g = _golden("toy_vectors.json")
    A, B = np.array(g["A"], np.float32), np.array(g["B"], np.float32)
    assert np.mean(A == 0) == g["zero_fraction_A"] and np.mean(B == 0) == g["zero_fraction_B"]
    bad_a, first_a = sp24.check(_codes_of(A))
    bad_b, first_b = sp24.check(_codes_of(B))
    assert bad_a == 0 and first_a == -1
    assert bad_b == 1 and first_b == g["B_groups_pass"].index(False)
    # the same rule on raw code rows with unit-ish scale: [2,0,4,0 | 5,0,6,0] and [2,4,5,0 | 6,0,0,0]
    ca = quant.pack_nibbles(np.array([[2, 0, 4, 0, 5, 0, 6, 0]]))
    cb = quant.pack_nibbles(np.array([[2, 4, 5, 0, 6, 0, 0, 0]]))
    assert sp24.check(ca) == (0, -1) and sp24.check(cb) == (1, 0)


def test_toy_vectors_compress_bytes():
    # A: groups [2,0,4,0], [5,0,6,0] keep positions (0,2): vals 0x42, 0x65; nib = 0 | 2<<2 = 8 -> meta 0x88
    ca = quant.pack_nibbles(np.array([[2, 0, 4, 0, 5, 0, 6, 0]]))
    vals, meta, bad = sp24.compress(ca)
    assert vals.tolist() == [[0x42, 0x65]] and meta.tolist() == [[0x88]] and bad == 0
    # B: group 0 fails -> vals 0x00, positions (0,1) (nib 0x4); group 1 [6,0,0,0] keeps the nonzero
    # position 0 and the lowest zero 1: vals 0x06, nib 0x4 -> meta 0x44
    cb = quant.pack_nibbles(np.array([[2, 4, 5, 0, 6, 0, 0, 0]]))
    vals, meta, bad = sp24.compress(cb)
    assert vals.tolist() == [[0x00, 0x06]] and meta.tolist() == [[0x44]] and bad == 1


def test_mechanism_figure_positions():
    g = _golden("mechanism_figure.json")
    # w0 0 0 w3 with nonzero codes 3 and 5 (plus a passing second group to fill a meta byte)
    codes = quant.pack_nibbles(np.array([[3, 0, 0, 5, 0, 0, 0, 0]]))
    vals, meta, bad = sp24.compress(codes)
    i0, i1 = sp24.positions(meta)
    assert [int(i0[0, 0]), int(i1[0, 0])] == g["kept_positions"]
    assert meta[0, 0] & 0xF == 0xC and vals[0, 0] == 0x53 and bad == 0


def _brute_group(c):
    """Plain per-group rule for one group of 4 codes: (passes, (i0, i1), vals byte)."""
    zeros = [i for i in range(4) if c[i] & 7 == 0]
    nonzeros = [i for i in range(4) if c[i] & 7 != 0]
    if len(zeros) < 2:
        return False, (0, 1), 0
    pick = sorted((nonzeros + zeros)[:2])
    return True, tuple(pick), c[pick[0]] | (c[pick[1]] << 4)


def test_exhaustive_all_groups():
    groups = np.array(list(itertools.product(range(16), repeat=4)), dtype=np.uint8)   # 65536 x 4
    # two groups per row so that each meta byte holds two groups: pair group i with group i
    rows = np.concatenate([groups, groups], axis=1)
    codes = quant.pack_nibbles(rows)
    vals, meta, bad = sp24.compress(codes)
    i0, i1 = sp24.positions(meta)
    n_bad = 0
    for r in range(len(groups)):
        ok, (p0, p1), vb = _brute_group(groups[r].tolist())
        n_bad += not ok
        assert (int(i0[r, 0]), int(i1[r, 0])) == (p0, p1)
        assert int(vals[r, 0]) == vb
    assert bad == 2 * n_bad
    assert sp24.check(codes)[0] == 2 * n_bad
    # count of failing groups: groups with at most one zero code (2 zero codes of 16: 0x0, 0x8)
    assert n_bad == sum(1 for g in groups if sum((x & 7) == 0 for x in g) < 2)


def test_first_bad_index_is_flat_and_minimal():
    rows = np.zeros((3, 16), np.uint8)
    rows[1, 8:12] = [1, 2, 3, 0]      # row 1, group 2
    rows[2, 0:4] = [1, 1, 1, 1]       # row 2, group 0
    bad, first = sp24.check(quant.pack_nibbles(rows))
    assert bad == 2 and first == 1 * 4 + 2


def test_round_trip():
    rng = np.random.default_rng(4)
    w = sp24.prune24((rng.standard_normal((16, 64)) * 0.02).astype(np.float32))
    codes, _, _ = quant.quantize(w)
    assert sp24.check(codes) == (0, -1)
    vals, meta, bad = sp24.compress(codes)
    assert bad == 0 and vals.shape == (16, 16) and meta.shape == (16, 8)
    back = sp24.decompress(vals, meta)
    nib, nib_back = quant.unpack_nibbles(codes), quant.unpack_nibbles(back)
    # unselected positions come back as +0 code; selected ones verbatim
    assert np.array_equal(np.where(nib & 7 == 0, nib_back & 7, nib), nib_back)
    assert np.array_equal(nib & 7, nib_back & 7)


def test_prune_keeps_two_largest_ties_to_lower_index():
    rng = np.random.default_rng(6)
    w = rng.standard_normal((8, 32)).astype(np.float32)
    w[0, 0:4] = [1.0, -1.0, 1.0, 0.5]        # tie among three: keep positions 0 and 1
    w[1, 4:8] = [0.0, 0.0, 0.0, 0.0]
    p = sp24.prune24(w)
    for n in range(8):
        for g in range(8):
            grp = w[n, 4 * g:4 * g + 4].tolist()
            order = sorted(range(4), key=lambda i: (-abs(grp[i]), i))
            keep = set(order[:2])
            for i in range(4):
                want = grp[i] if i in keep else 0.0
                assert p[n, 4 * g + i] == want
    assert p[0, 0:4].tolist() == [1.0, -1.0, 0.0, 0.0]
    assert sp24.check(quant.quantize(p)[0]) == (0, -1)
