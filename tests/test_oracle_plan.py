"""Pins of the oracle's schedule table: exhaustive enumeration of small routings
against a library stable sort, invariants, invalid ids and the tile list."""
import itertools

import numpy as np
import pytest

import oracle



def check_plan_against_stable_sort(idx, E):
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    p = oracle.build_plan(idx, E)
    flat = idx.reshape(-1)
    order = np.argsort(flat, kind="stable")                 # library stable sort
    np.testing.assert_array_equal(p["counts"], np.bincount(flat, minlength=E))
    np.testing.assert_array_equal(p["offsets"], np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    np.testing.assert_array_equal(p["src_token"], order // k)
    np.testing.assert_array_equal(p["src_slot"], order % k)
    inv = np.empty_like(order)
    inv[order] = np.arange(order.size)
    np.testing.assert_array_equal(p["pos"].reshape(-1), inv)
    return p


def check_invariants(idx, E, p):
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    R = T * k
    assert p["counts"].sum() == R
    assert p["offsets"][0] == 0 and p["offsets"][E] == R
    assert np.all(np.diff(p["offsets"]) >= 0)
    rows = p["src_token"] * k + p["src_slot"]
    assert sorted(rows.tolist()) == list(range(R))         # a permutation of the pairs
    for e in range(E):
        seg = slice(p["offsets"][e], p["offsets"][e + 1])
        assert np.all(idx[p["src_token"][seg], p["src_slot"][seg]] == e)
        assert np.all(np.diff(p["src_token"][seg]) > 0)    # strictly ascending tokens
    pos = p["pos"]
    for t in range(T):
        for j in range(k):
            r = pos[t, j]
            assert p["src_token"][r] == t and p["src_slot"][r] == j


def test_exhaustive_T4_E4_k2():
    E, k = 4, 2
    choices = list(itertools.permutations(range(E), k))    # 12 ordered distinct pairs
    n = 0
    for rows in itertools.product(choices, repeat=4):
        idx = np.array(rows)
        p = check_plan_against_stable_sort(idx, E)
        if n % 97 == 0:
            check_invariants(idx, E, p)
        n += 1
    assert n == 12 ** 4


@pytest.mark.parametrize("seed", range(20))
def test_random_small(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(1, 17))
    E = int(rng.integers(2, 40))
    k = int(rng.integers(1, min(E, 8) + 1))
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    p = check_plan_against_stable_sort(idx, E)
    check_invariants(idx, E, p)


def test_degenerate_routings():
    # every token on the same expert set, empty experts, k = E, T = 1
    for idx, E in [(np.tile([[3, 1]], (9, 1)), 5), (np.array([[0, 1, 2, 3]]), 4),
                   (np.tile(np.arange(6)[None], (5, 1)), 6)]:
        p = check_plan_against_stable_sort(idx, E)
        check_invariants(idx, E, p)


def test_invalid_expert_ids_are_excluded():
    idx = np.array([[0, 5], [-1, 1], [1, 0]])
    p = oracle.build_plan(idx, 3)
    assert p["err"]
    np.testing.assert_array_equal(p["counts"], [2, 2, 0])
    np.testing.assert_array_equal(p["src_token"], [0, 2, 1, 2, -1, -1])
    np.testing.assert_array_equal(p["src_slot"], [0, 1, 1, 0, -1, -1])
    np.testing.assert_array_equal(p["pos"], [[0, -1], [-1, 2], [3, 1]])


def test_tile_list_covers_segments():
    rng = np.random.default_rng(5)
    counts = rng.integers(0, 300, size=37)
    counts[[3, 4, 20]] = 0
    offsets = np.concatenate([[0], np.cumsum(counts)])
    for bm in (16, 64, 128):
        tl = oracle.tile_list(counts, offsets, bm)
        assert len(tl) == sum(-(-c // bm) for c in counts)
        covered = np.zeros(offsets[-1], dtype=int)
        for e, r0 in tl:
            r1 = min(r0 + bm, offsets[e + 1])
            assert offsets[e] <= r0 < offsets[e + 1]
            covered[r0:r1] += 1
        assert np.all(covered == 1)
