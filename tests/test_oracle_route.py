"""Pins of the oracle's router: brute force over k-subsets, softmax identities,
finite differences and autograd for the router backward."""
import itertools

import numpy as np
import pytest
import scipy.special
import torch

import oracle



def brute_topk(row, k):
    """All k-subsets; keep the max-sum ones; the lexicographically smallest id set wins."""
    E = len(row)
    best, best_set = None, None
    for S in itertools.combinations(range(E), k):   # ascending lexicographic order
        s = sum(row[e] for e in S)
        if best is None or s > best:
            best, best_set = s, S
    return best_set


@pytest.mark.parametrize("E,k", [(4, 1), (5, 2), (6, 3), (8, 2), (10, 4), (7, 7)])
def test_topk_matches_bruteforce(E, k):
    rng = np.random.default_rng(E * 31 + k)
    for trial in range(60):
        if trial % 2:
            row = rng.integers(-2, 3, size=E).astype(np.float64)   # many ties
        else:
            row = rng.standard_normal(E)
        idx, w = oracle.route(row[None, :], k)
        assert tuple(sorted(idx[0].tolist())) == brute_topk(row.tolist(), k)
        # selection order: logit descending, ties by ascending id
        keys = [(-row[e], e) for e in idx[0]]
        assert keys == sorted(keys)


def test_gates_are_renormalised_full_softmax():
    rng = np.random.default_rng(1)
    L = rng.standard_normal((50, 12)) * 3
    for k in (1, 2, 5, 12):
        idx, w = oracle.route(L, k)
        np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-14)
        full = scipy.special.softmax(L, axis=1)
        sel = np.take_along_axis(full, idx.astype(np.int64), 1)
        np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-13)
        # invariant under per-row shifts of the logits
        idx2, w2 = oracle.route(L + rng.standard_normal((50, 1)) * 10, k)
        assert (idx2 == idx).all()
        np.testing.assert_allclose(w2, w, rtol=1e-12)


def test_negative_zero_ties_with_zero():
    idx, _ = oracle.route(np.array([[-0.0, 0.0, -1.0]]), 1)
    assert idx[0, 0] == 0


def test_route_backward_finite_differences():
    rng = np.random.default_rng(2)
    T, E, k = 6, 7, 3
    L = rng.standard_normal((T, E))
    dg = rng.standard_normal((T, k))
    idx, w = oracle.route(L, k)
    dL = oracle.route_backward(idx, w, dg, E)
    eps = 1e-6
    num = np.zeros_like(L)
    for t in range(T):
        for e in range(E):
            Lp, Lm = L.copy(), L.copy()
            Lp[t, e] += eps
            Lm[t, e] -= eps
            ip, wp = oracle.route(Lp, k)
            im, wm = oracle.route(Lm, k)
            assert (ip == idx).all() and (im == idx).all()
            num[t, e] = ((wp - wm) * dg).sum() / (2 * eps)
    np.testing.assert_allclose(dL, num, rtol=1e-6, atol=1e-9)


def test_route_backward_autograd():
    rng = np.random.default_rng(3)
    T, E, k = 9, 16, 4
    L = rng.standard_normal((T, E))
    dg = rng.standard_normal((T, k))
    idx, w = oracle.route(L, k)
    Lt = torch.tensor(L, requires_grad=True)
    sel = torch.gather(Lt, 1, torch.tensor(idx, dtype=torch.int64))
    g = torch.softmax(sel, dim=1)
    (g * torch.tensor(dg)).sum().backward()
    np.testing.assert_allclose(oracle.route_backward(idx, w, dg, E), Lt.grad.numpy(),
                               rtol=1e-12, atol=1e-14)
