"""Pins of the permutation oracle (gather, scatter, inverse, padded forms):
a hand-derived fixture, the identities that tie the three together, and
NumPy's own indexing and argsort as independent routines."""
import json
import os

import numpy as np
import pytest

from oracle import permute as P

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold():
    with open(os.path.join(GOLD, "permute_hand.json")) as f:
        return json.load(f)


def test_golden_hand():
    g = _gold()
    x, p = np.array(g["rows"]), np.array(g["perm"])
    assert P.gather(x, p).tolist() == g["gather"]
    assert P.scatter(x, p).tolist() == g["scatter"]
    assert P.invert(p).tolist() == g["invert"]


def test_golden_hand_padded():
    g = _gold()["padded"]
    x, p = np.array(g["rows"]), np.array(g["perm"])
    assert P.gather_padded(x, p).tolist() == g["gather"]
    assert P.scatter_padded(np.array(g["slots"]), p, len(g["rows"])).tolist() == g["scatter"]


@pytest.mark.parametrize("n,shape,dtype", [(1, (3,), np.float32), (7, (2, 5), np.int16),
                                           (1000, (8, 4), np.float64), (513, (), np.int32)])
def test_identities(n, shape, dtype):
    rng = np.random.default_rng(n)
    x = (rng.standard_normal((n,) + shape) * 1000).astype(dtype)
    p = rng.permutation(n)
    g, s, inv = P.gather(x, p), P.scatter(x, p), P.invert(p)
    assert np.array_equal(P.scatter(g, p), x)            # scatter undoes gather
    assert np.array_equal(P.gather(s, p), x)             # gather undoes scatter
    assert np.array_equal(P.gather(x, inv), s)           # gather by the inverse
    assert np.array_equal(P.invert(inv), p)              # the inverse of the inverse
    assert np.array_equal(P.gather(x, np.arange(n)), x)  # identity permutation
    # composition: gathering twice is gathering by the composed permutation
    p2 = rng.permutation(n)
    assert np.array_equal(P.gather(P.gather(x, p), p2), P.gather(x, p[p2]))


def test_numpy_indexing_and_argsort():
    """Library routines that compute the same maps: fancy indexing, indexed
    assignment, argsort."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((300, 6))
    p = rng.permutation(300)
    assert np.array_equal(P.gather(x, p), x[p])
    ref = np.empty_like(x)
    ref[p] = x
    assert np.array_equal(P.scatter(x, p), ref)
    assert np.array_equal(P.invert(p), np.argsort(p))


def test_padded_round_trip_and_reduction():
    rng = np.random.default_rng(5)
    n, slots = 97, 128
    x = rng.standard_normal((n, 3))
    p = np.full(slots, -1)
    p[rng.permutation(slots)[:n]] = rng.permutation(n)
    g = P.gather_padded(x, p)
    assert np.array_equal(g[p < 0], np.zeros(((p < 0).sum(), 3)))
    assert np.array_equal(P.scatter_padded(g, p, n), x)
    q = rng.permutation(n)                     # no unused slot: the plain forms
    assert np.array_equal(P.gather_padded(x, q), P.gather(x, q))
    assert np.array_equal(P.scatter_padded(x, q, n), P.scatter(x, q))


@pytest.mark.parametrize("bad", [[0, 0, 1], [0, 1, 3], [-1, 0, 1], [0, 1]])
def test_rejects_non_permutations(bad):
    with pytest.raises(ValueError):
        P.gather(np.zeros((3, 2)), bad)


def test_planted_swap_is_caught():
    """A gather written as a scatter (or the inverse left out) fails the
    fixture: the two maps differ for any permutation that is not an
    involution."""
    g = _gold()
    x, p = np.array(g["rows"]), np.array(g["perm"])
    assert P.scatter(x, p).tolist() != g["gather"]
    assert P.gather(x, P.invert(p)).tolist() != g["gather"]
