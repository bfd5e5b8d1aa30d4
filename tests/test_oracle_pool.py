"""Pins for the coarsening / refinement oracle: closed forms and the nesting
of tree levels, not a restatement of its formula."""
import numpy as np

from oracle import pool as P
from oracle import tree as T


def _data(n=256, H=2, d=8, seed=0):
    g = np.random.default_rng(seed)
    return g.standard_normal((n, H, d)), g.permutation(n)


def test_constant_children_give_that_constant():
    x, perm = _data()
    parents = np.random.default_rng(1).standard_normal((256 // 8, 2, 8))
    xt = np.repeat(parents, 8, axis=0)            # tree order: 8 equal children
    x = np.empty_like(xt)
    x[perm] = xt
    assert np.allclose(P.coarsen(x, perm, 8), parents, atol=1e-15, rtol=0)


def test_coarsen_after_refine_is_identity():
    xc = np.random.default_rng(2).standard_normal((32, 2, 8))
    perm = np.random.default_rng(3).permutation(256)
    assert np.allclose(P.coarsen(P.refine(xc, perm, 8), perm, 8), xc, atol=1e-15, rtol=0)


def test_levels_nest():
    """Coarsening by 4 then by 2 (tree order, no permutation) equals
    coarsening by 8: the parents of parents are the grandparents."""
    x, perm = _data()
    once = P.coarsen(x, perm, 8)
    twice = P.coarsen(P.coarsen(x, perm, 4), None, 2)
    assert np.allclose(once, twice, atol=1e-14, rtol=0)


def test_s1_is_the_gather_and_full_is_the_mean():
    x, perm = _data()
    assert np.array_equal(P.coarsen(x, perm, 1), x[perm])
    assert np.allclose(P.coarsen(x, perm, 256)[0], x.mean(axis=0), atol=1e-14, rtol=0)


def test_parents_are_tree_nodes():
    """With a real tree of leaf 8, each parent of s = 8 averages exactly one
    leaf's points (the points of a ball are contiguous at every level)."""
    g = np.random.default_rng(4)
    c = g.random((256, 3)).astype(np.float32)
    perm = T.build(c, 8)
    x = g.standard_normal((256, 1, 4))
    leaves = perm.reshape(-1, 8)
    want = np.stack([x[sorted(lf)].mean(axis=0) for lf in leaves])
    assert np.allclose(P.coarsen(x, perm, 8), want, atol=1e-14, rtol=0)


def test_refine_scatters_to_original_order():
    xc = np.arange(4, dtype=np.float64).reshape(4, 1, 1)
    perm = np.array([3, 0, 2, 1, 7, 5, 6, 4])
    out = P.refine(xc, perm, 2)[:, 0, 0]
    # tree positions 0,1 -> parent 0 at original rows 3, 0; 2,3 -> parent 1 at 2, 1; ...
    assert out.tolist() == [0, 1, 1, 0, 3, 2, 3, 2]
