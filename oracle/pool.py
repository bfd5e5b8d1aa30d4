"""Coarsening and refinement of tree-ordered features (test infrastructure
only; parity is pinned by tests/test_oracle_pool.py).

Erwin coarsens and then refines the ball tree while the attention ball size
stays fixed, U-Net fashion (Erwin thread on Bluesky, post 8/N); because every
level of the tree is stored contiguously, the operations reduce to views and
means (post 9/N).  Reading taken here (the non-learned half of that U-Net):

* coarsen by s = 2^k: the feature of a parent is the plain mean of its s
  children, i.e. of s consecutive tree positions; the coarse level is in
  tree order.
* refine by s: every child takes its parent's feature.

Inputs in original order are gathered into tree order first (x[perm]); a
refined output is scattered back (out[perm] = ...).  fp64 throughout.
"""
from __future__ import annotations

import numpy as np

from .attention import _f64


def coarsen(x, perm, s: int) -> np.ndarray:
    """[N,H,d] (original order if perm is given) -> [N/s,H,d] in tree order."""
    x = _f64(x)
    n = x.shape[0]
    if n % s:
        raise ValueError("s must divide N")
    xt = x if perm is None else x[np.asarray(perm, dtype=np.int64)]
    return xt.reshape(n // s, s, *xt.shape[1:]).mean(axis=1)


def refine(xc, perm, s: int) -> np.ndarray:
    """[N/s,H,d] coarse level -> [N,H,d], original order if perm is given."""
    xc = _f64(xc)
    xt = np.repeat(xc, s, axis=0)
    if perm is None:
        return xt
    out = np.empty_like(xt)
    out[np.asarray(perm, dtype=np.int64)] = xt
    return out


__all__ = ["coarsen", "refine"]
