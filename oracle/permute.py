"""Row permutations between original order and tree order (test
infrastructure only; see oracle/__init__).

The ball tree stores the points of every ball next to each other at every
level (Erwin thread on Bluesky, post 9/N), so moving features into a tree's
order is one gather of rows, and moving them back is one scatter.  Alternate
layers use a rotated tree instead of shifted windows (Erwin thread, the post on
rotating trees), so a feature tensor leaves tree A by a scatter back to
original order and enters tree B by a gather.

``perm[t]`` is the original index of the row at tree position ``t``:

* gather:  dst[t] = src[perm[t]]        (original order -> tree order)
* scatter: dst[perm[t]] = src[t]        (tree order -> original order)
* invert:  inv[perm[t]] = t             (so gather by inv == scatter by perm)

Padded trees (an uneven point count) have more slots than rows; an unused slot
holds -1.  Gathering gives such a slot a zero row, and scattering skips it.

Rows are copied as they are (any dtype): no arithmetic, so results are
byte-exact.  Plain loops over rows, one row at a time.
"""
from __future__ import annotations

import numpy as np


def _check_perm(perm, n: int) -> np.ndarray:
    p = np.asarray(perm)
    if p.ndim != 1 or p.shape[0] != n:
        raise ValueError("perm must hold one entry per row")
    if n and (p.min() < 0 or p.max() >= n or np.unique(p).shape[0] != n):
        raise ValueError("perm must be a permutation of 0..n-1")
    return p.astype(np.int64)


def gather(src, perm) -> np.ndarray:
    """dst[t] = src[perm[t]] over the rows (first axis) of src."""
    src = np.asarray(src)
    p = _check_perm(perm, src.shape[0])
    dst = np.empty_like(src)
    for t in range(src.shape[0]):
        dst[t] = src[p[t]]
    return dst


def scatter(src, perm) -> np.ndarray:
    """dst[perm[t]] = src[t] over the rows (first axis) of src."""
    src = np.asarray(src)
    p = _check_perm(perm, src.shape[0])
    dst = np.empty_like(src)
    for t in range(src.shape[0]):
        dst[p[t]] = src[t]
    return dst


def invert(perm) -> np.ndarray:
    """inv[perm[t]] = t (int32)."""
    p = _check_perm(perm, np.asarray(perm).shape[0])
    inv = np.empty(p.shape[0], dtype=np.int32)
    for t in range(p.shape[0]):
        inv[p[t]] = t
    return inv


def _check_padded(perm, n_rows: int) -> np.ndarray:
    p = np.asarray(perm).astype(np.int64)
    used = p[p >= 0]
    if p.ndim != 1 or (p < -1).any() or used.shape[0] != n_rows or \
            (n_rows and (used.max() >= n_rows or np.unique(used).shape[0] != n_rows)):
        raise ValueError("a padded perm holds each row index once and -1 elsewhere")
    return p


def gather_padded(src, perm) -> np.ndarray:
    """[n_rows, ...] -> [slots, ...]: dst[t] = src[perm[t]], zeros where
    perm[t] == -1."""
    src = np.asarray(src)
    p = _check_padded(perm, src.shape[0])
    dst = np.zeros((p.shape[0],) + src.shape[1:], dtype=src.dtype)
    for t in range(p.shape[0]):
        if p[t] >= 0:
            dst[t] = src[p[t]]
    return dst


def scatter_padded(src, perm, n_rows: int) -> np.ndarray:
    """[slots, ...] -> [n_rows, ...]: dst[perm[t]] = src[t] for used slots."""
    src = np.asarray(src)
    p = _check_padded(perm, n_rows)
    if src.shape[0] != p.shape[0]:
        raise ValueError("src must hold one row per slot")
    dst = np.empty((n_rows,) + src.shape[1:], dtype=src.dtype)
    for t in range(p.shape[0]):
        if p[t] >= 0:
            dst[p[t]] = src[t]
    return dst
