"""Tree invariant checkers (test infrastructure only).

These checkers do not call ``oracle.tree``: each one restates one defining
property of the ball tree directly on a candidate permutation, so they can pin
the oracle (and any other builder) from outside.  Together they characterise
the unique tree of the split rule described in ``oracle.tree``:

* ``is_bijection``       -- perm is a permutation of 0..N-1;
* ``leaf_sizes_ok``      -- N = leaf * 2^L (every leaf then holds ``leaf``);
* ``split_property``     -- at every internal node the left half precedes the
                            right half in (coordinate, index) order on the
                            node's split axis;
* ``axis_is_max_spread`` -- that split axis has the largest fp32 spread, the
                            lowest axis on ties;
* ``ascending_in_leaves``-- indices ascend inside every leaf.

Each returns ``(ok: bool, message: str)``.
"""
from __future__ import annotations

import numpy as np


def _coords(coords):
    c = np.array(coords, dtype=np.float32, copy=True)
    c[c == 0] = np.float32(0.0)        # -0.0 and +0.0 are the same key
    return c


def is_bijection(perm, n):
    p = np.asarray(perm)
    if p.shape != (n,):
        return False, f"shape {p.shape} != ({n},)"
    seen = np.zeros(n, dtype=bool)
    if p.min() < 0 or p.max() >= n:
        return False, "index out of range"
    seen[p] = True
    if not seen.all():
        return False, "repeated index"
    return True, ""


def leaf_sizes_ok(n, leaf):
    if leaf < 1 or n % leaf:
        return False, "leaf does not divide N"
    q = n // leaf
    if q & (q - 1):
        return False, "N/leaf is not a power of two"
    return True, ""


def _axis(pts):
    best, arg = None, 0
    for a in range(3):
        s = np.float32(pts[:, a].max()) - np.float32(pts[:, a].min())
        if best is None or s > best:          # strict: first maximum wins
            best, arg = s, a
    return arg


def _nodes(n, leaf):
    size = n
    while size > leaf:
        for start in range(0, n, size):
            yield start, size
        size //= 2


def axis_is_max_spread(coords, perm, leaf):
    c = _coords(coords)
    p = np.asarray(perm)
    for start, size in _nodes(len(p), leaf):
        ids = p[start:start + size]
        pts = c[ids]
        spreads = [np.float32(pts[:, a].max()) - np.float32(pts[:, a].min())
                   for a in range(3)]
        a = _axis(pts)
        if any(s > spreads[a] for s in spreads) or \
           any(spreads[b] == spreads[a] for b in range(a)):
            return False, f"node [{start},{start+size}): axis {a} not first max"
    return True, ""


def split_property(coords, perm, leaf):
    """Left half <= right half in (coord on split axis, index) order."""
    c = _coords(coords)
    p = np.asarray(perm)
    for start, size in _nodes(len(p), leaf):
        ids = p[start:start + size]
        a = _axis(c[ids])
        half = size // 2
        L, R = ids[:half], ids[half:]
        lv, rv = c[L, a], c[R, a]
        lmax = lv.max()
        rmin = rv.min()
        if lmax > rmin:
            return False, f"node [{start},{start+size}): left {lmax} > right {rmin}"
        if lmax == rmin:
            # among points with the boundary value, left indices < right ones
            li = L[lv == lmax].max()
            ri = R[rv == rmin].min()
            if li > ri:
                return False, f"node [{start},{start+size}): tie broken wrong"
    return True, ""


def ascending_in_leaves(perm, leaf):
    p = np.asarray(perm).reshape(-1, leaf)
    if np.any(np.diff(p, axis=1) <= 0):
        return False, "indices not ascending inside a leaf"
    return True, ""


def check_tree(coords, perm, leaf):
    n = len(coords)
    for name, res in (
        ("bijection", is_bijection(perm, n)),
        ("leaf_sizes", leaf_sizes_ok(n, leaf)),
        ("ascending_in_leaves", ascending_in_leaves(perm, leaf)),
        ("axis", axis_is_max_spread(coords, perm, leaf)),
        ("split", split_property(coords, perm, leaf)),
    ):
        if not res[0]:
            return False, f"{name}: {res[1]}"
    return True, ""


def check_padded_tree(coords, perm, leaf):
    """The padded tree of an uneven N: slots = the smallest leaf * 2^L >= N;
    the points fill each leaf's first slots in ascending index, -1 after; at
    every internal node the left child holds ceil(n/2) of the node's n points,
    on the axis of largest fp32 spread, all of them before the right child's
    in (coordinate, index) order."""
    c = _coords(coords)
    n = len(c)
    p = np.asarray(perm)
    cap = leaf
    while cap < n:
        cap *= 2
    if p.shape != (cap,):
        return False, f"slot count {p.shape} != ({cap},)"
    real = p[p >= 0]
    if np.any(p < -1):
        return False, "entry below -1"
    ok, msg = is_bijection(real, n)
    if not ok:
        return False, "points: " + msg
    for j in range(0, cap, leaf):
        row = p[j:j + leaf]
        m = int((row >= 0).sum())
        if np.any(row[:m] < 0) or np.any(np.diff(row[:m]) <= 0):
            return False, f"leaf at {j}: points not first or not ascending"
    size = cap
    while size > leaf:
        for start in range(0, cap, size):
            ids = p[start:start + size]
            ids = ids[ids >= 0]
            half = size // 2
            L = p[start:start + half]
            L = L[L >= 0]
            R = p[start + half:start + size]
            R = R[R >= 0]
            if len(L) != (len(ids) + 1) // 2:
                return False, f"node at {start}: left holds {len(L)} of {len(ids)}"
            if len(ids) < 2:
                continue
            a = _axis(c[ids])
            if len(R) == 0:
                continue
            lv, rv = c[L, a], c[R, a]
            if lv.max() > rv.min():
                return False, f"node at {start}: left {lv.max()} > right {rv.min()}"
            if lv.max() == rv.min() and L[lv == lv.max()].max() > R[rv == rv.min()].min():
                return False, f"node at {start}: tie broken wrong"
        size //= 2
    return True, ""
