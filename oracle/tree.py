"""Ball-tree partition oracle (test infrastructure only; see oracle/__init__).

What it computes
----------------
A ball tree recursively partitions the points into nested sets of similar
size, each covered by a ball (Erwin thread on Bluesky, post 6/N), and the
points of each ball are stored next to each other at every level (post 9/N),
so that a ball at any level is a contiguous range of the tree order (post 7/N:
attention is computed inside the balls of a chosen level).

The pages leave the split rule open.  The reading used here:

* split axis: the axis of largest spread, spread = fp32(max - min) over the
  node's coordinates; ties go to the lower axis (x, then y, then z);
* split position: two equal halves; the left half is the n/2 smallest points
  ordered by (coordinate on the split axis, original index); -0.0 counts as
  +0.0;
* inside every node the points keep ascending original index, so the output
  permutation is unique;
* recursion stops at exactly ``leaf`` points, which requires N = leaf * 2^L.

``perm[t]`` is the original index of the point at tree position ``t``.

Uneven N (``build_padded``): the sets only need to be of similar size, while
contiguous storage with equal-size balls at every level is what turns ball
operations into views and means (posts 6/N and 9/N).  Reading: the tree has
``leaf * 2^L`` slots, L the smallest with ``leaf * 2^L >= N``; a node of n
points (and 2c slots) gives its left child the ceil(n/2) smallest points in
(coordinate, index) order and its right child the rest, each child owning c
slots; a leaf stores its points first (ascending index) and marks the unused
slots with -1.  Sibling point counts differ by at most one, and for
N = leaf * 2^L the result is exactly ``build``.

Rotation: the second tree of a rotated pair is the same tree built on
coordinates rotated by a caller-supplied 3x3 matrix (Erwin thread: trees are
rotated, instead of shifting windows as Swin does, so that alternate layers mix
information across balls).  Each product and each sum of the rotation is
rounded to fp32 separately: x'_a = ((R[a,0]*x + R[a,1]*y) + R[a,2]*z).
"""
from __future__ import annotations

import numpy as np


def _levels(n: int, leaf: int) -> int:
    if leaf < 1 or n < leaf or n % leaf:
        raise ValueError("N must be leaf * 2^L")
    q = n // leaf
    if q & (q - 1):
        raise ValueError("N must be leaf * 2^L")
    return q.bit_length() - 1


def canonical(coords) -> np.ndarray:
    """fp32 copy with -0.0 replaced by +0.0; rejects NaN/Inf."""
    c = np.array(coords, dtype=np.float32, copy=True)
    if c.ndim != 2 or c.shape[1] != 3:
        raise ValueError("coords must be [N,3]")
    if not np.all(np.isfinite(c)):
        raise ValueError("coordinates must be finite")
    c[c == 0] = np.float32(0.0)
    return c


def split_axis(pts: np.ndarray) -> int:
    """Axis of largest fp32 spread; the first one on ties."""
    spread = pts.max(axis=0) - pts.min(axis=0)        # fp32 subtraction
    assert spread.dtype == np.float32
    return int(np.argmax(spread))                      # first maximum


def build(coords, leaf: int) -> np.ndarray:
    """Tree permutation of the points (int64 array, length N)."""
    c = canonical(coords)
    n = c.shape[0]
    _levels(n, leaf)

    def rec(ids: np.ndarray) -> list:
        if len(ids) == leaf:
            return [ids]
        a = split_axis(c[ids])
        order = np.lexsort((ids, c[ids, a]))          # by (coord, index)
        half = len(ids) // 2
        left = np.sort(ids[order[:half]])
        right = np.sort(ids[order[half:]])
        return rec(left) + rec(right)

    return np.concatenate(rec(np.arange(n, dtype=np.int64)))


def padded_size(n: int, leaf: int) -> int:
    """Slots of the padded tree: the smallest leaf * 2^L that is >= n."""
    if leaf < 1 or n < 1:
        raise ValueError("need N >= 1 and leaf >= 1")
    cap = leaf
    while cap < n:
        cap *= 2
    return cap


def build_padded(coords, leaf: int) -> np.ndarray:
    """Padded tree permutation (int64, length padded_size(N, leaf)); -1 marks
    an unused slot."""
    c = canonical(coords)
    n = c.shape[0]
    cap = padded_size(n, leaf)

    def rec(ids: np.ndarray, slots: int) -> list:
        if slots == leaf:
            return [ids, np.full(leaf - len(ids), -1, dtype=np.int64)]
        if len(ids) == 0:
            return [np.full(slots, -1, dtype=np.int64)]
        a = split_axis(c[ids])
        order = np.lexsort((ids, c[ids, a]))          # by (coord, index)
        nl = (len(ids) + 1) // 2                      # ceil(n/2) go left
        left = np.sort(ids[order[:nl]])
        right = np.sort(ids[order[nl:]])
        return rec(left, slots // 2) + rec(right, slots // 2)

    return np.concatenate(rec(np.arange(n, dtype=np.int64), cap))


def rotate_build_padded(coords, leaf: int, R) -> np.ndarray:
    return build_padded(rotate(coords, R), leaf)


def rotate(coords, R) -> np.ndarray:
    """Rotate fp32 coordinates, rounding every product and sum to fp32."""
    c = np.asarray(coords, dtype=np.float32)
    R = np.asarray(R, dtype=np.float32).reshape(3, 3)
    if not np.all(np.isfinite(R)):
        raise ValueError("rotation must be finite")
    out = np.empty_like(c)
    x, y, z = c[:, 0], c[:, 1], c[:, 2]
    for a in range(3):
        t = R[a, 0] * x                                # fp32 product
        t = t + R[a, 1] * y                            # fp32 product, fp32 sum
        t = t + R[a, 2] * z
        out[:, a] = t
    return out


def rotate_build(coords, leaf: int, R) -> np.ndarray:
    return build(rotate(coords, R), leaf)


def node_ranges(n: int, leaf: int):
    """(level, node, start, stop) for every node of the implicit tree."""
    L = _levels(n, leaf)
    for lev in range(L + 1):
        size = n >> lev
        for i in range(1 << lev):
            yield lev, i, i * size, (i + 1) * size
