"""Ball attention and full attention in fp64 (test infrastructure only).

Ball Tree Attention computes scaled dot-product attention inside each ball of
a chosen tree level, all balls in parallel (Erwin thread on Bluesky, post 7/N;
Pith review of arXiv 2506.12541, "What carries the argument": scaled
dot-product attention within each ball).  The pages give no mask, bias or
causality, so none is applied; the scale is 1/sqrt(d) and the softmax
subtracts the row maximum before exponentiating.

Layout: q, k, v are [N, H, d] in original point order; ``perm`` is the tree
permutation (``perm[t]`` = original index at tree position t), or ``None`` if
the inputs are already in tree order.  A ball is ``ball`` contiguous tree
positions.  The output is returned in the same order as the inputs.
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):                 # torch tensor (bf16 or f32)
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def softmax_rows(s: np.ndarray) -> np.ndarray:
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def sdpa(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """softmax(q k^T / sqrt(d)) v over the last two axes ([..., n, d])."""
    d = q.shape[-1]
    s = q @ np.swapaxes(k, -1, -2) / np.sqrt(d)
    return softmax_rows(s) @ v


def ball_attn(q, k, v, perm, ball: int, chunk_balls: int = 64) -> np.ndarray:
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, H, d = q.shape
    if ball < 1 or n % ball:
        raise ValueError("ball must divide N")
    if perm is not None:
        perm = np.asarray(perm, dtype=np.int64)
        q, k, v = q[perm], k[perm], v[perm]          # tree order
    nb = n // ball
    out = np.empty_like(q)
    for b0 in range(0, nb, chunk_balls):
        b1 = min(nb, b0 + chunk_balls)
        sl = slice(b0 * ball, b1 * ball)
        # [balls, ball, H, d] -> [balls, H, ball, d]
        qb = q[sl].reshape(b1 - b0, ball, H, d).transpose(0, 2, 1, 3)
        kb = k[sl].reshape(b1 - b0, ball, H, d).transpose(0, 2, 1, 3)
        vb = v[sl].reshape(b1 - b0, ball, H, d).transpose(0, 2, 1, 3)
        ob = sdpa(qb, kb, vb)
        out[sl] = ob.transpose(0, 2, 1, 3).reshape(-1, H, d)
    if perm is not None:
        res = np.empty_like(out)
        res[perm] = out                               # back to original order
        return res
    return out


def ball_attn_rows(q, k, v, perm, ball: int, rows) -> np.ndarray:
    """Ball attention for selected tree positions only: [len(rows), H, d].

    Used to check full-size runs on a sample; row t of the result is the
    output of the point at tree position ``rows[t]``.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    perm = np.arange(q.shape[0]) if perm is None else np.asarray(perm)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows),) + q.shape[1:])
    for i, t in enumerate(rows):
        b = t // ball
        keys = perm[b * ball:(b + 1) * ball]
        qt = q[perm[t]][:, None, :]                   # [H,1,d]
        kb = k[keys].transpose(1, 0, 2)               # [H,ball,d]
        vb = v[keys].transpose(1, 0, 2)
        out[i] = sdpa(qt, kb, vb)[:, 0, :]
    return out


def full_attn(q, k, v) -> np.ndarray:
    """Full (all-pairs) attention per head, [N,H,d] -> [N,H,d]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    o = sdpa(q.transpose(1, 0, 2), k.transpose(1, 0, 2), v.transpose(1, 0, 2))
    return o.transpose(1, 0, 2)


def ball_attn_padded(q, k, v, perm, ball: int) -> np.ndarray:
    """Ball attention on a padded tree (``oracle.tree.build_padded``): ``perm``
    has one entry per slot, -1 for an unused slot, and the points of a ball are
    its slots that hold a point.  Each point attends to the points of its own
    ball (every head); output in original order."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, H, d = q.shape
    perm = np.asarray(perm, dtype=np.int64)
    if ball < 1 or len(perm) % ball:
        raise ValueError("ball must divide the slot count")
    real = perm[perm >= 0]
    if len(real) != n or len(np.unique(real)) != n:
        raise ValueError("the slots must hold every point exactly once")
    out = np.zeros_like(q)
    for b0 in range(0, len(perm), ball):
        ids = perm[b0:b0 + ball]
        ids = ids[ids >= 0]
        if len(ids) == 0:
            continue
        # [H, m, d] per ball
        qb, kb, vb = (x[ids].transpose(1, 0, 2) for x in (q, k, v))
        out[ids] = sdpa(qb, kb, vb).transpose(1, 0, 2)
    return out
