"""Backward pass of ball attention in fp64 (test infrastructure only; pinned
by tests/test_oracle_attn_bwd.py against autograd of a library attention
routine and against finite differences).

The branches of BSA, its gates and Erwin's layers are learned (Pith review
of arXiv 2506.12541, "What carries the argument": learned sigmoid gates;
Erwin thread on Bluesky, post 7/N: attention inside balls), so training
needs the gradient of ball attention with respect to q, k and v.  Per ball
and head, with S = Q K^T / sqrt(d), P = softmax(S) row by row, O = P V and
an incoming gradient dO, the chain rule gives:

    dV = P^T dO
    dP = dO V^T
    D_i = sum_e dO[i, e] O[i, e]          (= sum_j P[i, j] dP[i, j])
    dS = P * (dP - D)                     (softmax backward, row by row)
    dQ = dS K / sqrt(d)
    dK = dS^T Q / sqrt(d)

Layout as in attention.py: [N, H, d] in original order with ``perm`` the
tree permutation (or ``None`` for tree order); gradients are returned in the
inputs' order.
"""
from __future__ import annotations

import numpy as np

from .attention import _f64, softmax_rows


def ball_attn_bwd(q, k, v, dout, perm, ball: int):
    """(dq, dk, dv) of ball attention for the output gradient ``dout``."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(dout)
    n, H, d = q.shape
    if ball < 1 or n % ball:
        raise ValueError("ball must divide N")
    if perm is not None:
        perm = np.asarray(perm, dtype=np.int64)
        q, k, v, do = q[perm], k[perm], v[perm], do[perm]      # tree order
    nb = n // ball
    shape = lambda x: x.reshape(nb, ball, H, d).transpose(0, 2, 1, 3)   # [nb,H,ball,d]
    Q, K, V, dO = shape(q), shape(k), shape(v), shape(do)
    scale = 1.0 / np.sqrt(d)
    P = softmax_rows(Q @ np.swapaxes(K, -1, -2) * scale)
    O = P @ V
    dV = np.swapaxes(P, -1, -2) @ dO
    dP = dO @ np.swapaxes(V, -1, -2)
    D = (dO * O).sum(axis=-1, keepdims=True)
    dS = P * (dP - D)
    dQ = dS @ K * scale
    dK = np.swapaxes(dS, -1, -2) @ Q * scale
    back = lambda x: x.transpose(0, 2, 1, 3).reshape(n, H, d)
    res = []
    for g in (dQ, dK, dV):
        g = back(g)
        if perm is not None:
            o = np.empty_like(g)
            o[perm] = g
            g = o
        res.append(g)
    return tuple(res)


__all__ = ["ball_attn_bwd"]
