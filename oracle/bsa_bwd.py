"""Backward pass of Ball Sparse Attention in fp64 (test infrastructure only;
pinned by tests/test_oracle_bsa_bwd.py against central finite differences
of the forward oracle ``oracle.bsa.bsa`` and against ball attention's
backward where the gates reduce BSA to it).

The branches and gates of BSA are learned (Pith review of arXiv
2506.12541, "What carries the argument": learned sigmoid gates merge the
branch outputs), so training needs the gradients of the BSA output with
respect to q, k, v and the gate parameters.  Forward, per token t and head h
in tree order (module docstring of oracle/bsa.py):

    out = G0 O_ball + G1 O_cmp + G2 O_slc,    G = sigmoid(W q + b)

Backward for an incoming gradient dO:

* gates: dG_i = sum_e dO[e] O_i[e]; with learned gates dz_i = dG_i G_i (1 -
  G_i), dq += sum_i dz_i W[i], dW[i] = sum_{t,h} dz_i q, db[i] = sum_{t,h}
  dz_i.  Constant gates have no parameters and pass no gradient to q.
* each branch is softmax attention whose output gradient is G_i dO; its
  (dQ, dK, dV) follow the chain rule written out in attention_bwd.py.
  Compression: the keys and values are block means of K and V, so every
  token of block j receives dKc[j] / l and dVc[j] / l.  Selection: the keys
  and values are rows of K and V, which receive the sum over every group
  that selected their block.
* top-k: the selection is a step function of the scores, so it passes no
  gradient (the straight-through reading of a top-k; the scores are not
  differentiated).  The finite differences that pin this file move inputs by
  amounts too small to change a selection.

Group compression (``query_compression``) is not covered.
"""
from __future__ import annotations

import numpy as np

from .attention import _f64, softmax_rows
from .bsa import gates, pool_blocks, select


def attn_bwd(Q, K, V, dO):
    """Softmax attention over the last two axes and its backward:
    returns (O, dQ, dK, dV) for S = Q K^T / sqrt(d), P = softmax(S), O = P V."""
    d = Q.shape[-1]
    scale = 1.0 / np.sqrt(d)
    P = softmax_rows(Q @ np.swapaxes(K, -1, -2) * scale)
    O = P @ V
    dV = np.swapaxes(P, -1, -2) @ dO
    dP = dO @ np.swapaxes(V, -1, -2)
    D = (dO * O).sum(axis=-1, keepdims=True)
    dS = P * (dP - D)
    dQ = dS @ K * scale
    dK = np.swapaxes(dS, -1, -2) @ Q * scale
    return O, dQ, dK, dV


def bsa_bwd(q, k, v, dout, perm, ball: int, block: int, group: int, topk: int,
            mask_own_ball: bool = True, W=None, b=None, gate_const=None, sel_override=None):
    """(dq, dk, dv, dW, db) of BSA (without group compression) for ``dout``.

    Inputs and gradients are [N,H,d] in original order (``perm`` is the tree
    permutation, or None for tree order).  dW [3,d] and db [3] are None with
    constant gates.  ``sel_override`` ([H, N/g, k*]) replaces the oracle's own
    top-k choice, as in ``oracle.bsa.bsa`` (a numerical near-tie admits
    another valid set).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(dout)
    n, H, d = q.shape
    if n % ball or ball % block or n % group:
        raise ValueError("need ball | N, block | ball, group | N")
    if (W is None) == (gate_const is None):
        raise ValueError("give exactly one of W or gate_const")
    perm = np.arange(n) if perm is None else np.asarray(perm, dtype=np.int64)
    qt, kt, vt, dot = q[perm], k[perm], v[perm], do[perm]

    if gate_const is not None:
        G = np.broadcast_to(np.asarray(gate_const, dtype=np.float64), (n, H, 3))
    else:
        G = gates(qt, W, b)
    dqt = np.zeros_like(qt)
    dkt = np.zeros_like(kt)
    dvt = np.zeros_like(vt)
    dG = np.zeros((n, H, 3))

    # ball branch: [nb, H, ball, d] blocks
    nb = n // ball
    split = lambda x: x.reshape(nb, ball, H, d).transpose(0, 2, 1, 3)
    join = lambda x: x.transpose(0, 2, 1, 3).reshape(n, H, d)
    dO0 = G[..., 0:1] * dot
    O, dQ, dK, dV = attn_bwd(split(qt), split(kt), split(vt), split(dO0))
    O = join(O)
    dG[..., 0] = (dot * O).sum(-1)
    dqt += join(dQ)
    dkt += join(dK)
    dvt += join(dV)

    # compression branch: every query against every block mean
    kc, vc = pool_blocks(kt, block), pool_blocks(vt, block)
    th = lambda x: x.transpose(1, 0, 2)                      # [N,H,d] <-> [H,N,d]
    dO1 = G[..., 1:2] * dot
    O, dQ, dKc, dVc = attn_bwd(th(qt), th(kc), th(vc), th(dO1))
    dG[..., 1] = (dot * th(O)).sum(-1)
    dqt += th(dQ)
    dkt += np.repeat(th(dKc), block, axis=0) / block
    dvt += np.repeat(th(dVc), block, axis=0) / block

    # selection branch: each group over the union of its selected blocks
    if sel_override is None:
        sel, _ = select(qt, kc, ball, block, group, topk, mask_own_ball)
    else:
        sel = np.asarray(sel_override)
    dO2 = G[..., 2:3] * dot
    r = np.arange(block)
    for h in range(H):
        for g_ in range(n // group):
            keys = (sel[h, g_][:, None] * block + r[None, :]).reshape(-1)
            rows = slice(g_ * group, (g_ + 1) * group)
            O, dQ, dK, dV = attn_bwd(qt[rows, h], kt[keys, h], vt[keys, h], dO2[rows, h])
            dG[rows, h, 2] = (dot[rows, h] * O).sum(-1)
            dqt[rows, h] += dQ
            np.add.at(dkt[:, h], keys, dK)
            np.add.at(dvt[:, h], keys, dV)

    dW = db = None
    if gate_const is None:
        Wm = np.asarray(W, dtype=np.float64).reshape(3, d)
        dz = dG * G * (1.0 - G)                               # [N,H,3]
        dqt += np.einsum("nhc,cd->nhd", dz, Wm)
        dW = np.einsum("nhc,nhd->cd", dz, qt)
        db = dz.sum(axis=(0, 1))

    res = []
    for g in (dqt, dkt, dvt):
        o = np.empty_like(g)
        o[perm] = g
        res.append(o)
    return res[0], res[1], res[2], dW, db


__all__ = ["bsa_bwd", "attn_bwd"]
