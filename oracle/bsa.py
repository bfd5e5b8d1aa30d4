"""Brute-force Ball Sparse Attention in fp64 (test infrastructure only).

BSA keeps the compression and selection branches of Native Sparse Attention
and replaces its sliding window with Ball Tree Attention; the three branch
outputs are merged by learned sigmoid gates (Pith review of arXiv 2506.12541,
"What carries the argument" and Figure 1 caption; edgentiq blog "The Erwin NSA
Innovation").  Everything below runs in tree order (contiguous ranges of the
ball tree) and the result is scattered back to original order.

Branches, in the pages' order and notation (l = compression block size,
g = group size, k* = selected blocks):

1. ball: scaled dot-product attention inside each ball (see attention.py).
2. compression: K and V are pooled over contiguous blocks of l tree positions
   into coarse tokens K_cmp, V_cmp of length ceil(N/l) (referee report, major
   comment 1, Eqs. 13-15).  Pooling is the plain mean (the Feb-2025 thread on
   Bluesky, post 11/N, "simple mean pooling"; the MLP pooling of Figure 1 needs
   trained weights).  Every full-resolution query attends to all coarse tokens
   (Figure 3 surrounding text: compression attends to all coarse key-value
   representations).
3. selection: query positions form contiguous groups of g; the coarse scores
   of a group are averaged, i.e. the pooled query of the group (Eq. 11, major
   comment 2) scores each coarse key; the k* best blocks are fetched at full
   resolution for the whole group ("What carries the argument"; "Core
   claim").  Blocks inside a ball that holds a position of the group are
   masked so that selection reaches distant regions (Figure 3 surrounding
   text).  Ties in the top-k go to the smaller block index.  Each query of the
   group runs one softmax over the union of the selected keys.
4. gates: G = sigmoid(W q + b) in R^3 per token and head, one W [3, d] shared
   by all heads; out = G0 * O_ball + G1 * O_cmp + G2 * O_slc.  ``gate_const``
   replaces G by a constant triple so that the (1, 0, 0) reduction can be
   tested exactly.

Group (query) compression (``query_compression=True``): queries are pooled
before the compression and selection branches ("Core claim": an optional
coarsening step pools queries before selection and compression; the
compression branch then runs over Q_cmp, K_cmp, V_cmp of length ceil(N/l),
referee report major comment 1 on Eq. 15; the runtime it saves is quoted
under "If this is right").  Reading taken here: the mean query of each block
of l tree positions attends to all coarse tokens and every token of the
block takes that result; the mean query of each group (the one that scores
the blocks) attends once over the union of the group's selected blocks and
every query of the group takes that result.  The ball branch and the gates
stay per token.
"""
from __future__ import annotations

import numpy as np

from .attention import _f64, ball_attn, sdpa, softmax_rows


def own_ball_blocks(gamma: int, group: int, ball: int, block: int):
    """Block indices that overlap a ball holding a position of group gamma."""
    t0, t1 = gamma * group, (gamma + 1) * group          # [t0, t1)
    b0, b1 = t0 // ball, (t1 - 1) // ball                 # balls touched
    lo, hi = b0 * ball, (b1 + 1) * ball                   # their positions
    j0 = lo // block
    j1 = -(-hi // block)                                  # ceil
    return range(j0, j1)


def pool_blocks(x: np.ndarray, block: int) -> np.ndarray:
    """Mean over contiguous blocks of tree positions: [N,H,d] -> [N/l,H,d]."""
    n = x.shape[0]
    return x.reshape(n // block, block, *x.shape[1:]).mean(axis=1)


def group_scores(qt: np.ndarray, kc: np.ndarray, group: int) -> np.ndarray:
    """s[gamma, h, j] = mean_{t in gamma}(q_t) . kc_j / sqrt(d)."""
    n, H, d = qt.shape
    qbar = qt.reshape(n // group, group, H, d).mean(axis=1)      # [G,H,d]
    return np.einsum("ghd,jhd->ghj", qbar, kc) / np.sqrt(d)


def topk_blocks(s: np.ndarray, topk: int, masked) -> np.ndarray:
    """Indices of the top-k scores (descending; ties -> smaller index)."""
    s = s.copy()
    s[list(masked)] = -np.inf
    order = np.lexsort((np.arange(len(s)), -s))
    sel = order[:topk]
    if not np.all(np.isfinite(s[sel])):
        raise ValueError("top-k exceeds the unmasked blocks")
    return sel


def select(qt, kc, ball, block, group, topk, mask_own_ball):
    """Selected blocks per group and head: [H, N/g, k*] (int64)."""
    n, H, _ = qt.shape
    s = group_scores(qt, kc, group)
    G = n // group
    sel = np.empty((H, G, topk), dtype=np.int64)
    for g_ in range(G):
        masked = own_ball_blocks(g_, group, ball, block) if mask_own_ball else ()
        for h in range(H):
            sel[h, g_] = topk_blocks(s[g_, h], topk, masked)
    return sel, s


def selection_attn(qt, kt, vt, sel, block, group) -> np.ndarray:
    """Each query attends once over the union of its group's selected blocks."""
    n, H, d = qt.shape
    out = np.empty_like(qt)
    r = np.arange(block)
    for h in range(H):
        for g_ in range(n // group):
            keys = (sel[h, g_][:, None] * block + r[None, :]).reshape(-1)
            rows = slice(g_ * group, (g_ + 1) * group)
            out[rows, h] = sdpa(qt[rows, h], kt[keys, h], vt[keys, h])
    return out


def compression_attn(qt, kc, vc, chunk: int = 4096) -> np.ndarray:
    n, H, d = qt.shape
    out = np.empty_like(qt)
    kh, vh = kc.transpose(1, 0, 2), vc.transpose(1, 0, 2)     # [H,Nc,d]
    for a in range(0, n, chunk):
        qa = qt[a:a + chunk].transpose(1, 0, 2)              # [H,c,d]
        out[a:a + chunk] = sdpa(qa, kh, vh).transpose(1, 0, 2)
    return out


def pooled_compression_attn(qt, kc, vc, block: int) -> np.ndarray:
    """Group compression: the mean query of each block of l tree positions
    attends to all coarse tokens; every token of the block takes the result."""
    qc = pool_blocks(qt, block)                          # [N/l, H, d]
    return np.repeat(compression_attn(qc, kc, vc), block, axis=0)


def pooled_selection_attn(qt, kt, vt, sel, block, group) -> np.ndarray:
    """Group compression: the mean query of each group attends once over the
    union of the group's selected blocks; every query of the group takes it."""
    n, H, d = qt.shape
    qbar = qt.reshape(n // group, group, H, d).mean(axis=1)   # [G,H,d]
    out = np.empty_like(qt)
    r = np.arange(block)
    for h in range(H):
        for g_ in range(n // group):
            keys = (sel[h, g_][:, None] * block + r[None, :]).reshape(-1)
            o = sdpa(qbar[g_, h][None, :], kt[keys, h], vt[keys, h])[0]
            out[g_ * group:(g_ + 1) * group, h] = o
    return out


def gates(qt: np.ndarray, W, b) -> np.ndarray:
    """sigmoid(W q + b) for every token and head: [N,H,3]."""
    W = np.asarray(W, dtype=np.float64).reshape(3, -1)
    b = np.zeros(3) if b is None else np.asarray(b, dtype=np.float64)
    z = np.einsum("nhd,cd->nhc", qt, W) + b
    return 1.0 / (1.0 + np.exp(-z))


def bsa(q, k, v, perm, ball: int, block: int, group: int, topk: int,
        mask_own_ball: bool = True, W=None, b=None, gate_const=None,
        sel_override=None, return_parts: bool = False, query_compression: bool = False):
    """Three-branch BSA output in original order ([N,H,d], fp64).

    ``sel_override`` ([H, N/g, k*]) replaces the oracle's own top-k choice, so
    that a row whose selection is a numerical near-tie can be recomputed with
    another valid set.  ``query_compression`` pools the queries of the
    compression and selection branches (module docstring).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, H, d = q.shape
    if n % ball or ball % block or n % group:
        raise ValueError("need ball | N, block | ball, group | N")
    if (W is None) == (gate_const is None):
        raise ValueError("give exactly one of W or gate_const")
    perm = np.arange(n) if perm is None else np.asarray(perm, dtype=np.int64)
    qt, kt, vt = q[perm], k[perm], v[perm]

    o_ball = ball_attn(qt, kt, vt, None, ball)
    kc, vc = pool_blocks(kt, block), pool_blocks(vt, block)
    if query_compression:
        o_cmp = pooled_compression_attn(qt, kc, vc, block)
    else:
        o_cmp = compression_attn(qt, kc, vc)
    if sel_override is None:
        sel, scores = select(qt, kc, ball, block, group, topk, mask_own_ball)
    else:
        sel, scores = np.asarray(sel_override), group_scores(qt, kc, group)
    if query_compression:
        o_slc = pooled_selection_attn(qt, kt, vt, sel, block, group)
    else:
        o_slc = selection_attn(qt, kt, vt, sel, block, group)
    if gate_const is not None:
        G = np.broadcast_to(np.asarray(gate_const, dtype=np.float64), (n, H, 3))
    else:
        G = gates(qt, W, b)
    o = G[..., 0:1] * o_ball + G[..., 1:2] * o_cmp + G[..., 2:3] * o_slc
    res = np.empty_like(o)
    res[perm] = o
    if return_parts:
        return res, dict(sel=sel, scores=scores, o_ball=o_ball, o_cmp=o_cmp,
                         o_slc=o_slc, G=G, kc=kc, vc=vc)
    return res


__all__ = ["bsa", "select", "own_ball_blocks", "pool_blocks", "group_scores",
           "topk_blocks", "selection_attn", "compression_attn", "pooled_compression_attn",
           "pooled_selection_attn", "gates", "softmax_rows"]
