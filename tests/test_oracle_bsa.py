"""Pins for the BSA oracle: reductions to ball / full / pooled attention
(library routines), closed forms for zero queries, a hand-derived selection
golden case, the gate formula, and planted mistakes."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import bsa as B

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand(n, H, d, seed):
    g = np.random.default_rng(seed)
    return [g.standard_normal((n, H, d)) for _ in range(3)]


def _sdpa_t(q, k, v):
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x.transpose(1, 0, 2)))
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v)).numpy().transpose(1, 0, 2)


N, H, D = 512, 2, 16
BALL, BLK, GRP, TOPK = 64, 16, 32, 4


@pytest.fixture(scope="module")
def data():
    q, k, v = _rand(N, H, D, 0)
    perm = np.random.default_rng(1).permutation(N)
    return q, k, v, perm


def test_gates_100_is_ball_attention(data):
    q, k, v, perm = data
    o = B.bsa(q, k, v, perm, BALL, BLK, GRP, TOPK, gate_const=(1, 0, 0))
    np.testing.assert_allclose(o, A.ball_attn(q, k, v, perm, BALL), atol=1e-12)


def test_gates_010_is_sdpa_over_pooled(data):
    q, k, v, perm = data
    o = B.bsa(q, k, v, perm, BALL, BLK, GRP, TOPK, gate_const=(0, 1, 0))
    pool = lambda x: torch.nn.functional.avg_pool1d(
        torch.from_numpy(x[perm].reshape(N, -1).T.copy())[None], BLK, BLK
    )[0].T.numpy().reshape(N // BLK, H, D)
    ref_t = _sdpa_t(q[perm], pool(k), pool(v))
    ref = np.empty_like(ref_t); ref[perm] = ref_t
    np.testing.assert_allclose(o, ref, atol=1e-12)


def test_block_one_compression_is_full_attention(data):
    q, k, v, perm = data
    o = B.bsa(q, k, v, perm, BALL, 1, GRP, TOPK, gate_const=(0, 1, 0))
    np.testing.assert_allclose(o, _sdpa_t(q, k, v), atol=1e-12)


def test_selection_of_all_blocks_is_full_attention(data):
    q, k, v, perm = data
    o = B.bsa(q, k, v, perm, BALL, BLK, GRP, N // BLK, mask_own_ball=False,
              gate_const=(0, 0, 1))
    np.testing.assert_allclose(o, _sdpa_t(q, k, v), atol=1e-12)


def test_zero_queries_closed_form(data):
    _, k, v, perm = data
    q = np.zeros_like(k)
    o, parts = B.bsa(q, k, v, perm, BALL, BLK, GRP, TOPK, gate_const=(0, 1, 0),
                     return_parts=True)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=0), v.shape), atol=1e-12)
    # every selection score is 0 -> the lowest-index unmasked blocks win
    sel = parts["sel"]
    per_ball = BALL // BLK
    for g in range(N // GRP):
        b = (g * GRP) // BALL
        masked = set(range(b * per_ball, (b + 1) * per_ball))
        want = [j for j in range(N // BLK) if j not in masked][:TOPK]
        assert sel[0, g].tolist() == want
    o2 = B.bsa(q, k, v, perm, BALL, BLK, GRP, TOPK, gate_const=(0, 0, 1))
    vt = v[perm]
    g0 = sel[0, 0]
    rows = (g0[:, None] * BLK + np.arange(BLK)).ravel()
    np.testing.assert_allclose(o2[perm[0]], vt[rows].mean(axis=0), atol=1e-12)


def test_golden_selection():
    with open(os.path.join(GOLD, "bsa_hand_select.json")) as f:
        g = json.load(f)
    q, k = np.array(g["q"]), np.array(g["k"])
    kc = B.pool_blocks(k, g["block"])
    sel, _ = B.select(q, kc, g["ball"], g["block"], g["group"], g["topk"], True)
    assert sel.tolist() == g["sel"]


def test_own_ball_blocks():
    assert list(B.own_ball_blocks(0, 64, 128, 64)) == [0, 1]
    assert list(B.own_ball_blocks(1, 64, 128, 64)) == [0, 1]
    assert list(B.own_ball_blocks(2, 64, 128, 64)) == [2, 3]
    assert list(B.own_ball_blocks(1, 256, 128, 64)) == [4, 5, 6, 7]   # g > ball


def test_pooled_query_equals_mean_of_logits(data):
    q, k, v, perm = data
    kc = B.pool_blocks(k[perm], BLK)
    s = B.group_scores(q[perm], kc, GRP)
    qt = q[perm]
    logits = np.einsum("nhd,jhd->nhj", qt, kc) / np.sqrt(D)
    mean_logits = logits.reshape(N // GRP, GRP, H, -1).mean(axis=1)
    np.testing.assert_allclose(s, mean_logits, atol=1e-12)


def test_gate_formula(data):
    q, *_ = data
    W = np.random.default_rng(3).standard_normal((3, D)) * 0.02
    b = np.array([0.1, -0.2, 0.3])
    G = B.gates(q, W, b)
    ref = torch.sigmoid(torch.nn.functional.linear(
        torch.from_numpy(q), torch.from_numpy(W), torch.from_numpy(b))).numpy()
    np.testing.assert_allclose(G, ref, atol=1e-14)


def test_gated_merge_is_linear(data):
    q, k, v, perm = data
    W = np.random.default_rng(4).standard_normal((3, D)) * 0.02
    o, parts = B.bsa(q, k, v, perm, BALL, BLK, GRP, TOPK, W=W, return_parts=True)
    G = parts["G"]
    want_t = (G[..., :1] * parts["o_ball"] + G[..., 1:2] * parts["o_cmp"]
              + G[..., 2:] * parts["o_slc"])
    want = np.empty_like(want_t); want[perm] = want_t
    np.testing.assert_allclose(o, want, atol=1e-14)


def test_selection_blocks_exclude_own_ball(data):
    q, k, v, perm = data
    _, parts = B.bsa(q, k, v, perm, BALL, BLK, GRP, TOPK, gate_const=(0, 0, 1),
                     return_parts=True)
    for g in range(N // GRP):
        own = set(B.own_ball_blocks(g, GRP, BALL, BLK))
        assert not (set(parts["sel"][0, g].tolist()) & own)


def test_mutation_per_block_softmax_is_caught(data, monkeypatch):
    """A planted mistake: one softmax per selected block instead of one over
    the union.  The full-attention reduction must catch it."""
    q, k, v, perm = data

    def bad(qt, kt, vt, sel, block, group):
        n, H_, d = qt.shape
        out = np.zeros_like(qt)
        for h in range(H_):
            for g_ in range(n // group):
                rows = slice(g_ * group, (g_ + 1) * group)
                for j in sel[h, g_]:
                    ks = slice(j * block, (j + 1) * block)
                    out[rows, h] += A.sdpa(qt[rows, h], kt[ks, h], vt[ks, h])
                out[rows, h] /= len(sel[h, g_])
        return out
    monkeypatch.setattr(B, "selection_attn", bad)
    o = B.bsa(q, k, v, perm, BALL, BLK, GRP, N // BLK, mask_own_ball=False,
              gate_const=(0, 0, 1))
    assert not np.allclose(o, _sdpa_t(q, k, v), atol=1e-6)


def test_mutation_unmasked_is_caught(data):
    q, k, v, perm = data
    _, parts = B.bsa(q, k, v, perm, BALL, BLK, GRP, TOPK, mask_own_ball=False,
                     gate_const=(0, 0, 1), return_parts=True)
    hit = 0
    for g in range(N // GRP):
        own = set(B.own_ball_blocks(g, GRP, BALL, BLK))
        hit += bool(set(parts["sel"][0, g].tolist()) & own)
    assert hit > 0        # without the mask the own ball is usually selected


# ---- group (query) compression ------------------------------------------

def _tree_const_queries(q, perm, span, seed):
    """q whose tree-ordered rows are constant over each run of `span`."""
    n, H, d = q.shape
    runs = np.random.default_rng(seed).standard_normal((n // span, H, d))
    qt = np.repeat(runs, span, axis=0)
    out = np.empty_like(qt)
    out[perm] = qt
    return out


def test_query_compression_equals_bsa_for_constant_queries(data):
    """With every block and group holding one query, pooling changes nothing."""
    _, k, v, perm = data
    q = _tree_const_queries(data[0], perm, max(BLK, GRP), seed=5)
    W = 0.3 * np.random.default_rng(6).standard_normal((3, D))
    a = B.bsa(q, k, v, perm, BALL, BLK, GRP, TOPK, True, W=W, query_compression=True)
    b = B.bsa(q, k, v, perm, BALL, BLK, GRP, TOPK, True, W=W)
    assert np.allclose(a, b, atol=1e-12, rtol=0)


def test_query_compression_pools_compression_by_block(data):
    """Queries constant over blocks of l but not over groups: the compression
    part equals the per-token one, the selection part does not; pooling the
    compression queries over the group instead is caught."""
    _, k, v, perm = data
    assert GRP > BLK
    q = _tree_const_queries(data[0], perm, BLK, seed=7)
    gc = (0.0, 1.0, 0.0)
    _, pq = B.bsa(q, k, v, perm, BALL, BLK, GRP, TOPK, True, gate_const=gc,
                  query_compression=True, return_parts=True)
    _, ps = B.bsa(q, k, v, perm, BALL, BLK, GRP, TOPK, True, gate_const=gc, return_parts=True)
    assert np.allclose(pq["o_cmp"], ps["o_cmp"], atol=1e-12, rtol=0)
    assert not np.allclose(pq["o_slc"], ps["o_slc"], atol=1e-6)
    qt = np.asarray(q)[perm]
    wrong = np.repeat(B.compression_attn(B.pool_blocks(qt, GRP), pq["kc"], pq["vc"]), GRP, axis=0)
    assert not np.allclose(wrong, ps["o_cmp"], atol=1e-6)


def test_query_compression_selection_is_group_mean_query(data):
    """Each group's selection output is the attention of its mean query over
    the selected keys (written out with the library SDPA), shared by the group."""
    q, k, v, perm = data
    _, p = B.bsa(q, k, v, perm, BALL, BLK, GRP, TOPK, True, gate_const=(0, 0, 1),
                 query_compression=True, return_parts=True)
    qt, kt, vt = q[perm], k[perm], v[perm]
    for h in range(H):
        for g_ in (0, N // GRP - 1):
            rows = slice(g_ * GRP, (g_ + 1) * GRP)
            keys = (p["sel"][h, g_][:, None] * BLK + np.arange(BLK)[None, :]).reshape(-1)
            qb = qt[rows, h].mean(axis=0)
            t = lambda x: torch.from_numpy(np.ascontiguousarray(x))
            want = torch.nn.functional.scaled_dot_product_attention(
                t(qb[None, None, :]), t(kt[keys, h][None]), t(vt[keys, h][None])).numpy()[0, 0]
            assert np.allclose(p["o_slc"][rows, h], want[None, :], atol=1e-12, rtol=0)


def test_query_compression_single_block_is_global_mean(data):
    """ball = block = N: one coarse token, so compression gives every token the
    mean of V (closed form)."""
    q, k, v, perm = data
    out = B.bsa(q, k, v, perm, N, N, GRP, 1, False, gate_const=(0, 1, 0), query_compression=True)
    assert np.allclose(out, np.broadcast_to(v.mean(axis=0), v.shape), atol=1e-12, rtol=0)
