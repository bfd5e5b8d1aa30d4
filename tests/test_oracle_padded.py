"""Pins of the uneven-N oracle (padded tree and padded ball attention)."""
import json
import os

import numpy as np
import pytest

from ball_tree_sparse_amd import synth
from oracle import attention as A
from oracle import checks as C
from oracle import tree as T

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_derived_padded_trees():
    g = json.load(open(os.path.join(GOLD, "tree_hand_padded.json")))
    for case in g["cases"]:
        got = T.build_padded(np.array(case["coords"], np.float32), case["leaf"])
        assert got.tolist() == case["perm"], case


@pytest.mark.parametrize("n,leaf", [(1, 1), (1, 4), (2, 1), (5, 2), (972, 32), (1000, 16),
                                    (3586, 128), (4095, 64)])
def test_padded_tree_invariants(n, leaf):
    rng = np.random.default_rng(n + leaf)
    c = synth.uniform_cube(rng, n)
    p = T.build_padded(c, leaf)
    assert len(p) == T.padded_size(n, leaf)
    ok, msg = C.check_padded_tree(c, p, leaf)
    assert ok, msg
    # leaf counts: floor or ceil of N over the number of leaves
    cnt = (p.reshape(-1, leaf) >= 0).sum(1)
    nl = len(p) // leaf
    assert set(cnt.tolist()) <= {n // nl, -(-n // nl)} and cnt.sum() == n


def test_padded_equals_plain_tree_when_n_fits():
    rng = np.random.default_rng(4)
    c = synth.gaussian_mixture(rng, 2048, k=8)
    assert np.array_equal(T.build_padded(c, 64), T.build(c, 64))
    R = synth.random_rotation(rng)
    assert np.array_equal(T.rotate_build_padded(c, 64, R), T.rotate_build(c, 64, R))


def test_padded_checker_catches_planted_mistakes():
    rng = np.random.default_rng(6)
    c = synth.uniform_cube(rng, 300)
    p = T.build_padded(c, 16)
    bad = p.copy()                       # a point moved behind the padding of its leaf
    j = int(np.argmax(bad.reshape(-1, 16)[:, -1] < 0)) * 16
    m = int((bad[j:j + 16] >= 0).sum())
    bad[j + m], bad[j] = bad[j], -1
    assert not C.check_padded_tree(c, bad, 16)[0]
    bad = p.copy()                       # two points swapped across the root split
    half = len(p) // 2
    a, b = 0, half
    bad[a], bad[b] = bad[b], bad[a]
    assert not C.check_padded_tree(c, bad, 16)[0]


def test_padded_attention_without_padding_is_ball_attention():
    rng = np.random.default_rng(7)
    q, k, v = (synth.normal_features(rng, 256, 2, 16, "f32") for _ in range(3))
    perm = rng.permutation(256)
    assert np.allclose(A.ball_attn_padded(q, k, v, perm, 32), A.ball_attn(q, k, v, perm, 32),
                       rtol=0, atol=1e-12)


def test_padded_attention_closed_forms():
    rng = np.random.default_rng(8)
    n, H, d = 5, 3, 8
    q, k, v = (rng.standard_normal((n, H, d)) for _ in range(3))
    k[3] = k[2]                          # 2 and 3 share a ball and have equal keys
    perm = np.array([0, -1, -1, -1, 2, 3, -1, -1, 1, 4, -1, -1], np.int64)   # ball 4
    out = A.ball_attn_padded(q, k, v, perm, 4)
    assert np.array_equal(out[0], v[0])                     # alone: its own value
    assert np.allclose(out[2], (v[2] + v[3]) / 2, atol=1e-14)   # equal logits: the mean
    assert np.allclose(out[3], (v[2] + v[3]) / 2, atol=1e-14)
    # two points: weights are the logistic function of the logit difference
    s = np.einsum("hd,hd->h", q[1], k[4] - k[1]) / np.sqrt(d)
    w4 = 1 / (1 + np.exp(-s))
    assert np.allclose(out[1], (1 - w4)[:, None] * v[1] + w4[:, None] * v[4], atol=1e-13)


def test_padded_attention_ignores_slot_order_inside_a_ball():
    rng = np.random.default_rng(9)
    n = 200
    q, k, v = (synth.normal_features(rng, n, 2, 16, "f32") for _ in range(3))
    c = synth.uniform_cube(rng, n)
    p = T.build_padded(c, 32)                      # 256 slots
    out = A.ball_attn_padded(q, k, v, p, 64)
    p2 = p.reshape(-1, 64).copy()
    for row in p2:
        rng.shuffle(row)
    assert np.allclose(A.ball_attn_padded(q, k, v, p2.reshape(-1), 64), out, atol=1e-13)
