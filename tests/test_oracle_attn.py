"""Pins for the ball-attention oracle: a hand-computed golden case, library
routines (torch SDPA in fp64 on the CPU), closed forms and mutations."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import attention as A

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand(n, H, d, seed):
    g = np.random.default_rng(seed)
    return [g.standard_normal((n, H, d)) for _ in range(3)]


def _torch_sdpa(q, k, v, mask=None):
    """torch's SDPA in fp64 over [N,H,d] inputs (heads as batch)."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x.transpose(1, 0, 2)))
    o = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=mask)
    return o.numpy().transpose(1, 0, 2)


def test_golden_hand():
    with open(os.path.join(GOLD, "attn_hand.json")) as f:
        g = json.load(f)
    out = A.ball_attn(np.array(g["q"]), np.array(g["k"]), np.array(g["v"]),
                      np.array(g["perm"]), g["ball"])
    np.testing.assert_allclose(out, np.array(g["out"]), rtol=0, atol=1e-12)


def test_ball_equals_N_is_full_attention():
    q, k, v = _rand(256, 3, 16, 0)
    perm = np.random.default_rng(1).permutation(256)
    out = A.ball_attn(q, k, v, perm, 256)
    np.testing.assert_allclose(out, _torch_sdpa(q, k, v), atol=1e-12)
    np.testing.assert_allclose(A.full_attn(q, k, v), _torch_sdpa(q, k, v), atol=1e-12)


def test_block_diagonal_mask_equivalence():
    """Ball attention in tree order == SDPA with a block-diagonal mask."""
    n, ball = 512, 64
    q, k, v = _rand(n, 2, 32, 2)
    perm = np.random.default_rng(3).permutation(n)
    out = A.ball_attn(q, k, v, perm, ball)
    qt, kt, vt = q[perm], k[perm], v[perm]
    blk = np.arange(n) // ball
    mask = torch.from_numpy(blk[:, None] == blk[None, :])
    ref_t = _torch_sdpa(qt, kt, vt, mask)
    ref = np.empty_like(ref_t)
    ref[perm] = ref_t
    np.testing.assert_allclose(out, ref, atol=1e-12)


def test_ball_one_returns_v():
    q, k, v = _rand(64, 2, 8, 4)
    np.testing.assert_allclose(A.ball_attn(q, k, v, None, 1), v, atol=0)


def test_zero_query_is_ball_mean():
    q, k, v = _rand(128, 2, 8, 5)
    q[:] = 0
    perm = np.random.default_rng(6).permutation(128)
    out = A.ball_attn(q, k, v, perm, 32)
    vt = v[perm].reshape(4, 32, 2, 8).mean(axis=1)          # [balls,H,d]
    want_t = np.repeat(vt, 32, axis=0)
    want = np.empty_like(want_t)
    want[perm] = want_t
    np.testing.assert_allclose(out, want, atol=1e-12)


def test_constant_v_per_ball():
    q, k, v = _rand(128, 1, 4, 7)
    vt = np.repeat(np.arange(4.0)[:, None, None] * np.ones((1, 1, 4)), 32, axis=0)
    out = A.ball_attn(q, k, vt, None, 32)
    np.testing.assert_allclose(out, vt, atol=1e-12)


def test_equivariance_within_ball():
    q, k, v = _rand(128, 2, 8, 8)
    perm = np.arange(128)
    sh = perm.copy()
    sh[32:64] = np.random.default_rng(9).permutation(np.arange(32, 64))
    a = A.ball_attn(q, k, v, perm, 32)
    b = A.ball_attn(q, k, v, sh, 32)
    np.testing.assert_allclose(a, b, atol=1e-12)


def test_rows_helper_matches():
    q, k, v = _rand(256, 2, 16, 10)
    perm = np.random.default_rng(11).permutation(256)
    full = A.ball_attn(q, k, v, perm, 64)
    rows = np.array([0, 5, 63, 64, 200, 255])
    part = A.ball_attn_rows(q, k, v, perm, 64, rows)
    np.testing.assert_allclose(part, full[perm[rows]], atol=1e-12)


def test_bf16_inputs_upcast_exactly():
    x = torch.randn(64, 2, 8).to(torch.bfloat16)
    y = A._f64(x)
    assert y.dtype == np.float64
    assert np.array_equal(y, x.float().numpy().astype(np.float64))


def test_mutation_missing_scale_is_caught(monkeypatch):
    def bad(q, k, v):
        return A.softmax_rows(q @ np.swapaxes(k, -1, -2)) @ v
    monkeypatch.setattr(A, "sdpa", bad)
    q, k, v = _rand(128, 2, 16, 12)
    with pytest.raises(AssertionError):
        np.testing.assert_allclose(A.ball_attn(q, k, v, None, 128),
                                   _torch_sdpa(q, k, v), atol=1e-9)


def test_mutation_scatter_instead_of_gather_is_caught(monkeypatch):
    q, k, v = _rand(128, 1, 8, 13)
    perm = np.random.default_rng(14).permutation(128)
    inv = np.argsort(perm)
    good = A.ball_attn(q, k, v, perm, 32)
    bad = A.ball_attn(q, k, v, inv, 32)                    # wrong direction
    ref_t = _torch_sdpa(q[perm], k[perm], v[perm],
                        torch.from_numpy((np.arange(128)[:, None] // 32) ==
                                         (np.arange(128)[None, :] // 32)))
    ref = np.empty_like(ref_t); ref[perm] = ref_t
    np.testing.assert_allclose(good, ref, atol=1e-12)
    assert not np.allclose(bad, ref, atol=1e-6)
