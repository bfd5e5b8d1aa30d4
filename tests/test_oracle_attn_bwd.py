"""Pins for the ball-attention backward oracle: torch autograd through the
library SDPA in fp64 (an independent routine), central finite differences,
and the ball = N reduction."""
import numpy as np
import torch

from oracle import attention as A
from oracle import attention_bwd as AB


def _data(n, H, d, seed):
    g = np.random.default_rng(seed)
    return [g.standard_normal((n, H, d)) for _ in range(4)] + [g.permutation(n)]


def _autograd(q, k, v, do, perm, ball):
    n, H, d = q.shape
    t = lambda x: torch.tensor(x[perm], dtype=torch.float64, requires_grad=True)
    Q, K, V = t(q), t(k), t(v)
    sh = lambda x: x.reshape(n // ball, ball, H, d).transpose(1, 2)
    O = torch.nn.functional.scaled_dot_product_attention(sh(Q), sh(K), sh(V))
    O = O.transpose(1, 2).reshape(n, H, d)
    O.backward(torch.tensor(do[perm], dtype=torch.float64))
    res = []
    for g in (Q.grad, K.grad, V.grad):
        o = np.empty((n, H, d))
        o[perm] = g.numpy()
        res.append(o)
    return res


def test_matches_autograd_of_library_sdpa():
    q, k, v, do, perm = _data(256, 2, 16, 0)
    got = AB.ball_attn_bwd(q, k, v, do, perm, 32)
    want = _autograd(q, k, v, do, perm, 32)
    for a, b in zip(got, want):
        assert np.allclose(a, b, atol=1e-12, rtol=0)


def test_finite_differences():
    q, k, v, do, perm = _data(16, 1, 4, 1)
    ball, eps = 8, 1e-6
    dq, dk, dv = AB.ball_attn_bwd(q, k, v, do, perm, ball)
    f = lambda q_, k_, v_: float((A.ball_attn(q_, k_, v_, perm, ball) * do).sum())
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in [(0, 0, 0), (5, 0, 3), (11, 0, 1), (15, 0, 2)]:
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": (q, k, v), "k": (q, k, v), "v": (q, k, v)}[name]
            ap = [xp if a is x else a for a in args]
            am = [xm if a is x else a for a in args]
            num = (f(*ap) - f(*am)) / (2 * eps)
            assert abs(num - g[idx]) < 1e-7, (name, idx, num, g[idx])


def test_v_gradient_of_uniform_attention():
    """q = 0: every query attends uniformly, so dV_j is the mean of dO over the
    ball, and dK = dS^T Q vanishes."""
    q, k, v, do, perm = _data(64, 1, 8, 2)
    q = np.zeros_like(q)
    dq, dk, dv = AB.ball_attn_bwd(q, k, v, do, None, 64)
    assert np.allclose(dv, np.broadcast_to(do.mean(axis=0), dv.shape), atol=1e-13, rtol=0)
    assert np.allclose(dk, 0.0, atol=1e-13)        # dK = dS^T Q = 0
