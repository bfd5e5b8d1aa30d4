"""Pins of the BSA backward oracle (CPU): central finite differences of the
forward oracle, the reduction to ball attention's backward under constant
gates (1, 0, 0), and the block-constant gradient of the compression branch."""
import numpy as np
import pytest

from oracle import attention_bwd as AB
from oracle import bsa as B
from oracle import bsa_bwd as BB

# a tiny instance in which every branch, the own-ball mask and the gates act
N, H, D = 64, 2, 4
P = dict(ball=16, block=4, group=8, topk=3)


def _inputs(seed):
    rng = np.random.default_rng(seed)
    q, k, v, do = (rng.standard_normal((N, H, D)) for _ in range(4))
    perm = rng.permutation(N)
    W = rng.standard_normal((3, D)) * 0.5
    b = rng.standard_normal(3) * 0.5
    return q, k, v, do, perm, W, b


def _loss(q, k, v, do, perm, W=None, b=None, gate_const=None):
    out, parts = B.bsa(q, k, v, perm, **P, W=W, b=b, gate_const=gate_const,
                       return_parts=True)
    return float((out * do).sum()), parts["sel"]


def _fd_check(x, grad, f, rng, count, eps=1e-6):
    """Central differences of f at `count` random entries of x (in place)."""
    flat = x.reshape(-1)
    gflat = grad.reshape(-1)
    idx = rng.choice(flat.size, size=min(count, flat.size), replace=False)
    base_sel = f()[1]
    worst = 0.0
    for i in idx:
        x0 = flat[i]
        flat[i] = x0 + eps
        lp, sp = f()
        flat[i] = x0 - eps
        lm, sm = f()
        flat[i] = x0
        # a selection that flips under the perturbation has no derivative
        assert np.array_equal(sp, base_sel) and np.array_equal(sm, base_sel)
        fd = (lp - lm) / (2 * eps)
        worst = max(worst, abs(fd - gflat[i]) / max(1.0, abs(fd)))
    return worst


@pytest.mark.parametrize("seed", [0, 1])
def test_bsa_bwd_matches_finite_differences(seed):
    q, k, v, do, perm, W, b = _inputs(seed)
    dq, dk, dv, dW, db = BB.bsa_bwd(q, k, v, do, perm, **P, W=W, b=b)
    rng = np.random.default_rng(100 + seed)
    f = lambda: _loss(q, k, v, do, perm, W=W, b=b)
    for x, g in ((q, dq), (k, dk), (v, dv), (W, dW), (b, db)):
        assert _fd_check(x, g, f, rng, 48) < 1e-6


def test_bsa_bwd_constant_gates_finite_differences():
    q, k, v, do, perm, _, _ = _inputs(2)
    gc = (0.3, 0.5, 0.7)
    dq, dk, dv, dW, db = BB.bsa_bwd(q, k, v, do, perm, **P, gate_const=gc)
    assert dW is None and db is None
    rng = np.random.default_rng(7)
    f = lambda: _loss(q, k, v, do, perm, gate_const=gc)
    for x, g in ((q, dq), (k, dk), (v, dv)):
        assert _fd_check(x, g, f, rng, 48) < 1e-6


def test_bsa_bwd_reduces_to_ball_attention_bwd():
    """Gates (1, 0, 0): BSA is ball attention, so are its gradients."""
    q, k, v, do, perm, _, _ = _inputs(3)
    dq, dk, dv, _, _ = BB.bsa_bwd(q, k, v, do, perm, **P, gate_const=(1.0, 0.0, 0.0))
    rq, rk, rv = AB.ball_attn_bwd(q, k, v, do, perm, P["ball"])
    for a, r in ((dq, rq), (dk, rk), (dv, rv)):
        np.testing.assert_allclose(a, r, rtol=0, atol=1e-12)


def test_bsa_bwd_compression_gradient_is_block_constant():
    """Gates (0, 1, 0): k and v reach the output only through block means,
    so every token of a block gets the same dk and dv (tree order)."""
    q, k, v, do, perm, _, _ = _inputs(4)
    _, dk, dv, _, _ = BB.bsa_bwd(q, k, v, do, perm, **P, gate_const=(0.0, 1.0, 0.0))
    l = P["block"]
    for g in (dk, dv):
        gt = g[perm].reshape(N // l, l, H, D)
        np.testing.assert_allclose(gt, np.broadcast_to(gt[:, :1], gt.shape), rtol=0, atol=1e-12)
