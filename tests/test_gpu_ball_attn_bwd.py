"""GPU parity of ball_attn_bwd against the fp64 backward oracle (through the
C ABI)."""
import numpy as np
import pytest

from ball_tree_sparse_amd import ops, synth
from oracle import attention_bwd as AB
from tests.helpers import gpu, max_abs, say

pytestmark = pytest.mark.gpu

import torch  # noqa: E402

TOL = {"bf16": 2e-2, "f32": 1e-5}   # fp32: measured max abs errors 0.4-1.2e-6


@pytest.mark.parametrize("n,H,d,ball,dtype", [
    (1024, 4, 16, 32, "f32"),
    (2048, 2, 32, 128, "f32"),
    (1536, 3, 32, 96, "f32"),       # ball not a power of two
    (1024, 1, 16, 1024, "f32"),     # the largest ball the backward takes
    (512, 2, 64, 64, "f32"),
    (4096, 8, 32, 128, "bf16"),     # MFMA kernel from here on ...
    (1024, 4, 32, 32, "bf16"),
    (1536, 2, 32, 64, "bf16"),
    (2048, 2, 64, 64, "bf16"),
    (1024, 3, 64, 32, "bf16"),
    (4096, 2, 64, 128, "bf16"),
    (4096, 2, 32, 256, "bf16"),
    (2048, 2, 64, 256, "bf16"),
    (2048, 2, 32, 512, "bf16"),     # ... VALU kernel again (ball above 256)
    (1024, 2, 16, 64, "bf16"),      # d = 16: VALU kernel
])
def test_parity(n, H, d, ball, dtype):
    dev = gpu()
    rng = np.random.default_rng(n + H + d + ball)
    q, k, v, do = (synth.normal_features(rng, n, H, d, dtype) for _ in range(4))
    perm = rng.permutation(n)
    say("ball_attn_bwd", n, H, d, ball, dtype)
    pd = torch.from_numpy(perm.astype(np.int32)).to(dev)
    g = ops.ball_attn_bwd(q.to(dev), k.to(dev), v.to(dev), do.to(dev), pd, ball)
    torch.cuda.synchronize()
    want = AB.ball_attn_bwd(q, k, v, do, perm, ball)
    for name, a, b in zip("qkv", g, want):
        err = max_abs(a.cpu(), b)
        assert err <= TOL[dtype], (name, err)


def test_tree_order_no_perm():
    dev = gpu()
    rng = np.random.default_rng(3)
    q, k, v, do = (synth.normal_features(rng, 2048, 2, 32, "f32") for _ in range(4))
    say("ball_attn_bwd perm=None")
    g = ops.ball_attn_bwd(q.to(dev), k.to(dev), v.to(dev), do.to(dev), None, 64)
    torch.cuda.synchronize()
    for a, b in zip(g, AB.ball_attn_bwd(q, k, v, do, None, 64)):
        assert max_abs(a.cpu(), b) <= TOL["f32"]


def test_tree_order_no_perm_bf16():
    dev = gpu()
    rng = np.random.default_rng(4)
    q, k, v, do = (synth.normal_features(rng, 2048, 2, 32, "bf16") for _ in range(4))
    say("ball_attn_bwd bf16 perm=None")
    g = ops.ball_attn_bwd(q.to(dev), k.to(dev), v.to(dev), do.to(dev), None, 128)
    torch.cuda.synchronize()
    for a, b in zip(g, AB.ball_attn_bwd(q, k, v, do, None, 128)):
        assert max_abs(a.cpu(), b) <= TOL["bf16"]


def test_full_size_sphere():
    """The 65,536-point sphere shape (ball 128, 8 heads, d 32, bf16) with a
    random permutation, every output checked."""
    dev = gpu()
    w = synth.make("sphere")
    do = synth.normal_features(np.random.default_rng(8), w.coords.shape[0], w.H, w.d, "bf16")
    perm = np.random.default_rng(7).permutation(w.coords.shape[0])
    say("ball_attn_bwd sphere", w.coords.shape[0], w.H, w.d, w.ball)
    pd = torch.from_numpy(perm.astype(np.int32)).to(dev)
    g = ops.ball_attn_bwd(w.q.to(dev), w.k.to(dev), w.v.to(dev), do.to(dev), pd, w.ball)
    torch.cuda.synchronize()
    want = AB.ball_attn_bwd(w.q, w.k, w.v, do, perm, w.ball)
    for name, a, b in zip("qkv", g, want):
        assert max_abs(a.cpu(), b) <= TOL["bf16"], name
