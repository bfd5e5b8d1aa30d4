"""GPU parity of bt_coarsen / bt_refine against the fp64 oracle (through
the C ABI), and one U-Net level: coarsen, ball attention at the coarse
level, refine."""
import numpy as np
import pytest
import torch

from ball_tree_sparse_amd import ops, synth
from oracle import attention as A
from oracle import pool as P
from oracle import tree as T
from tests.helpers import gpu, max_abs, say

pytestmark = pytest.mark.gpu


def _feats(n, H, d, dtype, seed):
    return synth.normal_features(np.random.default_rng(seed), n, H, d, dtype)


@pytest.mark.parametrize("n,H,d,s,dtype,use_perm", [
    (4096, 8, 32, 2, "bf16", True),
    (4096, 8, 32, 8, "bf16", False),
    (8192, 4, 16, 64, "f32", True),
    (1000, 2, 64, 8, "bf16", True),       # ragged N (not a power of two)
    (2048, 1, 16, 2048, "f32", True),     # s = N: one parent
    (512, 3, 32, 1, "bf16", True),        # s = 1: the gather
])
def test_coarsen_parity(n, H, d, s, dtype, use_perm):
    dev = gpu()
    x = _feats(n, H, d, dtype, seed=n + s)
    perm = np.random.default_rng(s).permutation(n) if use_perm else None
    say("coarsen", n, H, d, s, dtype, use_perm)
    pd = None if perm is None else torch.from_numpy(perm.astype(np.int32)).to(dev)
    got = ops.bt_coarsen(x.to(dev), pd, s)
    torch.cuda.synchronize()
    want = P.coarsen(x, perm, s)
    # bf16: the fp32 mean rounded once (half a bf16 unit of |mean| <= 4)
    tol = 1e-5 if dtype == "f32" else 2 ** -8 * 4
    assert max_abs(got.cpu(), want) <= tol


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_refine_bit_exact(dtype):
    dev = gpu()
    n, H, d, s = 4096, 4, 32, 16
    xc = _feats(n // s, H, d, dtype, seed=3)
    perm = np.random.default_rng(4).permutation(n)
    say("refine", dtype)
    got = ops.bt_refine(xc.to(dev), torch.from_numpy(perm.astype(np.int32)).to(dev), s)
    torch.cuda.synchronize()
    want = P.refine(xc.float().numpy() if dtype == "bf16" else xc.numpy(), perm, s)
    assert np.array_equal(got.float().cpu().numpy(), want.astype(np.float32))


def test_unet_level_round_trip():
    """Coarsen a real tree's features by 8 (leaves of 8 points), run ball
    attention at the coarse level (ball 32, tree order), refine back."""
    dev = gpu()
    rng = np.random.default_rng(9)
    n, H, d = 8192, 4, 32
    c = synth.deformed_sphere(rng, n)
    q, k, v = (synth.normal_features(rng, n, H, d, "bf16") for _ in range(3))
    perm = T.build(c, 8)
    pd = torch.from_numpy(perm.astype(np.int32)).to(dev)
    say("U-Net level")
    qc, kc, vc = (ops.bt_coarsen(t.to(dev), pd, 8) for t in (q, k, v))
    oc = ops.ball_attn(qc, kc, vc, None, 32)
    out = ops.bt_refine(oc, pd, 8)
    torch.cuda.synchronize()
    # coarse inputs: within bf16 rounding of the oracle's means
    for g_, x in ((qc, q), (kc, k), (vc, v)):
        assert max_abs(g_.cpu(), P.coarsen(x, perm, 8)) <= 2 ** -8 * 4
    # attention at the coarse level on the GPU's coarse tensors, then refine
    want = P.refine(A.ball_attn(qc.cpu(), kc.cpu(), vc.cpu(), None, 32), perm, 8)
    assert max_abs(out.cpu(), want) <= 2e-2
