"""GPU parity of the uneven-N path (padded tree, padded permute, padded ball
attention) against the oracle, through the C ABI."""
import numpy as np
import pytest

from ball_tree_sparse_amd import ops, synth
from oracle import attention as A
from oracle import permute as P
from oracle import checks as CK
from oracle import tree as T
from tests.helpers import gpu, max_abs, say

pytestmark = pytest.mark.gpu

import torch  # noqa: E402


@pytest.mark.parametrize("n,leaf", [(972, 32), (1000, 16), (513, 64), (5, 2), (3, 1), (1, 1),
                                    (700, 700), (1024, 32), (129, 1), (4000, 4096),
                                    # one-workgroup LDS builder (1,025-8,192 slots)
                                    (3586, 32), (5000, 64), (1025, 1), (6001, 3), (8192, 64),
                                    (2049, 2048),
                                    # streamed splits above 8,192 slots
                                    (9000, 64), (12289, 3), (16385, 128), (20000, 8192),
                                    (65000, 128)])
def test_padded_tree_bit_exact(n, leaf):
    dev = gpu()
    rng = np.random.default_rng(n * 7 + leaf)
    c = synth.uniform_cube(rng, n)
    say("bt_build_padded", n, leaf)
    p = ops.bt_build_padded(torch.from_numpy(c).to(dev), leaf)
    torch.cuda.synchronize()
    got = p.cpu().numpy()
    assert np.array_equal(got, T.build_padded(c, leaf))
    assert CK.check_padded_tree(c, got, leaf)[0]


def test_padded_tree_equals_plain_tree_when_n_fits():
    dev = gpu()
    c = synth.uniform_cube(np.random.default_rng(3), 1024)
    cd = torch.from_numpy(c).to(dev)
    say("bt_build_padded vs bt_build 1024")
    a = ops.bt_build_padded(cd, 32)
    b = ops.bt_build(cd, 32)
    torch.cuda.synchronize()
    assert torch.equal(a.cpu(), b.cpu())


def test_padded_tree_rotated_and_ties():
    dev = gpu()
    rng = np.random.default_rng(12)
    c = rng.integers(-1, 2, size=(900, 3)).astype(np.float32)
    c[rng.random(c.shape) < 0.5] *= -1.0
    R = synth.random_rotation(rng)
    w = synth.uniform_cube(rng, 600)
    say("bt_build_padded ties / rotated")
    p1 = ops.bt_build_padded(torch.from_numpy(c).to(dev), 8)
    p2 = ops.bt_build_padded(torch.from_numpy(w).to(dev), 16, R=R)
    torch.cuda.synchronize()
    assert np.array_equal(p1.cpu().numpy(), T.build_padded(c, 8))
    assert np.array_equal(p2.cpu().numpy(), T.rotate_build_padded(w, 16, R))


@pytest.mark.parametrize("n,shape,dtype", [(972, (8, 32), torch.bfloat16),
                                           (3586, (3,), torch.float32),
                                           (5000, (5, 7), torch.float32)])
def test_permute_padded(n, shape, dtype):
    dev = gpu()
    rng = np.random.default_rng(n)
    slots = T.padded_size(n, 64)
    perm = np.full(slots, -1, np.int32)
    perm[np.sort(rng.choice(slots, n, replace=False))] = rng.permutation(n)
    x = torch.from_numpy(rng.standard_normal((n,) + shape).astype(np.float32)).to(dtype)
    pd = torch.from_numpy(perm).to(dev)
    say("bt_permute_padded", n, shape, dtype)
    g = ops.bt_permute_padded(x.to(dev), pd, n, ops.BT_GATHER)
    back = ops.bt_permute_padded(g, pd, n, ops.BT_SCATTER)
    torch.cuda.synchronize()
    as_np = lambda t: (t.cpu().view(torch.int16) if t.dtype == torch.bfloat16 else t.cpu()).numpy()
    assert np.array_equal(as_np(g), P.gather_padded(as_np(x), perm))
    assert np.array_equal(as_np(back), P.scatter_padded(as_np(g), perm, n))
    assert np.array_equal(as_np(back), as_np(x))


@pytest.mark.parametrize("n,leaf,H,d,ball,dtype", [
    (972, 32, 8, 32, 128, "bf16"),      # Elasticity-sized cloud
    (3586, 64, 8, 32, 128, "bf16"),     # ShapeNet-Car-sized cloud
    (5000, 64, 4, 64, 64, "bf16"),      # cosmology-sized cloud
    (3586, 64, 2, 32, 256, "bf16"),
    (2000, 32, 2, 32, 32, "bf16"),
    (972, 32, 4, 16, 32, "f32"),        # VALU kernel
    (1500, 16, 2, 64, 512, "bf16"),     # VALU kernel (ball above 256)
])
def test_ball_attn_padded(n, leaf, H, d, ball, dtype):
    dev = gpu()
    rng = np.random.default_rng(n + ball + d)
    c = synth.deformed_sphere(rng, n)
    perm = T.build_padded(c, leaf).astype(np.int32)
    if len(perm) % ball:
        perm = np.concatenate([perm, np.full(ball - len(perm) % ball, -1, np.int32)])
    q, k, v = (synth.normal_features(rng, n, H, d, dtype) for _ in range(3))
    say("ball_attn_padded", n, len(perm), H, d, ball, dtype)
    out = ops.ball_attn_padded(q.to(dev), k.to(dev), v.to(dev),
                               torch.from_numpy(perm).to(dev), ball)
    torch.cuda.synchronize()
    err = max_abs(out.cpu(), A.ball_attn_padded(q, k, v, perm, ball))
    assert err <= (2e-2 if dtype == "bf16" else 1e-5), err


def test_ball_attn_padded_full_size():
    """65,000 points of the sphere workload in 65,536 slots (ball 128, 8 heads,
    d 32): the padded GPU tree bit for bit, then every output row of padded
    attention through it against the oracle."""
    dev = gpu()
    w = synth.make("sphere", n=65000)
    say("bt_build_padded + ball_attn_padded sphere 65000")
    p = ops.bt_build_padded(torch.from_numpy(w.coords).to(dev), w.leaf)
    out = ops.ball_attn_padded(w.q.to(dev), w.k.to(dev), w.v.to(dev), p, w.ball)
    torch.cuda.synchronize()
    perm = T.build_padded(w.coords, w.leaf).astype(np.int32)
    assert len(perm) == 65536
    assert np.array_equal(p.cpu().numpy(), perm)
    assert max_abs(out.cpu(), A.ball_attn_padded(w.q, w.k, w.v, perm, w.ball)) <= 2e-2


def test_padded_pipeline_972():
    """Elasticity-sized pipeline: GPU padded tree, padded attention, gather
    into tree order and back, all against the oracle."""
    dev = gpu()
    rng = np.random.default_rng(21)
    n = 972
    c = synth.uniform_cube(rng, n)
    q, k, v = (synth.normal_features(rng, n, 4, 32, "bf16") for _ in range(3))
    say("padded pipeline 972")
    p = ops.bt_build_padded(torch.from_numpy(c).to(dev), 32)
    out = ops.ball_attn_padded(q.to(dev), k.to(dev), v.to(dev), p, 64)
    ot = ops.bt_permute_padded(out, p, n, ops.BT_GATHER)      # tree order, zero rows
    torch.cuda.synchronize()
    pr = T.build_padded(c, 32)
    assert np.array_equal(p.cpu().numpy(), pr)
    ref = A.ball_attn_padded(q, k, v, pr, 64)
    assert max_abs(out.cpu(), ref) <= 2e-2
    assert torch.equal(ot.cpu()[torch.from_numpy(pr < 0)],
                       torch.zeros(int((pr < 0).sum()), 4, 32, dtype=torch.bfloat16))


@pytest.mark.parametrize("name,n,leaf,ball,H,d", [
    ("shapenet_car", 3586, 32, 128, 8, 32),   # ShapeNet-Car's point count
    ("cosmology", 5000, 64, 64, 4, 64),       # a cosmology-sized cloud
])
def test_padded_pipeline_pages_sizes(name, n, leaf, ball, H, d):
    """The pages' uneven clouds end to end on the GPU: padded tree (bit for
    bit), padded ball attention through the GPU permutation, gather into
    tree order."""
    dev = gpu()
    rng = np.random.default_rng(n)
    c = synth.deformed_sphere(rng, n)
    q, k, v = (synth.normal_features(rng, n, H, d, "bf16") for _ in range(3))
    say("padded pipeline", name, n, leaf, ball)
    p = ops.bt_build_padded(torch.from_numpy(c).to(dev), leaf)
    out = ops.ball_attn_padded(q.to(dev), k.to(dev), v.to(dev), p, ball)
    ot = ops.bt_permute_padded(out, p, n, ops.BT_GATHER)
    torch.cuda.synchronize()
    pr = T.build_padded(c, leaf)
    assert np.array_equal(p.cpu().numpy(), pr)
    assert max_abs(out.cpu(), A.ball_attn_padded(q, k, v, pr, ball)) <= 2e-2
    as_i16 = lambda t: t.cpu().view(torch.int16).numpy()
    assert np.array_equal(as_i16(ot), P.gather_padded(as_i16(out), pr))
