"""GPU parity of ball_attn against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

from ball_tree_sparse_amd import ops, synth
from oracle import attention as A
from oracle import tree as T
from tests.helpers import gpu, max_abs, ramp_scores, say

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-5}


def _feats(n, H, d, dtype, seed):
    rng = np.random.default_rng(seed)
    return [synth.normal_features(rng, n, H, d, dtype) for _ in range(3)]


def _run(q, k, v, perm, ball, dev):
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    pd = None if perm is None else torch.from_numpy(np.asarray(perm, np.int32)).to(dev)
    out = ops.ball_attn(qd, kd, vd, pd, ball)
    torch.cuda.synchronize()
    return out.cpu()


@pytest.mark.parametrize("n,H,d,ball,dtype", [
    (1024, 4, 16, 32, "f32"),      # the tiny workload's shape, fp32 path
    (2048, 3, 32, 64, "f32"),
    (512, 2, 64, 128, "f32"),
    (1536, 3, 32, 96, "f32"),      # ball not a power of two
    (4096, 8, 32, 128, "bf16"),    # MFMA, several tiles
    (2560, 3, 32, 128, "bf16"),    # 60 (ball, head) pairs: no XCD remap, ragged
    (4096, 2, 64, 128, "bf16"),
    (2048, 5, 32, 32, "bf16"),
    (2048, 4, 32, 64, "bf16"),
    (4096, 4, 32, 256, "bf16"),
    (2048, 2, 64, 256, "bf16"),
    (1024, 4, 16, 32, "bf16"),     # d=16 bf16 -> VALU kernel
    (960, 2, 32, 48, "bf16"),      # ball not a multiple of 32 -> VALU kernel
    (98432, 4, 32, 128, "bf16"),   # 1,538 head-pair items: persistent pipelined form,
                                   # two workgroups walk a second item, no XCD remap
    (98304, 6, 32, 128, "bf16"),   # 2,304 items, pipelined, XCD remap, 3 pairs per ball
    (16384, 8, 32, 256, "bf16"),   # ball 256: single-head items
])
def test_parity_random_perm(n, H, d, ball, dtype):
    dev = gpu()
    q, k, v = _feats(n, H, d, dtype, seed=n + H + d + ball)
    perm = np.random.default_rng(7).permutation(n)
    say("ball_attn", n, H, d, ball, dtype)
    got = _run(q, k, v, perm, ball, dev)
    want = A.ball_attn(q, k, v, perm, ball)
    err = max_abs(got, want)
    assert err <= TOL[dtype], err


@pytest.mark.parametrize("big", [False, True])
@pytest.mark.parametrize("n,H,d,ball", [(4096, 4, 32, 256), (2048, 2, 64, 256),
                                        (2048, 3, 32, 256), (4096, 4, 32, 128)])
def test_parity_scores_stepping_along_the_ball(n, H, d, ball, big):
    """Scores that climb (or fall) by 2^8 and more from one 64-key stretch of
    a ball to the next.  big: one key per ball with a large component no
    query has, so that the bound |q| max|k| on the scores is far above them
    (a running maximum is then raised part way through)."""
    dev = gpu()
    q, k, v = _feats(n, H, d, "bf16", seed=n + d + 11)
    perm = np.random.default_rng(8).permutation(n)
    q, k = ramp_scores(q, k, perm, ball, seed=9, big_key=big)
    say("ball_attn stepped scores", n, H, d, ball)
    got = _run(q, k, v, perm, ball, dev)
    assert max_abs(got, A.ball_attn(q, k, v, perm, ball)) <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_parity_tree_order_no_perm(dtype):
    dev = gpu()
    q, k, v = _feats(4096, 4, 32, dtype, seed=3)
    say("ball_attn perm=None", dtype)
    got = _run(q, k, v, None, 128, dev)
    assert max_abs(got, A.ball_attn(q, k, v, None, 128)) <= TOL[dtype]


def test_full_attention_when_ball_is_n():
    dev = gpu()
    q, k, v = _feats(1024, 2, 32, "f32", seed=4)
    say("ball_attn ball=N")
    got = _run(q, k, v, np.random.default_rng(0).permutation(1024), 1024, dev)
    assert max_abs(got, A.full_attn(q, k, v)) <= 1e-5


def test_largest_ball_is_full_attention():
    """ball = 4,096 (the largest accepted; fp32 VALU kernel) equals full attention."""
    dev = gpu()
    q, k, v = _feats(4096, 1, 16, "f32", seed=6)
    say("ball_attn ball=4096")
    got = _run(q, k, v, np.random.default_rng(1).permutation(4096), 4096, dev)
    assert max_abs(got, A.full_attn(q, k, v)) <= 1e-5


def test_empty_input_is_a_noop():
    dev = gpu()
    say("ball_attn / permute with N = 0")
    for dt in (torch.bfloat16, torch.float32):
        q = torch.empty((0, 4, 32), dtype=dt, device=dev)
        out = ops.ball_attn(q, q.clone(), q.clone(), None, 32)
        assert out.shape == (0, 4, 32)
    src = torch.empty((0, 64), dtype=torch.int32, device=dev)
    p = torch.empty((0,), dtype=torch.int32, device=dev)
    assert ops.bt_permute(src, p, ops.BT_GATHER).shape == (0, 64)
    torch.cuda.synchronize()


def test_ball_one_returns_v():
    dev = gpu()
    q, k, v = _feats(256, 2, 16, "f32", seed=5)
    say("ball_attn ball=1")
    got = _run(q, k, v, None, 1, dev)
    assert max_abs(got, v) == 0.0


def test_tiny_workload_end_to_end():
    """N=1,024 cube, leaf = ball = 32, H=4, d=16 fp32: GPU tree + GPU attention."""
    dev = gpu()
    w = synth.make("tiny")
    c = torch.from_numpy(w.coords).to(dev)
    say("tiny: bt_build + ball_attn")
    perm = ops.bt_build(c, w.leaf)
    qd, kd, vd = (t.to(dev) for t in (w.q, w.k, w.v))
    out = ops.ball_attn(qd, kd, vd, perm, w.ball)
    torch.cuda.synchronize()
    p_ref = T.build(w.coords, w.leaf)
    assert np.array_equal(perm.cpu().numpy(), p_ref)
    assert max_abs(out.cpu(), A.ball_attn(w.q, w.k, w.v, p_ref, w.ball)) <= 1e-5


def test_sphere_workload_full_size():
    """N=65,536 deformed sphere, ball 128, H=8, d=32 bf16 (the measured shape)."""
    dev = gpu()
    w = synth.make("sphere")
    p_ref = T.build(w.coords, w.leaf)
    say("sphere: ball_attn full size")
    got = _run(w.q, w.k, w.v, p_ref, w.ball, dev)
    want = A.ball_attn(w.q, w.k, w.v, p_ref, w.ball)
    assert max_abs(got, want) <= 2e-2


def test_cosmo_workload_sampled():
    """N=1,048,576 mixture, ball 256: oracle on 3,000 sampled tree positions."""
    dev = gpu()
    w = synth.make("cosmo")
    p_ref = T.build(w.coords, w.leaf)
    say("cosmo: ball_attn full size")
    got = _run(w.q, w.k, w.v, p_ref, w.ball, dev)
    rows = np.random.default_rng(1).choice(w.coords.shape[0], 3000, replace=False)
    rows = np.concatenate([rows, [0, w.coords.shape[0] - 1]])
    want = A.ball_attn_rows(w.q, w.k, w.v, p_ref, w.ball, rows)
    assert max_abs(got[torch.from_numpy(p_ref[rows])], want) <= 2e-2
    # every output row is finite and a convex combination bound holds
    g = got.float()
    assert torch.isfinite(g).all()
    assert g.abs().max() <= w.v.float().abs().max() + 1e-2


@pytest.mark.parametrize("name", ["sphere", "cosmo"])
def test_workload_gpu_tree_then_attention(name):
    """The workload's build and pass on the GPU: bt_build (bit for bit
    against the oracle's tree), then ball_attn through that device
    permutation; every output (sphere) or 3,002 sampled rows (cosmology)
    against the oracle."""
    dev = gpu()
    w = synth.make(name)
    say(name, ": GPU tree then ball_attn")
    perm = ops.bt_build(torch.from_numpy(w.coords).to(dev), w.leaf)
    out = ops.ball_attn(w.q.to(dev), w.k.to(dev), w.v.to(dev), perm, w.ball)
    torch.cuda.synchronize()
    p_ref = T.build(w.coords, w.leaf)
    assert np.array_equal(perm.cpu().numpy(), p_ref)
    got = out.cpu()
    if name == "sphere":
        assert max_abs(got, A.ball_attn(w.q, w.k, w.v, p_ref, w.ball)) <= 2e-2
    else:
        rows = np.random.default_rng(2).choice(w.coords.shape[0], 3000, replace=False)
        rows = np.concatenate([rows, [0, w.coords.shape[0] - 1]])
        want = A.ball_attn_rows(w.q, w.k, w.v, p_ref, w.ball, rows)
        assert max_abs(got[torch.from_numpy(p_ref[rows])], want) <= 2e-2


def test_deterministic():
    dev = gpu()
    q, k, v = _feats(8192, 8, 32, "bf16", seed=9)
    perm = np.random.default_rng(2).permutation(8192)
    say("ball_attn determinism")
    a = _run(q, k, v, perm, 128, dev)
    b = _run(q, k, v, perm, 128, dev)
    assert torch.equal(a, b)
