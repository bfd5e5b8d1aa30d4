"""GPU tree builder: bit-exact against the oracle (ties broken by index)."""
import numpy as np
import pytest
import torch

from ball_tree_sparse_amd import ops, synth
from oracle import checks
from oracle import tree as T
from tests.helpers import gpu, say

pytestmark = pytest.mark.gpu

# The GPU builder's passes for nodes above 1,024 points faulted the GPU in
# two runs (first failing case: tests/test_gpu_permute.py::
# test_rotated_pair_pipeline_small) and the cause has not been found; the
# library refuses such trees, and these cases stay skipped until it is.
GLOBAL_PASSES_OFF = pytest.mark.skip(
    reason="GPU tree passes above 1,024 points are switched off: they faulted the GPU twice "
           "and the cause is not found (the same kernels are checked on the CPU by "
           "tests/test_kernel_cpu_sim.py)")


def _gpu_tree(coords, leaf, R=None):
    dev = gpu()
    c = torch.from_numpy(np.ascontiguousarray(coords, dtype=np.float32)).to(dev)
    p = ops.bt_build(c, leaf) if R is None else ops.bt_rotate_build(c, leaf, R)
    torch.cuda.synchronize()
    return p.cpu().numpy().astype(np.int64)


def _clouds():
    rng = np.random.default_rng(21)
    yield "cube1k", synth.uniform_cube(rng, 1024), 32
    yield "cube1k_leaf1", synth.uniform_cube(rng, 1024), 1
    yield "sphere1k", synth.deformed_sphere(rng, 1024), 64
    yield "mixture512", synth.gaussian_mixture(rng, 512, k=8), 16
    yield "lattice1k", rng.integers(0, 5, size=(1024, 3)).astype(np.float32), 16
    yield "dups1k", np.repeat(rng.random((64, 3)).astype(np.float32), 16, axis=0), 4
    z = rng.integers(-1, 2, size=(1024, 3)).astype(np.float32)
    z[rng.random((1024, 3)) < 0.5] *= 0.0
    z[rng.random((1024, 3)) < 0.5] *= -1.0                 # +-0 and +-1
    yield "signed_zeros1k", z, 2
    yield "identical512", np.full((512, 3), 0.5, np.float32), 16
    yield "n_eq_leaf", synth.uniform_cube(rng, 256), 256
    yield "big_range1k", (rng.standard_normal((1024, 3)) * 1e30).astype(np.float32), 32
    tiny = np.array([[0, 0, 0], [3, 1, 0], [0, 5, 0], [2, 2, 0], [-1, 4, 1], [2, 2, 0],
                     [1, 0, 0], [-0.0, 5, 1]], np.float32)
    yield "golden8", tiny, 2


def _big_clouds():
    rng = np.random.default_rng(22)
    yield "cube4k_leaf8", synth.uniform_cube(rng, 4096), 8
    yield "sphere16k", synth.deformed_sphere(rng, 16384), 64
    yield "mixture32k", synth.gaussian_mixture(rng, 32768, k=32), 128
    yield "lattice8k", rng.integers(0, 5, size=(8192, 3)).astype(np.float32), 16
    yield "leaf2048", synth.uniform_cube(rng, 8192), 2048


@pytest.mark.parametrize("name,coords,leaf", list(_clouds()), ids=[c[0] for c in _clouds()])
def test_bit_exact(name, coords, leaf):
    say("bt_build", name, coords.shape, leaf)
    got = _gpu_tree(coords, leaf)
    want = T.build(coords, leaf)
    assert np.array_equal(got, want), np.flatnonzero(got != want)[:10]
    assert checks.check_tree(coords, got, leaf)[0]


@GLOBAL_PASSES_OFF
@pytest.mark.parametrize("name,coords,leaf", list(_big_clouds()),
                         ids=[c[0] for c in _big_clouds()])
def test_bit_exact_above_1024(name, coords, leaf):
    say("bt_build", name, coords.shape, leaf)
    assert np.array_equal(_gpu_tree(coords, leaf), T.build(coords, leaf))


def test_tiny_workload_bit_exact():
    w = synth.make("tiny", features=False)
    say("bt_build workload tiny")
    assert np.array_equal(_gpu_tree(w.coords, w.leaf), T.build(w.coords, w.leaf))


def test_rejects_above_limit():
    dev = gpu()
    c = torch.zeros((2048, 3), device=dev)
    with pytest.raises(ops.BtError):
        ops.bt_build(c, 2)


@GLOBAL_PASSES_OFF
@pytest.mark.parametrize("name", ["sphere", "rotpair", "cosmo"])
def test_workloads_bit_exact(name):
    w = synth.make(name, features=False)
    say("bt_build workload", name)
    got = _gpu_tree(w.coords, w.leaf)
    assert np.array_equal(got, T.build(w.coords, w.leaf))


@GLOBAL_PASSES_OFF
def test_sphere_leaf64_nests_leaf128():
    w = synth.make("sphere", features=False)
    say("bt_build sphere leaf 64")
    p64 = _gpu_tree(w.coords, 64)
    assert np.array_equal(p64, T.build(w.coords, 64))
    p128 = _gpu_tree(w.coords, 128)
    # every 128-ball holds the same points in both trees
    a = np.sort(p64.reshape(-1, 128), axis=1)
    b = np.sort(p128.reshape(-1, 128), axis=1)
    assert np.array_equal(a, b)


@GLOBAL_PASSES_OFF
def test_rotate_build_rotpair():
    w = synth.make("rotpair", features=False)
    say("bt_rotate_build rotpair")
    got = _gpu_tree(w.coords, w.leaf, R=w.R)
    assert np.array_equal(got, T.rotate_build(w.coords, w.leaf, w.R))


def test_rotate_identity_equals_build():
    rng = np.random.default_rng(4)
    c = synth.box_4x1x1(rng, 1024)
    say("bt_rotate_build identity")
    assert np.array_equal(_gpu_tree(c, 32, R=np.eye(3)), _gpu_tree(c, 32))


def test_rotate_rounding_small():
    rng = np.random.default_rng(5)
    c = rng.standard_normal((1024, 3)).astype(np.float32)
    R = synth.random_rotation(rng)
    say("bt_rotate_build random small")
    assert np.array_equal(_gpu_tree(c, 4, R=R), T.rotate_build(c, 4, R))
    w = synth.make("rotpair", n=1024, features=False)
    say("bt_rotate_build rotpair recipe at 1024")
    assert np.array_equal(_gpu_tree(w.coords, 32, R=w.R), T.rotate_build(w.coords, 32, w.R))


def test_deterministic_and_workspace_reuse():
    dev = gpu()
    w = synth.make("sphere", n=1024, features=False)
    c = torch.from_numpy(w.coords).to(dev)
    ws = torch.empty(ops.bt_build_workspace_size(c.shape[0], 32), dtype=torch.uint8, device=dev)
    ws.fill_(0xAB)                                       # garbage workspace
    say("bt_build determinism")
    a = ops.bt_build(c, 32, workspace=ws).clone()
    b = ops.bt_build(c, 32, workspace=ws).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)
