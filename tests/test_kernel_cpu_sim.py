"""The HIP kernel sources, compiled for the host and run on the CPU.

tests/cpu_sim/ holds a host SIMT emulation of the HIP constructs the kernels
use (see its header); the kernel .hip files are included unchanged, built
with clang++ and AddressSanitizer, and run on small inputs.  The results are
compared with the oracle: tree permutations bit for bit (including the
global passes above 1,024 points, which the library switches off on the
GPU), attention within the GPU tolerances.  An out-of-bounds access in a
kernel aborts the run under AddressSanitizer.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

from ball_tree_sparse_amd import synth
from oracle import attention as A
from oracle import attention_bwd as AB
from oracle import bsa as B
from oracle import bsa_bwd as BB
from oracle import tree as T

HERE = os.path.dirname(os.path.abspath(__file__))
SIM = os.path.join(HERE, "cpu_sim")
ROOT = os.path.dirname(HERE)
CXX = shutil.which("clang++") or "/opt/rocm/llvm/bin/clang++"


@pytest.fixture(scope="module")
def sim(tmp_path_factory):
    if not os.path.exists(CXX):
        pytest.skip("clang++ not available")
    d = tmp_path_factory.mktemp("cpu_sim")
    flags = ["-std=c++20", "-O1", "-fsanitize=address", "-fno-omit-frame-pointer",
             "-I", SIM, "-I", os.path.join(ROOT, "include")]
    bins = {}
    procs = []
    for name, src, extra in (("tree", "tree_driver.cpp", []), ("attn", "attn_driver.cpp", []),
                             ("bsa_bwd", "attn_driver.cpp", ["-DBT_SIM_BSA_BWD"])):
        out = str(d / name)
        procs.append(subprocess.Popen([CXX, *flags, *extra, os.path.join(SIM, src),
                                       os.path.join(SIM, "emu.cpp"), "-o", out, "-lpthread"],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                      text=True))
        bins[name] = out
    for p in procs:
        o, _ = p.communicate()
        assert p.returncode == 0, o[-4000:]
    bins["dir"] = d
    return bins


def _tree(sim, coords, leaf, R=None):
    d = sim["dir"]
    c = d / "c.bin"
    np.ascontiguousarray(coords, np.float32).tofile(c)
    args = [sim["tree"], str(c), str(len(coords)), str(leaf), str(d / "p.bin")]
    if R is not None:
        np.asarray(R, np.float32).tofile(d / "R.bin")
        args.append(str(d / "R.bin"))
    r = subprocess.run(args, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and "done" in r.stdout, r.stderr[-4000:]
    return np.fromfile(d / "p.bin", np.int32)


@pytest.mark.parametrize("case", ["cube4k_leaf32", "lattice2k_leaf8", "signed_zeros2k_leaf2",
                                  "mixture4k_leaf16", "leaf2048", "cube1536_leaf3",
                                  "cube2000_leaf1000"])
def test_tree_kernels_bit_exact(sim, case):
    rng = np.random.default_rng(31)
    if case == "cube4k_leaf32":
        c, leaf = synth.uniform_cube(rng, 4096), 32
    elif case == "lattice2k_leaf8":
        c, leaf = rng.integers(0, 4, size=(2048, 3)).astype(np.float32), 8
    elif case == "signed_zeros2k_leaf2":
        c = rng.integers(-1, 2, size=(2048, 3)).astype(np.float32)
        c[rng.random(c.shape) < 0.5] *= 0.0
        c[rng.random(c.shape) < 0.5] *= -1.0
        leaf = 2
    elif case == "mixture4k_leaf16":
        c, leaf = synth.gaussian_mixture(rng, 4096, k=16), 16
    elif case == "leaf2048":
        c, leaf = synth.uniform_cube(rng, 4096), 2048
    elif case == "cube1536_leaf3":        # a 1,536-point node: not a multiple of 1,024
        c, leaf = synth.uniform_cube(rng, 3 << 9), 3
    else:                                 # chunks that are not a multiple of 256
        c, leaf = synth.uniform_cube(rng, 2000), 1000
    assert np.array_equal(_tree(sim, c, leaf), T.build(c, leaf))


def test_rotated_tree_kernels_bit_exact(sim):
    w = synth.make("rotpair", n=4096, features=False)
    assert np.array_equal(_tree(sim, w.coords, 64, R=w.R),
                          T.rotate_build(w.coords, 64, w.R))


def _dump(t, path):
    if t.dtype == torch.bfloat16:
        t.contiguous().view(torch.int16).numpy().tofile(path)
    else:
        t.contiguous().numpy().tofile(path)


def _read_out(path, n, H, d, dtype):
    raw = np.fromfile(path, np.uint8)
    if dtype == "bf16":
        return torch.from_numpy(raw.view(np.int16).copy()).view(torch.bfloat16).float() \
            .numpy().reshape(n, H, d)
    return raw.view(np.float32).reshape(n, H, d)


@pytest.mark.parametrize("n,H,d,ball,dtype", [(1024, 2, 32, 128, "bf16"), (1024, 1, 32, 256, "bf16"),
                                             (512, 2, 32, 256, "bf16"),
                                             (256, 3, 32, 32, "bf16"), (512, 1, 64, 256, "bf16"),
                                             (512, 2, 64, 64, "bf16"), (2048, 4, 32, 64, "bf16"),
                                             (1024, 6, 64, 128, "bf16"),
                                             (512, 2, 16, 32, "f32")])
def test_ball_attn_kernels(sim, n, H, d, ball, dtype):
    d_ = sim["dir"]
    rng = np.random.default_rng(n + d)
    q, k, v = (synth.normal_features(rng, n, H, d, dtype) for _ in range(3))
    perm = rng.permutation(n).astype(np.int32)
    for t, nm in ((q, "q.bin"), (k, "k.bin"), (v, "v.bin")):
        _dump(t, d_ / nm)
    perm.tofile(d_ / "perm.bin")
    r = subprocess.run([sim["attn"], "ball", str(n), str(H), str(d), str(ball),
                        "1" if dtype == "bf16" else "0"], cwd=d_, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0 and "done" in r.stdout, r.stderr[-4000:]
    out = _read_out(d_ / "out.bin", n, H, d, dtype)
    err = np.abs(out - A.ball_attn(q, k, v, perm, ball)).max()
    assert err <= (2e-2 if dtype == "bf16" else 1e-5), err


def test_ball_attn_kernel_tree_order_input(sim):
    """perm == NULL: inputs already in tree order."""
    d_ = sim["dir"]
    n, H, d, ball = 1024, 2, 32, 64
    rng = np.random.default_rng(9)
    q, k, v = (synth.normal_features(rng, n, H, d, "bf16") for _ in range(3))
    for t, nm in ((q, "q.bin"), (k, "k.bin"), (v, "v.bin")):
        _dump(t, d_ / nm)
    np.arange(n, dtype=np.int32).tofile(d_ / "perm.bin")
    r = subprocess.run([sim["attn"], "ball_noperm", str(n), str(H), str(d), str(ball), "1"],
                       cwd=d_, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and "done" in r.stdout, r.stderr[-4000:]
    out = _read_out(d_ / "out.bin", n, H, d, "bf16")
    assert np.abs(out - A.ball_attn(q, k, v, None, ball)).max() <= 2e-2


@pytest.mark.parametrize("qc,group", [(0, 64), (1, 64), (0, 128)])
def test_bsa_kernels(sim, qc, group):
    """BSA, and BSA with group compression (qc = 1); group 128 runs two waves
    of 64 queries per workgroup."""
    d_ = sim["dir"]
    n, H, d, ball, block, topk = 2048, 2, 32, 128, 64, 4
    rng = np.random.default_rng(5)
    c = synth.deformed_sphere(rng, n)
    q, k, v = (synth.normal_features(rng, n, H, d, "bf16") for _ in range(3))
    W = (0.02 * rng.standard_normal((3, d))).astype(np.float32)
    perm = T.build(c, block).astype(np.int32)
    for t, nm in ((q, "q.bin"), (k, "k.bin"), (v, "v.bin")):
        _dump(t, d_ / nm)
    perm.tofile(d_ / "perm.bin")
    W.tofile(d_ / "w.bin")
    r = subprocess.run([sim["attn"], "bsa", str(n), str(H), str(d), str(ball), "1", str(block),
                        str(group), str(topk), "1", "0", str(qc)], cwd=d_, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0 and "done" in r.stdout, r.stderr[-4000:]
    out = _read_out(d_ / "out.bin", n, H, d, "bf16")
    sel = np.fromfile(d_ / "sel.out", np.int32).reshape(H, n // group, topk)
    ref, parts = B.bsa(q, k, v, perm, ball, block, group, topk, True, W=W, return_parts=True,
                       query_compression=bool(qc))
    assert np.array_equal(np.sort(sel, -1), np.sort(parts["sel"], -1))
    assert np.abs(out - ref).max() <= 2e-2


@pytest.mark.parametrize("n,d,block,group,gm", [(2048, 32, 64, 64, 0), (2048, 32, 32, 32, 1),
                                               (1024, 64, 32, 128, 0)])
def test_bsa_bwd_kernels(sim, n, d, block, group, gm):
    """BSA backward: learned gates (gm 0, with dW and db) and constant gates
    (gm 1); groups of one, two and four waves; key passes with two key blocks
    per wave (ball and 64-key blocks; 64 coarse tokens) and with one."""
    d_ = sim["dir"]
    H, ball, topk = 2, 128, 4
    rng = np.random.default_rng(11 + d + group)
    c = synth.deformed_sphere(rng, n)
    q, k, v, do = (synth.normal_features(rng, n, H, d, "bf16") for _ in range(4))
    W = (0.2 * rng.standard_normal((3, d))).astype(np.float32)
    b = (0.5 * rng.standard_normal(3)).astype(np.float32)
    perm = T.build(c, block).astype(np.int32)
    for t, nm in ((q, "q.bin"), (k, "k.bin"), (v, "v.bin"), (do, "do.bin")):
        _dump(t, d_ / nm)
    perm.tofile(d_ / "perm.bin")
    W.tofile(d_ / "w.bin")
    b.tofile(d_ / "b.bin")
    r = subprocess.run([sim["bsa_bwd"], "bsa_bwd", str(n), str(H), str(d), str(ball), "1",
                        str(block), str(group), str(topk), "1", str(gm)], cwd=d_,
                       capture_output=True, text=True, timeout=900)
    assert r.returncode == 0 and "done" in r.stdout, r.stderr[-4000:]
    if gm == 0:
        want = BB.bsa_bwd(q, k, v, do, perm, ball, block, group, topk, True, W=W, b=b)
    else:
        want = BB.bsa_bwd(q, k, v, do, perm, ball, block, group, topk, True,
                          gate_const=(0.3, 0.5, 0.7))
    for name, w in zip("qkv", want[:3]):
        got = _read_out(d_ / f"d{name}.bin", n, H, d, "bf16")
        err = np.abs(got - w).max()
        assert err <= 2e-2, (name, err)
    if gm == 0:
        # sums over all N*H tokens: 2e-2 relative to the largest entry
        dw = np.fromfile(d_ / "dw.bin", np.float32).reshape(3, d)
        db = np.fromfile(d_ / "db.bin", np.float32)
        assert np.abs(dw - want[3]).max() <= 2e-2 * max(1.0, np.abs(want[3]).max())
        assert np.abs(db - want[4]).max() <= 2e-2 * max(1.0, np.abs(want[4]).max())


@pytest.mark.parametrize("n,H,d,ball,dtype", [(512, 2, 32, 128, "bf16"), (256, 2, 32, 32, "bf16"),
                                             (256, 1, 64, 64, "bf16"), (384, 2, 32, 64, "bf16"),
                                             (256, 1, 64, 128, "bf16"), (512, 1, 32, 256, "bf16"),
                                             (256, 2, 16, 64, "bf16"), (256, 2, 32, 32, "f32")])
def test_ball_attn_bwd_kernels(sim, n, H, d, ball, dtype):
    """Backward: the MFMA kernel (bf16, d 32 or 64, balls of 32 to 256) and
    the VALU kernel (the rest)."""
    d_ = sim["dir"]
    rng = np.random.default_rng(3 * n + d + ball)
    q, k, v, do = (synth.normal_features(rng, n, H, d, dtype) for _ in range(4))
    perm = rng.permutation(n).astype(np.int32)
    for t, nm in ((q, "q.bin"), (k, "k.bin"), (v, "v.bin"), (do, "do.bin")):
        _dump(t, d_ / nm)
    perm.tofile(d_ / "perm.bin")
    r = subprocess.run([sim["attn"], "bwd", str(n), str(H), str(d), str(ball),
                        "1" if dtype == "bf16" else "0"], cwd=d_, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0 and "done" in r.stdout, r.stderr[-4000:]
    want = AB.ball_attn_bwd(q, k, v, do, perm, ball)
    for name, w in zip("qkv", want):
        got = _read_out(d_ / f"d{name}.bin", n, H, d, dtype)
        err = np.abs(got - w).max()
        assert err <= (2e-2 if dtype == "bf16" else 2e-5), (name, err)


def _tree_padded(sim, coords, leaf, R=None):
    d = sim["dir"]
    c = d / "c.bin"
    np.ascontiguousarray(coords, np.float32).tofile(c)
    args = [sim["tree"], "padded", str(c), str(len(coords)), str(leaf), str(d / "p.bin")]
    if R is not None:
        np.asarray(R, np.float32).tofile(d / "R.bin")
        args.append(str(d / "R.bin"))
    r = subprocess.run(args, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and "done" in r.stdout, r.stderr[-4000:]
    return np.fromfile(d / "p.bin", np.int32)


@pytest.mark.parametrize("n,leaf", [(972, 32), (1000, 16), (513, 64), (5, 2), (3, 1), (1, 1),
                                    (2, 1), (700, 700), (1024, 32), (129, 1)])
def test_padded_tree_kernels_bit_exact(sim, n, leaf):
    """Uneven N: the padded tree (one workgroup in LDS), bit for bit."""
    rng = np.random.default_rng(n * 7 + leaf)
    c = synth.uniform_cube(rng, n)
    assert np.array_equal(_tree_padded(sim, c, leaf), T.build_padded(c, leaf))


def test_padded_tree_kernels_rotated_and_ties(sim):
    rng = np.random.default_rng(12)
    c = rng.integers(-1, 2, size=(900, 3)).astype(np.float32)    # many equal keys
    c[rng.random(c.shape) < 0.5] *= -1.0                          # signed zeros
    R = synth.random_rotation(rng)
    assert np.array_equal(_tree_padded(sim, c, 8), T.build_padded(c, 8))
    w = synth.uniform_cube(rng, 600)
    assert np.array_equal(_tree_padded(sim, w, 16, R=R), T.rotate_build_padded(w, 16, R))


@pytest.mark.parametrize("n,H,d,ball,dtype", [(972, 2, 32, 128, "bf16"), (1000, 3, 64, 64, "bf16"),
                                             (300, 2, 32, 256, "bf16"), (972, 2, 16, 32, "f32"),
                                             (500, 2, 16, 64, "bf16")])
def test_ball_attn_padded_kernels(sim, n, H, d, ball, dtype):
    """Ball attention on a padded tree: unused slots take no weight and get no
    output row (the MFMA kernel for bf16 d 32/64, the VALU kernel otherwise)."""
    d_ = sim["dir"]
    rng = np.random.default_rng(n + ball)
    c = synth.uniform_cube(rng, n)
    perm = T.build_padded(c, 16).astype(np.int32)
    if len(perm) % ball:
        perm = np.concatenate([perm, np.full(ball - len(perm) % ball, -1, np.int32)])
    q, k, v = (synth.normal_features(rng, n, H, d, dtype) for _ in range(3))
    for t, nm in ((q, "q.bin"), (k, "k.bin"), (v, "v.bin")):
        _dump(t, d_ / nm)
    perm.tofile(d_ / "perm.bin")
    r = subprocess.run([sim["attn"], "ball_padded", str(n), str(H), str(d), str(ball),
                        "1" if dtype == "bf16" else "0", str(len(perm))], cwd=d_,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and "done" in r.stdout, r.stderr[-4000:]
    out = _read_out(d_ / "out.bin", n, H, d, dtype)
    err = np.abs(out - A.ball_attn_padded(q, k, v, perm, ball)).max()
    assert err <= (2e-2 if dtype == "bf16" else 1e-5), err


@pytest.mark.parametrize("mode,ball,dtype", [("ball", 128, "bf16"), ("ball", 64, "f32"),
                                             ("bwd", 128, "bf16"), ("bwd", 32, "f32")])
def test_out_of_range_perm_stays_in_bounds(sim, mode, ball, dtype):
    """A 'permutation' with entries far outside [0, N) (negative and huge):
    every kernel that reads rows through it forces the indices into range,
    so AddressSanitizer sees no access outside q/k/v/dO or the outputs."""
    d_ = sim["dir"]
    n, H, d = 512, 2, 32
    rng = np.random.default_rng(77)
    ts = [synth.normal_features(rng, n, H, d, dtype) for _ in range(4)]
    for t, nm in zip(ts, ("q.bin", "k.bin", "v.bin", "do.bin")):
        _dump(t, d_ / nm)
    perm = rng.integers(-2**31, 2**31 - 1, size=n, dtype=np.int64).astype(np.int32)
    perm[:8] = [-1, n, n + 1, 2**31 - 1, -2**31, 0, n - 1, 7]
    perm.tofile(d_ / "perm.bin")
    r = subprocess.run([sim["attn"], mode, str(n), str(H), str(d), str(ball),
                        "1" if dtype == "bf16" else "0"], cwd=d_, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0 and "done" in r.stdout, r.stderr[-4000:]
