"""The HIP kernel sources, compiled for the host and run on the CPU.

tests/cpu_sim/ holds a host SIMT emulation of the HIP constructs the kernels
use (see its header); the kernel .hip files are included unchanged, built
with clang++ and AddressSanitizer, and run on small inputs.  The results are
compared with the oracle: tree permutations bit for bit (the one-workgroup
LDS builder of trees up to 8,192 points and the streamed one-workgroup-per-
node splits above that), attention within the GPU tolerances.  An out-of-bounds access in a
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
                             ("bsa_bwd", "attn_driver.cpp", ["-DBT_SIM_BSA_BWD"]),
                             ("pipeline", "pipeline_driver.cpp", [])):
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


@pytest.fixture(scope="module")
def sim_tsan(tmp_path_factory):
    """The tree and pipeline drivers under ThreadSanitizer: the emulation runs
    every lane as a host thread, so LDS or memory shared between the lanes or
    waves of a workgroup without a barrier or an atomic is reported as a race."""
    if not os.path.exists(CXX):
        pytest.skip("clang++ not available")
    d = tmp_path_factory.mktemp("cpu_sim_tsan")
    flags = ["-std=c++20", "-O1", "-g", "-fsanitize=thread", "-fno-omit-frame-pointer",
             "-I", SIM, "-I", os.path.join(ROOT, "include")]
    bins, procs = {"dir": d}, []
    for name, src in (("tree", "tree_driver.cpp"), ("pipeline", "pipeline_driver.cpp")):
        out = str(d / name)
        procs.append(subprocess.Popen([CXX, *flags, os.path.join(SIM, src),
                                       os.path.join(SIM, "emu.cpp"), "-o", out, "-lpthread"],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                      text=True))
        bins[name] = out
    for p in procs:
        o, _ = p.communicate()
        assert p.returncode == 0, o[-4000:]
    return bins


@pytest.fixture(scope="module")
def sim_msan(tmp_path_factory):
    """The tree driver under MemorySanitizer, with its workspace left
    uninitialised and every LDS array marked uninitialised when a workgroup
    starts (tests/cpu_sim/msan_lds.h): a read of either before any write that
    steers a branch or an address is reported."""
    if not os.path.exists(CXX):
        pytest.skip("clang++ not available")
    d = tmp_path_factory.mktemp("cpu_sim_msan")
    out = str(d / "tree")
    r = subprocess.run([CXX, "-std=c++20", "-O1", "-g", "-fsanitize=memory",
                        "-fno-omit-frame-pointer", "-DBT_SIM_UNINIT_WS", "-include",
                        os.path.join(SIM, "msan_lds.h"), "-I", SIM, "-I",
                        os.path.join(ROOT, "include"), os.path.join(SIM, "tree_driver.cpp"),
                        os.path.join(SIM, "emu.cpp"), "-o", out, "-lpthread"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    return {"dir": d, "tree": out}


@pytest.mark.parametrize("case", ["lds_builder", "streamed", "padded", "padded_lds"])
def test_tree_kernels_no_uninitialised_reads(sim_msan, case):
    """The rotated-pair recipe rotated, leaf 128, at 4,096 points (in LDS by
    one workgroup) and 16,384 points (streamed splits, then LDS), and padded
    trees of 972 and 5,000 points: nothing uninitialised is read, and the
    permutations are the oracle's."""
    d_ = sim_msan["dir"]
    env = dict(os.environ, EMU_SHUFFLE="4")
    if case.startswith("padded"):
        n, leaf = (972, 32) if case == "padded" else (5000, 64)
        c = synth.uniform_cube(np.random.default_rng(11), n)
        c.astype(np.float32).tofile(d_ / "coords.bin")
        args, want = ["padded", "coords.bin", str(n), str(leaf), "out.bin"], T.build_padded(c, leaf)
    else:
        n = 4096 if case == "lds_builder" else 16384
        w = synth.make("rotpair", n=n, features=False)
        w.coords.astype(np.float32).tofile(d_ / "coords.bin")
        w.R.astype(np.float32).tofile(d_ / "R.bin")
        args = ["coords.bin", str(n), "128", "out.bin", "R.bin"]
        want = T.rotate_build(w.coords, 128, w.R)
    r = subprocess.run([sim_msan["tree"], *args], cwd=d_, capture_output=True, text=True,
                       timeout=900, env=env)
    assert r.returncode == 0 and "MemorySanitizer" not in r.stderr, r.stderr[-4000:]
    assert np.array_equal(np.fromfile(d_ / "out.bin", np.int32), want)


def _tsan_env(shuffle):
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1 report_signal_unsafe=0")
    env["EMU_SHUFFLE"] = str(shuffle)
    return env


@pytest.mark.parametrize("n", [4096, 16384], ids=["lds_builder", "streamed"])
def test_tree_kernels_no_races(sim_tsan, n):
    """The rotated-pair recipe at 4,096 points (built in LDS by one
    workgroup) and 16,384 points (streamed splits, then one workgroup per
    node in LDS), leaf 128, plain and rotated: no data race, and the
    permutations are the oracle's."""
    d_ = sim_tsan["dir"]
    w = synth.make("rotpair", n=n, features=False)
    w.coords.astype(np.float32).tofile(d_ / "coords.bin")
    w.R.astype(np.float32).tofile(d_ / "R.bin")
    for rot in (False, True):
        args = [sim_tsan["tree"], "coords.bin", str(n), "128", "out.bin"] + (["R.bin"] if rot else [])
        r = subprocess.run(args, cwd=d_, capture_output=True, text=True, timeout=900,
                           env=_tsan_env(3))
        assert r.returncode == 0 and "ThreadSanitizer" not in r.stderr, r.stderr[-4000:]
        want = T.rotate_build(w.coords, 128, w.R) if rot else T.build(w.coords, 128)
        assert np.array_equal(np.fromfile(d_ / "out.bin", np.int32), want)


def test_rotated_pair_pipeline_no_races(sim_tsan):
    """The rotated-pair pipeline (both trees, ball attention, gathers,
    scatter, inverse) at 4,096 points and 2 heads: no data race."""
    from oracle import permute as P
    d_ = sim_tsan["dir"]
    n, H = 4096, 2
    w = synth.make("rotpair", n=n, features=False)
    rng = np.random.default_rng(n)
    q, k, v = (synth.normal_features(rng, n, H, 32, "bf16") for _ in range(3))
    w.coords.astype(np.float32).tofile(d_ / "coords.bin")
    w.R.astype(np.float32).tofile(d_ / "R.bin")
    for t, nm in ((q, "q.bin"), (k, "k.bin"), (v, "v.bin")):
        _dump(t, d_ / nm)
    r = subprocess.run([sim_tsan["pipeline"], str(n), str(w.leaf), str(w.ball), str(H), "32"],
                       cwd=d_, capture_output=True, text=True, timeout=1800, env=_tsan_env(9))
    assert r.returncode == 0 and "done" in r.stdout and "ThreadSanitizer" not in r.stderr, \
        r.stderr[-4000:]
    pb = np.fromfile(d_ / "pb.bin", np.int32)
    assert np.array_equal(pb, T.rotate_build(w.coords, w.leaf, w.R))
    assert np.array_equal(np.fromfile(d_ / "inv.bin", np.int32), P.invert(pb))


# Cases that take minutes of emulation run only with BT_SIM_SLOW=1 (their
# results are recorded with the tree notes of the design document).
SLOW = pytest.mark.skipif(os.environ.get("BT_SIM_SLOW") != "1",
                          reason="long emulation: set BT_SIM_SLOW=1")


def _env(shuffle):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    if shuffle is not None:
        env["EMU_SHUFFLE"] = str(shuffle)
    return env


def _tree(sim, coords, leaf, R=None, shuffle=None, timeout=600):
    d = sim["dir"]
    c = d / "c.bin"
    np.ascontiguousarray(coords, np.float32).tofile(c)
    args = [sim["tree"], str(c), str(len(coords)), str(leaf), str(d / "p.bin")]
    if R is not None:
        np.asarray(R, np.float32).tofile(d / "R.bin")
        args.append(str(d / "R.bin"))
    r = subprocess.run(args, capture_output=True, text=True, timeout=timeout,
                       env=_env(shuffle))
    assert r.returncode == 0 and "done" in r.stdout, r.stderr[-4000:]
    return np.fromfile(d / "p.bin", np.int32)


@pytest.mark.parametrize("case", ["cube4k_leaf32", "lattice2k_leaf8", "signed_zeros2k_leaf2",
                                  "mixture4k_leaf16", "leaf2048", "cube1536_leaf3",
                                  "cube2000_leaf1000", "lattice8k_leaf16"])
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
    elif case == "cube2000_leaf1000":     # chunks that are not a multiple of 256
        c, leaf = synth.uniform_cube(rng, 2000), 1000
    else:                                 # the largest tree built in LDS
        c, leaf = rng.integers(0, 5, size=(8192, 3)).astype(np.float32), 16
    assert np.array_equal(_tree(sim, c, leaf), T.build(c, leaf))


@pytest.mark.parametrize("n,leaf,rot", [(16384, 128, True), (32768, 16384, False)],
                         ids=["rotpair16k_rotated", "leaf16384"])
def test_streamed_tree_kernels_bit_exact(sim, n, leaf, rot):
    """Trees above 8,192 points: one workgroup per node streamed through the
    workspace's two record arrays (AddressSanitizer on the exact-size
    workspace), then one workgroup per node in LDS, or the leaves directly."""
    w = synth.make("rotpair", n=n, features=False)
    R = w.R if rot else None
    want = T.rotate_build(w.coords, leaf, R) if rot else T.build(w.coords, leaf)
    assert np.array_equal(_tree(sim, w.coords, leaf, R=R, shuffle=6), want)


def test_rotated_tree_kernels_bit_exact(sim):
    w = synth.make("rotpair", n=4096, features=False)
    assert np.array_equal(_tree(sim, w.coords, 64, R=w.R), T.rotate_build(w.coords, 64, w.R))


@pytest.mark.parametrize("shuffle", [1, 2])
def test_tree_kernels_shuffled_workgroups(sim, shuffle):
    """Workgroups of every launch in a seeded random order (32,768 points,
    leaf 16: streamed levels of up to eight workgroups, then sixteen
    workgroups in LDS): the result does not depend on the order (no
    workgroup reads what another one of the same launch writes)."""
    w = synth.make("rotpair", n=32768, features=False)
    assert np.array_equal(_tree(sim, w.coords, 16, R=w.R, shuffle=shuffle),
                          T.rotate_build(w.coords, 16, w.R))


def _pipeline(sim, n, H, shuffle):
    """The rotated-pair pipeline of the rotated-pair workload's recipe at n
    points, every array in an allocation of its own (AddressSanitizer
    catches an access past any of them), compared with the oracle."""
    from oracle import permute as P
    d_ = sim["dir"]
    w = synth.make("rotpair", n=n, features=False)
    rng = np.random.default_rng(n)
    q, k, v = (synth.normal_features(rng, n, H, 32, "bf16") for _ in range(3))
    w.coords.astype(np.float32).tofile(d_ / "coords.bin")
    w.R.astype(np.float32).tofile(d_ / "R.bin")
    for t, nm in ((q, "q.bin"), (k, "k.bin"), (v, "v.bin")):
        _dump(t, d_ / nm)
    r = subprocess.run([sim["pipeline"], str(n), str(w.leaf), str(w.ball), str(H), "32"],
                       cwd=d_, capture_output=True, text=True, timeout=3600, env=_env(shuffle))
    assert r.returncode == 0 and "done" in r.stdout, r.stderr[-4000:]
    pa, pb = (np.fromfile(d_ / f, np.int32) for f in ("pa.bin", "pb.bin"))
    pa_ref, pb_ref = T.build(w.coords, w.leaf), T.rotate_build(w.coords, w.leaf, w.R)
    assert np.array_equal(pa, pa_ref) and np.array_equal(pb, pb_ref)
    assert np.array_equal(np.fromfile(d_ / "inv.bin", np.int32), P.invert(pb_ref))
    o1 = torch.from_numpy(_read_out(d_ / "o1.bin", n, H, 32, "bf16")).to(torch.bfloat16)
    assert np.abs(o1.float().numpy() - A.ball_attn(q, k, v, pa_ref, w.ball)).max() <= 2e-2
    o2 = _read_out(d_ / "o2.bin", n, H, 32, "bf16")
    assert np.abs(o2 - A.ball_attn(q, k, o1, pb_ref, w.ball)).max() <= 2e-2


def test_rotated_pair_pipeline(sim):
    """4,096 points, leaf = ball 128: both trees in LDS; ball attention in
    tree A, gather into tree B, attention, scatter back."""
    _pipeline(sim, 4096, 2, shuffle=5)


@SLOW
def test_rotated_pair_pipeline_16k_8_heads(sim):
    """The inputs of the pipeline case that faulted the GPU: the rotated-pair
    recipe at 16,384 points, leaf = ball 128, 8 heads of 32."""
    _pipeline(sim, 16384, 8, shuffle=7)


@SLOW
@pytest.mark.parametrize("leaf", [128, 64])
def test_sphere_65536_tree(sim, leaf):
    w = synth.make("sphere", features=False)
    assert np.array_equal(_tree(sim, w.coords, leaf, shuffle=leaf, timeout=3600),
                          T.build(w.coords, leaf))


@SLOW
def test_tree_many_nodes(sim):
    """524,288 points, leaf 128: eight streamed levels (up to 128
    workgroups), then 256 workgroups of 2,048 points in LDS."""
    w = synth.make("rotpair", n=524288, features=False)
    assert np.array_equal(_tree(sim, w.coords, 128, shuffle=11, timeout=7200),
                          T.build(w.coords, 128))


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


@pytest.mark.parametrize("n,H,d,big", [(512, 2, 32, False), (512, 1, 64, False),
                                       (768, 3, 32, False), (512, 2, 32, True),
                                       (512, 1, 64, True), (768, 3, 32, True)])
def test_ball_attn_kernels_stepped_scores(sim, n, H, d, big):
    """256-point balls whose scores climb or fall by 2^8 and more from one
    64-key stretch to the next.  big: one key per ball with a large
    component no query has, so that |q| max|k| is far above every score
    (the kernel then keeps a running maximum, raised mid-ball)."""
    from tests.helpers import ramp_scores
    d_ = sim["dir"]
    rng = np.random.default_rng(n + d + 5)
    q, k, v = (synth.normal_features(rng, n, H, d, "bf16") for _ in range(3))
    perm = rng.permutation(n).astype(np.int32)
    q, k = ramp_scores(q, k, perm, 256, seed=n, big_key=big)
    for t, nm in ((q, "q.bin"), (k, "k.bin"), (v, "v.bin")):
        _dump(t, d_ / nm)
    perm.tofile(d_ / "perm.bin")
    r = subprocess.run([sim["attn"], "ball", str(n), str(H), str(d), "256", "1"], cwd=d_,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and "done" in r.stdout, r.stderr[-4000:]
    out = _read_out(d_ / "out.bin", n, H, d, "bf16")
    err = np.abs(out - A.ball_attn(q, k, v, perm, 256)).max()
    assert err <= 2e-2, err


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


@pytest.mark.parametrize("qc,group,ball,block,topk,steps",
                         [(0, 64, 128, 64, 4, None), (1, 64, 128, 64, 4, None),
                          (0, 128, 128, 64, 4, None), (0, 32, 32, 32, 5, None),
                          (0, 64, 128, 64, 4, "halves"), (0, 64, 128, 64, 4, "halves+big"),
                          (1, 64, 128, 64, 4, "halves+big")])
def test_bsa_kernels(sim, qc, group, ball, block, topk, steps):
    """BSA, and BSA with group compression (qc = 1); group 128 runs two waves
    of 64 queries per workgroup; 32-point balls and 5 selected 32-key blocks
    leave 32-key tails in the ball and selection branches.  steps: scores
    that step up by about 2^12 half way through every ball, with the bound
    |q| max|k| small, or (big) far above every score, so that the kernel
    keeps a running maximum and raises it."""
    from tests.helpers import step_ball_halves
    d_ = sim["dir"]
    n, H, d = 2048, 2, 32
    rng = np.random.default_rng(5)
    c = synth.deformed_sphere(rng, n)
    q, k, v = (synth.normal_features(rng, n, H, d, "bf16") for _ in range(3))
    W = (0.02 * rng.standard_normal((3, d))).astype(np.float32)
    perm = T.build(c, block).astype(np.int32)
    if steps:
        q, k = step_ball_halves(q, k, perm, ball, big_key=steps.endswith("big"))
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


@pytest.mark.parametrize("n,d,block,group,gm", [
    pytest.param(2048, 32, 64, 64, 0, marks=SLOW),      # minutes of emulation each
    (2048, 32, 32, 32, 1),
    pytest.param(1024, 64, 32, 128, 0, marks=SLOW)])
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
        assert err <= (2e-2 if dtype == "bf16" else 1e-5), (name, err)


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
                                    (2, 1), (700, 700), (1024, 32), (129, 1),
                                    (3586, 32), (5000, 64), (1025, 1), (6001, 3), (2049, 2048),
                                    (9000, 64), (20000, 8192)])
def test_padded_tree_kernels_bit_exact(sim, n, leaf):
    """Uneven N: the padded tree (one workgroup in LDS up to 8,192 slots;
    above that streamed splits of the padded segments, then LDS or the
    leaves directly), bit for bit."""
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
