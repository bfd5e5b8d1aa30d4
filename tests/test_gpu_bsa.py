"""GPU parity of bsa_attn against the brute-force fp64 oracle.

Top-k selection is discontinuous: one fp32 rounding can swap a block near
the k-th score.  The GPU returns its selected blocks; a (group, head) whose
set differs from the oracle's is accepted only if every differing block's
fp64 score is within tau = 1e-4 * max|s| of the oracle's k-th score, and the
oracle output is then recomputed with the GPU's set.
"""
import numpy as np
import pytest
import torch

from ball_tree_sparse_amd import ops, synth
from oracle import attention as A
from oracle import bsa as B
from oracle import tree as T
from tests.helpers import gpu, max_abs, say, step_ball_halves

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _setup(n, H, d, seed, leaf):
    rng = np.random.default_rng(seed)
    c = synth.deformed_sphere(rng, n)
    q, k, v = [synth.normal_features(rng, n, H, d, "bf16") for _ in range(3)]
    W = (0.02 * rng.standard_normal((3, d))).astype(np.float32)
    perm = T.build(c, leaf)
    return c, q, k, v, W, perm


def _check_sel(sel_gpu, parts, topk, tau_rel=1e-4):
    """Returns the selection the oracle must use and the count of rows whose
    set differs (each difference must be a near-tie)."""
    sel_o, s = parts["sel"], parts["scores"]          # [H,G,k], [G,H,Nc]
    H, G, _ = sel_o.shape
    use = sel_o.copy()
    ambiguous = 0
    for h in range(H):
        for g in range(G):
            a, b = set(sel_o[h, g].tolist()), set(sel_gpu[h, g].tolist())
            if a == b:
                continue
            ambiguous += 1
            sc = s[g, h]
            kth = np.sort(sc[sel_o[h, g]])[0]
            tau = tau_rel * np.max(np.abs(sc[np.isfinite(sc)]))
            for j in a ^ b:
                assert abs(sc[j] - kth) <= tau, (h, g, j, sc[j], kth)
            use[h, g] = sel_gpu[h, g]
    return use, ambiguous


def _run(q, k, v, perm, W, ball, block, group, topk, mask, gate_const=None, qc=False):
    dev = gpu()
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    pd = torch.from_numpy(np.asarray(perm, np.int32)).to(dev)
    Wd = None if gate_const is not None else torch.from_numpy(W).to(dev)
    out, sel = ops.bsa_attn(qd, kd, vd, pd, ball, block, group, topk, mask, gate_w=Wd,
                            gate_const=gate_const, return_sel=True, query_compression=qc)
    torch.cuda.synchronize()
    return out.cpu(), sel.cpu().numpy()


@pytest.mark.parametrize("n,H,d,ball,block,group,topk,mask,gates", [
    (4096, 2, 32, 128, 64, 64, 4, True, None),
    (4096, 2, 32, 128, 64, 64, 4, True, (1, 0, 0)),
    (4096, 2, 32, 128, 64, 64, 4, True, (0, 1, 0)),
    (4096, 2, 32, 128, 64, 64, 4, True, (0, 0, 1)),
    (4096, 3, 64, 256, 128, 128, 3, False, None),
    (8192, 2, 32, 64, 32, 32, 5, True, None),
    (4096, 1, 32, 128, 32, 64, 64, True, None),       # 64 blocks selected
    (65536, 1, 32, 64, 32, 32, 8, True, None),        # 2,048 blocks: scores kept in LDS
    (8192, 2, 32, 256, 64, 128, 8, True, None),       # two 64-query waves per group
    (8192, 2, 32, 256, 128, 256, 4, False, None),     # four 64-query waves per group
    (4096, 2, 32, 32, 32, 32, 4, True, None),         # 32-point balls: one 32-key block
    (4096, 2, 64, 64, 32, 32, 3, True, None),         # d 64, 96 selected keys: a 32-key tail
])
def test_parity(n, H, d, ball, block, group, topk, mask, gates):
    _, q, k, v, W, perm = _setup(n, H, d, seed=n + H + d + topk, leaf=block)
    say("bsa_attn", n, H, d, ball, block, group, topk, mask, gates)
    out, sel = _run(q, k, v, perm, W, ball, block, group, topk, mask, gates)
    ref, parts = B.bsa(q, k, v, perm, ball, block, group, topk, mask,
                       W=None if gates else W, gate_const=gates, return_parts=True)
    use, amb = _check_sel(sel, parts, topk)
    if amb:
        ref = B.bsa(q, k, v, perm, ball, block, group, topk, mask,
                    W=None if gates else W, gate_const=gates, sel_override=use)
    assert max_abs(out, ref) <= TOL


@pytest.mark.parametrize("qc", [False, True])
@pytest.mark.parametrize("big", [False, True])
def test_parity_scores_stepping_within_balls(big, qc):
    """Keys of the second 64-key stretch of every ball score about 2^12
    higher than those of the first.  big: one key per block with a large
    component no query has, so that the bound |q| max|k| is far above every
    score and the branches keep a running maximum, raised part way through
    each ball."""
    n, H, d, ball, block, group, topk = 4096, 2, 32, 128, 64, 64, 4
    _, q, k, v, W, perm = _setup(n, H, d, seed=17, leaf=block)
    q, k = step_ball_halves(q, k, perm, ball, big_key=big)
    say("bsa stepped scores", big, qc)
    out, sel = _run(q, k, v, perm, W, ball, block, group, topk, True, qc=qc)
    ref, parts = B.bsa(q, k, v, perm, ball, block, group, topk, True, W=W, return_parts=True,
                       query_compression=qc)
    use, amb = _check_sel(sel, parts, topk)
    if amb:
        ref = B.bsa(q, k, v, perm, ball, block, group, topk, True, W=W, sel_override=use,
                    query_compression=qc)
    assert max_abs(out, ref) <= TOL


def test_gates_100_equal_ball_attention_on_gpu():
    """BSA with gates (1,0,0) reduces to ball attention."""
    dev = gpu()
    _, q, k, v, W, perm = _setup(4096, 4, 32, seed=5, leaf=64)
    say("bsa gates (1,0,0) vs ball_attn")
    out, _ = _run(q, k, v, perm, W, 128, 64, 64, 4, True, (1, 0, 0))
    pd = torch.from_numpy(np.asarray(perm, np.int32)).to(dev)
    ba = ops.ball_attn(q.to(dev), k.to(dev), v.to(dev), pd, 128)
    torch.cuda.synchronize()
    assert max_abs(out, ba.cpu()) <= TOL
    assert max_abs(out, A.ball_attn(q, k, v, perm, 128)) <= TOL


def test_zero_queries_select_lowest_blocks():
    """Q = 0: all selection scores tie at 0, so the lowest-index unmasked
    blocks are taken (pins the tie-break on the GPU)."""
    _, q, k, v, W, perm = _setup(4096, 2, 32, seed=6, leaf=64)
    q = torch.zeros_like(q)
    say("bsa zero queries")
    out, sel = _run(q, k, v, perm, W, 128, 64, 64, 4, True, None)
    for g in range(4096 // 64):
        b = (g * 64) // 128
        masked = {2 * b, 2 * b + 1}
        want = [j for j in range(64) if j not in masked][:4]
        assert sel[0, g].tolist() == want and sel[1, g].tolist() == want
    ref = B.bsa(q, k, v, perm, 128, 64, 64, 4, True, W=W)
    assert max_abs(out, ref) <= TOL


def test_bsa_workload_full_size():
    """N=65,536 sphere, ball 128, block 64, group 64, top-16, gates from a
    random Linear(d->3) with weights N(0, 0.02^2)."""
    w = synth.make("bsa")
    perm = T.build(w.coords, w.leaf)
    x = w.extra
    say("bsa workload full size")
    out, sel = _run(w.q, w.k, w.v, perm, w.gate_w, w.ball, x["block"], x["group"], x["topk"],
                    bool(x["mask_own_ball"]))
    ref, parts = B.bsa(w.q, w.k, w.v, perm, w.ball, x["block"], x["group"], x["topk"], True,
                       W=w.gate_w, return_parts=True)
    use, amb = _check_sel(sel, parts, x["topk"])
    if amb:
        ref = B.bsa(w.q, w.k, w.v, perm, w.ball, x["block"], x["group"], x["topk"], True,
                    W=w.gate_w, sel_override=use)
    print(f"ambiguous top-k rows: {amb}")
    assert max_abs(out, ref) <= TOL


def test_deterministic():
    _, q, k, v, W, perm = _setup(8192, 4, 32, seed=8, leaf=64)
    say("bsa determinism")
    a, sa = _run(q, k, v, perm, W, 128, 64, 64, 8, True)
    b, sb = _run(q, k, v, perm, W, 128, 64, 64, 8, True)
    assert torch.equal(a, b) and np.array_equal(sa, sb)


# ---- group (query) compression --------------------------------------------

@pytest.mark.parametrize("n,H,d,ball,block,group,topk,mask,gates", [
    (4096, 2, 32, 128, 64, 64, 4, True, None),
    (4096, 2, 32, 128, 64, 64, 4, True, (0, 1, 0)),   # compression only
    (4096, 2, 32, 128, 64, 64, 4, True, (0, 0, 1)),   # selection only
    (8192, 2, 32, 128, 32, 64, 6, True, None),        # block != group
    (4096, 3, 64, 256, 128, 128, 3, False, None),
])
def test_parity_query_compression(n, H, d, ball, block, group, topk, mask, gates):
    _, q, k, v, W, perm = _setup(n, H, d, seed=n + H + d + topk + 1, leaf=block)
    say("bsa_attn group compression", n, H, d, ball, block, group, topk, mask, gates)
    out, sel = _run(q, k, v, perm, W, ball, block, group, topk, mask, gates, qc=True)
    kw = dict(W=None if gates else W, gate_const=gates, query_compression=True)
    ref, parts = B.bsa(q, k, v, perm, ball, block, group, topk, mask, return_parts=True, **kw)
    use, amb = _check_sel(sel, parts, topk)
    if amb:
        ref = B.bsa(q, k, v, perm, ball, block, group, topk, mask, sel_override=use, **kw)
    assert max_abs(out, ref) <= TOL


def test_query_compression_full_size():
    """The 65,536-point BSA workload with group compression."""
    w = synth.make("bsa")
    perm = T.build(w.coords, w.leaf)
    x = w.extra
    say("bsa group compression full size")
    out, sel = _run(w.q, w.k, w.v, perm, w.gate_w, w.ball, x["block"], x["group"], x["topk"],
                    bool(x["mask_own_ball"]), qc=True)
    kw = dict(W=w.gate_w, query_compression=True)
    ref, parts = B.bsa(w.q, w.k, w.v, perm, w.ball, x["block"], x["group"], x["topk"], True,
                       return_parts=True, **kw)
    use, amb = _check_sel(sel, parts, x["topk"])
    if amb:
        ref = B.bsa(w.q, w.k, w.v, perm, w.ball, x["block"], x["group"], x["topk"], True,
                    sel_override=use, **kw)
    assert max_abs(out, ref) <= TOL
