"""Calls are stateless and re-entrant: the same calls on two streams at once,
each with its own workspace, give the results of running them one at a time
(bit for bit)."""
import numpy as np
import pytest
import torch

from ball_tree_sparse_amd import ops, synth
from tests.helpers import gpu, say

pytestmark = pytest.mark.gpu


def _inputs(dev, seed, n=16384):
    rng = np.random.default_rng(seed)
    q, k, v = (synth.normal_features(rng, n, 8, 32, "bf16").to(dev) for _ in range(3))
    perm = torch.from_numpy(rng.permutation(n).astype(np.int32)).to(dev)
    return q, k, v, perm


def _work(q, k, v, perm):
    a = ops.ball_attn(q, k, v, perm, 128)
    b = ops.bsa_attn(q, k, v, perm, 128, 64, 64, 8, True,
                     gate_const=(0.5, 0.25, 0.25))
    g = ops.ball_attn_bwd(q, k, v, a, perm, 128)
    gb = ops.bsa_attn_bwd(q, k, v, perm, a, 128, 64, 64, 8, True,
                          gate_const=(0.5, 0.25, 0.25))
    return [a, b, *g, *gb[:3]]


def test_two_streams_match_serial_runs():
    dev = gpu()
    x1, x2 = _inputs(dev, 1), _inputs(dev, 2)
    say("two streams: ball_attn, bsa_attn, ball_attn_bwd, bsa_attn_bwd")
    ref1 = _work(*x1)
    ref2 = _work(*x2)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    torch.cuda.current_stream().synchronize()
    with torch.cuda.stream(s1):
        out1 = _work(*x1)
    with torch.cuda.stream(s2):
        out2 = _work(*x2)
    torch.cuda.synchronize()
    for a, b in zip(out1, ref1):
        assert torch.equal(a, b)
    for a, b in zip(out2, ref2):
        assert torch.equal(a, b)
