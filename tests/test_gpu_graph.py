"""ball_attn and bt_permute captured in a HIP graph (as bench.py times them):
every replay, with eager work and synchronisations in between, must equal the
eager result bit for bit."""
import numpy as np
import pytest
import torch

from ball_tree_sparse_amd import ops, synth
from tests.helpers import gpu, say

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    dev = gpu()
    rng = np.random.default_rng(3)
    q, k, v = (synth.normal_features(rng, 8192, 8, 32, "bf16").to(dev) for _ in range(3))
    perm = torch.from_numpy(rng.permutation(8192).astype(np.int32)).to(dev)
    say("graph capture ball_attn + bt_permute")
    eager = ops.ball_attn(q, k, v, perm, 128)
    eager_g = ops.bt_permute(eager, perm, ops.BT_GATHER)
    torch.cuda.synchronize()
    out = torch.empty_like(q)
    gat = torch.empty_like(q)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ops.ball_attn(q, k, v, perm, 128, out=out)
        ops.bt_permute(out, perm, ops.BT_GATHER, dst=gat)
    for r in range(4):
        out.zero_()
        gat.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), r
        assert torch.equal(gat, eager_g), r
        junk = (q.float() * 2).sum()          # eager work between replays
        torch.cuda.synchronize()
        del junk
