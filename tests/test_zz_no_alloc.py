"""bsa_attn_noalloc (the static-workspace variant of bsa_attn for callers
that cannot allocate) against bsa_attn itself, through the C ABI: two calls
in a row, the second with a smaller input, each bit-identical to bsa_attn
(same kernels, same inputs); a call that needs more workspace than the static
array holds is refused before any launch."""
import numpy as np
import pytest
import torch

from ball_tree_sparse_amd import ops, synth
from tests.helpers import gpu, say

pytestmark = pytest.mark.gpu


def _case(dev, n, H, topk, qc):
    w = synth.make("bsa", n=n)
    if H != w.H:
        rng = np.random.default_rng(n + H)
        w.q, w.k, w.v = (synth.normal_features(rng, n, H, w.d, "bf16") for _ in range(3))
    x = w.extra
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(n)).to(torch.int32).to(dev)
    q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
    W = torch.from_numpy(w.gate_w).to(dev)
    args = (q, k, v, perm, w.ball, x["block"], x["group"], topk, True)
    return args, W


@pytest.mark.parametrize("qc", [False, True])
def test_noalloc_matches_bsa_attn_two_calls(qc):
    dev = gpu()
    for n, H, topk in ((65536, 8, 16), (4096, 4, 4)):          # second call smaller
        say("bsa_attn_noalloc", n, H, topk, "qc" if qc else "")
        args, W = _case(dev, n, H, topk, qc)
        ref, sel_ref = ops.bsa_attn(*args, gate_w=W, return_sel=True, query_compression=qc)
        got, sel = ops.bsa_attn_noalloc(*args, gate_w=W, return_sel=True, query_compression=qc)
        torch.cuda.synchronize()
        assert torch.equal(got.cpu(), ref.cpu())
        assert torch.equal(sel.cpu(), sel_ref.cpu())


def test_noalloc_refuses_oversized_call():
    dev = gpu()
    say("bsa_attn_noalloc oversized")
    n, H, d = 131072, 8, 64                 # needs about 269 MiB of workspace
    assert ops.bsa_workspace_size(n, H, d, 128, 64, 64, 16) > ops.lib().bsa_attn_noalloc_max_bytes()
    q = torch.zeros((n, H, d), dtype=torch.bfloat16, device=dev)
    perm = torch.arange(n, dtype=torch.int32, device=dev)
    with pytest.raises(ops.BtError) as e:
        ops.bsa_attn_noalloc(q, q.clone(), q.clone(), perm, 128, 64, 64, 16, True,
                             gate_const=(1.0, 0.0, 0.0))
    assert e.value.status == ops.BT_EINVAL
    torch.cuda.synchronize()
