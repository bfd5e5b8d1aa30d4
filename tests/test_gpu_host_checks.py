"""Malformed arguments are refused by the binding before the library is
called: a short permutation, malformed coordinates or gate parameters of the
wrong shape raise ValueError, and the C ABI refuses a misaligned permutation
with BT_EINVAL, so no kernel ever indexes past an allocation."""
import pytest
import torch

from ball_tree_sparse_amd import ops
from tests.helpers import gpu, say

pytestmark = pytest.mark.gpu


def _qkv(dev, n=256, H=2, d=32):
    return [torch.zeros((n, H, d), dtype=torch.bfloat16, device=dev) for _ in range(3)]


def test_shape_errors_raise_before_launch():
    dev = gpu()
    say("host checks")
    q, k, v = _qkv(dev)
    short = torch.arange(255, dtype=torch.int32, device=dev)
    with pytest.raises(ValueError):
        ops.ball_attn(q, k, v, short, 128)
    with pytest.raises(ValueError):
        ops.bt_permute(q, short, ops.BT_GATHER)
    with pytest.raises(ValueError):
        ops.ball_attn_bwd(q, k, v, q.clone(), short, 128)
    with pytest.raises(ValueError):
        ops.bt_coarsen(q, short, 2)
    with pytest.raises(ValueError):
        ops.bt_build(torch.zeros((256, 2), device=dev), 32)          # not [N,3]
    with pytest.raises(ValueError):
        ops.bt_build(torch.zeros((256, 3), device=dev), 32,
                     perm=torch.empty(128, dtype=torch.int32, device=dev))
    perm = torch.arange(256, dtype=torch.int32, device=dev)
    with pytest.raises(ValueError):
        ops.bsa_attn(q, k, v, perm, 128, 64, 64, 2,
                     gate_w=torch.zeros((3, 16), device=dev))          # d is 32
    with pytest.raises(ValueError):
        ops.bsa_attn(q, k, v, perm, 128, 64, 64, 2,
                     gate_w=torch.zeros((3, 32), device=dev), gate_b=torch.zeros(4, device=dev))
    with pytest.raises(ValueError):
        ops.ball_attn(q, k, v, perm, 128, out=torch.empty((128, 2, 32), dtype=torch.bfloat16,
                                                          device=dev))
    torch.cuda.synchronize()


def test_misaligned_perm_is_refused():
    dev = gpu()
    say("misaligned perm")
    q, k, v = _qkv(dev)
    buf = torch.arange(257, dtype=torch.int32, device=dev)
    with pytest.raises(ops.BtError) as e:
        ops.ball_attn(q, k, v, buf[1:], 128)                          # 4 bytes off
    assert e.value.status == ops.BT_EINVAL
    torch.cuda.synchronize()
