"""CPU checks of the C ABI: the library loads, exports every symbol that
include/bt.h declares, and rejects bad arguments before touching a device."""
import ctypes as C
import os
import re

import pytest

from ball_tree_sparse_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "bt.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", src)
    keep = [n for n in names if n.startswith(("bt_", "ball_attn", "bsa_"))]
    return sorted(set(keep))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ops.LIB_PATH):
        pytest.skip("library not built")
    return ops.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert "bt_build" in names and "ball_attn" in names and "bsa_attn" in names
    for n in names:
        assert hasattr(L, n), n
    assert sorted(names) == sorted(ops.EXPORTS)


def test_status_strings(L):
    for s in range(4):
        assert L.bt_status_str(s)
    assert b"gfx950" in L.bt_version()


def _fake(n=1):
    """Host buffers used as stand-in pointers: every call below is rejected
    before the library could dereference them."""
    return C.cast(C.create_string_buffer(max(n, 16) + 256), C.c_void_p)


def test_build_rejects(L):
    f = _fake()
    assert L.bt_build(None, 8, 2, f, f, 1 << 20, None) == ops.BT_EINVAL
    assert L.bt_build(f, 12, 4, f, f, 1 << 20, None) == ops.BT_EINVAL      # 12/4 not 2^L
    assert b"leaf" in L.bt_last_error()
    assert L.bt_build(f, 0, 1, f, f, 1 << 20, None) == ops.BT_EINVAL
    assert L.bt_build(f, 1 << 31, 1, f, f, 1 << 20, None) == ops.BT_EINVAL
    assert L.bt_build(f, 8, 2, f, None, 1 << 20, None) == ops.BT_EINVAL
    assert L.bt_build_workspace_size(12, 4) == 0
    assert L.bt_build_workspace_size(1024, 32) == 256    # built in LDS from coords
    assert L.bt_build_workspace_size(8192, 32) == 256
    assert L.bt_build_workspace_size(16384, 32) >= 2 * 16384 * 16   # two record arrays


def test_build_rejects_short_workspace(L):
    buf = C.create_string_buffer(4096 + 512)
    addr = (C.addressof(buf) + 255) & ~255
    f = _fake()
    assert L.bt_build(f, 16384, 32, f, C.c_void_p(addr), 4096, None) == ops.BT_ENOMEM
    assert L.bt_build(f, 16384, 32, f, C.c_void_p(addr + 8), 1 << 30, None) == ops.BT_EINVAL


def test_rotate_rejects_nonfinite(L):
    f = _fake()
    R = (C.c_float * 9)(1, 0, 0, 0, float("nan"), 0, 0, 0, 1)
    assert L.bt_rotate_build(f, 8, 2, R, f, f, 1 << 20, None) == ops.BT_EINVAL
    R = (C.c_float * 9)(1, 0, 0, 0, float("inf"), 0, 0, 0, 1)
    assert L.bt_rotate_build(f, 8, 2, R, f, f, 1 << 20, None) == ops.BT_EINVAL
    assert L.bt_rotate_build(f, 8, 2, None, f, f, 1 << 20, None) == ops.BT_EINVAL


def test_permute_rejects(L):
    a, b = _fake(1024), _fake(1024)
    assert L.bt_permute(a, a, 8, 6, 0, b, None) == ops.BT_EINVAL          # row_bytes % 4
    assert L.bt_permute(a, a, 8, 16, 2, b, None) == ops.BT_EINVAL         # bad mode
    assert L.bt_permute(a, a, 8, 16, 0, a, None) == ops.BT_EINVAL         # src == dst
    assert L.bt_permute(a, a, -1, 16, 0, b, None) == ops.BT_EINVAL
    assert L.bt_permute(None, None, 0, 16, 0, None, None) == ops.BT_OK    # empty is a no-op
    assert L.bt_invert_perm(a, 4, a, None) == ops.BT_EINVAL               # overlap


def test_count_nonfinite_rejects(L):
    a = _fake(64)
    assert L.bt_count_nonfinite(a, -1, a, None) == ops.BT_EINVAL
    assert L.bt_count_nonfinite(a, 4, None, None) == ops.BT_EINVAL
    assert L.bt_count_nonfinite(None, 4, a, None) == ops.BT_EINVAL
    assert L.bt_count_nonfinite(a, 4, C.c_void_p(a.value + 2), None) == ops.BT_EINVAL


def test_ball_attn_rejects(L):
    q, k, v, o = (_fake(1 << 16) for _ in range(4))
    args = lambda **kw: dict(dict(q=q, k=k, v=v, perm=None, N=1024, ball=32, H=4, d=16,
                                  dt=ops.BT_F32, out=o), **kw)
    call = lambda a: L.ball_attn(a["q"], a["k"], a["v"], a["perm"], a["N"], a["ball"], a["H"],
                                 a["d"], a["dt"], a["out"], None)
    assert call(args(ball=48)) == ops.BT_EINVAL          # 48 does not divide 1024
    assert call(args(d=24)) == ops.BT_EINVAL
    assert call(args(H=0)) == ops.BT_EINVAL
    assert call(args(dt=7)) == ops.BT_EINVAL
    assert call(args(out=q)) == ops.BT_EINVAL            # aliasing
    assert call(args(q=None)) == ops.BT_EINVAL
    assert call(args(ball=8192, N=8192)) == ops.BT_EINVAL
    buf = C.create_string_buffer(64)
    pa = (C.addressof(buf) + 15) & ~15
    assert call(args(perm=C.c_void_p(pa + 4), N=64)) == ops.BT_EINVAL    # perm misaligned
    assert b"aligned" in L.bt_last_error()
    # no points: a no-op that touches no pointer; shape checks still apply
    assert call(args(N=0, q=None, k=None, v=None, out=None)) == ops.BT_OK
    assert call(args(N=0, d=24, q=None, k=None, v=None, out=None)) == ops.BT_EINVAL


def test_bsa_rejects(L):
    q, k, v, o, p, ws = (_fake(1 << 16) for _ in range(6))
    P = ops.BsaParams
    gc = (C.c_float * 3)(1, 0, 0)
    def call(params, N=4096, H=2, d=32, dt=ops.BT_BF16, gw=None, gcc=gc, wsb=1 << 30):
        return L.bsa_attn(q, k, v, p, N, H, d, dt, C.byref(params), gw, None, gcc, None, ws,
                          wsb, o, None)
    assert call(P(128, 64, 64, 4, 1), dt=ops.BT_F32) == ops.BT_EINVAL
    assert call(P(128, 48, 64, 4, 1)) == ops.BT_EINVAL    # block not multiple of 32
    assert call(P(128, 64, 96, 4, 1)) == ops.BT_EINVAL    # group vs ball
    assert call(P(128, 64, 64, 65, 1)) == ops.BT_EINVAL   # topk too large
    assert call(P(128, 64, 64, 4, 1), d=16) == ops.BT_EINVAL
    assert call(P(128, 64, 64, 4, 1), gw=ws) == ops.BT_EINVAL   # both gates given
    assert call(P(128, 64, 64, 4, 1), gcc=None) == ops.BT_EINVAL  # no gate
    assert L.bsa_workspace_size(4096, 2, 32, C.byref(P(128, 64, 64, 4, 1))) > 0
    assert L.bsa_workspace_size(4096, 2, 32, C.byref(P(100, 64, 64, 4, 1))) == 0


def test_bsa_bwd_rejects(L):
    # distinct, 256-byte aligned stand-ins, each as large as a [4096, 2, 32] bf16 tensor
    bufs = [C.create_string_buffer(4096 * 2 * 32 * 2 + 512) for _ in range(9)]
    a = [C.c_void_p((C.addressof(b) + 255) & ~255) for b in bufs]
    q, k, v, perm, do, dq, dk, dv, ws = a
    P = ops.BsaParams
    gc = (C.c_float * 3)(1, 0, 0)
    gw = _fake(3 * 32 * 4)

    def call(params=None, N=4096, H=2, d=32, dt=ops.BT_BF16, gates=(None, gc), grads=(None, None),
             outs=(dq, dk, dv), wsb=1 << 30):
        params = params or P(128, 64, 64, 4, 1, 0)
        return L.bsa_attn_bwd(q, k, v, perm, do, N, H, d, dt, C.byref(params), gates[0], None,
                              gates[1], outs[0], outs[1], outs[2], grads[0], grads[1], ws, wsb,
                              None)
    assert call(dt=ops.BT_F32) == ops.BT_EINVAL
    assert call(P(128, 64, 64, 4, 1, 1)) == ops.BT_EINVAL          # group compression
    assert call(P(128, 48, 64, 4, 1, 0)) == ops.BT_EINVAL          # block not multiple of 32
    assert call(d=16) == ops.BT_EINVAL
    assert call(gates=(gw, gc)) == ops.BT_EINVAL                   # both gates given
    assert call(gates=(None, None)) == ops.BT_EINVAL               # no gate
    assert call(grads=(gw, None)) == ops.BT_EINVAL                 # constant gates: no dW
    assert call(outs=(q, dk, dv)) == ops.BT_EINVAL                 # dq is q
    assert call(outs=(dq, dq, dv)) == ops.BT_EINVAL                # dk is dq
    assert call(outs=(dq, dk, None)) == ops.BT_EINVAL
    assert call(wsb=4096) == ops.BT_ENOMEM
    assert L.bsa_attn_bwd_workspace_size(4096, 2, 32, C.byref(P(128, 64, 64, 4, 1, 0))) > \
        L.bsa_workspace_size(4096, 2, 32, C.byref(P(128, 64, 64, 4, 1, 0)))
    assert L.bsa_attn_bwd_workspace_size(4096, 2, 32, C.byref(P(128, 64, 64, 4, 1, 1))) == 0


def test_coarsen_refine_reject(L):
    x, o = _fake(1 << 16), _fake(1 << 16)
    for f in (L.bt_coarsen, L.bt_refine):
        assert f(x, None, 1024, 4, 32, 3, ops.BT_BF16, o, None) == ops.BT_EINVAL   # 3 does not divide
        assert f(x, None, 1024, 1, 2, 2, ops.BT_F32, o, None) == ops.BT_EINVAL     # 8-byte rows
        assert f(x, None, 1024, 4, 32, 0, ops.BT_BF16, o, None) == ops.BT_EINVAL
        assert f(x, None, 1024, 4, 32, 2, 7, o, None) == ops.BT_EINVAL
        assert f(None, None, 1024, 4, 32, 2, ops.BT_BF16, o, None) == ops.BT_EINVAL
        assert f(x, None, 1024, 4, 32, 2, ops.BT_BF16, x, None) == ops.BT_EINVAL   # overlap
        assert f(None, None, 0, 4, 32, 2, ops.BT_BF16, None, None) == ops.BT_OK    # empty


def test_ball_attn_bwd_rejects(L):
    t = [_fake(1 << 16) for _ in range(7)]
    def call(N=1024, ball=32, H=4, d=16, dt=ops.BT_F32, ptrs=None):
        p = t if ptrs is None else ptrs
        return L.ball_attn_bwd(p[0], p[1], p[2], p[3], None, N, ball, H, d, dt, p[4], p[5], p[6],
                               None)
    assert call(ball=2048, N=2048) == ops.BT_EINVAL           # ball above 1024
    assert call(ball=48) == ops.BT_EINVAL                      # 48 does not divide 1024
    assert call(d=24) == ops.BT_EINVAL
    assert call(ptrs=[t[0], t[1], t[2], t[3], t[0], t[5], t[6]]) == ops.BT_EINVAL   # dq aliases q
    assert call(ptrs=[t[0], t[1], t[2], t[3], t[4], t[4], t[6]]) == ops.BT_EINVAL   # dq is dk
    assert call(N=0, ptrs=[None] * 7) == ops.BT_OK


def test_padded_size_and_workspace(L):
    assert L.bt_padded_size(972, 32) == 1024
    assert L.bt_padded_size(1024, 32) == 1024
    assert L.bt_padded_size(3586, 128) == 4096
    assert L.bt_padded_size(1, 1) == 1
    assert L.bt_padded_size(700, 700) == 700
    assert L.bt_padded_size(0, 4) == -1
    assert L.bt_padded_size(5, 0) == -1
    assert L.bt_padded_size((1 << 31) - 1, 3) == -1          # slots would reach 2^31
    assert L.bt_build_padded_workspace_size(0, 4) == 0
    assert L.bt_build_padded_workspace_size(972, 32) == 256


def test_build_padded_rejects(L):
    f = _fake()
    assert L.bt_build_padded(None, 10, 2, None, f, f, 1 << 20, None) == ops.BT_EINVAL
    assert L.bt_build_padded(f, 0, 2, None, f, f, 1 << 20, None) == ops.BT_EINVAL
    assert L.bt_build_padded_workspace_size(9000, 128) > 2 * 9000 * 16   # streamed
    assert L.bt_build_padded_workspace_size(5000, 64) == 256                 # in LDS
    bad = (C.c_float * 9)(1, 0, 0, 0, float("inf"), 0, 0, 0, 1)
    assert L.bt_build_padded(f, 10, 2, bad, f, f, 1 << 20, None) == ops.BT_EINVAL
    buf = C.create_string_buffer(4096 + 512)
    addr = (C.addressof(buf) + 255) & ~255
    assert L.bt_build_padded(f, 10, 2, None, f, C.c_void_p(addr), 16, None) == ops.BT_ENOMEM
    assert L.bt_build_padded(f, 10, 2, None, f, C.c_void_p(addr + 8), 4096, None) == \
        ops.BT_EINVAL


def test_permute_padded_rejects(L):
    f = _fake(4096)
    assert L.bt_permute_padded(f, f, 5, 8, 6, ops.BT_GATHER, _fake(4096), None) == ops.BT_EINVAL
    assert L.bt_permute_padded(f, f, 9, 8, 16, ops.BT_GATHER, _fake(4096), None) == ops.BT_EINVAL
    assert L.bt_permute_padded(f, f, 0, 8, 16, ops.BT_GATHER, _fake(4096), None) == ops.BT_EINVAL
    assert L.bt_permute_padded(f, f, 5, 8, 16, 7, _fake(4096), None) == ops.BT_EINVAL
    assert L.bt_permute_padded(f, None, 5, 8, 16, ops.BT_SCATTER, _fake(4096), None) == \
        ops.BT_EINVAL
    assert L.bt_permute_padded(f, f, 5, 8, 16, ops.BT_GATHER, f, None) == ops.BT_EINVAL
    assert L.bt_permute_padded(None, None, 0, 0, 16, ops.BT_GATHER, None, None) == ops.BT_OK


def test_ball_attn_padded_rejects(L):
    a, b, c, o, p = (_fake(1 << 16) for _ in range(5))
    bf = ops.BT_BF16
    assert L.ball_attn_padded(a, b, c, p, 100, 96, 32, 2, 32, bf, o, None) == ops.BT_EINVAL
    assert b"n_rows" in L.bt_last_error()                       # more rows than slots
    assert L.ball_attn_padded(a, b, c, p, 90, 100, 32, 2, 32, bf, o, None) == ops.BT_EINVAL
    assert L.ball_attn_padded(a, b, c, None, 90, 96, 32, 2, 32, bf, o, None) == ops.BT_EINVAL
    assert L.ball_attn_padded(a, b, c, p, 90, 96, 32, 2, 48, bf, o, None) == ops.BT_EINVAL
    assert L.ball_attn_padded(a, b, c, p, 90, 96, 32, 2, 32, bf, a, None) == ops.BT_EINVAL
    assert L.ball_attn_padded(a, b, c, p, 0, 96, 32, 2, 32, bf, o, None) == ops.BT_EINVAL
