"""ctypes binding of libbtsparse (include/bt.h).

Argument marshalling only: torch tensors become device pointers and the
current HIP stream; every step of the computation runs in the library's HIP
kernels.  There is no CPU fallback: if the library is missing or a tensor is
not on the GPU, the call raises.

Names follow the C ABI: ``bt_build``, ``bt_rotate_build``, ``bt_permute``,
``bt_invert_perm``, ``ball_attn``, ``bsa_attn``.  Output tensors and
workspaces are allocated with torch (device memory plumbing); the library
itself allocates nothing.
"""
from __future__ import annotations

import ctypes as C
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbtsparse.so")

BT_OK, BT_EINVAL, BT_EHIP, BT_ENOMEM = 0, 1, 2, 3
BT_F32, BT_BF16 = 0, 1
BT_GATHER, BT_SCATTER = 0, 1


class BtError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class BsaParams(C.Structure):
    _fields_ = [("ball", C.c_int32), ("block", C.c_int32), ("group", C.c_int32),
                ("topk", C.c_int32), ("mask_own_ball", C.c_int32),
                ("query_compression", C.c_int32)]


_lib = None

# (name, restype, argtypes) for every entry point in include/bt.h
_P = C.c_void_p
_SIGS = [
    ("bt_status_str", C.c_char_p, [C.c_int]),
    ("bt_last_error", C.c_char_p, []),
    ("bt_version", C.c_char_p, []),
    ("bt_build_workspace_size", C.c_size_t, [C.c_int64, C.c_int32]),
    ("bt_build", C.c_int, [_P, C.c_int64, C.c_int32, _P, _P, C.c_size_t, _P]),
    ("bt_rotate_build", C.c_int, [_P, C.c_int64, C.c_int32, C.POINTER(C.c_float), _P, _P,
                                  C.c_size_t, _P]),
    ("bt_permute", C.c_int, [_P, _P, C.c_int64, C.c_int64, C.c_int, _P, _P]),
    ("bt_invert_perm", C.c_int, [_P, C.c_int64, _P, _P]),
    ("bt_count_nonfinite", C.c_int, [_P, C.c_int64, _P, _P]),
    ("ball_attn", C.c_int, [_P, _P, _P, _P, C.c_int64, C.c_int32, C.c_int32, C.c_int32,
                            C.c_int, _P, _P]),
    ("bsa_workspace_size", C.c_size_t, [C.c_int64, C.c_int32, C.c_int32,
                                        C.POINTER(BsaParams)]),
    ("bsa_attn", C.c_int, [_P, _P, _P, _P, C.c_int64, C.c_int32, C.c_int32, C.c_int,
                           C.POINTER(BsaParams), _P, _P, C.POINTER(C.c_float), _P, _P,
                           C.c_size_t, _P, _P]),
    ("bt_coarsen", C.c_int, [_P, _P, C.c_int64, C.c_int32, C.c_int32, C.c_int32, C.c_int, _P,
                             _P]),
    ("bt_refine", C.c_int, [_P, _P, C.c_int64, C.c_int32, C.c_int32, C.c_int32, C.c_int, _P,
                            _P]),
    ("ball_attn_bwd", C.c_int, [_P, _P, _P, _P, _P, C.c_int64, C.c_int32, C.c_int32,
                                C.c_int32, C.c_int, _P, _P, _P, _P]),
    ("bsa_attn_bwd_workspace_size", C.c_size_t, [C.c_int64, C.c_int32, C.c_int32,
                                                 C.POINTER(BsaParams)]),
    ("bsa_attn_bwd", C.c_int, [_P, _P, _P, _P, _P, C.c_int64, C.c_int32, C.c_int32, C.c_int,
                               C.POINTER(BsaParams), _P, _P, C.POINTER(C.c_float), _P, _P, _P,
                               _P, _P, _P, C.c_size_t, _P]),
    ("bsa_attn_noalloc_max_bytes", C.c_size_t, []),
    ("bsa_attn_noalloc", C.c_int, [_P, _P, _P, _P, C.c_int64, C.c_int32, C.c_int32, C.c_int,
                                   C.POINTER(BsaParams), _P, _P, C.POINTER(C.c_float), _P, _P,
                                   _P]),
    ("bt_padded_size", C.c_int64, [C.c_int64, C.c_int32]),
    ("bt_build_padded_workspace_size", C.c_size_t, [C.c_int64, C.c_int32]),
    ("bt_build_padded", C.c_int, [_P, C.c_int64, C.c_int32, C.POINTER(C.c_float), _P, _P,
                                  C.c_size_t, _P]),
    ("bt_permute_padded", C.c_int, [_P, _P, C.c_int64, C.c_int64, C.c_int64, C.c_int, _P, _P]),
    ("ball_attn_padded", C.c_int, [_P, _P, _P, _P, C.c_int64, C.c_int64, C.c_int32, C.c_int32,
                                   C.c_int32, C.c_int, _P, _P]),
]
EXPORTS = [s[0] for s in _SIGS]


def lib():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run __graft_entry__.build() first")
        L = C.CDLL(LIB_PATH)
        for name, res, args in _SIGS:
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int):
    if status != BT_OK:
        L = lib()
        raise BtError(status, f"{L.bt_status_str(status).decode()}: "
                              f"{L.bt_last_error().decode()}")


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(device):
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(t, name, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU (no CPU fallback)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _dtype_code(t):
    if t.dtype == torch.float32:
        return BT_F32
    if t.dtype == torch.bfloat16:
        return BT_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _coords(coords):
    _dev(coords, "coords", torch.float32)
    if coords.dim() != 2 or coords.shape[1] != 3:
        raise ValueError(f"coords must be [N,3], got {tuple(coords.shape)}")
    return coords.shape[0]


def _perm(perm, n, name="perm"):
    """A permutation argument: int32, 1-D, n entries (checked before any
    launch, so a short array never reaches a kernel)."""
    _dev(perm, name, torch.int32)
    if perm.dim() != 1 or perm.numel() != n:
        raise ValueError(f"{name} must be int32 [{n}], got {tuple(perm.shape)}")
    return perm


def _same_shape(t, ref, name):
    if tuple(t.shape) != tuple(ref.shape):
        raise ValueError(f"{name} must have shape {tuple(ref.shape)}, got {tuple(t.shape)}")


def _gates(gate_w, gate_b, d):
    if gate_w is not None:
        _dev(gate_w, "gate_w", torch.float32)
        if tuple(gate_w.shape) != (3, d):
            raise ValueError(f"gate_w must be [3,{d}], got {tuple(gate_w.shape)}")
    if gate_b is not None:
        _dev(gate_b, "gate_b", torch.float32)
        if tuple(gate_b.shape) != (3,):
            raise ValueError(f"gate_b must be [3], got {tuple(gate_b.shape)}")


# --------------------------------------------------------------------- tree --

def bt_build_workspace_size(N: int, leaf: int) -> int:
    return lib().bt_build_workspace_size(N, leaf)


def _workspace(nbytes, device):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def bt_build(coords, leaf: int, perm=None, workspace=None):
    """Tree permutation of ``coords`` [N,3] fp32 -> int32 [N] (device)."""
    N = _coords(coords)
    if perm is None:
        perm = torch.empty(N, dtype=torch.int32, device=coords.device)
    _perm(perm, N)
    need = lib().bt_build_workspace_size(N, leaf)
    if workspace is None:
        workspace = _workspace(need, coords.device)
    _check(lib().bt_build(_ptr(coords), N, leaf, _ptr(perm), _ptr(workspace),
                          workspace.numel(), _stream(coords.device)))
    return perm


def bt_rotate_build(coords, leaf: int, R, perm=None, workspace=None):
    """Tree of the coordinates rotated by the 3x3 matrix R (host values)."""
    N = _coords(coords)
    r = torch.as_tensor(R, dtype=torch.float32).reshape(9).cpu().tolist()
    rarr = (C.c_float * 9)(*r)
    if perm is None:
        perm = torch.empty(N, dtype=torch.int32, device=coords.device)
    _perm(perm, N)
    need = lib().bt_build_workspace_size(N, leaf)
    if workspace is None:
        workspace = _workspace(need, coords.device)
    _check(lib().bt_rotate_build(_ptr(coords), N, leaf, rarr, _ptr(perm), _ptr(workspace),
                                 workspace.numel(), _stream(coords.device)))
    return perm


def bt_padded_size(N: int, leaf: int) -> int:
    """Slots of the padded tree of N points (-1 if invalid)."""
    return lib().bt_padded_size(N, leaf)


def bt_build_padded(coords, leaf: int, R=None, perm=None, workspace=None):
    """Padded tree of an uneven point count: int32 [bt_padded_size(N, leaf)]
    with -1 in unused slots (R: optional host 3x3 rotation)."""
    N = _coords(coords)
    S = lib().bt_padded_size(N, leaf)
    rarr = None
    if R is not None:
        r = torch.as_tensor(R, dtype=torch.float32).reshape(9).cpu().tolist()
        rarr = (C.c_float * 9)(*r)
    if perm is None:
        perm = torch.empty(max(S, 0), dtype=torch.int32, device=coords.device)
    _dev(perm, "perm", torch.int32)
    if perm.dim() != 1 or perm.numel() != S:
        raise ValueError(f"perm must be int32 [{S}] (the slot count)")
    need = lib().bt_build_padded_workspace_size(N, leaf)
    if workspace is None:
        workspace = _workspace(need, coords.device)
    _check(lib().bt_build_padded(_ptr(coords), N, leaf, rarr, _ptr(perm), _ptr(workspace),
                                 workspace.numel(), _stream(coords.device)))
    return perm


# ------------------------------------------------------------------ permute --

def bt_permute(src, perm, mode: int, dst=None):
    """GATHER dst[t] = src[perm[t]]; SCATTER dst[perm[t]] = src[t] (rows)."""
    _dev(src, "src")
    if src.dim() < 1:
        raise ValueError("src must have a row axis")
    N = src.shape[0]
    _perm(perm, N)
    row_bytes = math.prod(src.shape[1:]) * src.element_size()
    if dst is None:
        dst = torch.empty_like(src)
    _dev(dst, "dst", src.dtype)
    _same_shape(dst, src, "dst")
    _check(lib().bt_permute(_ptr(src), _ptr(perm), N, row_bytes, mode, _ptr(dst),
                            _stream(src.device)))
    return dst


def bt_permute_padded(src, perm, n_rows: int, mode: int, dst=None):
    """Padded permutation (perm: one entry per slot, -1 unused).  GATHER:
    [n_rows, ...] -> [slots, ...] with zero rows in unused slots; SCATTER:
    [slots, ...] -> [n_rows, ...] from the used slots."""
    _dev(src, "src")
    _dev(perm, "perm", torch.int32)
    if perm.dim() != 1:
        raise ValueError("perm must be 1-D (one entry per slot)")
    S = perm.numel()
    row_bytes = math.prod(src.shape[1:]) * src.element_size()
    if dst is None:
        rows = S if mode == BT_GATHER else n_rows
        dst = torch.empty((rows,) + tuple(src.shape[1:]), dtype=src.dtype, device=src.device)
    _dev(dst, "dst", src.dtype)
    if src.shape[0] != (n_rows if mode == BT_GATHER else S) or \
            dst.shape[0] != (S if mode == BT_GATHER else n_rows):
        raise ValueError("src/dst rows do not match n_rows and the slot count")
    _check(lib().bt_permute_padded(_ptr(src), _ptr(perm), n_rows, S, row_bytes, mode, _ptr(dst),
                                   _stream(src.device)))
    return dst


def bt_count_nonfinite(x, count=None):
    """Number of NaN or infinite values in the fp32 tensor x (device int32
    [1] holding the count; the debug check of the builders' precondition)."""
    _dev(x, "x", torch.float32)
    if count is None:
        count = torch.empty(1, dtype=torch.int32, device=x.device)
    _dev(count, "count", torch.int32)
    if count.numel() != 1:
        raise ValueError("count must hold one int32")
    _check(lib().bt_count_nonfinite(_ptr(x), x.numel(), _ptr(count), _stream(x.device)))
    return count


def bt_invert_perm(perm, inv=None):
    _dev(perm, "perm", torch.int32)
    if perm.dim() != 1:
        raise ValueError("perm must be 1-D")
    if inv is None:
        inv = torch.empty_like(perm)
    _perm(inv, perm.numel(), "inv")
    _check(lib().bt_invert_perm(_ptr(perm), perm.numel(), _ptr(inv), _stream(perm.device)))
    return inv


# ------------------------------------------------------ coarsen / refine --

def bt_coarsen(x, perm, s: int, out=None):
    """[N,H,d] -> coarse level [N/s,H,d] in tree order (perm None: x is
    already in tree order)."""
    _dev(x, "x")
    if x.dim() != 3:
        raise ValueError("x must be [N,H,d]")
    N, H, d = x.shape
    if perm is not None:
        _perm(perm, N)
    if out is None:
        out = torch.empty((N // s if s > 0 else 0, H, d), dtype=x.dtype, device=x.device)
    _dev(out, "out", x.dtype)
    if s > 0 and tuple(out.shape) != (N // s, H, d):
        raise ValueError(f"out must be [{N // s},{H},{d}]")
    _check(lib().bt_coarsen(_ptr(x), _ptr(perm), N, H, d, s, _dtype_code(x), _ptr(out),
                            _stream(x.device)))
    return out


def bt_refine(xc, perm, s: int, out=None):
    """Coarse level [N/s,H,d] -> [N,H,d]: every child takes its parent's row
    (original order when perm is given)."""
    _dev(xc, "xc")
    if xc.dim() != 3:
        raise ValueError("xc must be [N/s,H,d]")
    Nc, H, d = xc.shape
    if perm is not None:
        _perm(perm, Nc * s)
    if out is None:
        out = torch.empty((Nc * s, H, d), dtype=xc.dtype, device=xc.device)
    _dev(out, "out", xc.dtype)
    if tuple(out.shape) != (Nc * s, H, d):
        raise ValueError(f"out must be [{Nc * s},{H},{d}]")
    _check(lib().bt_refine(_ptr(xc), _ptr(perm), Nc * s, H, d, s, _dtype_code(xc), _ptr(out),
                           _stream(xc.device)))
    return out


# ---------------------------------------------------------------- attention --

def ball_attn(q, k, v, perm, ball: int, out=None):
    """Ball attention over [N,H,d] tensors (perm None = already tree order)."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev(t, name, q.dtype)
        if t.shape != q.shape or t.dim() != 3:
            raise ValueError("q, k, v must share one [N,H,d] shape")
    N, H, d = q.shape
    if perm is not None:
        _perm(perm, N)
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype)
    _same_shape(out, q, "out")
    _check(lib().ball_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(perm), N, ball, H, d,
                           _dtype_code(q), _ptr(out), _stream(q.device)))
    return out


def ball_attn_padded(q, k, v, perm, ball: int, out=None):
    """Ball attention on a padded tree: q, k, v [N,H,d] in original order,
    perm int32 [slots] with -1 in unused slots."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev(t, name, q.dtype)
        if t.shape != q.shape or t.dim() != 3:
            raise ValueError("q, k, v must share one [N,H,d] shape")
    _dev(perm, "perm", torch.int32)
    if perm.dim() != 1:
        raise ValueError("perm must be 1-D (one entry per slot)")
    N, H, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype)
    _same_shape(out, q, "out")
    _check(lib().ball_attn_padded(_ptr(q), _ptr(k), _ptr(v), _ptr(perm), N, perm.numel(), ball,
                                  H, d, _dtype_code(q), _ptr(out), _stream(q.device)))
    return out


def ball_attn_bwd(q, k, v, dout, perm, ball: int, dq=None, dk=None, dv=None):
    """Gradients (dq, dk, dv) of ball attention for the output gradient dout."""
    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _dev(t, name, q.dtype)
        if t.shape != q.shape or t.dim() != 3:
            raise ValueError("q, k, v, dout must share one [N,H,d] shape")
    N, H, d = q.shape
    if perm is not None:
        _perm(perm, N)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _dev(t, name, q.dtype)
        _same_shape(t, q, name)
    _check(lib().ball_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(perm), N, ball, H,
                               d, _dtype_code(q), _ptr(dq), _ptr(dk), _ptr(dv),
                               _stream(q.device)))
    return dq, dk, dv


def bsa_workspace_size(N: int, H: int, d: int, ball: int, block: int, group: int,
                       topk: int, mask_own_ball: bool = True,
                       query_compression: bool = False) -> int:
    p = BsaParams(ball, block, group, topk, int(bool(mask_own_ball)),
                  int(bool(query_compression)))
    return lib().bsa_workspace_size(N, H, d, C.byref(p))


def bsa_attn_bwd_workspace_size(N: int, H: int, d: int, ball: int, block: int, group: int,
                                topk: int, mask_own_ball: bool = True) -> int:
    p = BsaParams(ball, block, group, topk, int(bool(mask_own_ball)), 0)
    return lib().bsa_attn_bwd_workspace_size(N, H, d, C.byref(p))


def bsa_attn(q, k, v, perm, ball: int, block: int, group: int, topk: int,
             mask_own_ball: bool = True, gate_w=None, gate_b=None, gate_const=None,
             return_sel: bool = False, out=None, workspace=None,
             query_compression: bool = False):
    """Ball Sparse Attention; returns out (and sel [H, N/group, topk]).
    ``query_compression`` selects BSA with group compression."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev(t, name, q.dtype)
        if t.shape != q.shape or t.dim() != 3:
            raise ValueError("q, k, v must share one [N,H,d] shape")
    N, H, d = q.shape
    _perm(perm, N)
    p = BsaParams(ball, block, group, topk, int(bool(mask_own_ball)),
                  int(bool(query_compression)))
    _gates(gate_w, gate_b, d)
    gc = None
    if gate_const is not None:
        gc = (C.c_float * 3)(*[float(x) for x in gate_const])
    sel = None
    if return_sel:
        sel = torch.empty((H, N // group, topk), dtype=torch.int32, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype)
    _same_shape(out, q, "out")
    need = lib().bsa_workspace_size(N, H, d, C.byref(p))
    if workspace is None:
        workspace = _workspace(need, q.device)
    _check(lib().bsa_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(perm), N, H, d, _dtype_code(q),
                          C.byref(p), _ptr(gate_w), _ptr(gate_b), gc, _ptr(sel),
                          _ptr(workspace), workspace.numel(), _ptr(out), _stream(q.device)))
    return (out, sel) if return_sel else out


def bsa_attn_noalloc(q, k, v, perm, ball: int, block: int, group: int, topk: int,
                     mask_own_ball: bool = True, gate_w=None, gate_b=None, gate_const=None,
                     return_sel: bool = False, out=None, query_compression: bool = False):
    """bsa_attn with the library's static workspace (no device allocation by
    the library; ``out`` and ``sel`` are allocated here unless given)."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev(t, name, q.dtype)
        if t.shape != q.shape or t.dim() != 3:
            raise ValueError("q, k, v must share one [N,H,d] shape")
    N, H, d = q.shape
    _perm(perm, N)
    p = BsaParams(ball, block, group, topk, int(bool(mask_own_ball)),
                  int(bool(query_compression)))
    _gates(gate_w, gate_b, d)
    gc = None
    if gate_const is not None:
        gc = (C.c_float * 3)(*[float(x) for x in gate_const])
    sel = None
    if return_sel:
        sel = torch.empty((H, N // group, topk), dtype=torch.int32, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype)
    _same_shape(out, q, "out")
    _check(lib().bsa_attn_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(perm), N, H, d,
                                  _dtype_code(q), C.byref(p), _ptr(gate_w), _ptr(gate_b), gc,
                                  _ptr(sel), _ptr(out), _stream(q.device)))
    return (out, sel) if return_sel else out


def bsa_attn_bwd(q, k, v, perm, dout, ball: int, block: int, group: int, topk: int,
                 mask_own_ball: bool = True, gate_w=None, gate_b=None, gate_const=None,
                 grads=None, workspace=None):
    """Backward of BSA (without group compression): returns (dq, dk, dv,
    dgate_w, dgate_b); the gate gradients are None with ``gate_const``.
    ``grads`` optionally gives the (dq, dk, dv) tensors to write."""
    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _dev(t, name, q.dtype)
        if t.shape != q.shape or t.dim() != 3:
            raise ValueError("q, k, v, dout must share one [N,H,d] shape")
    N, H, d = q.shape
    _perm(perm, N)
    p = BsaParams(ball, block, group, topk, int(bool(mask_own_ball)), 0)
    _gates(gate_w, gate_b, d)
    gc = None
    dgw = dgb = None
    if gate_const is not None:
        gc = (C.c_float * 3)(*[float(x) for x in gate_const])
    else:
        dgw = torch.empty((3, d), dtype=torch.float32, device=q.device)
        dgb = torch.empty(3, dtype=torch.float32, device=q.device)
    if grads is None:
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    else:
        dq, dk, dv = grads
        for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            _dev(t, name, q.dtype)
            if t.shape != q.shape:
                raise ValueError(f"{name} must have the shape of q")
    need = lib().bsa_attn_bwd_workspace_size(N, H, d, C.byref(p))
    if workspace is None:
        workspace = _workspace(need, q.device)
    _check(lib().bsa_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(perm), _ptr(dout), N, H, d,
                              _dtype_code(q), C.byref(p), _ptr(gate_w), _ptr(gate_b), gc,
                              _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dgw), _ptr(dgb),
                              _ptr(workspace), workspace.numel(), _stream(q.device)))
    return dq, dk, dv, dgw, dgb
