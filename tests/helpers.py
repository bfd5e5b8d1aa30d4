"""Shared helpers for the GPU parity tests."""
import sys

import numpy as np
import pytest
import torch


def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")


def say(*a):
    """Name the case before a GPU step (flushed, so a fault still shows it)."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def max_abs(a, b):
    a = a.detach().float().cpu().double().numpy() if hasattr(a, "detach") else np.asarray(a)
    b = b.detach().float().cpu().double().numpy() if hasattr(b, "detach") else np.asarray(b)
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def ramp_scores(q, k, perm, ball, seed, big_key=False):
    """q and k altered so that scores move in steps along each ball.

    Coordinate 0 of every key gets -8 * ((ball - 1 - t) // 64) added, t its
    slot in the ball (perm[slot] is its row), and coordinate 0 of every query
    gets +4 or -4 (random): against a head dimension of 32 or 64, a query of
    the first kind sees its largest scores climb by 2^8 or more (in base-2
    units) from one 64-key stretch to the next, one of the second kind sees
    them fall.  A kernel that keeps a running maximum must raise it within a
    ball for some queries while others in the same wave stay put.

    big_key: coordinate 1 of every query is set to 0 and the key in slot 5
    of every ball gets 256 there.  The scores do not change, but the product
    of the norms |q| |k| (a bound on every score) becomes large.
    """
    dt = q.dtype
    q, k = q.float().clone(), k.float().clone()
    n, H, _ = q.shape
    rng = np.random.default_rng(seed)
    q[:, :, 0] += torch.from_numpy(rng.choice([-4.0, 4.0], size=(n, H)).astype(np.float32))
    t = np.arange(len(perm)) % ball
    off = np.zeros(n, np.float32)
    off[np.asarray(perm)] = -8.0 * ((ball - 1 - t) // 64)
    k[:, :, 0] += torch.from_numpy(off)[:, None]
    if big_key:
        q[:, :, 1] = 0.0
        rows = np.asarray(perm)[t == 5]
        k[torch.from_numpy(rows.astype(np.int64)), :, 1] = 256.0
    return q.to(dt), k.to(dt)


def step_ball_halves(q, k, perm, ball, big_key=False):
    """q and k altered so that, within every ball, the keys of its second
    64-key stretch score about 2^12 higher (base-2 units, head dimension 32)
    than those of its first: coordinate 0 of every query is set to 4 plus its
    draw, and coordinate 0 of the key in slot t gets +6 or -6 as t % ball is
    past 64 or not.  A kernel with a running maximum must raise it part way
    through each ball.

    big_key: coordinate 1 of every query is set to 0 and the key in slot 3 of
    every 64-slot block gets 256 there: no score changes, but |q| max|k| (a
    bound on every score) becomes large.
    """
    dt = q.dtype
    q, k = q.float().clone(), k.float().clone()
    n = q.shape[0]
    p = np.asarray(perm)
    t = np.arange(len(p))
    q[:, :, 0] += 4.0
    off = np.zeros(n, np.float32)
    off[p] = np.where(t % ball >= 64, 6.0, -6.0)
    k[:, :, 0] += torch.from_numpy(off)[:, None]
    if big_key:
        q[:, :, 1] = 0.0
        rows = p[t % 64 == 3]
        k[torch.from_numpy(rows.astype(np.int64)), :, 1] = 256.0
    return q.to(dt), k.to(dt)
