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
