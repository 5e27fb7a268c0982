"""Host <-> device plumbing for the GPU tests (torch provides memory only)."""

from __future__ import annotations

import sys

import numpy as np
import pytest


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch


def say(*a):
    """Name the case before a GPU step, flushed, so a failed run names it."""
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, pad_before: int = 0, pad_after: int = 0, fill: int = 0):
    """Upload a uint16 (bf16 bits) or float32 array; optional guard elements
    around it hold ``fill`` (bit pattern). Returns (full, view)."""
    import torch
    a = np.ascontiguousarray(a).reshape(-1)
    if a.dtype == np.uint16:
        dt = torch.bfloat16
        host = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    elif a.dtype == np.float32:
        dt = torch.float32
        host = torch.from_numpy(a)
    else:
        raise TypeError(a.dtype)
    if pad_before == 0 and pad_after == 0:
        t = host.to("cuda")
        return t, t
    full = empty_dev(a.size + pad_before + pad_after, dt, fill)
    view = full[pad_before:pad_before + a.size]
    view.copy_(host.to("cuda"))
    return full, view


def empty_dev(n: int, dtype, fill: int = 0):
    """n elements of dtype on the device, every element = bit pattern fill."""
    import torch
    if dtype == torch.bfloat16:
        t = torch.full((n,), int(np.int16(np.uint16(fill))), dtype=torch.int16, device="cuda")
        return t.view(torch.bfloat16)
    t = torch.full((n,), int(np.int32(np.uint32(fill))), dtype=torch.int32, device="cuda")
    return t.view(torch.float32)


def from_dev(t) -> np.ndarray:
    import torch
    c = t.detach().contiguous().cpu()
    if c.dtype == torch.bfloat16:
        return c.view(torch.int16).numpy().view(np.uint16)
    return c.numpy()


def out_buffers(sizes, dtype, guard: int = 0, fill: int = 0xDEAD & 0xFFFF):
    """Output buffers with `guard` canary elements on each side.
    Returns (fulls, views)."""
    fulls, views = [], []
    for n in sizes:
        f = empty_dev(n + 2 * guard, dtype, fill)
        fulls.append(f)
        views.append(f[guard:guard + n])
    return fulls, views


def check_guards(fulls, sizes, guard: int, fill: int = 0xDEAD & 0xFFFF):
    for f, n in zip(fulls, sizes):
        h = from_dev(f)
        bits = h.view(np.uint16) if h.dtype == np.uint16 else h.view(np.uint32)
        want = np.uint16(fill) if h.dtype == np.uint16 else np.uint32(fill)
        assert (bits[:guard] == want).all(), "canary before an output was overwritten"
        assert (bits[guard + n:] == want).all(), "canary after an output was overwritten"
