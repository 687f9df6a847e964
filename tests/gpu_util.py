"""Helpers for GPU parity tests: device transfer of BF16 bit arrays, progress lines."""

import sys

import numpy as np


def say(*a):
    """Name the case before each GPU step (flushed, so a crash still shows it)."""
    print("[case]", *a, file=sys.stderr, flush=True)


def dev_bf16(bits, device="cuda:0"):
    """BF16 device tensor [R, C]; the row stride is padded to a multiple of 8 elements (16 bytes)."""
    import torch
    R, C = bits.shape
    ld = -(-max(C, 1) // 8) * 8
    buf = np.zeros((R, ld), dtype=np.uint16)
    buf[:, :C] = bits
    t = torch.from_numpy(buf.view(np.int16)).to(device).view(torch.bfloat16)
    return t[:, :C]


def host(t):
    """Device tensor -> numpy (BF16 comes back as uint16 bit patterns)."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def sample_index(n, k, rng, must=()):
    """k sorted distinct indices in [0, n), always including `must` (edges, tails)."""
    base = set(int(m) % n for m in must if n > 0)
    rest = [i for i in rng.choice(n, size=min(n, k), replace=False) if i not in base]
    idx = sorted(base | set(int(i) for i in rest[: max(0, k - len(base))]))
    return np.array(idx, dtype=np.int64)
