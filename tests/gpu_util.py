"""Helpers shared by the GPU parity tests (host <-> device marshalling, logging)."""
import sys

import numpy as np


def note(msg: str) -> None:
    """Name the case on stdout before a GPU step (flushed, so it survives a crash)."""
    sys.stdout.write(f"[gpu-case] {msg}\n")
    sys.stdout.flush()


def dev(a, dtype=None):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    t = torch.from_numpy(a)
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t):
    import torch
    if t.dtype == torch.int16:
        return t.cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def sample_rows(L: int, topk: int, n: int, seed: int = 0):
    """Seeded row sample that always contains the edge rows."""
    rng = np.random.default_rng(seed)
    edges = [0, 1, topk - 2, topk - 1, topk, topk + 1, L - 2, L - 1]
    rows = set(r for r in edges if 0 <= r < L)
    rows |= set(rng.choice(L, size=min(n, L), replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def check_structure_all(idx_t, topk: int, row0: int = 0):
    """Invariants on every row of a device index tensor: count, causality,
    order.  Row r holds query position row0 + r."""
    import torch
    L = idx_t.shape[0]
    t = torch.arange(row0, row0 + L, device=idx_t.device).unsqueeze(1)
    n = torch.clamp(t + 1, max=topk)
    pos = torch.arange(topk, device=idx_t.device).unsqueeze(0)
    valid = pos < n
    assert bool(torch.all((idx_t >= 0) == valid)), "padding / count wrong"
    assert bool(torch.all(torch.where(valid, idx_t <= t, True))), "non-causal index"
    d = idx_t[:, 1:] - idx_t[:, :-1]
    both = valid[:, 1:]
    assert bool(torch.all(torch.where(both, d > 0, True))), "not strictly ascending"
