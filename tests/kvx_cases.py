"""Shared helpers of the GPU parity tests: tolerances, row sampling and the
bf16 rounding floor.  No translation arithmetic lives here."""
from __future__ import annotations

import numpy as np
import torch

from oracle import kvx_oracle as O

# max|err| / RMS bounds of the parity bar: fp32 caches, bf16 caches.
TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def sample_rows(token_map, n: int, seed: int) -> np.ndarray:
    """Receiver rows to compare at full size: the first and last 8, every
    row before the first shared boundary (map 0 at the start), at least 32
    rows at run boundaries, the rest uniform."""
    m = np.asarray(token_map)
    N = m.size
    rng = np.random.default_rng(seed)
    pick = set(range(min(8, N))) | set(range(max(0, N - 8), N))
    lead = np.flatnonzero(m == m[0])
    pick |= set(lead[:64].tolist())
    starts = np.flatnonzero(np.diff(m) != 0) + 1
    if starts.size:
        for s in rng.choice(starts, size=min(32, starts.size), replace=False):
            pick |= {int(s) - 1, int(s)}
    while len(pick) < min(n, N):
        pick.add(int(rng.integers(0, N)))
    return np.array(sorted(pick), dtype=np.int64)


def bf16_floor(ref) -> float:
    """max over elements of half a bf16 ulp of the exact value, / RMS: the
    error that rounding the exact result to bf16 alone can cause."""
    ref = np.asarray(ref, dtype=np.float64)
    a = np.abs(ref[ref != 0])
    if a.size == 0:
        return 0.0
    half_ulp = 2.0 ** (np.floor(np.log2(a)) - 8)
    return float(half_ulp.max() / np.sqrt(np.mean(ref * ref)))


def host(t: torch.Tensor) -> torch.Tensor:
    return t.detach().cpu()


def rows_of(cache: torch.Tensor, rows) -> np.ndarray:
    """[L][len(rows)][H*d] float64 of a device cache at the given rows."""
    idx = torch.as_tensor(np.asarray(rows), device=cache.device, dtype=torch.long)
    sub = cache.index_select(1, idx)
    return O.as_f64(sub).reshape(sub.shape[0], sub.shape[1], -1)
