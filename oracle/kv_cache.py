"""CPU oracle of the KV-cache update -- test infrastructure.

Only the test-suite, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this module; the product never does, and it
imports nothing from the product.

It follows the onnx-tensorrt "TensorRT Custom Operator Schemas" page,
section TRT_KVCacheUpdate (mode "linear", axis -2 of the [B, H, N, D]
cache; update in "padded_bhnd" [B, H, N_u, D] or "packed_nhd" [T, H, D]
form; write_indices [B]; update_lengths cumulative [B+1]).  Readings where
the page is silent:

  * write_indices absent: every sequence writes from position 0;
  * update_lengths absent (padded update only): each sequence writes all
    N_u rows of its update; present: sequence b writes
    L_b = update_lengths[b+1] - update_lengths[b] rows (the first L_b of
    update[b] when padded, rows update_lengths[b] .. +L_b when packed);
  * row t of sequence b lands at position write_indices[b] + t of every
    head; positions outside [0, N) are dropped (nothing is written there);
  * every other element of Y equals past_cache.

The arithmetic is byte copying only, so the arrays are handled as raw
integer views of any element type (fp8, f16, bf16 all copy bit for bit).
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def _raw(x) -> np.ndarray:
    """A host numpy view of the bytes of an array or torch tensor."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            es = x.element_size()
            dt = {1: torch.uint8, 2: torch.int16, 4: torch.int32}[es]
            return x.view(dt).numpy()
    except ImportError:  # pragma: no cover - torch is always present here
        pass
    return np.asarray(x)


def kv_cache_update(past_cache, update, *, write_indices=None, update_lengths=None,
                    update_form: str = "padded_bhnd") -> np.ndarray:
    """Y = past_cache with each sequence's update rows written along the
    sequence axis (TRT_KVCacheUpdate, linear mode).  Returns a new array of
    past_cache's raw integer type and shape."""
    cache = _raw(past_cache)
    upd = _raw(update)
    if cache.ndim != 4:
        raise ValueError("past_cache must be [B, H, N, D]")
    B, H, N, D = cache.shape
    y = cache.copy()
    w = None if write_indices is None else np.asarray(_raw(write_indices), dtype=np.int64)
    ul = None if update_lengths is None else np.asarray(_raw(update_lengths), dtype=np.int64)
    if update_form == "packed_nhd":
        if ul is None:
            raise ValueError("a packed update needs update_lengths")
        if upd.ndim != 3 or upd.shape[1:] != (H, D):
            raise ValueError("packed update must be [T, H, D]")
    elif update_form == "padded_bhnd":
        if upd.ndim != 4 or upd.shape[0] != B or upd.shape[1] != H or upd.shape[3] != D:
            raise ValueError("padded update must be [B, H, N_u, D]")
    else:
        raise ValueError(update_form)
    for b in range(B):
        start = 0 if w is None else int(w[b])
        if update_form == "packed_nhd":
            first, count = int(ul[b]), int(ul[b + 1] - ul[b])
        else:
            first, count = 0, (upd.shape[2] if ul is None else int(ul[b + 1] - ul[b]))
        for t in range(count):
            pos = start + t
            if pos < 0 or pos >= N:
                continue
            for h in range(H):
                if update_form == "packed_nhd":
                    y[b, h, pos, :] = upd[first + t, h, :]
                else:
                    y[b, h, pos, :] = upd[b, h, t, :]
    return y


def written_rows(B: int, N: int, count_per_seq, write_indices: Optional[np.ndarray] = None) -> int:
    """Number of (b, position) rows the update writes (for bandwidth counts)."""
    n = 0
    for b in range(B):
        start = 0 if write_indices is None else int(write_indices[b])
        lo, hi = max(start, 0), min(start + int(count_per_seq[b]), N)
        n += max(0, hi - lo)
    return n
