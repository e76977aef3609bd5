"""Reference order of the segment scheduler's (user, q-tile) worklist.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages launch a dense grid (cdiv(max_seqlen, 64), num_users, n_heads) in
which programs past a user's end exit at once (cti2026 README,
FlashAttention_Varlen section, "operator design", and the CUDA Graph section,
"fixed attention grid": an oversized grid leaves results unchanged; zero-length
padding users are skipped).  The scheduler here replaces the empty programs by
a compact list that holds exactly the (user, q-tile) pairs that have rows:

* user ``u`` with length ``L`` owns ``ceil(L / tile_rows)`` q-tiles; zero-length
  users own none;
* q-tile ``k`` of a user needs ``k + 1`` key tiles (it stops at the diagonal), so
  items are emitted longest first: for ``k`` from the largest tile index down to
  0, every user that has a tile ``k``, in ascending user order.

The order is a design choice of this library (longest-processing-time first
for the persistent kernel); the list is unique under it, so the GPU-built list
must match this one element for element.
"""
from __future__ import annotations

import numpy as np


def tiles_per_user(cu_seqlens, tile_rows: int, max_tiles: int | None = None) -> np.ndarray:
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    lengths = np.diff(cu)
    if np.any(lengths < 0):
        raise ValueError("cu_seqlens must be non-decreasing")
    nt = (lengths + tile_rows - 1) // tile_rows
    if max_tiles is not None:
        nt = np.minimum(nt, max_tiles)
    return nt


def reference_worklist(cu_seqlens, tile_rows: int, max_tiles: int | None = None) -> np.ndarray:
    """int32 ``[N, 2]`` array of (user, q_tile) in the scheduler's order, by plain loops."""
    nt = tiles_per_user(cu_seqlens, tile_rows, max_tiles)
    items = []
    top = int(nt.max()) if nt.size else 0
    for k in range(top - 1, -1, -1):
        for u in range(nt.shape[0]):
            if nt[u] > k:
                items.append((u, k))
    return np.asarray(items, dtype=np.int32).reshape(-1, 2)
