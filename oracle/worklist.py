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
* q-tile ``k`` of a user needs ``k + 1`` key tiles (it stops at the diagonal).

Order (a design choice of this library, not of the pages).  Users are grouped
by length class ``floor(log2(tiles))``, longest class first, so the longest
users' work starts first; inside a class users ascend; each user's q-tiles are
listed together, from the last one (the most key tiles) down to q-tile 0.
Keeping a user's q-tiles adjacent makes the work items that run at the same
time share that user's key/value rows.  The list is unique under this rule,
so the GPU-built list must match this one element for element.
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


def length_class(tiles: int) -> int:
    """floor(log2(tiles)) for tiles >= 1."""
    c = 0
    while (2 << c) <= tiles:
        c += 1
    return c


def reference_worklist(cu_seqlens, tile_rows: int, max_tiles: int | None = None) -> np.ndarray:
    """int32 ``[N, 2]`` array of (user, q_tile) in the scheduler's order, by plain loops."""
    nt = tiles_per_user(cu_seqlens, tile_rows, max_tiles)
    items = []
    users = [u for u in range(nt.shape[0]) if nt[u] > 0]
    top = max((length_class(int(nt[u])) for u in users), default=-1)
    for c in range(top, -1, -1):
        for u in users:
            if length_class(int(nt[u])) == c:
                for k in range(int(nt[u]) - 1, -1, -1):
                    items.append((u, k))
    return np.asarray(items, dtype=np.int32).reshape(-1, 2)
