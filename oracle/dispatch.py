"""Oracle: token-to-expert dispatch.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Batch-union ("Show HN: Getting GLM-5.2 running on my slow computer", section "What's implemented"): a prefill
or verification batch loads every expert it selects one time, for all of the
positions that chose it. That needs the positions grouped by expert.

The routing gives idx [T, k]; assignment f = t*k + j sends token t to expert
idx[t, j]. The dispatch is:
    counts[e]  = number of assignments to e
    offsets    = [0, cumulative counts]                  (E + 1 entries)
    perm       = assignments sorted by (expert, f)      (a stable sort)
    inv_perm   = the inverse permutation: inv_perm[perm[p]] = p
Rows offsets[e] .. offsets[e+1]-1 of the permuted order belong to expert e,
in increasing f (so in increasing token) order.

An assignment to expert -1 is a slot dropped by the adaptive expert top-p: it
is not counted, its inv_perm entry is -1, and perm lists the kept assignments
only, followed by -1 up to T*k entries.
"""
from __future__ import annotations

import numpy as np


def dispatch(idx: np.ndarray, n_experts: int):
    """Returns (counts, offsets, perm, inv_perm), all int32."""
    flat = np.asarray(idx).reshape(-1).astype(np.int64)
    if flat.size and (flat.min() < -1 or flat.max() >= n_experts):
        raise ValueError("expert index out of range")
    kept = np.nonzero(flat >= 0)[0]
    counts = np.bincount(flat[kept], minlength=n_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    order = kept[np.argsort(flat[kept], kind="stable")]
    perm = np.full(flat.size, -1, dtype=np.int64)
    perm[:order.size] = order
    inv = np.full(flat.size, -1, dtype=np.int64)
    inv[order] = np.arange(order.size)
    return (counts.astype(np.int32), offsets.astype(np.int32),
            perm.astype(np.int32), inv.astype(np.int32))
