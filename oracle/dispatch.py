"""Oracle: token-to-expert dispatch.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Batch-union ("Show HN: Getting GLM-5.2 running on my slow computer", section "What's implemented"): in prefill and
verification each distinct expert of the batch is read once and applied to
every position routed to it. That needs the positions grouped by expert.

The routing gives idx [T, k]; assignment f = t*k + j sends token t to expert
idx[t, j]. The dispatch is:
    counts[e]  = number of assignments to e
    offsets    = [0, cumulative counts]                  (E + 1 entries)
    perm       = assignments sorted by (expert, f)      (a stable sort)
    inv_perm   = the inverse permutation: inv_perm[perm[p]] = p
Rows offsets[e] .. offsets[e+1]-1 of the permuted order belong to expert e,
in increasing f (so in increasing token) order.
"""
from __future__ import annotations

import numpy as np


def dispatch(idx: np.ndarray, n_experts: int):
    """Returns (counts, offsets, perm, inv_perm), all int32."""
    flat = np.asarray(idx).reshape(-1).astype(np.int64)
    if flat.size and (flat.min() < 0 or flat.max() >= n_experts):
        raise ValueError("expert index out of range")
    counts = np.bincount(flat, minlength=n_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    perm = np.argsort(flat, kind="stable")
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    return (counts.astype(np.int32), offsets.astype(np.int32),
            perm.astype(np.int32), inv.astype(np.int32))
