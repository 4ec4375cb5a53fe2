"""Oracle: the two routers, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Softmax top-k ("I ran a 7B Mixture-of-Experts LLM...", section
"Mixture-of-Experts": OLMoE picks the top 8 of 64 experts per token).
Logits L = X Wg^T. The experts with the k largest logits are selected (the
softmax is monotone, so ranking logits ranks probabilities). A selected
expert's weight is its softmax probability p = exp(L - max) / sum exp(L - max),
divided by the sum of the selected probabilities when renormalising.

Sigmoid noaux_tc ("Show HN: Getting GLM-5.2 running on my slow computer", section "What's implemented": a
DeepSeek-V3-style sigmoid router with noaux_tc and routed_scaling_factor). The
page names the router only; its steps are the DeepSeek-V3 ones:
    s = sigmoid(L);  c = s + b          (b: score-correction bias, selection only)
    experts fall into n_group contiguous groups of E / n_group;
    group score = sum of the two largest c in the group;
    the topk_group best groups stay eligible, the others are excluded;
    the k largest c among eligible experts are selected;
    w_j = s_j / sum_j s_j * routed_scaling_factor.

Ordering and ties, everywhere: larger key first; equal keys go to the lower
expert (or group) id. Output slot j holds the j-th selected expert.

Adaptive expert top-p ("Show HN: Getting GLM-5.2 running on my slow
computer", section "Useful knobs": an adaptive expert top-p of 0.7 reads
30-40% fewer expert bytes). The page gives the knob and its effect only; the
plain reading taken here: with S the sum of a token's k selected weights, slot
j is kept when it is the first slot or the weights of the slots before it sum
to less than top_p * S (the shortest prefix, in selection order, reaching the
mass top_p); the kept weights are rescaled to sum to S again, and a dropped
slot is marked by expert -1 and weight 0. top_p = 0 or top_p >= 1 keeps every
slot.
"""
from __future__ import annotations

import numpy as np


def logits(x: np.ndarray, wg: np.ndarray) -> np.ndarray:
    """L = X Wg^T in fp64. X [T, d], Wg [E, d] -> [T, E]."""
    return np.asarray(x, np.float64) @ np.asarray(wg, np.float64).T


def top_k_desc(keys: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest keys per row, larger first, ties to lower id.

    A stable sort of the negated keys keeps equal keys in ascending id order.
    """
    return np.argsort(-keys, axis=1, kind="stable")[:, :k]


def softmax(l: np.ndarray) -> np.ndarray:
    m = l.max(axis=1, keepdims=True)
    e = np.exp(l - m)
    return e / e.sum(axis=1, keepdims=True)


def route_softmax(x, wg, k: int, renormalize: bool):
    """Returns (idx int32 [T, k], w fp64 [T, k], logits fp64 [T, E])."""
    l = logits(x, wg)
    if not 1 <= k <= l.shape[1]:
        raise ValueError("top_k out of range")
    idx = top_k_desc(l, k)
    p = softmax(l)
    w = np.take_along_axis(p, idx, axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return idx.astype(np.int32), w, l


def apply_top_p(idx: np.ndarray, w: np.ndarray, top_p: float):
    """Adaptive expert top-p over the selected slots (see the module text).

    idx [T, k], w [T, k] in selection order -> (idx, w) with the dropped
    trailing slots set to -1 / 0 and the kept weights rescaled to the same sum.
    """
    idx = np.array(idx, dtype=np.int32, copy=True)
    w = np.array(w, dtype=np.float64, copy=True)
    if top_p <= 0.0 or top_p >= 1.0:
        return idx, w
    total = w.sum(axis=1, keepdims=True)
    before = np.cumsum(w, axis=1) - w                 # mass of the slots before j
    keep = before < top_p * total
    keep[:, 0] = True
    kept_sum = np.where(keep, w, 0.0).sum(axis=1, keepdims=True)
    w = np.where(keep, w * (total / kept_sum), 0.0)
    idx[~keep] = -1
    return idx, w


def top_p_margin(w: np.ndarray, top_p: float) -> np.ndarray:
    """Per token: the smallest |mass before slot j - top_p * S| over slots j >= 1,
    relative to S (inf when top-p is off); a small value means the fp32 and the
    fp64 keep decisions may differ."""
    w = np.asarray(w, np.float64)
    if top_p <= 0.0 or top_p >= 1.0 or w.shape[1] < 2:
        return np.full(w.shape[0], np.inf)
    total = w.sum(axis=1, keepdims=True)
    before = (np.cumsum(w, axis=1) - w)[:, 1:]
    return (np.abs(before - top_p * total) / total).min(axis=1)


def sigmoid(l: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-l))


def group_scores(c: np.ndarray, n_group: int) -> np.ndarray:
    """Sum of the two largest selection keys in each contiguous expert group."""
    t, e = c.shape
    gs = e // n_group
    cg = np.sort(c.reshape(t, n_group, gs), axis=2)[:, :, ::-1]
    return cg[:, :, :min(2, gs)].sum(axis=2)


def route_noaux_tc(x, wg, bias, k: int, n_group: int, topk_group: int,
                   routed_scaling_factor: float):
    """Returns (idx int32 [T, k], w fp64 [T, k], logits fp64 [T, E])."""
    l = logits(x, wg)
    t, e = l.shape
    if e % n_group or not 1 <= topk_group <= n_group:
        raise ValueError("bad group configuration")
    gs = e // n_group
    if not 1 <= k <= topk_group * gs:
        raise ValueError("top_k exceeds the eligible experts")
    s = sigmoid(l)
    c = s + (0.0 if bias is None else np.asarray(bias, np.float64)[None, :])
    gsc = group_scores(c, n_group)
    keep = top_k_desc(gsc, topk_group)
    eligible_group = np.zeros((t, n_group), dtype=bool)
    np.put_along_axis(eligible_group, keep, True, axis=1)
    eligible = np.repeat(eligible_group, gs, axis=1)
    masked = np.where(eligible, c, -np.inf)
    idx = top_k_desc(masked, k)
    ssel = np.take_along_axis(s, idx, axis=1)
    w = ssel / ssel.sum(axis=1, keepdims=True) * routed_scaling_factor
    return idx.astype(np.int32), w, l


def selection_keys(l: np.ndarray, mode: str, bias=None, n_group=1, topk_group=1):
    """Per-expert selection keys (for margins): L (softmax) or masked s + b."""
    if mode == "softmax":
        return l
    s = sigmoid(l)
    c = s + (0.0 if bias is None else np.asarray(bias, np.float64)[None, :])
    gs = l.shape[1] // n_group
    keep = top_k_desc(group_scores(c, n_group), topk_group)
    eligible_group = np.zeros((l.shape[0], n_group), dtype=bool)
    np.put_along_axis(eligible_group, keep, True, axis=1)
    return np.where(np.repeat(eligible_group, gs, axis=1), c, -np.inf)


def boundary_margin(keys: np.ndarray, k: int) -> np.ndarray:
    """Per token: k-th largest key minus the (k+1)-th (inf if none follows)."""
    srt = -np.sort(-keys, axis=1)
    if k >= keys.shape[1]:
        return np.full(keys.shape[0], np.inf)
    a, b = srt[:, k - 1], srt[:, k]
    with np.errstate(invalid="ignore"):
        m = a - b
    return np.where(np.isfinite(b), m, np.inf)


def group_margin(l: np.ndarray, bias, n_group: int, topk_group: int) -> np.ndarray:
    """Per token: gap between the last kept group score and the next one."""
    if topk_group >= n_group:
        return np.full(l.shape[0], np.inf)
    c = sigmoid(l) + (0.0 if bias is None else np.asarray(bias, np.float64)[None, :])
    g = -np.sort(-group_scores(c, n_group), axis=1)
    return g[:, topk_group - 1] - g[:, topk_group]
