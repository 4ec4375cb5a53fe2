"""Oracle: the whole routed MoE FFN layer.

TEST INFRASTRUCTURE ONLY (see the package docstring).

route -> dispatch -> each distinct expert applied once to all of its rows
(batch-union; "Show HN: Getting GLM-5.2 running on my slow computer", section "What's implemented") -> combine:

    out[t] = sum_j w[t, j] * Y[inv_perm[t*k + j]]  +  S[t]

where Y holds the un-weighted expert outputs in permuted order and S is the
shared expert ("Show HN: Getting GLM-5.2 running on my slow computer": shared expert), an FFN of the same format
applied to every token with weight 1: the pages name no gate on it.

Gated shared expert (an option, off by default): some model families scale
the shared expert's output per token by a learned scalar gate, the sigmoid of
one more linear projection of the hidden state. With that vector u [d]:

    S[t] = sigmoid(x[t] . u) * FFN_shared(x[t])

The pages do not describe it; this is the plain form of the option, taken in
fp64 on the layer's input rows (the same rows the router sees).
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Optional

import numpy as np

from . import dispatch as dispatch_mod
from . import ffn, router


@dataclasses.dataclass
class RouterSpec:
    mode: str                    # "softmax" | "noaux_tc"
    top_k: int
    renormalize: bool = False
    n_group: int = 1
    topk_group: int = 1
    routed_scaling_factor: float = 1.0
    bias: Optional[np.ndarray] = None
    top_p: float = 0.0           # adaptive expert top-p; 0 (or >= 1) keeps all k
    shared_gate: Optional[np.ndarray] = None   # [d]: gate the shared expert by sigmoid(x . u)


def rmsnorm(x, gamma, eps: float):
    """RMSNorm of each row, in fp64: x / sqrt(mean(x^2) + eps) * gamma.

    The hidden states the layer takes are "after RMSNorm"; the normalisation
    itself is the transformer block's (the mtlm-7m-base page lists RMSNorm
    among the model's layers, section "What is and is not machin").
    """
    x = np.asarray(x, np.float64)
    inv = 1.0 / np.sqrt((x * x).mean(axis=1, keepdims=True) + eps)
    return x * inv * np.asarray(gamma, np.float64)[None, :]


def route(x, wg, spec: RouterSpec):
    if spec.mode == "softmax":
        idx, w, l = router.route_softmax(x, wg, spec.top_k, spec.renormalize)
    elif spec.mode == "noaux_tc":
        idx, w, l = router.route_noaux_tc(x, wg, spec.bias, spec.top_k, spec.n_group,
                                          spec.topk_group, spec.routed_scaling_factor)
    else:
        raise ValueError(f"unknown router mode {spec.mode}")
    idx, w = router.apply_top_p(idx, w, spec.top_p)
    return idx, w, l


def expert_rows(x, ex: ffn.QuantExpert, act_mode: str):
    if act_mode == "f32":
        return ffn.ffn_f32(x, ex)
    if act_mode == "q8_0":
        return ffn.ffn_q8(x, ex)[0]
    raise ValueError(f"unknown act_mode {act_mode}")


def shared_gate_values(x, u) -> np.ndarray:
    """sigmoid(x[t] . u) per row, fp64 [T]."""
    z = np.asarray(x, np.float64) @ np.asarray(u, np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def combine(y_perm, w, inv_perm, shared_y=None):
    t, k = w.shape
    inv = np.asarray(inv_perm).reshape(t, k)
    gathered = y_perm[np.maximum(inv, 0)]                         # [T, k, d]
    wk = np.where(inv >= 0, np.asarray(w, np.float64), 0.0)       # dropped slots add nothing
    out = np.einsum("tk,tkd->td", wk, gathered)
    if shared_y is not None:
        out = out + shared_y
    return out


def layer_forward(x, wg, spec: RouterSpec, get_expert: Callable[[int], ffn.QuantExpert],
                  shared: Optional[ffn.QuantExpert], act_mode: str):
    """Returns a dict with idx, w, counts, offsets, perm, inv_perm, y_perm,
    shared_y and out (fp64 [T, d])."""
    x = np.asarray(x, np.float32)
    n_experts = wg.shape[0]
    idx, w, l = route(x, wg, spec)
    counts, offsets, perm, inv = dispatch_mod.dispatch(idx, n_experts)
    k = spec.top_k
    t, d = x.shape
    y_perm = np.zeros((t * k, d), dtype=np.float64)
    for e in np.nonzero(counts)[0]:
        lo, hi = offsets[e], offsets[e + 1]
        tokens = perm[lo:hi] // k
        y_perm[lo:hi] = expert_rows(x[tokens], get_expert(int(e)), act_mode)
    shared_y = expert_rows(x, shared, act_mode) if shared is not None else None
    gate = None
    if shared_y is not None and spec.shared_gate is not None:
        gate = shared_gate_values(x, spec.shared_gate)
        shared_y = gate[:, None] * shared_y
    out = combine(y_perm, w, inv, shared_y)
    return dict(idx=idx, w=w, logits=l, counts=counts, offsets=offsets, perm=perm,
                inv_perm=inv, y_perm=y_perm, shared_y=shared_y, shared_gate=gate, out=out)


def block_forward(x, gamma, eps: float, wg, spec: RouterSpec, get_expert: Callable[[int], ffn.QuantExpert],
                  shared: Optional[ffn.QuantExpert], act_mode: str):
    """The layer between its neighbours: out = x + layer(RMSNorm(x)).

    The normalised states enter the layer in fp32 (the layer's input type);
    gamma = None skips the normalisation. Returns layer_forward's dict with
    out replaced by the residual sum and x_norm added.
    """
    x = np.asarray(x, np.float32)
    xn = x if gamma is None else rmsnorm(x, gamma, eps).astype(np.float32)
    res = layer_forward(xn, wg, spec, get_expert, shared, act_mode)
    res["x_norm"] = xn
    res["out"] = np.asarray(x, np.float64) + res["out"]
    return res
