"""A synthetic MoE layer resident in GPU memory, built through the library.

Raw fp32 tensors come from the seeded generators in ``synth``; they are copied
to the GPU one chunk of experts at a time and quantised there by
moe_quantize_weights, so no host copy of a whole large layer is ever held.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np
import torch

import synth
from . import _lib


@dataclasses.dataclass
class DeviceLayer:
    shape: synth.LayerShape
    gate_w: torch.Tensor                  # [E, d] fp32
    bias: Optional[torch.Tensor]          # [E] fp32 or None
    shared_gate: Optional[torch.Tensor]   # [d] fp32 or None
    routed: List[_lib.QuantExperts]       # one or more copies of the routed stack
    shared: List[Optional[_lib.QuantExperts]]
    params: _lib.RouterParams

    @property
    def copies(self) -> int:
        return len(self.routed)


def _quantize_stack(shape: synth.LayerShape, experts, device, chunk: int, out: _lib.QuantExperts, base: int):
    f = _lib.FORMATS[shape.wformat]
    for lo in range(0, len(experts), chunk):
        ids = experts[lo:lo + chunk]
        for which, q, s in (("gate", out.gate_q, out.gate_s), ("up", out.up_q, out.up_s),
                            ("down", out.down_q, out.down_s)):
            host = synth.expert_weights_stacked(shape, which, ids)
            dev = torch.from_numpy(host).to(device, non_blocking=False)
            _lib.moe_quantize_weights(dev, f, q[base + lo:base + lo + len(ids)], s[base + lo:base + lo + len(ids)])
            del dev
    torch.cuda.synchronize(device)


def build(shape: synth.LayerShape, device="cuda", copies: int = 1, chunk: Optional[int] = None) -> DeviceLayer:
    """Quantise the layer on the GPU. copies > 1 duplicates the routed and
    shared experts (device-to-device), so repeated timing can rotate through
    more bytes than the last-level caches hold."""
    E, d, I = shape.n_experts, shape.d_model, shape.d_ff
    if chunk is None:
        per = 3 * d * I * 4
        chunk = max(1, min(E, (2 << 30) // per))
    routed = _lib.QuantExperts.empty(E, d, I, shape.wformat, device=device)
    _quantize_stack(shape, list(range(E)), device, chunk, routed, 0)
    shared = None
    if shape.shared_expert:
        shared = _lib.QuantExperts.empty(1, d, I, shape.wformat, device=device)
        _quantize_stack(shape, [E], device, 1, shared, 0)
    routed_list = [routed]
    shared_list = [shared]
    for _ in range(1, copies):
        routed_list.append(_lib.QuantExperts(shape.wformat, *(t.clone() for t in (
            routed.gate_q, routed.gate_s, routed.up_q, routed.up_s, routed.down_q, routed.down_s))))
        shared_list.append(None if shared is None else _lib.QuantExperts(shape.wformat, *(t.clone() for t in (
            shared.gate_q, shared.gate_s, shared.up_q, shared.up_s, shared.down_q, shared.down_s))))
    gate_w = torch.from_numpy(synth.gate_weight(shape)).to(device)
    b = synth.score_bias(shape)
    bias = torch.from_numpy(b).to(device) if b is not None else None
    u = synth.shared_gate_weight(shape)
    sg = torch.from_numpy(u).to(device) if u is not None else None
    params = _lib.router_params(E, shape.top_k, shape.router, shape.renormalize, shape.n_group,
                                shape.topk_group, shape.routed_scaling_factor, bias, shape.top_p, sg)
    return DeviceLayer(shape, gate_w, bias, sg, routed_list, shared_list, params)


def add_copies(layer: DeviceLayer, total: int) -> None:
    """Grow the layer to `total` device copies of its experts (device-to-device
    clones of the first copy)."""
    r0, s0 = layer.routed[0], layer.shared[0]
    while len(layer.routed) < total:
        layer.routed.append(_lib.QuantExperts(r0.fmt, *(t.clone() for t in (
            r0.gate_q, r0.gate_s, r0.up_q, r0.up_s, r0.down_q, r0.down_s))))
        layer.shared.append(None if s0 is None else _lib.QuantExperts(s0.fmt, *(t.clone() for t in (
            s0.gate_q, s0.gate_s, s0.up_q, s0.up_s, s0.down_q, s0.down_s))))


def activations(shape: synth.LayerShape, tokens: int, device="cuda") -> torch.Tensor:
    return torch.from_numpy(synth.activations(shape, tokens)).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()
