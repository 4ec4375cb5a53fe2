"""Seeded synthetic inputs for the routed MoE FFN layer.

This module only draws numbers and states workload shapes. It holds none of the
layer's arithmetic (no quantisation, routing, dispatch or matmul): the oracle
under ``oracle/`` and the HIP library each turn these raw fp32 tensors into
their own results.

Every tensor comes from its own numpy PCG64 stream keyed by
``(seed, tag, index)``, so a tensor never depends on which other tensors were
drawn before it, and a single expert can be regenerated without the rest.

Shapes follow the layers the pages run:
  * OLMoE-1B-7B, top-8 of 64 experts per layer (dev.to, "I ran a 7B
    Mixture-of-Experts LLM...", section "Mixture-of-Experts");
  * GLM-5.2 with a DeepSeek-V3-style sigmoid router and a shared expert
    (note.crab.center, "Show HN: Getting GLM-5.2 running on my slow computer", section "What's implemented");
  * a 512-expert Qwen-Next-class model (scholarbro.com, "FLE: Fast Local
    Experts", abstract).
The pages run trained checkpoints on real prompts; none is available here, so
weights are N(0, 0.02) before quantisation and activations N(0, 1).
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

# stream tags
TAG_X = 1
TAG_GATE_W = 2
TAG_BIAS = 3
TAG_ZIPF_RANK = 4
TAG_NORM_W = 5
TAG_RESID = 6
TAG_SHARED_GATE = 7
TAG_W_GATE = 10
TAG_W_UP = 11
TAG_W_DOWN = 12

WEIGHT_STD = 0.02
BIAS_STD = 0.01


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """One MoE layer: sizes, router mode and expert weight format."""
    name: str
    seed: int
    d_model: int
    n_experts: int
    d_ff: int
    top_k: int
    router: str                 # "softmax" | "noaux_tc"
    renormalize: bool = False
    n_group: int = 1
    topk_group: int = 1
    routed_scaling_factor: float = 1.0
    has_bias: bool = False
    shared_expert: bool = False
    shared_gate: bool = False   # shared expert scaled by sigmoid(x . u) per token
    wformat: str = "int8"       # "int8" | "int4" | "int2" (group 32, fp32 scales); "..._row": a scale per row
    zipf_s: float = 0.0         # > 0: Zipf(s) log-prior on the router logits
    top_p: float = 0.0          # adaptive expert top-p (0: keep all k)


@dataclasses.dataclass(frozen=True)
class Workload:
    """A layer shape plus a token count and an activation mode."""
    name: str
    layer: LayerShape
    tokens: int
    act_mode: str               # "f32" (decode GEMV) | "q8_0" (integer-dot path)
    top_p: float = 0.0          # > 0: adaptive expert top-p for this workload
    block: bool = False         # run as a block: out = x + layer(RMSNorm(x))


LAYERS = {
    "tiny": LayerShape("tiny", 1001, d_model=64, n_experts=8, d_ff=128, top_k=2,
                       router="softmax", renormalize=True, wformat="int8"),
    "olmoe": LayerShape("olmoe", 1002, d_model=2048, n_experts=64, d_ff=1024, top_k=8,
                        router="softmax", renormalize=False, wformat="int8"),
    "olmoe_int4": LayerShape("olmoe_int4", 1003, d_model=2048, n_experts=64, d_ff=1024,
                             top_k=8, router="softmax", renormalize=False, wformat="int4"),
    "glm": LayerShape("glm", 1004, d_model=6144, n_experts=256, d_ff=2048, top_k=8,
                      router="noaux_tc", n_group=8, topk_group=4,
                      routed_scaling_factor=2.5, has_bias=True, shared_expert=True,
                      wformat="int4"),
    # per-row scales: the OLMoE shape with one fp32 scale per matrix row
    "olmoe_int4_row": LayerShape("olmoe_int4_row", 1006, d_model=2048, n_experts=64, d_ff=1024,
                                 top_k=8, router="softmax", renormalize=False, wformat="int4_row"),
    # packed int2 (ternary codes): the OLMoE shape and the GLM shape
    "olmoe_int2": LayerShape("olmoe_int2", 1007, d_model=2048, n_experts=64, d_ff=1024,
                             top_k=8, router="softmax", renormalize=False, wformat="int2"),
    "glm_int2": LayerShape("glm_int2", 1008, d_model=6144, n_experts=256, d_ff=2048, top_k=8,
                           router="noaux_tc", n_group=8, topk_group=4,
                           routed_scaling_factor=2.5, has_bias=True, shared_expert=True,
                           wformat="int2"),
    # the 512-expert layer as its configuration states it: one ungated shared expert
    "qwen": LayerShape("qwen", 1005, d_model=2048, n_experts=512, d_ff=512, top_k=10,
                       router="softmax", renormalize=True, shared_expert=True,
                       wformat="int4", zipf_s=1.1),
    # the same weights with the shared expert scaled by sigmoid(x . u) per token
    "qwen_gated": LayerShape("qwen_gated", 1005, d_model=2048, n_experts=512, d_ff=512, top_k=10,
                             router="softmax", renormalize=True, shared_expert=True, shared_gate=True,
                             wformat="int4", zipf_s=1.1),
}

WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", LAYERS["tiny"], 16, "f32"),
    "tiny_q8": Workload("tiny_q8", LAYERS["tiny"], 16, "q8_0"),
    "olmoe_b1": Workload("olmoe_b1", LAYERS["olmoe"], 1, "f32"),
    "olmoe_b16": Workload("olmoe_b16", LAYERS["olmoe"], 16, "f32"),
    "olmoe_int4_prefill": Workload("olmoe_int4_prefill", LAYERS["olmoe_int4"], 2048, "q8_0"),
    "glm_b1": Workload("glm_b1", LAYERS["glm"], 1, "f32"),
    "glm_verify4": Workload("glm_verify4", LAYERS["glm"], 4, "q8_0"),
    "qwen_prefill": Workload("qwen_prefill", LAYERS["qwen"], 4096, "q8_0"),
    "qwen_gated_prefill": Workload("qwen_gated_prefill", LAYERS["qwen_gated"], 4096, "q8_0"),
    # the pages' decode knob: adaptive expert top-p 0.7
    "glm_b1_topp": Workload("glm_b1_topp", LAYERS["glm"], 1, "f32", top_p=0.7),
    "olmoe_b16_topp": Workload("olmoe_b16_topp", LAYERS["olmoe"], 16, "f32", top_p=0.7),
    "olmoe_b16_int4": Workload("olmoe_b16_int4", LAYERS["olmoe_int4"], 16, "f32"),
    # per-row weight scales (decode and prefill)
    "olmoe_b16_int4_row": Workload("olmoe_b16_int4_row", LAYERS["olmoe_int4_row"], 16, "f32"),
    "olmoe_int4_row_prefill": Workload("olmoe_int4_row_prefill", LAYERS["olmoe_int4_row"], 2048, "q8_0"),
    # packed int2 weights
    "olmoe_b16_int2": Workload("olmoe_b16_int2", LAYERS["olmoe_int2"], 16, "f32"),
    "olmoe_int2_prefill": Workload("olmoe_int2_prefill", LAYERS["olmoe_int2"], 2048, "q8_0"),
    "glm_b1_int2": Workload("glm_b1_int2", LAYERS["glm_int2"], 1, "f32"),
    # the layer with its neighbours fused in: RMSNorm before, residual after
    "olmoe_b16_block": Workload("olmoe_b16_block", LAYERS["olmoe"], 16, "f32", block=True),
    "olmoe_int4_prefill_block": Workload("olmoe_int4_prefill_block", LAYERS["olmoe_int4"], 2048, "q8_0", block=True),
}


def weight_bits(layer: LayerShape) -> int:
    """Code width of the layer's weight format: 8, 4 or 2."""
    return {"int8": 8, "int4": 4, "int2": 2}[layer.wformat.split("_")[0]]


def weight_per_row(layer: LayerShape) -> bool:
    """True for the per-row-scale formats ("..._row")."""
    return layer.wformat.endswith("_row")


def _rng(seed: int, tag: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, tag, index])


def _normal(seed: int, tag: int, index: int, shape, std: float) -> np.ndarray:
    out = _rng(seed, tag, index).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def zipf_ranks(layer: LayerShape) -> np.ndarray:
    """A seeded permutation of 1..E: expert e has popularity rank zipf_ranks[e]."""
    return _rng(layer.seed, TAG_ZIPF_RANK).permutation(layer.n_experts) + 1


def activations(layer: LayerShape, tokens: int) -> np.ndarray:
    """Hidden states X [T, d] fp32 ~ N(0, 1). Row t does not depend on T.

    With a Zipf prior the last feature is the constant 1, so that the router's
    last column acts as a per-expert logit offset (see ``gate_weight``).
    """
    x = _normal(layer.seed, TAG_X, 0, (tokens, layer.d_model), 1.0)
    if layer.zipf_s > 0:
        x[:, -1] = 1.0
    return x


def block_states(layer: LayerShape, tokens: int) -> np.ndarray:
    """Hidden states before the block's RMSNorm [T, d] fp32: N(0, 1) rows with
    a per-row scale in [0.25, 4) (the norm removes it); row t does not depend
    on T."""
    x = _normal(layer.seed, TAG_RESID, 0, (tokens, layer.d_model), 1.0)
    scale = np.exp2(_rng(layer.seed, TAG_RESID, 1).uniform(-2.0, 2.0, size=(65536,)))[:tokens]
    return (x * scale[:, None].astype(np.float32)).astype(np.float32)


def norm_weight(layer: LayerShape) -> np.ndarray:
    """The RMSNorm gain [d] fp32 ~ 1 + N(0, 0.1)."""
    return (1.0 + _normal(layer.seed, TAG_NORM_W, 0, (layer.d_model,), 0.1)).astype(np.float32)


def gate_weight(layer: LayerShape) -> np.ndarray:
    """Router weight Wg [E, d] fp32 ~ N(0, 0.02).

    With a Zipf prior the last column holds -s*ln(rank_e), so that an expert's
    logit carries the log of a Zipf(s) popularity on top of the N(0, .) noise.
    """
    wg = _normal(layer.seed, TAG_GATE_W, 0, (layer.n_experts, layer.d_model), WEIGHT_STD)
    if layer.zipf_s > 0:
        ranks = zipf_ranks(layer).astype(np.float64)
        wg[:, -1] = (-layer.zipf_s * np.log(ranks)).astype(np.float32)
    return wg


def shared_gate_weight(layer: LayerShape) -> Optional[np.ndarray]:
    """The shared expert's gate vector u [d] fp32 ~ N(0, 0.02), or None
    (ungated, or no shared expert)."""
    if not (layer.shared_expert and layer.shared_gate):
        return None
    return _normal(layer.seed, TAG_SHARED_GATE, 0, (layer.d_model,), WEIGHT_STD)


def score_bias(layer: LayerShape) -> Optional[np.ndarray]:
    """e_score_correction_bias [E] fp32 ~ N(0, 0.01), or None."""
    if not layer.has_bias:
        return None
    return _normal(layer.seed, TAG_BIAS, 0, (layer.n_experts,), BIAS_STD)


def expert_weight(layer: LayerShape, e: int, which: str) -> np.ndarray:
    """Unquantised fp32 weights of expert e (e == E is the shared expert).

    which: "gate" / "up" -> [I, d]; "down" -> [d, I]; each ~ N(0, 0.02).
    """
    if not (0 <= e <= layer.n_experts):
        raise ValueError(f"expert index {e} out of range")
    tag = {"gate": TAG_W_GATE, "up": TAG_W_UP, "down": TAG_W_DOWN}[which]
    shape = (layer.d_ff, layer.d_model) if which != "down" else (layer.d_model, layer.d_ff)
    return _normal(layer.seed, tag, e, shape, WEIGHT_STD)


def expert_weights_stacked(layer: LayerShape, which: str, experts=None,
                           threads: Optional[int] = None) -> np.ndarray:
    """Stack expert_weight over a list of experts (default: all routed experts)."""
    if experts is None:
        experts = range(layer.n_experts)
    experts = list(experts)
    shape = (layer.d_ff, layer.d_model) if which != "down" else (layer.d_model, layer.d_ff)
    out = np.empty((len(experts),) + shape, dtype=np.float32)

    def fill(i):
        out[i] = expert_weight(layer, experts[i], which)

    n = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=n) as pool:
        list(pool.map(fill, range(len(experts))))
    return out


def workload(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}") from None


def variant(layer: LayerShape, **changes) -> LayerShape:
    """A copy of a layer shape with some fields changed (for tiny test variants)."""
    return dataclasses.replace(layer, **changes)
