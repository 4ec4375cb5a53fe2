"""Helpers shared by the GPU parity tests: device layers built through the
library, oracle experts built by the oracle from the same seeded fp32 weights,
and the comparison rules."""
from __future__ import annotations

import functools
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import ffn as offn
from oracle import layer as olayer

REL_TOL = 2e-3          # max|gpu - ref| <= REL_TOL * max|ref| (per output tensor)


def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")


def say(*args):
    print(*args, file=sys.stderr, flush=True)


@functools.lru_cache(maxsize=4)
def device_layer(name: str):
    from quantized_expert_ffn_amd import device_layer as dl
    shape = synth.LAYERS[name]
    say(f"[gpu] building device layer {name}")
    return dl.build(shape, "cuda")


@functools.lru_cache(maxsize=2048)
def oracle_expert(name: str, e: int) -> offn.QuantExpert:
    shape = synth.LAYERS[name] if isinstance(name, str) else name
    bits = synth.weight_bits(shape)
    return offn.QuantExpert.from_fp32(synth.expert_weight(shape, e, "gate"), synth.expert_weight(shape, e, "up"),
                                      synth.expert_weight(shape, e, "down"), bits, synth.weight_per_row(shape))


def router_spec(shape, top_p=None) -> olayer.RouterSpec:
    return olayer.RouterSpec(mode=shape.router, top_k=shape.top_k, renormalize=shape.renormalize,
                             n_group=shape.n_group, topk_group=shape.topk_group,
                             routed_scaling_factor=shape.routed_scaling_factor, bias=synth.score_bias(shape),
                             top_p=shape.top_p if top_p is None else top_p,
                             shared_gate=synth.shared_gate_weight(shape))


def assert_close_rel(gpu: np.ndarray, ref: np.ndarray, tol: float = REL_TOL, what: str = "output"):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU values"
    scale = np.abs(ref).max()
    err = np.abs(gpu - ref).max()
    say(f"[parity] {what}: max|gpu-ref| = {err:.3e}, max|ref| = {scale:.3e}, rel = {err / max(scale, 1e-300):.3e}")
    assert err <= tol * scale, f"{what}: max|gpu-ref| {err:.3e} > {tol} * max|ref| {scale:.3e}"


def t2n(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def untile_codes(tiled: np.ndarray, n_rows: int, n_cols: int, fmt: str) -> np.ndarray:
    """Library weight codes (lane-tiled, group-major layout of include/moe.h) back to the
    row-major storage the oracle keeps: int8 [N, K], packed int4 [N, K/2]
    (element 2i in the low nibble of byte i) or packed int2 [N, K/4] (element
    4i + j in bits 2j of byte i)."""
    flat = np.asarray(tiled).reshape(-1).view(np.uint8)
    nt, g = n_rows // 32, n_cols // 32
    if fmt.startswith("int8"):
        # (group, tile, h, nl, half, byte) -> row = 32 tile + 16 half + nl, k = 32 group + 8 h + byte
        a = flat.reshape(g, nt, 4, 16, 2, 8).transpose(1, 4, 3, 0, 2, 5)
        return a.reshape(n_rows, n_cols).view(np.int8)
    if fmt.startswith("int2"):
        # (quad, tile, h, nl, group of quad, half, byte) -> byte column 8 group + 2 h + byte
        a = flat.reshape(g // 4, nt, 4, 16, 4, 2, 2).transpose(1, 5, 3, 0, 4, 2, 6)
        return a.reshape(n_rows, n_cols // 4)
    # (pair, tile, h, nl, group of pair, half, byte) -> byte column 16 group + 4 h + byte
    a = flat.reshape(g // 2, nt, 4, 16, 2, 2, 4).transpose(1, 5, 3, 0, 4, 2, 6)
    return a.reshape(n_rows, n_cols // 2)


def untile_scales(tiled: np.ndarray, n_rows: int, n_cols: int, fmt: str = "int8") -> np.ndarray:
    """Library scales back to the oracle's shape: group scales (lane-tiled
    layout) to row-major [N, K/32]; per-row scales (row order) to [N, 1]."""
    flat = np.asarray(tiled).reshape(-1)
    if fmt.endswith("_row"):
        return flat.reshape(n_rows, 1)
    nt, g = n_rows // 32, n_cols // 32
    a = flat.reshape(nt, g // 2, 16, 2, 2).transpose(0, 4, 2, 1, 3)   # (tile, half, nl, pair, group of pair)
    return a.reshape(n_rows, g)


# operand-slot order of H's codes in the workspace (include/moe.h,
# MOE_WS_H_CODES): slot j of each 8-wide slice holds k offset SLOT_K[codes][j]
SLOT_K = {"int8": [0, 2, 1, 3, 4, 6, 5, 7], "int4": [0, 4, 1, 5, 2, 6, 3, 7], "int2": list(range(8))}


def workspace_sections(ws: torch.Tensor, T: int, shape, act_mode: str, has_shared: bool):
    """The routing results (and, in Q8_0 mode, H's codes and scales) a layer
    call left in its workspace, as numpy arrays."""
    import quantized_expert_ffn_amd as qe
    k, E, d, I = shape.top_k, shape.n_experts, shape.d_model, shape.d_ff
    off = qe.moe_debug_workspace_sections(T, k, E, d, I, qe.ACT_MODES[act_mode], has_shared)
    raw = ws.detach().cpu().numpy().view(np.uint8)

    def take(name, dtype, count):
        o = off[name]
        return raw[o:o + count * np.dtype(dtype).itemsize].view(dtype).copy()

    n = T * k
    out = dict(idx=take("topk_idx", np.int32, n).reshape(T, k), w=take("topk_w", np.float32, n).reshape(T, k),
               counts=take("counts", np.int32, E), offsets=take("offsets", np.int32, E + 1),
               perm=take("perm", np.int32, n), inv_perm=take("inv_perm", np.int32, n))
    if act_mode == "q8_0":
        R = n + (T if has_shared else 0)
        codes = take("h_codes", np.float16, R * I).reshape(R, I // 8, 8)
        order = SLOT_K[shape.wformat.split("_")[0]]
        nat = np.empty_like(codes)
        nat[:, :, order] = codes
        # rows no slot was dispatched to hold whatever the workspace held
        out["hq"] = np.where(np.isfinite(nat), nat, 0).reshape(R, I).astype(np.int64)
        out["hd"] = take("h_scales", np.float32, R * (I // 32)).reshape(R, I // 32)
    return out


def h_code_flips(sec, shape, x, rows, oracle_expert_fn, shared_expert=None):
    """H's Q8_0 codes the GPU left for the given token rows against the
    oracle's, per routed slot (and the shared expert): returns (flips, total);
    asserts that no code differs by more than one step."""
    from oracle import ffn as offn
    k = shape.top_k
    T = sec["idx"].shape[0]
    flips = total = 0
    for t in rows:
        for j in range(k):
            e = int(sec["idx"][t, j])
            if e < 0:
                continue
            p = int(sec["inv_perm"][t * k + j])
            _, parts = offn.ffn_q8(x[t:t + 1], oracle_expert_fn(e))
            diff = sec["hq"][p] - parts["hq"][0].astype(np.int64)
            assert np.abs(diff).max() <= 1, f"token {t} slot {j}: H code off by {np.abs(diff).max()}"
            flips += int(np.count_nonzero(diff))
            total += diff.size
        if shared_expert is not None:
            _, parts = offn.ffn_q8(x[t:t + 1], shared_expert)
            diff = sec["hq"][T * k + t] - parts["hq"][0].astype(np.int64)
            assert np.abs(diff).max() <= 1, f"token {t} shared expert: H code off by {np.abs(diff).max()}"
            flips += int(np.count_nonzero(diff))
            total += diff.size
    return flips, total
