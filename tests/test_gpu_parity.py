"""GPU parity: the HIP library (through its C ABI) against the oracle.

Bit-exact: quantised weight bytes and scales, Q8_0 codes and scales, expert
indices (tokens whose selection margin is wider than fp32 logit rounding),
counts, offsets, the permutation and its inverse, int32 group dots.
Tolerance: every floating-point output tensor within 2e-3 * max|ref|.
"""
import dataclasses

import numpy as np
import pytest
import torch

import synth
import quantized_expert_ffn_amd as qe
from oracle import dispatch as odispatch
from oracle import ffn as offn
from oracle import layer as olayer
from oracle import quant as oquant
from oracle import router as orouter

from gpu_common import (REL_TOL, assert_close_rel, device_layer, h_code_flips, need_gpu, oracle_expert, router_spec,
                        say, t2n, untile_codes, untile_scales, workspace_sections)

pytestmark = pytest.mark.gpu

MARGIN_EPS = 1e-5      # logits closer than this may rank differently in fp32 vs fp64
TOPP_EPS = 1e-5        # top-p mass this close (relative) to the threshold may decide differently


# ---------------------------------------------------------------------------
# quantisers
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("fmt", ["int8", "int4", "int2", "int8_row", "int4_row", "int2_row"])
def test_quantize_weights_bit_exact(fmt):
    """A stack of two 64 x 256 matrices, with rows scaled over eight decades,
    an all-zero group and row, and a group of tiny values."""
    need_gpu()
    rng = np.random.default_rng(21)
    w = (rng.standard_normal((2, 64, 256)) * rng.uniform(1e-4, 3, (2, 64, 1))).astype(np.float32)
    w[0, 3, 32:64] = 0.0
    w[0, 4, :32] = 1e-30
    w[1, 5, :] = 0.0
    bits = {"int8": 8, "int4": 4, "int2": 2}[fmt.split("_")[0]]
    per_row = fmt.endswith("_row")
    qz = oquant.quantize_rows if per_row else oquant.quantize_weights
    refs = [qz(w[m], bits) for m in range(2)]
    stored = [oquant.pack_codes(q, bits) for q, _ in refs]
    q = torch.empty((2,) + stored[0].shape, dtype=torch.int8 if bits == 8 else torch.uint8, device="cuda")
    s = torch.empty((2,) + refs[0][1].shape, dtype=torch.float32, device="cuda")
    qe.moe_quantize_weights(torch.from_numpy(w).cuda(), qe.FORMATS[fmt], q, s)
    torch.cuda.synchronize()
    for m in range(2):
        assert np.array_equal(untile_scales(t2n(s[m]), 64, 256, fmt), refs[m][1])
        assert np.array_equal(untile_codes(t2n(q[m]), 64, 256, fmt), stored[m])


def test_quantize_q8_0_bit_exact(golden_dir):
    need_gpu()
    rng = np.random.default_rng(22)
    x = (rng.standard_normal((33, 96)) * rng.uniform(1e-3, 50, (33, 1))).astype(np.float32)
    x[2, :32] = 0.0
    fx = [l for l in open(f"{golden_dir}/q8_0_rounding.txt") if l.strip() and not l.startswith("#")][0]
    x[5, :32] = np.array([float(v) for v in fx.split("|")[0].split()], np.float32)
    q_ref, d_ref = oquant.quantize_q8_0(x)
    q = torch.empty(x.shape, dtype=torch.int8, device="cuda")
    d = torch.empty(d_ref.shape, dtype=torch.float32, device="cuda")
    qe.moe_quantize_q8_0(torch.from_numpy(x).cuda(), q, d)
    torch.cuda.synchronize()
    assert np.array_equal(t2n(d), d_ref)
    assert np.array_equal(t2n(q), q_ref)


# ---------------------------------------------------------------------------
# router
# ---------------------------------------------------------------------------
def gpu_route(x, wg, params, k):
    T = x.shape[0]
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    wgd = torch.from_numpy(np.ascontiguousarray(wg)).cuda()
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ws = qe.workspace(T, k, params.n_experts, x.shape[1], 32, qe.MOE_ACT_F32, False)
    qe.moe_route(xd, wgd, params, idx, w, ws)
    torch.cuda.synchronize()
    return t2n(idx), t2n(w)


def check_route(x, wg, spec: olayer.RouterSpec, bias=None):
    E = wg.shape[0]
    bias_d = torch.from_numpy(bias).cuda() if bias is not None else None
    params = qe.router_params(E, spec.top_k, spec.mode, spec.renormalize, spec.n_group, spec.topk_group,
                              spec.routed_scaling_factor, bias_d, spec.top_p)
    gi, gw = gpu_route(x, wg, params, spec.top_k)
    ri0, rw0, l = olayer.route(x, wg, dataclasses.replace(spec, top_p=0.0))
    ri, rw = orouter.apply_top_p(ri0, rw0, spec.top_p)
    keys = orouter.selection_keys(l, spec.mode, spec.bias, spec.n_group, spec.topk_group)
    margin = orouter.boundary_margin(keys, spec.top_k)
    if spec.mode == "noaux_tc":
        margin = np.minimum(margin, orouter.group_margin(l, spec.bias, spec.n_group, spec.topk_group))
    near = margin < MARGIN_EPS
    # top-p: a token whose kept mass lies within fp32 rounding of the threshold
    near_p = orouter.top_p_margin(rw0, spec.top_p) < TOPP_EPS
    say(f"[route] T={x.shape[0]} E={E} k={spec.top_k} mode={spec.mode} top_p={spec.top_p}: "
        f"min margin {margin.min():.3e}, near-ties {int(near.sum())}, near top-p {int(near_p.sum())}")
    # bit-exact wherever fp32 rounding cannot reorder the boundary
    ok = ~near & ~near_p
    assert np.array_equal(gi[ok], ri[ok])
    # near-tie tokens: the GPU choice must be a valid top-k within the margin
    for t in np.nonzero(near)[0]:
        kept = gi[t][gi[t] >= 0]
        rest = np.setdiff1d(np.arange(E), kept)
        if rest.size:
            assert keys[t, kept].min() >= keys[t, rest].max() - MARGIN_EPS
    # near top-p tokens: the kept slots are a prefix of the oracle's selection,
    # one slot longer or shorter at most
    for t in np.nonzero(near_p & ~near)[0]:
        n_gpu, n_ref = int((gi[t] >= 0).sum()), int((ri[t] >= 0).sum())
        assert abs(n_gpu - n_ref) <= 1 and np.array_equal(gi[t][:n_gpu], ri0[t][:n_gpu])
    assert np.all(gi[:, 0] >= 0)
    assert np.allclose(gw[ok], rw[ok], rtol=1e-5, atol=1e-7)
    return gi, gw


def test_route_tiny_softmax():
    need_gpu()
    lay = synth.LAYERS["tiny"]
    check_route(synth.activations(lay, 16), synth.gate_weight(lay), router_spec(lay))


@pytest.mark.parametrize("renorm", [False, True])
def test_route_exact_ties(renorm):
    need_gpu()
    x = np.random.default_rng(0).standard_normal((5, 64)).astype(np.float32)
    wg = np.zeros((8, 64), np.float32)
    p = qe.router_params(8, 3, "softmax", renorm)
    gi, gw = gpu_route(x, wg, p, 3)
    assert np.all(gi == [0, 1, 2])
    assert np.allclose(gw, 1 / 3 if renorm else 1 / 8, rtol=1e-6)
    wg = (np.random.default_rng(1).standard_normal((8, 64)) * 0.02).astype(np.float32)
    wg[6] = wg[2] = x[0] * 0.5
    gi, _ = gpu_route(x[:1], wg, qe.router_params(8, 2, "softmax", renorm), 2)
    assert list(gi[0]) == [2, 6]
    # sigmoid ties: all logits 0 -> all scores 0.5 -> lowest ids, weights rsf / k
    gi, gw = gpu_route(x, np.zeros((16, 64), np.float32), qe.router_params(16, 4, "noaux_tc", False, 4, 2, 2.5), 4)
    assert np.all(gi == [0, 1, 2, 3]) and np.allclose(gw, 2.5 / 4, rtol=1e-6)


@pytest.mark.parametrize("e,n_group,topk_group,k", [(8, 4, 2, 2), (16, 4, 2, 3), (64, 8, 3, 6), (256, 8, 4, 8)])
def test_route_noaux_tc_variants(e, n_group, topk_group, k):
    need_gpu()
    lay = synth.variant(synth.LAYERS["tiny"], router="noaux_tc", n_experts=e, n_group=n_group,
                        topk_group=topk_group, top_k=k, has_bias=True, routed_scaling_factor=2.5)
    x = synth.activations(lay, 64)
    wg = (synth.gate_weight(lay) * 15).astype(np.float32)      # logits of order 1
    spec = router_spec(lay)
    check_route(x, wg, spec, synth.score_bias(lay))


@pytest.mark.parametrize("mode", ["softmax", "noaux_tc"])
@pytest.mark.parametrize("top_p", [0.3, 0.7, 0.95])
def test_route_top_p(mode, top_p):
    need_gpu()
    if mode == "softmax":
        lay = synth.variant(synth.LAYERS["tiny"], n_experts=64, top_k=8, renormalize=False, top_p=top_p)
    else:
        lay = synth.variant(synth.LAYERS["tiny"], router="noaux_tc", n_experts=64, n_group=8, topk_group=4,
                            top_k=8, has_bias=True, routed_scaling_factor=2.5, top_p=top_p)
    x = synth.activations(lay, 300)
    wg = (synth.gate_weight(lay) * 15).astype(np.float32)
    gi, gw = check_route(x, wg, router_spec(lay), synth.score_bias(lay))
    kept = (gi >= 0).sum(axis=1)
    say(f"[route] top_p {top_p} {mode}: mean kept slots {kept.mean():.2f} of {lay.top_k}")


@pytest.mark.parametrize("e,k", [(1024, 64), (1024, 8), (128, 6), (100, 7), (40, 40), (512, 16)])
def test_route_max_experts_and_k(e, k):
    """Expert counts and k around the selection's limits: 64 lanes of 1..16
    experts each, k * experts-per-lane candidates up to 128 (ranked) and
    beyond (arg-max rounds), E not a multiple of 64, k = E."""
    need_gpu()
    lay = synth.variant(synth.LAYERS["tiny"], n_experts=e, top_k=k, renormalize=True)
    x = synth.activations(lay, 37)
    wg = (synth.gate_weight(lay) * 15).astype(np.float32)
    check_route(x, wg, router_spec(lay))


@pytest.mark.parametrize("name,tokens", [("olmoe", 16), ("olmoe_int4", 2048), ("glm", 4), ("qwen", 4096)])
def test_route_full_size(name, tokens):
    need_gpu()
    lay = synth.LAYERS[name]
    check_route(synth.activations(lay, tokens), synth.gate_weight(lay), router_spec(lay), synth.score_bias(lay))


def router_slices(T, E, d):
    """How many d-slices the router's logits come in for a batch of T
    (moe_route, no RMSNorm): the library's own choice, restated; a wrong
    count would make the sums below wrong and the test fail."""
    if T <= 16:
        if T <= 4:
            return 1
        u = -(-d // 256)
        pu = -(-u // 8)
        return -(-u // pu)
    tiles = -(-T // 128) * -(-E // 64)
    return max(1, min(-(-1024 // tiles), max(d // 128, 1)))


@pytest.mark.parametrize("T,E,d,name", [(1, 64, 2048, None), (8, 64, 2048, None), (16, 512, 2048, None),
                                        (300, 64, 2048, None), (300, 512, 2048, None), (200, 100, 196, None),
                                        (4096, 512, 2048, "qwen")])
def test_route_logits_values(T, E, d, name):
    """The router's logits (the slice sums moe_route leaves at the start of
    its workspace) against fp64 X Wg^T, within 1e-6 of sum_k |x_k w_k| for
    every logit: each decode path multiplies in fp32, the prefill path f16
    hi/lo parts of each value with a power of two per row (products within
    about 2^-21 of x w), all of them sum in fp32. Shapes cover the one-row,
    split-d and matrix-core logits kernels, both tile widths of the last,
    and rows that are not a multiple of 32 (padded parts)."""
    need_gpu()
    if name:
        lay = synth.LAYERS[name]
        x, wg = synth.activations(lay, T), synth.gate_weight(lay)
    else:
        rng = np.random.default_rng(T * 7 + E)
        x = (rng.standard_normal((T, d)) * rng.uniform(0.01, 100, (T, 1))).astype(np.float32)
        wg = (rng.standard_normal((E, d)) * 0.02).astype(np.float32)
    params = qe.router_params(E, min(8, E), "softmax", False)
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    wgd = torch.from_numpy(np.ascontiguousarray(wg)).cuda()
    idx = torch.empty((T, params.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, params.top_k), dtype=torch.float32, device="cuda")
    # (the workspace of d rounded up to 32 covers moe_route's need for d)
    ws = qe.workspace(T, params.top_k, E, -(-d // 32) * 32, 32, qe.MOE_ACT_F32, False)
    qe.moe_route(xd, wgd, params, idx, w, ws)
    torch.cuda.synchronize()
    S = router_slices(T, E, d)
    raw = ws.detach().cpu().numpy().view(np.uint8)[:S * T * E * 4].view(np.float32).reshape(S, T, E)
    got = raw.astype(np.float64).sum(axis=0)
    ref = x.astype(np.float64) @ wg.astype(np.float64).T
    scale = np.abs(x).astype(np.float64) @ np.abs(wg).astype(np.float64).T
    err = np.abs(got - ref) / (scale + 1e-30)
    say(f"[route logits] T={T} E={E} d={d} slices={S}: max error {err.max():.2e} of sum |x w|")
    assert err.max() <= 1e-6


# ---------------------------------------------------------------------------
# dispatch
# ---------------------------------------------------------------------------
def gpu_dispatch(idx, E, scratch=True):
    """scratch: pass a workspace (large batches then dispatch over many
    blocks); without one the single-block dispatch runs."""
    T, k = idx.shape
    n = max(1, T * k)
    ws = qe.workspace(T, k, E, 64, 64, qe.MOE_ACT_Q8_0, False) if scratch else None
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(n, dtype=torch.int32, device="cuda")
    inv = torch.empty(n, dtype=torch.int32, device="cuda")
    qe.moe_dispatch(torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).cuda(), E, counts, offsets,
                    perm, inv, ws)
    torch.cuda.synchronize()
    return t2n(counts), t2n(offsets), t2n(perm)[:T * k], t2n(inv)[:T * k]


@pytest.mark.parametrize("scratch", [True, False])
@pytest.mark.parametrize("T,k,E,zipf", [(16, 2, 8, False), (1, 8, 64, False), (16, 8, 64, False),
                                        (2048, 8, 64, False), (4, 8, 256, False), (4096, 10, 512, True),
                                        (64, 64, 1024, False), (3, 1, 1, False), (777, 3, 5, True),
                                        (2049, 1, 3, False), (1000, 9, 1024, True)])
def test_dispatch_bit_exact(T, k, E, zipf, scratch):
    need_gpu()
    rng = np.random.default_rng(T * 31 + k * 7 + E)
    if zipf:
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        p /= p.sum()
        idx = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)])
    else:
        idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    got = gpu_dispatch(idx, E, scratch)
    want = odispatch.dispatch(idx, E)
    for g, w, nm in zip(got, want, ("counts", "offsets", "perm", "inv_perm")):
        assert np.array_equal(g, w), nm


def test_dispatch_empty_and_out_of_range():
    need_gpu()
    c, o, _, _ = gpu_dispatch(np.zeros((0, 2), np.int32), 8)
    assert np.all(c == 0) and np.all(o == 0)
    idx = np.array([[0, 3], [7, 9], [-1, 3]], np.int32)         # 9 and -1 are outside [0, 8)
    c, o, perm, inv = gpu_dispatch(idx, 8)
    assert c.tolist() == [1, 0, 0, 2, 0, 0, 0, 1] and o[-1] == 4
    assert sorted(perm[:4].tolist()) == [0, 1, 2, 5]
    # a large batch (the multi-block dispatch) with dropped and out-of-range ids
    rng = np.random.default_rng(8)
    idx = rng.integers(0, 8, size=(1500, 3)).astype(np.int32)
    idx[::7, 2] = -1
    idx[5, 0], idx[901, 1], idx[1499, 2] = 8, 1 << 20, -5
    for scratch in (True, False):
        c, o, perm, inv = gpu_dispatch(idx, 8, scratch)
        # ids outside [0, E) are skipped like -1
        wc, wo, wp, wi = odispatch.dispatch(np.where((idx >= 0) & (idx < 8), idx, -1), 8)
        assert np.array_equal(c, wc) and np.array_equal(o, wo)
        assert np.array_equal(perm, wp) and np.array_equal(inv, wi)


# ---------------------------------------------------------------------------
# whole layer, small shapes (every output element)
# ---------------------------------------------------------------------------
def run_layer(dl, x_np, act_mode, copy=0, timed=False, top_p=None, return_ws=False):
    T = x_np.shape[0]
    lay = dl.shape
    params = dl.params if top_p is None else qe.with_top_p(dl.params, top_p)
    x = torch.from_numpy(np.ascontiguousarray(x_np)).cuda()
    out = torch.empty((T, lay.d_model), dtype=torch.float32, device="cuda")
    ws = qe.workspace(T, lay.top_k, lay.n_experts, lay.d_model, lay.d_ff, qe.ACT_MODES[act_mode],
                      dl.shared[copy] is not None)
    if timed:
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * qe.MOE_STAGE_COUNT)]
        qe.moe_layer_forward_timed(x, dl.gate_w, params, dl.routed[copy], dl.shared[copy],
                                   qe.ACT_MODES[act_mode], out, ws, evs)
        torch.cuda.synchronize()
        for s in range(qe.MOE_STAGE_COUNT):      # every stage that runs as its own launch was timed
            if qe.STAGES[s] == "quant_x":
                continue                         # done inside the router's logits launch
            ms = evs[2 * s].elapsed_time(evs[2 * s + 1])
            assert 0.0 < ms < 1000.0, (qe.STAGES[s], ms)
    else:
        qe.moe_layer_forward(x, dl.gate_w, params, dl.routed[copy], dl.shared[copy], qe.ACT_MODES[act_mode],
                             out, ws)
    torch.cuda.synchronize()
    if return_ws:
        return t2n(out), ws
    return t2n(out)


def oracle_layer(shape, x, act_mode, name=None, top_p=None):
    key = name or shape
    shared = oracle_expert(key, shape.n_experts) if shape.shared_expert else None
    wg = synth.gate_weight(shape)
    return olayer.layer_forward(x, wg, router_spec(shape, top_p), lambda e: oracle_expert(key, e), shared,
                                act_mode)


def report_h_flips(ws, shape, x, rows, what, key):
    """H's Q8_0 codes the layer left in its workspace against the oracle's, for
    the given tokens: every code within one step, and the count of one-step
    differences (the fp32 H on the GPU against fp64 in the oracle) reported."""
    sec = workspace_sections(ws, x.shape[0], shape, "q8_0", shape.shared_expert)
    shared = oracle_expert(key, shape.n_experts) if shape.shared_expert else None
    flips, total = h_code_flips(sec, shape, x, rows, lambda e: oracle_expert(key, e), shared)
    say(f"[q8] {what}: {flips} of {total} H codes differ by one step from the oracle's ({flips / max(total, 1):.2e})")
    assert flips <= max(2, total // 100)


def top_p_settled(shape, x, top_p=None):
    """Tokens whose top-p keep decisions are far from the threshold (fp32 and
    fp64 decide them alike); all tokens when top-p is off."""
    spec = router_spec(shape, top_p)
    if not 0.0 < spec.top_p < 1.0:
        return np.ones(x.shape[0], dtype=bool)
    _, w0, _ = olayer.route(x, synth.gate_weight(shape), dataclasses.replace(spec, top_p=0.0))
    return orouter.top_p_margin(w0, spec.top_p) >= TOPP_EPS


TINY_VARIANTS = {
    "tiny": {},
    "tiny_shared_noaux": dict(router="noaux_tc", n_experts=16, n_group=4, topk_group=2, top_k=3, has_bias=True,
                              routed_scaling_factor=2.5, shared_expert=True),
    "tiny_int4": dict(wformat="int4"),
    "tiny_e1k1": dict(n_experts=1, top_k=1, renormalize=True),
    "tiny_kE": dict(top_k=8, renormalize=False),
    "tiny_wide": dict(d_model=192, d_ff=320, n_experts=6, top_k=3),
    "tiny_topp": dict(n_experts=16, top_k=6, renormalize=False, top_p=0.6),
    "tiny_noaux_topp": dict(router="noaux_tc", n_experts=16, n_group=4, topk_group=2, top_k=4, has_bias=True,
                            routed_scaling_factor=2.5, shared_expert=True, top_p=0.7),
    # per-row scales; the wide one has odd group-pair counts on both axes
    "tiny_int8_row": dict(wformat="int8_row", shared_expert=True),
    "tiny_int4_row_wide": dict(wformat="int4_row", d_model=192, d_ff=320, n_experts=6, top_k=3),
    # a shared expert gated by sigmoid(x . u)
    "tiny_gated": dict(shared_expert=True, shared_gate=True),
    # packed int2 (K % 128 == 0 on both axes); the second has odd quad counts
    # along d_ff and a K-split along d_model in the decode kernel
    "tiny_int2": dict(wformat="int2", d_model=128, d_ff=256, shared_expert=True),
    "tiny_int2_row": dict(wformat="int2_row", d_model=512, d_ff=384, n_experts=6, top_k=3),
}


def tiny_layer(variant):
    from quantized_expert_ffn_amd import device_layer as dl
    shape = synth.variant(synth.LAYERS["tiny"], **TINY_VARIANTS[variant])
    if variant not in _TINY:
        _TINY[variant] = (shape, dl.build(shape, "cuda"))
    return _TINY[variant]


_TINY = {}


@pytest.mark.parametrize("act_mode", ["f32", "q8_0"])
@pytest.mark.parametrize("variant", list(TINY_VARIANTS))
def test_layer_tiny(variant, act_mode):
    need_gpu()
    shape, dl = tiny_layer(variant)
    # 600 tokens: experts span several 128-row prefill tiles, the last one short
    for T in (16, 1, 67, 600):
        x = synth.activations(shape, T)
        got, ws = run_layer(dl, x, act_mode, return_ws=True)
        ref = oracle_layer(shape, x, act_mode)
        ok = top_p_settled(shape, x)
        assert ok.sum() >= 0.98 * T
        assert_close_rel(got[ok], ref["out"][ok], what=f"{variant}/{act_mode}/T={T} out")
        if act_mode == "q8_0":
            report_h_flips(ws, shape, x, np.nonzero(ok)[0], f"{variant}/T={T}", shape)


def test_layer_zero_tokens_is_noop():
    need_gpu()
    shape, dl = tiny_layer("tiny")
    out = torch.full((1, shape.d_model), 7.0, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    x = torch.empty((0, shape.d_model), dtype=torch.float32, device="cuda")
    qe.moe_layer_forward(x, dl.gate_w, dl.params, dl.routed[0], None, qe.MOE_ACT_F32, out, ws)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


@pytest.mark.parametrize("act_mode", ["f32", "q8_0"])
def test_layer_deterministic(act_mode):
    need_gpu()
    shape, dl = tiny_layer("tiny_shared_noaux")
    x = synth.activations(shape, 67)
    a = run_layer(dl, x, act_mode)
    for _ in range(2):
        assert np.array_equal(run_layer(dl, x, act_mode, timed=True), a)


@pytest.mark.parametrize("act_mode", ["f32", "q8_0"])
@pytest.mark.parametrize("variant", ["tiny_wide", "tiny_int4_row_wide", "tiny_int2_row"])
def test_expert_ffn_and_combine_pieces(act_mode, variant):
    """moe_route -> moe_dispatch -> moe_expert_ffn -> moe_combine against the oracle's
    y_perm and out (routed only)."""
    need_gpu()
    shape, dl = tiny_layer(variant)
    T = 41
    x = synth.activations(shape, T)
    ref = oracle_layer(synth.variant(shape, shared_expert=False), x, act_mode, name=shape)
    k, E = shape.top_k, shape.n_experts
    xd = torch.from_numpy(x).cuda()
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    am = qe.ACT_MODES[act_mode]
    ws = qe.workspace(T, k, E, shape.d_model, shape.d_ff, am, False)
    qe.moe_route(xd, dl.gate_w, dl.params, idx, w, ws)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
    inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
    qe.moe_dispatch(idx, E, counts, offsets, perm, inv)
    y = torch.empty((T * k, shape.d_model), dtype=torch.float32, device="cuda")
    qe.moe_expert_ffn(xd, k, dl.routed[0], counts, offsets, perm, am, y, ws)
    out = torch.empty((T, shape.d_model), dtype=torch.float32, device="cuda")
    qe.moe_combine(y, w, inv, None, out)
    torch.cuda.synchronize()
    assert np.array_equal(t2n(idx), ref["idx"])
    assert np.array_equal(t2n(perm), ref["perm"])
    assert_close_rel(t2n(y), ref["y_perm"], what="y_perm")
    assert_close_rel(t2n(out), ref["out"], what="out")


@pytest.mark.parametrize("T", [29, 1, 4, 16])
@pytest.mark.parametrize("variant", ["tiny", "tiny_int4", "tiny_wide", "tiny_int4_row_wide", "tiny_int2",
                                     "tiny_int2_row"])
def test_q8_group_dots_bit_exact(variant, T):
    """The production Q8_0 kernels' exact int32 group dots, Q8_0(H) codes
    and the down projection's dots fed the GPU's own H codes: the tiled
    matrix-core GEMM above 16 tokens (T = 29), the small-batch GEMV up to 16
    (T = 1, 4, 16: the verification batches)."""
    need_gpu()
    shape, dl = tiny_layer(variant)
    k, E, d, I = shape.top_k, shape.n_experts, shape.d_model, shape.d_ff
    x = synth.activations(shape, T)
    ref = oracle_layer(shape, x, "q8_0")
    R = T * k
    xd = torch.from_numpy(x).cuda()
    counts = torch.from_numpy(ref["counts"]).cuda()
    offsets = torch.from_numpy(ref["offsets"]).cuda()
    perm = torch.from_numpy(ref["perm"]).cuda()
    dg = torch.empty((R, I, d // 32), dtype=torch.int32, device="cuda")
    du = torch.empty_like(dg)
    hq = torch.empty((R, I), dtype=torch.int8, device="cuda")
    hd = torch.empty((R, I // 32), dtype=torch.float32, device="cuda")
    dd = torch.empty((R, d, I // 32), dtype=torch.int32, device="cuda")
    y = torch.empty((R, d), dtype=torch.float32, device="cuda")
    ws = qe.workspace(T, k, E, d, I, qe.MOE_ACT_Q8_0, False)
    qe.moe_debug_q8_expert_ffn(xd, k, dl.routed[0], counts, offsets, perm, dg, du, hq, hd, dd, y, ws)
    torch.cuda.synchronize()
    dg, du, hq, hd, dd, y = map(t2n, (dg, du, hq, hd, dd, y))
    xq, xdq = oquant.quantize_q8_0(x)
    n_diff = 0
    for e in range(E):
        lo, hi = ref["offsets"][e], ref["offsets"][e + 1]
        if hi == lo:
            continue
        ex = oracle_expert(shape, e)
        toks = ref["perm"][lo:hi] // k
        assert np.array_equal(dg[lo:hi], offn.group_dots(xq[toks], ex.gate_q)), f"gate dots e={e}"
        assert np.array_equal(du[lo:hi], offn.group_dots(xq[toks], ex.up_q)), f"up dots e={e}"
        assert np.array_equal(dd[lo:hi], offn.group_dots(hq[lo:hi], ex.down_q)), f"down dots e={e}"
        _, parts = offn.ffn_q8(x[toks], ex)
        diff = hq[lo:hi].astype(int) - parts["hq"].astype(int)
        assert np.abs(diff).max() <= 1
        n_diff += int(np.count_nonzero(diff))
        y_ref, _ = offn.ffn_q8(x[toks], ex, hq_override=(hq[lo:hi], hd[lo:hi]))
        assert_close_rel(y[lo:hi], y_ref, what=f"y e={e} (GPU H codes)")
    say(f"[q8] {variant} T={T}: {n_diff} of {hq.size} H codes differ by 1 from the oracle's")
    assert n_diff <= max(2, hq.size // 100)


# ---------------------------------------------------------------------------
# full-size workloads
# ---------------------------------------------------------------------------
SAMPLE = 48


@pytest.mark.parametrize("wname", ["olmoe_b1", "olmoe_b16", "glm_b1", "glm_verify4", "olmoe_int4_prefill",
                                   "qwen_prefill", "qwen_gated_prefill", "glm_b1_topp", "olmoe_b16_topp", "olmoe_b16_int4_row",
                                   "olmoe_int4_row_prefill", "olmoe_b16_int2", "olmoe_int2_prefill",
                                   "glm_b1_int2"])
def test_layer_full_size(wname):
    need_gpu()
    wl = synth.workload(wname)
    shape = wl.layer
    dl = device_layer(shape.name)
    x = synth.activations(shape, wl.tokens)
    say(f"[gpu] {wname}: running the layer on T={wl.tokens}")
    top_p = wl.top_p or None
    got, ws = run_layer(dl, x, wl.act_mode, top_p=top_p, return_ws=True)
    rows = np.arange(wl.tokens)
    if wl.tokens > SAMPLE:
        rows = np.sort(np.random.default_rng(5).choice(wl.tokens, SAMPLE, replace=False))
    rows = rows[top_p_settled(shape, x[rows], top_p)]
    say(f"[oracle] {wname}: {len(rows)} tokens")
    ref = oracle_layer(shape, x[rows], wl.act_mode, name=shape.name, top_p=top_p)
    if top_p:
        say(f"[gpu] {wname}: top-p {top_p} keeps {(ref['idx'] >= 0).sum()} of {ref['idx'].size} slots")
    assert_close_rel(got[rows], ref["out"], what=f"{wname} out")
    if wl.act_mode == "q8_0":
        report_h_flips(ws, shape, x, rows, wname, shape.name)
    # the same weights, byte for byte, on both sides (a few experts)
    used = np.unique(ref["idx"][ref["idx"] >= 0])[:3]
    for e in used:
        ox = oracle_expert(shape.name, int(e))
        assert np.array_equal(untile_codes(t2n(dl.routed[0].gate_q[e]), shape.d_ff, shape.d_model, shape.wformat),
                              ox.stored("gate"))
        assert np.array_equal(untile_codes(t2n(dl.routed[0].down_q[e]), shape.d_model, shape.d_ff, shape.wformat),
                              ox.stored("down"))
        assert np.array_equal(untile_scales(t2n(dl.routed[0].down_s[e]), shape.d_model, shape.d_ff, shape.wformat),
                              ox.down_s)


def check_layer_routing(sec, shape, x, top_p=None):
    """The routing a layer call left in its workspace against the oracle's:
    expert ids bit for bit wherever the selection margin exceeds fp32 logit
    rounding (and top-p keep decisions are settled), weights to fp32
    rounding, and counts / offsets / perm / inv_perm bit for bit (equal to
    the oracle's dispatch of the GPU's own ids, and to the oracle's routing
    where no token is near a tie)."""
    spec = router_spec(shape, top_p)
    ri0, rw0, l = olayer.route(x, synth.gate_weight(shape), dataclasses.replace(spec, top_p=0.0))
    ri, rw = orouter.apply_top_p(ri0, rw0, spec.top_p)
    keys = orouter.selection_keys(l, spec.mode, spec.bias, spec.n_group, spec.topk_group)
    margin = orouter.boundary_margin(keys, spec.top_k)
    if spec.mode == "noaux_tc":
        margin = np.minimum(margin, orouter.group_margin(l, spec.bias, spec.n_group, spec.topk_group))
    ok = (margin >= MARGIN_EPS) & (orouter.top_p_margin(rw0, spec.top_p) >= TOPP_EPS)
    gi, gw = sec["idx"], sec["w"]
    assert np.array_equal(gi[ok], ri[ok])
    assert np.allclose(gw[ok], rw[ok], rtol=1e-5, atol=1e-7)
    mine = odispatch.dispatch(gi, shape.n_experts)
    for g, w, nm in zip((sec["counts"], sec["offsets"], sec["perm"], sec["inv_perm"]), mine,
                        ("counts", "offsets", "perm", "inv_perm")):
        assert np.array_equal(g, w), nm
    if ok.all():
        ref = odispatch.dispatch(ri, shape.n_experts)
        for g, w, nm in zip((sec["counts"], sec["offsets"], sec["perm"], sec["inv_perm"]), ref,
                            ("counts", "offsets", "perm", "inv_perm")):
            assert np.array_equal(g, w), nm
    return int((~ok).sum()), float(margin.min())


@pytest.mark.parametrize("wname,tokens", [("olmoe_b1", 1), ("olmoe_b16", 4), ("olmoe_b16", 16), ("glm_b1", 1),
                                          ("glm_verify4", 4), ("glm_verify4", 16), ("olmoe_b16_topp", 16),
                                          ("qwen_gated_prefill", 16)])
def test_layer_fused_routing_bit_exact(wname, tokens):
    """Up to 16 tokens the layer's top-k and dispatch run as one fused kernel
    whose results never leave the workspace: read them back after the call
    (include/moe.h, moe_debug_workspace_sections) and compare with the
    oracle's routing and dispatch."""
    need_gpu()
    wl = synth.workload(wname)
    shape = wl.layer
    dl = device_layer(shape.name)
    x = synth.activations(shape, tokens)
    _, ws = run_layer(dl, x, wl.act_mode, top_p=wl.top_p or None, return_ws=True)
    sec = workspace_sections(ws, tokens, shape, wl.act_mode, shape.shared_expert)
    near, margin = check_layer_routing(sec, shape, x, wl.top_p or None)
    say(f"[route] {wname} T={tokens}: fused routing read back, min margin {margin:.3e}, unsettled tokens {near}")


@pytest.mark.parametrize("act_mode", ["f32", "q8_0"])
@pytest.mark.parametrize("variant", ["tiny_noaux_topp", "tiny_shared_noaux", "tiny_topp", "tiny_kE", "tiny_e1k1"])
def test_layer_fused_routing_tiny(variant, act_mode):
    need_gpu()
    shape, dl = tiny_layer(variant)
    for T in (1, 4, 16, 67):
        x = synth.activations(shape, T)
        _, ws = run_layer(dl, x, act_mode, return_ws=True)
        sec = workspace_sections(ws, T, shape, act_mode, shape.shared_expert)
        check_layer_routing(sec, shape, x)


@pytest.mark.parametrize("variant,T", [("tiny_shared_noaux", 700), ("tiny", 1400), ("tiny_int4", 1100)])
def test_layer_prefill_tile_layout(variant, T):
    """Batches large enough for the multi-block dispatch (T*k > 2048), whose
    work lists lay the full 128-row tiles out in 8 runs, one per XCD, with
    empty tiles evening the runs out. For each case the host counts, from the
    oracle's routing, how many full tiles there are: the cases are chosen so
    that the count is not a multiple of 8 (empty tiles exist and are skipped)
    or a run boundary splits an expert's tiles. Q8_0 outputs against the
    oracle."""
    need_gpu()
    shape, dl = tiny_layer(variant)
    assert T * shape.top_k > 2048
    x = synth.activations(shape, T)
    spec = router_spec(shape)
    idx, _, _ = olayer.route(x, synth.gate_weight(shape), spec)
    counts = np.bincount(idx[idx >= 0].ravel(), minlength=shape.n_experts)
    n_full = int((counts // 128).sum()) + (T // 128 if shape.shared_expert else 0)
    run = (n_full + 7) // 8
    empty = 8 * run - n_full
    starts = np.concatenate([[0], np.cumsum(counts // 128)])
    split = any(s0 // run != (s0 + c - 1) // run for s0, c in zip(starts[:-1], counts // 128) if c > 0)
    say(f"[tiles] {variant}/T={T}: {n_full} full tiles, runs of {run}, {empty} empty, expert split across runs: {split}")
    assert empty > 0 or split
    got = run_layer(dl, x, "q8_0")
    ref = oracle_layer(shape, x, "q8_0")
    ok = top_p_settled(shape, x)
    assert_close_rel(got[ok], ref["out"][ok], what=f"{variant}/q8_0/T={T} out")


@pytest.mark.parametrize("act_mode", ["f32", "q8_0"])
@pytest.mark.parametrize("variant,T", [("tiny_shared_noaux", 67), ("tiny_gated", 1100)])
def test_layer_hip_graph_replay(act_mode, variant, T):
    """The layer captured in a HIP graph: every replay, with eager work and
    synchronisation between replays, equals the eager result bit for bit.
    1100 tokens x top-2 take the multi-block dispatch and the tiled router
    (with the shared-expert gate row)."""
    need_gpu()
    shape, dl = tiny_layer(variant)
    x = torch.from_numpy(synth.activations(shape, T)).cuda()
    am = qe.ACT_MODES[act_mode]
    ws = qe.workspace(T, shape.top_k, shape.n_experts, shape.d_model, shape.d_ff, am, True)
    eager = torch.empty((T, shape.d_model), dtype=torch.float32, device="cuda")
    qe.moe_layer_forward(x, dl.gate_w, dl.params, dl.routed[0], dl.shared[0], am, eager, ws)
    torch.cuda.synchronize()
    out = torch.zeros_like(eager)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qe.moe_layer_forward(x, dl.gate_w, dl.params, dl.routed[0], dl.shared[0], am, out, ws)
    for r in range(4):
        out.zero_()
        ws.fill_(0xAB)                      # eager work between replays, scrambling the workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs"


# ---------------------------------------------------------------------------
# the layer between its neighbours: RMSNorm before, residual after
# ---------------------------------------------------------------------------
def run_block(dl, x_np, act_mode, norm_w, eps, in_place=False):
    T = x_np.shape[0]
    lay = dl.shape
    x = torch.from_numpy(np.ascontiguousarray(x_np)).cuda()
    out = x if in_place else torch.empty_like(x)
    g = torch.from_numpy(norm_w).cuda() if norm_w is not None else None
    ws = qe.workspace(T, lay.top_k, lay.n_experts, lay.d_model, lay.d_ff, qe.ACT_MODES[act_mode],
                      dl.shared[0] is not None)
    qe.moe_block_forward(x, g, eps, dl.gate_w, dl.params, dl.routed[0], dl.shared[0], qe.ACT_MODES[act_mode], out, ws)
    torch.cuda.synchronize()
    return t2n(out)


def oracle_block(shape, x, act_mode, norm_w, eps, name=None):
    key = name or shape
    shared = oracle_expert(key, shape.n_experts) if shape.shared_expert else None
    return olayer.block_forward(x, norm_w, eps, synth.gate_weight(shape), router_spec(shape),
                                lambda e: oracle_expert(key, e), shared, act_mode)


@pytest.mark.parametrize("act_mode", ["f32", "q8_0"])
@pytest.mark.parametrize("variant", ["tiny", "tiny_shared_noaux", "tiny_int4", "tiny_topp", "tiny_gated"])
def test_block_forward_tiny(variant, act_mode):
    need_gpu()
    shape, dl = tiny_layer(variant)
    gamma = synth.norm_weight(shape)
    for T, norm, in_place in ((16, True, False), (67, True, True), (16, False, True), (67, False, False), (1, True, False)):
        x = synth.block_states(shape, T)
        g = gamma if norm else None
        got = run_block(dl, x, act_mode, g, 1e-6, in_place)
        ref = oracle_block(shape, x, act_mode, g, 1e-6)
        ok = top_p_settled(shape, ref["x_norm"])
        assert_close_rel(got[ok], ref["out"][ok], what=f"{variant}/{act_mode}/T={T}/norm={norm} block out")
        # the layer's own part, against the same tolerance (the residual is exact)
        assert_close_rel(got[ok] - x[ok], ref["out"][ok] - x[ok].astype(np.float64),
                         what=f"{variant}/{act_mode}/T={T} layer part")


@pytest.mark.parametrize("wname", ["olmoe_b16", "glm_verify4", "olmoe_int4_prefill"])
def test_block_forward_full_size(wname):
    need_gpu()
    wl = synth.workload(wname)
    shape = wl.layer
    dl = device_layer(shape.name)
    x = synth.block_states(shape, wl.tokens)
    gamma = synth.norm_weight(shape)
    got = run_block(dl, x, wl.act_mode, gamma, 1e-5)
    rows = np.arange(wl.tokens)
    if wl.tokens > SAMPLE:
        rows = np.sort(np.random.default_rng(6).choice(wl.tokens, SAMPLE, replace=False))
    ref = oracle_block(shape, x[rows], wl.act_mode, gamma, 1e-5, name=shape.name)
    assert_close_rel(got[rows] - x[rows], ref["out"] - x[rows].astype(np.float64), what=f"{wname} block layer part")


# ---------------------------------------------------------------------------
# tokens of very different magnitudes in one batch
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("act_mode", ["f32", "q8_0"])
@pytest.mark.parametrize("name", ["tiny", "tiny_int4", "tiny_shared_noaux", "olmoe", "glm"])
def test_layer_mixed_token_magnitudes(name, act_mode):
    """16 tokens whose rows are scaled by 2^-10 .. 2^10. Every token is checked
    against the oracle relative to its own largest output: the f32 path keeps
    one power of two per 32-column group of X over the whole batch and one per
    row and group of H, so a small token next to a large one keeps its own
    precision. Tokens whose top-k boundary lies within fp32 rounding of their
    own logits are left out of the comparison."""
    need_gpu()
    T = 16
    if name in ("olmoe", "glm"):
        shape, dl, key = synth.LAYERS[name], device_layer(name), name
    else:
        shape, dl = tiny_layer(name)
        key = shape
    scales = np.exp2(np.linspace(-10.0, 10.0, T))
    x = (synth.activations(shape, T) * scales[:, None]).astype(np.float32)
    got = run_layer(dl, x, act_mode)
    ref = oracle_layer(shape, x, act_mode, name=key)
    spec = router_spec(shape)
    keys = orouter.selection_keys(ref["logits"], spec.mode, spec.bias, spec.n_group, spec.topk_group)
    margin = orouter.boundary_margin(keys, spec.top_k)
    if spec.mode == "noaux_tc":
        margin = np.minimum(margin, orouter.group_margin(ref["logits"], spec.bias, spec.n_group, spec.topk_group))
    key_scale = np.abs(np.where(np.isfinite(keys), keys, 0.0)).max(axis=1)   # ineligible experts hold -inf
    settled = margin >= 1e-5 * key_scale + 1e-30
    assert settled.sum() >= T - 2
    worst = 0.0
    for t in np.nonzero(settled)[0]:
        scale = np.abs(ref["out"][t]).max()
        err = np.abs(got[t] - ref["out"][t]).max() / scale
        worst = max(worst, err)
        assert err <= REL_TOL, f"token {t} (row scale 2^{np.log2(scales[t]):.1f}): rel err {err:.3e}"
    say(f"[mixed] {name}/{act_mode}: worst per-token rel err {worst:.3e} over {int(settled.sum())} tokens "
        f"(row scales 2^-10 .. 2^10)")
