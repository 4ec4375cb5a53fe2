"""Pins for the oracle's expert FFN and whole layer (CPU only).

Dense masked evaluation (every expert applied to every token, weighted by the
routing mask) against the sparse batch-union path; special cases that reduce
to a dense SwiGLU or a dense softmax mixture; closed forms of SiLU and the
SwiGLU orientation; brute-force integer dots; the Q8_0 error bound.
"""
import math

import numpy as np
import pytest

from oracle import ffn, layer, quant
import synth


def _tiny_experts(lay, bits=None):
    bits = bits or (synth.weight_bits(lay))
    return [ffn.QuantExpert.from_fp32(synth.expert_weight(lay, e, "gate"),
                                      synth.expert_weight(lay, e, "up"),
                                      synth.expert_weight(lay, e, "down"), bits, synth.weight_per_row(lay))
            for e in range(lay.n_experts + (1 if lay.shared_expert else 0))]


def _spec(lay, **over):
    kw = dict(mode=lay.router, top_k=lay.top_k, renormalize=lay.renormalize,
              n_group=lay.n_group, topk_group=lay.topk_group,
              routed_scaling_factor=lay.routed_scaling_factor, bias=synth.score_bias(lay))
    kw.update(over)
    return layer.RouterSpec(**kw)


def test_silu_closed_forms():
    g = np.array([0.0, 30.0, -30.0, 1.0, -1.0])
    s = ffn.silu(g)
    assert s[0] == 0.0
    assert abs(s[1] - 30.0) < 1e-9 and abs(s[2]) < 1e-9
    assert abs((s[3] - s[4]) - 1.0) < 1e-15          # silu(x) - silu(-x) = x
    assert abs(s[3] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15


def test_swiglu_orientation_is_silu_of_gate_times_up():
    # one-hot token through hand-built weights whose group scales are exact
    # powers of two (amax = 127 * 2^-n): G = 127/64, U = 127/256
    d, i = 32, 32
    gate = np.zeros((i, d), np.float32)
    up = np.zeros((i, d), np.float32)
    down = np.zeros((d, i), np.float32)
    gate[0, 0] = 127 / 64
    up[0, 0] = 127 / 256
    down[0, 0] = 127 / 128
    ex = ffn.QuantExpert.from_fp32(gate, up, down, 8)
    x = np.zeros((1, d), np.float32)
    x[0, 0] = 1.0
    y = ffn.ffn_f32(x, ex)
    g, u = 127 / 64, 127 / 256
    want = g / (1.0 + math.exp(-g)) * u * (127 / 128)  # silu(gate) * up, through down
    assert ex.gate_s[0, 0] == 1 / 64 and ex.up_s[0, 0] == 1 / 256
    assert abs(y[0, 0] - want) < 1e-12
    assert abs(y[0, 0] - u / (1 + math.exp(-u)) * g * (127 / 128)) > 0.1   # swapped orientation


@pytest.mark.parametrize("act_mode", ["f32", "q8_0"])
def test_dense_masked_equals_sparse_tiny(act_mode):
    lay = synth.LAYERS["tiny"]
    x = synth.activations(lay, 16)
    wg = synth.gate_weight(lay)
    exps = _tiny_experts(lay)
    spec = _spec(lay)
    r = layer.layer_forward(x, wg, spec, lambda e: exps[e], None, act_mode)
    # dense: every expert on every token, weighted by the routing mask
    mask = np.zeros((16, lay.n_experts))
    for t in range(16):
        for j in range(lay.top_k):
            mask[t, r["idx"][t, j]] += r["w"][t, j]
    dense = np.zeros((16, lay.d_model))
    for e in range(lay.n_experts):
        ye = layer.expert_rows(x, exps[e], act_mode)
        dense += mask[:, e:e + 1] * ye
    assert np.allclose(r["out"], dense, rtol=0, atol=1e-12 * np.abs(dense).max())


@pytest.mark.parametrize("wformat", ["int8", "int4", "int2", "int2_row"])
def test_single_expert_is_dense_swiglu(wformat):
    lay = synth.variant(synth.LAYERS["tiny"], n_experts=1, top_k=1, renormalize=True, wformat=wformat)
    x = synth.activations(lay, 16)
    wg = synth.gate_weight(lay)
    exps = _tiny_experts(lay)
    r = layer.layer_forward(x, wg, _spec(lay), lambda e: exps[e], None, "f32")
    assert np.all(r["idx"] == 0) and np.allclose(r["w"], 1.0)
    wgt, wup, wdn = (quant.dequantize(q, s) for q, s in
                     [(exps[0].gate_q, exps[0].gate_s), (exps[0].up_q, exps[0].up_s),
                      (exps[0].down_q, exps[0].down_s)])
    x64 = x.astype(np.float64)
    g = x64 @ wgt.T
    dense = ((g / (1 + np.exp(-g))) * (x64 @ wup.T)) @ wdn.T
    assert np.allclose(r["out"], dense, rtol=1e-12, atol=1e-14)


def test_all_experts_is_softmax_mixture():
    lay = synth.variant(synth.LAYERS["tiny"], top_k=8, renormalize=False)
    x = synth.activations(lay, 16)
    wg = synth.gate_weight(lay)
    exps = _tiny_experts(lay)
    r = layer.layer_forward(x, wg, _spec(lay), lambda e: exps[e], None, "f32")
    l = x.astype(np.float64) @ wg.astype(np.float64).T
    p = np.exp(l - l.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    mix = sum(p[:, e:e + 1] * ffn.ffn_f32(x, exps[e]) for e in range(8))
    assert np.allclose(r["out"], mix, rtol=1e-11, atol=1e-14)


def test_shared_expert_adds_with_weight_one():
    lay = synth.variant(synth.LAYERS["tiny"], shared_expert=True)
    x = synth.activations(lay, 16)
    wg = synth.gate_weight(lay)
    exps = _tiny_experts(lay)
    base = layer.layer_forward(x, wg, _spec(lay), lambda e: exps[e], None, "f32")
    withs = layer.layer_forward(x, wg, _spec(lay), lambda e: exps[e], exps[lay.n_experts], "f32")
    s = ffn.ffn_f32(x, exps[lay.n_experts])
    assert np.allclose(withs["out"] - base["out"], s, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("act_mode", ["f32", "q8_0"])
def test_gated_shared_expert_closed_forms(act_mode):
    """A zero gate vector halves the shared expert (sigmoid(0) = 1/2); a gate
    vector along token 0's hidden state gives that token sigmoid(alpha)."""
    lay = synth.variant(synth.LAYERS["tiny"], shared_expert=True)
    x = synth.activations(lay, 5)
    wg = synth.gate_weight(lay)
    exps = _tiny_experts(lay)
    sh = exps[lay.n_experts]
    routed = layer.layer_forward(x, wg, _spec(lay), lambda e: exps[e], None, act_mode)["out"]
    full = layer.layer_forward(x, wg, _spec(lay), lambda e: exps[e], sh, act_mode)["out"]
    s = full - routed
    half = layer.layer_forward(x, wg, _spec(lay, shared_gate=np.zeros(lay.d_model)), lambda e: exps[e], sh,
                               act_mode)
    assert np.allclose(half["out"] - routed, 0.5 * s, rtol=1e-12, atol=1e-15)
    assert np.all(half["shared_gate"] == 0.5)
    alpha = 1.7
    x0 = x[0].astype(np.float64)
    u = alpha * x0 / (x0 @ x0)
    r = layer.layer_forward(x, wg, _spec(lay, shared_gate=u), lambda e: exps[e], sh, act_mode)
    g0 = 1.0 / (1.0 + math.exp(-alpha))
    assert abs(r["shared_gate"][0] - g0) < 1e-12
    assert np.allclose(r["out"][0] - routed[0], g0 * s[0], rtol=1e-10, atol=1e-15)
    # the gate is per token: x[t] . u for the other rows too, and never enters the routing
    z = x.astype(np.float64) @ u
    assert np.allclose(r["shared_gate"], 1.0 / (1.0 + np.exp(-z)), rtol=1e-14)
    assert np.array_equal(r["idx"], half["idx"])
    # without a shared expert the gate is ignored
    assert np.array_equal(layer.layer_forward(x, wg, _spec(lay, shared_gate=u), lambda e: exps[e], None,
                                              act_mode)["out"], routed)


def test_group_dots_brute_force_python_ints():
    rng = np.random.default_rng(4)
    a = rng.integers(-127, 128, size=(3, 64)).astype(np.int8)
    b = rng.integers(-127, 128, size=(5, 64)).astype(np.int8)
    a[0, :32] = -127
    b[0, :32] = -127                                   # the extreme group: 32*127*127
    got = ffn.group_dots(a, b)
    for m in range(3):
        for n in range(5):
            for g in range(2):
                want = sum(int(a[m, k]) * int(b[n, k]) for k in range(32 * g, 32 * g + 32))
                assert got[m, n, g] == want
    assert got[0, 0, 0] == 32 * 127 * 127 and got[0, 0, 0] < 2 ** 31


def test_q8_integer_dots_equal_product_form():
    lay = synth.LAYERS["tiny"]
    x = synth.activations(lay, 16)
    ex = _tiny_experts(lay)[3]
    _, parts = ffn.ffn_q8(x, ex)
    dots = ffn.group_dots(parts["xq"], ex.gate_q)                     # [16, I, G]
    g_int = np.einsum("mg,ng,mng->mn", parts["xd"].astype(np.float64),
                      ex.gate_s.astype(np.float64), dots.astype(np.float64))
    assert np.allclose(g_int, parts["g"], rtol=1e-13, atol=1e-15)


def test_q8_vs_f32_first_projection_bound():
    lay = synth.LAYERS["olmoe"]
    x = synth.activations(lay, 4)
    gate = synth.expert_weight(lay, 0, "gate")[:64]
    q, s = quant.quantize_weights(gate, 8)
    w = quant.dequantize(q, s)
    xq, xd = quant.quantize_q8_0(x)
    g_q8 = quant.dequantize(xq, xd) @ w.T
    g_f32 = x.astype(np.float64) @ w.T
    # |x - dequant(Q8_0(x))| <= d/2 per element, so the error is bounded by sum |w| d/2
    bound = (np.abs(w)[None, :, :] * np.repeat(xd.astype(np.float64), 32, axis=1)[:, None, :] / 2).sum(-1)
    assert np.all(np.abs(g_q8 - g_f32) <= bound * (1 + 1e-6))


def test_layer_noaux_tc_weights_sum_to_scaling_factor():
    lay = synth.variant(synth.LAYERS["tiny"], router="noaux_tc", n_group=4, topk_group=2,
                        routed_scaling_factor=2.5, has_bias=True, n_experts=16, top_k=3)
    x = synth.activations(lay, 16)
    wg = synth.gate_weight(lay)
    exps = _tiny_experts(lay)
    r = layer.layer_forward(x, wg, _spec(lay), lambda e: exps[e], None, "f32")
    assert np.allclose(r["w"].sum(1), 2.5, rtol=1e-12)


# ---------------------------------------------------------------------------
# the neighbours of the layer: RMSNorm before it, the residual after it
# ---------------------------------------------------------------------------
def test_rmsnorm_closed_forms():
    d = 64
    gamma = np.linspace(0.5, 1.5, d)
    # a constant row c: mean(x^2) = c^2, so x_norm = sign(c) * gamma / sqrt(1 + eps / c^2)
    for c, eps in ((3.0, 0.0), (-0.25, 1e-6), (2.0, 1e-2)):
        got = layer.rmsnorm(np.full((1, d), c), gamma, eps)[0]
        assert np.allclose(got, np.sign(c) * gamma / math.sqrt(1.0 + eps / c ** 2), rtol=1e-14, atol=0)
    # a row of one +a and (d-1) zeros: mean(x^2) = a^2/d, x_norm[0] = sqrt(d) * gamma[0]
    x = np.zeros((1, d))
    x[0, 0] = 7.0
    got = layer.rmsnorm(x, gamma, 0.0)[0]
    assert math.isclose(got[0], math.sqrt(d) * gamma[0], rel_tol=1e-14) and np.all(got[1:] == 0)
    # with eps = 0: invariant to a positive scale of the row, unit root-mean-square before gamma
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, d))
    a = layer.rmsnorm(x, np.ones(d), 0.0)
    assert np.allclose(layer.rmsnorm(37.5 * x, np.ones(d), 0.0), a, rtol=1e-13, atol=0)
    assert np.allclose(np.sqrt((a * a).mean(axis=1)), 1.0, rtol=1e-13)


def test_block_residual_only_when_the_norm_gain_is_zero():
    # gamma = 0: the layer sees zero states, every logit is 0 (experts 0..k-1
    # by the tie rule), every expert output is 0, so out is the residual x
    lay = synth.variant(synth.LAYERS["tiny"], shared_expert=True)
    x = synth.activations(lay, 9)
    exps = _tiny_experts(lay)
    for act in ("f32", "q8_0"):
        r = layer.block_forward(x, np.zeros(lay.d_model), 1e-6, synth.gate_weight(lay), _spec(lay),
                                lambda e: exps[e], exps[lay.n_experts], act)
        assert np.array_equal(r["out"], x.astype(np.float64))
        assert np.all(r["idx"] == np.arange(lay.top_k))


def test_block_without_norm_is_residual_plus_layer():
    lay = synth.variant(synth.LAYERS["tiny"], shared_expert=True)
    x = synth.activations(lay, 9)
    exps = _tiny_experts(lay)
    wg = synth.gate_weight(lay)
    r = layer.block_forward(x, None, 0.0, wg, _spec(lay), lambda e: exps[e], exps[lay.n_experts], "f32")
    base = layer.layer_forward(x, wg, _spec(lay), lambda e: exps[e], exps[lay.n_experts], "f32")
    assert np.array_equal(r["out"], x.astype(np.float64) + base["out"])


# ---------------------------------------------------------------------------
# the Q8_0 path's second half, worked with exact integers
# ---------------------------------------------------------------------------
def _round_binary(q, mant_bits: int):
    """Round a rational to the nearest binary floating-point number with
    mant_bits significant bits, ties to the even mantissa (IEEE round to
    nearest in the normal range; the values used here are all normal)."""
    from fractions import Fraction
    q = Fraction(q)
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    ulp = Fraction(2) ** (e - mant_bits + 1)
    m = a / ulp
    whole = m.numerator // m.denominator
    rest = m - whole
    if rest > Fraction(1, 2) or (rest == Fraction(1, 2) and whole % 2 == 1):
        whole += 1
    return sign * whole * ulp


def _rne_int(q) -> int:
    from fractions import Fraction
    q = Fraction(q)
    whole = q.numerator // q.denominator
    rest = q - whole
    if rest > Fraction(1, 2) or (rest == Fraction(1, 2) and whole % 2 == 1):
        whole += 1
    return whole


def _q8_0_exact(row):
    """Q8_0 of one group of 32 exact rationals in the quantiser's fp32 steps
    ("Show HN: Getting GLM-5.2 running on my slow computer", section "What's
    implemented": Q8_0-style int8 activations), each step rounded to fp32 by
    _round_binary: d = fp32(amax / 127), id = fp32(1 / d), q = rne(fp32(v * id))."""
    from fractions import Fraction
    f32 = lambda v: _round_binary(v, 24)  # noqa: E731
    amax = max(abs(v) for v in row)
    d = f32(amax / 127)
    idv = f32(Fraction(1) / d) if d != 0 else Fraction(0)
    return [max(-127, min(127, _rne_int(f32(v * idv)))) for v in row], d


def test_q8_second_half_hand_worked_exact_integers():
    """d = I = 32, two tokens, one int8 expert with dyadic weights chosen by
    hand. Every quantity of the Q8_0 path is recomputed here with Python
    integers and exact fractions (no numpy arithmetic): the Q8_0 codes of X,
    the integer group dots and G, U; H = silu(G) * U taken in fp64 and then
    rounded to fp32 (silu(G) = G exactly: every G here is either 0 or >= 38,
    where 1 + e^-G rounds to 1 in fp64); the Q8_0 codes and scale of that fp32
    H; the down projection's integer dots over those codes and Y = hd * sw * dot.
    The oracle must reproduce each one bit for bit."""
    from fractions import Fraction as Fr
    d = i_ff = 32
    x = np.zeros((2, d), np.float32)
    x[0, :3] = [100.0, -37.25, 3.0]      # amax 100: a scale that is no power of two
    x[1, 3:5] = [50.0, 50.0]
    # gate row n: code 127 at k = 0 (the group's largest, so the scale is 2^-1),
    # codes g1 at k = 1 and g3 at k = 3 (g3 = 0 or >= 2 keeps token 1's G at 0 or >= 38)
    g1 = [(-1) ** n * (7 * n % 120) for n in range(i_ff)]
    g3 = [0 if n % 5 == 0 else 2 + (11 * n) % 100 for n in range(i_ff)]
    gate = np.zeros((i_ff, d), np.float32)
    gate[:, 0] = 127 * 0.5
    gate[:, 1] = np.array(g1, np.float32) * 0.5
    gate[:, 3] = np.array(g3, np.float32) * 0.5
    # up row n: codes on k = 0..4 and the largest code, 127, at k = 31 (where
    # both tokens are 0), so the scale is 2^-6
    u_codes = [[(5 * n + 3 * j) % 255 - 127 for j in range(5)] for n in range(i_ff)]
    up = np.zeros((i_ff, d), np.float32)
    up[:, :5] = np.array(u_codes, np.float32) * 2.0 ** -6
    up[:, 31] = 127 * 2.0 ** -6
    # down row j: scale 2^-(7 + j % 3), codes spread over [-127, 127], 127 at n = j
    down = np.zeros((d, i_ff), np.float32)
    for j in range(d):
        c = [((13 * j + 29 * n) % 255) - 127 for n in range(i_ff)]
        c[j] = 127
        down[j] = np.array(c, np.float32) * 2.0 ** -(7 + j % 3)
    ex = ffn.QuantExpert.from_fp32(gate, up, down, 8)
    y, parts = ffn.ffn_q8(x, ex)

    f32 = lambda v: _round_binary(v, 24)  # noqa: E731
    f64 = lambda v: _round_binary(v, 53)  # noqa: E731
    gq = [[int(round(float(gate[n, k]) * 2)) for k in range(d)] for n in range(i_ff)]
    uq = [[int(round(float(up[n, k]) * 64)) for k in range(d)] for n in range(i_ff)]
    dq = [[int(round(float(down[j, n]) * 2 ** (7 + j % 3))) for n in range(i_ff)] for j in range(d)]
    assert ex.gate_q.tolist() == gq and ex.up_q.tolist() == uq and ex.down_q.tolist() == dq
    sw_gate, sw_up = Fr(1, 2), Fr(1, 64)
    sw_down = [Fr(1, 2 ** (7 + j % 3)) for j in range(d)]
    n_diff_fp32_arith = 0
    for t in range(2):
        xq, dx = _q8_0_exact([Fr(float(v)) for v in x[t]])
        assert parts["xq"][t].tolist() == xq and Fr(float(parts["xd"][t, 0])) == dx
        h32 = []
        for n in range(i_ff):
            dot_g = sum(a * b for a, b in zip(xq, gq[n]))         # integer group dots
            dot_u = sum(a * b for a, b in zip(xq, uq[n]))
            G = dx * sw_gate * dot_g                              # exact rationals
            U = dx * sw_up * dot_u
            assert G == 0 or G >= 38
            assert Fr(float(parts["g"][t, n])) == G and Fr(float(parts["u"][t, n])) == U
            h = f32(f64(G * U))                                   # silu(G) = G; fp64 product, then fp32
            h32.append(h)
            assert Fr(float(parts["h32"][t, n])) == h, (t, n)
            # a quantiser fed H computed in fp32 arithmetic instead would see another value here
            n_diff_fp32_arith += f32(f32(G) * f32(U)) != h
        hq, hd = _q8_0_exact(h32)
        assert parts["hq"][t].tolist() == hq
        assert parts["hd"].dtype == np.float32 and Fr(float(parts["hd"][t, 0])) == hd
        for j in range(d):
            dot_d = sum(a * b for a, b in zip(hq, dq[j]))         # down integer dots over H's codes
            assert Fr(float(y[t, j])) == hd * sw_down[j] * dot_d, (t, j)
        # the activation scale in the down projection's place would move Y
        assert any(dx * sw_down[j] * sum(a * b for a, b in zip(hq, dq[j])) != Fr(float(y[t, j])) for j in range(d))
    assert n_diff_fp32_arith > 0
    assert set(g3) >= {0} and parts["h32"].dtype == np.float32
