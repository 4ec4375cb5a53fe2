"""Pins for the oracle's routers and dispatch (CPU only).

Exhaustive search over expert and group subsets on tiny layers, exact-tie
fixtures, closed-form weight sums, and special cases that reduce to a plainer
router.
"""
import itertools

import numpy as np
import pytest

from oracle import dispatch, router
import synth


def _beats(ka, ia, kb, ib):
    """(key a, id a) is ranked before (key b, id b) under the tie rule."""
    return ka > kb or (ka == kb and ia < ib)


def _exhaustive_topk(keys, k):
    """The unique subset whose every member beats every non-member."""
    n = len(keys)
    found = []
    for sub in itertools.combinations(range(n), k):
        rest = [j for j in range(n) if j not in sub]
        if all(_beats(keys[a], a, keys[b], b) for a in sub for b in rest):
            found.append(sub)
    assert len(found) == 1
    sub = list(found[0])
    # order inside the subset: descending key, ties to lower id
    sub.sort(key=lambda e: (-keys[e], e))
    return sub


@pytest.mark.parametrize("k", [1, 2, 3, 8])
def test_softmax_topk_exhaustive_tiny(k):
    lay = synth.LAYERS["tiny"]
    x = synth.activations(lay, 16)
    wg = synth.gate_weight(lay)
    idx, w, l = router.route_softmax(x, wg, k, renormalize=False)
    for t in range(16):
        assert list(idx[t]) == _exhaustive_topk(list(l[t]), k)


def test_softmax_weights_closed_forms():
    lay = synth.LAYERS["tiny"]
    x = synth.activations(lay, 16)
    wg = synth.gate_weight(lay)
    _, w_all, l = router.route_softmax(x, wg, 8, renormalize=False)
    # k = E without renormalisation: the full softmax, which sums to 1
    assert np.allclose(w_all.sum(axis=1), 1.0, atol=1e-12)
    idx, w, _ = router.route_softmax(x, wg, 2, renormalize=False)
    assert np.all(w.sum(axis=1) < 1.0)
    # probability ratios are exp of logit differences
    r = w[:, 0] / w[:, 1]
    d = np.take_along_axis(l, idx, 1)
    assert np.allclose(r, np.exp(d[:, 0] - d[:, 1]), rtol=1e-12)
    idx2, w2, _ = router.route_softmax(x, wg, 2, renormalize=True)
    assert np.array_equal(idx, idx2)
    assert np.allclose(w2.sum(axis=1), 1.0, atol=1e-12)
    assert np.allclose(w2, w / w.sum(axis=1, keepdims=True), rtol=1e-12)


def test_exact_ties_go_to_lower_id():
    x = np.random.default_rng(0).standard_normal((5, 64)).astype(np.float32)
    wg = np.zeros((8, 64), np.float32)
    idx, w, _ = router.route_softmax(x, wg, 3, renormalize=False)
    assert np.all(idx == [0, 1, 2])
    assert np.allclose(w, 1 / 8)
    idx, w, _ = router.route_softmax(x, wg, 3, renormalize=True)
    assert np.allclose(w, 1 / 3)
    # duplicated rows: the lower id of the pair wins the tie
    wg = (np.random.default_rng(1).standard_normal((8, 64)) * 0.02).astype(np.float32)
    wg[6] = wg[2] = x[0] * 0.5       # both strongly aligned with token 0
    idx, _, _ = router.route_softmax(x[:1], wg, 1, renormalize=False)
    assert idx[0, 0] == 2
    idx, _, _ = router.route_softmax(x[:1], wg, 2, renormalize=False)
    assert list(idx[0]) == [2, 6]


def _noaux_brute(l, b, k, n_group, topk_group, rsf):
    s = 1 / (1 + np.exp(-l))
    c = s + b
    e = len(l)
    gs = e // n_group
    gscore = [sorted(c[g * gs:(g + 1) * gs])[::-1][:2] for g in range(n_group)]
    gscore = [sum(v) for v in gscore]
    kept = _exhaustive_topk(gscore, topk_group)
    elig = [j for j in range(e) if j // gs in kept]
    sub = _exhaustive_topk([c[j] for j in elig], k)
    idx = [elig[j] for j in sub]
    w = np.array([s[j] for j in idx])
    return idx, w / w.sum() * rsf


@pytest.mark.parametrize("e,n_group,topk_group,k", [(8, 4, 2, 2), (16, 4, 2, 3), (16, 8, 3, 4), (16, 2, 1, 8)])
def test_noaux_tc_exhaustive(e, n_group, topk_group, k):
    rng = np.random.default_rng(e * 100 + k)
    x = rng.standard_normal((12, 64)).astype(np.float32)
    wg = (rng.standard_normal((e, 64)) * 0.3).astype(np.float32)
    b = (rng.standard_normal(e) * 0.1).astype(np.float32)
    idx, w, l = router.route_noaux_tc(x, wg, b, k, n_group, topk_group, 2.5)
    for t in range(12):
        bi, bw = _noaux_brute(l[t], b.astype(np.float64), k, n_group, topk_group, 2.5)
        assert list(idx[t]) == bi
        assert np.allclose(w[t], bw, rtol=1e-12)
    assert np.allclose(w.sum(axis=1), 2.5, rtol=1e-12)


def test_noaux_tc_reduces_to_sigmoid_topk():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((10, 32)).astype(np.float32)
    wg = (rng.standard_normal((16, 32)) * 0.3).astype(np.float32)
    idx, w, l = router.route_noaux_tc(x, wg, None, 4, 1, 1, 1.0)
    idx_s, _, _ = router.route_softmax(x, wg, 4, renormalize=False)
    assert np.array_equal(idx, idx_s)       # sigmoid is monotone
    s = 1 / (1 + np.exp(-np.take_along_axis(l, idx, 1)))
    assert np.allclose(w, s / s.sum(axis=1, keepdims=True), rtol=1e-12)


def test_noaux_tc_group_score_is_top2_sum_not_max():
    # group 0 = experts 0..3, group 1 = experts 4..7 (n_group 2, keep 1)
    # group 0 has the single best expert; group 1 has the better top-2 sum
    s = np.array([0.95, 0.05, 0.05, 0.05, 0.80, 0.78, 0.05, 0.05])
    l = np.log(s / (1 - s))
    wg = np.zeros((8, 8), np.float32)
    wg[:, 0] = l.astype(np.float32)                       # logit_e = l_e
    x = np.zeros((1, 8), np.float32)
    x[0, 0] = 1.0
    idx, w, _ = router.route_noaux_tc(x, wg, None, 2, 2, 1, 1.0)
    assert sorted(idx[0]) == [4, 5]


def test_noaux_tc_bias_selects_but_does_not_weigh():
    x = np.zeros((1, 8), np.float32)
    x[0, 0] = 1.0
    wg = np.zeros((8, 8), np.float32)
    wg[:, 0] = np.array([2.0, 1.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0], np.float32)
    b = np.zeros(8, np.float32)
    b[7] = 0.9                                            # lifts expert 7 above expert 1
    idx, w, _ = router.route_noaux_tc(x, wg, b, 2, 1, 1, 1.0)
    assert list(idx[0]) == [7, 0]         # c7 = 0.5 + 0.9 > c0 = sigmoid(2)
    s0, s7 = 1 / (1 + np.exp(-2.0)), 0.5
    want = {0: s0 / (s0 + s7), 7: s7 / (s0 + s7)}
    for j in range(2):
        assert np.isclose(w[0, j], want[idx[0, j]], rtol=1e-12)


def test_dispatch_invariants_and_brute_force():
    rng = np.random.default_rng(9)
    for t, k, e in [(16, 2, 8), (1, 8, 64), (33, 3, 5), (0, 2, 4)]:
        idx = np.stack([rng.choice(e, size=k, replace=False) for _ in range(t)]) if t else np.zeros((0, k), int)
        counts, offsets, perm, inv = dispatch.dispatch(idx, e)
        flat = idx.reshape(-1)
        assert counts.sum() == t * k and offsets[0] == 0 and offsets[-1] == t * k
        assert sorted(perm.tolist()) == list(range(t * k))
        assert np.array_equal(inv[perm], np.arange(t * k))
        want = [f for ex in range(e) for f in range(t * k) if flat[f] == ex]
        assert perm.tolist() == want
        for ex in range(e):
            seg = perm[offsets[ex]:offsets[ex + 1]]
            assert np.all(flat[seg] == ex) and np.all(np.diff(seg) > 0)


# ---------------------------------------------------------------------------
# adaptive expert top-p (the reading: shortest prefix in selection order whose
# mass reaches top_p of the selected total, kept weights rescaled to that total)
# ---------------------------------------------------------------------------
def test_top_p_off_keeps_everything():
    rng = np.random.default_rng(5)
    idx = rng.integers(0, 64, size=(7, 8)).astype(np.int32)
    w = rng.random((7, 8))
    for p in (0.0, 1.0, 1.5):
        i2, w2 = router.apply_top_p(idx, w, p)
        assert np.array_equal(i2, idx) and np.array_equal(w2, w)


def test_top_p_hand_worked_example():
    # weights 0.5, 0.3, 0.2 (sum 1), top_p 0.7: the mass before the slots is
    # 0, 0.5, 0.8, so slots 0 and 1 stay (0.5 < 0.7) and slot 2 goes; the kept
    # 0.8 is rescaled to 1: 0.625, 0.375
    idx = np.array([[11, 4, 9]], dtype=np.int32)
    w = np.array([[0.5, 0.3, 0.2]])
    i2, w2 = router.apply_top_p(idx, w, 0.7)
    assert i2.tolist() == [[11, 4, -1]]
    assert np.allclose(w2, [[0.625, 0.375, 0.0]], rtol=0, atol=1e-15)


@pytest.mark.parametrize("k,p", [(8, 0.7), (8, 0.3), (10, 0.55), (4, 0.9), (6, 0.01)])
def test_top_p_equal_weights_keep_ceil_pk(k, p):
    # equal weights: the mass before slot j is j/k of the total, so slot j
    # stays iff j < p*k, which keeps ceil(p*k) slots (p*k not an integer)
    w = np.full((3, k), 2.5 / k)
    idx = np.tile(np.arange(k, dtype=np.int32), (3, 1))
    i2, w2 = router.apply_top_p(idx, w, p)
    n_keep = int(np.ceil(p * k))
    assert (i2 >= 0).sum(axis=1).tolist() == [n_keep] * 3
    assert np.allclose(w2[:, :n_keep], 2.5 / n_keep) and np.all(w2[:, n_keep:] == 0)


def test_top_p_dominant_first_slot_and_invariants():
    rng = np.random.default_rng(9)
    w = rng.random((200, 8)) + 0.01
    w[0] = [0.9, 0.05, 0.02, 0.01, 0.01, 0.005, 0.003, 0.002]      # slot 0 alone reaches 0.7
    w = -np.sort(-w, axis=1) * 2.5 / w.sum(axis=1, keepdims=True)  # selection order, sum 2.5
    idx = np.tile(np.arange(8, dtype=np.int32), (200, 1))
    i2, w2 = router.apply_top_p(idx, w, 0.7)
    assert i2[0].tolist() == [0, -1, -1, -1, -1, -1, -1, -1] and np.isclose(w2[0, 0], 2.5)
    assert np.allclose(w2.sum(axis=1), 2.5)                        # total mass kept
    kept = i2 >= 0
    assert np.all(kept[:, 0])                                      # at least one slot
    assert np.all(kept[:, :-1] >= kept[:, 1:])                     # dropped slots form a suffix
    # a larger top_p never keeps fewer slots
    for p_lo, p_hi in ((0.3, 0.5), (0.5, 0.7), (0.7, 0.95)):
        a, _ = router.apply_top_p(idx, w, p_lo)
        b, _ = router.apply_top_p(idx, w, p_hi)
        assert np.all((a >= 0).sum(axis=1) <= (b >= 0).sum(axis=1))


def test_dispatch_skips_dropped_slots():
    idx = np.array([[3, 1, -1], [1, -1, -1], [0, 3, 2]], dtype=np.int32)
    counts, offsets, perm, inv = dispatch.dispatch(idx, 4)
    assert counts.tolist() == [1, 2, 1, 2]
    assert offsets.tolist() == [0, 1, 3, 4, 6]
    # kept flat assignments sorted by (expert, f): e0: 6; e1: 1, 3; e2: 8; e3: 0, 7
    assert perm.tolist() == [6, 1, 3, 8, 0, 7, -1, -1, -1]
    assert inv.tolist() == [4, 1, -1, 2, -1, -1, 0, 5, 3]
    with pytest.raises(ValueError):
        dispatch.dispatch(np.array([[4, -2]]), 4)
