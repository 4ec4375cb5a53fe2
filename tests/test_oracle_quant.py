"""Pins for the oracle's quantisers (CPU only).

Each check ties the oracle to something other than itself: numbers printed on
the pages, hand-worked examples of the adopted definitions, bounds that hold
for any correct round-to-nearest quantiser, and brute force over integer
codes.
"""
import json
import os

import numpy as np
import pytest

from oracle import quant
import synth


def test_int8_g32_error_within_page_bound(golden_dir):
    # mtlm-7m-base, section Files: the int8 export in groups of 32 reports a largest absolute error of 1.7e-3.
    bound = json.load(open(os.path.join(golden_dir, "page_numbers.json")))["int8_g32_max_abs_error"]["value"]
    w = synth.expert_weight(synth.LAYERS["olmoe"], 0, "gate")
    q, s = quant.quantize_weights(w, 8)
    err = np.abs(quant.dequantize(q, s) - w.astype(np.float64)).max()
    assert err <= bound
    # and it is a round-to-nearest error, i.e. well below half a step of the largest scale
    assert err <= 0.5 * s.max() * (1 + 1e-5)


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_round_trip_half_step_and_amax(bits):
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((37, 96)) * rng.uniform(1e-4, 3, (37, 1))).astype(np.float32)
    w[3, 32:64] = 0.0                                   # an all-zero group
    q, s = quant.quantize_weights(w, bits)
    qmax = {8: 127, 4: 7, 2: 1}[bits]
    assert q.dtype == np.int8 and s.dtype == np.float32
    assert q.min() >= -qmax and q.max() <= qmax
    deq = quant.dequantize(q, s)
    step = np.repeat(s.astype(np.float64), 32, axis=1)
    assert np.all(np.abs(w - deq) <= 0.5 * step * (1 + 1e-5) + 1e-30)
    # the amax element of each non-zero group maps to +-qmax
    g = w.reshape(37, 3, 32)
    qa = q.reshape(37, 3, 32)
    for r in range(37):
        for j in range(3):
            if s[r, j] == 0:
                assert np.all(qa[r, j] == 0) and np.all(g[r, j] == 0)
                continue
            a = np.argmax(np.abs(g[r, j]))
            assert abs(int(qa[r, j, a])) == qmax
            assert np.sign(qa[r, j, a]) == np.sign(g[r, j, a])
    assert s[3, 1] == 0 and np.all(q[3, 32:64] == 0)


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_codes_are_nearest_integers_brute_force(bits):
    # brute force: for each element, no other code in range lands closer to w/s
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((4, 64)) * 0.02).astype(np.float32)
    q, s = quant.quantize_weights(w, bits)
    qmax = {8: 127, 4: 7, 2: 1}[bits]
    codes = np.arange(-qmax, qmax + 1)
    for r in range(4):
        for c in range(64):
            sc = float(s[r, c // 32])
            ratio = float(w[r, c]) / sc
            dist = np.abs(ratio - codes)
            best = dist.min()
            assert abs(ratio - int(q[r, c])) <= best + 1e-6


def test_scale_is_amax_over_qmax_in_fp32():
    w = np.zeros((1, 32), np.float32)
    w[0, 5] = -0.3
    w[0, 9] = 0.1
    q8, s8 = quant.quantize_weights(w, 8)
    q4, s4 = quant.quantize_weights(w, 4)
    assert s8[0, 0] == np.float32(np.float32(0.3) / np.float32(127))
    assert s4[0, 0] == np.float32(np.float32(0.3) / np.float32(7))
    assert q8[0, 5] == -127 and q4[0, 5] == -7
    # 0.1 / (0.3/127) = 42.33 -> 42 ; 0.1 / (0.3/7) = 2.33 -> 2
    assert q8[0, 9] == 42 and q4[0, 9] == 2


def test_int4_pack_matches_hand_worked_bytes(golden_dir):
    for line in open(os.path.join(golden_dir, "int4_nibbles.txt")):
        if line.startswith("#") or not line.strip():
            continue
        left, right = line.split("|")
        codes = np.array([int(v) for v in left.split()], dtype=np.int8)
        want = np.array([int(v, 16) for v in right.split()], dtype=np.uint8)
        assert np.array_equal(quant.pack_int4(codes), want)
        assert np.array_equal(quant.unpack_int4(want), codes)


def test_int4_unpack_equals_int8_container():
    # Show HN: Getting GLM-5.2 running on my slow computer, section What's implemented: the page checks
    # that packed codes unpack to exactly the int8 codes. Every byte value round-trips.
    allbytes = np.arange(256, dtype=np.uint8)
    codes = quant.unpack_int4(allbytes)
    assert codes.min() == -8 and codes.max() == 7
    assert np.array_equal(quant.pack_int4(codes), allbytes)
    w = (np.random.default_rng(3).standard_normal((16, 128)) * 0.02).astype(np.float32)
    q, _ = quant.quantize_weights(w, 4)
    assert np.array_equal(quant.unpack_int4(quant.pack_int4(q)), q)


def test_int2_pack_matches_hand_worked_bytes(golden_dir):
    for line in open(os.path.join(golden_dir, "int2_fields.txt")):
        if line.startswith("#") or not line.strip():
            continue
        left, right = line.split("|")
        codes = np.array([int(v) for v in left.split()], dtype=np.int8)
        want = np.array([int(v, 16) for v in right.split()], dtype=np.uint8)
        assert np.array_equal(quant.pack_int2(codes), want)
        assert np.array_equal(quant.unpack_int2(want), codes)


def test_int2_unpack_equals_int8_container():
    # every byte value round-trips; quantised codes survive packing unchanged
    allbytes = np.arange(256, dtype=np.uint8)
    codes = quant.unpack_int2(allbytes)
    assert codes.min() == -2 and codes.max() == 1
    assert np.array_equal(quant.pack_int2(codes), allbytes)
    w = (np.random.default_rng(3).standard_normal((16, 128)) * 0.02).astype(np.float32)
    for qz in (quant.quantize_weights, quant.quantize_rows):
        q, _ = qz(w, 2)
        assert set(np.unique(q).tolist()) <= {-1, 0, 1}
        assert np.array_equal(quant.unpack_int2(quant.pack_int2(q)), q)


def test_int2_hand_worked():
    # group [0.8, -0.8, 0.4, 0.41, -0.39, 0...]: s = amax / 1 = 0.8; 0.4 / 0.8 is
    # exactly 1/2 in fp32 -> 0 (half to even); 0.41 -> 1; -0.39 -> -0
    w = np.zeros((1, 32), np.float32)
    w[0, :5] = [0.8, -0.8, 0.4, 0.41, -0.39]
    q, s = quant.quantize_weights(w, 2)
    assert s[0, 0] == np.float32(0.8)
    assert q[0, :5].tolist() == [1, -1, 0, 1, 0] and np.all(q[0, 5:] == 0)
    # the mean absolute error of ternary codes on a Gaussian group is far from
    # zero but below half the scale
    g = (np.random.default_rng(9).standard_normal((64, 32)) * 0.02).astype(np.float32)
    qg, sg = quant.quantize_weights(g, 2)
    err = np.abs(quant.dequantize(qg, sg) - g)
    assert np.all(err <= 0.5 * np.repeat(sg, 32, axis=1) * (1 + 1e-6))


def test_q8_0_hand_worked_rounding(golden_dir):
    for line in open(os.path.join(golden_dir, "q8_0_rounding.txt")):
        if line.startswith("#") or not line.strip():
            continue
        xs, ds, qs = line.split("|")
        x = np.array([float(v) for v in xs.split()], dtype=np.float32)[None, :]
        want_q = np.array([int(v) for v in qs.split()], dtype=np.int8)[None, :]
        assert x.shape == (1, 32) and want_q.shape == (1, 32)
        q, d = quant.quantize_q8_0(x)
        assert d[0, 0] == np.float32(float(ds))
        assert np.array_equal(q, want_q)


def test_q8_0_bounds_and_zero_group():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((9, 64)).astype(np.float32)
    x[2, :32] = 0
    q, d = quant.quantize_q8_0(x)
    assert np.all(q[2, :32] == 0) and d[2, 0] == 0
    deq = quant.dequantize(q, d)
    step = np.repeat(d.astype(np.float64), 32, axis=1)
    assert np.all(np.abs(deq - x) <= 0.5 * step * (1 + 1e-5) + 1e-30)
    g = np.abs(x.reshape(9, 2, 32))
    a = g.argmax(axis=2)
    qq = np.abs(q.reshape(9, 2, 32))
    for r in range(9):
        for j in range(2):
            if d[r, j] > 0:
                assert qq[r, j, a[r, j]] == 127


def test_page_byte_accounting(golden_dir):
    # Show HN: Getting GLM-5.2 running on my slow computer, section The idea: ~19 MB per routed expert at int4;
    # section Got a better machine?: a cold token reads about 11.4 GB of experts.
    pn = json.load(open(os.path.join(golden_dir, "page_numbers.json")))
    glm = synth.LAYERS["glm"]
    payload = 0
    for shape in [(glm.d_ff, glm.d_model), (glm.d_ff, glm.d_model), (glm.d_model, glm.d_ff)]:
        payload += quant.pack_int4(np.zeros(shape, np.int8)).nbytes
    assert abs(payload / 1e6 - pn["glm_routed_expert_mb_int4"]["value"]) < 0.5
    cold = pn["glm_moe_layers"]["value"] * pn["glm_experts_per_token"]["value"] * payload
    assert abs(cold / 1e9 - pn["glm_cold_token_gb"]["value"]) / pn["glm_cold_token_gb"]["value"] < 0.02


# ---------------------------------------------------------------------------
# per-row scales (the GLM engine's kernels: one scale per row)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("bits", [8, 4, 2])
def test_per_row_on_one_group_rows_equals_group_32(bits):
    # a row of exactly 32 values is one group: both quantisers must agree
    w = (np.random.default_rng(11).standard_normal((40, 32)) * 0.02).astype(np.float32)
    qr, sr = quant.quantize_rows(w, bits)
    qg, sg = quant.quantize_weights(w, bits)
    assert np.array_equal(qr, qg) and np.array_equal(sr[:, 0], sg[:, 0])


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_per_row_round_trip_and_amax(bits):
    rng = np.random.default_rng(12)
    w = (rng.standard_normal((33, 256)) * 0.02).astype(np.float32)
    w[5] = 0.0                                                   # an all-zero row: scale 0, codes 0
    q, s = quant.quantize_rows(w, bits)
    qmax = {8: 127, 4: 7, 2: 1}[bits]
    assert s.shape == (33, 1) and s[5, 0] == 0 and np.all(q[5] == 0)
    err = np.abs(quant.dequantize(q, s) - w.astype(np.float64))
    assert np.all(err <= s.astype(np.float64) / 2 * (1 + 1e-6))  # nearest code
    rows = [r for r in range(33) if r != 5]
    am = np.argmax(np.abs(w[rows]), axis=1)
    assert np.all(np.abs(q[rows, am]) == qmax)                   # the row's amax maps to +-qmax
    # one scale per row: the error of a per-row code can exceed the group
    # quantiser's, never its own half step
    qg, sg = quant.quantize_weights(w, bits)
    assert np.abs(quant.dequantize(qg, sg) - w).max() <= np.abs(quant.dequantize(q, s) - w).max()


def test_per_row_hand_worked():
    # row [0.7, -0.35, 0.1, ...zeros]: amax 0.7, int4 scale 0.1: codes 7, -3.5 -> -4 (half to even), 1
    w = np.zeros((1, 64), np.float32)
    w[0, :3] = [0.7, -0.35, 0.1]
    q, s = quant.quantize_rows(w, 4)
    assert np.isclose(s[0, 0], np.float32(0.7) / np.float32(7))
    assert q[0, :3].tolist() == [7, -4, 1] and np.all(q[0, 3:] == 0)
    # int4 packing of per-row codes unpacks to the same int8 container
    assert np.array_equal(quant.unpack_int4(quant.pack_int4(q)), q)
