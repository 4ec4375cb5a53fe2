"""The C ABI on the host, without a GPU: the library loads, exports every
entry point include/moe.h declares, and rejects bad arguments with the right
status before anything is enqueued (no call here reaches a kernel)."""
import ctypes
import os
import re

import numpy as np
import pytest

from conftest import ROOT

import quantized_expert_ffn_amd as qe
from quantized_expert_ffn_amd import _lib

HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
FAKE = 0x10000          # an aligned, never dereferenced address


def declared_functions():
    text = "\n".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(moe_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libmoe.so is not built: run `python -m quantized_expert_ffn_amd.build`")
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"
    assert set(names) == set(_lib.exported_names()), "binding and header disagree"


def test_status_strings(lib):
    assert qe.moe_status_string(0) == "MOE_OK"
    for st in (INVALID, UNSUPPORTED, WORKSPACE, -4):
        assert qe.moe_status_string(st).startswith("MOE_ERR_")


def test_workspace_size_rules(lib):
    ws = qe.moe_workspace_size
    assert ws(16, 2, 8, 64, 128, 0, 0) > 0
    assert ws(16, 2, 8, 64, 128, 1, 1) > ws(16, 2, 8, 64, 128, 1, 0)
    assert ws(2048, 8, 64, 2048, 1024, 1, 0) > ws(16, 8, 64, 2048, 1024, 1, 0)
    assert ws(0, 2, 8, 64, 128, 0, 0) > 0                     # T = 0 still valid
    assert ws(16, 9, 8, 64, 128, 0, 0) == 0                   # k > E
    assert ws(16, 2, 8, 65, 128, 0, 0) == 0                   # d % 32
    assert ws(16, 2, 8, 64, 128, 7, 0) == 0                   # unknown act_mode
    assert ws(-1, 2, 8, 64, 128, 0, 0) == 0


def _params(**kw):
    p = _lib.RouterParams()
    p.n_experts, p.top_k, p.mode, p.renormalize = 8, 2, 0, 1
    p.n_group, p.topk_group, p.routed_scaling_factor, p.score_bias = 1, 1, 1.0, None
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def _experts(**kw):
    e = _lib.Experts()
    e.n_experts, e.d_model, e.d_ff, e.format = 8, 64, 128, 0
    for f in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s"):
        setattr(e, f, FAKE)
    for k, v in kw.items():
        setattr(e, k, v)
    return e


def _fwd(lib, T=4, params=None, routed=None, shared=None, act=0, ws_bytes=1 << 30, x=FAKE, out=FAKE, ws=FAKE):
    params = params or _params()
    routed = routed or _experts()
    return lib.moe_layer_forward(x, T, FAKE, ctypes.byref(params), ctypes.byref(routed),
                                 ctypes.byref(shared) if shared else None, act, out, ws, ws_bytes, None)


def test_layer_forward_validation(lib):
    assert _fwd(lib, T=0) == OK                                   # no-op, nothing enqueued
    assert _fwd(lib, T=-1) == INVALID
    assert _fwd(lib, x=None) == INVALID
    assert _fwd(lib, act=5) == INVALID
    assert _fwd(lib, params=_params(top_k=9)) == INVALID          # k > E
    assert _fwd(lib, params=_params(top_k=0)) == INVALID
    assert _fwd(lib, params=_params(n_experts=7)) == INVALID      # router E != experts E
    assert _fwd(lib, params=_params(mode=3)) == INVALID
    assert _fwd(lib, routed=_experts(d_model=65)) == UNSUPPORTED  # d % 32
    assert _fwd(lib, routed=_experts(d_model=96)) == UNSUPPORTED  # d % 64 (pairs of groups)
    assert _fwd(lib, routed=_experts(d_ff=100)) == UNSUPPORTED    # I % 32
    assert _fwd(lib, routed=_experts(format=9)) == INVALID
    assert _fwd(lib, routed=_experts(format=6)) == INVALID
    assert _fwd(lib, routed=_experts(format=4)) == UNSUPPORTED   # int2 needs d % 128
    assert _fwd(lib, T=0, routed=_experts(format=4, d_model=128, d_ff=256)) == OK
    assert _fwd(lib, T=0, routed=_experts(format=3)) == OK        # the per-row formats are valid
    assert _fwd(lib, shared=_experts(n_experts=1, format=2)) == UNSUPPORTED   # shared format != routed
    assert _fwd(lib, params=_params(shared_gate=FAKE + 4), shared=_experts(n_experts=1)) == INVALID  # misaligned
    assert _fwd(lib, routed=_experts(up_s=None)) == INVALID
    assert _fwd(lib, routed=_experts(gate_q=FAKE + 4)) == INVALID  # misaligned codes
    assert _fwd(lib, shared=_experts(n_experts=2)) == INVALID
    assert _fwd(lib, shared=_experts(n_experts=1, d_ff=96)) == UNSUPPORTED
    assert _fwd(lib, ws_bytes=16) == WORKSPACE
    assert _fwd(lib, ws=None) == WORKSPACE
    assert "workspace" in qe.moe_last_error_detail()


def test_noaux_tc_validation(lib):
    E = 16
    base = dict(n_experts=E, mode=1, n_group=4, topk_group=2, top_k=3, routed_scaling_factor=2.5)
    r = _experts(n_experts=E)

    def run(**kw):
        d = dict(base)
        d.update(kw)
        return _fwd(lib, T=0, params=_params(**d), routed=r)

    assert run() == OK
    assert run(n_group=5) == INVALID            # E % n_group
    assert run(topk_group=5) == INVALID         # topk_group > n_group
    assert run(top_k=9) == INVALID              # more than the 2 kept groups of 4 hold
    assert run(n_group=0) == INVALID
    assert run(routed_scaling_factor=float("inf")) == INVALID


def test_route_dispatch_combine_validation(lib):
    p = _params()
    assert lib.moe_route(FAKE, 0, 64, FAKE, ctypes.byref(p), FAKE, FAKE, FAKE, 0, None) == OK
    assert lib.moe_route(FAKE, 4, 64, FAKE, None, FAKE, FAKE, FAKE, 1 << 20, None) == INVALID
    assert lib.moe_route(FAKE, 4, 64, FAKE, ctypes.byref(p), FAKE, FAKE, FAKE, 8, None) == WORKSPACE
    big = _params(n_experts=2048, top_k=2)
    assert lib.moe_route(FAKE, 4, 64, FAKE, ctypes.byref(big), FAKE, FAKE, FAKE, 1 << 30, None) == UNSUPPORTED
    assert lib.moe_dispatch(FAKE, 4, 3, 2, FAKE, FAKE, FAKE, FAKE, None, 0, None) == INVALID   # k > E
    assert lib.moe_dispatch(FAKE, 4, 2, 2000, FAKE, FAKE, FAKE, FAKE, None, 0, None) == UNSUPPORTED
    assert lib.moe_dispatch(FAKE, 4, 2, 8, None, FAKE, FAKE, FAKE, None, 0, None) == INVALID
    assert lib.moe_combine(FAKE, FAKE, FAKE, None, 0, 2, 64, FAKE, None) == OK
    assert lib.moe_combine(FAKE, FAKE, FAKE, None, 4, 2, 66, FAKE, None) == UNSUPPORTED
    assert lib.moe_combine(None, FAKE, FAKE, None, 4, 2, 64, FAKE, None) == INVALID
    assert lib.moe_quantize_weights(FAKE, 32, 48, 32, 0, FAKE, FAKE, None) == UNSUPPORTED   # cols % 32
    assert lib.moe_quantize_weights(FAKE, 32, 96, 32, 1, FAKE, FAKE, None) == UNSUPPORTED   # cols % 64
    assert lib.moe_quantize_weights(FAKE, 40, 64, 40, 0, FAKE, FAKE, None) == UNSUPPORTED   # matrix rows % 32
    assert lib.moe_quantize_weights(FAKE, 96, 64, 64, 0, FAKE, FAKE, None) == INVALID       # not whole matrices
    assert lib.moe_quantize_weights(FAKE, 64, 64, 0, 0, FAKE, FAKE, None) == INVALID
    assert lib.moe_quantize_weights(FAKE, 32, 64, 32, 6, FAKE, FAKE, None) == INVALID      # unknown format
    assert lib.moe_quantize_weights(FAKE, 32, 64, 32, 4, FAKE, FAKE, None) == UNSUPPORTED  # int2: cols % 128
    assert lib.moe_quantize_weights(FAKE, 0, 128, 32, 5, FAKE, FAKE, None) == OK
    assert lib.moe_quantize_weights(FAKE, 32, 64, 32, -1, FAKE, FAKE, None) == INVALID
    assert lib.moe_quantize_weights(FAKE, 40, 64, 40, 3, FAKE, FAKE, None) == UNSUPPORTED  # per-row: same layout
    assert lib.moe_quantize_weights(FAKE, 0, 64, 32, 1, FAKE, FAKE, None) == OK
    assert lib.moe_quantize_weights(FAKE, 0, 64, 32, 3, FAKE, FAKE, None) == OK
    assert lib.moe_quantize_q8_0(FAKE, 4, 40, FAKE, FAKE, None) == UNSUPPORTED
    e = _experts()
    assert lib.moe_expert_ffn(FAKE, 4, 9, ctypes.byref(e), FAKE, FAKE, FAKE, 0, FAKE, FAKE, 1 << 30, None) == INVALID
    assert lib.moe_expert_ffn(FAKE, 4, 2, ctypes.byref(e), FAKE, FAKE, FAKE, 0, FAKE, FAKE, 64, None) == WORKSPACE
    assert lib.moe_expert_ffn(FAKE, 0, 2, ctypes.byref(e), FAKE, FAKE, FAKE, 1, FAKE, FAKE, 0, None) == OK
    assert lib.moe_debug_q8_expert_ffn(FAKE, 4, 2, ctypes.byref(e), FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE,
                                       FAKE, FAKE, 1 << 30, None) == INVALID


def test_accounting_matches_page_figures():
    from quantized_expert_ffn_amd import accounting as acc
    # ~19 MB per GLM routed expert at int4 is the payload; the scales add a quarter
    glm = (6144, 2048)
    payload = 3 * glm[0] * glm[1] // 2
    assert abs(payload / 1e6 - 19) < 0.5
    assert acc.expert_bytes(*glm, "int4") == payload + 3 * glm[0] * glm[1] // 32 * 4
    assert acc.useful_ops([2, 0, 1], 3, 64, 128, False) == 2 * 3 * 3 * 64 * 128
    # per-row scales: one float per matrix row
    assert acc.expert_bytes(*glm, "int4_row") == payload + (2 * glm[1] + glm[0]) * 4
    assert acc.expert_bytes(*glm, "int8_row") == 2 * payload + (2 * glm[1] + glm[0]) * 4
    assert acc.expert_bytes(*glm, "int2") == payload // 2 + 3 * glm[0] * glm[1] // 32 * 4
    assert acc.expert_bytes(*glm, "int2_row") == payload // 2 + (2 * glm[1] + glm[0]) * 4


@pytest.mark.parametrize("fmt", ["int8", "int4", "int2"])
def test_untile_helpers_invert_the_documented_layout(fmt):
    """The GPU tests read library weights back through untile_*; check those
    against the layout formulas of include/moe.h, written out element by element."""
    from gpu_common import untile_codes, untile_scales
    rng = np.random.default_rng(3)
    N, K = 96, 256
    G, P, NT = K // 32, K // 64, N // 32
    qmax = {"int8": 127, "int4": 7, "int2": 1}[fmt]
    codes = rng.integers(-qmax, qmax + 1, (N, K))
    scales = rng.standard_normal((N, G)).astype(np.float32)
    sflat = np.zeros(N * G, np.float32)
    if fmt == "int8":
        qflat = np.zeros(N * K, np.int8)
    elif fmt == "int4":
        qflat = np.zeros(N * K // 8, np.uint32)
    else:
        qflat = np.zeros(N * K // 8, np.uint16)
    for row in range(N):
        t, r = divmod(row, 32)
        nl, half = r % 16, r // 16
        for g in range(G):
            sflat[(t * P + g // 2) * 64 + 4 * nl + 2 * (g % 2) + half] = scales[row, g]
            for h in range(4):
                lane = nl + 16 * h
                ks = range(32 * g + 8 * h, 32 * g + 8 * h + 8)
                if fmt == "int8":
                    for k in ks:
                        qflat[((g * NT + t) * 64 + lane) * 16 + 8 * half + k % 8] = codes[row, k]
                elif fmt == "int4":
                    word = 0
                    for k in ks:
                        word |= (int(codes[row, k]) & 0xF) << (4 * (k % 8))
                    qflat[((g // 2 * NT + t) * 64 + lane) * 4 + 2 * (g % 2) + half] = word
                else:
                    word = 0
                    for k in ks:
                        word |= (int(codes[row, k]) & 0x3) << (2 * (k % 8))
                    qflat[((g // 4 * NT + t) * 64 + lane) * 8 + 2 * (g % 4) + half] = word
    from oracle import quant as oquant
    stored = oquant.pack_codes(codes.astype(np.int8), {"int8": 8, "int4": 4, "int2": 2}[fmt])
    assert np.array_equal(untile_codes(qflat, N, K, fmt), stored)
    assert np.array_equal(untile_scales(sflat, N, K), scales)


def test_router_top_p_validation(lib):
    for bad in (-0.1, float("nan")):
        p = _params(top_p=bad)
        assert lib.moe_route(FAKE, 4, 64, FAKE, ctypes.byref(p), FAKE, FAKE, FAKE, 1 << 30, None) == INVALID
        assert _fwd(lib, params=p) == INVALID
    # a struct built field by field leaves top_p at 0: every slot kept
    assert _params().top_p == 0.0


def test_block_forward_validation(lib):
    p = _params()
    e = _experts()
    def blk(eps=1e-6, norm=FAKE, x=FAKE):
        return lib.moe_block_forward(x, 4, norm, ctypes.c_float(eps), FAKE, ctypes.byref(p), ctypes.byref(e), None, 0,
                                     FAKE, FAKE, 1 << 30, None, None)
    assert blk(eps=-1.0) == INVALID
    assert blk(eps=float("nan")) == INVALID
    assert blk(eps=float("inf")) == INVALID
    assert blk(x=None) == INVALID
    assert blk(norm=FAKE + 4) == INVALID        # norm_w not 16-byte aligned
    assert lib.moe_block_forward(FAKE, 0, None, ctypes.c_float(0.0), FAKE, ctypes.byref(p), ctypes.byref(e), None, 0,
                                 FAKE, FAKE, 0, None, None) == OK      # T = 0


def test_workspace_sections_inside_the_workspace(lib):
    """The test hook's section offsets: 256-byte aligned, in bounds, the
    routing sections large enough and disjoint; H's sections only in Q8_0
    mode; sizes the workspace rejects are rejected too."""
    for act, shared in ((0, False), (1, False), (1, True)):
        T, k, E, d, I = 16, 2, 8, 64, 128
        size = qe.moe_workspace_size(T, k, E, d, I, act, shared)
        sec = qe.moe_debug_workspace_sections(T, k, E, d, I, act, shared)
        need = {"topk_idx": T * k * 4, "topk_w": T * k * 4, "counts": E * 4, "offsets": (E + 1) * 4,
                "perm": T * k * 4, "inv_perm": T * k * 4}
        if act == 1:
            R = T * k + (T if shared else 0)
            need.update(h_codes=R * I * 2, h_scales=R * (I // 32) * 4)
        else:
            assert sec["h_codes"] == -1 and sec["h_scales"] == -1
        spans = sorted((sec[n], sec[n] + b) for n, b in need.items())
        for (a0, a1), (b0, _) in zip(spans, spans[1:]):
            assert a1 <= b0
        assert all(o % 256 == 0 for o, _ in spans) and spans[-1][1] <= size
    with pytest.raises(qe.MoeError) as e:
        qe.moe_debug_workspace_sections(16, 9, 8, 64, 128, 0, False)        # k > E
    assert e.value.status == INVALID


def test_calib_stream_read_rejects_bad_arguments(lib):
    f = lib.moe_calib_stream_read
    assert f(None, 1 << 20, FAKE, 64, None) == INVALID
    assert f(FAKE, 1 << 20, None, 64, None) == INVALID
    assert f(FAKE + 4, 1 << 20, FAKE, 64, None) == INVALID            # unaligned
    assert f(FAKE, 1000, FAKE, 64, None) == INVALID                   # not a multiple of 16
    assert f(FAKE, 0, FAKE, 64, None) == INVALID
    assert f(FAKE, 1 << 20, FAKE, 0, None) == INVALID


def test_calib_prefill_mix_rejects_bad_arguments(lib):
    f = lib.moe_calib_prefill_mix
    assert f(16, 8, None, None, None) == INVALID
    assert f(0, 8, FAKE, None, None) == INVALID
    assert f(16, 7, FAKE, None, None) == INVALID                     # odd stage count
    assert f(16, 0, FAKE, None, None) == INVALID


def test_noalloc_entry_point_checks_before_any_gpu_call(lib):
    """The allocation-free layer entry point: null arguments and calls whose
    workspace would exceed its scratch are rejected on the host, before any
    HIP call (no GPU here)."""
    p, r = _params(), _experts()
    f = lib.moe_layer_forward_noalloc
    assert f(FAKE, 4, FAKE, None, ctypes.byref(r), None, 0, FAKE, None) == INVALID
    assert f(FAKE, 4, FAKE, ctypes.byref(p), None, None, 0, FAKE, None) == INVALID
    assert f(FAKE, -1, FAKE, ctypes.byref(p), ctypes.byref(r), None, 0, FAKE, None) == INVALID
    big_t = 200_000           # this layer's workspace at this T is far beyond the scratch
    assert qe.moe_workspace_size(big_t, 2, 8, 64, 128, 0, 0) > qe.MOE_NOALLOC_SCRATCH_BYTES
    assert f(FAKE, big_t, FAKE, ctypes.byref(p), ctypes.byref(r), None, 0, FAKE, None) == UNSUPPORTED
    assert "scratch" in qe.moe_last_error_detail()
    # sizes the layer itself rejects still name the bad argument
    bad = _experts(d_model=96)
    assert f(FAKE, 4, FAKE, ctypes.byref(p), ctypes.byref(bad), None, 0, FAKE, None) == UNSUPPORTED
    assert f(FAKE, 4, FAKE, ctypes.byref(_params(top_k=9)), ctypes.byref(r), None, 0, FAKE, None) == INVALID


def test_host_abi_layer_under_address_sanitizer(tmp_path):
    """The ABI layer's host code built with AddressSanitizer (its device code
    and the kernels unchanged) and driven through every host-side check of
    tests/abi_host_check.cpp without a GPU: the validation tables, a sweep of
    workspace sizes and sections from 1 to 65536 tokens and 1 to 1024
    experts, the error details. Any out-of-bounds or use-after-free access in
    that code ends the run with a sanitizer report."""
    import subprocess
    from quantized_expert_ffn_amd import build as qbuild
    exe = qbuild.build_host_check(str(tmp_path), os.path.join(ROOT, "tests", "abi_host_check.cpp"))
    assert b"__asan_report_load" in open(exe, "rb").read(), "the check was not built with the sanitizer"
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert "AddressSanitizer" not in res.stderr, res.stderr[-4000:]
    assert res.returncode == 0, res.stdout + res.stderr[-4000:]
    assert "passed" in res.stdout


def test_binding_rejects_mismatched_shapes():
    """The binding checks every tensor against the sizes it passes to the
    library before any pointer is taken: a tensor of the wrong shape is a
    ValueError on the host, never a kernel reading or writing past its end
    (CPU tensors here; the checks come before the device check)."""
    import torch
    E, d, I, T, k = 8, 64, 128, 4, 2
    routed = _lib.QuantExperts.empty(E, d, I, "int8", device="cpu")
    p = _lib.router_params(E, k)
    x = torch.zeros((T, d))
    gate_w = torch.zeros((E, d))
    out = torch.zeros((T, d))
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    for bad in (dict(x=torch.zeros((T, d + 32))), dict(gate_w=torch.zeros((E - 1, d))),
                dict(out=torch.zeros((T - 1, d))), dict(x=torch.zeros(T * d))):
        a = dict(x=x, gate_w=gate_w, out=out)
        a.update(bad)
        with pytest.raises(ValueError):
            qe.moe_layer_forward(a["x"], a["gate_w"], p, routed, None, 0, a["out"], ws)
        with pytest.raises(ValueError):
            qe.moe_layer_forward_noalloc(a["x"], a["gate_w"], p, routed, None, 0, a["out"])
    with pytest.raises(ValueError):
        qe.moe_block_forward(x, torch.zeros(d + 1), 1e-5, gate_w, p, routed, None, 0, out, ws)
    with pytest.raises(ValueError):   # codes of a stack that does not match its scales
        _lib.QuantExperts("int8", routed.gate_q[:, :-32], routed.gate_s, routed.up_q, routed.up_s, routed.down_q,
                          routed.down_s)
    with pytest.raises(ValueError):
        qe.moe_combine(torch.zeros((T * k, d)), torch.zeros((T, k)), torch.zeros(T * k - 1, dtype=torch.int32),
                       None, torch.zeros((T, d)))
    with pytest.raises(ValueError):
        qe.moe_calib_prefill_mix(4, 2, torch.zeros(4 * 512 - 1))
