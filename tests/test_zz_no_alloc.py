"""The allocation-free layer entry point (include/moe.h,
moe_layer_forward_noalloc) through the C ABI, against moe_layer_forward
with a caller workspace: bitwise equal outputs on two calls in a row, the
second with a smaller batch (the shared scratch then still holds the first
call's contents), in both activation modes and on the tiled prefill path."""
import numpy as np
import pytest
import torch

import synth
import quantized_expert_ffn_amd as qe

from gpu_common import device_layer, need_gpu, say, t2n

pytestmark = pytest.mark.gpu


def _tiny(**over):
    from quantized_expert_ffn_amd import device_layer as dl
    shape = synth.variant(synth.LAYERS["tiny"], **over)
    return shape, dl.build(shape, "cuda")


def _both(dl, shape, T, act_mode):
    x = torch.from_numpy(synth.activations(shape, T)).cuda()
    am = qe.ACT_MODES[act_mode]
    ref = torch.empty((T, shape.d_model), dtype=torch.float32, device="cuda")
    ws = qe.workspace(T, shape.top_k, shape.n_experts, shape.d_model, shape.d_ff, am, dl.shared[0] is not None)
    qe.moe_layer_forward(x, dl.gate_w, dl.params, dl.routed[0], dl.shared[0], am, ref, ws)
    got = torch.full_like(ref, float("nan"))
    qe.moe_layer_forward_noalloc(x, dl.gate_w, dl.params, dl.routed[0], dl.shared[0], am, got)
    torch.cuda.synchronize()
    return t2n(got), t2n(ref)


@pytest.mark.parametrize("case", ["olmoe_f32", "glm_q8", "tiny_shared_q8_prefill", "tiny_f32"])
def test_noalloc_matches_workspace_entry_point(case):
    need_gpu()
    if case == "olmoe_f32":
        shape, dl, act, sizes = synth.LAYERS["olmoe"], device_layer("olmoe"), "f32", (16, 4)
    elif case == "glm_q8":
        shape, dl, act, sizes = synth.LAYERS["glm"], device_layer("glm"), "q8_0", (4, 1)
    elif case == "tiny_shared_q8_prefill":
        shape, dl = _tiny(shared_expert=True, router="noaux_tc", n_experts=16, n_group=4, topk_group=2, top_k=3,
                          has_bias=True, routed_scaling_factor=2.5)
        act, sizes = "q8_0", (600, 67)
    else:
        shape, dl = _tiny(shared_expert=True)
        act, sizes = "f32", (67, 16)
    for T in sizes:
        assert qe.moe_workspace_size(T, shape.top_k, shape.n_experts, shape.d_model, shape.d_ff,
                                     qe.ACT_MODES[act], shape.shared_expert) <= qe.MOE_NOALLOC_SCRATCH_BYTES
        say(f"[noalloc] {case}: T={T} {act}")
        got, ref = _both(dl, shape, T, act)
        assert np.all(np.isfinite(got))
        assert np.array_equal(got, ref), f"{case} T={T}: outputs differ (max {np.abs(got - ref).max():.3e})"


def test_noalloc_rejects_calls_beyond_its_scratch():
    need_gpu()
    shape, dl = _tiny(shared_expert=True)
    T = 60000          # the workspace of this call is larger than the scratch
    assert qe.moe_workspace_size(T, shape.top_k, shape.n_experts, shape.d_model, shape.d_ff, qe.MOE_ACT_F32,
                                 True) > qe.MOE_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, shape.d_model), dtype=torch.float32, device="cuda")
    out = torch.full_like(x, 7.0)
    with pytest.raises(qe.MoeError) as e:
        qe.moe_layer_forward_noalloc(x, dl.gate_w, dl.params, dl.routed[0], dl.shared[0], qe.MOE_ACT_F32, out)
    assert e.value.status == qe._lib.MOE_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)       # nothing was enqueued
