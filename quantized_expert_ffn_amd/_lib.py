"""ctypes binding of libmoe (include/moe.h): argument marshalling only.

Every function here has the name of the C entry point it calls, takes torch
tensors that already live in GPU memory, passes their device pointers and the
current HIP stream, and raises MoeError when the library returns an error.
No arithmetic of the layer happens in Python; there is no CPU fallback: if the
built library is missing, loading fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4

MOE_ROUTER_SOFTMAX_TOPK = 0
MOE_ROUTER_SIGMOID_NOAUX_TC = 1
MOE_W_INT8_G32 = 0
MOE_W_INT4_G32 = 1
MOE_W_INT8_ROW = 2
MOE_W_INT4_ROW = 3
MOE_W_INT2_G32 = 4
MOE_W_INT2_ROW = 5
MOE_ACT_F32 = 0
MOE_ACT_Q8_0 = 1

STAGES = ("route", "dispatch", "quant_x", "gateup", "down", "combine")
# workspace sections the test hook moe_debug_workspace_sections locates
WS_SECTIONS = ("topk_idx", "topk_w", "counts", "offsets", "perm", "inv_perm", "h_codes", "h_scales")
MOE_STAGE_COUNT = len(STAGES)

FORMATS = {"int8": MOE_W_INT8_G32, "int4": MOE_W_INT4_G32, "int2": MOE_W_INT2_G32,
           "int8_row": MOE_W_INT8_ROW, "int4_row": MOE_W_INT4_ROW, "int2_row": MOE_W_INT2_ROW}
ACT_MODES = {"f32": MOE_ACT_F32, "q8_0": MOE_ACT_Q8_0}
ROUTERS = {"softmax": MOE_ROUTER_SOFTMAX_TOPK, "noaux_tc": MOE_ROUTER_SIGMOID_NOAUX_TC}


class MoeError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__(f"{func}: {moe_status_string(status)} ({detail})")


class RouterParams(ctypes.Structure):
    _fields_ = [("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("mode", ctypes.c_int32),
                ("renormalize", ctypes.c_int32), ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32),
                ("routed_scaling_factor", ctypes.c_float), ("score_bias", ctypes.c_void_p),
                ("top_p", ctypes.c_float), ("shared_gate", ctypes.c_void_p)]


class Experts(ctypes.Structure):
    _fields_ = [("n_experts", ctypes.c_int32), ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("format", ctypes.c_int32),
                ("gate_q", ctypes.c_void_p), ("gate_s", ctypes.c_void_p),
                ("up_q", ctypes.c_void_p), ("up_s", ctypes.c_void_p),
                ("down_q", ctypes.c_void_p), ("down_s", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "moe_workspace_size": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32, _I32]),
    "moe_quantize_weights": (_I32, [_P, _I64, _I32, _I32, _I32, _P, _P, _P]),
    "moe_quantize_q8_0": (_I32, [_P, _I64, _I32, _P, _P, _P]),
    "moe_route": (_I32, [_P, _I32, _I32, _P, ctypes.POINTER(RouterParams), _P, _P, _P, _SZ, _P]),
    "moe_dispatch": (_I32, [_P, _I32, _I32, _I32, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_expert_ffn": (_I32, [_P, _I32, _I32, ctypes.POINTER(Experts), _P, _P, _P, _I32, _P, _P, _SZ, _P]),
    "moe_combine": (_I32, [_P, _P, _P, _P, _I32, _I32, _I32, _P, _P]),
    "moe_layer_forward": (_I32, [_P, _I32, _P, ctypes.POINTER(RouterParams), ctypes.POINTER(Experts),
                                 ctypes.POINTER(Experts), _I32, _P, _P, _SZ, _P]),
    "moe_layer_forward_noalloc": (_I32, [_P, _I32, _P, ctypes.POINTER(RouterParams), ctypes.POINTER(Experts),
                                         ctypes.POINTER(Experts), _I32, _P, _P]),
    "moe_layer_forward_timed": (_I32, [_P, _I32, _P, ctypes.POINTER(RouterParams), ctypes.POINTER(Experts),
                                       ctypes.POINTER(Experts), _I32, _P, _P, _SZ, _P, _P]),
    "moe_block_forward": (_I32, [_P, _I32, _P, ctypes.c_float, _P, ctypes.POINTER(RouterParams),
                                 ctypes.POINTER(Experts), ctypes.POINTER(Experts), _I32, _P, _P, _SZ, _P, _P]),
    "moe_debug_q8_expert_ffn": (_I32, [_P, _I32, _I32, ctypes.POINTER(Experts), _P, _P, _P, _P, _P, _P, _P, _P,
                                       _P, _P, _SZ, _P]),
    "moe_debug_workspace_sections": (_I32, [_I32, _I32, _I32, _I32, _I32, _I32, _I32, _P]),
    "moe_status_string": (ctypes.c_char_p, [_I32]),
    # include/moe_calib.h: measurement references
    "moe_calib_stream_read": (_I32, [_P, ctypes.c_uint64, _P, _I32, _P]),
    "moe_calib_prefill_mix": (_I32, [_I32, _I32, _P, ctypes.POINTER(ctypes.c_uint64), _P]),
    "moe_last_error_detail": (ctypes.c_char_p, []),
}

_lib: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    """Load libmoe.so once. Fails loudly when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m quantized_expert_ffn_amd.build` "
                              "(the HIP library is the only implementation; there is no fallback)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def exported_names() -> Sequence[str]:
    return tuple(_SIGNATURES)


def moe_status_string(status: int) -> str:
    return load().moe_status_string(status).decode()


def moe_last_error_detail() -> str:
    return load().moe_last_error_detail().decode()


def _check(status: int, func: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, func, moe_last_error_detail())


def _ptr(t: Optional[torch.Tensor], dtype=None, name: str = "tensor") -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _shape(t: Optional[torch.Tensor], shape, name: str) -> None:
    """The kernels index the tensors by the sizes the call passes: a tensor of
    another shape is an error here, not an access past its end there."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _at_least(t: Optional[torch.Tensor], numel: int, name: str) -> None:
    if t is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, the call uses {numel}")


def _rows(t: torch.Tensor, rows: int, cols: int, name: str) -> None:
    """An output of rows x cols: rows of exactly cols elements, at least rows of them."""
    if t.dim() != 2 or t.shape[1] != cols or t.shape[0] < rows:
        raise ValueError(f"{name} must be [>= {rows}, {cols}], got {tuple(t.shape)}")


def _layer_shapes(x, gate_w, params, routed, out, norm_w=None) -> None:
    if x.dim() != 2:
        raise ValueError(f"x must be [T, d_model], got {tuple(x.shape)}")
    T, d = x.shape[0], routed.d_model
    _shape(x, (T, d), "x")
    _shape(gate_w, (params.n_experts, d), "gate_w")
    _rows(out, T, d, "out")
    _shape(norm_w, (d,), "norm_w")


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def router_params(n_experts: int, top_k: int, mode: str = "softmax", renormalize: bool = False,
                  n_group: int = 1, topk_group: int = 1, routed_scaling_factor: float = 1.0,
                  score_bias: Optional[torch.Tensor] = None, top_p: float = 0.0,
                  shared_gate: Optional[torch.Tensor] = None) -> RouterParams:
    """shared_gate: [d] fp32 device vector gating the shared expert by
    sigmoid(x . shared_gate), or None."""
    p = RouterParams()
    p.n_experts = n_experts
    p.top_k = top_k
    p.mode = ROUTERS[mode]
    p.renormalize = int(bool(renormalize))
    p.n_group = n_group
    p.topk_group = topk_group
    p.routed_scaling_factor = routed_scaling_factor
    p.score_bias = _ptr(score_bias, torch.float32, "score_bias")
    p.top_p = top_p
    p.shared_gate = _ptr(shared_gate, torch.float32, "shared_gate")
    p._keep = (score_bias, shared_gate)   # keep the tensors alive with the struct
    return p


def with_top_p(params: RouterParams, top_p: float) -> RouterParams:
    """A copy of a router parameter set with another adaptive expert top-p."""
    q = RouterParams()
    ctypes.memmove(ctypes.addressof(q), ctypes.addressof(params), ctypes.sizeof(RouterParams))
    q.top_p = top_p
    q._keep = getattr(params, "_keep", None)
    return q


class QuantExperts:
    """A stack of quantised SwiGLU experts in the library's layout (GPU tensors).

    Tensor shapes give the per-expert storage size only: gate_q / up_q hold
    I*d bytes (int8), I*d/2 (packed int4) or I*d/4 (packed int2) per expert,
    shaped [E, I, d], [E, I, d/2] or [E, I, d/4]; scales I*d/32 floats, shaped [E, I, d/32] (the per-row
    formats: I floats, shaped [E, I, 1]); down_q / down_s likewise with d and
    I swapped. The bytes inside are in the lane-tiled layout of
    include/moe.h (32-row tiles, lane-ordered), not row-major; per-row scales
    are in row order.
    """

    def __init__(self, fmt: str, gate_q, gate_s, up_q, up_s, down_q, down_s):
        self.fmt = fmt
        self.gate_q, self.gate_s = gate_q, gate_s
        self.up_q, self.up_s = up_q, up_s
        self.down_q, self.down_s = down_q, down_s
        self.n_experts, self.d_ff = gate_s.shape[0], gate_s.shape[1]
        self.d_model = down_s.shape[1]
        if fmt not in FORMATS:
            raise ValueError(f"unknown weight format {fmt!r}")
        div = {"int8": 1, "int4": 2, "int2": 4}[fmt.split("_")[0]]
        per_row = fmt.endswith("_row")
        E, I, d = self.n_experts, self.d_ff, self.d_model
        need = {"gate_q": (gate_q, E * I * d // div), "up_q": (up_q, E * I * d // div),
                "down_q": (down_q, E * d * I // div),
                "gate_s": (gate_s, E * I * (1 if per_row else d // 32)),
                "up_s": (up_s, E * I * (1 if per_row else d // 32)),
                "down_s": (down_s, E * d * (1 if per_row else I // 32))}
        for name, (t, n) in need.items():
            if t.numel() * t.element_size() // (4 if name.endswith("_s") else 1) != n:
                raise ValueError(f"{name} of a {fmt} stack of {E} experts (d_model {d}, d_ff {I}) must hold {n} "
                                 f"{'floats' if name.endswith('_s') else 'bytes'}")

    @classmethod
    def empty(cls, n_experts: int, d_model: int, d_ff: int, fmt: str, device="cuda"):
        if fmt not in FORMATS:
            raise ValueError(f"unknown weight format {fmt!r}")
        int8 = fmt.startswith("int8")
        div = {"int8": 1, "int4": 2, "int2": 4}[fmt.split("_")[0]]
        qdt = torch.int8 if int8 else torch.uint8
        per_row = fmt.endswith("_row")
        sg_d = 1 if per_row else d_model // 32    # scales per gate / up row
        sg_i = 1 if per_row else d_ff // 32       # scales per down row
        return cls(fmt,
                   torch.empty((n_experts, d_ff, d_model // div), dtype=qdt, device=device),
                   torch.empty((n_experts, d_ff, sg_d), dtype=torch.float32, device=device),
                   torch.empty((n_experts, d_ff, d_model // div), dtype=qdt, device=device),
                   torch.empty((n_experts, d_ff, sg_d), dtype=torch.float32, device=device),
                   torch.empty((n_experts, d_model, d_ff // div), dtype=qdt, device=device),
                   torch.empty((n_experts, d_model, sg_i), dtype=torch.float32, device=device))

    def abi(self) -> Experts:
        ex = Experts()
        ex.n_experts, ex.d_model, ex.d_ff = self.n_experts, self.d_model, self.d_ff
        ex.format = FORMATS[self.fmt]
        ex.gate_q, ex.gate_s = _ptr(self.gate_q, name="gate_q"), _ptr(self.gate_s, torch.float32, "gate_s")
        ex.up_q, ex.up_s = _ptr(self.up_q, name="up_q"), _ptr(self.up_s, torch.float32, "up_s")
        ex.down_q, ex.down_s = _ptr(self.down_q, name="down_q"), _ptr(self.down_s, torch.float32, "down_s")
        return ex

    def select(self, e: int) -> "QuantExperts":
        """A one-expert view (e.g. to pass a shared expert stored in a stack)."""
        return QuantExperts(self.fmt, *(t[e:e + 1] for t in (self.gate_q, self.gate_s, self.up_q, self.up_s,
                                                              self.down_q, self.down_s)))

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.gate_q, self.gate_s, self.up_q, self.up_s,
                                                         self.down_q, self.down_s))


# --------------------------------------------------------------------------
# entry points
# --------------------------------------------------------------------------
def moe_workspace_size(T: int, k: int, E: int, d: int, d_ff: int, act_mode: int, has_shared: bool) -> int:
    return int(load().moe_workspace_size(T, k, E, d, d_ff, act_mode, int(bool(has_shared))))


def moe_quantize_weights(w: torch.Tensor, fmt: int, q: torch.Tensor, s: torch.Tensor, stream=None,
                         matrix_rows: Optional[int] = None) -> None:
    """w: one matrix [N, K] or a stack [..., N, K]; each N-row matrix is
    written in the lane-tiled layout, one after the other."""
    rows = w.numel() // w.shape[-1]
    mr = int(matrix_rows) if matrix_rows is not None else w.shape[-2]
    _check(load().moe_quantize_weights(_ptr(w, torch.float32, "w"), rows, w.shape[-1], mr, fmt, _ptr(q, None, "q"),
                                       _ptr(s, torch.float32, "s"), _stream(stream)), "moe_quantize_weights")


def moe_quantize_q8_0(x: torch.Tensor, q: torch.Tensor, d: torch.Tensor, stream=None) -> None:
    rows = x.numel() // x.shape[-1]
    _check(load().moe_quantize_q8_0(_ptr(x, torch.float32, "x"), rows, x.shape[-1], _ptr(q, torch.int8, "q"),
                                    _ptr(d, torch.float32, "d"), _stream(stream)), "moe_quantize_q8_0")


def moe_route(x: torch.Tensor, gate_w: torch.Tensor, params: RouterParams, topk_idx: torch.Tensor,
              topk_w: torch.Tensor, ws: torch.Tensor, stream=None) -> None:
    T, d = x.shape
    _shape(gate_w, (params.n_experts, d), "gate_w")
    _at_least(topk_idx, T * params.top_k, "topk_idx")
    _at_least(topk_w, T * params.top_k, "topk_w")
    _check(load().moe_route(_ptr(x, torch.float32, "x"), T, d, _ptr(gate_w, torch.float32, "gate_w"),
                            ctypes.byref(params), _ptr(topk_idx, torch.int32, "topk_idx"),
                            _ptr(topk_w, torch.float32, "topk_w"), _ptr(ws, None, "ws"),
                            ws.numel() * ws.element_size(), _stream(stream)), "moe_route")


def moe_dispatch(topk_idx: torch.Tensor, E: int, counts: torch.Tensor, offsets: torch.Tensor,
                 perm: torch.Tensor, inv_perm: torch.Tensor, ws: Optional[torch.Tensor] = None,
                 stream=None) -> None:
    """ws (optional): scratch that lets large batches dispatch over many blocks."""
    T, k = topk_idx.shape
    _at_least(counts, E, "counts")
    _at_least(offsets, E + 1, "offsets")
    _at_least(perm, T * k, "perm")
    _at_least(inv_perm, T * k, "inv_perm")
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(load().moe_dispatch(_ptr(topk_idx, torch.int32, "topk_idx"), T, k, E, _ptr(counts, torch.int32, "counts"),
                               _ptr(offsets, torch.int32, "offsets"), _ptr(perm, torch.int32, "perm"),
                               _ptr(inv_perm, torch.int32, "inv_perm"), _ptr(ws, None, "ws"), nbytes,
                               _stream(stream)), "moe_dispatch")


def moe_expert_ffn(x: torch.Tensor, k: int, experts: QuantExperts, counts: torch.Tensor, offsets: torch.Tensor,
                   perm: torch.Tensor, act_mode: int, y_perm: torch.Tensor, ws: torch.Tensor, stream=None) -> None:
    ex = experts.abi()
    T, d = x.shape[0], experts.d_model
    _shape(x, (T, d), "x")
    _at_least(counts, experts.n_experts, "counts")
    _at_least(offsets, experts.n_experts + 1, "offsets")
    _at_least(perm, T * k, "perm")
    _at_least(y_perm, T * k * d, "y_perm")
    _check(load().moe_expert_ffn(_ptr(x, torch.float32, "x"), x.shape[0], k, ctypes.byref(ex),
                                 _ptr(counts, torch.int32, "counts"), _ptr(offsets, torch.int32, "offsets"),
                                 _ptr(perm, torch.int32, "perm"), act_mode, _ptr(y_perm, torch.float32, "y_perm"),
                                 _ptr(ws, None, "ws"), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_expert_ffn")


def moe_debug_q8_expert_ffn(x, k, experts: QuantExperts, counts, offsets, perm, dots_gate, dots_up, hq, hd,
                            dots_down, y_perm, ws, stream=None) -> None:
    ex = experts.abi()
    _check(load().moe_debug_q8_expert_ffn(
        _ptr(x, torch.float32, "x"), x.shape[0], k, ctypes.byref(ex), _ptr(counts, torch.int32, "counts"),
        _ptr(offsets, torch.int32, "offsets"), _ptr(perm, torch.int32, "perm"),
        _ptr(dots_gate, torch.int32, "dots_gate"), _ptr(dots_up, torch.int32, "dots_up"),
        _ptr(hq, torch.int8, "hq"), _ptr(hd, torch.float32, "hd"), _ptr(dots_down, torch.int32, "dots_down"),
        _ptr(y_perm, torch.float32, "y_perm"), _ptr(ws, None, "ws"), ws.numel() * ws.element_size(),
        _stream(stream)), "moe_debug_q8_expert_ffn")


def moe_debug_workspace_sections(T: int, k: int, E: int, d: int, d_ff: int, act_mode: int,
                                 has_shared: bool) -> dict:
    """Byte offsets inside the layer's workspace where moe_layer_forward leaves
    its routing results and (Q8_0 mode) H's codes and scales: a dict keyed by
    WS_SECTIONS (-1 for a section the mode does not have)."""
    arr = (ctypes.c_int64 * len(WS_SECTIONS))()
    _check(load().moe_debug_workspace_sections(T, k, E, d, d_ff, act_mode, int(bool(has_shared)), arr),
           "moe_debug_workspace_sections")
    return dict(zip(WS_SECTIONS, (int(v) for v in arr)))


def moe_calib_stream_read(buf: torch.Tensor, sink: torch.Tensor, blocks: int, stream=None) -> None:
    """Reference streaming read of every byte of buf (include/moe_calib.h);
    sink: uint32-sized [blocks] device tensor."""
    if sink.numel() * sink.element_size() < 4 * blocks:
        raise ValueError(f"sink holds {sink.numel() * sink.element_size()} bytes, the launch writes {4 * blocks}")
    _check(load().moe_calib_stream_read(_ptr(buf, None, "buf"), buf.numel() * buf.element_size(),
                                        _ptr(sink, None, "sink"), blocks, _stream(stream)), "moe_calib_stream_read")


def moe_calib_prefill_mix(blocks: int, stages: int, sink: torch.Tensor, stream=None) -> int:
    """The prefill GEMM's inner loop alone (include/moe_calib.h); sink: fp32
    [blocks * 512] device tensor. Returns the useful int8 operations launched."""
    if sink.numel() < blocks * 512:
        raise ValueError(f"sink holds {sink.numel()} floats, the launch writes {blocks * 512}")
    ops = ctypes.c_uint64(0)
    _check(load().moe_calib_prefill_mix(blocks, stages, _ptr(sink, torch.float32, "sink"), ctypes.byref(ops),
                                        _stream(stream)), "moe_calib_prefill_mix")
    return int(ops.value)


def moe_combine(y_perm: torch.Tensor, topk_w: torch.Tensor, inv_perm: torch.Tensor,
                shared_y: Optional[torch.Tensor], out: torch.Tensor, stream=None) -> None:
    T, k = topk_w.shape
    d = out.shape[1]
    _rows(out, T, d, "out")
    _at_least(inv_perm, T * k, "inv_perm")
    _at_least(y_perm, T * k * d, "y_perm")
    _shape(shared_y, (T, d), "shared_y")
    _check(load().moe_combine(_ptr(y_perm, torch.float32, "y_perm"), _ptr(topk_w, torch.float32, "topk_w"),
                              _ptr(inv_perm, torch.int32, "inv_perm"), _ptr(shared_y, torch.float32, "shared_y"),
                              T, k, out.shape[1], _ptr(out, torch.float32, "out"), _stream(stream)), "moe_combine")


def moe_layer_forward(x: torch.Tensor, gate_w: torch.Tensor, params: RouterParams, routed: QuantExperts,
                      shared: Optional[QuantExperts], act_mode: int, out: torch.Tensor, ws: torch.Tensor,
                      stream=None, _abi_cache=None) -> None:
    _layer_shapes(x, gate_w, params, routed, out)
    r = routed.abi()
    s = shared.abi() if shared is not None else None
    _check(load().moe_layer_forward(_ptr(x, torch.float32, "x"), x.shape[0], _ptr(gate_w, torch.float32, "gate_w"),
                                    ctypes.byref(params), ctypes.byref(r), ctypes.byref(s) if s is not None else None,
                                    act_mode, _ptr(out, torch.float32, "out"), _ptr(ws, None, "ws"),
                                    ws.numel() * ws.element_size(), _stream(stream)), "moe_layer_forward")


MOE_NOALLOC_SCRATCH_BYTES = 32 << 20   # include/moe.h


def moe_layer_forward_noalloc(x: torch.Tensor, gate_w: torch.Tensor, params: RouterParams, routed: QuantExperts,
                              shared: Optional[QuantExperts], act_mode: int, out: torch.Tensor, stream=None) -> None:
    """moe_layer_forward with the library's own per-GPU scratch instead of a
    workspace (no allocation); calls needing more than
    MOE_NOALLOC_SCRATCH_BYTES of workspace are rejected."""
    _layer_shapes(x, gate_w, params, routed, out)
    r = routed.abi()
    s = shared.abi() if shared is not None else None
    _check(load().moe_layer_forward_noalloc(_ptr(x, torch.float32, "x"), x.shape[0],
                                            _ptr(gate_w, torch.float32, "gate_w"), ctypes.byref(params),
                                            ctypes.byref(r), ctypes.byref(s) if s is not None else None, act_mode,
                                            _ptr(out, torch.float32, "out"), _stream(stream)),
           "moe_layer_forward_noalloc")


def moe_layer_forward_timed(x, gate_w, params: RouterParams, routed: QuantExperts, shared: Optional[QuantExperts],
                            act_mode: int, out, ws, events: Sequence[Optional[torch.cuda.Event]],
                            stream=None) -> None:
    """events: 2 * MOE_STAGE_COUNT torch.cuda.Event(enable_timing=True) or None;
    entry 2s is recorded before stage s and 2s+1 after it."""
    if len(events) != 2 * MOE_STAGE_COUNT:
        raise ValueError(f"need {2 * MOE_STAGE_COUNT} events")
    handles = []
    for ev in events:
        if ev is None:
            handles.append(None)
            continue
        if not ev.cuda_event:
            ev.record()        # torch creates the HIP event on its first record
        handles.append(ev.cuda_event)
    arr = (ctypes.c_void_p * len(events))(*handles)
    _layer_shapes(x, gate_w, params, routed, out)
    r = routed.abi()
    s = shared.abi() if shared is not None else None
    _check(load().moe_layer_forward_timed(
        _ptr(x, torch.float32, "x"), x.shape[0], _ptr(gate_w, torch.float32, "gate_w"), ctypes.byref(params),
        ctypes.byref(r), ctypes.byref(s) if s is not None else None, act_mode, _ptr(out, torch.float32, "out"),
        _ptr(ws, None, "ws"), ws.numel() * ws.element_size(), arr, _stream(stream)), "moe_layer_forward_timed")


def _event_array(events):
    if len(events) != 2 * MOE_STAGE_COUNT:
        raise ValueError(f"need {2 * MOE_STAGE_COUNT} events")
    handles = []
    for ev in events:
        if ev is None:
            handles.append(None)
            continue
        if not ev.cuda_event:
            ev.record()        # torch creates the HIP event on its first record
        handles.append(ev.cuda_event)
    return (ctypes.c_void_p * len(events))(*handles)


def moe_block_forward(x, norm_w: Optional[torch.Tensor], eps: float, gate_w, params: RouterParams,
                      routed: QuantExperts, shared: Optional[QuantExperts], act_mode: int, out, ws,
                      events: Optional[Sequence[Optional[torch.cuda.Event]]] = None, stream=None) -> None:
    """out = x + layer(RMSNorm(x)) (norm_w None: out = x + layer(x)); out may be x."""
    arr = _event_array(events) if events is not None else None
    _layer_shapes(x, gate_w, params, routed, out, norm_w)
    r = routed.abi()
    s = shared.abi() if shared is not None else None
    _check(load().moe_block_forward(
        _ptr(x, torch.float32, "x"), x.shape[0], _ptr(norm_w, torch.float32, "norm_w"), eps,
        _ptr(gate_w, torch.float32, "gate_w"), ctypes.byref(params), ctypes.byref(r),
        ctypes.byref(s) if s is not None else None, act_mode, _ptr(out, torch.float32, "out"),
        _ptr(ws, None, "ws"), ws.numel() * ws.element_size(), arr, _stream(stream)), "moe_block_forward")


def quantize_experts(gate: torch.Tensor, up: torch.Tensor, down: torch.Tensor, fmt: str, stream=None) -> QuantExperts:
    """Quantise fp32 expert stacks (gate/up [E, I, d], down [E, d, I]) on the GPU."""
    E, I, d = gate.shape
    ex = QuantExperts.empty(E, d, I, fmt, device=gate.device)
    f = FORMATS[fmt]
    moe_quantize_weights(gate.contiguous(), f, ex.gate_q, ex.gate_s, stream)
    moe_quantize_weights(up.contiguous(), f, ex.up_q, ex.up_s, stream)
    moe_quantize_weights(down.contiguous(), f, ex.down_q, ex.down_s, stream)
    return ex


def workspace(T: int, k: int, E: int, d: int, d_ff: int, act_mode: int, has_shared: bool,
              device="cuda") -> torch.Tensor:
    n = moe_workspace_size(T, k, E, d, d_ff, act_mode, has_shared)
    if n == 0:
        raise ValueError("invalid sizes for moe_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=device)
