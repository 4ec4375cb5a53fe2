"""Oracle: one quantised SwiGLU expert, in two activation modes.

TEST INFRASTRUCTURE ONLY (see the package docstring).

An expert is a SwiGLU FFN ("mtlm-7m-base": SwiGLU blocks, SiLU) whose three
matrices are stored group-32 quantised ("Show HN: Getting GLM-5.2 running on my slow computer", section "What's
implemented": int8 / packed int4, dequantised on use):
    gate, up: [I, d]    down: [d, I]
    G = X gate^T,  U = X up^T,  H = silu(G) * U,  Y = H down^T
with silu(g) = g * sigmoid(g).

Two activation modes, after the same page (batches take integer dots on
Q8_0-quantised activations, while a single int4 row keeps f32 activations):
  * "f32": activations stay fp32 and meet the dequantised weights s*q. The
    oracle evaluates every product and sum in fp64.
  * "q8_0": activations are Q8_0-quantised per 32 (see oracle.quant). Per
    output and per group g the int8 codes give an exact integer dot
    I_g = sum_{k in g} xq_k * wq_k, and G = sum_g dx_g * sw_g * I_g. H is
    rounded to fp32 and Q8_0-quantised again before the down projection.
    The integer-dot sum equals dequant(Xq) dequant(W)^T exactly up to fp64
    rounding, so that product form is used for speed; group_dots() gives the
    integers themselves.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from . import quant


@dataclasses.dataclass
class QuantExpert:
    """One expert's quantised matrices as integer codes plus fp32 scales.

    bits = 8: codes in [-127, 127]; bits = 4: codes in [-7, 7]; bits = 2:
    codes in [-1, 1].
    gate_q, up_q [I, d]; down_q [d, I]; *_s the matching group scales, or one
    scale per row ([rows, 1]) when per_row.
    """
    bits: int
    gate_q: np.ndarray
    gate_s: np.ndarray
    up_q: np.ndarray
    up_s: np.ndarray
    down_q: np.ndarray
    down_s: np.ndarray
    per_row: bool = False

    @classmethod
    def from_fp32(cls, gate, up, down, bits: int, per_row: bool = False) -> "QuantExpert":
        qz = quant.quantize_rows if per_row else quant.quantize_weights
        gq, gs = qz(gate, bits)
        uq, us = qz(up, bits)
        dq, ds = qz(down, bits)
        return cls(bits, gq, gs, uq, us, dq, ds, per_row)

    def dequantized(self):
        return (quant.dequantize(self.gate_q, self.gate_s),
                quant.dequantize(self.up_q, self.up_s),
                quant.dequantize(self.down_q, self.down_s))

    def stored(self, which: str) -> np.ndarray:
        """Bytes as the library stores them: int8 codes, or packed int4 / int2."""
        return quant.pack_codes(getattr(self, which + "_q"), self.bits)


def silu(g: np.ndarray) -> np.ndarray:
    return g / (1.0 + np.exp(-g))


def ffn_f32(x: np.ndarray, ex: QuantExpert) -> np.ndarray:
    """Expert output for fp32 activation rows x [n, d] -> [n, d] fp64."""
    wg, wu, wd = ex.dequantized()
    x64 = np.asarray(x, np.float32).astype(np.float64)
    g = x64 @ wg.T
    u = x64 @ wu.T
    h = silu(g) * u
    return h @ wd.T


def ffn_q8(x: np.ndarray, ex: QuantExpert, hq_override=None):
    """Expert output in Q8_0 mode for rows x [n, d].

    Returns (y fp64 [n, d], parts) where parts holds the intermediate
    quantities: xq, xd (Q8_0 of x), h32 (fp32 H), hq, hd (Q8_0 of h32).
    hq_override = (hq, hd) replaces the oracle's own Q8_0(H) in the down
    projection (used to check a down projection fed the same int8 codes).
    """
    wg, wu, wd = ex.dequantized()
    xq, xd = quant.quantize_q8_0(x)
    xdeq = quant.dequantize(xq, xd)
    g = xdeq @ wg.T
    u = xdeq @ wu.T
    h32 = (silu(g) * u).astype(np.float32)
    hq, hd = quant.quantize_q8_0(h32)
    if hq_override is not None:
        hq, hd = hq_override
    y = quant.dequantize(hq, hd) @ wd.T
    return y, dict(xq=xq, xd=xd, g=g, u=u, h32=h32, hq=hq, hd=hd)


def group_dots(aq: np.ndarray, bq: np.ndarray) -> np.ndarray:
    """Exact per-group integer dots: I[m, n, g] = sum_{k in g} aq[m,k]*bq[n,k]."""
    a = quant._groups(np.asarray(aq).astype(np.int64))     # [M, G, 32]
    b = quant._groups(np.asarray(bq).astype(np.int64))     # [N, G, 32]
    return np.einsum("mgk,ngk->mng", a, b)
