"""Algorithmic bytes and operations of the MoE layer, for roofline pricing.

Bytes count what the method must move at least once: each distinct selected
expert's quantised weights and scales once (batch-union), the router weight,
the hidden states in and the layer output out. Operations count useful
multiply-adds (2 ops each) of the expert matmuls, padding excluded.

The pages give the same accounting for their GLM-5.2 layer: a routed expert is
about 19 MB of int4 payload and a cold token reads about 11.4 GB of experts
over 75 layers of 8 experts ("Show HN: Getting GLM-5.2 running on my slow computer", sections "The idea" and "Got
a better machine?"). Group-32 fp32 scales add 4 bytes per 32 weights on top of
that payload; per-row scales add 4 bytes per matrix row.
"""
from __future__ import annotations

from typing import Sequence

GROUP = 32


def matrix_bytes(rows: int, cols: int, fmt: str) -> int:
    """Quantised codes + fp32 scales (per group of 32, or per row for the
    "_row" formats) of one [rows, cols] matrix."""
    payload = rows * cols * {"int8": 8, "int4": 4, "int2": 2}[fmt.split("_")[0]] // 8
    scales = rows if fmt.endswith("_row") else rows * (cols // GROUP)
    return payload + scales * 4


def expert_bytes(d: int, d_ff: int, fmt: str) -> int:
    """gate [I, d] + up [I, d] + down [d, I]."""
    return 2 * matrix_bytes(d_ff, d, fmt) + matrix_bytes(d, d_ff, fmt)


def gateup_bytes(d: int, d_ff: int, fmt: str) -> int:
    return 2 * matrix_bytes(d_ff, d, fmt)


def down_bytes(d: int, d_ff: int, fmt: str) -> int:
    return matrix_bytes(d, d_ff, fmt)


def distinct_experts(counts: Sequence[int]) -> int:
    return sum(1 for c in counts if c > 0)


def layer_bytes(counts: Sequence[int], T: int, d: int, d_ff: int, fmt: str, n_experts: int,
                has_shared: bool, has_bias: bool = False) -> int:
    """Minimum HBM bytes of one layer call (weights once, router, x in, out)."""
    n = distinct_experts(counts) + (1 if has_shared else 0)
    return (n * expert_bytes(d, d_ff, fmt) + n_experts * d * 4 + (n_experts * 4 if has_bias else 0)
            + 2 * T * d * 4)


def gateup_kernel_bytes(counts: Sequence[int], T: int, k: int, d: int, d_ff: int, fmt: str,
                        has_shared: bool, act_mode: str) -> int:
    """Algorithmic bytes of the gate/up kernel: distinct experts' gate and up
    weights once, the activations once, H written once."""
    n = distinct_experts(counts) + (1 if has_shared else 0)
    rows = int(sum(counts)) + (T if has_shared else 0)     # routed rows (T*k unless top-p dropped some)
    if act_mode == "f32":
        x_bytes = T * d * 4
        h_bytes = rows * d_ff * 4
    else:
        x_bytes = T * d + T * (d // GROUP) * 4
        h_bytes = rows * d_ff + rows * (d_ff // GROUP) * 4
    return n * gateup_bytes(d, d_ff, fmt) + x_bytes + h_bytes


def useful_ops(counts: Sequence[int], T: int, d: int, d_ff: int, has_shared: bool) -> int:
    """2 * multiply-adds of the three expert matmuls over real rows."""
    rows = sum(int(c) for c in counts) + (T if has_shared else 0)
    return 2 * rows * 3 * d * d_ff


def gateup_ops(counts: Sequence[int], T: int, d: int, d_ff: int, has_shared: bool) -> int:
    rows = sum(int(c) for c in counts) + (T if has_shared else 0)
    return 2 * rows * 2 * d * d_ff
