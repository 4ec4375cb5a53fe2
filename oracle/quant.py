"""Oracle: group-32 weight quantisation, int4 packing, Q8_0 activations.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Weights ("mtlm-7m-base", section "Files": int8 export with group size 32;
"Show HN: Getting GLM-5.2 running on my slow computer", section "What's implemented": int8 / packed int4
quantisation, dequantised on use). Each row of a matrix is cut into groups of
32 consecutive elements along its input (reduction) axis; a group keeps one
fp32 scale s and signed integer codes q with s*q approximating the weights:

    amax = max |w| over the group
    s    = amax / qmax            (qmax = 127 for int8, 7 for int4, 1 for int2;
                                   fp32 divide)
    q    = clamp(rne(w / s), -qmax, qmax)   (fp32 divide, round half to even)
    amax == 0  ->  s = 0, q = 0

The pages give no formula beyond "group size 32", "per-group scale" and
"symmetric"; the symmetric absmax scale with round-half-to-even is the plainest
reading. Codes are decided in fp32 so that a GPU quantiser can match them bit
for bit.

Packed int4 ("two nibbles per byte", symmetric): element 2i sits in the low
nibble of byte i and element 2i+1 in the high nibble, each as a 4-bit two's
complement number.

Packed int2 (same section: "packed int2", next to int4 and validated against
the int8 container): four 2-bit two's complement codes per byte, element
4i + j in bits 2j, 2j+1 of byte i. Symmetric like the other widths, so
qmax = 2^(bits-1) - 1 = 1: the codes are -1, 0 and 1 (the pattern of -2 is
never produced by the quantiser, though unpacking reads it).

Activations ("Show HN: Getting GLM-5.2 running on my slow computer", section "What's implemented": Q8_0-style int8
activations). Each row is cut into groups of 32; a group keeps an fp32 scale d
and int8 codes, all steps in fp32:

    amax = max |x|;  d = amax / 127;  id = (d == 0) ? 0 : 1 / d
    q    = clamp(rne(x * id), -127, 127)
"""
from __future__ import annotations

import numpy as np

GROUP = 32


def _groups(a: np.ndarray) -> np.ndarray:
    if a.shape[-1] % GROUP:
        raise ValueError(f"last dimension {a.shape[-1]} is not a multiple of {GROUP}")
    return a.reshape(a.shape[:-1] + (a.shape[-1] // GROUP, GROUP))


def qmax_for_bits(bits: int) -> int:
    if bits == 8:
        return 127
    if bits == 4:
        return 7
    if bits == 2:
        return 1
    raise ValueError(f"unsupported weight bits {bits}")


def quantize_weights(w: np.ndarray, bits: int):
    """Group-32 symmetric quantisation of fp32 weights along the last axis.

    Returns (q, s): q int8 codes with the shape of w, s fp32 scales with the
    last axis divided by 32.
    """
    w = np.asarray(w, dtype=np.float32)
    g = _groups(w)
    qmax = np.float32(qmax_for_bits(bits))
    amax = np.max(np.abs(g), axis=-1)
    s = (amax / qmax).astype(np.float32)
    q = np.zeros(g.shape, dtype=np.float32)
    nz = s > 0
    if np.any(nz):
        r = g[nz] / s[nz][:, None]          # fp32 / fp32 -> fp32, IEEE rounding
        q[nz] = np.clip(np.rint(r), -qmax, qmax)
    return q.astype(np.int8).reshape(w.shape), s


def quantize_rows(w: np.ndarray, bits: int):
    """Per-row symmetric quantisation ("Show HN: Getting GLM-5.2 running on my
    slow computer", section "What's implemented": int8 / packed int4 kernels
    with per-row scales): one fp32 scale per row over the whole last axis,
    s = amax / qmax, q = clamp(round_half_even(w / s), -qmax, qmax), in the
    same fp32 steps as the group quantiser.

    Returns (q, s): q int8 codes with the shape of w, s fp32 [..., 1] (the
    shape dequantize broadcasts over the groups of a row).
    """
    w = np.asarray(w, dtype=np.float32)
    qmax = np.float32(qmax_for_bits(bits))
    amax = np.max(np.abs(w), axis=-1, keepdims=True)
    s = (amax / qmax).astype(np.float32)
    q = np.zeros(w.shape, dtype=np.float32)
    nz = (s > 0)[..., 0]
    if np.any(nz):
        q[nz] = np.clip(np.rint(w[nz] / s[nz]), -qmax, qmax)
    return q.astype(np.int8), s


def dequantize(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """s * q in fp64 (exact: an fp32 scale times a small integer). s holds one
    scale per group, or one per row as [..., 1]."""
    g = _groups(np.asarray(q).astype(np.float64))
    return (g * np.asarray(s, dtype=np.float64)[..., None]).reshape(np.shape(q))


def pack_int4(q: np.ndarray) -> np.ndarray:
    """Pack int4 codes (int8 array, values in [-8, 7]) two per byte."""
    q = np.asarray(q)
    if q.shape[-1] % 2:
        raise ValueError("int4 packing needs an even last dimension")
    if q.min(initial=0) < -8 or q.max(initial=0) > 7:
        raise ValueError("int4 code out of range")
    u = q.astype(np.int16) & 0xF
    lo = u[..., 0::2]
    hi = u[..., 1::2]
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_int4(b: np.ndarray) -> np.ndarray:
    """Inverse of pack_int4: bytes -> int8 codes (sign-extended nibbles)."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int16)
    lo = b & 0xF
    hi = (b >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def pack_int2(q: np.ndarray) -> np.ndarray:
    """Pack int2 codes (int8 array, values in [-2, 1]) four per byte."""
    q = np.asarray(q)
    if q.shape[-1] % 4:
        raise ValueError("int2 packing needs a last dimension divisible by 4")
    if q.min(initial=0) < -2 or q.max(initial=0) > 1:
        raise ValueError("int2 code out of range")
    u = q.astype(np.int16) & 0x3
    out = u[..., 0::4] | (u[..., 1::4] << 2) | (u[..., 2::4] << 4) | (u[..., 3::4] << 6)
    return out.astype(np.uint8)


def unpack_int2(b: np.ndarray) -> np.ndarray:
    """Inverse of pack_int2: bytes -> int8 codes (sign-extended 2-bit fields)."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int16)
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 4,), dtype=np.int8)
    for j in range(4):
        f = (b >> (2 * j)) & 0x3
        out[..., j::4] = np.where(f >= 2, f - 4, f)
    return out


def pack_codes(q: np.ndarray, bits: int) -> np.ndarray:
    """The stored bytes of int8 codes at a weight width: int8 as is, int4 and
    int2 packed."""
    if bits == 8:
        return np.asarray(q, np.int8)
    if bits == 4:
        return pack_int4(q)
    if bits == 2:
        return pack_int2(q)
    raise ValueError(f"unsupported weight bits {bits}")


def quantize_q8_0(x: np.ndarray):
    """Q8_0-style activation quantisation along the last axis, fp32 steps.

    Returns (q int8 with the shape of x, d fp32 with the last axis / 32).
    """
    x = np.asarray(x, dtype=np.float32)
    g = _groups(x)
    amax = np.max(np.abs(g), axis=-1)
    d = (amax / np.float32(127)).astype(np.float32)
    idv = np.zeros_like(d)
    nz = d != 0
    idv[nz] = np.float32(1) / d[nz]
    prod = (g * idv[..., None]).astype(np.float32)   # fp32 multiply, no fusion
    q = np.clip(np.rint(prod), -127, 127).astype(np.int8)
    return q.reshape(x.shape), d
