"""Block quantizers: amax6, four_six, mxfp4_search, amax2_or_amax6, and the
two-term residual query.

Oracle module (test infrastructure only; see the package docstring).

Scale-mode names and their assignment come from "BitDecoding-FP4
evaluation/config.py": ``recipe_additional_config`` maps RECIPE to
``nvfp4_scale_mode = {key: four_six | amax6, value: amax6, query: amax6}``
and ``nvfp4_query_terms = 2 | 1``; ``probability_environment`` selects the
probability scale mode ``amax6`` (scaling disabled) or ``amax2_or_amax6_c8`` /
``amax2_or_amax6`` (c = 8 / c = 1, threshold tau); the ``bitdecoding-mxfp4``
KV_MODES entry uses ``mxfp4_search``. The page gives the names only; the
rules below are the plainest readings consistent with them:

* ``amax6``: one E4M3 scale per 16 consecutive elements,
  s = E4M3(float32(amax / 6)), so the block maximum lands on the E2M1 maximum.
* ``four_six`` (adaptive block-scale search, keys): candidates
  s6 = E4M3(float32(amax/6)) and s4 = E4M3(float32(amax/4)); quantize with
  each and keep s4 only if its squared error is strictly smaller. The squared
  error is sum_j (x_j - s*g_j)**2 with every subtract, square and add a
  float32 operation, summed as a balanced pairwise tree over consecutive pairs.
* ``mxfp4_search``: one E8M0 scale 2**E per 32 elements; candidates E_hi, the
  least integer with amax <= 6 * 2**E, and E_hi - 1; keep E_hi - 1 only if its
  squared error (same tree over 32) is strictly smaller. The E8M0 code is
  E + 127, E limited to [-127, 127]. An all-zero block has code 0 and zero
  element codes.
* ``amax2_or_amax6`` (underflow-aware probability scaling, c and tau): on
  p' = c * p, per 16-token block with a = max p': s = E4M3(float32(a / 2)) if
  a < tau, else E4M3(float32(a / 6)). Dequantized P is s * e2m1 / c.
* two-term query: Q1 = quantize(q_r), r = float32(q_r - deq(Q1)),
  Q2 = quantize(r); the query used in Q.K is deq(Q1) + deq(Q2).
"""
from __future__ import annotations

import numpy as np

from .formats import (
    E2M1_GRID,
    e2m1_encode,
    e2m1_value,
    e4m3_encode,
    e4m3_value,
    e8m0_value,
)

NONE = "none"
AMAX6 = "amax6"
FOUR_SIX = "four_six"
MXFP4_SEARCH = "mxfp4_search"
AMAX2_OR_AMAX6 = "amax2_or_amax6"

NV_BLOCK = 16
MX_BLOCK = 32


def block_size(mode: str) -> int:
    return MX_BLOCK if mode == MXFP4_SEARCH else NV_BLOCK


def sse_tree(e: np.ndarray) -> np.ndarray:
    """Balanced pairwise float32 sum over the last axis (a power of two):
    ((e0+e1)+(e2+e3))+... level by level."""
    s = np.asarray(e, dtype=np.float32)
    while s.shape[-1] > 1:
        s = (s[..., 0::2] + s[..., 1::2]).astype(np.float32)
    return s[..., 0]


def _blocks(x: np.ndarray, n: int) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    assert x.shape[-1] % n == 0
    return x.reshape(x.shape[:-1] + (x.shape[-1] // n, n))


def _deq_f32(nib: np.ndarray, s_val: np.ndarray) -> np.ndarray:
    """s * e2m1 in float32 (exact: at most 6 significant bits)."""
    return (np.float32(1.0) * e2m1_value(nib).astype(np.float32) * s_val.astype(np.float32)).astype(np.float32)


def _sse(xb: np.ndarray, nib: np.ndarray, s_val: np.ndarray) -> np.ndarray:
    d = (xb - _deq_f32(nib, s_val[..., None])).astype(np.float32)
    return sse_tree((d * d).astype(np.float32))


def quantize_amax6(x: np.ndarray):
    """NVFP4 amax6 over blocks of 16: returns (nibbles [...,n], e4m3 codes [...,n/16])."""
    xb = _blocks(x, NV_BLOCK)
    a = np.max(np.abs(xb), axis=-1)
    sc = e4m3_encode((a / np.float32(6.0)).astype(np.float32))
    s_val = e4m3_value(sc).astype(np.float32)
    nib = e2m1_encode(xb, s_val[..., None])
    return nib.reshape(np.shape(x)), sc


def quantize_four_six(x: np.ndarray):
    """NVFP4 adaptive {4,6} block-scale search over blocks of 16."""
    xb = _blocks(x, NV_BLOCK)
    a = np.max(np.abs(xb), axis=-1)
    sc6 = e4m3_encode((a / np.float32(6.0)).astype(np.float32))
    sc4 = e4m3_encode((a / np.float32(4.0)).astype(np.float32))
    s6 = e4m3_value(sc6).astype(np.float32)
    s4 = e4m3_value(sc4).astype(np.float32)
    nib6 = e2m1_encode(xb, s6[..., None])
    nib4 = e2m1_encode(xb, s4[..., None])
    err6 = _sse(xb, nib6, s6)
    err4 = _sse(xb, nib4, s4)
    take4 = err4 < err6
    nib = np.where(take4[..., None], nib4, nib6)
    sc = np.where(take4, sc4, sc6).astype(np.uint8)
    return nib.reshape(np.shape(x)), sc


def mx_exponent_hi(a: np.ndarray) -> np.ndarray:
    """Least integer E with a <= 6 * 2**E (a > 0, float32), found by exact
    float64 comparisons around a first guess."""
    a64 = np.asarray(a, dtype=np.float32).astype(np.float64)
    e = np.ceil(np.log2(a64 / 6.0)).astype(np.int64)
    for _ in range(3):
        e = np.where(6.0 * np.exp2(e.astype(np.float64)) < a64, e + 1, e)
        e = np.where(6.0 * np.exp2((e - 1).astype(np.float64)) >= a64, e - 1, e)
    return e


def quantize_mxfp4_search(x: np.ndarray):
    """MXFP4 two-candidate search over blocks of 32: (nibbles, e8m0 codes)."""
    xb = _blocks(x, MX_BLOCK)
    a = np.max(np.abs(xb), axis=-1)
    zero = a == 0
    e_hi = np.clip(mx_exponent_hi(np.where(zero, np.float32(1.0), a)), -127, 127)
    e_lo = np.maximum(e_hi - 1, -127)
    s_hi = np.exp2(e_hi.astype(np.float64)).astype(np.float32)
    s_lo = np.exp2(e_lo.astype(np.float64)).astype(np.float32)
    nib_hi = e2m1_encode(xb, s_hi[..., None])
    nib_lo = e2m1_encode(xb, s_lo[..., None])
    err_hi = _sse(xb, nib_hi, s_hi)
    err_lo = _sse(xb, nib_lo, s_lo)
    take_lo = (err_lo < err_hi) & (e_lo < e_hi)
    nib = np.where(take_lo[..., None], nib_lo, nib_hi)
    e = np.where(take_lo, e_lo, e_hi)
    code = (e + 127).astype(np.uint8)
    nib = np.where(zero[..., None], np.uint8(0), nib).astype(np.uint8)
    code = np.where(zero, np.uint8(0), code).astype(np.uint8)
    return nib.reshape(np.shape(x)), code


def quantize(x: np.ndarray, mode: str):
    """Quantize rows (last axis a multiple of the block) with a scale mode."""
    if mode == AMAX6:
        return quantize_amax6(x)
    if mode == FOUR_SIX:
        return quantize_four_six(x)
    if mode == MXFP4_SEARCH:
        return quantize_mxfp4_search(x)
    raise ValueError(f"not an element scale mode: {mode!r}")


def scale_value(codes: np.ndarray, mode: str) -> np.ndarray:
    if mode == MXFP4_SEARCH:
        return e8m0_value(codes)
    return e4m3_value(codes)


def dequantize(nib: np.ndarray, scales: np.ndarray, mode: str) -> np.ndarray:
    """s * e2m1 per element, float64 (exact)."""
    n = block_size(mode)
    s = scale_value(scales, mode)
    v = e2m1_value(nib)
    vb = v.reshape(v.shape[:-1] + (v.shape[-1] // n, n))
    return (vb * s[..., None]).reshape(v.shape)


def quantize_p(pp: np.ndarray, mode: str, tau) -> tuple:
    """Probability quantizer over aligned 16-token blocks of p' = c * p
    (float32, non-negative). Returns (nibbles, e4m3 codes)."""
    pb = _blocks(pp, NV_BLOCK)
    a = np.max(pb, axis=-1)
    s6 = e4m3_encode((a / np.float32(6.0)).astype(np.float32))
    if mode == AMAX6:
        sc = s6
    elif mode == AMAX2_OR_AMAX6:
        s2 = e4m3_encode((a / np.float32(2.0)).astype(np.float32))
        sc = np.where(a < np.float32(tau), s2, s6).astype(np.uint8)
    else:
        raise ValueError(f"not a probability scale mode: {mode!r}")
    s_val = e4m3_value(sc).astype(np.float32)
    nib = e2m1_encode(pb, s_val[..., None])
    return nib.reshape(np.shape(pp)), sc


def quantize_query(q_r: np.ndarray, mode: str, terms: int):
    """Two-term (or one-term) residual quantization of an already rotated
    float32 query row [..., 128].

    Returns (terms_list, qhat) where terms_list holds (nibbles, scales) per
    term and qhat = sum of the dequantized terms (float64, exact)."""
    q_r = np.asarray(q_r, dtype=np.float32)
    if mode == NONE:
        return [], q_r.astype(np.float64)
    nib1, sc1 = quantize(q_r, mode)
    deq1 = dequantize(nib1, sc1, mode)
    out = [(nib1, sc1)]
    qhat = deq1.copy()
    if terms == 2:
        r = (q_r - deq1.astype(np.float32)).astype(np.float32)
        nib2, sc2 = quantize(r, mode)
        out.append((nib2, sc2))
        qhat = qhat + dequantize(nib2, sc2, mode)
    elif terms != 1:
        raise ValueError("query_terms is 1 or 2")
    return out, qhat


__all__ = [
    "NONE", "AMAX6", "FOUR_SIX", "MXFP4_SEARCH", "AMAX2_OR_AMAX6",
    "NV_BLOCK", "MX_BLOCK", "E2M1_GRID", "block_size", "sse_tree",
    "quantize_amax6", "quantize_four_six", "quantize_mxfp4_search",
    "mx_exponent_hi", "quantize", "scale_value", "dequantize", "quantize_p",
    "quantize_query",
]
