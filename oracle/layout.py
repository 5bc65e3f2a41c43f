"""Physical layout of one quantized page of the KV cache.

Oracle module (test infrastructure only; see the package docstring).

A page holds 128 tokens ("block_size": 128 in PARITY_ENGINE_KWARGS of
"BitDecoding-FP4 evaluation/config.py") of one KV head; each token row has
128 head-dim elements. The pages fix only the logical content (E2M1 codes,
one scale per 16 elements for NVFP4 or per 32 for MXFP4). The byte order
inside a page is this library's own format; it is stated here as plain index
maps and is the same one the C-ABI header documents. Each cache tensor is a
dense array [num_pages, num_kv_heads, bytes_per_page_head]; the block of page
p, head h starts at (p * num_kv_heads + h) * bytes_per_page_head.

Codes: two 4-bit codes per byte; which two, and which goes in bits 3..0,
depends on the array.

K codes (8192 B per page-head), token t, element d (element d even in bits 3..0):
    byte = (t >> 4) * 1024 + (d >> 5) * 256 + (t & 15) * 16 + ((d & 31) >> 1)
V codes, NVFP4 (8192 B): a byte holds tokens t and t+1 (t even, in bits 3..0)
of one element d:
    byte = (t >> 5) * 2048 + (((t >> 3) & 3) * 16 + (d >> 3)) * 32 + (d & 7) * 4 + ((t & 7) >> 1)
V codes, MXFP4 (8192 B), element d even in bits 3..0:
    byte = ((((t >> 5) * 4 + ((t >> 3) & 3)) * 16 + (d >> 3)) * 8 + (t & 7)) * 4 + ((d & 7) >> 1)
NVFP4 K scales (1024 B), token t, 16-block j (0..7):
    byte = (((j >> 1) * 16 + (t & 15)) * 8 + (t >> 4)) * 2 + (j & 1)
MXFP4 K scales (512 B), token t, 32-block j (0..3):
    byte = (j * 16 + (t & 15)) * 8 + (t >> 4)
NVFP4 K scales of the channel geometry (1024 B), token block b = t >> 4 (0..7), channel c:
    byte = b * 128 + c
NVFP4 V scales (1024 B), token t, block j (0..7):
    byte = (((t >> 5) * 4 + ((t >> 3) & 3)) * 8 + j) * 8 + (t & 7)
MXFP4 V scales (512 B), token t, block j (0..3):
    byte = (((t >> 5) * 4 + ((t >> 3) & 3)) * 4 + j) * 8 + (t & 7)
"""
from __future__ import annotations

import numpy as np

PAGE = 128
D = 128
CODE_BYTES = PAGE * D // 2  # 8192


def scale_bytes(mx: bool) -> int:
    return PAGE * (D // 32 if mx else D // 16)


def k_code_byte(t, d):
    return (t >> 4) * 1024 + (d >> 5) * 256 + (t & 15) * 16 + ((d & 31) >> 1)


def v_code_byte(t, d, mx: bool):
    if mx:
        return ((((t >> 5) * 4 + ((t >> 3) & 3)) * 16 + (d >> 3)) * 8 + (t & 7)) * 4 + ((d & 7) >> 1)
    return (t >> 5) * 2048 + (((t >> 3) & 3) * 16 + (d >> 3)) * 32 + (d & 7) * 4 + ((t & 7) >> 1)


def _code_map(which: str, mx: bool):
    """(byte index, bit shift) of every (token, element) of a page-head."""
    t = np.arange(PAGE)[:, None]
    d = np.arange(D)[None, :]
    if which == "k":
        byte, hi = k_code_byte(t, d), d & 1
    elif mx:
        byte, hi = v_code_byte(t, d, True), d & 1
    else:
        byte, hi = v_code_byte(t, d, False), t & 1
    return (np.broadcast_to(byte, (PAGE, D)).reshape(-1),
            np.broadcast_to(hi * 4, (PAGE, D)).reshape(-1).astype(np.uint8))


def k_scale_byte(t, j, mx: bool):
    if mx:
        return (j * 16 + (t & 15)) * 8 + (t >> 4)
    return (((j >> 1) * 16 + (t & 15)) * 8 + (t >> 4)) * 2 + (j & 1)


def k_scale_byte_channel(b, c):
    """K scale of token block b (16 tokens) and channel c, channel geometry."""
    return b * 128 + c


def pack_k_scales_channel(sc: np.ndarray) -> np.ndarray:
    """sc: uint8 [..., 8 token blocks, 128 channels] -> bytes [..., 1024]."""
    sc = np.asarray(sc, dtype=np.uint8)
    assert sc.shape[-2:] == (PAGE // 16, D)
    b = np.arange(PAGE // 16)[:, None]
    c = np.arange(D)[None, :]
    out = np.zeros(sc.shape[:-2] + (scale_bytes(False),), dtype=np.uint8)
    out[..., k_scale_byte_channel(b, c).reshape(-1)] = sc.reshape(sc.shape[:-2] + (-1,))
    return out


def unpack_k_scales_channel(buf: np.ndarray) -> np.ndarray:
    buf = np.asarray(buf, dtype=np.uint8)
    b = np.arange(PAGE // 16)[:, None]
    c = np.arange(D)[None, :]
    return buf[..., k_scale_byte_channel(b, c)].astype(np.uint8)


def v_scale_byte(t, j, mx: bool):
    if mx:
        return (((t >> 5) * 4 + ((t >> 3) & 3)) * 4 + j) * 8 + (t & 7)
    return (((t >> 5) * 4 + ((t >> 3) & 3)) * 8 + j) * 8 + (t & 7)


def pack_codes(nib: np.ndarray, which: str, mx: bool = False) -> np.ndarray:
    """nib: uint8 [..., 128 tokens, 128 elements] (4-bit codes) -> bytes [..., 8192]."""
    nib = np.asarray(nib, dtype=np.uint8)
    lead = nib.shape[:-2]
    out = np.zeros(lead + (CODE_BYTES,), dtype=np.uint8)
    flat_b, flat_s = _code_map(which, mx)
    vals = (nib.reshape(lead + (PAGE * D,)) & 0xF) << flat_s
    # every byte receives exactly two nibbles, one at shift 0 and one at shift 4
    for sh in (0, 4):
        sel = flat_s == sh
        out[..., flat_b[sel]] |= vals[..., sel].astype(np.uint8)
    return out


def unpack_codes(buf: np.ndarray, which: str, mx: bool = False) -> np.ndarray:
    """bytes [..., 8192] -> nibbles [..., 128 tokens, 128 elements]."""
    buf = np.asarray(buf, dtype=np.uint8)
    flat_b, flat_s = _code_map(which, mx)
    return ((buf[..., flat_b] >> flat_s) & 0xF).astype(np.uint8).reshape(buf.shape[:-1] + (PAGE, D))


def pack_scales(sc: np.ndarray, which: str, mx: bool) -> np.ndarray:
    """sc: uint8 [..., 128 tokens, nblocks] -> bytes [..., scale_bytes(mx)]."""
    sc = np.asarray(sc, dtype=np.uint8)
    nb = D // (32 if mx else 16)
    assert sc.shape[-1] == nb and sc.shape[-2] == PAGE
    lead = sc.shape[:-2]
    out = np.zeros(lead + (scale_bytes(mx),), dtype=np.uint8)
    t = np.arange(PAGE)[:, None]
    j = np.arange(nb)[None, :]
    fn = k_scale_byte if which == "k" else v_scale_byte
    byte = np.broadcast_to(fn(t, j, mx), (PAGE, nb))
    out[..., byte.reshape(-1)] = sc.reshape(lead + (PAGE * nb,))
    return out


def unpack_scales(buf: np.ndarray, which: str, mx: bool) -> np.ndarray:
    buf = np.asarray(buf, dtype=np.uint8)
    nb = D // (32 if mx else 16)
    t = np.arange(PAGE)[:, None]
    j = np.arange(nb)[None, :]
    fn = k_scale_byte if which == "k" else v_scale_byte
    byte = np.broadcast_to(fn(t, j, mx), (PAGE, nb))
    return buf[..., byte].astype(np.uint8)
