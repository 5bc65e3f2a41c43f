"""KV page writer: key centering, rotation, block quantization, page packing.

Oracle module (test infrastructure only; see the package docstring).

"How openbitsys/bitdecoding-fp4 works" (gitdiagram), Components and
Connections: the KV cache writer quantizes pages through KV quantization,
which uses block scaling and scale modes. "kv-landlords scripts/quant_ab.py",
module docstring and PageSim: a page is quantized once when it fills and kept
frozen; the partial hot page stays BF16. So the writer takes whole 128-token
pages only.

Key path (readings, from "BitDecoding-FP4 evaluation/config.py": RECIPE
outlier_aware_key_quantization, the module docstring's "K centering" and
the comment that the runner creates missing key means):

    x = float32(k) - mu            (static per-channel key mean, float32)
    y = rotate(x)                  (Hadamard; see rotation.py)
    codes, scales = quantize(y, scale_mode_k)

With the channel key scale geometry (KV_MODES key_scale_geometry; quant_ab.py
SCHEMES per-channel keys) the same y is quantized in blocks of 16 tokens of
one channel instead of 16 channels of one token; its scales are stored
[token block][channel].

Value path: codes, scales = quantize(float32(v), scale_mode_v); the rotation
is listed under key quantization only, so values are not rotated - except in
the rotate_v recipe variant (the alternative reading: rotate V as well and
rotate the attention output back), where v is rotated like a key (no
centering) before quantization.
"""
from __future__ import annotations

import numpy as np

from . import layout
from . import quant as Q
from .formats import bf16_to_f32
from .recipe import CHANNEL, Recipe
from .rotation import rotate


def key_rows(k_f32: np.ndarray, mu, rotation: bool) -> np.ndarray:
    """Centered, rotated float32 key rows (the values that get quantized)."""
    x = np.asarray(k_f32, dtype=np.float32)
    if mu is not None:
        x = (x - np.asarray(mu, dtype=np.float32)).astype(np.float32)
    return rotate(x) if rotation else x


def quantize_k_rows(k_f32, mu, rotation: bool, mode: str):
    return Q.quantize(key_rows(k_f32, mu, rotation), mode)


def quantize_k_page_channel(y: np.ndarray, mode: str):
    """Channel key geometry: y [..., 128 tokens, 128 channels] float32 (the
    centered, rotated keys of whole pages). Every channel's column is cut into
    8 blocks of 16 consecutive tokens, each quantized with the key scale mode
    exactly as a 16-channel block would be. Returns (nibbles [..., tok, ch],
    e4m3 codes [..., 8 token blocks, ch])."""
    y = np.asarray(y, dtype=np.float32)
    cols = np.swapaxes(y, -1, -2)                 # [..., ch, tok]
    nib, sc = Q.quantize(cols, mode)              # blocks of 16 along tokens
    return np.swapaxes(nib, -1, -2), np.swapaxes(sc, -1, -2)


def value_rows(v_f32, rotate_v: bool) -> np.ndarray:
    """The float32 value rows that get quantized."""
    x = np.asarray(v_f32, dtype=np.float32)
    return rotate(x) if rotate_v else x


def quantize_v_rows(v_f32, mode: str, rotate_v: bool = False):
    return Q.quantize(value_rows(v_f32, rotate_v), mode)


def empty_cache(num_pages: int, num_kv_heads: int, recipe: Recipe) -> dict:
    kmx = recipe.scale_mode_k == Q.MXFP4_SEARCH
    vmx = recipe.scale_mode_v == Q.MXFP4_SEARCH
    z = lambda n: np.zeros((num_pages, num_kv_heads, n), dtype=np.uint8)
    return {
        "k_codes": z(layout.CODE_BYTES), "k_scales": z(layout.scale_bytes(kmx)),
        "v_codes": z(layout.CODE_BYTES), "v_scales": z(layout.scale_bytes(vmx)),
    }


def write_pages(recipe: Recipe, cache: dict, k_bf16: np.ndarray, v_bf16: np.ndarray,
                page_ids, key_shift=None) -> dict:
    """Quantize n whole pages into the cache (in place; also returned).

    k_bf16, v_bf16: uint16 bf16 patterns [n*128, Hkv, 128], page i holding
    rows [128 i, 128 i + 128); page_ids: destination physical pages [n];
    key_shift: float32 [Hkv, 128] key means (required when key_smoothing)."""
    page_ids = np.asarray(page_ids, dtype=np.int64)
    n = page_ids.shape[0]
    k = bf16_to_f32(k_bf16).reshape(n, layout.PAGE, -1, layout.D)
    v = bf16_to_f32(v_bf16).reshape(n, layout.PAGE, -1, layout.D)
    hkv = k.shape[2]
    mu = None
    if recipe.key_smoothing:
        if key_shift is None:
            raise ValueError("key smoothing needs key means")
        mu = np.asarray(key_shift, dtype=np.float32).reshape(1, 1, hkv, layout.D)
    kmx = recipe.scale_mode_k == Q.MXFP4_SEARCH
    vmx = recipe.scale_mode_v == Q.MXFP4_SEARCH
    vn, vs = quantize_v_rows(v, recipe.scale_mode_v, recipe.rotate_v)
    if recipe.key_scale_geometry == CHANNEL:
        y = key_rows(k, mu, recipe.rotation).transpose(0, 2, 1, 3)     # [n, h, tok, ch]
        kn, ks = quantize_k_page_channel(y, recipe.scale_mode_k)
        cache["k_scales"][page_ids] = layout.pack_k_scales_channel(ks)
    else:
        kn, ks = quantize_k_rows(k, mu, recipe.rotation, recipe.scale_mode_k)
        # [n, tok, h, ...] -> [n, h, tok, ...]
        kn = kn.transpose(0, 2, 1, 3)
        cache["k_scales"][page_ids] = layout.pack_scales(ks.transpose(0, 2, 1, 3), "k", kmx)
    vn = vn.transpose(0, 2, 1, 3)
    vs = vs.transpose(0, 2, 1, 3)
    cache["k_codes"][page_ids] = layout.pack_codes(kn, "k")
    cache["v_codes"][page_ids] = layout.pack_codes(vn, "v", vmx)
    cache["v_scales"][page_ids] = layout.pack_scales(vs, "v", vmx)
    return cache


def read_page_head(recipe: Recipe, cache: dict, page: int, head: int):
    """Dequantized (k_hat, v_hat) of one page-head, float64 [128, 128] each,
    in the quantized domain (keys centered and rotated; values rotated in the
    rotate_v variant)."""
    kmx = recipe.scale_mode_k == Q.MXFP4_SEARCH
    vmx = recipe.scale_mode_v == Q.MXFP4_SEARCH
    kn = layout.unpack_codes(cache["k_codes"][page, head], "k")
    vn = layout.unpack_codes(cache["v_codes"][page, head], "v", vmx)
    vs = layout.unpack_scales(cache["v_scales"][page, head], "v", vmx)
    if recipe.key_scale_geometry == CHANNEL:
        ks = layout.unpack_k_scales_channel(cache["k_scales"][page, head])     # [8, 128]
        k_hat = Q.dequantize(kn.T, ks.T, recipe.scale_mode_k).T                # blocks along tokens
    else:
        ks = layout.unpack_scales(cache["k_scales"][page, head], "k", kmx)
        k_hat = Q.dequantize(kn, ks, recipe.scale_mode_k)
    return k_hat, Q.dequantize(vn, vs, recipe.scale_mode_v)
