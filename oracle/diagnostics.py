"""Quantization diagnostics: squared errors of stored pages.

Oracle module (test infrastructure only; see the package docstring).

"kv-landlords scripts/quant_ab.py" compares KV-cache quantization schemes by
their reconstruction error and memory ("BitDecoding-FP4 evaluation/config.py"
lists the recipe ablations: rotation, key smoothing, K four_six vs amax6,
query terms, c). Reading: the error of a page is measured in the domain it
was quantized in - keys centered and rotated (what the codes approximate),
values as stored (rotated in the rotate_v variant) - as float64 sums over every element of the written pages:

    [sum (k_hat - y)^2, sum y^2, sum (v_hat - v)^2, sum v^2]

so RMSE = sqrt(err / n) and relative error = sqrt(err / ref) follow.
Pages whose destination lies outside the pool are skipped, as the writer
skips them.
"""
from __future__ import annotations

import numpy as np

from . import layout
from .formats import bf16_to_f32
from .recipe import Recipe
from .writer import key_rows, read_page_head, value_rows


def page_errors(recipe: Recipe, cache: dict, k_bf16: np.ndarray, v_bf16: np.ndarray, page_ids,
                key_shift=None) -> np.ndarray:
    """k_bf16, v_bf16: uint16 [n*128, Hkv, 128] (the writer's input rows);
    page_ids [n]. Returns float64 [4]."""
    page_ids = np.asarray(page_ids, dtype=np.int64)
    n = page_ids.shape[0]
    num_pages = cache["k_codes"].shape[0]
    k = bf16_to_f32(k_bf16).reshape(n, layout.PAGE, -1, layout.D)
    v = bf16_to_f32(v_bf16).reshape(n, layout.PAGE, -1, layout.D)
    hkv = k.shape[2]
    out = np.zeros(4)
    for i in range(n):
        p = int(page_ids[i])
        if p < 0 or p >= num_pages:
            continue
        for h in range(hkv):
            mu = None if key_shift is None or not recipe.key_smoothing else np.asarray(key_shift)[h]
            y = key_rows(k[i, :, h], mu, recipe.rotation).astype(np.float64)
            kh, vh = read_page_head(recipe, cache, p, h)
            vv = value_rows(v[i, :, h], recipe.rotate_v).astype(np.float64)
            out += [np.sum((kh - y) ** 2), np.sum(y ** 2), np.sum((vh - vv) ** 2), np.sum(vv ** 2)]
    return out
