"""Decode-time append with freeze-at-fill.

Oracle module (test infrastructure only; see the package docstring).

"kv-landlords scripts/quant_ab.py", module docstring and PageSim: new tokens
go to a hot page kept in BF16; a page is quantized once, when it fills, and
then stays frozen. "BitDecoding-FP4 evaluation/config.py", KV_MODES
("sink_tokens": 16, "block_size": 128 in PARITY_ENGINE_KWARGS): the first 16
tokens of a sequence are also kept in BF16 for good. "How
openbitsys/bitdecoding-fp4 works" (gitdiagram), Components: the KV cache
writer hands full pages to KV quantization.

Readings (the pages give the policy, not the buffers):

* the hot page of sequence b is the tail buffer [Hkv, 128, 128]; the token at
  position pos lands in slot pos mod 128 (sink tokens too, because page 0 is
  quantized whole when it fills, sink slots included);
* a token with pos < sink_tokens is also stored in the sink buffer at pos;
* the token that fills slot 127 freezes the page: the 128 tail rows are
  quantized exactly as the page writer quantizes a whole page (writer.py),
  into physical page block_tables[b, pos // 128];
* rows with pos < 0 (padding) or pos >= 128 * max_pages_per_seq are skipped;
  a destination page outside the pool is skipped while the tail is still
  written (as the page writer skips such pages).
"""
from __future__ import annotations

import numpy as np

from . import layout
from .recipe import Recipe
from .writer import write_pages


def append_tokens(recipe: Recipe, cache: dict, tail_k: np.ndarray, tail_v: np.ndarray,
                  sink_k, sink_v, k_new: np.ndarray, v_new: np.ndarray, positions,
                  block_tables: np.ndarray, key_shift=None) -> None:
    """Append one token per sequence (in place).

    tail_k/v: uint16 bf16 [B, Hkv, 128, 128]; sink_k/v: uint16 [B, Hkv, S, 128]
    (None when S = 0); k_new/v_new: uint16 [B, Hkv, 128]; positions: int [B];
    block_tables: int32 [B, max_pages_per_seq]; cache as writer.empty_cache."""
    num_pages = cache["k_codes"].shape[0]
    max_pages = block_tables.shape[1]
    for b in range(k_new.shape[0]):
        pos = int(positions[b])
        if pos < 0 or pos >= layout.PAGE * max_pages:
            continue
        slot = pos % layout.PAGE
        tail_k[b, :, slot] = k_new[b]
        tail_v[b, :, slot] = v_new[b]
        if pos < recipe.sink_tokens:
            sink_k[b, :, pos] = k_new[b]
            sink_v[b, :, pos] = v_new[b]
        if slot == layout.PAGE - 1:
            page = int(block_tables[b, pos // layout.PAGE])
            if 0 <= page < num_pages:
                # tail [Hkv, tok, d] -> the writer's page rows [tok, Hkv, d]
                write_pages(recipe, cache, tail_k[b].transpose(1, 0, 2), tail_v[b].transpose(1, 0, 2),
                            [page], key_shift)
