"""Calibration drivers: the key means mu and the tau search.

Oracle module (test infrastructure only; see the package docstring).

"BitDecoding-FP4 evaluation/config.py": RECIPE outlier_aware_key_quantization
turns on key smoothing with a static per-channel key shift (the module
docstring's K centering, and the comment that the runner creates missing key
means, i.e. a calibration pass over activations); probability_environment
refuses tau "calibrate" outside calibration, so tau is searched before use.
The pages state neither the statistic nor the search objective. Readings:

* mu[h, c] = float32 of the mean, taken in float64, of float32(K[t, h, c])
  over the calibration tokens t (the mean is the plainest "key mean");
* tau: over a caller-given candidate grid, the value whose FP4 decode output
  has the smallest relative L2 error against exact attention over the BF16
  keys and values of the same calibration workload; ties keep the earlier
  candidate. Parity unpinned with respect to the pages' own objective (they
  state none): the pins below check the search's mechanics, not its target.
"""
from __future__ import annotations

import numpy as np

from .decode import decode
from .formats import bf16_to_f32


def key_means(k_bf16: np.ndarray) -> np.ndarray:
    """k_bf16: uint16 [T, Hkv, 128] calibration keys -> float32 [Hkv, 128]."""
    x = bf16_to_f32(k_bf16).astype(np.float64)
    # the plain sum 0 + x_0 + x_1 + ...: it starts from +0.0
    return (x.sum(axis=0, initial=0.0) / x.shape[0]).astype(np.float32)


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.linalg.norm(np.asarray(got, np.float64) - ref) / np.linalg.norm(ref))


def tau_search(recipe, candidates, cache, q, block_tables, seq_lens, sink_k, sink_v, tail_k, tail_v,
               key_shift, sigma, pages_per_partition, reference):
    """Returns (best tau, [error per candidate]); reference = the exact
    attention output (decode.bf16_decode over the same tokens)."""
    errs = []
    for t in candidates:
        out = decode(recipe.with_(tau=float(t)), cache, q, block_tables, seq_lens, sink_k, sink_v,
                     tail_k, tail_v, key_shift, sigma, pages_per_partition)
        errs.append(rel_l2(out, reference))
    best = int(np.argmin(errs))          # the first of equal minima
    return float(candidates[best]), errs
