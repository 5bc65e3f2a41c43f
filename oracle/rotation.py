"""128-point Hadamard rotation of key and query rows.

Oracle module (test infrastructure only; see the package docstring).

"BitDecoding-FP4 evaluation/config.py" turns on
``outlier_aware_key_quantization.hadamard_rotation`` in RECIPE, which
``recipe_additional_config`` maps to ``nvfp4_rotation: "hadamard"``; the
``bitdecoding-mxfp4`` entry of KV_MODES fixes ``rotation: "hadamard"``. The
page gives no matrix, order or normalisation. Reading taken here:

* the Sylvester-ordered Hadamard matrix of order 128,
  H[i][j] = (-1)**popcount(i & j), normalised by 1/sqrt(128) so that the
  rotation is orthonormal and q.k is preserved when both sides are rotated;
* evaluated as the fast Walsh-Hadamard transform in float32: stages
  h = 1, 2, 4, ..., 64, each replacing the pair (x[i], x[i+h]) (i with bit h
  clear) by (x[i] + x[i+h], x[i] - x[i+h]), every add/sub rounded to float32;
  then one float32 multiply by float32(1/sqrt(128)).

Because every output of a stage is one rounded operation on two outputs of
the previous stage, this fixes the float32 result bit for bit.
"""
from __future__ import annotations

import numpy as np

D = 128
#: float32 nearest to 1/sqrt(128)
INV_SQRT_D = np.float32(1.0 / np.sqrt(128.0))


def hadamard_matrix(n: int = D) -> np.ndarray:
    """Integer Sylvester Hadamard matrix, H[i][j] = (-1)**popcount(i & j)."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    bits = np.bitwise_and(i, j)
    pop = np.zeros_like(bits)
    b = bits.copy()
    while np.any(b):
        pop += b & 1
        b >>= 1
    return np.where(pop % 2 == 0, 1, -1).astype(np.int64)


def fwht(x: np.ndarray) -> np.ndarray:
    """Unnormalised fast Walsh-Hadamard transform over the last axis (128),
    float32 throughout, stage order h = 1, 2, ..., 64."""
    y = np.array(x, dtype=np.float32, copy=True)
    n = y.shape[-1]
    assert n == D
    lead = y.shape[:-1]
    h = 1
    while h < n:
        blocks = y.reshape(lead + (n // (2 * h), 2, h))
        a = blocks[..., 0, :]
        b = blocks[..., 1, :]
        s = (a + b).astype(np.float32)
        d = (a - b).astype(np.float32)
        y = np.stack([s, d], axis=-2).reshape(lead + (n,))
        h *= 2
    return y


def rotate(x: np.ndarray) -> np.ndarray:
    """Normalised rotation: fwht(x) * float32(1/sqrt(128)), in float32."""
    return (fwht(x) * INV_SQRT_D).astype(np.float32)
