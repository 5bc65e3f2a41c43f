"""Oracle pins for the quantization diagnostics (CPU only).

* pages whose values lie on the quantization grid (codes times scales, key
  rotation and centering off) have zero error and the exact reference sums;
* doubling K, V and the key means doubles every quantized value exactly
  (scales double, codes stay), so every sum grows by exactly 4;
* a page outside the pool contributes nothing.
"""
import numpy as np

from oracle import diagnostics as DG
from oracle import quant as Q
from oracle import recipe as RC
from oracle import writer as W

PAGE, D = 128, 128
GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _bf16(x):
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def test_on_grid_pages_have_zero_error():
    rng = np.random.default_rng(4)
    r = RC.nvfp4_default().with_(tau=1.0, rotation=False, key_smoothing=False, scale_mode_k=Q.AMAX6)
    n, hkv = 2, 2
    # each 16-block: one element 6 (fixes the amax6 scale to 1 * 2^e), the rest on the grid
    def grid_rows():
        g = rng.choice(GRID, size=(n * PAGE, hkv, D)) * rng.choice([-1.0, 1.0], size=(n * PAGE, hkv, D))
        g[..., ::16] = 6.0
        return g * 2.0 ** rng.integers(-3, 4, size=(n * PAGE, hkv, 1))
    k, v = grid_rows(), grid_rows()
    kb, vb = _bf16(k), _bf16(v)
    cache = W.empty_cache(4, hkv, r)
    W.write_pages(r, cache, kb, vb, [3, 1])
    e = DG.page_errors(r, cache, kb, vb, [3, 1])
    assert e[0] == 0.0 and e[2] == 0.0
    assert e[1] == np.sum(k.astype(np.float64) ** 2) and e[3] == np.sum(v.astype(np.float64) ** 2)


def test_scaling_by_two_scales_sums_by_four_and_foreign_pages_are_skipped():
    rng = np.random.default_rng(5)
    r = RC.nvfp4_default().with_(tau=1.0)
    n, hkv = 2, 1
    k = rng.standard_normal((n * PAGE, hkv, D)).astype(np.float32) * 0.5
    v = rng.standard_normal((n * PAGE, hkv, D)).astype(np.float32) * 0.5
    mu = rng.standard_normal((hkv, D)).astype(np.float32) * 0.25
    kb, vb, kb2, vb2 = _bf16(k), _bf16(v), _bf16(2 * k), _bf16(2 * v)
    c1, c2 = W.empty_cache(3, hkv, r), W.empty_cache(3, hkv, r)
    W.write_pages(r, c1, kb, vb, [0, 2], mu)
    W.write_pages(r, c2, kb2, vb2, [0, 2], 2 * mu)
    e1 = DG.page_errors(r, c1, kb, vb, [0, 2], mu)
    e2 = DG.page_errors(r, c2, kb2, vb2, [0, 2], 2 * mu)
    assert np.all(e1 > 0) and np.array_equal(e2, 4 * e1)
    # the second input page aimed outside the pool: only the first counts
    e_first = DG.page_errors(r, c1, kb[:PAGE], vb[:PAGE], [0], mu)
    assert np.array_equal(DG.page_errors(r, c1, kb, vb, [0, 7], mu), e_first)
