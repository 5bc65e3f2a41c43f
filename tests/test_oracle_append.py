"""Oracle pins for decode-time append with freeze-at-fill (CPU only).

* appending a sequence one token at a time leaves the cache exactly as the
  bulk page writer leaves it for the same full pages, the sink holding the
  first sink_tokens tokens and every tail slot j the last token whose
  position is j mod 128;
* padding rows (position < 0), positions past the block table and
  destination pages outside the pool change what the reading says they change
  and nothing else.
"""
import numpy as np

from oracle import append as OA
from oracle import recipe as RC
from oracle import writer as W

PAGE, D = 128, 128


def _tokens(rng, n, hkv):
    x = rng.standard_normal((n, hkv, D)).astype(np.float32)
    x[:, :, 5] += 6.0                              # an outlier channel, as keys have
    u = x.view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def _state(B, hkv, S, num_pages):
    tk = np.zeros((B, hkv, PAGE, D), dtype=np.uint16)
    sk = np.zeros((B, hkv, S, D), dtype=np.uint16) if S else None
    return tk, tk.copy(), sk, (sk.copy() if S else None)


def test_append_one_by_one_equals_bulk_writer():
    rng = np.random.default_rng(11)
    r = RC.nvfp4_default().with_(tau=1.0)
    hkv, lens = 2, [3 * PAGE + 37, PAGE + 5]
    num_pages, max_pages = 9, 5
    bt = np.full((2, max_pages), -1, dtype=np.int32)
    perm = rng.permutation(num_pages).astype(np.int32)
    bt[0, :4], bt[1, :2] = perm[:4], perm[4:6]
    k = [_tokens(rng, L, hkv) for L in lens]
    v = [_tokens(rng, L, hkv) for L in lens]
    mu = rng.standard_normal((hkv, D)).astype(np.float32)
    cache = W.empty_cache(num_pages, hkv, r)
    tk, tv, sk, sv = _state(2, hkv, r.sink_tokens, num_pages)
    for step in range(max(lens)):
        pos = np.array([step if step < L else -1 for L in lens])
        kn = np.stack([k[b][min(step, lens[b] - 1)] for b in range(2)])
        vn = np.stack([v[b][min(step, lens[b] - 1)] for b in range(2)])
        OA.append_tokens(r, cache, tk, tv, sk, sv, kn, vn, pos, bt, mu)

    want = W.empty_cache(num_pages, hkv, r)
    for b, L in enumerate(lens):
        n = L // PAGE
        W.write_pages(r, want, k[b][:n * PAGE], v[b][:n * PAGE], bt[b, :n], mu)
    for name in want:
        assert np.array_equal(cache[name], want[name]), name
    for b, L in enumerate(lens):
        n, rem = divmod(L, PAGE)
        for j in range(PAGE):
            t = n * PAGE + j if j < rem else (n - 1) * PAGE + j   # last token written to slot j
            assert np.array_equal(tk[b, :, j], k[b][t]) and np.array_equal(tv[b, :, j], v[b][t])
        assert np.array_equal(sk[b], k[b][:16].transpose(1, 0, 2))
        assert np.array_equal(sv[b], v[b][:16].transpose(1, 0, 2))


def test_append_skips_padding_past_table_and_foreign_pages():
    rng = np.random.default_rng(12)
    r = RC.mxfp4_default().with_(tau=1.0, sink_tokens=0)
    hkv, num_pages = 1, 4
    cache = W.empty_cache(num_pages, hkv, r)
    tk, tv, sk, sv = _state(3, hkv, 0, num_pages)
    # seq 0: its page slot names a page outside the pool; seq 1: padding;
    # seq 2: position past its one-page block table
    bt = np.array([[num_pages], [0], [1]], dtype=np.int32)
    k = _tokens(rng, PAGE, hkv)
    for step in range(PAGE):
        kn = np.stack([k[step]] * 3)
        OA.append_tokens(r, cache, tk, tv, sk, sv, kn, kn, np.array([step, -1, PAGE + step]), bt, None)
    assert all(not c.any() for c in cache.values())          # nothing frozen anywhere
    assert np.array_equal(tk[0, 0], k[:, 0])                    # but seq 0's tail is written
    assert not tk[1].any() and not tk[2].any()
