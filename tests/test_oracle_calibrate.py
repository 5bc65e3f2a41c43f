"""Oracle pins for the calibration drivers (CPU only).

* key means: an arithmetic progression of exactly representable keys has the
  closed-form mean a + d (T - 1) / 2; a constant channel has its own value;
* tau search: one candidate is returned as is; candidates that cannot change
  any P scale (all at or below every block maximum, so every block takes
  amax6 - the disabled-mode setting) give identical errors and the first
  wins; tau = 0 reproduces the amax6 P mode exactly.
"""
import numpy as np

from fp4_kv_cache_nvfp4_amd import synth
from oracle import calibrate as OC
from oracle import decode as OD
from oracle import quant as Q
from oracle import recipe as RC

from gpu_helpers import oracle_write


def test_key_means_closed_forms():
    T, hkv = 1000, 2
    t = np.arange(T)
    x = np.zeros((T, hkv, 128), dtype=np.float32)
    x[:, 1, :] = 1.5                                  # constant channel: its own value
    x[:, 0, 7] = 0.5 * (t % 4)                        # period 4 over 1000 tokens: mean 0.75
    x[:, 0, 9] = np.where(t < 10, 100.0, 0.0)         # one burst: 10 * 100 / 1000 = 1
    u = synth.f32_to_bf16(x)
    assert np.array_equal(synth.bf16_to_f32(u), x)    # every value exact in bf16
    mu = OC.key_means(u)
    assert mu[0, 7] == np.float32(0.75) and mu[0, 9] == np.float32(1.0) and mu[0, 0] == 0.0
    assert np.all(mu[1] == np.float32(1.5))


def test_key_means_progression_exact():
    # small integers and halves are exact in bf16: a = -2, d = 0.5, T = 200
    T = 200
    t = np.arange(T, dtype=np.float32)
    x = np.broadcast_to((-2.0 + 0.5 * t)[:, None, None], (T, 1, 128)).astype(np.float32)
    u = synth.f32_to_bf16(x)
    assert np.array_equal(synth.bf16_to_f32(u), x)
    assert np.all(OC.key_means(u) == np.float32(-2.0 + 0.5 * (T - 1) / 2))


def _small():
    wl = synth.decode_workload("cal", 5, [3 * 128 + 40], 8, 2, "qwen")
    return wl


def _args(r, wl):
    cache = oracle_write(r, wl)
    sk, sv, tk, tv = wl.sink_tail()
    return (cache, wl.q, wl.block_tables, wl.seq_lens, sk, sv, tk, tv, wl.key_shift, wl.sigma, 1)


def test_tau_search_mechanics():
    wl = _small()
    r = RC.nvfp4_default().with_(tau=1.0)
    args = _args(r, wl)
    kp, vp = wl.bf16_pages()
    ref = OD.bf16_decode(wl.q, kp, vp, wl.block_tables, wl.seq_lens, wl.sigma)
    best, errs = OC.tau_search(r, [0.5], *args, ref)
    assert best == 0.5 and len(errs) == 1 and 0.0 < errs[0] < 0.5
    # p' = c p <= c = 8 and every block holds a token of p' >= c e^(sigma (t - m)) > 0;
    # tau values at or below 0 never select amax2: all equal, the first wins
    best, errs = OC.tau_search(r, [0.0, -0.0], *args, ref)
    assert best == 0.0 and errs[0] == errs[1]
    # tau = 0 is exactly the amax6 P mode
    a = OD.decode(r.with_(tau=0.0), *args)
    b = OD.decode(r.with_(scale_mode_p=Q.AMAX6), *args)
    assert np.array_equal(a, b)
