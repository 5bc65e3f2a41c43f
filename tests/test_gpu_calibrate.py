"""Calibration kernels through the C ABI against the oracle: key means
bit-identical with the oracle's float64 means (ragged chunk tail, and the
full 131,072-token x 8-head prefill); error sums against float64 sums; the
tau search on the device reporting the oracle's per-candidate errors and its
choice."""
import numpy as np
import pytest
import torch

import fp4_kv_cache_nvfp4_amd as bd
from fp4_kv_cache_nvfp4_amd import synth
from oracle import calibrate as OC
from oracle import decode as OD
from oracle import recipe as RC

from gpu_helpers import dev, dev_bf16, gpu_write, oracle_write, to_c

pytestmark = pytest.mark.gpu


def _u16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("tokens,hkv", [(1, 1), (50_000, 3)])
def test_key_means_bit_exact(tokens, hkv):
    rng = np.random.default_rng(tokens)
    x = rng.standard_normal((tokens, hkv, 128)).astype(np.float32)
    x[:, :, 11] += 9.0                                  # an outlier channel with a large mean
    x[:, 0, 20] = -0.0                                  # zeros of either sign sum to +0.0
    x[:, 0, 21] = 0.0
    k = synth.f32_to_bf16(x)
    mu = bd.key_means(dev_bf16(k), hkv)
    torch.cuda.synchronize()
    want = OC.key_means(k)
    assert not np.signbit(want[0, 20]) and not np.signbit(want[0, 21])
    assert np.array_equal(mu.cpu().numpy().view(np.uint32), want.view(np.uint32))


def test_key_means_full_prefill_bit_exact():
    w = synth.torch_write_rows(0)                       # 131,072 tokens x 8 heads, on the device
    mu = bd.key_means(w["k"], 8)
    torch.cuda.synchronize()
    assert np.array_equal(mu.cpu().numpy().view(np.uint32), OC.key_means(_u16(w["k"])).view(np.uint32))


def test_error_sums_match_float64():
    rng = np.random.default_rng(2)
    for n in (0, 1, 4097, 300_000):
        a = rng.standard_normal(n).astype(np.float32)
        b = rng.standard_normal(n).astype(np.float32)
        out = torch.zeros(2, dtype=torch.float64, device="cuda")
        bd.error_sums(dev(a), dev(b), out)
        got = out.cpu().numpy()
        want = np.array([np.sum((a.astype(np.float64) - b) ** 2), np.sum(b.astype(np.float64) ** 2)])
        assert np.allclose(got, want, rtol=1e-12, atol=0.0), (n, got, want)


def test_tau_search_matches_oracle():
    wl = synth.decode_workload("cal", 5, [3 * 128 + 40, 2 * 128 + 3], 8, 2, "qwen")
    r = RC.nvfp4_default().with_(tau=1.0)
    rc = to_c(r)
    cands = [0.0, 0.125, 0.5, 1.0, 2.0, 4.0, 8.0]
    # oracle
    ocache = oracle_write(r, wl)
    sk, sv, tk, tv = wl.sink_tail()
    kp, vp = wl.bf16_pages()
    ref = OD.bf16_decode(wl.q, kp, vp, wl.block_tables, wl.seq_lens, wl.sigma)
    o_best, o_errs = OC.tau_search(r, cands, ocache, wl.q, wl.block_tables, wl.seq_lens, sk, sv, tk, tv,
                                   wl.key_shift, wl.sigma, 1, ref)
    # device: reference from the BF16-KV decode, the search from the FP4 decode
    B, Hq, msl = wl.batch, wl.num_q_heads, int(wl.seq_lens.max())
    q, bt, sl = dev_bf16(wl.q), dev(wl.block_tables), dev(wl.seq_lens)
    ws = bd.alloc_workspace(bd.decode_workspace_size(B, Hq, wl.num_kv_heads, msl, 1))
    gref = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")
    bd.bf16_decode_attention(q, dev_bf16(kp), dev_bf16(vp), bt, sl, msl, wl.sigma, 1, ws, gref)
    args = dict(cache=gpu_write(r, wl), q=q, block_tables=bt, seq_lens=sl, max_seq_len=msl,
                sink_k=dev_bf16(sk), sink_v=dev_bf16(sv), tail_k=dev_bf16(tk), tail_v=dev_bf16(tv),
                key_shift=dev(wl.key_shift), softmax_scale=wl.sigma, pages_per_partition=1, workspace=ws)
    g_best, g_errs = bd.calibrate_tau(rc, cands, gref, args)
    print("[tau] oracle", np.round(o_errs, 6), "device", np.round(g_errs, 6), flush=True)
    assert np.allclose(g_errs, o_errs, rtol=1e-4, atol=0.0)
    srt = sorted(o_errs)
    if srt[1] - srt[0] > 1e-3 * srt[0]:                 # a clear winner must be found again
        assert g_best == o_best
    else:
        assert g_errs[cands.index(g_best)] <= srt[0] * (1 + 1e-3)
