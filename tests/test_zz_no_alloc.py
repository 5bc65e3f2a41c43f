"""The allocation-free decode entry point (bdfp4_decode_attention_noalloc)
against bdfp4_decode_attention through the C ABI: two calls in a row on the
library's per-GPU scratch array, the second with a smaller input (fewer
sequences, KV heads and pages), each bit-identical to the workspace entry
point's output on the same inputs and within the parity tolerance of the
float64 oracle."""
import numpy as np
import pytest
import torch

import fp4_kv_cache_nvfp4_amd as bd
from fp4_kv_cache_nvfp4_amd import synth
from oracle import recipe as RC

from gpu_helpers import assert_close, cache_to_dev, dev, dev_bf16, oracle_decode, oracle_write, to_c

pytestmark = pytest.mark.gpu

NV = RC.nvfp4_default().with_(tau=1.0)


def _both(r, wl, ppp, what):
    print(f"[noalloc] {what}", flush=True)
    host = oracle_write(r, wl)
    cache = cache_to_dev(r, host, wl.num_kv_heads)
    rc = to_c(r)
    B, Hq = wl.batch, wl.num_q_heads
    msl = int(wl.seq_lens.max())
    sk, sv, tk, tv = wl.sink_tail()
    a = dict(q=dev_bf16(wl.q), bt=dev(wl.block_tables.astype(np.int32)), sl=dev(wl.seq_lens.astype(np.int32)),
             sk=dev_bf16(sk), sv=dev_bf16(sv), tk=dev_bf16(tk), tv=dev_bf16(tv), mu=dev(wl.key_shift))
    want = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    ws = bd.alloc_workspace(bd.decode_workspace_size(B, Hq, wl.num_kv_heads, msl, ppp))
    bd.decode_attention(rc, cache, a["q"], a["bt"], a["sl"], msl, a["sk"], a["sv"], a["tk"], a["tv"], a["mu"],
                        wl.sigma, ppp, ws, want)
    got = torch.full_like(want, float("nan"))
    bd.decode_attention_noalloc(rc, cache, a["q"], a["bt"], a["sl"], msl, a["sk"], a["sv"], a["tk"], a["tv"],
                                a["mu"], wl.sigma, ppp, got)
    torch.cuda.synchronize()
    g, w = got.cpu().numpy(), want.cpu().numpy()
    assert np.array_equal(g.view(np.uint32), w.view(np.uint32)), f"{what}: outputs differ from the workspace entry"
    assert_close(g.astype(np.float64), oracle_decode(r, wl, host, ppp), what)


def test_noalloc_two_calls_second_smaller():
    big = synth.decode_workload("noalloc_big", 11, [5000, 2179, 4096], 16, 4, "qwen", extra_pages=2)
    small = synth.decode_workload("noalloc_small", 12, [1300], 4, 1, "qwen")
    _both(NV, big, 1, "3 sequences x 4 KV heads, one page per partition")
    _both(NV, small, 4, "1 sequence x 1 KV head")


def test_noalloc_rejects_oversize_plan():
    r = bd.recipe_default_nvfp4(tau=1.0)
    need = bd.decode_workspace_size(64, 32, 8, 131072, 1)
    assert need > bd.decode_noalloc_max_workspace()
    wl = synth.tiny(0)
    cache = bd.PagedCache.allocate(r, 4, 8)
    q = torch.zeros((64, 32, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((64, 1024), dtype=torch.int32, device="cuda")
    sl = torch.full((64,), 131072, dtype=torch.int32, device="cuda")
    rows = torch.zeros((64, 8, 128, 128), dtype=torch.bfloat16, device="cuda")
    mu = torch.zeros((8, 128), dtype=torch.float32, device="cuda")
    out = torch.zeros((64, 32, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(bd.Bdfp4Error) as ei:
        bd.decode_attention_noalloc(r, cache, q, bt, sl, 131072, rows, rows, rows, rows, mu, wl.sigma, 1, out)
    assert ei.value.status == bd.E_WORKSPACE
    assert torch.count_nonzero(out).item() == 0
