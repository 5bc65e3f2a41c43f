"""The decode captured in a HIP graph (torch.cuda.CUDAGraph over the C-ABI
launch on the capturing stream), for the workspace entry point and the
allocation-free one: each of several replays, with the program's own eager
work and a synchronization between them, gives outputs bit-identical to the
eager call's. The decode records no memset into the graph: its tickets are
put back to zero by the kernel itself, and the allocation-free entry's
one-time zeroing of its scratch tickets is a fill kernel that runs on the
first (eager) call. A workload with several FP4 workgroups per sequence
(tickets and the final merge) and one that fits a single workgroup."""
import numpy as np
import pytest
import torch

import fp4_kv_cache_nvfp4_amd as bd
from fp4_kv_cache_nvfp4_amd import synth
from oracle import recipe as RC

from gpu_helpers import cache_to_dev, dev, dev_bf16, oracle_write, to_c

pytestmark = pytest.mark.gpu

NV = RC.nvfp4_default().with_(tau=1.0)
MX = RC.mxfp4_default().with_(tau=1.0)


def _inputs(r, wl):
    host = oracle_write(r, wl)
    cache = cache_to_dev(r, host, wl.num_kv_heads)
    sk, sv, tk, tv = wl.sink_tail()
    return cache, dict(q=dev_bf16(wl.q), bt=dev(wl.block_tables.astype(np.int32)),
                       sl=dev(wl.seq_lens.astype(np.int32)), sk=dev_bf16(sk), sv=dev_bf16(sv), tk=dev_bf16(tk),
                       tv=dev_bf16(tv), mu=dev(wl.key_shift))


@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
@pytest.mark.parametrize("r", [NV, MX], ids=["nvfp4", "mxfp4"])
def test_decode_graph_replays_match_eager(r, noalloc):
    rc = to_c(r)
    cases = (("ragged, 1 page per partition", synth.decode_workload("graph", 31, [5000, 1234, 300], 8, 2, "qwen",
                                                                     extra_pages=2), 1),
             ("tiny 2K", synth.tiny(0), 4))
    for what, wl, ppp in cases:
        print(f"[graph] {what} noalloc={noalloc}", flush=True)
        cache, a = _inputs(r, wl)
        B, Hq = wl.batch, wl.num_q_heads
        msl = int(wl.seq_lens.max())
        ws = None if noalloc else bd.alloc_workspace(bd.decode_workspace_size(B, Hq, wl.num_kv_heads, msl, ppp))
        out = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device="cuda")

        def call():
            if noalloc:
                bd.decode_attention_noalloc(rc, cache, a["q"], a["bt"], a["sl"], msl, a["sk"], a["sv"], a["tk"],
                                            a["tv"], a["mu"], wl.sigma, ppp, out)
            else:
                bd.decode_attention(rc, cache, a["q"], a["bt"], a["sl"], msl, a["sk"], a["sv"], a["tk"], a["tv"],
                                    a["mu"], wl.sigma, ppp, ws, out)

        call()
        torch.cuda.synchronize()
        want = out.clone()
        assert torch.isfinite(want).all()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            call()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call()
        torch.cuda.synchronize()
        for rep in range(4):
            out.fill_(float("nan"))
            junk = torch.randn(1 << 16, device="cuda").sum()          # eager work between replays
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int32), want.view(torch.int32)), (what, noalloc, rep, float(junk))
        del g
