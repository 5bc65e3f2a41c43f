"""Decode-time append with freeze-at-fill through the C ABI, against the
oracle append on the same seeded inputs: after a run of appends that crosses
page boundaries (sink positions, a padding row, a destination page outside
the pool and positions past the block table included), the cache, the tails
and the sinks are bit-identical; a decode over a sequence built by appends
alone matches the oracle decode over the oracle's state."""
import numpy as np
import pytest
import torch

import fp4_kv_cache_nvfp4_amd as bd
from oracle import append as OA
from oracle import decode as OD
from oracle import quant as Q
from oracle import recipe as RC
from oracle import writer as W

from gpu_helpers import assert_close, cache_to_host, dev, dev_bf16, to_c

pytestmark = pytest.mark.gpu

PAGE, D = 128, 128
RECIPES = {
    "nvfp4": RC.nvfp4_default().with_(tau=1.0),
    "nvfp4_plain": RC.nvfp4_default().with_(tau=1.0, rotation=False, key_smoothing=False),
    "mxfp4": RC.mxfp4_default().with_(tau=1.0),
    "nvfp4_rotv": RC.nvfp4_default().with_(tau=1.0, rotate_v=True),
    "nvfp4_chan": RC.nvfp4_default().with_(tau=1.0, key_scale_geometry=RC.CHANNEL),
}


def _bf16(rng, shape, outlier=True):
    x = rng.standard_normal(shape).astype(np.float32)
    if outlier:
        x[..., 3] += 8.0
    u = x.view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def _u16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("name", list(RECIPES))
def test_append_run_bit_exact(name):
    r = RECIPES[name]
    rc = to_c(r)
    rng = np.random.default_rng(31)
    B, hkv, num_pages, max_pages, steps = 4, 4, 18, 4, 140
    # seq 0 starts empty; seq 1 mid-page, its second page outside the pool;
    # seq 2 padding for 10 steps; seq 3 runs past its 4-page block table
    starts = [0, 120, 250, 500]
    bt = rng.permutation(num_pages)[:B * max_pages].astype(np.int32).reshape(B, max_pages)
    bt[1, 1] = num_pages
    mu = (rng.standard_normal((hkv, D)) * 2).astype(np.float32) if r.key_smoothing else None
    S = r.sink_tokens
    tail_k, tail_v = _bf16(rng, (B, hkv, PAGE, D)), _bf16(rng, (B, hkv, PAGE, D), False)
    sink_k, sink_v = _bf16(rng, (B, hkv, S, D)), _bf16(rng, (B, hkv, S, D), False)
    kn_all, vn_all = _bf16(rng, (steps, B, hkv, D)), _bf16(rng, (steps, B, hkv, D), False)
    pos_all = np.array([[s + i for s in starts] for i in range(steps)], dtype=np.int32)
    pos_all[:10, 2] = -1
    pos_all[10:, 2] -= 10

    ocache = W.empty_cache(num_pages, hkv, r)
    otk, otv, osk, osv = tail_k.copy(), tail_v.copy(), sink_k.copy(), sink_v.copy()
    cache = bd.PagedCache.allocate(rc, num_pages, hkv)
    gtk, gtv, gsk, gsv = dev_bf16(tail_k), dev_bf16(tail_v), dev_bf16(sink_k), dev_bf16(sink_v)
    gbt, gmu = dev(bt), (dev(mu) if mu is not None else None)
    for i in range(steps):
        OA.append_tokens(r, ocache, otk, otv, osk, osv, kn_all[i], vn_all[i], pos_all[i], bt, mu)
        bd.append_tokens(rc, cache, dev_bf16(kn_all[i]), dev_bf16(vn_all[i]), dev(pos_all[i]), gbt,
                         gsk, gsv, gtk, gtv, gmu)
    torch.cuda.synchronize()
    got = cache_to_host(cache)
    frozen = 0
    for n in ocache:
        bad = np.argwhere(got[n] != ocache[n])
        assert bad.size == 0, f"{n}: {len(bad)} bytes differ, first at {bad[:3].tolist()}"
        frozen += int(ocache[n].any(axis=(1, 2)).sum())
    assert frozen > 0
    for nm, g, o in (("tail_k", gtk, otk), ("tail_v", gtv, otv), ("sink_k", gsk, osk), ("sink_v", gsv, osv)):
        assert np.array_equal(_u16(g), o), nm


def test_append_then_decode_matches_oracle():
    r = RECIPES["nvfp4"]
    rc = to_c(r)
    rng = np.random.default_rng(32)
    hkv, hq, L, num_pages = 2, 8, 2 * PAGE + 44, 5
    bt = np.array([[3, 0, 4]], dtype=np.int32)
    mu = rng.standard_normal((hkv, D)).astype(np.float32)
    k, v = _bf16(rng, (L, 1, hkv, D)), _bf16(rng, (L, 1, hkv, D), False)
    q = _bf16(rng, (1, hq, D), False)
    z = lambda *s: np.zeros(s, dtype=np.uint16)
    ocache = W.empty_cache(num_pages, hkv, r)
    otk, otv, osk, osv = z(1, hkv, PAGE, D), z(1, hkv, PAGE, D), z(1, hkv, 16, D), z(1, hkv, 16, D)
    cache = bd.PagedCache.allocate(rc, num_pages, hkv)
    gtk, gtv, gsk, gsv = (dev_bf16(a) for a in (otk, otv, osk, osv))
    gbt, gmu = dev(bt), dev(mu)
    for t in range(L):
        pos = np.array([t], dtype=np.int32)
        OA.append_tokens(r, ocache, otk, otv, osk, osv, k[t], v[t], pos, bt, mu)
        bd.append_tokens(rc, cache, dev_bf16(k[t]), dev_bf16(v[t]), dev(pos), gbt, gsk, gsv, gtk, gtv, gmu)
    sigma = float(np.float32(1.0 / np.sqrt(128.0)))
    sl = np.array([L], dtype=np.int32)
    ws = bd.alloc_workspace(bd.decode_workspace_size(1, hq, hkv, L, 1))
    out = torch.full((1, hq, D), float("nan"), dtype=torch.float32, device="cuda")
    bd.decode_attention(rc, cache, dev_bf16(q), gbt, dev(sl), L, gsk, gsv, gtk, gtv, gmu, sigma, 1, ws, out)
    torch.cuda.synchronize()
    want = OD.decode(r, ocache, q, bt, sl, osk, osv, otk, otv, mu, sigma, 1)
    assert_close(out.cpu().numpy().astype(np.float64), want, "decode after 300 appends")
