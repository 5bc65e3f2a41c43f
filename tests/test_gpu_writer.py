"""GPU page writer parity through the C ABI: codes and scales of every
written page bit-exact with the oracle (NVFP4 four_six / amax6, MXFP4, with
and without rotation and centering, the channel key scale geometry),
untouched pages left alone, invalid
destination pages skipped; at the full 131,072-token x 8-head prefill size,
every page-head compared byte for byte."""
import numpy as np
import pytest
import torch

import fp4_kv_cache_nvfp4_amd as bd
from fp4_kv_cache_nvfp4_amd import synth
from oracle import layout as LY
from oracle import quant as Q
from oracle import recipe as RC
from oracle import writer as W

import oracle_pool as OP
from gpu_helpers import cache_to_host, dev, dev_bf16, gpu_write, oracle_write, to_c

pytestmark = pytest.mark.gpu

RECIPES = {
    "nvfp4": RC.nvfp4_default().with_(tau=1.0),
    "nvfp4_amax6": RC.nvfp4_default().with_(tau=1.0, scale_mode_k=Q.AMAX6),
    "nvfp4_plain": RC.nvfp4_default().with_(tau=1.0, rotation=False, key_smoothing=False),
    "mxfp4": RC.mxfp4_default().with_(tau=1.0),
    "mxfp4_plain": RC.mxfp4_default().with_(tau=1.0, rotation=False, key_smoothing=False),
    "nvfp4_rotv": RC.nvfp4_default().with_(tau=1.0, rotate_v=True),
    "mxfp4_rotv": RC.mxfp4_default().with_(tau=1.0, rotate_v=True),
    "nvfp4_chan": RC.nvfp4_default().with_(tau=1.0, key_scale_geometry=RC.CHANNEL),
    "nvfp4_chan_amax6": RC.nvfp4_default().with_(tau=1.0, key_scale_geometry=RC.CHANNEL, scale_mode_k=Q.AMAX6),
    "nvfp4_chan_plain": RC.nvfp4_default().with_(tau=1.0, key_scale_geometry=RC.CHANNEL, rotation=False,
                                                 key_smoothing=False),
}


def _compare(got: dict, want: dict, pages=None):
    for name in ("k_codes", "k_scales", "v_codes", "v_scales"):
        g, w = got[name], want[name]
        if pages is not None:
            g, w = g[pages], w[pages]
        bad = np.argwhere(g != w)
        assert bad.size == 0, f"{name}: {len(bad)} bytes differ, first at {bad[:3].tolist()}"


@pytest.mark.parametrize("name", list(RECIPES))
def test_writer_tiny_bit_exact(name):
    r = RECIPES[name]
    wl = synth.tiny(0)
    _compare(cache_to_host(gpu_write(r, wl)), oracle_write(r, wl))


@pytest.mark.parametrize("name", ["nvfp4", "mxfp4", "nvfp4_chan"])
def test_writer_multihead_permuted_bit_exact(name):
    r = RECIPES[name]
    wl = synth.decode_workload("w", 7, [128 * 11 + 5, 128 * 3], 32, 8, "qwen", extra_pages=3)
    got = cache_to_host(gpu_write(r, wl))
    want = oracle_write(r, wl)
    _compare(got, want)
    # pages nobody wrote stay zero
    used = set(int(p) for b in range(wl.batch) for p in wl.block_tables[b, :wl.full_pages(b)])
    for p in range(wl.num_pages):
        if p not in used:
            assert not got["k_codes"][p].any() and not got["v_scales"][p].any()


def test_writer_skips_invalid_page_ids():
    r = RECIPES["nvfp4"]
    wl = synth.write_workload(seed=2, tokens=512, num_kv_heads=2)
    rc = to_c(r)
    cache = bd.PagedCache.allocate(rc, wl.num_pages, 2)
    ids = wl.page_ids.copy()
    ids[1] = -1
    ids[2] = wl.num_pages + 5
    bd.quantize_pages(rc, cache, dev_bf16(wl.k_rows), dev_bf16(wl.v_rows), dev(ids), dev(wl.key_shift))
    torch.cuda.synchronize()
    got = cache_to_host(cache)
    want = W.empty_cache(wl.num_pages, 2, r)
    keep = [0, 3]
    W.write_pages(r, want, wl.k_rows.reshape(4, 128, 2, 128)[keep].reshape(-1, 2, 128),
                  wl.v_rows.reshape(4, 128, 2, 128)[keep].reshape(-1, 2, 128), ids[keep], wl.key_shift)
    _compare(got, want)


@pytest.mark.parametrize("name", ["nvfp4", "mxfp4", "nvfp4_chan"])
def test_writer_full_prefill(name):
    """131,072 tokens x 8 KV heads in one launch; the oracle writes the same
    1,024 pages x 8 KV heads and all four cache arrays are compared byte for
    byte."""
    r = RECIPES[name]
    print(f"[writer full] {name}", flush=True)
    wl = synth.write_workload(seed=0)
    rc = to_c(r)
    cache = bd.PagedCache.allocate(rc, wl.num_pages, 8)
    bd.quantize_pages(rc, cache, dev_bf16(wl.k_rows), dev_bf16(wl.v_rows), dev(wl.page_ids), dev(wl.key_shift))
    torch.cuda.synchronize()
    want = W.empty_cache(wl.num_pages, 8, r)
    OP.write_pages(r, want, wl.k_rows, wl.v_rows, wl.page_ids, wl.key_shift)
    for name_ in ("k_codes", "k_scales", "v_codes", "v_scales"):
        got = getattr(cache, name_).cpu().numpy()
        bad = np.argwhere(got != want[name_])
        assert bad.size == 0, (name_, bad.shape[0], bad[:4].tolist())