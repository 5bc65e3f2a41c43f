"""Quantization diagnostics through the C ABI against the oracle: the page
squared-error sums of pages the HIP writer wrote equal the oracle's sums
over the oracle's pages (float64, to summation order), for NVFP4 four_six /
amax6, without rotation and centering, and MXFP4; a destination page outside
the pool contributes nothing; sampled pages of the full 131,072-token x
8-head prefill."""
import numpy as np
import pytest
import torch

import fp4_kv_cache_nvfp4_amd as bd
from fp4_kv_cache_nvfp4_amd import synth
from oracle import diagnostics as DG
from oracle import quant as Q
from oracle import recipe as RC
from oracle import writer as W

from gpu_helpers import dev, dev_bf16, gpu_write, oracle_write, to_c

pytestmark = pytest.mark.gpu

RECIPES = {
    "nvfp4": RC.nvfp4_default().with_(tau=1.0),
    "nvfp4_amax6": RC.nvfp4_default().with_(tau=1.0, scale_mode_k=Q.AMAX6),
    "nvfp4_plain": RC.nvfp4_default().with_(tau=1.0, rotation=False, key_smoothing=False),
    "mxfp4": RC.mxfp4_default().with_(tau=1.0),
    "nvfp4_rotv": RC.nvfp4_default().with_(tau=1.0, rotate_v=True),
    "nvfp4_chan": RC.nvfp4_default().with_(tau=1.0, key_scale_geometry=RC.CHANNEL),
}


def _u16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("name", list(RECIPES))
def test_page_errors_match_oracle(name):
    r = RECIPES[name]
    wl = synth.decode_workload("d", 9, [128 * 5 + 7, 128 * 2], 16, 4, "qwen", extra_pages=2)
    k, v, ids = wl.writer_inputs()
    mu = wl.key_shift if r.key_smoothing else None
    cache = gpu_write(r, wl)
    ids_f = ids.copy()
    ids_f[1] = wl.num_pages + 3                         # this input page is not stored anywhere
    got = bd.page_errors(to_c(r), cache, dev_bf16(k), dev_bf16(v), dev(ids_f),
                         dev(mu) if mu is not None else None).cpu().numpy()
    want = DG.page_errors(r, oracle_write(r, wl), k, v, ids_f, mu)
    print(f"[diag] {name}: K rel {np.sqrt(got[0] / got[1]):.4f} V rel {np.sqrt(got[2] / got[3]):.4f}", flush=True)
    assert np.allclose(got, want, rtol=1e-12, atol=0.0), (got, want)


def test_page_errors_full_prefill_sampled():
    r = RECIPES["nvfp4"]
    rc = to_c(r)
    w = synth.torch_write_rows(0)
    cache = bd.PagedCache.allocate(rc, w["num_pages"], 8)
    bd.quantize_pages(rc, cache, w["k"], w["v"], w["page_ids"], w["key_shift"])
    rng = np.random.default_rng(1)
    pick = np.sort(rng.choice(w["tokens"] // 128, size=12, replace=False))
    rows = torch.from_numpy(np.concatenate([np.arange(p * 128, p * 128 + 128) for p in pick])).cuda()
    ks, vs = w["k"][rows].contiguous(), w["v"][rows].contiguous()
    ids = w["page_ids"][torch.from_numpy(pick).cuda()].contiguous()
    got = bd.page_errors(rc, cache, ks, vs, ids, w["key_shift"]).cpu().numpy()
    # the oracle writes the sampled pages itself and measures its own pages
    kh, vh, ih, muh = _u16(ks), _u16(vs), ids.cpu().numpy(), w["key_shift"].cpu().numpy()
    ocache = W.empty_cache(w["num_pages"], 8, r)
    W.write_pages(r, ocache, kh, vh, ih, muh)
    want = DG.page_errors(r, ocache, kh, vh, ih, muh)
    assert np.allclose(got, want, rtol=1e-12, atol=0.0), (got, want)


def _from_c(rc) -> RC.Recipe:
    mode = {bd.SCALE_NONE: Q.NONE, bd.SCALE_AMAX6: Q.AMAX6, bd.SCALE_FOUR_SIX: Q.FOUR_SIX,
            bd.SCALE_MXFP4_SEARCH: Q.MXFP4_SEARCH, bd.SCALE_AMAX2_OR_AMAX6: Q.AMAX2_OR_AMAX6}
    return RC.Recipe(sink_tokens=rc.sink_tokens, rotation=bool(rc.rotation), key_smoothing=bool(rc.key_smoothing),
                     scale_mode_k=mode[rc.scale_mode_k], scale_mode_v=mode[rc.scale_mode_v],
                     scale_mode_q=mode[rc.scale_mode_q], scale_mode_p=mode[rc.scale_mode_p],
                     query_terms=rc.query_terms, c=rc.c, tau=float(rc.tau), rotate_v=bool(rc.rotate_v),
                     p_running_max=bool(rc.p_running_max),
                     key_scale_geometry=RC.CHANNEL if rc.key_scale_geometry == bd.KEY_GEOMETRY_CHANNEL else RC.LOCAL)


@pytest.mark.parametrize("keys", ["qwen", "write"])
def test_ablation_report_matches_oracle(keys):
    from fp4_kv_cache_nvfp4_amd import diagnostics as D
    from oracle import decode as OD

    L, layer = 1024 + 77, 3
    rep = D.ablation_report(context=L, layer=layer, keys=keys)
    d = synth.torch_decode_layer(layer, seq_len=L, outliers=keys)   # the same seeded inputs
    k, v, q = _u16(d["k"]), _u16(d["v"]), _u16(d["q"])
    bt, sl = d["block_tables"].cpu().numpy(), d["seq_lens"].cpu().numpy()
    ids, n_full, mu = d["page_ids"].cpu().numpy(), d["n_full"], d["key_shift"].cpu().numpy()
    sk, sv, tk, tv = (_u16(d[n]) for n in ("sink_k", "sink_v", "tail_k", "tail_v"))
    kp = _u16(synth.bf16_pages_from_tokens(d["k"], d["block_tables"], d["num_pages"]))
    vp = _u16(synth.bf16_pages_from_tokens(d["v"], d["block_tables"], d["num_pages"]))
    ref = OD.bf16_decode(q, kp, vp, bt, sl, d["sigma"])
    for name, rc in D.recipes().items():
        r = _from_c(rc)
        m = mu if r.key_smoothing else None
        cache = W.empty_cache(d["num_pages"], 8, r)
        W.write_pages(r, cache, k[:n_full * 128], v[:n_full * 128], ids, m)
        pe = DG.page_errors(r, cache, k[:n_full * 128], v[:n_full * 128], ids, m)
        out = OD.decode(r, cache, q, bt, sl, sk, sv, tk, tv, m, d["sigma"], rep["pages_per_partition"])
        want = {"k_rel": np.sqrt(pe[0] / pe[1]), "v_rel": np.sqrt(pe[2] / pe[3]),
                "out_rel_l2": np.linalg.norm(out - ref) / np.linalg.norm(ref)}
        got = rep["recipes"][name]
        print(f"[ablation] keys={keys} {name}: {got}", flush=True)
        assert abs(got["k_rel"] - want["k_rel"]) <= 1e-9 * want["k_rel"], name
        assert abs(got["v_rel"] - want["v_rel"]) <= 1e-9 * want["v_rel"], name
        assert abs(got["out_rel_l2"] - want["out_rel_l2"]) <= 1e-3 * want["out_rel_l2"], name
