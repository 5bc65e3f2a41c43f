"""The C ABI on the host (no GPU): the library loads and exports every entry
point include/bdfp4.h declares; recipe defaults and validation follow the
BitDecoding-FP4 config page (golden/recipe_modes.json,
golden/probability_environment.json); every invalid argument returns its
documented status before anything is launched; sizes and the split plan.

Only failing calls and pure host functions are made here: a call that passed
validation would launch a kernel.
"""
import ctypes
import json
import math
import os
import re

import pytest

import fp4_kv_cache_nvfp4_amd as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")
FAKE = 0x7F0000000000          # 16-byte aligned stand-in device address (never dereferenced)
TICKETS = 16384 * 128          # the workspace's ticket region: 16,384 tickets, one 128-byte line each


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _declared():
    src = open(os.path.join(ROOT, "include", "bdfp4.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bdfp4_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_entry_point():
    names = _declared()
    assert len(names) >= 12
    L = bd.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    assert bd.status_string(0) == "BDFP4_OK"
    assert bd.status_string(-2) == "BDFP4_E_UNCALIBRATED"
    assert bd.status_string(-99) == "BDFP4_E_UNKNOWN"


def test_recipe_defaults_follow_kv_modes():
    g = _golden("recipe_modes.json")
    nv = bd.recipe_default_nvfp4()
    e = g["bitdecoding-nvfp4"]
    assert nv.sink_tokens == e["sink_tokens"] and nv.query_terms == e["query_terms"]
    assert (nv.scale_mode_k, nv.scale_mode_v, nv.scale_mode_q) == (bd.SCALE_FOUR_SIX, bd.SCALE_AMAX6, bd.SCALE_AMAX6)
    assert nv.rotation == 1 and nv.key_smoothing == 1
    assert nv.scale_mode_p == bd.SCALE_AMAX2_OR_AMAX6 and nv.c == g["probability"]["c"]
    assert math.isnan(nv.tau)
    mx = bd.recipe_default_mxfp4()
    assert mx.scale_mode_k == mx.scale_mode_v == mx.scale_mode_q == bd.SCALE_MXFP4_SEARCH
    assert mx.sink_tokens == g["bitdecoding-mxfp4"]["sink_tokens"] and mx.rotation == 1


def test_recipe_validation_follows_probability_environment():
    g = _golden("probability_environment.json")
    for case in g["cases"]:
        r = bd.recipe_default_nvfp4()
        r.c = case["c"]
        r.tau = math.nan if case["tau"] is None else float(case["tau"])
        r.scale_mode_p = bd.SCALE_AMAX2_OR_AMAX6 if case["enabled"] else bd.SCALE_AMAX6
        want = {"ok": bd.OK, "invalid": bd.E_INVALID, "uncalibrated": bd.E_UNCALIBRATED}[case["expect"]]
        if want == bd.OK:
            bd.recipe_validate(r)
        else:
            with pytest.raises(bd.Bdfp4Error) as ei:
                bd.recipe_validate(r)
            assert ei.value.status == want


@pytest.mark.parametrize("field,value,status", [
    ("sink_tokens", 8, bd.E_INVALID), ("sink_tokens", 128, bd.E_INVALID), ("sink_tokens", -16, bd.E_INVALID),
    ("query_terms", 3, bd.E_INVALID), ("rotation", 2, bd.E_INVALID), ("key_smoothing", 5, bd.E_INVALID),
    ("rotate_v", 2, bd.E_INVALID), ("p_running_max", 3, bd.E_INVALID),
    ("scale_mode_k", 9, bd.E_INVALID), ("scale_mode_v", bd.SCALE_FOUR_SIX, bd.E_INVALID),
    ("scale_mode_p", 7, bd.E_INVALID), ("scale_mode_p", bd.SCALE_NONE, bd.E_UNSUPPORTED),
    ("scale_mode_q", bd.SCALE_MXFP4_SEARCH, bd.E_UNSUPPORTED),
    ("scale_mode_v", bd.SCALE_MXFP4_SEARCH, bd.E_UNSUPPORTED),
    ("key_scale_geometry", 2, bd.E_INVALID), ("key_scale_geometry", -1, bd.E_INVALID),
])
def test_recipe_field_checks(field, value, status):
    r = bd.recipe_default_nvfp4(tau=1.0)
    setattr(r, field, value)
    with pytest.raises(bd.Bdfp4Error) as ei:
        bd.recipe_validate(r)
    assert ei.value.status == status


def test_sizes_and_plan():
    nv = bd.recipe_default_nvfp4(tau=1.0)
    mx = bd.recipe_default_mxfp4(tau=1.0)
    assert bd.cache_bytes(nv, 10, 8) == (10 * 8 * 8192, 10 * 8 * 1024, 10 * 8 * 8192, 10 * 8 * 1024)
    assert bd.cache_bytes(mx, 3, 2) == (3 * 2 * 8192, 3 * 2 * 512, 3 * 2 * 8192, 3 * 2 * 512)
    # explicit plan
    assert bd.decode_plan(1, 8, 131072, 2) == (2, 512)
    assert bd.decode_plan(1, 1, 2048, 4) == (4, 4)
    assert bd.decode_plan(1, 1, 100, 4) == (4, 0)
    ppp, parts = bd.decode_plan(1, 8, 131072, 0)
    assert ppp == 4 and parts == -(-1024 // ppp)
    # the automatic plan: at most 256 FP4 workgroups of four partitions while
    # 4 pages per partition suffice, else about 512
    assert [bd.decode_plan(1, 8, L, 0) for L in (8192, 16384, 32768, 49152, 65536, 98304)] == \
        [(1, 64), (1, 128), (2, 128), (3, 128), (4, 128), (3, 256)]
    assert bd.decode_plan(16, 8, 16384, 0) == (4, 32)
    assert bd.decode_plan(1, 1, 2048, 0) == (1, 16)
    ws = bd.decode_workspace_size(1, 32, 8, 131072, 4)
    assert ws == TICKETS + 8 * (256 + 2) * 520 * 4
    # a partial last page adds a BF16-decode partition
    assert bd.decode_workspace_size(2, 8, 2, 1000, 3) == TICKETS + 4 * 6 * 520 * 4      # 3 + 2 slots, rounded up to even
    with pytest.raises(bd.Bdfp4Error) as ei:
        bd.decode_workspace_size(1, 24, 8, 1000, 0)
    assert ei.value.status == bd.E_UNSUPPORTED
    for args in [(0, 8, 1000, 0), (1, 8, 0, 0), (1, 8, 1000, 5), (1, 8, 1000, -1)]:
        with pytest.raises(bd.Bdfp4Error) as ei:
            bd.decode_plan(*args)
        assert ei.value.status == bd.E_INVALID


def test_bf16_plan_and_workspace():
    # the BF16-KV decode's own plan: about 512 workgroups, up to 16 pages
    # (the partial last page counted) per partition
    assert [bd.bf16_decode_plan(1, 8, L, 0) for L in (8192, 32768, 65536, 131072)] == \
        [(1, 64), (4, 64), (8, 64), (16, 64)]
    assert bd.bf16_decode_plan(1, 8, 131072 + 77, 0) == (16, 65)
    assert bd.bf16_decode_plan(16, 8, 16384, 0) == (16, 8)
    assert bd.bf16_decode_plan(5, 2, 2100, 0) == (1, 17)
    assert bd.bf16_decode_plan(1, 1, 100, 16) == (16, 1)
    for args in [(1, 8, 1000, 17), (1, 8, 1000, -1), (0, 8, 1000, 0)]:
        with pytest.raises(bd.Bdfp4Error) as ei:
            bd.bf16_decode_plan(*args)
        assert ei.value.status == bd.E_INVALID
    # 0 sizes for both automatic plans (the FP4 one needs more here), 5 .. 16
    # for the BF16 decode alone
    assert bd.decode_workspace_size(1, 32, 8, 131072, 0) == TICKETS + 8 * (256 + 2) * 520 * 4
    assert bd.decode_workspace_size(1, 32, 8, 131072, 16) == TICKETS + 8 * (64 + 2) * 520 * 4
    assert bd.decode_workspace_size(1, 32, 8, 131072 + 77, 16) == TICKETS + 8 * 68 * 520 * 4   # 65 + 2, even
    for L in (100, 2048, 8192, 32768 + 77, 131072):
        for b, h in ((1, 1), (1, 8), (16, 8)):
            auto = bd.decode_workspace_size(b, 4 * h, h, L, 0)
            assert auto >= bd.decode_workspace_size(b, 4 * h, h, L, bd.bf16_decode_plan(b, h, L, 0)[0])
            assert auto >= bd.decode_workspace_size(b, 4 * h, h, L, bd.decode_plan(b, h, L, 0)[0])


def _cache(**kw):
    c = bd.Cache(FAKE, FAKE, FAKE, FAKE, 16, 1, 128, 128)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _decode(r, cache=None, **kw):
    a = dict(q=FAKE, batch=1, hq=4, bt=FAKE, maxp=16, seq=FAKE, maxlen=2048, sk=FAKE, sv=FAKE, tk=FAKE,
             tv=FAKE, mu=FAKE, scale=0.088, ppp=4, ws=None, wsb=None, out=FAKE)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = bd.decode_workspace_size(1, 4, 1, 2048, 4)
    if a["ws"] is None:
        a["ws"] = FAKE
    c = cache or _cache()
    return bd.lib().bdfp4_decode_attention(
        ctypes.byref(r), ctypes.byref(c), a["q"], a["batch"], a["hq"], a["bt"], a["maxp"], a["seq"],
        a["maxlen"], a["sk"], a["sv"], a["tk"], a["tv"], a["mu"], a["scale"], a["ppp"], a["ws"], a["wsb"],
        a["out"], None)


def test_decode_rejects_before_launch():
    r = bd.recipe_default_nvfp4(tau=1.0)
    assert _decode(bd.recipe_default_nvfp4()) == bd.E_UNCALIBRATED
    assert _decode(r.replace(c=2)) == bd.E_INVALID
    assert _decode(r, cache=_cache(head_dim=64)) == bd.E_UNSUPPORTED
    assert _decode(r, cache=_cache(block_size=16)) == bd.E_UNSUPPORTED
    assert _decode(r, cache=_cache(k_codes=None)) == bd.E_INVALID
    assert _decode(r, cache=_cache(v_scales=FAKE + 4)) == bd.E_INVALID
    assert _decode(r, hq=8) == bd.E_UNSUPPORTED
    assert _decode(r, q=None) == bd.E_INVALID
    assert _decode(r, q=FAKE + 2) == bd.E_INVALID
    assert _decode(r, mu=None) == bd.E_INVALID                     # key smoothing without key means
    assert "key_shift" in bd.lib().bdfp4_last_error().decode()
    assert _decode(r.replace(key_smoothing=0)) == bd.E_INVALID     # key means without smoothing
    assert _decode(r, sk=None) == bd.E_INVALID
    assert _decode(r, tk=None) == bd.E_INVALID
    assert _decode(r, ws=None, wsb=0) == bd.E_WORKSPACE
    assert _decode(r, wsb=100) == bd.E_WORKSPACE
    assert _decode(r, maxp=15) == bd.E_INVALID                     # 2048 tokens need 16 pages
    assert _decode(r, maxlen=0) == bd.E_INVALID
    assert _decode(r, ppp=40) == bd.E_INVALID
    assert _decode(r, scale=float("inf")) == bd.E_INVALID
    assert _decode(r, batch=0) == bd.E_INVALID
    assert "batch" in bd.lib().bdfp4_last_error().decode()


def _write(r, cache=None, k=FAKE, v=FAKE, ids=FAKE, n=4, mu=FAKE):
    c = cache or _cache()
    return bd.lib().bdfp4_quantize_pages(ctypes.byref(r), ctypes.byref(c), k, v, ids, n, mu, None)


def test_writer_rejects_before_launch():
    r = bd.recipe_default_nvfp4()          # tau is not needed to write pages
    assert _write(r, n=0) == bd.OK          # empty write is a no-op
    assert _write(r, n=-1) == bd.E_INVALID
    assert _write(r, k=None) == bd.E_INVALID
    assert _write(r, v=FAKE + 8) == bd.E_INVALID
    assert _write(r, ids=None) == bd.E_INVALID
    assert _write(r, mu=None) == bd.E_INVALID
    assert _write(r.replace(key_smoothing=0)) == bd.E_INVALID
    assert _write(r.replace(scale_mode_k=bd.SCALE_MXFP4_SEARCH)) == bd.E_UNSUPPORTED
    assert _write(r, cache=_cache(num_pages=0)) == bd.E_INVALID
    assert _write(r, cache=_cache(head_dim=256)) == bd.E_UNSUPPORTED


def test_codec_entries_reject_before_launch():
    L = bd.lib()
    assert L.bdfp4_quantize_rows(FAKE, 4, None, 1, 7, 1, FAKE, FAKE, None) == bd.E_INVALID
    assert L.bdfp4_quantize_rows(FAKE, 4, None, 1, 1, 3, FAKE, FAKE, None) == bd.E_INVALID
    assert L.bdfp4_quantize_rows(FAKE, 0, None, 1, 1, 1, None, None, None) == bd.OK
    assert L.bdfp4_quantize_p_blocks(FAKE, 4, 4, ctypes.c_float(math.nan), FAKE, FAKE, None) == bd.E_UNCALIBRATED
    assert L.bdfp4_quantize_p_blocks(FAKE, 4, 4, ctypes.c_float(500.0), FAKE, FAKE, None) == bd.E_INVALID
    assert L.bdfp4_quantize_p_blocks(FAKE, 4, 2, ctypes.c_float(1.0), FAKE, FAKE, None) == bd.E_INVALID


def test_bf16_decode_rejects_before_launch():
    L = bd.lib()
    wsb = bd.decode_workspace_size(1, 4, 1, 2048, 4)
    call = lambda **k: L.bdfp4_bf16_decode_attention(
        k.get("q", FAKE), 1, k.get("hq", 4), 1, k.get("kp", FAKE), FAKE, 16, FAKE, k.get("maxp", 16), FAKE,
        k.get("maxlen", 2048), 0.088, 4, FAKE, k.get("wsb", wsb), FAKE, None)
    assert call(hq=12) == bd.E_UNSUPPORTED
    assert call(kp=None) == bd.E_INVALID
    assert call(maxlen=2049) == bd.E_INVALID       # 17 pages needed, 16 in the table
    assert call(wsb=64) == bd.E_WORKSPACE


def test_stream_read_rejects_before_launch():
    L = bd.lib()
    ok_sink = 512 * 256 * 4
    assert L.bdfp4_stream_read(FAKE, 4096, FAKE, ok_sink, 0, None) == bd.E_INVALID          # no workgroups
    assert L.bdfp4_stream_read(FAKE, 4096, FAKE, ok_sink, 70000, None) == bd.E_INVALID      # too many
    assert L.bdfp4_stream_read(FAKE, 4100, FAKE, ok_sink, 512, None) == bd.E_INVALID        # not 16-byte words
    assert L.bdfp4_stream_read(None, 4096, FAKE, ok_sink, 512, None) == bd.E_INVALID
    assert L.bdfp4_stream_read(FAKE + 8, 4096, FAKE, ok_sink, 512, None) == bd.E_INVALID    # misaligned source
    assert L.bdfp4_stream_read(FAKE, 4096, FAKE, ok_sink - 4, 512, None) == bd.E_INVALID    # sink too small


def test_append_rejects_before_launch():
    r = bd.recipe_default_nvfp4()
    c = _cache()
    L = bd.lib()

    def call(r=r, batch=2, kn=FAKE, maxp=8, sink=FAKE, tail=FAKE, mu=FAKE, cache=c):
        return L.bdfp4_append_tokens(ctypes.byref(r), ctypes.byref(cache), kn, FAKE, batch, FAKE, FAKE, maxp,
                                     sink, sink, tail, tail, mu, None)
    assert call(batch=0) == bd.OK                 # nothing to append: no launch
    assert call(batch=-1) == bd.E_INVALID
    assert call(maxp=0) == bd.E_INVALID
    assert call(kn=None) == bd.E_INVALID
    assert call(kn=FAKE + 8) == bd.E_INVALID      # misaligned token rows
    assert call(sink=None) == bd.E_INVALID        # sink_tokens = 16 needs the sink buffers
    assert call(tail=None) == bd.E_INVALID
    assert call(mu=None) == bd.E_INVALID          # key smoothing needs the key means
    assert call(r.replace(key_smoothing=0)) == bd.E_INVALID
    assert call(r.replace(scale_mode_k=bd.SCALE_MXFP4_SEARCH)) == bd.E_UNSUPPORTED
    assert call(cache=_cache(num_pages=0)) == bd.E_INVALID


def test_calibration_entries_reject_before_launch():
    L = bd.lib()
    n = ctypes.c_size_t()
    assert L.bdfp4_key_means_workspace_size(131072, 8, ctypes.byref(n)) == bd.OK
    assert n.value == 64 * 8 * 128 * 8                     # float64 sums per 2048-token chunk
    assert L.bdfp4_key_means_workspace_size(0, 8, ctypes.byref(n)) == bd.E_INVALID
    assert L.bdfp4_key_means_workspace_size(16, 0, ctypes.byref(n)) == bd.E_INVALID
    assert L.bdfp4_key_means(FAKE, 1000, 2, FAKE, 16, FAKE, None) == bd.E_WORKSPACE
    assert L.bdfp4_key_means(None, 1000, 2, FAKE, 1 << 20, FAKE, None) == bd.E_INVALID
    assert L.bdfp4_key_means(FAKE + 8, 1000, 2, FAKE, 1 << 20, FAKE, None) == bd.E_INVALID
    assert L.bdfp4_error_sums(FAKE, FAKE, -1, FAKE, None) == bd.E_INVALID
    assert L.bdfp4_error_sums(FAKE, None, 16, FAKE, None) == bd.E_INVALID
    assert L.bdfp4_error_sums(FAKE, FAKE, 16, None, None) == bd.E_INVALID
    assert L.bdfp4_error_sums(FAKE, FAKE, 16, FAKE + 4, None) == bd.E_INVALID


def test_key_mean_sidecar_round_trip(tmp_path):
    import numpy as np
    rng = np.random.default_rng(3)
    means = {f"layer.{i}.key_shift": rng.standard_normal((8, 128)).astype(np.float32) for i in range(3)}
    p = str(tmp_path / "key_means.safetensors")
    bd.save_key_means(p, means)
    back = bd.load_key_means(p)
    assert sorted(back) == sorted(means)
    assert all(np.array_equal(back[k], means[k]) and back[k].dtype == np.float32 for k in means)


def test_page_errors_reject_before_launch():
    r = bd.recipe_default_nvfp4()
    L = bd.lib()
    n = ctypes.c_size_t()
    assert L.bdfp4_page_errors_workspace_size(4, 2, ctypes.byref(n)) == bd.OK and n.value == 4 * 2 * 4 * 8
    assert L.bdfp4_page_errors_workspace_size(0, 2, ctypes.byref(n)) == bd.E_INVALID

    def call(r=r, n_pages=4, wsb=1 << 20, mu=FAKE, out=FAKE, cache=None):
        c = cache or _cache()
        return L.bdfp4_page_errors(ctypes.byref(r), ctypes.byref(c), FAKE, FAKE, FAKE, n_pages, mu, FAKE, wsb,
                                   out, None)
    assert call(wsb=16) == bd.E_WORKSPACE
    assert call(n_pages=0) == bd.E_INVALID
    assert call(mu=None) == bd.E_INVALID
    assert call(out=FAKE + 4) == bd.E_INVALID
    assert call(r.replace(scale_mode_v=bd.SCALE_MXFP4_SEARCH)) == bd.E_UNSUPPORTED


def test_running_max_variant_combinations():
    nv = bd.recipe_default_nvfp4(tau=1.0)
    bd.recipe_validate(nv.replace(p_running_max=1))
    for r in (bd.recipe_default_mxfp4(tau=1.0).replace(p_running_max=1),
              nv.replace(p_running_max=1, query_terms=1),
              nv.replace(p_running_max=1, scale_mode_p=bd.SCALE_AMAX6)):
        with pytest.raises(bd.Bdfp4Error) as ei:
            bd.recipe_validate(r)
        assert ei.value.status == bd.E_UNSUPPORTED


def test_noalloc_decode_rejects_before_launch():
    """The allocation-free decode validates like the workspace entry point
    and refuses a plan larger than its fixed array, enqueuing nothing (no GPU
    is touched on these paths)."""
    r = bd.recipe_default_nvfp4(tau=1.0)
    L = bd.lib()
    cap = bd.decode_noalloc_max_workspace()
    assert cap == 16 << 20

    def call(r, batch, hkv, maxp, maxlen, ppp, q=FAKE):
        c = _cache(num_kv_heads=hkv)
        return L.bdfp4_decode_attention_noalloc(ctypes.byref(r), ctypes.byref(c), q, batch, 4 * hkv, FAKE, maxp,
                                                FAKE, maxlen, FAKE, FAKE, FAKE, FAKE, FAKE, 0.088, ppp, FAKE, None)

    # 64 sequences x 8 KV heads x 128K tokens at one page per partition need
    # far more than the array holds
    assert bd.decode_workspace_size(64, 32, 8, 131072, 1) > cap
    assert call(r, 64, 8, 1024, 131072, 1) == bd.E_WORKSPACE
    assert "allocation-free" in L.bdfp4_last_error().decode()
    # argument errors are reported first, as by bdfp4_decode_attention
    assert call(bd.recipe_default_nvfp4(), 1, 1, 16, 2048, 4) == bd.E_UNCALIBRATED
    assert call(r, 1, 1, 16, 2048, 4, q=None) == bd.E_INVALID
    assert call(r, 1, 1, 16, 2048, 40) == bd.E_INVALID


def test_channel_key_geometry_support():
    nv = bd.recipe_default_nvfp4(tau=1.0)
    assert nv.key_scale_geometry == bd.KEY_GEOMETRY_LOCAL
    assert bd.recipe_default_mxfp4(tau=1.0).key_scale_geometry == bd.KEY_GEOMETRY_LOCAL
    bd.recipe_validate(nv.replace(key_scale_geometry=bd.KEY_GEOMETRY_CHANNEL))
    bd.recipe_validate(nv.replace(key_scale_geometry=bd.KEY_GEOMETRY_CHANNEL, scale_mode_k=bd.SCALE_AMAX6))
    for r in (bd.recipe_default_mxfp4(tau=1.0).replace(key_scale_geometry=bd.KEY_GEOMETRY_CHANNEL),
              nv.replace(key_scale_geometry=bd.KEY_GEOMETRY_CHANNEL, p_running_max=1)):
        with pytest.raises(bd.Bdfp4Error) as ei:
            bd.recipe_validate(r)
        assert ei.value.status == bd.E_UNSUPPORTED
    # the cache sizes do not depend on the key geometry
    assert bd.cache_bytes(nv.replace(key_scale_geometry=bd.KEY_GEOMETRY_CHANNEL), 3, 2) == bd.cache_bytes(nv, 3, 2)


def test_select_tau_host():
    """bdfp4_select_tau: relative L2 errors sqrt(err / ref), the smallest
    wins, ties keep the earlier candidate, NaN never wins, zero references."""
    import numpy as np
    cand = [0.0, 0.5, 1.0, 4.0]
    sums = np.array([[4.0, 100.0], [1.0, 100.0], [1.0, 100.0], [9.0, 100.0]])
    best, errs = bd.select_tau(sums, cand)
    assert best == 0.5 and np.allclose(errs, [0.2, 0.1, 0.1, 0.3], rtol=0, atol=1e-15)
    sums2 = np.array([[np.nan, 1.0], [0.0, 0.0], [1.0, 0.0], [0.25, 1.0]])
    best, errs = bd.select_tau(sums2, cand)
    assert best == 0.5 and errs[1] == 0.0 and errs[2] == float("inf") and np.isnan(errs[0])
    with pytest.raises(bd.Bdfp4Error) as ei:
        bd.select_tau(np.array([[np.nan, 1.0]]), [1.0])
    assert ei.value.status == bd.E_INVALID
    with pytest.raises(bd.Bdfp4Error):
        bd.select_tau(np.array([[-1.0, 1.0]]), [1.0])
