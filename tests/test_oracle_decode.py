"""Oracle pins for the page layout, the writer, the split plan and the decode
(CPU only).

* layout: every nibble and scale byte of a page is used exactly once;
* writer: on-grid pages (rotation and centering off) dequantize to the input;
* decode with every quantizer off equals textbook softmax attention;
  with values rotated (rotate_v) and the outputs rotated back, too; and with
  P normalised by the running block maximum (p_running_max), which with P
  quantized equals the partition-maximum reading when every partition peaks
  in its first block;
  centering + rotation with quantizers off equals it to float32 rounding;
  on-grid pages read through the packed cache equal textbook attention;
* with P unquantized the result is independent of the split plan;
* permuting the physical pool and the block table changes nothing;
* bytes per token-head reproduce the memory ratio of "kv-landlords
  scripts/quant_ab.py" mem_ratio (golden/mem_ratio.json);
* recipe validation follows "BitDecoding-FP4 evaluation/config.py"
  probability_environment (golden/probability_environment.json).
"""
import json
import math
import os

import numpy as np
import pytest

from fp4_kv_cache_nvfp4_amd import synth
from oracle import decode as OD
from oracle import formats as F
from oracle import layout as LY
from oracle import quant as Q
from oracle import recipe as RC
from oracle import writer as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- layout

@pytest.mark.parametrize("which,mx", [("k", False), ("v", False), ("v", True)])
def test_code_layout_is_a_bijection(which, mx):
    b, sh = LY._code_map(which, mx)
    slot = b.astype(np.int64) * 2 + sh // 4
    assert np.array_equal(np.sort(slot), np.arange(128 * 128))
    rng = np.random.default_rng(0)
    nib = rng.integers(0, 16, size=(3, 128, 128)).astype(np.uint8)
    assert np.array_equal(LY.unpack_codes(LY.pack_codes(nib, which, mx), which, mx), nib)


@pytest.mark.parametrize("which", ["k", "v"])
@pytest.mark.parametrize("mx", [False, True])
def test_scale_layout_is_a_bijection(which, mx):
    nb = 4 if mx else 8
    fn = LY.k_scale_byte if which == "k" else LY.v_scale_byte
    t, j = np.meshgrid(np.arange(128), np.arange(nb), indexing="ij")
    b = fn(t, j, mx)
    assert np.array_equal(np.sort(b.ravel()), np.arange(128 * nb))
    rng = np.random.default_rng(1)
    sc = rng.integers(0, 256, size=(2, 128, nb)).astype(np.uint8)
    assert np.array_equal(LY.unpack_scales(LY.pack_scales(sc, which, mx), which, mx), sc)


def test_bytes_per_token_head_match_mem_ratio():
    g = _golden("mem_ratio.json")
    for case in g["cases"]:
        ratio = 2.0 / (case["bits"] / 8.0 + 1.0 / case["block"])
        assert ratio == pytest.approx(case["ratio"], rel=1e-15)
    # one K row + one V row of one page-head: codes and NVFP4 scales
    per_tok = 2 * (LY.CODE_BYTES + LY.scale_bytes(False)) / 128
    assert per_tok == 144
    assert 2 * 2 * 128 / per_tok == pytest.approx(g["cases"][0]["ratio"], rel=1e-12)
    assert 2 * (LY.CODE_BYTES + LY.scale_bytes(True)) / 128 == 136


# ----------------------------------------------------------------- recipe

def test_recipe_validation_follows_probability_environment():
    g = _golden("probability_environment.json")
    for case in g["cases"]:
        tau = case["tau"]
        tau = float("nan") if tau is None else float(tau)
        r = RC.nvfp4_default().with_(
            c=case["c"], tau=tau,
            scale_mode_p=Q.AMAX2_OR_AMAX6 if case["enabled"] else Q.AMAX6)
        if case["expect"] == "ok":
            RC.validate(r)
        elif case["expect"] == "uncalibrated":
            with pytest.raises(RC.UncalibratedError):
                RC.validate(r)
        else:
            with pytest.raises(RC.RecipeError) as ei:
                RC.validate(r)
            assert not isinstance(ei.value, RC.UncalibratedError)


def test_recipe_defaults_follow_kv_modes():
    g = _golden("recipe_modes.json")
    nv = RC.nvfp4_default()
    e = g["bitdecoding-nvfp4"]
    assert nv.sink_tokens == e["sink_tokens"] and nv.query_terms == e["query_terms"]
    assert (nv.scale_mode_k, nv.scale_mode_v, nv.scale_mode_q) == (
        e["scale_mode"]["key"], e["scale_mode"]["value"], e["scale_mode"]["query"])
    assert nv.rotation and nv.key_smoothing and nv.c == g["probability"]["c"]
    assert math.isnan(nv.tau)
    mx = RC.mxfp4_default()
    assert mx.scale_mode_k == mx.scale_mode_v == mx.scale_mode_q == g["bitdecoding-mxfp4"]["scale_mode"]


# ----------------------------------------------------------------- split plan

@pytest.mark.parametrize("sink", [0, 16, 48, 112])
def test_split_plan_covers_every_token_once(sink):
    for L in list(range(1, 300)) + [1000, 2048, 2049, 32845, 131072]:
        for ppp in (1, 2, 3, 4, 16):
            n, bf, parts = OD.split_plan(L, sink, ppp)
            toks = list(bf)
            for lo, hi in parts:
                assert lo % 16 == 0 and hi % 16 == 0 and lo < hi
                toks += list(range(lo, hi))
            assert sorted(toks) == list(range(L))
            assert len(parts) == (-(-n // ppp) if n else 0)


# ----------------------------------------------------------------- writer

def _on_grid_rows(rng, n):
    """Rows whose 16-blocks sit exactly on the NVFP4 grid with max 6*s."""
    s = np.exp2(rng.integers(-4, 3, size=(n, 8))).astype(np.float32)
    g = rng.choice(GRID, size=(n, 8, 16)) * rng.choice([-1.0, 1.0], size=(n, 8, 16))
    g[..., 0] = 6.0
    return (g * s[..., None]).reshape(n, 128).astype(np.float32)


def test_writer_on_grid_pages_round_trip():
    rng = np.random.default_rng(2)
    hkv, npg = 2, 3
    k = _on_grid_rows(rng, npg * 128 * hkv).reshape(npg * 128, hkv, 128)
    v = _on_grid_rows(rng, npg * 128 * hkv).reshape(npg * 128, hkv, 128)
    r = RC.nvfp4_default().with_(rotation=False, key_smoothing=False, scale_mode_k=Q.AMAX6, tau=1.0)
    cache = W.empty_cache(5, hkv, r)
    ids = np.array([4, 0, 2])
    W.write_pages(r, cache, synth.f32_to_bf16(k), synth.f32_to_bf16(v), ids)
    for i, p in enumerate(ids):
        for h in range(hkv):
            kh, vh = W.read_page_head(r, cache, p, h)
            assert np.array_equal(kh, k[i * 128:(i + 1) * 128, h].astype(np.float64))
            assert np.array_equal(vh, v[i * 128:(i + 1) * 128, h].astype(np.float64))
    assert not cache["k_codes"][1].any() and not cache["k_codes"][3].any()


def test_writer_rows_match_row_quantizer():
    wl = synth.write_workload(seed=3, tokens=256, num_kv_heads=2)
    r = RC.nvfp4_default().with_(tau=1.0)
    cache = W.empty_cache(wl.num_pages, 2, r)
    W.write_pages(r, cache, wl.k_rows, wl.v_rows, wl.page_ids, wl.key_shift)
    kf = F.bf16_to_f32(wl.k_rows)
    x = W.key_rows(kf, wl.key_shift[None], True)
    nib, sc = Q.quantize_four_six(x)
    p = int(wl.page_ids[1])
    got_n = LY.unpack_codes(cache["k_codes"][p, 1], "k")
    got_s = LY.unpack_scales(cache["k_scales"][p, 1], "k", False)
    assert np.array_equal(got_n, nib[128:256, 1]) and np.array_equal(got_s, sc[128:256, 1])


# ----------------------------------------------------------------- decode

def _workload(seed=0, L=(700, 300, 1), hkv=2, g=4):
    return synth.decode_workload("t", seed, list(L), hkv * g, hkv, "tiny", extra_pages=2)


def _run(r, wl, ppp=2, fp4_rows=None, cache=None):
    sk, sv, tk, tv = wl.sink_tail()
    if cache is None and fp4_rows is None:
        cache = W.empty_cache(wl.num_pages, wl.num_kv_heads, r)
        k, v, ids = wl.writer_inputs()
        W.write_pages(r, cache, k, v, ids, wl.key_shift if r.key_smoothing else None)
    return OD.decode(r, cache, wl.q, wl.block_tables, wl.seq_lens, sk, sv, tk, tv,
                     wl.key_shift if r.key_smoothing else None, wl.sigma, ppp, fp4_rows=fp4_rows)


def _textbook(wl):
    q = F.bf16_to_f32(wl.q)
    G = wl.num_q_heads // wl.num_kv_heads
    out = np.zeros((wl.batch, wl.num_q_heads, 128))
    for b in range(wl.batch):
        L = int(wl.seq_lens[b])
        k = F.bf16_to_f32(wl.k_tokens[b])
        v = F.bf16_to_f32(wl.v_tokens[b])
        for h in range(wl.num_kv_heads):
            out[b, h * G:(h + 1) * G] = OD.textbook_attention(q[b, h * G:(h + 1) * G], k[:L, h], v[:L, h], wl.sigma)
    return out


def _rows_unquantized(wl, r):
    def rows(b, h, n):
        k = F.bf16_to_f32(wl.k_tokens[b][: n * 128, h])
        v = F.bf16_to_f32(wl.v_tokens[b][: n * 128, h])
        x = W.key_rows(k, wl.key_shift[h] if r.key_smoothing else None, r.rotation)
        return x.astype(np.float64), W.value_rows(v, r.rotate_v).astype(np.float64)
    return rows


OFF = dict(scale_mode_k=Q.NONE, scale_mode_v=Q.NONE, scale_mode_q=Q.NONE, scale_mode_p=Q.NONE)


def test_quantization_off_is_textbook_attention():
    wl = _workload()
    r = RC.nvfp4_default().with_(rotation=False, key_smoothing=False, **OFF)
    got = _run(r, wl, fp4_rows=_rows_unquantized(wl, r))
    assert np.max(np.abs(got - _textbook(wl))) <= 1e-12


def test_centering_and_rotation_preserve_attention():
    wl = _workload(seed=1)
    r = RC.nvfp4_default().with_(**OFF)
    got = _run(r, wl, fp4_rows=_rows_unquantized(wl, r))
    assert np.max(np.abs(got - _textbook(wl))) <= 1e-6


def test_value_rotation_preserves_attention():
    # rotating the values and the partition outputs back changes nothing but
    # float32 rounding of the rotated values
    wl = _workload(seed=2)
    r = RC.nvfp4_default().with_(rotate_v=True, **OFF)
    got = _run(r, wl, fp4_rows=_rows_unquantized(wl, r))
    assert np.max(np.abs(got - _textbook(wl))) <= 1e-6
    # and without the rotation back the result is visibly different
    plain = _run(r.with_(rotate_v=False), wl, fp4_rows=_rows_unquantized(wl, r))
    assert np.max(np.abs(plain - _textbook(wl))) > 1e-2


def test_on_grid_cache_through_packed_layout_is_textbook():
    rng = np.random.default_rng(5)
    wl = _workload(seed=2, L=(640, 257))
    hkv = wl.num_kv_heads
    for b in range(wl.batch):
        L = int(wl.seq_lens[b])
        wl.k_tokens[b] = synth.f32_to_bf16(_on_grid_rows(rng, L * hkv).reshape(L, hkv, 128))
        wl.v_tokens[b] = synth.f32_to_bf16(_on_grid_rows(rng, L * hkv).reshape(L, hkv, 128))
    r = RC.nvfp4_default().with_(rotation=False, key_smoothing=False, scale_mode_k=Q.AMAX6,
                                 scale_mode_q=Q.NONE, scale_mode_p=Q.NONE)
    got = _run(r, wl)
    assert np.max(np.abs(got - _textbook(wl))) <= 1e-12


def test_split_plan_invariance_without_p_quantization():
    wl = _workload(seed=3)
    r = RC.nvfp4_default().with_(scale_mode_p=Q.NONE)
    outs = [_run(r, wl, ppp=ppp) for ppp in (1, 2, 3, 8)]
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) <= 1e-12


def test_paging_invariance():
    wl = _workload(seed=4)
    r = RC.nvfp4_default().with_(tau=1.0)
    base = _run(r, wl)
    perm = np.random.default_rng(9).permutation(wl.num_pages).astype(np.int32)
    wl.block_tables = perm[wl.block_tables]
    assert np.array_equal(_run(r, wl), base)


def test_quantized_decode_is_close_to_textbook():
    wl = _workload(seed=5)
    ref = _textbook(wl)
    for r in (RC.nvfp4_default().with_(tau=1.0), RC.mxfp4_default().with_(tau=1.0)):
        got = _run(r, wl)
        rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        assert rel < 0.15, rel


def test_p_blocks_follow_bruteforce_quantizer():
    """The P_hat of one FP4 partition equals a brute-force per-block search."""
    from fractions import Fraction
    r = RC.nvfp4_default().with_(tau=1.0)
    rng = np.random.default_rng(6)
    t = rng.standard_normal((4, 64)) * 3
    p = np.exp(t - t.max(axis=1, keepdims=True))
    pp = (8.0 * p).astype(np.float32)
    ph = OD._p_hat(r, pp)
    for g in range(4):
        for blk in range(4):
            x = pp[g, blk * 16:(blk + 1) * 16]
            a = np.max(x)
            k = np.float32(2.0) if a < np.float32(1.0) else np.float32(6.0)
            s = Fraction(float(F.e4m3_value(F.e4m3_encode(np.float32(a) / k))))
            for j in range(16):
                r_ = Fraction(float(x[j])) / s
                m = min(range(8), key=lambda i: (abs(r_ - Fraction(GRID[i])), i % 2))
                assert ph[g, blk * 16 + j] == float(Fraction(GRID[m]) * s / 8)


def test_p_prime_is_c_exp_sigma_t_minus_max_in_float32():
    """p' (the float32 probabilities the P codes are decided on): c exactly at
    the maximum, c * exp(sigma (r - m)) to float32 rounding elsewhere (within
    a few units in the last place: the argument is rounded twice), float32,
    non-negative, and increasing with r; against the running maximum it is
    c * exp(sigma (r - ref)) for the given reference."""
    rng = np.random.default_rng(11)
    sigma = 1.0 / np.sqrt(128.0)
    raw = rng.standard_normal((4, 96)) * 20.0
    for c in (1, 8):
        r = RC.nvfp4_default().with_(tau=1.0, c=c)
        m32 = raw.astype(np.float32).max(axis=1)
        pp = OD.p_prime(r, sigma, raw, m32)
        assert pp.dtype == np.float32 and np.all(pp >= 0)
        want = c * np.exp(sigma * (raw.astype(np.float32).astype(np.float64) - m32[:, None].astype(np.float64)))
        assert np.all(np.abs(pp - want) <= 4e-6 * want + 1e-30)
        assert np.all(pp[np.arange(4), raw.argmax(axis=1)] == np.float32(c))
        order = np.argsort(raw, axis=1)
        assert np.all(np.diff(np.take_along_axis(pp, order, axis=1), axis=1) >= 0)
        ref = np.maximum.accumulate(raw.astype(np.float32), axis=1)
        pr = OD.p_prime(r, sigma, raw, ref)
        assert np.all(np.abs(pr - c * np.exp(sigma * (raw.astype(np.float32) - ref).astype(np.float64)))
                      <= 4e-6 * c)


def test_bf16_baseline_is_textbook():
    wl = _workload(seed=7)
    kp, vp = wl.bf16_pages()
    got = OD.bf16_decode(wl.q, kp, vp, wl.block_tables, wl.seq_lens, wl.sigma)
    assert np.max(np.abs(got - _textbook(wl))) <= 1e-12


def test_running_max_variant_reduces_to_partition_max_and_to_textbook():
    wl = _workload(seed=3)
    # P unquantized: the normaliser cancels, both readings are textbook attention
    r = RC.nvfp4_default().with_(p_running_max=True, rotation=False, key_smoothing=False, **OFF)
    got = _run(r, wl, fp4_rows=_rows_unquantized(wl, r))
    assert np.max(np.abs(got - _textbook(wl))) <= 1e-12
    # P quantized, each partition's maximum in its first 16-token block: the
    # running maximum is the partition maximum throughout, the results coincide.
    # One query head per KV head, whose key at the partition's first token is
    # 50 q / |q| (logit 50 |q| sigma, far above the others).
    wl1 = _workload(seed=3, g=1)
    q = RC.nvfp4_default().with_(tau=1.0, rotation=False, key_smoothing=False, scale_mode_k=Q.NONE,
                                 scale_mode_v=Q.NONE, scale_mode_q=Q.NONE)
    rows = _rows_unquantized(wl1, q)
    qf = np.asarray(F.bf16_to_f32(wl1.q), dtype=np.float64)

    def peaked(b, h, n):
        k, v = rows(b, h, n)
        k = k.copy()
        for lo in ([16] if n else []) + [128 * p for p in range(1, n)]:   # each one-page partition's first token
            k[lo] = 50.0 * qf[b, h] / np.linalg.norm(qf[b, h])
        return k, v
    a = _run(q.with_(p_running_max=True), wl1, fp4_rows=peaked, ppp=1)
    b = _run(q, wl1, fp4_rows=peaked, ppp=1)
    assert np.array_equal(a, b)
    # and in general they differ (the variant is not a no-op)
    c = _run(q.with_(p_running_max=True), wl1, fp4_rows=rows, ppp=1)
    d = _run(q, wl1, fp4_rows=rows, ppp=1)
    assert not np.array_equal(c, d)
