"""Oracle pins for the channel key scale geometry (CPU only).

"BitDecoding-FP4 evaluation/config.py", KV_MODES bitdecoding-nvfp4: a key
scale geometry that defaults to "local"; "kv-landlords scripts/quant_ab.py",
SCHEMES: keys quantized per "channel" as against per "headdim". Reading: with
the channel geometry an NVFP4 key block is 16 consecutive tokens of one
channel inside a frozen page, quantized with the key scale mode exactly as a
16-channel block is. The pins tie it to the pinned local quantizer and to
exact arithmetic:

* with rotation and centering off, the channel geometry of a page is the
  local geometry of the transposed page (codes and scales, read back through
  both packed layouts);
* pages whose 16-token column blocks are exactly a scale times grid values
  come back exactly (amax6, and four_six choosing 4);
* the scale byte map is a bijection onto the 1024 scale bytes;
* the decode over such pages with the query and P unquantized is textbook
  softmax attention, so the dequantization indexes scales by (token block,
  channel) and not the other way round.
"""
import numpy as np
import pytest

from fp4_kv_cache_nvfp4_amd import synth
from oracle import decode as OD
from oracle import formats as F
from oracle import layout as LY
from oracle import quant as Q
from oracle import recipe as RC
from oracle import writer as W

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
CH = RC.nvfp4_default().with_(key_scale_geometry=RC.CHANNEL, tau=1.0)


def _pages(rng, npg, hkv, scale=1.0):
    return synth.f32_to_bf16((rng.standard_normal((npg * 128, hkv, 128)) * scale).astype(np.float32))


@pytest.mark.parametrize("mode", [Q.FOUR_SIX, Q.AMAX6])
def test_channel_geometry_is_local_geometry_of_transposed_page(mode):
    rng = np.random.default_rng(11)
    hkv = 2
    k = _pages(rng, 1, hkv, 3.0)
    v = _pages(rng, 1, hkv)
    rc = CH.with_(rotation=False, key_smoothing=False, scale_mode_k=mode)
    rl = rc.with_(key_scale_geometry=RC.LOCAL)
    cc = W.empty_cache(1, hkv, rc)
    W.write_pages(rc, cc, k, v, [0])
    # the transposed page: row t' = channel t' of every token
    kt = np.ascontiguousarray(k.transpose(2, 1, 0))          # [ch, h, tok]
    cl = W.empty_cache(1, hkv, rl)
    W.write_pages(rl, cl, kt, v, [0])
    for h in range(hkv):
        nib_c = LY.unpack_codes(cc["k_codes"][0, h], "k")                   # [tok, ch]
        sc_c = LY.unpack_k_scales_channel(cc["k_scales"][0, h])              # [block, ch]
        nib_l = LY.unpack_codes(cl["k_codes"][0, h], "k")                   # [ch, tok]
        sc_l = LY.unpack_scales(cl["k_scales"][0, h], "k", False)           # [ch, block]
        assert np.array_equal(nib_c, nib_l.T)
        assert np.array_equal(sc_c, sc_l.T)
    # values do not depend on the key geometry
    assert np.array_equal(cc["v_codes"], cl["v_codes"]) and np.array_equal(cc["v_scales"], cl["v_scales"])


def _on_grid_columns(rng, npg, hkv, gmax):
    """Key pages whose every (16-token, channel) block is s * g exactly, with
    s a power of two and max |g| = gmax in each block."""
    s = np.exp2(rng.integers(-4, 3, size=(npg, 8, hkv, 128))).astype(np.float32)
    g = rng.choice([x for x in GRID if x <= gmax], size=(npg, 8, 16, hkv, 128))
    g = g * rng.choice([-1.0, 1.0], size=g.shape)
    g[:, :, 0] = gmax * rng.choice([-1.0, 1.0], size=(npg, 8, hkv, 128))
    x = (g * s[:, :, None]).reshape(npg * 128, hkv, 128).astype(np.float32)
    return x


@pytest.mark.parametrize("mode,gmax", [(Q.AMAX6, 6.0), (Q.FOUR_SIX, 4.0)])
def test_on_grid_channel_blocks_round_trip(mode, gmax):
    rng = np.random.default_rng(12)
    hkv, npg = 2, 2
    k = _on_grid_columns(rng, npg, hkv, gmax)
    v = _on_grid_columns(rng, npg, hkv, 6.0)       # values use head-dim blocks; not on grid there
    r = CH.with_(rotation=False, key_smoothing=False, scale_mode_k=mode)
    cache = W.empty_cache(3, hkv, r)
    W.write_pages(r, cache, synth.f32_to_bf16(k), synth.f32_to_bf16(v), [2, 0])
    for i, p in enumerate((2, 0)):
        for h in range(hkv):
            kh, _ = W.read_page_head(r, cache, p, h)
            assert np.array_equal(kh, k[i * 128:(i + 1) * 128, h].astype(np.float64))
    # local geometry on the same pages is not exact: the blocks really run along tokens
    rl = r.with_(key_scale_geometry=RC.LOCAL)
    cl = W.empty_cache(3, hkv, rl)
    W.write_pages(rl, cl, synth.f32_to_bf16(k), synth.f32_to_bf16(v), [2, 0])
    kl, _ = W.read_page_head(rl, cl, 2, 0)
    assert not np.array_equal(kl, k[:128, 0].astype(np.float64))


def test_channel_scale_map_is_a_bijection():
    b = np.arange(8)[:, None]
    c = np.arange(128)[None, :]
    idx = LY.k_scale_byte_channel(b, c).reshape(-1)
    assert np.array_equal(np.sort(idx), np.arange(1024))
    sc = np.random.default_rng(0).integers(0, 127, size=(3, 8, 128)).astype(np.uint8)
    assert np.array_equal(LY.unpack_k_scales_channel(LY.pack_k_scales_channel(sc)), sc)


def test_channel_decode_of_on_grid_pages_is_textbook():
    rng = np.random.default_rng(13)
    hkv, G = 2, 4
    wl = synth.decode_workload("g", 14, [640, 300], hkv * G, hkv, "tiny", extra_pages=1)
    for b in range(wl.batch):
        L = int(wl.seq_lens[b])
        n = -(-L // 128)
        wl.k_tokens[b] = synth.f32_to_bf16(_on_grid_columns(rng, n, hkv, 6.0)[:L])
        # values on the head-dim grid: one power-of-two scale per 16 channels
        s = np.exp2(rng.integers(-3, 2, size=(L, hkv, 8))).astype(np.float32)
        g = rng.choice(GRID, size=(L, hkv, 8, 16)) * rng.choice([-1.0, 1.0], size=(L, hkv, 8, 16))
        g[..., 0] = 6.0
        wl.v_tokens[b] = synth.f32_to_bf16((g * s[..., None]).reshape(L, hkv, 128).astype(np.float32))
    r = CH.with_(rotation=False, key_smoothing=False, scale_mode_k=Q.AMAX6, scale_mode_q=Q.NONE,
                 scale_mode_p=Q.NONE)
    cache = W.empty_cache(wl.num_pages, hkv, r)
    k, v, ids = wl.writer_inputs()
    W.write_pages(r, cache, k, v, ids)
    sk, sv, tk, tv = wl.sink_tail()
    got = OD.decode(r, cache, wl.q, wl.block_tables, wl.seq_lens, sk, sv, tk, tv, None, wl.sigma, 2)
    q = F.bf16_to_f32(wl.q)
    for b in range(wl.batch):
        L = int(wl.seq_lens[b])
        kf = F.bf16_to_f32(wl.k_tokens[b])
        vf = F.bf16_to_f32(wl.v_tokens[b])
        for h in range(hkv):
            ref = OD.textbook_attention(q[b, h * G:(h + 1) * G], kf[:L, h], vf[:L, h], wl.sigma)
            assert np.max(np.abs(got[b, h * G:(h + 1) * G] - ref)) <= 1e-12


def test_channel_geometry_validation():
    RC.validate(CH)
    RC.validate(CH.with_(scale_mode_k=Q.AMAX6))
    with pytest.raises(RC.RecipeError):
        RC.validate(RC.mxfp4_default().with_(tau=1.0, key_scale_geometry=RC.CHANNEL))
    with pytest.raises(RC.RecipeError):
        RC.validate(CH.with_(key_scale_geometry="headdim_by_token"))
