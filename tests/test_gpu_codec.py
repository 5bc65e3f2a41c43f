"""GPU codec parity through the C ABI: the row quantizer (key / query path:
shift, rotation, amax6 / four_six / mxfp4_search, two residual terms) and the
probability quantizer (amax2_or_amax6 with tau, amax6) and the decode's own
query prologue (bdfp4_decode_query_codes) against the oracle, bit for bit,
including ties, zero blocks, subnormal and saturating scales."""
import numpy as np
import pytest
import torch

import fp4_kv_cache_nvfp4_amd as bd
from fp4_kv_cache_nvfp4_amd import synth
from oracle import formats as F
from oracle import quant as Q
from oracle import writer as W

from gpu_helpers import dev, dev_bf16

pytestmark = pytest.mark.gpu

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _pack_logical(nib):
    """[..., 128] nibbles -> [..., 64] bytes, element 2i in the low nibble."""
    nib = nib.astype(np.uint8)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


def _rows(seed, n):
    """A mix of row types: normal, outlier channels, tiny, huge, on-grid, zeros."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 128)).astype(np.float32)
    x[0::7, rng.integers(0, 128, 4)] += 10.0
    x[1::7] *= 1e-4
    x[2::7] *= 300.0
    x[2::14] *= 10.0                        # saturating E4M3 scales
    x[3::7] = 0.0
    x[4::7, :16] = 0.0
    g = rng.choice(GRID, size=(n, 128)) * rng.choice([-1.0, 1.0], size=(n, 128))
    x[5::7] = (g[5::7] * 0.375).astype(np.float32)
    x[6::7] = rng.integers(-12, 13, size=x[6::7].shape) * np.float32(0.25)   # many exact ties
    return synth.f32_to_bf16(x)


@pytest.mark.parametrize("mode", [Q.AMAX6, Q.FOUR_SIX, Q.MXFP4_SEARCH])
@pytest.mark.parametrize("rotation,shift", [(False, False), (True, False), (True, True)])
@pytest.mark.parametrize("terms", [1, 2])
def test_rows_bit_exact(mode, rotation, shift, terms):
    n = 4099                                  # several workgroups and a ragged tail
    u = _rows(11, n)
    mu = (np.random.default_rng(3).standard_normal(128) * 2).astype(np.float32) if shift else None
    cmode = {Q.AMAX6: bd.SCALE_AMAX6, Q.FOUR_SIX: bd.SCALE_FOUR_SIX, Q.MXFP4_SEARCH: bd.SCALE_MXFP4_SEARCH}[mode]
    nb = 4 if mode == Q.MXFP4_SEARCH else 8
    codes = torch.zeros((n, terms, 64), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((n, terms, nb), dtype=torch.uint8, device="cuda")
    bd.quantize_rows(dev_bf16(u), dev(mu) if shift else None, int(rotation), cmode, terms, codes, scales)
    torch.cuda.synchronize()
    gc, gs = codes.cpu().numpy(), scales.cpu().numpy()
    y = W.key_rows(F.bf16_to_f32(u), mu, rotation)
    if terms == 1:
        nib, sc = Q.quantize(y, mode)
        want = [(nib, sc)]
    else:
        want, _ = Q.quantize_query(y, mode, 2)
    for t, (nib, sc) in enumerate(want):
        assert np.array_equal(gc[:, t], _pack_logical(nib)), f"codes term {t}"
        assert np.array_equal(gs[:, t], sc.astype(np.uint8)), f"scales term {t}"


@pytest.mark.parametrize("mode", [Q.AMAX6, Q.FOUR_SIX, Q.MXFP4_SEARCH])
def test_rows_bit_exact_near_float32_underflow(mode):
    # block maxima around 2^-126: MXFP4 candidates at the float32 subnormal
    # 2^-127 (the threshold search), beside normal power-of-two candidates;
    # E4M3 scales of such blocks are zero
    rng = np.random.default_rng(5)
    n = 300
    x = rng.standard_normal((n, 128)).astype(np.float32) * np.float32(2.0 ** -122)
    x[1::3] *= np.float32(2.0 ** -4)
    x[2::3] *= np.float32(2.0 ** -7)
    u = synth.f32_to_bf16(x)
    cmode = {Q.AMAX6: bd.SCALE_AMAX6, Q.FOUR_SIX: bd.SCALE_FOUR_SIX, Q.MXFP4_SEARCH: bd.SCALE_MXFP4_SEARCH}[mode]
    nb = 4 if mode == Q.MXFP4_SEARCH else 8
    codes = torch.zeros((n, 1, 64), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((n, 1, nb), dtype=torch.uint8, device="cuda")
    bd.quantize_rows(dev_bf16(u), None, 0, cmode, 1, codes, scales)
    torch.cuda.synchronize()
    nib, sc = Q.quantize(W.key_rows(F.bf16_to_f32(u), None, False), mode)
    assert np.array_equal(codes.cpu().numpy()[:, 0], _pack_logical(nib))
    assert np.array_equal(scales.cpu().numpy()[:, 0], sc.astype(np.uint8))


def _p_blocks(seed, n):
    rng = np.random.default_rng(seed)
    p = np.exp(-rng.exponential(2.0, size=(n, 16)))
    p[::5, 0] = 1.0
    pp = (8.0 * p).astype(np.float32)
    pp[1::9] *= np.float32(1e-3)            # small blocks: subnormal / zero scales
    pp[2::9] = 0.0
    pp[3::9] = (rng.integers(0, 25, size=(len(pp[3::9]), 16)) * 0.25).astype(np.float32)   # ties
    pp[4::9, :] = np.float32(1.0)          # a == tau exactly
    pp[5::9] *= np.float32(80.0)           # large scales (c p' up to 640)
    return pp


@pytest.mark.parametrize("mode,tau", [(Q.AMAX2_OR_AMAX6, 1.0), (Q.AMAX2_OR_AMAX6, 0.0),
                                      (Q.AMAX2_OR_AMAX6, 448.0), (Q.AMAX2_OR_AMAX6, 0.37), (Q.AMAX6, 0.0)])
def test_p_blocks_bit_exact(mode, tau):
    n = 20011
    pp = _p_blocks(5, n)
    cmode = bd.SCALE_AMAX2_OR_AMAX6 if mode == Q.AMAX2_OR_AMAX6 else bd.SCALE_AMAX6
    codes = torch.zeros((n, 8), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((n,), dtype=torch.uint8, device="cuda")
    bd.quantize_p_blocks(dev(pp), cmode, tau, codes, scales)
    torch.cuda.synchronize()
    nib, sc = Q.quantize_p(pp, mode, np.float32(tau))
    assert np.array_equal(scales.cpu().numpy(), sc[:, 0])
    assert np.array_equal(codes.cpu().numpy(), _pack_logical(nib))


@pytest.mark.parametrize("nwords,wgs", [(1, 1), (1000, 3), (4096 * 7 + 5, 512), (1 << 20, 512)])
def test_stream_read_folds_every_word_once(nwords, wgs):
    # each 16-byte word is read by exactly one thread, which xors its four
    # 32-bit lanes into its sink word: the xor of the sink is the xor of the
    # whole buffer
    g = torch.Generator().manual_seed(nwords)
    host = torch.randint(-(1 << 31), (1 << 31) - 1, (nwords * 4,), generator=g, dtype=torch.int64).to(torch.int32)
    src = host.to("cuda")
    sink = torch.full((wgs * 256,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    bd.stream_read(src, sink, wgs)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert got == want


@pytest.mark.parametrize("recipe", ["nvfp4", "nvfp4_terms1", "nvfp4_norot", "mxfp4", "mxfp4_terms1", "mxfp4_norot"])
def test_decode_query_codes_bit_exact(recipe):
    """The decode's own query prologue (bdfp4_decode_query_codes runs the same
    device function the decode runs, two elements per lane with cross-lane
    rotation stages) against the oracle's query quantizer, bit for bit."""
    from oracle import recipe as RC
    r = {"nvfp4": RC.nvfp4_default(), "nvfp4_terms1": RC.nvfp4_default().with_(query_terms=1),
         "nvfp4_norot": RC.nvfp4_default().with_(rotation=False), "mxfp4": RC.mxfp4_default(),
         "mxfp4_terms1": RC.mxfp4_default().with_(query_terms=1),
         "mxfp4_norot": RC.mxfp4_default().with_(rotation=False)}[recipe].with_(tau=1.0)
    from gpu_helpers import to_c
    hkv, B = 8, 129                            # 129 x 32 query rows of every kind (the row mix above)
    u = _rows(17, B * 4 * hkv).reshape(B, 4 * hkv, 128)
    mode = r.scale_mode_q
    nb = 4 if mode == Q.MXFP4_SEARCH else 8
    T = r.query_terms
    codes = torch.zeros((B * 4 * hkv, T, 64), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((B * 4 * hkv, T, nb), dtype=torch.uint8, device="cuda")
    bd.decode_query_codes(to_c(r), dev_bf16(u), hkv, codes, scales)
    torch.cuda.synchronize()
    gc, gs = codes.cpu().numpy(), scales.cpu().numpy()
    y = W.key_rows(F.bf16_to_f32(u.reshape(-1, 128)), None, r.rotation)     # the query is rotated, not centered
    want, _ = Q.quantize_query(y, mode, T)
    for t, (nib, sc) in enumerate(want):
        bad = np.argwhere(gc[:, t] != _pack_logical(nib))
        assert bad.size == 0, f"codes term {t}: {len(bad)} bytes differ, first rows {bad[:3, 0].tolist()}"
        assert np.array_equal(gs[:, t], sc.astype(np.uint8)), f"scales term {t}"
