"""GPU decode parity through the C ABI against the float64 oracle on the same
quantized operands and the same split plan: max-abs <= 2e-3 and relative L2
<= 1e-3 on float32 outputs. Covers the tiny 2K case, ragged batches (sink
only, sink + tail, several partitions with a ragged last one), sink lengths,
the MXFP4 recipe, one query term, c = 1, tau = 0 and the amax6 P mode,
rotated values (NVFP4 and MXFP4, ragged batch included), P normalised by
the running block maximum (ragged batches with sink 16 and 112 included), the
32K Qwen3-4B-shaped layer with a 77-token tail and the full 128K layer in the
benchmark's launch configuration (every KV head), each for NVFP4 and MXFP4, long contexts at one
page per partition (the final merge over several batches of partials), 16 sequences of
2K..16K tokens (every sequence), determinism, paging
invariance, invalid inputs (NaN rows), the end-to-end writer + decode path,
16 seeded random shapes and recipes, the channel key scale geometry (recipe
variants, ragged batches at 1, 2 and 3 pages per partition, the 32K layer,
6 seeded random shapes through the HIP writer) and the BF16-KV baseline arm."""
import numpy as np
import pytest
import torch

import fp4_kv_cache_nvfp4_amd as bd
from fp4_kv_cache_nvfp4_amd import synth
from oracle import decode as OD
from oracle import quant as Q
from oracle import recipe as RC
from oracle import writer as OW

import oracle_pool as OP
from gpu_helpers import (assert_close, cache_to_dev, dev, dev_bf16, gpu_decode, gpu_write,
                         oracle_decode, oracle_write, to_c, TICKET_BYTES)

pytestmark = pytest.mark.gpu

NV = RC.nvfp4_default().with_(tau=1.0)
MX = RC.mxfp4_default().with_(tau=1.0)


def _run(r, wl, ppp, what):
    print(f"[decode] {what}", flush=True)
    host = oracle_write(r, wl)
    ref = oracle_decode(r, wl, host, ppp)
    got = gpu_decode(r, wl, cache_to_dev(r, host, wl.num_kv_heads), ppp)
    assert_close(got, ref, what)
    return got, ref, host


@pytest.mark.parametrize("ppp", [4, 1, 3, 2])
def test_tiny_2k(ppp):
    _run(NV, synth.tiny(0), ppp, f"tiny ppp={ppp}")


def test_tiny_2k_mxfp4():
    _run(MX, synth.tiny(0), 4, "tiny mxfp4")


@pytest.mark.parametrize("variant", ["terms1", "c1", "tau0", "p_amax6", "k_amax6", "norot", "nosmooth", "rotv",
                                     "rotv_mx", "runmax", "runmax_tau0", "kchan", "kchan_amax6", "kchan_terms1",
                                     "kchan_p_amax6"])
def test_recipe_variants(variant):
    r = {"terms1": NV.with_(query_terms=1), "c1": NV.with_(c=1), "tau0": NV.with_(tau=0.0),
         "p_amax6": NV.with_(scale_mode_p=Q.AMAX6), "k_amax6": NV.with_(scale_mode_k=Q.AMAX6),
         "norot": NV.with_(rotation=False), "nosmooth": NV.with_(key_smoothing=False),
         "rotv": NV.with_(rotate_v=True), "rotv_mx": MX.with_(rotate_v=True),
         "runmax": NV.with_(p_running_max=True), "runmax_tau0": NV.with_(p_running_max=True, tau=0.0),
         "kchan": NV.with_(key_scale_geometry=RC.CHANNEL),
         "kchan_amax6": NV.with_(key_scale_geometry=RC.CHANNEL, scale_mode_k=Q.AMAX6),
         "kchan_terms1": NV.with_(key_scale_geometry=RC.CHANNEL, query_terms=1),
         "kchan_p_amax6": NV.with_(key_scale_geometry=RC.CHANNEL, scale_mode_p=Q.AMAX6)}[variant]
    wl = synth.decode_workload("v", 3, [1500, 777], 8, 2, "qwen", extra_pages=1)
    _run(r, wl, 2, variant)


@pytest.mark.parametrize("sink", [0, 16, 112])
def test_ragged_batch(sink):
    # L = 1 (sink only), 100 (< one page), 300 (2 pages + 44 tail), 2049 (16 pages + 1), 640 (5 pages)
    wl = synth.decode_workload("r", 4, [1, 100, 300, 2049, 640], 8, 2, "tiny", extra_pages=2, sink_tokens=sink)
    _run(NV.with_(sink_tokens=sink), wl, 3, f"ragged sink={sink}")


def test_ragged_batch_rotated_values():
    # sequences with no full page (BF16 only, written directly) beside ones
    # whose merged output is rotated back
    wl = synth.decode_workload("r", 6, [1, 100, 300, 2049, 640], 8, 2, "qwen", extra_pages=2)
    _run(NV.with_(rotate_v=True), wl, 3, "ragged rotate_v")


@pytest.mark.parametrize("sink", [16, 112])
def test_ragged_batch_running_max(sink):
    # leading blocks of sink slots only (no running maximum yet), ragged tails
    wl = synth.decode_workload("r", 7, [1, 100, 300, 2049, 640], 8, 2, "qwen", extra_pages=2, sink_tokens=sink)
    _run(NV.with_(p_running_max=True, sink_tokens=sink), wl, 3, f"ragged running max sink={sink}")


@pytest.mark.parametrize("seed", range(16))
def test_random_shapes(seed):
    # seeded random shapes: batch, lengths (ragged pages, sequences shorter
    # than the sink or a page), KV heads, sink, pages per partition, recipe
    # (NVFP4 / MXFP4, one or two query terms, tau, c), the HIP writer's pages
    rng = np.random.default_rng(1000 + seed)
    batch = int(rng.integers(1, 5))
    hkv = int(rng.choice([1, 2, 3]))
    sink = int(rng.choice([0, 16, 48, 112]))
    lens = [int(x) for x in rng.integers(1, 3000, size=batch)]
    ppp = int(rng.integers(1, 5))
    base = MX if rng.random() < 0.4 else NV
    r = base.with_(sink_tokens=sink, query_terms=int(rng.choice([1, 2])), tau=float(rng.choice([0.0, 0.5, 1.0, 4.0])),
                   c=int(rng.choice([1, 8])))
    wl = synth.decode_workload("rand", 2000 + seed, lens, 4 * hkv, hkv, "qwen",
                               extra_pages=int(rng.integers(0, 3)), sink_tokens=sink)
    what = f"random seed={seed}: B={batch} L={lens} hkv={hkv} sink={sink} ppp={ppp} {'mx' if base is MX else 'nv'}"
    print(f"[decode] {what}", flush=True)
    host = oracle_write(r, wl)
    ref = oracle_decode(r, wl, host, ppp)
    got = gpu_decode(r, wl, gpu_write(r, wl), ppp)
    assert_close(got, ref, what)


@pytest.mark.parametrize("seed", range(8))
def test_large_random_grids(seed):
    """Seeded batches whose grids leave the small-launch paths, 4, 8 or 3 KV
    heads by seed (with 3, a head's workgroups span XCDs): even seeds
    sequences of 3K-8K tokens at one page per partition (13-16 FP4
    workgroups per head, 312-640 in all: BF16 workgroups of their own,
    dispatched after the FP4 columns, and heads of up to 64 partials); odd
    seeds 160-250 (sequence, KV head) pairs of 1-6000 tokens at two pages per
    partition (a grid of 1,000-1,400 workgroups: compacted, last columns
    last, the BF16 partition folded, odd partial counts). NVFP4, MXFP4 or NVFP4 with
    channel key scales by seed; random sink, query terms and tau; every
    output row against the oracle."""
    hkv = [4, 8, 3][seed % 3]
    rng = np.random.default_rng(5000 + seed)
    if seed % 2 == 0:
        B, ppp = int(rng.integers(max(1, 24 // hkv), max(2, 44 // hkv))), 1
        lens = [int(x) for x in rng.integers(3000, 8192, size=B)]
    else:
        B, ppp = int(rng.integers(160 // hkv, 252 // hkv)), 2
        lens = [int(x) for x in rng.integers(1, 6000, size=B)]
    sink = int(rng.choice([0, 16, 48]))
    kind = ["nv", "mx", "chan"][seed % 3]
    base = MX if kind == "mx" else (NV.with_(key_scale_geometry=RC.CHANNEL) if kind == "chan" else NV)
    r = base.with_(sink_tokens=sink, query_terms=int(rng.choice([1, 2])), tau=float(rng.choice([0.5, 1.0, 4.0])))
    wl = synth.decode_workload("large", 6000 + seed, lens, 4 * hkv, hkv, "qwen", extra_pages=1, sink_tokens=sink)
    what = f"large grid seed={seed}: B={B} hkv={hkv} max L={max(lens)} ppp={ppp} sink={sink} {kind}"
    print(f"[decode] {what}", flush=True)
    host = oracle_write(r, wl)
    ref = oracle_decode(r, wl, host, ppp)
    got = gpu_decode(r, wl, cache_to_dev(r, host, hkv), ppp)
    assert_close(got, ref, what)


@pytest.mark.parametrize("ppp", [1, 2, 3])
def test_ragged_batch_channel_geometry(ppp):
    # the channel key scale geometry over ragged lengths, every page-slot count
    wl = synth.decode_workload("r", 8, [1, 100, 300, 2049, 640], 8, 2, "qwen", extra_pages=2)
    _run(NV.with_(key_scale_geometry=RC.CHANNEL), wl, ppp, f"ragged channel geometry ppp={ppp}")


@pytest.mark.parametrize("seed", range(6))
def test_random_shapes_channel_geometry(seed):
    rng = np.random.default_rng(3000 + seed)
    batch = int(rng.integers(1, 4))
    hkv = int(rng.choice([1, 2]))
    sink = int(rng.choice([0, 16, 112]))
    lens = [int(x) for x in rng.integers(1, 2600, size=batch)]
    ppp = int(rng.integers(1, 5))
    r = NV.with_(key_scale_geometry=RC.CHANNEL, sink_tokens=sink, query_terms=int(rng.choice([1, 2])),
                 scale_mode_k=str(rng.choice([Q.FOUR_SIX, Q.AMAX6])), tau=float(rng.choice([0.0, 1.0, 4.0])))
    wl = synth.decode_workload("randc", 4000 + seed, lens, 4 * hkv, hkv, "qwen", sink_tokens=sink)
    what = f"random channel geometry seed={seed}: B={batch} L={lens} hkv={hkv} sink={sink} ppp={ppp}"
    print(f"[decode] {what}", flush=True)
    host = oracle_write(r, wl)
    ref = oracle_decode(r, wl, host, ppp)
    got = gpu_decode(r, wl, gpu_write(r, wl), ppp)
    assert_close(got, ref, what)


def test_ragged_batch_mxfp4():
    wl = synth.decode_workload("r", 5, [129, 1000, 4096 + 77], 12, 3, "qwen", extra_pages=2)
    _run(MX, wl, 3, "ragged mxfp4")


@pytest.mark.parametrize("r", [NV, MX, NV.with_(key_scale_geometry=RC.CHANNEL)],
                         ids=["nvfp4", "mxfp4", "nvfp4_channel_geometry"])
def test_qwen_32k_layer(r):
    """32 query / 8 KV heads, 256 full pages + 77-token tail, permuted pool."""
    wl = synth.qwen_32k(0)
    ppp, _ = bd.decode_plan(1, 8, int(wl.seq_lens[0]), 0)
    _run(r, wl, ppp, f"qwen 32k ppp={ppp}")


@pytest.mark.parametrize("r", [NV, MX], ids=["nvfp4", "mxfp4"])
def test_determinism_and_paging_invariance(r):
    wl = synth.decode_workload("d", 6, [3000, 1234], 8, 2, "qwen", extra_pages=4)
    host = oracle_write(r, wl)
    cache = cache_to_dev(r, host, 2)
    a, b = gpu_decode(r, wl, cache, 2, repeat=2)
    assert np.array_equal(a, b)
    # move every physical page to a new slot and remap the tables
    perm = np.random.default_rng(0).permutation(wl.num_pages)
    moved = {k: np.empty_like(v) for k, v in host.items()}
    for k in host:
        moved[k][perm] = host[k]
    c = gpu_decode(r, wl, cache_to_dev(r, moved, 2), 2, block_tables=perm[wl.block_tables].astype(np.int32))
    assert np.array_equal(a, c)


@pytest.mark.parametrize("r", [NV, MX], ids=["nvfp4", "mxfp4"])
def test_invalid_inputs_give_nan_rows(r):
    wl = synth.decode_workload("n", 8, [700, 600, 500], 8, 2, "tiny", extra_pages=1)
    host = oracle_write(r, wl)
    cache = cache_to_dev(r, host, 2)
    ref = oracle_decode(r, wl, host, 2)
    sl = wl.seq_lens.copy()
    sl[1] = 0                                   # empty sequence
    bt = wl.block_tables.copy()
    bt[2, 1] = wl.num_pages + 7                 # page outside the pool
    got = gpu_decode(r, wl, cache, 2, max_seq_len=700, seq_lens=sl, block_tables=bt)
    assert np.all(np.isnan(got[1])) and np.all(np.isnan(got[2]))
    assert_close(got[0], ref[0], "valid row next to invalid ones")
    # a length above max_seq_len is rejected on the device too
    sl2 = wl.seq_lens.copy()
    got2 = gpu_decode(r, wl, cache, 2, max_seq_len=600, seq_lens=sl2)
    assert np.all(np.isnan(got2[0])) and np.all(np.isfinite(got2[1:]))


def test_workspace_reuse_across_shapes():
    """Tickets return to zero: one workspace serves different batches back to back."""
    big = synth.decode_workload("a", 9, [2000, 900, 129], 8, 2, "tiny", extra_pages=1)
    small = synth.decode_workload("b", 10, [700], 8, 2, "tiny")
    ws = bd.alloc_workspace(bd.decode_workspace_size(3, 8, 2, 2048, 1))
    for wl in (big, small, big):
        host = oracle_write(NV, wl)
        ref = oracle_decode(NV, wl, host, 1)
        rc = to_c(NV)
        sk, sv, tk, tv = wl.sink_tail()
        out = torch.empty((wl.batch, 8, 128), dtype=torch.float32, device="cuda")
        bd.decode_attention(rc, cache_to_dev(NV, host, 2), dev_bf16(wl.q), dev(wl.block_tables),
                            dev(wl.seq_lens), int(wl.seq_lens.max()), dev_bf16(sk), dev_bf16(sv), dev_bf16(tk),
                            dev_bf16(tv), dev(wl.key_shift), wl.sigma, 1, ws, out)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy().astype(np.float64), ref, f"reuse {wl.name}")
    assert not ws[:TICKET_BYTES].any()


def test_odd_partial_count_after_poisoned_call():
    """Partials are stored in slot pairs, so with an odd count n the merge's
    loads of the last pair also bring slot n, which still holds whatever an
    earlier call left there. Here an earlier call on the same workspace left
    a NaN partial in slot 3 of sequence 0 (an invalid page in its fourth FP4
    workgroup; a grid larger than the chip holds, so the BF16 partition is
    folded and slot 3 is no BF16 slot); the next call merges 3 partials for
    that sequence, and every row must match the oracle."""
    print("[odd partial count after a poisoned call] 48 x 8, ppp 1", flush=True)
    lens1 = [16 * 128] + [200] * 47
    lens2 = [12 * 128 + 50] + [200] * 47
    wl1 = synth.decode_workload("odd1", 41, lens1, 32, 8, "qwen", extra_pages=1)
    wl2 = synth.decode_workload("odd2", 42, lens2, 32, 8, "qwen")
    msl = 16 * 128
    ws = bd.alloc_workspace(bd.decode_workspace_size(48, 32, 8, msl, 1))
    rc = to_c(NV)
    outs = []
    for wl, poison in ((wl1, True), (wl2, False)):
        host = oracle_write(NV, wl)
        bt = np.zeros((48, 16), dtype=np.int32)          # both calls: 16 block-table columns
        bt[:, :wl.block_tables.shape[1]] = wl.block_tables
        if poison:
            bt[0, 13] = wl.num_pages + 7                 # a page outside the pool, FP4 workgroup 3's
        sk, sv, tk, tv = wl.sink_tail()
        out = torch.empty((48, 32, 128), dtype=torch.float32, device="cuda")
        bd.decode_attention(rc, cache_to_dev(NV, host, 8), dev_bf16(wl.q), dev(bt), dev(wl.seq_lens), msl,
                            dev_bf16(sk), dev_bf16(sv), dev_bf16(tk), dev_bf16(tv), dev(wl.key_shift), wl.sigma, 1,
                            ws, out)
        torch.cuda.synchronize()
        outs.append((wl, host, out.cpu().numpy().astype(np.float64)))
    wl, host, got = outs[0]
    assert np.all(np.isnan(got[0]))
    wl, host, got = outs[1]
    assert_close(got, oracle_decode(NV, wl, host, 1), "3 partials after a NaN partial in slot 3")
    assert not ws[:TICKET_BYTES].any()


@pytest.mark.parametrize("r", [NV, MX], ids=["nvfp4", "mxfp4"])
def test_end_to_end_writer_then_decode(r):
    wl = synth.decode_workload("e", 12, [5000, 2300], 16, 4, "qwen", extra_pages=2)
    cache = gpu_write(r, wl)
    ref = oracle_decode(r, wl, oracle_write(r, wl), 4)
    assert_close(gpu_decode(r, wl, cache, 4), ref, "end to end")


@pytest.mark.parametrize("ppp", [1, 4, 8, 16, 0])
def test_bf16_baseline(ppp):
    wl = synth.decode_workload("b", 13, [1, 127, 128, 1000, 2100], 8, 2, "qwen", extra_pages=2)
    kp, vp = wl.bf16_pages()
    ref = OD.bf16_decode(wl.q, kp, vp, wl.block_tables, wl.seq_lens, wl.sigma)
    msl = int(wl.seq_lens.max())
    ws = bd.alloc_workspace(bd.decode_workspace_size(wl.batch, 8, 2, msl, ppp))
    out = torch.empty((wl.batch, 8, 128), dtype=torch.float32, device="cuda")
    bd.bf16_decode_attention(dev_bf16(wl.q), dev_bf16(kp), dev_bf16(vp), dev(wl.block_tables),
                             dev(wl.seq_lens), msl, wl.sigma, ppp, ws, out)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy().astype(np.float64), ref, f"bf16 baseline ppp={ppp}")


@pytest.mark.parametrize("r", [NV, MX], ids=["nvfp4", "mxfp4"])
def test_full_128k_layer(r):
    """The headline shape in the launch configuration the benchmark times:
    batch 1, 131,072 tokens, 32 query / 8 KV heads, the library's own split
    plan (4 pages per partition: 512 FP4 workgroups, plus the BF16-partition
    workgroups where the occupancy leaves room). The HIP writer and decode run
    on all 8 KV heads; the oracle writes and decodes all 8 from the same
    seeded inputs, and every one of the 32 query-head rows is compared."""
    L = 131072
    print(f"[128k layer] {r.scale_mode_k}", flush=True)
    wl = synth.decode_workload("full128k", 11, [L], 32, 8, "qwen")
    ppp, parts = bd.decode_plan(1, 8, L, 0)
    assert (ppp, parts) == (4, 256)
    got = gpu_decode(r, wl, gpu_write(r, wl), ppp)
    k, v, ids = wl.writer_inputs()
    cache = OW.empty_cache(wl.num_pages, 8, r)
    OP.write_pages(r, cache, k, v, ids, wl.key_shift)
    sk, sv, tk, tv = wl.sink_tail()
    ref = OD.decode(r, cache, wl.q, wl.block_tables, wl.seq_lens, sk, sv, tk, tv, wl.key_shift, wl.sigma, ppp)
    assert_close(got, ref, "128k layer, all 8 KV heads")


def test_bf16_full_128k_layer():
    """The BF16-KV arm on the benchmark's 128K layer in its own automatic
    plan (16 pages per partition: 64 workgroups per KV head, 512 in all);
    every one of the 32 output rows against the oracle's exact attention."""
    L = 131072
    print("[128k layer] bf16", flush=True)
    wl = synth.decode_workload("full128k", 11, [L], 32, 8, "qwen")
    ppp, parts = bd.bf16_decode_plan(1, 8, L, 0)
    assert (ppp, parts) == (16, 64)
    kp, vp = wl.bf16_pages()
    ref = OD.bf16_decode(wl.q, kp, vp, wl.block_tables, wl.seq_lens, wl.sigma)
    ws = bd.alloc_workspace(bd.decode_workspace_size(1, 32, 8, L, 0))
    out = torch.full((1, 32, 128), float("nan"), dtype=torch.float32, device="cuda")
    bd.bf16_decode_attention(dev_bf16(wl.q), dev_bf16(kp), dev_bf16(vp), dev(wl.block_tables),
                             dev(wl.seq_lens), L, wl.sigma, 0, ws, out)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy().astype(np.float64), ref, "bf16 128k layer, auto plan")
    assert not ws[:TICKET_BYTES].any()


@pytest.mark.parametrize("r", [NV, MX], ids=["nvfp4", "mxfp4"])
def test_many_workgroups_per_head(r):
    """One page per partition over long contexts: 250 and 75 workgroups per
    (sequence, KV head), so the final merge takes its partials in several
    batches of 64 (64 + 64 + 64 + 58 and 64 + 11) and rescales the earlier
    batches; a 50-token and a 1-token tail, sink 16, every output row
    compared."""
    lens = [128 * 1000 + 50, 128 * 300 + 1]
    wl = synth.decode_workload("many_wgs", 23, lens, 4, 1, "qwen")
    ppp, parts = bd.decode_plan(2, 1, max(lens), 1)
    assert (ppp, parts) == (1, 1000)
    _run(r, wl, ppp, f"many workgroups per head, L={lens}, ppp=1")


def test_batched_16_sequences():
    """16 sequences with lengths drawn from 2K..16K over one shuffled pool,
    the library's own plan for the batch. The HIP path writes and decodes
    the whole batch; the oracle writes and decodes every sequence and KV
    head from the same inputs, and every output row is compared."""
    print("[batched 16]", flush=True)
    wl = synth.batched(0)
    B, msl = wl.batch, int(wl.seq_lens.max())
    ppp, _ = bd.decode_plan(B, 8, msl, 0)
    got = gpu_decode(NV, wl, gpu_write(NV, wl), ppp)
    cache = OW.empty_cache(wl.num_pages, 8, NV)
    full = [wl.full_pages(b) for b in range(B)]
    OP.write_pages(NV, cache, np.concatenate([wl.k_tokens[b][:n * 128] for b, n in enumerate(full)]),
                   np.concatenate([wl.v_tokens[b][:n * 128] for b, n in enumerate(full)]),
                   np.concatenate([wl.block_tables[b, :n] for b, n in enumerate(full)]), wl.key_shift)
    sk, sv, tk, tv = wl.sink_tail()
    ref = OD.decode(NV, cache, wl.q, wl.block_tables, wl.seq_lens, sk, sv, tk, tv, wl.key_shift, wl.sigma, ppp)
    assert_close(got, ref, f"batched 16 x 2k..16k ppp={ppp}, every sequence")


def test_compacted_grid():
    """A batch whose grid of every (sequence, KV head, column) exceeds what the
    chip holds at once (48 sequences x 8 KV heads x 3 columns against 768
    resident workgroups), so the launch is compacted: workgroup j serves the
    j-th unit with work. Sequences of every kind side by side: no full page
    (the BF16 partition alone), one to three FP4 workgroups, an empty one, one
    longer than max_seq_len and one whose block table names a page outside
    the pool (their rows NaN); every other row against the oracle."""
    print("[compacted grid] 48 x 8", flush=True)
    rng = np.random.Generator(np.random.PCG64(96))
    lens = rng.integers(1, 6000, 48).astype(np.int32)
    lens[::11] = rng.integers(1, 128, lens[::11].size)
    wl = synth.decode_workload("compact", 31, lens, 32, 8, "qwen", extra_pages=1)
    ppp, parts = bd.decode_plan(48, 8, 6000, 0)
    assert (ppp, parts) == (4, 12)                      # 3 FP4 workgroups per (sequence, KV head)
    host = oracle_write(NV, wl)
    ref = oracle_decode(NV, wl, host, ppp)
    cache = cache_to_dev(NV, host, 8)
    sl = wl.seq_lens.copy()
    bt = wl.block_tables.copy()
    victim = int([b for b in np.flatnonzero(sl >= 3 * 128) if b not in (5, 7)][2])
    sl[5] = 0                                          # empty
    sl[7] = 6500                                       # above max_seq_len
    bt[victim, 2] = wl.num_pages + 7                   # a page outside the pool
    got = gpu_decode(NV, wl, cache, ppp, max_seq_len=6000, seq_lens=sl, block_tables=bt)
    bad = [5, 7, victim]
    assert all(np.all(np.isnan(got[b])) for b in bad)
    good = np.setdiff1d(np.arange(48), bad)
    assert_close(got[good], ref[good], "compacted grid, 45 valid sequences")


def test_max_sequence_heads():
    """The largest call the library takes: 2,048 sequences x 8 KV heads =
    16,384 (sequence, KV head) pairs, every ticket word in use. Most
    sequences are shorter than a page (the BF16 partition alone), 64 hold
    1-4 full pages, 16 hold 17-23 (two FP4 workgroups of the plan's 4 pages
    per partition, so tickets and the merge run at the top of the ticket
    region). The FP4 and the BF16-KV decode against the oracle on every
    sequence, and the ticket words are zero again after each call."""
    print("[max sequence heads] 2048 x 8", flush=True)
    rng = np.random.Generator(np.random.PCG64(2048))
    lens = np.concatenate([rng.integers(1, 128, 1968), rng.integers(128, 601, 64), rng.integers(2200, 3001, 16)])
    lens = lens[rng.permutation(lens.size)].astype(np.int32)
    wl = synth.decode_workload("max_seq_heads", 29, lens, 32, 8, "qwen")
    assert wl.batch * wl.num_kv_heads == 16384
    ppp, parts = bd.decode_plan(wl.batch, 8, int(lens.max()), 0)
    assert (ppp, parts) == (4, 6)
    ref = oracle_decode(NV, wl, oracle_write(NV, wl), ppp)
    ws = bd.alloc_workspace(bd.decode_workspace_size(wl.batch, 32, 8, int(lens.max()), 0))
    cache = gpu_write(NV, wl)
    sk, sv, tk, tv = wl.sink_tail()
    out = torch.full((wl.batch, 32, 128), float("nan"), dtype=torch.float32, device="cuda")
    bd.decode_attention(to_c(NV), cache, dev_bf16(wl.q), dev(wl.block_tables), dev(wl.seq_lens), int(lens.max()),
                        dev_bf16(sk), dev_bf16(sv), dev_bf16(tk), dev_bf16(tv), dev(wl.key_shift), wl.sigma, ppp,
                        ws, out)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy().astype(np.float64), ref, "16,384 (sequence, KV head) pairs")
    assert not ws[:TICKET_BYTES].any()
    kp, vp = wl.bf16_pages()
    ref16 = OD.bf16_decode(wl.q, kp, vp, wl.block_tables, wl.seq_lens, wl.sigma)
    assert bd.bf16_decode_plan(wl.batch, 8, int(lens.max()), 0) == (16, 2)
    out.fill_(float("nan"))
    bd.bf16_decode_attention(dev_bf16(wl.q), dev_bf16(kp), dev_bf16(vp), dev(wl.block_tables), dev(wl.seq_lens),
                             int(lens.max()), wl.sigma, 0, ws, out)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy().astype(np.float64), ref16, "bf16, 16,384 (sequence, KV head) pairs")
    assert not ws[:TICKET_BYTES].any()


def test_p_flips_from_float32_logits():
    """P code and scale flips: the decode's own float32 logits
    (bdfp4_decode_attention_logits) and the oracle's float64 logits, both
    turned into float32 p' by the oracle (oracle.decode.p_prime) and fed
    through its P quantizer (same partitions, maxima, c and tau). The float32
    logits agree with the float64 ones to accumulation rounding, and the
    fraction of P codes or block scales that this rounding changes is
    reported and bounded."""
    from oracle import formats as F
    from oracle import writer as W
    r = NV
    cases = (("tiny 2K", synth.tiny(0), 1),
             ("ragged", synth.decode_workload("pf", 21, [3000, 1234, 640], 8, 2, "qwen", extra_pages=2), 2),
             ("batch of 16", synth.batched(0), 4))
    for what, wl, ppp in cases:
        host = oracle_write(r, wl)
        cache = cache_to_dev(r, host, wl.num_kv_heads)
        B, Hq, hkv = wl.batch, wl.num_q_heads, wl.num_kv_heads
        maxp = wl.block_tables.shape[1]
        msl = int(wl.seq_lens.max())
        sk, sv, tk, tv = wl.sink_tail()
        ws = bd.alloc_workspace(bd.decode_workspace_size(B, Hq, hkv, msl, ppp))
        out = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")
        lg = torch.full((B, hkv, 4, 128 * maxp), float("nan"), dtype=torch.float32, device="cuda")
        bd.decode_attention_logits(to_c(r), cache, dev_bf16(wl.q), dev(wl.block_tables.astype(np.int32)),
                                   dev(wl.seq_lens.astype(np.int32)), msl, dev_bf16(sk), dev_bf16(sv), dev_bf16(tk),
                                   dev_bf16(tv), dev(wl.key_shift), wl.sigma, ppp, ws, out, lg)
        torch.cuda.synchronize()
        lg = lg.cpu().numpy().astype(np.float64)
        q = F.bf16_to_f32(wl.q)
        n_el = n_blk = flip_el = flip_blk = 0
        worst = 0.0
        for b in range(B):
            L = int(wl.seq_lens[b])
            n_full, _, parts = OD.split_plan(L, r.sink_tokens, ppp)
            if n_full == 0:
                continue
            for h in range(hkv):
                qg = q[b, 4 * h:4 * h + 4]
                qhat = OD.query_hat(r, qg)
                qmu = qg.astype(np.float64) @ wl.key_shift[h].astype(np.float64)
                khat = np.concatenate([W.read_page_head(r, host, int(wl.block_tables[b, i]), h)[0]
                                       for i in range(n_full)])
                raw_o = qhat @ khat.T + qmu[:, None]
                raw_g = lg[b, h, :, :n_full * 128]
                for lo, hi in parts:
                    d = np.abs(raw_g[:, lo:hi] - raw_o[:, lo:hi])
                    worst = max(worst, float(np.max(d / np.maximum(1.0, np.abs(raw_o[:, lo:hi])))))
                    res = []
                    for raw in (raw_o, raw_g):
                        x = raw[:, lo:hi]
                        pp = OD.p_prime(r, wl.sigma, x, x.astype(np.float32).max(axis=1))
                        res.append(Q.quantize_p(pp, r.scale_mode_p, np.float32(r.tau)))
                    flip_el += int(np.count_nonzero(res[0][0] != res[1][0]))
                    flip_blk += int(np.count_nonzero(res[0][1] != res[1][1]))
                    n_el += res[0][0].size
                    n_blk += res[0][1].size
        print(f"[p flips] {what}: logits max rel diff {worst:.2e}; P codes {flip_el}/{n_el} differ, "
              f"block scales {flip_blk}/{n_blk}", flush=True)
        assert worst <= 1e-5, (what, worst)
        assert flip_el <= 1e-3 * n_el and flip_blk <= 1e-3 * n_blk, (what, flip_el, flip_blk)
