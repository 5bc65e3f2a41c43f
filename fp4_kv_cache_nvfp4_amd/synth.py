"""Seeded synthetic inputs for the page writer and the decode.

This module only draws numbers and lays them out; it contains none of the
quantization or attention arithmetic, so both the HIP path and the CPU oracle
can consume what it produces. Inputs are bf16 bit patterns in uint16 arrays.

Recipe (fixed draw order per workload: outlier channels, outlier offsets, K,
V, Q, page permutation; numpy Generator(PCG64(seed))):

* K, V, Q ~ N(0, 1) in float32, rounded to bf16 (round to nearest even);
* key outliers: a seeded set of channels per KV head gets a constant offset
  added before rounding - +8 on 4 channels ("tiny"), Student-t(3) offsets on 6
  channels ("qwen"), or +-10 with seeded signs on 8 channels ("write");
* key means mu = float32(mean over all K tokens of the layer, in float64),
  per (KV head, channel), standing in for the calibrated key-shift sidecar;
* pages: logical page i of sequence b maps to a physical page through a
  per-sequence block table drawn as a random permutation of the shared pool
  (identity for the tiny workload);
* the first 16 tokens are also handed over as the BF16 sink buffer and the
  tokens after the last full page as the BF16 tail page (slot = token - 128 n).

The workloads mirror the shapes of a Qwen3-4B-style decode (32 query heads,
8 KV heads, head_dim 128, block_size 128) at the context lengths the
BitDecoding-FP4 evaluation uses (up to 131,072 tokens, batch 1); no model
weights or benchmark data are involved.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

PAGE = 128
D = 128


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 bit patterns (nearest, ties to even; finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(u16: np.ndarray) -> np.ndarray:
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class DecodeWorkload:
    """One layer of a batched paged decode, all host arrays."""
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    seq_lens: np.ndarray            # int32 [B]
    num_pages: int                  # physical pool size
    block_tables: np.ndarray        # int32 [B, max_pages_per_seq]
    k_tokens: list                  # per sequence: uint16 [L_b, Hkv, 128]
    v_tokens: list
    q: np.ndarray                   # uint16 [B, Hq, 128]
    key_shift: np.ndarray           # float32 [Hkv, 128]
    sink_tokens: int = 16
    sigma: float = float(np.float32(1.0 / np.sqrt(128.0)))
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    def full_pages(self, b: int) -> int:
        return int(self.seq_lens[b]) // PAGE

    def writer_inputs(self):
        """(k_rows, v_rows, page_ids): every full page of every sequence, in
        order, with its destination physical page."""
        ks, vs, ids = [], [], []
        for b in range(self.batch):
            n = self.full_pages(b)
            if n == 0:
                continue
            ks.append(self.k_tokens[b][: n * PAGE])
            vs.append(self.v_tokens[b][: n * PAGE])
            ids.append(self.block_tables[b, :n])
        hkv = self.num_kv_heads
        if not ks:
            e = np.zeros((0, hkv, D), dtype=np.uint16)
            return e, e.copy(), np.zeros((0,), dtype=np.int32)
        return (np.concatenate(ks), np.concatenate(vs),
                np.concatenate(ids).astype(np.int32))

    def sink_tail(self):
        """sink_k/v uint16 [B, Hkv, S, 128]; tail_k/v uint16 [B, Hkv, 128, 128]."""
        B, hkv, S = self.batch, self.num_kv_heads, self.sink_tokens
        sk = np.zeros((B, hkv, S, D), dtype=np.uint16)
        sv = np.zeros_like(sk)
        tk = np.zeros((B, hkv, PAGE, D), dtype=np.uint16)
        tv = np.zeros_like(tk)
        for b in range(B):
            L = int(self.seq_lens[b])
            n = L // PAGE
            s = min(S, L)
            sk[b, :, :s] = self.k_tokens[b][:s].transpose(1, 0, 2)
            sv[b, :, :s] = self.v_tokens[b][:s].transpose(1, 0, 2)
            lo = max(S, n * PAGE)
            if L > lo:
                tk[b, :, lo - n * PAGE:L - n * PAGE] = self.k_tokens[b][lo:L].transpose(1, 0, 2)
                tv[b, :, lo - n * PAGE:L - n * PAGE] = self.v_tokens[b][lo:L].transpose(1, 0, 2)
        return sk, sv, tk, tv

    def bf16_pages(self):
        """BF16 paged cache holding every token (partial last page included):
        uint16 [num_pages, Hkv, 128, 128] for K and for V."""
        hkv = self.num_kv_heads
        kp = np.zeros((self.num_pages, hkv, PAGE, D), dtype=np.uint16)
        vp = np.zeros_like(kp)
        for b in range(self.batch):
            L = int(self.seq_lens[b])
            for i in range(-(-L // PAGE)):
                lo, hi = i * PAGE, min(L, (i + 1) * PAGE)
                p = int(self.block_tables[b, i])
                kp[p, :, : hi - lo] = self.k_tokens[b][lo:hi].transpose(1, 0, 2)
                vp[p, :, : hi - lo] = self.v_tokens[b][lo:hi].transpose(1, 0, 2)
        return kp, vp


def _outliers(rng, hkv: int, kind: str):
    """(channels [Hkv, n], offsets [Hkv, n]) for the key outlier recipe."""
    if kind == "tiny":
        n = 4
    elif kind == "qwen":
        n = 6
    elif kind == "write":
        n = 8
    elif kind == "none":
        return np.zeros((hkv, 0), dtype=np.int64), np.zeros((hkv, 0), dtype=np.float32)
    else:
        raise ValueError(kind)
    ch = np.stack([rng.choice(D, size=n, replace=False) for _ in range(hkv)])
    if kind == "tiny":
        off = np.full((hkv, n), 8.0)
    elif kind == "qwen":
        off = rng.standard_t(3, size=(hkv, n))
    else:
        off = 10.0 * rng.choice(np.array([-1.0, 1.0]), size=(hkv, n))
    return ch, off.astype(np.float32)


def _keys(rng, L: int, hkv: int, ch, off) -> np.ndarray:
    k = rng.standard_normal((L, hkv, D), dtype=np.float32)
    for h in range(hkv):
        k[:, h, ch[h]] += off[h]
    return f32_to_bf16(k)


def decode_workload(name: str, seed: int, seq_lens, num_q_heads: int, num_kv_heads: int,
                    outliers: str, shuffle: bool = True, extra_pages: int = 0,
                    sink_tokens: int = 16) -> DecodeWorkload:
    rng = np.random.Generator(np.random.PCG64(seed))
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    hkv = num_kv_heads
    ch, off = _outliers(rng, hkv, outliers)
    ks = [_keys(rng, int(L), hkv, ch, off) for L in seq_lens]
    vs = [f32_to_bf16(rng.standard_normal((int(L), hkv, D), dtype=np.float32)) for L in seq_lens]
    q = f32_to_bf16(rng.standard_normal((len(seq_lens), num_q_heads, D), dtype=np.float32))
    pages_per_seq = [-(-int(L) // PAGE) for L in seq_lens]
    num_pages = int(sum(pages_per_seq)) + extra_pages
    pool = rng.permutation(num_pages) if shuffle else np.arange(num_pages)
    maxp = max(1, max(pages_per_seq))
    bt = np.zeros((len(seq_lens), maxp), dtype=np.int32)
    pos = 0
    for b, n in enumerate(pages_per_seq):
        bt[b, :n] = pool[pos:pos + n]
        pos += n
    allk = np.concatenate([bf16_to_f32(k) for k in ks]).astype(np.float64)
    mu = allk.mean(axis=0).astype(np.float32) if allk.shape[0] else np.zeros((hkv, D), np.float32)
    return DecodeWorkload(name=name, seed=seed, num_q_heads=num_q_heads, num_kv_heads=hkv,
                          seq_lens=seq_lens, num_pages=num_pages, block_tables=bt,
                          k_tokens=ks, v_tokens=vs, q=q, key_shift=mu,
                          sink_tokens=sink_tokens,
                          meta={"outlier_channels": ch, "outlier_offsets": off})


def tiny(seed: int = 0) -> DecodeWorkload:
    """Batch 1, 1 KV head, 4 query heads, 2048 tokens (16 pages, identity
    table, no tail); +8 on 4 key channels."""
    return decode_workload("tiny_2k_1kv", seed, [2048], 4, 1, "tiny", shuffle=False)


def qwen_32k(seed: int = 0) -> DecodeWorkload:
    """Batch 1, 32 q / 8 KV heads, 256 full pages + a 77-token tail
    (L = 32,845), permuted 256-page pool; Student-t(3) key outliers."""
    return decode_workload("qwen3_4b_32k_tail77", seed, [256 * PAGE + 77], 32, 8, "qwen")


def qwen_128k_layer(layer: int) -> DecodeWorkload:
    """One layer of the 131,072-token decode (1024 pages, no tail); seed = layer."""
    return decode_workload("qwen3_4b_128k", layer, [131072], 32, 8, "qwen")


def batched_lengths(seed: int = 0, n_seqs: int = 16, lo: int = 2048, hi: int = 16384) -> np.ndarray:
    """The sequence lengths of ``batched``: L ~ U{lo..hi}, seeded."""
    rng = np.random.Generator(np.random.PCG64(seed + 1_000_003))
    return rng.integers(lo, hi + 1, size=n_seqs)


def batched(seed: int = 0, n_seqs: int = 16, lo: int = 2048, hi: int = 16384, num_kv_heads: int = 8) -> DecodeWorkload:
    """16 sequences with L ~ U{lo..hi}, shared shuffled pool, 4 query heads
    per KV head."""
    return decode_workload("batched_16x_2k_16k", seed, batched_lengths(seed, n_seqs, lo, hi), 4 * num_kv_heads,
                           num_kv_heads, "qwen")


@dataclass
class WriteWorkload:
    name: str
    seed: int
    k_rows: np.ndarray      # uint16 [n_pages*128, Hkv, 128]
    v_rows: np.ndarray
    page_ids: np.ndarray    # int32 [n_pages]
    num_pages: int
    key_shift: np.ndarray   # float32 [Hkv, 128]


def write_workload(seed: int = 0, tokens: int = 131072, num_kv_heads: int = 8,
                   shuffle: bool = True) -> WriteWorkload:
    """Prefill write of `tokens` tokens x 8 KV heads x 128; keys with +-10
    offsets (seeded signs) on 8 channels per head."""
    assert tokens % PAGE == 0
    rng = np.random.Generator(np.random.PCG64(seed))
    ch, off = _outliers(rng, num_kv_heads, "write")
    k = _keys(rng, tokens, num_kv_heads, ch, off)
    v = f32_to_bf16(rng.standard_normal((tokens, num_kv_heads, D), dtype=np.float32))
    n = tokens // PAGE
    ids = rng.permutation(n) if shuffle else np.arange(n)
    mu = bf16_to_f32(k).astype(np.float64).mean(axis=0).astype(np.float32)
    return WriteWorkload("prefill_write_128k_8kv", seed, k, v, ids.astype(np.int32), n, mu)


def torch_decode_layer(layer: int, seq_len: int = 131072, num_q_heads: int = 32, num_kv_heads: int = 8,
                       sink_tokens: int = 16, device="cuda", outliers: str = "qwen"):
    """One layer of the long-context decode drawn on the device with torch's
    generator (seed = layer): same recipe as ``decode_workload(..., "qwen")``
    (K, V, Q ~ N(0,1) in bf16; Student-t(3) offsets, formed as Z / sqrt(chi2_3 / 3),
    on 6 seeded key channels per KV head; mu = float32(mean of K in float64);
    one sequence; random permutation of a pool of ceil(L/128) pages). With
    outliers="write" the keys take the prefill write's outliers instead:
    +-10 (seeded signs) on 8 seeded channels per KV head.
    Returns a dict of device tensors."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(1_000_000 + layer)
    hkv = num_kv_heads
    if outliers == "write":
        ch = torch.stack([torch.randperm(D, generator=g, device=device)[:8] for _ in range(hkv)])
        off = 10.0 * torch.where(torch.rand((hkv, 8), generator=g, device=device) < 0.5, -1.0, 1.0)
    elif outliers == "qwen":
        ch = torch.stack([torch.randperm(D, generator=g, device=device)[:6] for _ in range(hkv)])
        z = torch.randn((hkv, 6), generator=g, device=device)
        chi = (torch.randn((hkv, 6, 3), generator=g, device=device) ** 2).sum(-1)
        off = z / torch.sqrt(chi / 3.0)
    else:
        raise ValueError(f"unknown key outlier recipe {outliers!r}")
    k = torch.randn((seq_len, hkv, D), generator=g, device=device)
    kf = k.view(seq_len, hkv, D)
    for h in range(hkv):
        kf[:, h, ch[h]] += off[h]
    k = kf.to(torch.bfloat16)
    v = torch.randn((seq_len, hkv, D), generator=g, device=device).to(torch.bfloat16)
    q = torch.randn((1, num_q_heads, D), generator=g, device=device).to(torch.bfloat16)
    n_pages = -(-seq_len // PAGE)
    perm = torch.randperm(n_pages, generator=g, device=device).to(torch.int32)
    mu = k.double().mean(dim=0).float().contiguous()
    n_full = seq_len // PAGE
    sink_k = k[:sink_tokens].permute(1, 0, 2).unsqueeze(0).contiguous()
    sink_v = v[:sink_tokens].permute(1, 0, 2).unsqueeze(0).contiguous()
    tail_k = torch.zeros((1, hkv, PAGE, D), dtype=torch.bfloat16, device=device)
    tail_v = torch.zeros_like(tail_k)
    lo = max(sink_tokens, n_full * PAGE)
    if seq_len > lo:
        tail_k[0, :, lo - n_full * PAGE:seq_len - n_full * PAGE] = k[lo:].permute(1, 0, 2)
        tail_v[0, :, lo - n_full * PAGE:seq_len - n_full * PAGE] = v[lo:].permute(1, 0, 2)
    return {
        "k": k, "v": v, "q": q, "key_shift": mu, "block_tables": perm.view(1, -1).contiguous(),
        "seq_lens": torch.tensor([seq_len], dtype=torch.int32, device=device),
        "num_pages": n_pages, "n_full": n_full, "page_ids": perm[:n_full].contiguous(),
        "sink_k": sink_k, "sink_v": sink_v, "tail_k": tail_k, "tail_v": tail_v,
        "seq_len": seq_len, "num_q_heads": num_q_heads, "num_kv_heads": hkv, "sink_tokens": sink_tokens,
        "sigma": float(np.float32(1.0 / np.sqrt(128.0))),
    }


def bf16_pages_from_tokens(k, block_tables, num_pages: int):
    """[L, Hkv, 128] bf16 tokens -> BF16 page pool [num_pages, Hkv, 128, 128]
    placed through the block table (zero-padded partial last page)."""
    import torch

    L, hkv, _ = k.shape
    n = -(-L // PAGE)
    pad = n * PAGE - L
    kk = torch.nn.functional.pad(k, (0, 0, 0, 0, 0, pad)) if pad else k
    pages = kk.view(n, PAGE, hkv, D).permute(0, 2, 1, 3)
    pool = torch.zeros((num_pages, hkv, PAGE, D), dtype=k.dtype, device=k.device)
    pool[block_tables[0, :n].long()] = pages
    return pool


def torch_write_rows(seed: int = 0, tokens: int = 131072, num_kv_heads: int = 8, device="cuda"):
    """The prefill-write workload drawn on the device (torch generator, seed):
    K, V ~ N(0,1) bf16 [tokens, Hkv, 128]; keys with +-10 offsets (seeded
    signs) on 8 seeded channels per head; mu = float32(mean of K); page_ids a
    random permutation of the tokens/128 pages."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(2_000_000 + seed)
    hkv = num_kv_heads
    ch = torch.stack([torch.randperm(D, generator=g, device=device)[:8] for _ in range(hkv)])
    sign = torch.where(torch.rand((hkv, 8), generator=g, device=device) < 0.5, -1.0, 1.0)
    k = torch.randn((tokens, hkv, D), generator=g, device=device)
    for h in range(hkv):
        k[:, h, ch[h]] += 10.0 * sign[h]
    k = k.to(torch.bfloat16)
    v = torch.randn((tokens, hkv, D), generator=g, device=device).to(torch.bfloat16)
    n = tokens // PAGE
    ids = torch.randperm(n, generator=g, device=device).to(torch.int32)
    mu = k.double().mean(dim=0).float().contiguous()
    return {"k": k, "v": v, "page_ids": ids, "key_shift": mu, "num_pages": n, "tokens": tokens, "num_kv_heads": hkv}
