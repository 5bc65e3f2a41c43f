"""Paged FP4 decode attention in float64 over the quantized operands.

Oracle module (test infrastructure only; see the package docstring).

Sources. "BitDecoding-FP4 evaluation/config.py": the ``bitdecoding-nvfp4``
KV_MODES entry (16-token BF16 sink, two-term query, rotation, key shift),
PARITY_ENGINE_KWARGS (block_size 128), RECIPE and ``probability_environment``
(P scale mode amax2_or_amax6 with c and tau). "How openbitsys/bitdecoding-fp4
works": the decode interface dispatches to the paged attention kernel, which
uses block scaling and scale modes; the tail control plane keeps the hybrid
(BF16 tail) cache. "kv-landlords scripts/quant_ab.py" PageSim: completed pages
are quantized, the partial page stays BF16.

The pages give no formulas for the decode. Readings taken here, in order:

1. Token sets. With L = seq_len and n = floor(L / 128) full pages: BF16
   tokens are the sink [0, min(S, L)) (S = sink_tokens, from the sink buffer)
   and the tail [max(S, 128 n), L) (from the BF16 tail page, slot t - 128 n).
   FP4 tokens are [S, 128 n), read through the block table.
2. Query. q = float32(q_bf16); q_r = rotate(q) (if rotation); two-term
   residual quantization of q_r (quant.quantize_query) gives q_hat.
3. Logits. FP4 token j: t_j = sigma * (q_hat . k_hat_j + q . mu), where
   k_hat_j is the dequantized centered, rotated key and q . mu (unrotated q,
   key mean mu) restores the logit of the uncentered key. BF16 token j:
   t_j = sigma * (q . k_j).
4. Partitions. Partition 0 holds all BF16 tokens. Partitions 1..S each hold a
   contiguous range of pages_per_partition FP4 pages (the first one starts
   after the sink).
5. Per partition s: m_s = max_j t_j, p_j = exp(t_j - m_s), l_s = sum_j p_j
   (unquantized). FP4 partitions quantize p'_j per 16-token block aligned to
   the logical token index with the P scale mode and use P_hat = s * e2m1 / c;
   the BF16 partition uses P_hat = p. o_s = sum_j P_hat_j * v_hat_j.
   The pages fix no precision for p', and p' decides integers (the P codes
   and block scales), so it is formed in float32, the precision in which the
   decode forms it: with r_j = float32(q_hat . k_hat_j + q . mu) and
   r_m = max_j r_j, p'_j = c * 2^a_j, a_j = fl32(fl32(r_j - r_m) * k) and
   k = fl32(fl32(sigma) * fl32(log2 e)), 2^a_j taken in float64 and rounded
   once to float32 (c is a power of two). Everything else about the
   partition (m_s, l_s, P_hat's values, o_s) is float64.
6. Merge: M = max_s m_s, L = sum_s l_s exp(m_s - M),
   out = sum_s o_s exp(m_s - M) / L (float output).

Everything after the quantized operands is float64.
"""
from __future__ import annotations

import math

import numpy as np

from . import quant as Q
from .formats import bf16_to_f32
from .recipe import Recipe
from .rotation import hadamard_matrix, rotate
from .writer import read_page_head

PAGE = 128
D = 128


def split_plan(seq_len: int, sink: int, pages_per_partition: int):
    """(n_full, bf16 token list, [(lo, hi) FP4 token range per partition 1..S])."""
    n_full = seq_len // PAGE
    bf16 = list(range(min(sink, seq_len))) + list(range(max(sink, PAGE * n_full), seq_len))
    parts = []
    if n_full >= 1:
        nparts = -(-n_full // pages_per_partition)
        for s in range(nparts):
            p0 = s * pages_per_partition
            p1 = min(n_full, (s + 1) * pages_per_partition)
            parts.append((max(sink, PAGE * p0), PAGE * p1))
    return n_full, bf16, parts


def query_hat(recipe: Recipe, q_f32: np.ndarray) -> np.ndarray:
    q_r = rotate(q_f32) if recipe.rotation else np.asarray(q_f32, dtype=np.float32)
    _, qhat = Q.quantize_query(q_r, recipe.scale_mode_q, recipe.query_terms)
    return qhat


def p_prime(recipe: Recipe, sigma: float, raw: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """p' = c * 2^(fl32(fl32(r - ref) * fl32(fl32(sigma) * fl32(log2 e)))) in
    float32 (reading 5): raw [G, n] logits without sigma (float64, rounded
    to float32 here), ref [G] or [G, n] the float32 reference maximum."""
    r32 = np.asarray(raw).astype(np.float32)
    k = np.float32(np.float32(sigma) * np.float32(math.log2(math.e)))
    ref32 = np.asarray(ref, dtype=np.float32)
    if ref32.ndim == 1:
        ref32 = ref32[:, None]
    a = ((r32 - ref32).astype(np.float32) * k).astype(np.float32)
    return (float(recipe.c) * np.exp2(a.astype(np.float64))).astype(np.float32)


def _p_hat(recipe: Recipe, pp: np.ndarray) -> np.ndarray:
    """Quantized probabilities of one FP4 partition from p' [G, n] float32
    (n a multiple of 16, blocks aligned to logical token index)."""
    nib, sc = Q.quantize_p(pp, recipe.scale_mode_p, np.float32(recipe.tau))
    return Q.dequantize(nib, sc, Q.AMAX6) / float(recipe.c)


def merge(parts):
    """Log-sum-exp merge of (o [G,D], m [G], l [G]) partials."""
    ms = np.stack([m for (_, m, _) in parts])          # [S, G]
    M = np.max(ms, axis=0)
    w = np.where(np.isneginf(ms), 0.0, np.exp(ms - np.where(np.isneginf(M), 0.0, M)))
    L = sum(w[i] * parts[i][2] for i in range(len(parts)))
    O = sum(w[i][:, None] * parts[i][0] for i in range(len(parts)))
    return O / L[:, None]


def attend_head(recipe: Recipe, q_f32: np.ndarray, seq_len: int,
                k_hat: np.ndarray, v_hat: np.ndarray,
                sink_k: np.ndarray, sink_v: np.ndarray,
                tail_k: np.ndarray, tail_v: np.ndarray,
                mu, sigma: float, pages_per_partition: int) -> np.ndarray:
    """Decode for one KV head and its G query heads.

    q_f32 [G, 128]; k_hat, v_hat [n_full*128, 128] float64 dequantized FP4
    tokens by logical index (rows before the sink are ignored); sink_k/v
    [S, 128] and tail_k/v [128, 128] float32 BF16 values; mu [128] or None."""
    G = q_f32.shape[0]
    if seq_len < 1:
        return np.full((G, D), np.nan)
    sigma = float(sigma)
    n_full, bf16_tok, parts = split_plan(seq_len, recipe.sink_tokens, pages_per_partition)
    q64 = q_f32.astype(np.float64)
    partials = []

    # partition 0: BF16 sink and tail, exact
    if bf16_tok:
        kb = np.stack([sink_k[t] if t < recipe.sink_tokens else tail_k[t - PAGE * n_full]
                       for t in bf16_tok]).astype(np.float64)
        vb = np.stack([sink_v[t] if t < recipe.sink_tokens else tail_v[t - PAGE * n_full]
                       for t in bf16_tok]).astype(np.float64)
        t = sigma * (q64 @ kb.T)
        m = t.max(axis=1)
        p = np.exp(t - m[:, None])
        partials.append((p @ vb, m, p.sum(axis=1)))

    if parts:
        qhat = query_hat(recipe, q_f32)
        qmu = q64 @ np.asarray(mu, dtype=np.float64) if recipe.key_smoothing else np.zeros(G)
        for lo, hi in parts:
            raw = qhat @ k_hat[lo:hi].T + qmu[:, None]
            t = sigma * raw
            m = t.max(axis=1)
            p = np.exp(t - m[:, None])
            r32 = raw.astype(np.float32)
            if recipe.scale_mode_p == Q.NONE:
                ph = p
            elif recipe.p_running_max:
                # recipe variant: each aligned 16-token block is normalised by
                # the running maximum over the partition's blocks up to it (as
                # a one-pass kernel would see it), quantized against that, and
                # weighted back to the partition maximum
                run = lambda x: np.repeat(np.maximum.accumulate(x.reshape(G, -1, 16).max(axis=2), axis=1), 16, axis=1)
                mrun = run(t)
                ph = _p_hat(recipe, p_prime(recipe, sigma, raw, run(r32))) * np.exp(mrun - m[:, None])
            else:
                ph = _p_hat(recipe, p_prime(recipe, sigma, raw, r32.max(axis=1)))
            o = ph @ v_hat[lo:hi]
            if recipe.rotate_v:
                # v_hat are rotated values: rotate this partition's output
                # back (H / sqrt(128) is symmetric and its own inverse)
                o = o @ (hadamard_matrix().astype(np.float64) / np.sqrt(128.0))
            partials.append((o, m, p.sum(axis=1)))
    return merge(partials)


def decode(recipe: Recipe, cache: dict, q_bf16: np.ndarray, block_tables: np.ndarray,
           seq_lens, sink_k, sink_v, tail_k, tail_v, key_shift, sigma: float,
           pages_per_partition: int, fp4_rows=None) -> np.ndarray:
    """Batched decode. q_bf16 [B, Hq, 128] uint16; block_tables [B, maxp] int;
    seq_lens [B]; sink_k/v [B, Hkv, S, 128] uint16; tail_k/v [B, Hkv, 128, 128]
    uint16; key_shift [Hkv, 128] float32 or None. Returns float64 [B, Hq, 128].

    fp4_rows, if given, is a callable (b, h, n_full) -> (k_hat, v_hat) used
    instead of reading the packed cache (quantization-off checks)."""
    q = bf16_to_f32(q_bf16)
    B, Hq, _ = q.shape
    Hkv = tail_k.shape[1]
    G = Hq // Hkv
    sk, sv = bf16_to_f32(sink_k), bf16_to_f32(sink_v)
    tk, tv = bf16_to_f32(tail_k), bf16_to_f32(tail_v)
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(seq_lens[b])
        n_full = max(L, 0) // PAGE
        for h in range(Hkv):
            if fp4_rows is not None:
                kh, vh = fp4_rows(b, h, n_full)
            else:
                kh = np.zeros((n_full * PAGE, D))
                vh = np.zeros((n_full * PAGE, D))
                for i in range(n_full):
                    kp, vp = read_page_head(recipe, cache, int(block_tables[b][i]), h)
                    kh[i * PAGE:(i + 1) * PAGE] = kp
                    vh[i * PAGE:(i + 1) * PAGE] = vp
            mu = None if key_shift is None else np.asarray(key_shift)[h]
            out[b, h * G:(h + 1) * G] = attend_head(
                recipe, q[b, h * G:(h + 1) * G], L, kh, vh, sk[b, h], sv[b, h],
                tk[b, h], tv[b, h], mu, sigma, pages_per_partition)
    return out


def textbook_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, sigma: float) -> np.ndarray:
    """softmax(sigma q K^T) V in float64; q [G, D], k/v [n, D]."""
    t = float(sigma) * (q.astype(np.float64) @ k.astype(np.float64).T)
    t = t - t.max(axis=1, keepdims=True)
    p = np.exp(t)
    return (p / p.sum(axis=1, keepdims=True)) @ v.astype(np.float64)


def bf16_decode(q_bf16: np.ndarray, k_pages: np.ndarray, v_pages: np.ndarray,
                block_tables: np.ndarray, seq_lens, sigma: float) -> np.ndarray:
    """BF16-KV paged decode (the unquantized baseline arm): exact attention
    over all L tokens of BF16 pages [P, Hkv, 128, 128] (uint16)."""
    q = bf16_to_f32(q_bf16)
    B, Hq, _ = q.shape
    Hkv = k_pages.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(seq_lens[b])
        if L < 1:
            out[b] = np.nan
            continue
        npg = -(-L // PAGE)
        pages = [int(block_tables[b][i]) for i in range(npg)]
        for h in range(Hkv):
            k = np.concatenate([bf16_to_f32(k_pages[p, h]) for p in pages])[:L]
            v = np.concatenate([bf16_to_f32(v_pages[p, h]) for p in pages])[:L]
            out[b, h * G:(h + 1) * G] = textbook_attention(q[b, h * G:(h + 1) * G], k, v, sigma)
    return out
