"""Recipe ablations on synthetic data: key/value reconstruction error and
attention output error, measured on the device through the library.

"BitDecoding-FP4 evaluation/config.py" lists the recipe's parts (Hadamard
rotation, key smoothing, K four_six, two query terms, P amax2_or_amax6 with
c and tau) and "kv-landlords scripts/quant_ab.py" compares cache schemes by
reconstruction error; this driver measures each part's effect by switching
it off alone, plus a plain NVFP4 cache (amax6 everywhere, no rotation or
centering, one query term, tau = 0), the rotated-values variant, the channel
key scale geometry and the MXFP4 recipe. For every recipe:

* bdfp4_quantize_pages writes the layer's full pages;
* bdfp4_page_errors gives the relative K error (centered, rotated domain)
  and V error;
* bdfp4_decode_attention against bdfp4_bf16_decode_attention (exact
  attention over the same BF16 tokens) through bdfp4_error_sums gives the
  relative L2 output error.

Inputs are the seeded synthetic decode layer (one sequence, Qwen3-4B shapes),
with the decode workload's mild key outliers or, with --keys write, the
prefill write's large ones (+-10 on 8 channels per KV head), which the
rotation and the centering exist for.
`python -m fp4_kv_cache_nvfp4_amd.diagnostics [--context L]` prints JSON.
"""
from __future__ import annotations

import argparse
import json
import math

from . import (KEY_GEOMETRY_CHANNEL, SCALE_AMAX6, alloc_workspace, bf16_decode_attention, decode_attention,
               decode_workspace_size, error_sums, page_errors, quantize_pages, recipe_default_mxfp4,
               recipe_default_nvfp4, PagedCache)
from . import synth

ABLATIONS = {
    "bitdecoding-nvfp4": {},
    "k_amax6": {"scale_mode_k": SCALE_AMAX6},
    "no_rotation": {"rotation": 0},
    "no_centering": {"key_smoothing": 0},
    "query_terms_1": {"query_terms": 1},
    "c_1": {"c": 1},
    "p_amax6_tau_0": {"tau": 0.0},
    "rotate_v": {"rotate_v": 1},
    "key_channel_geometry": {"key_scale_geometry": KEY_GEOMETRY_CHANNEL},
    "plain_nvfp4": {"scale_mode_k": SCALE_AMAX6, "rotation": 0, "key_smoothing": 0, "query_terms": 1,
                    "tau": 0.0},
    "bitdecoding-mxfp4": None,
}


def recipes(tau: float = 1.0) -> dict:
    out = {}
    for name, change in ABLATIONS.items():
        out[name] = recipe_default_mxfp4(tau) if change is None else recipe_default_nvfp4(tau).replace(**change)
    return out


def ablation_report(context: int = 32768, layer: int = 0, tau: float = 1.0, pages_per_partition: int = 0,
                    keys: str = "qwen") -> dict:
    """keys: "qwen" (the decode layer's Student-t(3) offsets on 6 channels
    per KV head) or "write" (the prefill write's +-10 offsets on 8)."""
    import torch

    d = synth.torch_decode_layer(layer, seq_len=context, outliers=keys)
    hq, hkv, L = d["num_q_heads"], d["num_kv_heads"], d["seq_len"]
    kp = synth.bf16_pages_from_tokens(d["k"], d["block_tables"], d["num_pages"])
    vp = synth.bf16_pages_from_tokens(d["v"], d["block_tables"], d["num_pages"])
    from . import decode_plan
    ppp, _ = decode_plan(1, hkv, L, pages_per_partition)
    ws = alloc_workspace(decode_workspace_size(1, hq, hkv, L, ppp))
    ref = torch.empty((1, hq, 128), dtype=torch.float32, device="cuda")
    bf16_decode_attention(d["q"], kp, vp, d["block_tables"], d["seq_lens"], L, d["sigma"], ppp, ws, ref)
    out = torch.empty_like(ref)
    sums = torch.zeros(2, dtype=torch.float64, device="cuda")
    report = {}
    for name, r in recipes(tau).items():
        mu = d["key_shift"] if r.key_smoothing else None
        cache = PagedCache.allocate(r, d["num_pages"], hkv)
        quantize_pages(r, cache, d["k"][:d["n_full"] * 128], d["v"][:d["n_full"] * 128], d["page_ids"], mu)
        pe = page_errors(r, cache, d["k"][:d["n_full"] * 128].contiguous(), d["v"][:d["n_full"] * 128].contiguous(),
                         d["page_ids"], mu).cpu().tolist()
        decode_attention(r, cache, d["q"], d["block_tables"], d["seq_lens"], L, d["sink_k"], d["sink_v"],
                         d["tail_k"], d["tail_v"], mu, d["sigma"], ppp, ws, out)
        error_sums(out, ref, sums)
        e, rr = sums.cpu().tolist()
        report[name] = {"k_rel": math.sqrt(pe[0] / pe[1]), "v_rel": math.sqrt(pe[2] / pe[3]),
                        "out_rel_l2": math.sqrt(e / rr)}
        del cache
    return {"context": L, "layer": layer, "tau": tau, "keys": keys, "pages_per_partition": ppp, "recipes": report}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--context", type=int, default=32768)
    ap.add_argument("--layer", type=int, default=0)
    ap.add_argument("--tau", type=float, default=1.0)
    ap.add_argument("--keys", choices=["qwen", "write"], default="qwen",
                    help="key outliers: the decode layer's Student-t(3) offsets or the prefill write's +-10")
    a = ap.parse_args()
    print(json.dumps(ablation_report(a.context, a.layer, a.tau, keys=a.keys)))


if __name__ == "__main__":
    main()
