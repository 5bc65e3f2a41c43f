"""NVFP4 / MXFP4 KV-cache page quantization and paged FP4 decode attention
for AMD MI355X (gfx950).

A thin ctypes binding over the C ABI of ``lib/libbdfp4.so`` (declared in
``include/bdfp4.h``). Each function has the name of its C entry point without
the ``bdfp4_`` prefix and only marshals arguments: tensors become device
pointers, the current torch stream becomes the launch stream, and a negative
status becomes a :class:`Bdfp4Error`. All computation happens in the HIP
kernels; if the library is not built, loading fails with an error (there is
no fallback).
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libbdfp4.so")

OK, E_INVALID, E_UNCALIBRATED, E_UNSUPPORTED, E_WORKSPACE, E_HIP = 0, -1, -2, -3, -4, -5
SCALE_NONE, SCALE_AMAX6, SCALE_FOUR_SIX, SCALE_MXFP4_SEARCH, SCALE_AMAX2_OR_AMAX6 = 0, 1, 2, 3, 4
KEY_GEOMETRY_LOCAL, KEY_GEOMETRY_CHANNEL = 0, 1


class Bdfp4Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_string(status)}: {message}")
        self.status = status


class Recipe(ctypes.Structure):
    _fields_ = [
        ("sink_tokens", ctypes.c_int32),
        ("rotation", ctypes.c_int32),
        ("key_smoothing", ctypes.c_int32),
        ("scale_mode_k", ctypes.c_int32),
        ("scale_mode_v", ctypes.c_int32),
        ("scale_mode_q", ctypes.c_int32),
        ("scale_mode_p", ctypes.c_int32),
        ("query_terms", ctypes.c_int32),
        ("c", ctypes.c_int32),
        ("tau", ctypes.c_float),
        ("rotate_v", ctypes.c_int32),
        ("p_running_max", ctypes.c_int32),
        ("key_scale_geometry", ctypes.c_int32),
    ]

    def replace(self, **kw) -> "Recipe":
        r = Recipe()
        ctypes.pointer(r)[0] = self
        for k, v in kw.items():
            setattr(r, k, v)
        return r

    @property
    def mx(self) -> bool:
        return self.scale_mode_k == SCALE_MXFP4_SEARCH


class Cache(ctypes.Structure):
    _fields_ = [
        ("k_codes", ctypes.c_void_p),
        ("k_scales", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p),
        ("v_scales", ctypes.c_void_p),
        ("num_pages", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
    ]


_lib_handle = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m fp4_kv_cache_nvfp4_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    RP = ctypes.POINTER(Recipe)
    CP = ctypes.POINTER(Cache)
    sig = {
        "bdfp4_recipe_default_nvfp4": [RP],
        "bdfp4_recipe_default_mxfp4": [RP],
        "bdfp4_recipe_validate": [RP],
        "bdfp4_cache_bytes": [RP, I32, I32, ctypes.POINTER(SZ), ctypes.POINTER(SZ), ctypes.POINTER(SZ), ctypes.POINTER(SZ)],
        "bdfp4_quantize_pages": [RP, CP, P, P, P, I32, P, P],
        "bdfp4_append_tokens": [RP, CP, P, P, I32, P, P, I32, P, P, P, P, P, P],
        "bdfp4_key_means_workspace_size": [I32, I32, ctypes.POINTER(SZ)],
        "bdfp4_key_means": [P, I32, I32, P, SZ, P, P],
        "bdfp4_error_sums": [P, P, ctypes.c_int64, P, P],
        "bdfp4_select_tau": [P, P, I32, ctypes.POINTER(F32), ctypes.POINTER(I32), P],
        "bdfp4_page_errors_workspace_size": [I32, I32, ctypes.POINTER(SZ)],
        "bdfp4_page_errors": [RP, CP, P, P, P, I32, P, P, SZ, P, P],
        "bdfp4_decode_plan": [I32, I32, I32, I32, ctypes.POINTER(I32), ctypes.POINTER(I32)],
        "bdfp4_bf16_decode_plan": [I32, I32, I32, I32, ctypes.POINTER(I32), ctypes.POINTER(I32)],
        "bdfp4_decode_workspace_size": [I32, I32, I32, I32, I32, ctypes.POINTER(SZ)],
        "bdfp4_decode_attention": [RP, CP, P, I32, I32, P, I32, P, I32, P, P, P, P, P, F32, I32, P, SZ, P, P],
        "bdfp4_decode_attention_noalloc": [RP, CP, P, I32, I32, P, I32, P, I32, P, P, P, P, P, F32, I32, P, P],
        "bdfp4_decode_attention_logits": [RP, CP, P, I32, I32, P, I32, P, I32, P, P, P, P, P, F32, I32, P, SZ, P, P,
                                          P],
        "bdfp4_bf16_decode_attention": [P, I32, I32, I32, P, P, I32, P, I32, P, I32, F32, I32, P, SZ, P, P],
        "bdfp4_quantize_rows": [P, I32, P, I32, I32, I32, P, P, P],
        "bdfp4_quantize_p_blocks": [P, I32, I32, F32, P, P, P],
        "bdfp4_decode_query_codes": [RP, P, I32, I32, I32, P, P, P],
        "bdfp4_stream_read": [P, SZ, P, SZ, I32, P],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int32
    L.bdfp4_decode_noalloc_max_workspace.argtypes = []
    L.bdfp4_decode_noalloc_max_workspace.restype = ctypes.c_size_t
    L.bdfp4_status_string.argtypes = [ctypes.c_int32]
    L.bdfp4_status_string.restype = ctypes.c_char_p
    L.bdfp4_last_error.argtypes = []
    L.bdfp4_last_error.restype = ctypes.c_char_p
    _lib_handle = L
    return L


def status_string(s: int) -> str:
    return lib().bdfp4_status_string(s).decode()


def _check(s: int) -> None:
    if s != OK:
        raise Bdfp4Error(s, lib().bdfp4_last_error().decode())


def _ptr(t) -> int | None:
    """Device (or host) address of a tensor, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        if not torch.cuda.is_available():
            return None
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


# ---------------------------------------------------------------- recipe

def recipe_default_nvfp4(tau: float = math.nan) -> Recipe:
    r = Recipe()
    _check(lib().bdfp4_recipe_default_nvfp4(ctypes.byref(r)))
    r.tau = tau
    return r


def recipe_default_mxfp4(tau: float = math.nan) -> Recipe:
    r = Recipe()
    _check(lib().bdfp4_recipe_default_mxfp4(ctypes.byref(r)))
    r.tau = tau
    return r


def recipe_validate(r: Recipe) -> None:
    _check(lib().bdfp4_recipe_validate(ctypes.byref(r)))


def cache_bytes(r: Recipe, num_pages: int, num_kv_heads: int):
    out = [ctypes.c_size_t() for _ in range(4)]
    _check(lib().bdfp4_cache_bytes(ctypes.byref(r), num_pages, num_kv_heads, *[ctypes.byref(o) for o in out]))
    return tuple(o.value for o in out)


@dataclass
class PagedCache:
    """The four cache arrays as uint8 device tensors [pages, heads, bytes]."""
    k_codes: object
    k_scales: object
    v_codes: object
    v_scales: object
    num_pages: int
    num_kv_heads: int

    @classmethod
    def allocate(cls, r: Recipe, num_pages: int, num_kv_heads: int, device="cuda"):
        import torch
        kc, ks, vc, vs = cache_bytes(r, num_pages, num_kv_heads)
        z = lambda n: torch.zeros((num_pages, num_kv_heads, n // max(1, num_pages * num_kv_heads)),
                                  dtype=torch.uint8, device=device)
        return cls(z(kc), z(ks), z(vc), z(vs), num_pages, num_kv_heads)

    def struct(self) -> Cache:
        return Cache(_ptr(self.k_codes), _ptr(self.k_scales), _ptr(self.v_codes), _ptr(self.v_scales),
                     self.num_pages, self.num_kv_heads, 128, 128)


# ---------------------------------------------------------------- writer

def quantize_pages(r: Recipe, cache: PagedCache, k, v, page_ids, key_shift=None, stream=None) -> None:
    n_pages = 0 if page_ids is None else int(page_ids.numel())
    c = cache.struct()
    _check(lib().bdfp4_quantize_pages(ctypes.byref(r), ctypes.byref(c), _ptr(k), _ptr(v), _ptr(page_ids),
                                      n_pages, _ptr(key_shift), _stream(stream)))


def append_tokens(r: Recipe, cache: PagedCache, k_new, v_new, positions, block_tables, sink_k, sink_v,
                  tail_k, tail_v, key_shift=None, stream=None) -> None:
    """One new token per sequence into its BF16 tail (and sink); a token that
    fills a page freezes that page into the cache. k_new/v_new [B, Hkv, 128]
    bf16, positions int32 [B] (device), block_tables int32 [B, max_pages]."""
    batch = int(positions.numel())
    c = cache.struct()
    _check(lib().bdfp4_append_tokens(ctypes.byref(r), ctypes.byref(c), _ptr(k_new), _ptr(v_new), batch,
                                     _ptr(positions), _ptr(block_tables), int(block_tables.shape[1]),
                                     _ptr(sink_k), _ptr(sink_v), _ptr(tail_k), _ptr(tail_v), _ptr(key_shift),
                                     _stream(stream)))


# ---------------------------------------------------------------- calibration

def key_means_workspace_size(tokens: int, num_kv_heads: int) -> int:
    need = ctypes.c_size_t()
    _check(lib().bdfp4_key_means_workspace_size(tokens, num_kv_heads, ctypes.byref(need)))
    return need.value


def key_means_into(k, num_kv_heads: int, workspace, mu, stream=None) -> None:
    """mu (float32 [Hkv, 128], device) = the key means of k [T, Hkv, 128] bf16,
    with a caller-given scratch of key_means_workspace_size bytes."""
    _check(lib().bdfp4_key_means(_ptr(k), int(k.shape[0]), num_kv_heads, _ptr(workspace),
                                 int(workspace.numel() * workspace.element_size()), _ptr(mu), _stream(stream)))


def key_means(k, num_kv_heads: int, stream=None):
    """float32 [Hkv, 128] device tensor of the key means of k [T, Hkv, 128]
    bf16 (the key-smoothing shift); the scratch is a torch allocation."""
    import torch
    tokens = int(k.shape[0])
    need = ctypes.c_size_t()
    _check(lib().bdfp4_key_means_workspace_size(tokens, num_kv_heads, ctypes.byref(need)))
    ws = torch.empty(max(need.value, 16), dtype=torch.uint8, device=k.device)
    mu = torch.empty((num_kv_heads, 128), dtype=torch.float32, device=k.device)
    _check(lib().bdfp4_key_means(_ptr(k), tokens, num_kv_heads, _ptr(ws), need.value, _ptr(mu), _stream(stream)))
    return mu


def error_sums(got, ref, out, stream=None) -> None:
    """out (float64 device, 2 values) = [sum (got - ref)^2, sum ref^2]."""
    _check(lib().bdfp4_error_sums(_ptr(got), _ptr(ref), int(ref.numel()), _ptr(out), _stream(stream)))


def calibrate_tau(r: Recipe, candidates, reference, decode_args: dict, stream=None):
    """The tau search: for each candidate, the FP4 decode (decode_attention
    with decode_args) and the error sums of its output against `reference`
    (exact attention of the same calibration batch, e.g. from
    bf16_decode_attention), all on the device; one copy of the sums to the
    host at the end, where bdfp4_select_tau picks the candidate. Returns
    (best tau, relative L2 error per candidate)."""
    import torch
    sums = torch.zeros((len(candidates), 2), dtype=torch.float64, device=reference.device)
    out = torch.empty_like(reference)
    for i, t in enumerate(candidates):
        decode_attention(r.replace(tau=float(t)), out=out, stream=stream, **decode_args)
        error_sums(out, reference, sums[i], stream)
    return select_tau(sums.cpu().numpy(), candidates)


def select_tau(sums, candidates):
    """bdfp4_select_tau on host error sums [n][2]: (chosen tau, relative L2
    error per candidate)."""
    import numpy as np
    s = np.ascontiguousarray(sums, dtype=np.float64).reshape(-1, 2)
    c = np.ascontiguousarray(candidates, dtype=np.float32).reshape(-1)
    errs = np.zeros(len(c), dtype=np.float64)
    best, idx = ctypes.c_float(), ctypes.c_int32()
    _check(lib().bdfp4_select_tau(s.ctypes.data, c.ctypes.data, len(c), ctypes.byref(best), ctypes.byref(idx),
                                  errs.ctypes.data))
    return float(best.value), [float(e) for e in errs]


def page_errors(r: Recipe, cache: PagedCache, k, v, page_ids, key_shift=None, stream=None):
    """Device float64 [4] = [sum (k_hat - y)^2, sum y^2, sum (v_hat - v)^2,
    sum v^2] of the pages quantize_pages wrote from these arguments."""
    import torch
    n_pages = int(page_ids.numel())
    need = ctypes.c_size_t()
    _check(lib().bdfp4_page_errors_workspace_size(n_pages, cache.num_kv_heads, ctypes.byref(need)))
    ws = torch.empty(need.value, dtype=torch.uint8, device=k.device)
    out = torch.empty(4, dtype=torch.float64, device=k.device)
    c = cache.struct()
    _check(lib().bdfp4_page_errors(ctypes.byref(r), ctypes.byref(c), _ptr(k), _ptr(v), _ptr(page_ids), n_pages,
                                   _ptr(key_shift), _ptr(ws), need.value, _ptr(out), _stream(stream)))
    return out


def save_key_means(path: str, means: dict) -> None:
    """Key-mean sidecar: {name: float32 [Hkv, 128] host array} to a
    safetensors file (host I/O only)."""
    import numpy as np
    from safetensors.numpy import save_file
    save_file({k: np.ascontiguousarray(v, dtype=np.float32) for k, v in means.items()}, path)


def load_key_means(path: str) -> dict:
    from safetensors.numpy import load_file
    return load_file(path)


# ---------------------------------------------------------------- decode

def decode_plan(batch: int, num_kv_heads: int, max_seq_len: int, pages_per_partition: int = 0):
    ppp, parts = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().bdfp4_decode_plan(batch, num_kv_heads, max_seq_len, pages_per_partition,
                                   ctypes.byref(ppp), ctypes.byref(parts)))
    return ppp.value, parts.value


def bf16_decode_plan(batch: int, num_kv_heads: int, max_seq_len: int, pages_per_partition: int = 0):
    ppp, parts = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().bdfp4_bf16_decode_plan(batch, num_kv_heads, max_seq_len, pages_per_partition,
                                        ctypes.byref(ppp), ctypes.byref(parts)))
    return ppp.value, parts.value


def decode_workspace_size(batch: int, num_q_heads: int, num_kv_heads: int, max_seq_len: int,
                          pages_per_partition: int = 0) -> int:
    n = ctypes.c_size_t()
    _check(lib().bdfp4_decode_workspace_size(batch, num_q_heads, num_kv_heads, max_seq_len,
                                             pages_per_partition, ctypes.byref(n)))
    return n.value


def alloc_workspace(nbytes: int, device="cuda"):
    """Zero-filled workspace (the ticket words must start at zero)."""
    import torch
    return torch.zeros(((nbytes + 15) // 16) * 16, dtype=torch.uint8, device=device)


def decode_attention(r: Recipe, cache: PagedCache, q, block_tables, seq_lens, max_seq_len: int,
                     sink_k, sink_v, tail_k, tail_v, key_shift, softmax_scale: float,
                     pages_per_partition: int, workspace, out, stream=None) -> None:
    B, Hq = int(q.shape[0]), int(q.shape[1])
    c = cache.struct()
    _check(lib().bdfp4_decode_attention(
        ctypes.byref(r), ctypes.byref(c), _ptr(q), B, Hq, _ptr(block_tables), int(block_tables.shape[1]),
        _ptr(seq_lens), int(max_seq_len), _ptr(sink_k), _ptr(sink_v), _ptr(tail_k), _ptr(tail_v),
        _ptr(key_shift), float(softmax_scale), int(pages_per_partition), _ptr(workspace),
        int(workspace.numel() * workspace.element_size()), _ptr(out), _stream(stream)))


def decode_attention_noalloc(r: Recipe, cache: PagedCache, q, block_tables, seq_lens, max_seq_len: int,
                             sink_k, sink_v, tail_k, tail_v, key_shift, softmax_scale: float,
                             pages_per_partition: int, out, stream=None) -> None:
    """decode_attention on the library's own per-GPU workspace array
    (bdfp4_decode_attention_noalloc): no workspace argument, no allocation."""
    B, Hq = int(q.shape[0]), int(q.shape[1])
    c = cache.struct()
    _check(lib().bdfp4_decode_attention_noalloc(
        ctypes.byref(r), ctypes.byref(c), _ptr(q), B, Hq, _ptr(block_tables), int(block_tables.shape[1]),
        _ptr(seq_lens), int(max_seq_len), _ptr(sink_k), _ptr(sink_v), _ptr(tail_k), _ptr(tail_v),
        _ptr(key_shift), float(softmax_scale), int(pages_per_partition), _ptr(out), _stream(stream)))


def decode_attention_logits(r: Recipe, cache: PagedCache, q, block_tables, seq_lens, max_seq_len: int,
                            sink_k, sink_v, tail_k, tail_v, key_shift, softmax_scale: float,
                            pages_per_partition: int, workspace, out, logits, stream=None) -> None:
    """bdfp4_decode_attention_logits (debug): the decode, plus its raw FP4-token
    logits in `logits` (float32 [B, Hkv, 4, 128 * max_pages_per_seq])."""
    B, Hq = int(q.shape[0]), int(q.shape[1])
    c = cache.struct()
    _check(lib().bdfp4_decode_attention_logits(
        ctypes.byref(r), ctypes.byref(c), _ptr(q), B, Hq, _ptr(block_tables), int(block_tables.shape[1]),
        _ptr(seq_lens), int(max_seq_len), _ptr(sink_k), _ptr(sink_v), _ptr(tail_k), _ptr(tail_v),
        _ptr(key_shift), float(softmax_scale), int(pages_per_partition), _ptr(workspace),
        int(workspace.numel() * workspace.element_size()), _ptr(out), _ptr(logits), _stream(stream)))


def decode_noalloc_max_workspace() -> int:
    return int(lib().bdfp4_decode_noalloc_max_workspace())


def bf16_decode_attention(q, k_pages, v_pages, block_tables, seq_lens, max_seq_len: int,
                          softmax_scale: float, pages_per_partition: int, workspace, out, stream=None) -> None:
    B, Hq = int(q.shape[0]), int(q.shape[1])
    _check(lib().bdfp4_bf16_decode_attention(
        _ptr(q), B, Hq, int(k_pages.shape[1]), _ptr(k_pages), _ptr(v_pages), int(k_pages.shape[0]),
        _ptr(block_tables), int(block_tables.shape[1]), _ptr(seq_lens), int(max_seq_len),
        float(softmax_scale), int(pages_per_partition), _ptr(workspace),
        int(workspace.numel() * workspace.element_size()), _ptr(out), _stream(stream)))


# ---------------------------------------------------------------- codec debug entries

def quantize_rows(rows, shift, rotation: int, mode: int, terms: int, codes, scales, stream=None) -> None:
    _check(lib().bdfp4_quantize_rows(_ptr(rows), int(rows.shape[0]) if rows is not None else 0, _ptr(shift),
                                     rotation, mode, terms, _ptr(codes), _ptr(scales), _stream(stream)))


def decode_query_codes(r: Recipe, q, num_kv_heads: int, codes, scales, stream=None) -> None:
    """bdfp4_decode_query_codes: the decode prologue's query codes and scales."""
    _check(lib().bdfp4_decode_query_codes(ctypes.byref(r), _ptr(q), int(q.shape[0]), int(q.shape[1]),
                                          int(num_kv_heads), _ptr(codes), _ptr(scales), _stream(stream)))


def quantize_p_blocks(pp, mode: int, tau: float, codes, scales, stream=None) -> None:
    _check(lib().bdfp4_quantize_p_blocks(_ptr(pp), int(pp.shape[0]) if pp is not None else 0, mode, float(tau),
                                         _ptr(codes), _ptr(scales), _stream(stream)))


def stream_read(src, sink, workgroups: int, nbytes: int | None = None, stream=None) -> None:
    """bdfp4_stream_read: a plain streaming read of `src` (the practical HBM
    read ceiling for a byte count); `sink` takes one uint32 per thread."""
    n = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    _check(lib().bdfp4_stream_read(_ptr(src), n, _ptr(sink), sink.numel() * sink.element_size(), int(workgroups),
                                   _stream(stream)))


class DecodeCall:
    """bdfp4_decode_attention with its arguments marshalled once; calling it
    launches on the given (or current) stream. For tight loops and graph
    capture, where per-call Python work would otherwise dominate."""

    def __init__(self, r: Recipe, cache: PagedCache, q, block_tables, seq_lens, max_seq_len: int,
                 sink_k, sink_v, tail_k, tail_v, key_shift, softmax_scale: float,
                 pages_per_partition: int, workspace, out):
        self._keep = (q, block_tables, seq_lens, sink_k, sink_v, tail_k, tail_v, key_shift, workspace, out, cache)
        self._r = r.replace()
        self._c = cache.struct()
        self._fn = lib().bdfp4_decode_attention
        self._args = [ctypes.byref(self._r), ctypes.byref(self._c), _ptr(q), int(q.shape[0]), int(q.shape[1]),
                      _ptr(block_tables), int(block_tables.shape[1]), _ptr(seq_lens), int(max_seq_len),
                      _ptr(sink_k), _ptr(sink_v), _ptr(tail_k), _ptr(tail_v), _ptr(key_shift),
                      float(softmax_scale), int(pages_per_partition), _ptr(workspace),
                      int(workspace.numel() * workspace.element_size()), _ptr(out)]

    def __call__(self, stream=None) -> None:
        _check(self._fn(*self._args, _stream(stream)))


class Bf16DecodeCall:
    """bdfp4_bf16_decode_attention with pre-marshalled arguments."""

    def __init__(self, q, k_pages, v_pages, block_tables, seq_lens, max_seq_len: int, softmax_scale: float,
                 pages_per_partition: int, workspace, out):
        self._keep = (q, k_pages, v_pages, block_tables, seq_lens, workspace, out)
        self._fn = lib().bdfp4_bf16_decode_attention
        self._args = [_ptr(q), int(q.shape[0]), int(q.shape[1]), int(k_pages.shape[1]), _ptr(k_pages),
                      _ptr(v_pages), int(k_pages.shape[0]), _ptr(block_tables), int(block_tables.shape[1]),
                      _ptr(seq_lens), int(max_seq_len), float(softmax_scale), int(pages_per_partition),
                      _ptr(workspace), int(workspace.numel() * workspace.element_size()), _ptr(out)]

    def __call__(self, stream=None) -> None:
        _check(self._fn(*self._args, _stream(stream)))
