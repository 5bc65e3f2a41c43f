"""The oracle's page writer over many pages in worker processes (test
infrastructure only). Pages are independent, so the writer's output for a
set of pages is the concatenation of its outputs for disjoint chunks of them;
each worker runs oracle.writer.write_pages on one chunk exactly as a single
call would. Workers are started with the spawn method: fresh interpreters
that import numpy and the oracle only, never the GPU runtime."""
import multiprocessing
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

from oracle import writer as W

MAX_WORKERS = 16


def _write_chunk(args):
    recipe, k_bf16, v_bf16, key_shift, n = args
    cache = W.empty_cache(n, k_bf16.shape[1], recipe)
    W.write_pages(recipe, cache, k_bf16, v_bf16, np.arange(n), key_shift)
    return cache


def write_pages(recipe, cache: dict, k_bf16: np.ndarray, v_bf16: np.ndarray, page_ids, key_shift=None,
                workers: int = 0) -> dict:
    """Same contract as oracle.writer.write_pages (cache updated in place and
    returned): k_bf16, v_bf16 [n*128, Hkv, 128] uint16, page i holding rows
    [128 i, 128 i + 128), written to physical page page_ids[i]."""
    page_ids = np.asarray(page_ids, dtype=np.int64)
    n = page_ids.shape[0]
    workers = workers or min(MAX_WORKERS, os.cpu_count() or 1)
    bounds = np.linspace(0, n, min(workers * 2, n) + 1).astype(int)
    jobs = [(recipe, k_bf16[128 * a:128 * b], v_bf16[128 * a:128 * b], key_shift, b - a)
            for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
    ctx = multiprocessing.get_context("spawn")
    with ProcessPoolExecutor(max_workers=workers, mp_context=ctx) as ex:
        parts = list(ex.map(_write_chunk, jobs))
    a = 0
    for part, (_, _, _, _, m) in zip(parts, jobs):
        for name, arr in part.items():
            cache[name][page_ids[a:a + m]] = arr
        a += m
    return cache
