"""The pooled oracle writer (tests/oracle_pool.py) equals the plain oracle
writer page for page (CPU only): it only splits the pages into chunks."""
import numpy as np
import pytest

from fp4_kv_cache_nvfp4_amd import synth
from oracle import recipe as RC
from oracle import writer as W

import oracle_pool as OP


@pytest.mark.parametrize("r", [RC.nvfp4_default().with_(tau=1.0), RC.mxfp4_default().with_(tau=1.0),
                               RC.nvfp4_default().with_(tau=1.0, key_scale_geometry=RC.CHANNEL)],
                         ids=["nvfp4", "mxfp4", "nvfp4_chan"])
def test_pooled_writer_equals_writer(r):
    wl = synth.write_workload(seed=3, tokens=128 * 12)
    a = W.empty_cache(wl.num_pages + 2, 8, r)
    W.write_pages(r, a, wl.k_rows, wl.v_rows, wl.page_ids + 2, wl.key_shift)
    b = W.empty_cache(wl.num_pages + 2, 8, r)
    OP.write_pages(r, b, wl.k_rows, wl.v_rows, wl.page_ids + 2, wl.key_shift, workers=3)
    for name in a:
        assert np.array_equal(a[name], b[name]), name
