"""The oracle's thread-pool form (used by bench.py's multi-core CPU baseline)
makes the same row calls as the serial step, so its results are identical
bit for bit, rejected rows and rows that append nothing included."""
import numpy as np
import pytest

import oracle
from autoregressive_kv_cache_amd.workloads import WORKLOADS, host_arrays, make_inputs


@pytest.mark.parametrize("name", ["tiny_mixed_f32", "mha_stress_f32", "chunk_gqa_bf16"])
@pytest.mark.parametrize("threads", [1, 3, 8])
def test_threaded_step_is_the_serial_step(name, threads):
    wl = WORKLOADS[name]
    inp = make_inputs(wl, 2, "cpu")
    inp["lengths"][0] = wl.M + 1  # a rejected row
    h = host_arrays(inp)
    args = (h["query"], h["new_key"], h["new_value"], h["key_cache"], h["value_cache"],
            h["lengths"], h["append_mask"])
    orc = oracle.default()
    a = orc.step(*args, scale=wl.scale)
    b = orc.step_threaded(*args, scale=wl.scale, threads=threads)
    for field in ("key_cache", "value_cache", "lengths", "attention", "context", "row_status"):
        assert np.array_equal(getattr(a, field), getattr(b, field)), field
