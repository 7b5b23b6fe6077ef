"""bench.py's byte accounting against the closed forms of the step.

In place the step must read the len cached rows and the n new rows, write the
n new rows, read q, write the full attention rows and the context; out of
place it must read every old slot and the new rows and write every slot of
the returned cache.  The attention kernel's share is what it visits."""
import numpy as np

import bench
from autoregressive_kv_cache_amd.workloads import WORKLOADS, draw_lengths_and_counts


def _closed_forms(wl, lengths, n):
    e = 2 if wl.dtype == "bf16" else 4
    row = (wl.D + wl.Dv) * e
    per_query = wl.B * wl.Hq * wl.Q * (wl.D + wl.M + wl.Dv) * e
    small = wl.B * (8 + 8 + 4 + wl.Q)
    inplace = sum(wl.Hk * (L + 2 * k) * row for L, k in zip(lengths, n)) + per_query + small
    oop = 2 * wl.B * wl.Hk * wl.M * row + sum(wl.Hk * k * row for k in n) + per_query + small
    return inplace, oop


def test_step_bytes_match_closed_forms():
    for name in ("tiny_mixed_f32", "decode_gqa_bf16", "mha_stress_f32"):
        wl = WORKLOADS[name]
        lengths, n = draw_lengths_and_counts(wl, 3)
        lengths = [int(x) for x in lengths]
        n = [int(x) for x in n]
        step, attend, _ = bench.algorithmic_bytes(wl, lengths, n)
        extra_step, extra_attend = bench.oop_extra_bytes(wl, lengths, n)
        inplace, oop = _closed_forms(wl, lengths, n)
        assert step == inplace
        assert step + extra_step == oop
        e = 2 if wl.dtype == "bf16" else 4
        visible = sum(wl.Hq * (L + t + 1) for L, k in zip(lengths, n) for t in range(k)) * e
        kv_read = sum(wl.Hk * (L + k) * (wl.D + wl.Dv) * e for L, k in zip(lengths, n))
        assert attend == kv_read + wl.B * wl.Hq * wl.Q * wl.D * e + visible + wl.B * (8 + wl.Q)
        assert extra_attend == sum(wl.Hk * L * (wl.D + wl.Dv) * e for L in lengths)


def test_decode_bytes_are_kv_dominated():
    wl = WORKLOADS["decode_gqa_bf16"]
    lengths, n = draw_lengths_and_counts(wl, 0)
    step, attend, kv = bench.algorithmic_bytes(wl, [int(x) for x in lengths], [int(x) for x in n])
    assert 0.95 < kv / step < 1.0
    assert attend < step
    assert np.isclose(attend / step, 1.0, atol=0.03)
