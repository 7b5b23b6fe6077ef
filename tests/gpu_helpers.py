"""Shared helpers of the GPU parity tests: run the HIP library through its C
ABI on seeded inputs and compare it with the CPU oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from autoregressive_kv_cache_amd import kvc
from autoregressive_kv_cache_amd.workloads import Workload, bf16_bits_to_f64, host_arrays

# Tolerances: fp32 inputs |gpu - ref| <= 1e-5 + 1e-5 |ref| on attention and
# context; bf16 inputs (fp32 accumulation, bf16 outputs) |d context| <= 2e-2
# and |d attention| <= 1e-2.  Cache contents and lengths are bit-exact.
F32_ATOL = F32_RTOL = 1e-5
BF16_CTX_ATOL = 2e-2
BF16_ATT_ATOL = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_gpu(inputs: dict[str, torch.Tensor], mode: str, scale=None, lengths_alias=False):
    """One step on the GPU; inputs are device tensors (left untouched by the
    out-of-place mode).  Returns device outputs."""
    q, nk, nv = inputs["query"], inputs["new_key"], inputs["new_value"]
    kc, vc = inputs["key_cache"], inputs["value_cache"]
    lens = inputs["lengths"]
    mask = inputs["append_mask"].to(torch.bool).contiguous().view(torch.uint8)
    B, Hq, Q, _ = q.shape
    M, Dv = kc.shape[2], vc.shape[3]
    dev = kc.device
    att = torch.full((B, Hq, Q, M), float("nan"), dtype=kc.dtype, device=dev)
    ctx = torch.full((B, Hq, Q, Dv), float("nan"), dtype=kc.dtype, device=dev)
    status = torch.full((B,), -99, dtype=torch.int32, device=dev)
    if mode == "oop":
        kc_out = torch.full_like(kc, float("nan"))
        vc_out = torch.full_like(vc, float("nan"))
        lens_out = torch.full_like(lens, -7)
        kvc.kvc_step_out_of_place(q, nk, nv, kc, vc, lens, mask, kc_out, vc_out, lens_out, att,
                                  ctx, status, scale=scale)
    else:
        kc_out, vc_out = kc, vc
        lens_out = lens if lengths_alias else torch.full_like(lens, -7)
        kvc.kvc_step_inplace(q, nk, nv, kc, vc, lens, mask, lens_out, att, ctx, status,
                             scale=scale)
    torch.cuda.synchronize()
    return {"key_cache": kc_out, "value_cache": vc_out, "lengths": lens_out, "attention": att,
            "context": ctx, "row_status": status}


def to_f64(t: torch.Tensor) -> np.ndarray:
    h = host_arrays({"x": t})["x"]
    return bf16_bits_to_f64(h) if h.dtype == np.uint16 else h.astype(np.float64)


def bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).numpy()


def check_floats(got: np.ndarray, ref: np.ndarray, dtype: str, what: str, kind: str):
    """Element-wise bar; the largest absolute and relative errors are printed
    beside it, so the margin each case leaves is on record."""
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    diff = np.abs(got - ref)
    max_abs = float(diff.max()) if diff.size else 0.0
    nz = np.abs(ref) > 0
    max_rel = float((diff[nz] / np.abs(ref[nz])).max()) if nz.any() else 0.0
    if dtype == "f32":
        err = diff - (F32_ATOL + F32_RTOL * np.abs(ref))
        worst = float(err.max()) if err.size else -1.0
        say(f"  {what}: max |d| {max_abs:.3e}, max |d|/|ref| {max_rel:.3e}; "
            f"bar |d| <= {F32_ATOL:g} + {F32_RTOL:g}|ref| (worst excess {worst:.3e})")
        assert worst <= 0.0, f"{what}: exceeds 1e-5 abs/rel by {worst:.3e}"
    else:
        tol = BF16_CTX_ATOL if kind == "context" else BF16_ATT_ATOL
        say(f"  {what}: max |d| {max_abs:.3e}, max |d|/|ref| {max_rel:.3e}; bar |d| <= {tol:g}")
        assert max_abs <= tol, f"{what}: max |diff| {max_abs:.3e} > {tol}"


def check_row_sums_ref(att: np.ndarray, ref_att: np.ndarray, dtype: str, what: str = ""):
    """Rows the oracle fills (valid query rows) sum to 1 within 1e-5 (fp32)
    or 2^-8 (bf16); rows the oracle leaves at zero are zero."""
    tol = 1e-5 if dtype == "f32" else 2.0 ** -8
    s_got = att.sum(axis=-1)
    s_ref = ref_att.sum(axis=-1)
    valid = s_ref > 0.5
    worst = float(np.abs(s_got[valid] - 1.0).max()) if valid.any() else 0.0
    say(f"  {what} row sums: max |sum - 1| {worst:.3e} over {int(valid.sum())} rows; bar {tol:.3e}")
    assert worst <= tol, f"{what}: row sum off by {worst:.3e} > {tol:.3e}"
    assert np.all(att[~valid] == 0.0), f"{what}: an invalid row is not zero"


def check_step(out: dict, ref: oracle.StepResult, dtype: str, what: str = ""):
    """Full comparison with an oracle result."""
    h_kc = host_arrays({"x": out["key_cache"]})["x"]
    h_vc = host_arrays({"x": out["value_cache"]})["x"]
    assert np.array_equal(h_kc.view(np.uint8), ref.key_cache.view(np.uint8)), \
        f"{what}: key cache differs"
    assert np.array_equal(h_vc.view(np.uint8), ref.value_cache.view(np.uint8)), \
        f"{what}: value cache differs"
    assert np.array_equal(out["lengths"].cpu().numpy(), ref.lengths), f"{what}: lengths differ"
    assert np.array_equal(out["row_status"].cpu().numpy(), ref.row_status), \
        f"{what}: row status differs"
    att = to_f64(out["attention"])
    ctx = to_f64(out["context"])
    # entries the oracle makes exactly zero (disallowed slots, invalid rows)
    zero = ref.attention == 0.0
    assert np.all(att[zero] == 0.0), f"{what}: non-zero attention where it must be 0"
    check_floats(att, ref.attention, dtype, f"{what} attention", "attention")
    check_floats(ctx, ref.context, dtype, f"{what} context", "context")
    if att.size:
        check_row_sums_ref(att, ref.attention, dtype, what)


def oracle_for(wl: Workload):
    return oracle.default()
