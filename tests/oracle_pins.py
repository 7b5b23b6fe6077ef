"""Pins for the CPU oracle: checks that tie it to something other than itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with what the pages or mathematics fix:

* the worked example that "Fixed-capacity KV cache" (section Examples) prints;
* PyTorch's own ``scaled_dot_product_attention`` (float64, CPU) with the
  library's lower-right causal bias -- the mask KempnerForge PR 542
  (Summary) switches to -- and its GQA head expansion; attention
  probabilities are read out of the same routine by attending an identity
  value matrix;
* the identity of "KV-Cache for Incremental Decoding" (Step-by-Step
  Approach, item 6): token-by-token steps equal one-shot causal attention,
  and so does any chunking (the chunk patterns of PR 542, Testing);
* closed forms (a single visible key, equal keys, scale folding);
* the invariants of "Autoregressive KV-cache append and causal attention"
  (Required behavior): untouched tail, no influence of the tail or future
  tokens, zero invalid rows, Q = 0 and n = 0 no-ops, inputs never modified;
* brute force over every mask pattern and length on a tiny shape.

The same functions run against deliberately broken copies of the oracle in
``test_oracle_mutants.py`` to show that each plausible mistake is caught.
"""
from __future__ import annotations

import os

import numpy as np
import torch
import torch.nn.functional as F
from torch.nn.attention.bias import causal_lower_right

from autoregressive_kv_cache_amd.workloads import (Workload, bf16_bits_to_f64, host_arrays,
                                                   make_inputs, prefix_mask)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# --------------------------------------------------------------------------
# helpers
# --------------------------------------------------------------------------
def widen(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


def small(name="s", B=2, Hq=4, Hk=2, Q=3, M=12, D=5, Dv=3, dtype="f32", **kw) -> Workload:
    kw.setdefault("len_range", (0, M - Q))
    kw.setdefault("n_rule", "uniform")
    return Workload(name, B=B, Hq=Hq, Hk=Hk, Q=Q, M=M, D=D, Dv=Dv, dtype=dtype, **kw)


def draw(wl: Workload, seed: int, **kw) -> dict[str, np.ndarray]:
    return host_arrays(make_inputs(wl, seed, "cpu", **kw))


def step(orc, h: dict[str, np.ndarray], scale=None):
    return orc.step(h["query"], h["new_key"], h["new_value"], h["key_cache"],
                    h["value_cache"], h["lengths"], h["append_mask"], scale=scale)


def counts(mask: np.ndarray) -> np.ndarray:
    return mask.astype(bool).sum(axis=1).astype(np.int64)


def sdpa_reference(h: dict[str, np.ndarray], scale=None):
    """Context and probabilities from torch SDPA (float64, CPU) per batch row,
    with K/V built by concatenating the old prefix and the appended rows."""
    q, nk, nv, kc, vc = (torch.from_numpy(widen(h[k])) for k in
                         ("query", "new_key", "new_value", "key_cache", "value_cache"))
    B, Hq, Q, _ = q.shape
    Hk, M = kc.shape[1], kc.shape[2]
    Dv = vc.shape[3]
    n = counts(h["append_mask"])
    ctx = torch.zeros(B, Hq, Q, Dv, dtype=torch.float64)
    att = torch.zeros(B, Hq, Q, M, dtype=torch.float64)
    for b in range(B):
        L0, nb = int(h["lengths"][b]), int(n[b])
        if nb == 0:
            continue
        K = torch.cat([kc[b, :, :L0], nk[b, :, :nb]], dim=1)
        V = torch.cat([vc[b, :, :L0], nv[b, :, :nb]], dim=1)
        L = L0 + nb
        bias = causal_lower_right(nb, L)
        qb = q[b, :, :nb]
        ctx[b, :, :nb] = F.scaled_dot_product_attention(qb, K, V, attn_mask=bias,
                                                        scale=scale, enable_gqa=True)
        eye = torch.eye(L, dtype=torch.float64).expand(Hk, L, L).contiguous()
        att[b, :, :nb, :L] = F.scaled_dot_product_attention(qb, K, eye, attn_mask=bias,
                                                            scale=scale, enable_gqa=True)
    return ctx.numpy(), att.numpy()


def close(a, b, tol, what):
    a, b = np.asarray(a), np.asarray(b)
    if a.shape != b.shape:
        raise AssertionError(f"{what}: shape {a.shape} vs {b.shape}")
    if not np.all(np.isfinite(a)):
        raise AssertionError(f"{what}: non-finite values")
    err = np.max(np.abs(a - b)) if a.size else 0.0
    if not err <= tol:
        raise AssertionError(f"{what}: max |diff| {err:.3e} > {tol:.1e}")


def read_golden(name: str) -> dict[str, list]:
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            rows = [[float(x) for x in r.split()] for r in rest.split(";")]
            out[key] = rows
    return out


# --------------------------------------------------------------------------
# pins
# --------------------------------------------------------------------------
def pin_page2_worked_example(orc):
    """"Fixed-capacity KV cache", Examples: lengths 2 then 3, the stored
    values, output [3, 4], weights 0.40111209/0.19777581/0.40111209, and a
    rejected append that leaves the length at 3."""
    g = read_golden("page2_worked_example.txt")
    M = int(g["capacity"][0][0])
    dk, dv = int(g["d_k"][0][0]), int(g["d_v"][0][0])
    f = np.float32
    kc = np.zeros((1, 1, M, dk), f)
    vc = np.zeros((1, 1, M, dv), f)
    # append 1: two steps into an empty cache (Q = 2, both True)
    k1 = np.array(g["append1_keys"], f)[None, None]
    v1 = np.array(g["append1_values"], f)[None, None]
    r1 = orc.step(np.zeros((1, 1, 2, dk), f), k1, v1, kc, vc, np.array([0]),
                  np.ones((1, 2), np.uint8))
    assert int(r1.lengths[0]) == int(g["len_after_append1"][0][0])
    # append 2 together with the query of decode_step: one step, Q = 1
    k2 = np.array(g["append2_keys"], f)[None, None]
    v2 = np.array(g["append2_values"], f)[None, None]
    q = np.array(g["query"], f)[None, None]
    r2 = orc.step(q, k2, v2, r1.key_cache, r1.value_cache, r1.lengths,
                  np.ones((1, 1), np.uint8))
    L = int(g["len_after_append2"][0][0])
    assert int(r2.lengths[0]) == L
    assert np.array_equal(r2.value_cache[0, 0, :L], np.array(g["values_after_append2"], f))
    decimals = int(g["weights_printed_decimals"][0][0])
    close(r2.attention[0, 0, 0, :L], np.array(g["weights"][0]), 0.5 * 10.0 ** -decimals,
          "page-2 weights")
    assert np.all(r2.attention[0, 0, 0, L:] == 0.0)
    # the output is exactly [3, 4]: the weights are symmetric (2a + b = 1)
    close(r2.context[0, 0, 0], np.array(g["output"][0]), 1e-12, "page-2 output")
    # append 3: two more steps do not fit in a capacity-4 cache
    k3 = np.array(g["append3_keys"], f)[None, None]
    v3 = np.array(g["append3_values"], f)[None, None]
    r3 = orc.step(np.zeros((1, 1, 2, dk), f), k3, v3, r2.key_cache, r2.value_cache,
                  r2.lengths, np.ones((1, 2), np.uint8))
    assert int(r3.lengths[0]) == int(g["len_after_append3"][0][0])
    assert int(r3.row_status[0]) != 0
    assert np.array_equal(r3.key_cache, r2.key_cache)
    assert np.array_equal(r3.value_cache, r2.value_cache)
    assert np.all(r3.attention == 0.0) and np.all(r3.context == 0.0)


def pin_sdpa_lower_right_gqa(orc):
    """Against torch SDPA with the lower-right causal bias and GQA expansion,
    over ragged lengths, partial masks, an empty row and an n = 0 row, with
    the default scale (SDPA's own 1/sqrt(D) default) and an explicit one."""
    for seed, wl, scale in [
        (0, small(B=3, Hq=6, Hk=2, Q=4, M=14, D=5, Dv=3), None),
        (1, small(B=2, Hq=4, Hk=4, Q=3, M=10, D=4, Dv=6, force_len0_row=0), 0.7),
        (2, small(B=2, Hq=8, Hk=1, Q=5, M=16, D=3, Dv=2, force_n0_row=1), None),
        (3, small(B=2, Hq=4, Hk=2, Q=3, M=16, D=8, Dv=8, dtype="bf16"), None),
    ]:
        h = draw(wl, seed)
        r = step(orc, h, scale)
        ctx, att = sdpa_reference(h, scale)
        close(r.context, ctx, 1e-12, f"context vs SDPA (seed {seed})")
        close(r.attention, att, 1e-12, f"attention vs SDPA (seed {seed})")


def pin_stable_softmax_large_scores(orc):
    """Scores far above 1000 ("Fixed-capacity KV cache", Constraints) must
    give finite output equal to SDPA's."""
    wl = small(B=2, Hq=2, Hk=2, Q=2, M=20, D=16, Dv=4, std=8.0, scale=4.0)
    h = draw(wl, 5)
    r = step(orc, h, 4.0)
    q = widen(h["query"])
    k = widen(h["key_cache"])
    assert np.max(np.abs(4.0 * np.einsum("d,jd->j", q[0, 0, 0], k[0, 0]))) > 1000.0
    ctx, att = sdpa_reference(h, 4.0)
    close(r.context, ctx, 1e-9, "context, large scores")
    close(r.attention, att, 1e-12, "attention, large scores")


def pin_identity_stepwise_chunked_oneshot(orc):
    """"KV-Cache for Incremental Decoding", Step-by-Step Approach item 6: the
    stepwise outputs equal one-shot causal attention; PR 542 (Testing)
    appends chunks 3+2+3, 1+7 and 5+1+2 to a filled cache with GQA, batch 2."""
    T, B, Hq, Hk, M, D, Dv, L0 = 8, 2, 4, 2, 24, 6, 5, 7
    gen = torch.Generator().manual_seed(11)
    q = torch.randn(B, Hq, T, D, generator=gen).numpy()
    k = torch.randn(B, Hk, T, D, generator=gen).numpy()
    v = torch.randn(B, Hk, T, Dv, generator=gen).numpy()
    kc0 = torch.randn(B, Hk, M, D, generator=gen).numpy()
    vc0 = torch.randn(B, Hk, M, Dv, generator=gen).numpy()
    results = {}
    for chunks in [(8,), (1,) * 8, (3, 2, 3), (1, 7), (5, 1, 2)]:
        kc, vc = kc0.copy(), vc0.copy()
        lengths = np.full(B, L0, np.int64)
        ctx = np.zeros((B, Hq, T, Dv))
        t0 = 0
        for c in chunks:
            sl = slice(t0, t0 + c)
            r = orc.step(q[:, :, sl].copy(), k[:, :, sl].copy(), v[:, :, sl].copy(), kc, vc,
                         lengths, np.ones((B, c), np.uint8))
            ctx[:, :, sl] = r.context
            kc, vc, lengths = r.key_cache, r.value_cache, r.lengths
            t0 += c
        results[chunks] = (ctx, kc, vc, lengths)
    ref_ctx, ref_kc, ref_vc, ref_len = results[(8,)]
    assert np.all(ref_len == L0 + T)
    for chunks, (ctx, kc, vc, lengths) in results.items():
        close(ctx, ref_ctx, 1e-12, f"chunks {chunks} vs one shot")
        assert np.array_equal(kc, ref_kc) and np.array_equal(vc, ref_vc)
        assert np.array_equal(lengths, ref_len)
    # one shot from an empty cache is ordinary causal attention, where the
    # lower-right and top-left alignments coincide
    r = orc.step(q, k, v, kc0, vc0, np.zeros(B, np.int64), np.ones((B, T), np.uint8))
    full = F.scaled_dot_product_attention(torch.from_numpy(q).double(),
                                          torch.from_numpy(k).double(),
                                          torch.from_numpy(v).double(), is_causal=True,
                                          enable_gqa=True).numpy()
    close(r.context, full, 1e-12, "empty-cache one shot vs is_causal SDPA")


def pin_chunk_sequence_40_32_24(orc):
    """PR 542 (Testing): chunks of 40, 32 and 24 appended in turn equal one
    96-token append, row for row."""
    B, Hq, Hk, M, D, Dv, L0 = 2, 4, 2, 160, 8, 8, 30
    T = 96
    gen = torch.Generator().manual_seed(3)
    q = torch.randn(B, Hq, T, D, generator=gen).numpy()
    k = torch.randn(B, Hk, T, D, generator=gen).numpy()
    v = torch.randn(B, Hk, T, Dv, generator=gen).numpy()
    kc = torch.randn(B, Hk, M, D, generator=gen).numpy()
    vc = torch.randn(B, Hk, M, Dv, generator=gen).numpy()
    lengths = np.full(B, L0, np.int64)
    one = orc.step(q, k, v, kc, vc, lengths, np.ones((B, T), np.uint8))
    t0, ctx = 0, np.zeros_like(one.context)
    for c in (40, 32, 24):
        sl = slice(t0, t0 + c)
        r = orc.step(q[:, :, sl].copy(), k[:, :, sl].copy(), v[:, :, sl].copy(), kc, vc,
                     lengths, np.ones((B, c), np.uint8))
        ctx[:, :, sl] = r.context
        kc, vc, lengths = r.key_cache, r.value_cache, r.lengths
        t0 += c
    close(ctx, one.context, 1e-12, "40/32/24 chunks vs one append")
    assert np.array_equal(kc, one.key_cache) and np.array_equal(lengths, one.lengths)


def pin_closed_forms(orc):
    """A single visible key gives probability 1 and context = that value,
    exactly; equal keys give uniform weights and the mean value; scaling q by
    c equals scaling the scale by c."""
    # single visible key: empty cache, first token
    wl = small(B=2, Hq=4, Hk=2, Q=1, M=6, D=4, Dv=3, len_range=(0, 0), n_rule="all")
    h = draw(wl, 21)
    r = step(orc, h)
    assert np.all(r.attention[:, :, 0, 0] == 1.0)
    assert np.all(r.attention[:, :, 0, 1:] == 0.0)
    nv = widen(h["new_value"])
    for hq in range(4):
        assert np.array_equal(r.context[:, hq, 0], nv[:, hq // 2, 0])
    # equal keys: uniform weights over len + t + 1 slots, context = mean of V
    B, Hq, Hk, Q, M, D, Dv = 1, 2, 1, 2, 9, 3, 4
    key = np.array([0.5, -1.0, 2.0], np.float32)
    kc = np.tile(key, (B, Hk, M, 1)).astype(np.float32)
    nk = np.tile(key, (B, Hk, Q, 1)).astype(np.float32)
    gen = torch.Generator().manual_seed(4)
    vc = torch.randn(B, Hk, M, Dv, generator=gen).numpy()
    nv = torch.randn(B, Hk, Q, Dv, generator=gen).numpy()
    q = torch.randn(B, Hq, Q, D, generator=gen).numpy()
    L0 = 5
    r = orc.step(q, nk, nv, kc, vc, np.array([L0]), np.ones((B, Q), np.uint8))
    vals = np.concatenate([vc[0, 0, :L0], nv[0, 0, :Q]], axis=0).astype(np.float64)
    for t in range(Q):
        close(r.attention[0, :, t, :L0 + t + 1], np.full((Hq, L0 + t + 1), 1.0 / (L0 + t + 1)),
              1e-15, "uniform weights")
        close(r.context[0, :, t], np.tile(vals[:L0 + t + 1].mean(axis=0), (Hq, 1)), 1e-12,
              "mean of values")
    # scale folding: (c q, s) == (q, c s), with c a power of two (exact)
    wl = small(B=2, Hq=4, Hk=2, Q=3, M=12, D=5, Dv=3)
    h = draw(wl, 8)
    r1 = step(orc, h, 0.75)
    h2 = dict(h)
    h2["query"] = (h["query"] * np.float32(4.0)).astype(np.float32)
    r2 = step(orc, h2, 0.1875)
    close(r1.attention, r2.attention, 1e-14, "scale folding, attention")
    close(r1.context, r2.context, 1e-13, "scale folding, context")


def pin_default_scale_uses_query_width(orc):
    """"Autoregressive KV-cache append and causal attention", Required
    behavior: the default scale is 1/sqrt(D) with D the query/key width (D
    differs from Dv here); a non-positive or non-finite scale is refused."""
    wl = small(B=2, Hq=2, Hk=1, Q=2, M=10, D=9, Dv=4)
    h = draw(wl, 6)
    r0 = step(orc, h, None)
    r1 = step(orc, h, 1.0 / 3.0)
    close(r0.attention, r1.attention, 1e-15, "default scale")
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        try:
            step(orc, h, bad)
        except ValueError:
            continue
        raise AssertionError(f"scale {bad} accepted")


def pin_gqa_equals_repeated_mha(orc):
    """GQA equals MHA with each KV head repeated for its Hq/Hk query heads
    (query head h reads KV head floor(h/(Hq/Hk)))."""
    wl = small(B=2, Hq=6, Hk=2, Q=3, M=12, D=4, Dv=5)
    h = draw(wl, 9)
    r = step(orc, h)
    G = 3
    h2 = dict(h)
    for k in ("new_key", "new_value", "key_cache", "value_cache"):
        h2[k] = np.ascontiguousarray(np.repeat(h[k], G, axis=1))
    r2 = step(orc, h2)
    close(r.attention, r2.attention, 0.0, "GQA vs repeated MHA attention")
    close(r.context, r2.context, 0.0, "GQA vs repeated MHA context")


def pin_bf16_widening(orc):
    """bfloat16 inputs are read exactly: the same values given as float32
    give bit-identical double outputs."""
    wl = small(B=2, Hq=4, Hk=2, Q=3, M=12, D=6, Dv=5, dtype="bf16")
    h = draw(wl, 13)
    r = step(orc, h)
    h32 = {k: (widen(v).astype(np.float32) if v.dtype == np.uint16 else v) for k, v in h.items()}
    r32 = step(orc, h32)
    close(r.attention, r32.attention, 0.0, "bf16 vs widened f32 attention")
    close(r.context, r32.context, 0.0, "bf16 vs widened f32 context")
    assert np.array_equal(widen(r.key_cache), r32.key_cache.astype(np.float64))


def pin_invariants(orc):
    """"Autoregressive KV-cache append and causal attention", Required
    behavior: unwritten entries (tail included) keep their bits; inputs are
    not modified; updated lengths are length + n; probabilities sum to 1 on
    valid rows and are 0 outside slots 0..length+t; invalid rows are zero;
    cache tail, future tokens and invalid query rows cannot change outputs."""
    wl = small(B=3, Hq=4, Hk=2, Q=4, M=15, D=5, Dv=3, len_range=(0, 11))
    h = draw(wl, 17)
    before = {k: v.copy() for k, v in h.items()}
    r = step(orc, h)
    for k in h:
        assert np.array_equal(h[k], before[k]), f"input {k} modified"
    n = counts(h["append_mask"])
    L = h["lengths"]
    assert np.array_equal(r.lengths, L + n)
    for b in range(wl.B):
        kc_exp = h["key_cache"][b].copy()
        vc_exp = h["value_cache"][b].copy()
        kc_exp[:, L[b]:L[b] + n[b]] = h["new_key"][b, :, :n[b]]
        vc_exp[:, L[b]:L[b] + n[b]] = h["new_value"][b, :, :n[b]]
        assert np.array_equal(r.key_cache[b], kc_exp)
        assert np.array_equal(r.value_cache[b], vc_exp)
        for t in range(wl.Q):
            if t < n[b]:
                s = r.attention[b, :, t].sum(axis=-1)
                close(s, np.ones_like(s), 1e-14, "row sums")
                assert np.all(r.attention[b, :, t, L[b] + t + 1:] == 0.0)
                assert np.all(r.attention[b, :, t, :L[b] + t + 1] > 0.0)
            else:
                assert np.all(r.attention[b, :, t] == 0.0)
                assert np.all(r.context[b, :, t] == 0.0)
    # perturb the tail beyond each new length, new rows t >= n, query rows t >= n
    h2 = {k: v.copy() for k, v in h.items()}
    for b in range(wl.B):
        h2["key_cache"][b, :, L[b] + n[b]:] = np.float32(123.0)
        h2["value_cache"][b, :, L[b] + n[b]:] = np.float32(-77.0)
        h2["key_cache"][b, :, L[b]:L[b] + n[b]] = np.float32(55.0)  # overwritten by append
        h2["new_key"][b, :, n[b]:] = np.float32(9.0)
        h2["new_value"][b, :, n[b]:] = np.float32(-9.0)
        h2["query"][b, :, n[b]:] = np.float32(1e3)
    r2 = step(orc, h2)
    assert np.array_equal(r.attention, r2.attention)
    assert np.array_equal(r.context, r2.context)


def pin_empty_and_noop_rows(orc):
    """Q = 0 and rows with n = 0 keep cache and lengths and give empty or
    zero outputs."""
    wl = small(B=2, Hq=2, Hk=1, Q=0, M=8, D=3, Dv=2, len_range=(0, 8), n_rule="all")
    h = draw(wl, 2)
    r = step(orc, h)
    assert r.attention.shape == (2, 2, 0, 8) and r.context.shape == (2, 2, 0, 2)
    assert np.array_equal(r.key_cache, h["key_cache"])
    assert np.array_equal(r.value_cache, h["value_cache"])
    assert np.array_equal(r.lengths, h["lengths"])
    wl = small(B=2, Hq=2, Hk=1, Q=3, M=8, D=3, Dv=2, n_rule="uniform", force_n0_row=0)
    h = draw(wl, 2)
    r = step(orc, h)
    assert r.lengths[0] == h["lengths"][0]
    assert np.array_equal(r.key_cache[0], h["key_cache"][0])
    assert np.all(r.attention[0] == 0.0) and np.all(r.context[0] == 0.0)


def pin_brute_force_all_masks(orc):
    """Every length 0..M and every one of the 2^Q mask patterns on a tiny
    shape: prefix masks that fit match SDPA; others leave the row as it was
    (status != 0, same length, same cache, zero outputs)."""
    B, Hq, Hk, Q, M, D, Dv = 1, 2, 1, 3, 4, 2, 3
    gen = torch.Generator().manual_seed(1)
    base = {
        "query": torch.randn(B, Hq, Q, D, generator=gen).numpy(),
        "new_key": torch.randn(B, Hk, Q, D, generator=gen).numpy(),
        "new_value": torch.randn(B, Hk, Q, Dv, generator=gen).numpy(),
        "key_cache": torch.randn(B, Hk, M, D, generator=gen).numpy(),
        "value_cache": torch.randn(B, Hk, M, Dv, generator=gen).numpy(),
    }
    for L0 in range(0, M + 1):
        for bits in range(2 ** Q):
            mask = np.array([[(bits >> t) & 1 for t in range(Q)]], np.uint8)
            h = dict(base, lengths=np.array([L0], np.int64), append_mask=mask)
            r = step(orc, h)
            nrun = 0
            while nrun < Q and mask[0, nrun]:
                nrun += 1
            is_prefix = mask[0].sum() == nrun
            fits = L0 + nrun <= M
            if is_prefix and fits:
                assert r.row_status[0] == 0
                ctx, att = sdpa_reference(h)
                close(r.context, ctx, 1e-12, f"len {L0} mask {bits:03b}")
                close(r.attention, att, 1e-12, f"len {L0} mask {bits:03b}")
                assert r.lengths[0] == L0 + nrun
            else:
                assert r.row_status[0] != 0
                assert r.lengths[0] == L0
                assert np.array_equal(r.key_cache, h["key_cache"])
                assert np.array_equal(r.value_cache, h["value_cache"])
                assert np.all(r.attention == 0.0) and np.all(r.context == 0.0)
    # lengths outside [0, M] are rejected the same way
    for L0 in (-1, M + 1):
        h = dict(base, lengths=np.array([L0], np.int64), append_mask=np.zeros((1, Q), np.uint8))
        r = step(orc, h)
        assert r.row_status[0] != 0 and r.lengths[0] == L0
        assert np.array_equal(r.key_cache, h["key_cache"])


def pin_attend_row_matches_sdpa(orc):
    """The one-row entry (used for sampled checks at full size) gives the
    same row as SDPA over the updated cache."""
    wl = small(B=2, Hq=4, Hk=2, Q=3, M=12, D=5, Dv=3, dtype="bf16")
    h = draw(wl, 31)
    kc, vc, _, n, _ = orc.append(h["new_key"], h["new_value"], h["key_cache"], h["value_cache"],
                                 h["lengths"], h["append_mask"], Hq=wl.Hq)
    ctx_ref, att_ref = sdpa_reference(h)
    for b in range(wl.B):
        for hq in range(wl.Hq):
            for t in range(wl.Q):
                a, c = orc.attend_row(h["query"], kc, vc, int(h["lengths"][b]), int(n[b]), b,
                                      hq, t)
                close(a, att_ref[b, hq, t], 1e-12, "row attention")
                close(c, ctx_ref[b, hq, t], 1e-12, "row context")


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
