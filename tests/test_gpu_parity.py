"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on
seeded inputs, element by element; cache contents and lengths bit-exact,
floats within the stated tolerances (tests/gpu_helpers.py)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from autoregressive_kv_cache_amd import kvc
from autoregressive_kv_cache_amd.workloads import (WORKLOADS, Workload, draw_lengths_and_counts,
                                                   host_arrays, make_inputs, paged_layout)
from gpu_helpers import bits, check_floats, check_step, run_gpu, say, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kvc.load()  # fail loudly when the HIP library is missing
    yield


def full_check(wl: Workload, seed: int, mode: str, scale="default", gen_device="cpu", **kw):
    scale = wl.scale if scale == "default" else scale
    say(f"[case] {wl.name} seed={seed} mode={mode} scale={scale} {kw}")
    inp = {k: v.cpu() for k, v in make_inputs(wl, seed, gen_device, **kw).items()}
    h = host_arrays(inp)
    ref = oracle.default().step(h["query"], h["new_key"], h["new_value"], h["key_cache"],
                                h["value_cache"], h["lengths"], h["append_mask"], scale=scale)
    dinp = {k: v.to(DEV) for k, v in inp.items()}
    out = run_gpu(dinp, mode, scale=scale)
    check_step(out, ref, wl.dtype, f"{wl.name}/{seed}/{mode}")
    if mode == "oop":  # inputs untouched
        for k, v in inp.items():
            assert torch.equal(dinp[k].cpu(), v), f"input {k} modified"
    return out, ref


# -- the small workloads, several seeds, both entry points -------------------
SMALL = ["tiny_mixed_f32", "chunk_gqa_bf16", "chunk_gqa_f32", "mha_stress_f32"]


@pytest.mark.parametrize("mode", ["oop", "inplace"])
@pytest.mark.parametrize("name", SMALL)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_small_workloads(name, seed, mode):
    full_check(WORKLOADS[name], seed, mode)


@pytest.mark.parametrize("seed", range(3, 8))
def test_tiny_more_seeds(seed):
    full_check(WORKLOADS["tiny_mixed_f32"], seed, "oop")


# -- reduced decode shapes: several splits, ragged tails, full oracle -------
@pytest.mark.parametrize("mode", ["oop", "inplace"])
@pytest.mark.parametrize("wl", [
    WORKLOADS["decode_gqa_bf16"].with_(name="decode_small", B=4, M=1536, len_range=(200, 1535)),
    WORKLOADS["long_decode_bf16"].with_(name="long_small", B=2, M=4099, len_range=(1000, 4098)),
    WORKLOADS["decode_gqa_bf16"].with_(name="decode_f32_small", B=3, M=777, dtype="f32",
                                       len_range=(0, 776)),
    WORKLOADS["chunk_gqa_bf16"].with_(name="chunk_ragged", M=700, len_range=(100, 640)),
    # stream path with two tokens per step: empty caches, rows that append
    # nothing, caches filled to capacity
    Workload(name="decode_q2_edges", B=8, Hq=4, Hk=2, Q=2, M=200, D=64, Dv=64, dtype="bf16",
             len_range=(0, 198), n_rule="uniform", force_len0_row=0, force_n0_row=1),
    # 9 to 15 packed rows: the stream kernel's two 8-row groups (two waves
    # per worker); ragged row counts, two tokens, rows that append nothing
    Workload(name="decode_r12", B=5, Hq=12, Hk=1, Q=1, M=777, D=128, Dv=128, dtype="bf16",
             len_range=(0, 776), n_rule="all"),
    Workload(name="decode_r9_d64", B=6, Hq=18, Hk=2, Q=1, M=640, D=64, Dv=64, dtype="bf16",
             len_range=(1, 639), n_rule="all"),
    Workload(name="decode_r15_q3", B=4, Hq=10, Hk=2, Q=3, M=300, D=128, Dv=128, dtype="bf16",
             len_range=(0, 297), n_rule="uniform", force_len0_row=0, force_n0_row=1),
    # more batch rows than the attend kernel prepares by itself (the
    # preparation kernel runs first)
    Workload(name="decode_b1030", B=1030, Hq=2, Hk=1, Q=1, M=96, D=64, Dv=64, dtype="bf16",
             len_range=(0, 95), n_rule="all"),
    # small heads (rows of at most 64 bytes): the one-slot-per-lane decode
    # kernel, fp32 and bf16, 1 to 8 packed rows, several chunks and ragged
    # tails, empty caches and rows that append nothing, and the preparation
    # kernel above 1024 rows
    Workload(name="small_f32_d8_r6", B=5, Hq=4, Hk=2, Q=3, M=300, D=8, Dv=8, dtype="f32",
             len_range=(0, 297), n_rule="uniform", force_len0_row=0, force_n0_row=1),
    Workload(name="small_f32_d16_r4", B=4, Hq=8, Hk=2, Q=1, M=700, D=16, Dv=16, dtype="f32",
             len_range=(0, 699), n_rule="all", std=4.0),
    Workload(name="small_bf16_d32_r8", B=4, Hq=8, Hk=2, Q=2, M=500, D=32, Dv=32, dtype="bf16",
             len_range=(0, 498), n_rule="uniform"),
    Workload(name="small_bf16_d16_r1", B=3, Hq=4, Hk=4, Q=1, M=200, D=16, Dv=16, dtype="bf16",
             len_range=(0, 199), n_rule="all"),
    Workload(name="small_b1030", B=1030, Hq=2, Hk=1, Q=1, M=96, D=8, Dv=8, dtype="f32",
             len_range=(0, 95), n_rule="all"),
], ids=lambda w: w.name)
def test_reduced_decode_shapes(wl, mode):
    full_check(wl, 0, mode)


# -- full sizes --------------------------------------------------------------
def test_decode_gqa_full_size_inplace_and_oop():
    """Single-token GQA decode at its full size (B=32, Hq=32, Hk=8, M=8192,
    D=Dv=128, bf16, 1e4 sentinel tail): full oracle comparison."""
    wl = WORKLOADS["decode_gqa_bf16"]
    for mode in ("inplace", "oop"):
        full_check(wl, 0, mode, gen_device=DEV)


def test_decode_write_through_full_check():
    """The decode step at twice the batch (B=64, 4 packed rows per KV head):
    its exp values pass 12 MiB per launch (16.3 MiB at seed 0), so the stream
    kernel writes its workspace through the L2 where the B=32 step (8.2 MiB)
    keeps the default policy.
    Every output against the oracle, in place and out of place."""
    wl = WORKLOADS["decode_gqa_bf16"].with_(name="decode_gqa_bf16_b64", B=64)
    lengths, n = draw_lengths_and_counts(wl, 0)
    chunks = sum(wl.Hk * (-(-int(l) // 64) + (1 if k > 0 else 0)) for l, k in zip(lengths, n))
    assert chunks * 4 * 64 * 2 > 12 << 20  # 4 rows of 64 bf16 exp values per chunk
    for mode in ("inplace", "oop"):
        full_check(wl, 0, mode, gen_device=DEV)


def test_long_decode_share_full_check():
    """One GPU's share of the slot-sharded long decode (M = 16384 of 131072,
    64 query heads over 8 KV heads): every output against the oracle, in
    place and out of place."""
    wl = WORKLOADS["long_decode_share8_bf16"]
    for mode in ("inplace", "oop"):
        full_check(wl, 0, mode, gen_device=DEV)


def test_long_decode_full_size():
    """Long-context GQA decode at its full size (B=4, Hq=64, Hk=8, M=131072,
    D=Dv=128, bf16): every output element against the oracle (one oracle
    step, ~7 s, serves both entry points), in place and out of place."""
    wl = WORKLOADS["long_decode_bf16"]
    say(f"[case] {wl.name} full size, oracle step")
    inp = {k: v.cpu() for k, v in make_inputs(wl, 0, "cpu").items()}
    h = host_arrays(inp)
    ref = oracle.default().step(h["query"], h["new_key"], h["new_value"], h["key_cache"],
                                h["value_cache"], h["lengths"], h["append_mask"], scale=wl.scale)
    for mode in ("inplace", "oop"):
        say(f"[case] {wl.name} full size mode={mode}")
        dinp = {k: v.to(DEV) for k, v in inp.items()}
        out = run_gpu(dinp, mode)
        check_step(out, ref, wl.dtype, f"{wl.name}/{mode}")
        del dinp, out
        torch.cuda.empty_cache()


# -- edge cases --------------------------------------------------------------
def tiny(**kw) -> Workload:
    base = dict(name="edge", B=3, Hq=4, Hk=2, Q=3, M=20, D=8, Dv=8, dtype="f32",
                len_range=(0, 17), n_rule="uniform")
    base.update(kw)
    return Workload(**base)


@pytest.mark.parametrize("mode", ["oop", "inplace"])
@pytest.mark.parametrize("wl", [
    tiny(name="q0", Q=0),
    tiny(name="all_n0", n_rule="choice", n_choices=(0,)),
    tiny(name="m1", M=1, Q=1, len_range=(0, 0), n_rule="all"),
    tiny(name="mha1", B=1, Hq=1, Hk=1, Q=1, M=5, len_range=(0, 4), n_rule="all"),
    tiny(name="odd_dims", D=3, Dv=5, M=37, len_range=(0, 30)),
    tiny(name="odd_dims_bf16", D=7, Dv=3, M=300, len_range=(0, 290), dtype="bf16"),
    tiny(name="fill_to_capacity", M=10, Q=3, len_range=(7, 7), n_rule="all"),
    tiny(name="full_cache", M=10, Q=2, len_range=(10, 10), n_rule="all"),
    tiny(name="many_rows", Hq=32, Hk=2, Q=3, M=300, len_range=(0, 290)),
    tiny(name="wide_head", Hq=2, Hk=1, D=512, Dv=256, M=64, len_range=(0, 60), dtype="bf16"),
], ids=lambda w: w.name)
def test_edge_shapes(wl, mode):
    full_check(wl, 0, mode)


@pytest.mark.parametrize("mode", ["oop", "inplace"])
def test_rejected_rows(mode):
    """Rows outside the contract (bad length, non-prefix mask, overflow) are
    no-ops with a status; other rows of the batch are unaffected."""
    wl = tiny(name="rejected", B=5, Q=3, M=12)
    lengths = np.array([3, -1, 13, 4, 11], np.int64)
    n = np.array([2, 1, 0, 1, 2], np.int64)
    inp = make_inputs(wl, 4, "cpu", lengths=lengths, n=n)
    inp["append_mask"][3] = torch.tensor([True, False, True])  # not a prefix
    h = host_arrays(inp)
    ref = oracle.default().step(h["query"], h["new_key"], h["new_value"], h["key_cache"],
                                h["value_cache"], h["lengths"], h["append_mask"])
    assert list(ref.row_status) == [0, 1, 1, 3, 2]
    out = run_gpu({k: v.to(DEV) for k, v in inp.items()}, mode)
    check_step(out, ref, "f32", f"rejected/{mode}")


def test_lengths_updated_in_place():
    wl = tiny(name="alias")
    inp = {k: v.to(DEV) for k, v in make_inputs(wl, 2, "cpu").items()}
    h = host_arrays(inp)
    ref = oracle.default().step(h["query"], h["new_key"], h["new_value"], h["key_cache"],
                                h["value_cache"], h["lengths"], h["append_mask"])
    out = run_gpu(inp, "inplace", lengths_alias=True)
    assert out["lengths"].data_ptr() == inp["lengths"].data_ptr()
    check_step(out, ref, "f32", "alias")


def test_inplace_repeat_is_idempotent():
    """With lengths_out != lengths, repeating the in-place step repeats the
    same step (what the benchmark relies on)."""
    wl = WORKLOADS["decode_gqa_bf16"].with_(B=4, M=2048, len_range=(100, 2047))
    inp = {k: v.to(DEV) for k, v in make_inputs(wl, 3, "cpu").items()}
    first = {k: v.clone() for k, v in run_gpu(inp, "inplace").items()}
    second = run_gpu(inp, "inplace")
    for k in ("key_cache", "value_cache", "lengths", "attention", "context"):
        assert torch.equal(bits_t(first[k]), bits_t(second[k])), k


def bits_t(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


@pytest.mark.parametrize("mode", ["oop", "inplace"])
def test_tail_future_invariance_bitwise(mode):
    """Cache tail beyond the new length, new rows t >= n and query rows
    t >= n cannot change any output (bitwise)."""
    wl = WORKLOADS["chunk_gqa_bf16"].with_(M=900, len_range=(100, 800))
    inp = make_inputs(wl, 6, "cpu")
    lengths, n = draw_lengths_and_counts(wl, 6)
    pert = {k: v.clone() for k, v in inp.items()}
    for b in range(wl.B):
        L, nb = int(lengths[b]), int(n[b])
        pert["key_cache"][b, :, L + nb:] = 77.0
        pert["value_cache"][b, :, L + nb:] = -55.0
        pert["key_cache"][b, :, L:L + nb] = 3.0
        pert["new_key"][b, :, nb:] = 1e3
        pert["new_value"][b, :, nb:] = -1e3
        pert["query"][b, :, nb:] = 1e3
    o1 = run_gpu({k: v.to(DEV) for k, v in inp.items()}, mode)
    o2 = run_gpu({k: v.to(DEV) for k, v in pert.items()}, mode)
    assert torch.equal(bits_t(o1["attention"]), bits_t(o2["attention"]))
    assert torch.equal(bits_t(o1["context"]), bits_t(o2["context"]))


def test_page_face_dict_and_inplace_twin():
    wl = WORKLOADS["tiny_mixed_f32"]
    inp = {k: v.to(DEV) for k, v in make_inputs(wl, 1, "cpu").items()}
    h = host_arrays(inp)
    ref = oracle.default().step(h["query"], h["new_key"], h["new_value"], h["key_cache"],
                                h["value_cache"], h["lengths"], h["append_mask"], scale=0.5)
    out = kvc.kv_cache_attention_step(inp["query"], inp["new_key"], inp["new_value"],
                                      inp["key_cache"], inp["value_cache"], inp["lengths"],
                                      inp["append_mask"], {"scale": 0.5})
    assert set(out) == {"key_cache", "value_cache", "lengths", "attention", "context"}
    check_floats(to_f64(out["attention"]), ref.attention, "f32", "face attention", "attention")
    check_floats(to_f64(out["context"]), ref.context, "f32", "face context", "context")
    assert np.array_equal(out["lengths"].cpu().numpy(), ref.lengths)
    out2 = kvc.kv_cache_attention_step_(inp["query"], inp["new_key"], inp["new_value"],
                                        inp["key_cache"], inp["value_cache"], inp["lengths"],
                                        inp["append_mask"], {"scale": 0.5})
    assert out2["key_cache"].data_ptr() == inp["key_cache"].data_ptr()
    assert np.array_equal(bits(inp["key_cache"]), ref.key_cache.view(np.int32))
    assert np.array_equal(inp["lengths"].cpu().numpy(), ref.lengths)
    bad = inp["append_mask"].clone()
    bad[0] = torch.tensor([False, True, False])
    with pytest.raises(ValueError):
        kvc.kv_cache_attention_step(inp["query"], inp["new_key"], inp["new_value"],
                                    inp["key_cache"], inp["value_cache"], inp["lengths"], bad,
                                    {}, validate=True)


def test_plan_paths():
    """The decode-shaped workloads (the tiny step's head size 8 included)
    take the vector decode path, the chunk workloads (160 packed rows) the
    matrix-core chunk path."""
    expect = {"decode_gqa_bf16": 1, "long_decode_bf16": 1, "mha_stress_f32": 1,
              "chunk_gqa_bf16": 2, "chunk_gqa_f32": 2, "tiny_mixed_f32": 1}
    for name, path in expect.items():
        w = WORKLOADS[name]
        d = kvc.KvcDims(w.B, w.Hq, w.Hk, w.Q, w.M, w.D, w.Dv)
        assert kvc.kvc_plan_step(d, kvc.dtype_code(w.torch_dtype))["path"] == path, name


# -- the matrix-core chunk path (more than 8 packed rows) --------------------
def chunk_wl(**kw) -> Workload:
    base = dict(name="chunk", B=2, Hq=4, Hk=1, Q=5, M=200, D=64, Dv=64, dtype="bf16",
                len_range=(0, 190), n_rule="uniform")
    base.update(kw)
    return Workload(**base)


CHUNK_CASES = [
    chunk_wl(name="rows20_ragged"),                                   # R = 20, not a multiple of 16
    chunk_wl(name="rows16_d128", Hq=2, Q=8, D=128, Dv=128, M=300, len_range=(0, 290)),
    chunk_wl(name="rows16_d256", Hq=1, Q=16, D=256, Dv=256, M=130, len_range=(0, 114)),
    chunk_wl(name="fill_to_capacity", Hq=1, Q=16, M=128, len_range=(112, 112), n_rule="all"),
    chunk_wl(name="prefill_len0", Hq=8, Hk=2, Q=40, M=96, len_range=(0, 0), n_rule="all"),
    chunk_wl(name="many_heads", B=3, Hq=16, Hk=2, Q=3, M=257, len_range=(0, 250)),
]
# fp32 inputs take the fp64 matrix-core variant (D = Dv in {64, 128});
# the stress scale (std 8, scale 4) pushes the scores into the hundreds
CHUNK_CASES += [
    chunk_wl(name="rows20_ragged_f32", dtype="f32"),
    chunk_wl(name="rows16_d128_f32", dtype="f32", Hq=2, Q=8, D=128, Dv=128, M=300,
             len_range=(0, 290)),
    chunk_wl(name="fill_to_capacity_f32", dtype="f32", Hq=1, Q=16, M=128,
             len_range=(112, 112), n_rule="all"),
    chunk_wl(name="prefill_len0_f32", dtype="f32", Hq=8, Hk=2, Q=40, M=96,
             len_range=(0, 0), n_rule="all"),
    chunk_wl(name="stress_f32", dtype="f32", B=3, Hq=16, Hk=2, Q=3, M=257,
             len_range=(0, 250), std=8.0, scale=4.0),
]


@pytest.mark.parametrize("mode", ["oop", "inplace"])
@pytest.mark.parametrize("wl", CHUNK_CASES, ids=lambda w: w.name)
def test_chunk_path_shapes(wl, mode):
    d = kvc.KvcDims(wl.B, wl.Hq, wl.Hk, wl.Q, wl.M, wl.D, wl.Dv)
    assert kvc.kvc_plan_step(d, kvc.dtype_code(wl.torch_dtype))["path"] == 2
    for seed in (0, 1):
        full_check(wl, seed, mode)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode", ["oop", "inplace"])
def test_chunk_path_rejected_rows(mode, dtype):
    """Outside-contract rows on the chunk path: no-ops with a status."""
    wl = chunk_wl(name="chunk_rejected", B=5, Q=5, M=70, dtype=dtype)
    lengths = np.array([3, -1, 71, 4, 68], np.int64)
    n = np.array([5, 1, 0, 2, 5], np.int64)
    inp = make_inputs(wl, 4, "cpu", lengths=lengths, n=n)
    inp["append_mask"][3] = torch.tensor([True, False, True, False, False])  # not a prefix
    h = host_arrays(inp)
    ref = oracle.default().step(h["query"], h["new_key"], h["new_value"], h["key_cache"],
                                h["value_cache"], h["lengths"], h["append_mask"])
    assert list(ref.row_status) == [0, 1, 1, 3, 2]
    out = run_gpu({k: v.to(DEV) for k, v in inp.items()}, mode)
    check_step(out, ref, dtype, f"chunk_rejected/{mode}/{dtype}")


def test_chunk_sequence_40_32_24():
    """Chunks of 40, 32 and 24 tokens appended in turn through the chunk path
    equal the oracle after every step (in place, lengths carried over)."""
    wl = chunk_wl(name="seq", B=2, Hq=8, Hk=2, Q=40, M=400, len_range=(50, 60), n_rule="all")
    inp = make_inputs(wl, 11, "cpu")
    h = host_arrays(inp)
    kc, vc, lens = h["key_cache"], h["value_cache"], h["lengths"]
    dk, dv = inp["key_cache"].to(DEV), inp["value_cache"].to(DEV)
    dlen = inp["lengths"].to(DEV)
    for step, cnt in enumerate((40, 32, 24)):
        step_in = make_inputs(wl, 100 + step, "cpu", lengths=lens, n=np.full(wl.B, cnt))
        hs = host_arrays(step_in)
        ref = oracle.default().step(hs["query"], hs["new_key"], hs["new_value"], kc, vc, lens,
                                    hs["append_mask"])
        dinp = {k: v.to(DEV) for k, v in step_in.items()}
        dinp["key_cache"], dinp["value_cache"], dinp["lengths"] = dk, dv, dlen
        out = run_gpu(dinp, "inplace")
        check_step(out, ref, "bf16", f"seq step {step}")
        kc, vc, lens = ref.key_cache, ref.value_cache, ref.lengths
        dk, dv, dlen = out["key_cache"], out["value_cache"], out["lengths"]


def misaligned(t: torch.Tensor) -> torch.Tensor:
    """A copy of t whose data starts 2 bytes past a 16-byte boundary."""
    flat = torch.empty(t.numel() + 8, dtype=t.dtype, device=t.device)
    view = flat[1:1 + t.numel()].view(t.shape)
    view.copy_(t)
    assert view.data_ptr() % 16 != 0
    return view


@pytest.mark.parametrize("mode", ["oop", "inplace"])
def test_misaligned_buffers_take_generic_path(mode):
    """Buffers that are not 16-byte aligned cannot use the vector path; the
    library falls back to the generic kernel with the same results."""
    wl = WORKLOADS["decode_gqa_bf16"].with_(name="misaligned", B=3, M=600, len_range=(10, 599))
    inp = make_inputs(wl, 9, "cpu")
    h = host_arrays(inp)
    ref = oracle.default().step(h["query"], h["new_key"], h["new_value"], h["key_cache"],
                                h["value_cache"], h["lengths"], h["append_mask"])
    dinp = {k: v.to(DEV) for k, v in inp.items()}
    for k in ("query", "key_cache", "value_cache"):
        dinp[k] = misaligned(dinp[k])
    out = run_gpu(dinp, mode)
    check_step(out, ref, wl.dtype, f"misaligned/{mode}")


# -- the paged cache (kvc_step_paged: block pools + block table) ------------
def run_paged(inp: dict, kp, vp, table, scale=None):
    """kvc_step_paged on device copies; returns the updated pools and outputs."""
    d = {k: v.to(DEV) for k, v in inp.items()}
    kp, vp, table = kp.to(DEV), vp.to(DEV), table.to(DEV)
    B, Hq, Q, _ = d["query"].shape
    M = table.shape[1] * kp.shape[2]
    att = torch.full((B, Hq, Q, M), 3.0, dtype=kp.dtype, device=DEV)  # stale values must go
    ctx = torch.full((B, Hq, Q, vp.shape[3]), 3.0, dtype=kp.dtype, device=DEV)
    lens_out = torch.empty_like(d["lengths"])
    status = torch.empty(B, dtype=torch.int32, device=DEV)
    mask = d["append_mask"].contiguous().view(torch.uint8)
    kvc.kvc_step_paged(d["query"], d["new_key"], d["new_value"], kp, vp, table, d["lengths"], mask,
                       lens_out, att, ctx, status, scale=scale)
    torch.cuda.synchronize()
    return {"key_cache": kp.cpu(), "value_cache": vp.cpu(), "lengths": lens_out.cpu(),
            "attention": att.cpu(), "context": ctx.cpu(), "row_status": status.cpu()}


def paged_ref(inp: dict, kp, vp, table, scale=None):
    h = host_arrays(dict(inp, key_pool=kp, value_pool=vp))
    r = oracle.default().step_paged(h["query"], h["new_key"], h["new_value"], h["key_pool"],
                                    h["value_pool"], table.numpy(), h["lengths"],
                                    h["append_mask"], scale=scale)
    # check_step reads the pools where it reads the caches
    return oracle.StepResult(r.key_pool, r.value_pool, r.lengths, r.attention, r.context,
                             r.row_status)


PAGED_CASES = [
    # (workload, block size): 4 packed rows (bf16 D = 128), 8 packed rows
    # (Q = 2, appends that cross a block edge), fp32 with D != Dv, bf16 D = 64
    (WORKLOADS["decode_gqa_bf16"].with_(name="paged_d128", B=5, M=1024,
                                        len_range=(0, 1023)), 64),
    (WORKLOADS["decode_gqa_bf16"].with_(name="paged_d128_b256", B=3, M=1024,
                                        len_range=(1, 1023)), 256),
    (chunk_wl(name="paged_rows8", B=4, Hq=4, Hk=1, Q=2, M=512, D=128, Dv=128,
              len_range=(60, 70), n_rule="all"), 64),
    (WORKLOADS["mha_stress_f32"].with_(name="paged_f32", B=4, M=512, len_range=(0, 508)), 128),
    (chunk_wl(name="paged_d64", B=3, Hq=8, Hk=2, Q=1, M=640, len_range=(0, 639), n_rule="all"),
     128),
    # more than 8 packed rows: the matrix-core chunk kernels over the pool
    (chunk_wl(name="paged_chunk_bf16", B=2, Hq=8, Hk=2, Q=40, M=512, len_range=(0, 470)), 64),
    (chunk_wl(name="paged_chunk_d128", B=3, Hq=4, Hk=1, Q=5, M=512, D=128, Dv=128,
              len_range=(0, 500)), 128),
    (chunk_wl(name="paged_chunk_f32", dtype="f32", B=2, Hq=8, Hk=2, Q=20, M=256,
              len_range=(0, 230), std=8.0, scale=4.0), 64),
    # the generic kernel: blocks smaller than the decode or chunk paths'
    # chunks, and head sizes without a decode or chunk kernel
    (WORKLOADS["decode_gqa_bf16"].with_(name="paged_gen_b16", B=3, M=512,
                                        len_range=(0, 511)), 16),
    (chunk_wl(name="paged_gen_chunk_b32", B=2, Hq=8, Hk=2, Q=40, M=256, len_range=(0, 200)), 32),
    (Workload(name="paged_small_d8", B=3, Hq=4, Hk=2, Q=3, M=512, D=8, Dv=8, dtype="f32",
              len_range=(0, 500), n_rule="uniform"), 64),
    (WORKLOADS["tiny_mixed_f32"].with_(name="paged_gen_tiny"), 4),
    (WORKLOADS["tiny_mixed_f32"].with_(name="paged_gen_tiny_b1"), 1),
    (chunk_wl(name="paged_gen_d96", B=3, Hq=6, Hk=2, Q=3, M=384, D=96, Dv=80,
              len_range=(0, 380), n_rule="uniform"), 128),
]


@pytest.mark.parametrize("wl,bs", PAGED_CASES, ids=lambda x: getattr(x, "name", str(x)))
def test_paged_against_oracle(wl, bs):
    for seed in (0, 1):
        say(f"[case] paged {wl.name} bs={bs} seed={seed}")
        inp = make_inputs(wl, seed, "cpu")
        kp, vp, table = paged_layout(inp["key_cache"], inp["value_cache"], bs, seed)
        inp = {k: v for k, v in inp.items() if k not in ("key_cache", "value_cache")}
        ref = paged_ref(inp, kp, vp, table, scale=wl.scale)
        out = run_paged(inp, kp, vp, table, scale=wl.scale)
        check_step(out, ref, wl.dtype, f"paged {wl.name}/{seed}")


def test_paged_misaligned_pools_take_generic_path():
    """Pools that start 2 bytes past a 16-byte boundary: the generic kernel,
    results as the oracle's."""
    wl = WORKLOADS["decode_gqa_bf16"].with_(name="paged_misaligned", B=3, M=512,
                                            len_range=(0, 511))
    say(f"[case] paged misaligned pools")
    inp = make_inputs(wl, 0, "cpu")
    kp, vp, table = paged_layout(inp["key_cache"], inp["value_cache"], 64, 0)
    ref = paged_ref(inp, kp, vp, table)
    d = {k: v.to(DEV) for k, v in inp.items()}
    kpd, vpd = misaligned(kp.to(DEV)), misaligned(vp.to(DEV))
    tab = table.to(DEV)
    B, Hq, Q, _ = d["query"].shape
    att = torch.full((B, Hq, Q, wl.M), 3.0, dtype=kp.dtype, device=DEV)
    ctx = torch.full((B, Hq, Q, wl.Dv), 3.0, dtype=kp.dtype, device=DEV)
    lens_out = torch.empty_like(d["lengths"])
    status = torch.empty(B, dtype=torch.int32, device=DEV)
    mask = d["append_mask"].contiguous().view(torch.uint8)
    kvc.kvc_step_paged(d["query"], d["new_key"], d["new_value"], kpd, vpd, tab, d["lengths"],
                       mask, lens_out, att, ctx, status)
    torch.cuda.synchronize()
    out = {"key_cache": kpd.cpu(), "value_cache": vpd.cpu(), "lengths": lens_out.cpu(),
           "attention": att.cpu(), "context": ctx.cpu(), "row_status": status.cpu()}
    check_step(out, ref, wl.dtype, "paged misaligned pools")


def test_paged_full_size_bench_configuration():
    """The paged step at the full decode size in the configuration bench.py
    times (B=32, Hq=32, Hk=8, M=8192, 64-slot blocks permuted over the pool):
    every output against the oracle."""
    wl = WORKLOADS["decode_gqa_bf16"]
    say(f"[case] paged {wl.name} full size bs=64")
    inp = make_inputs(wl, 0, "cpu")
    kp, vp, table = paged_layout(inp["key_cache"], inp["value_cache"], 64, 0)
    inp = {k: v for k, v in inp.items() if k not in ("key_cache", "value_cache")}
    ref = paged_ref(inp, kp, vp, table, scale=wl.scale)
    out = run_paged(inp, kp, vp, table, scale=wl.scale)
    check_step(out, ref, wl.dtype, f"paged {wl.name} full size")
    del inp, kp, vp, out
    torch.cuda.empty_cache()


def test_paged_identity_table_matches_dense_bitwise():
    """A table that lays the pool out like the dense cache gives bit-identical
    outputs to kvc_step_inplace on that dense cache (same kernels, same order)."""
    wl = WORKLOADS["decode_gqa_bf16"].with_(name="paged_ident", B=3, M=512, len_range=(0, 511))
    inp = make_inputs(wl, 5, "cpu")
    B, Hk, M, D = inp["key_cache"].shape
    bs = 64
    mb = M // bs
    kp = inp["key_cache"].reshape(B, Hk, mb, bs, D).permute(0, 2, 1, 3, 4).reshape(
        B * mb, Hk, bs, D).contiguous()
    vp = inp["value_cache"].reshape(B, Hk, mb, bs, D).permute(0, 2, 1, 3, 4).reshape(
        B * mb, Hk, bs, D).contiguous()
    table = torch.arange(B * mb, dtype=torch.int32).reshape(B, mb)
    dense = run_gpu({k: v.to(DEV) for k, v in inp.items()}, "inplace")
    rest = {k: v for k, v in inp.items() if k not in ("key_cache", "value_cache")}
    paged = run_paged(rest, kp, vp, table)
    assert torch.equal(bits_t(paged["attention"]), bits_t(dense["attention"].cpu()))
    assert torch.equal(bits_t(paged["context"]), bits_t(dense["context"].cpu()))
    back = paged["key_cache"].reshape(B, mb, Hk, bs, D).permute(0, 2, 1, 3, 4).reshape(B, Hk, M, D)
    assert torch.equal(bits_t(back), bits_t(dense["key_cache"].cpu()))


def bits_t(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32)


def test_paged_shared_prefix_and_spare_blocks():
    """Rows 0 and 1 map the same first block (a prefix below both lengths);
    spare pool blocks and the shared block keep their bits."""
    wl = WORKLOADS["decode_gqa_bf16"].with_(name="paged_shared", B=3, M=512, len_range=(70, 500))
    inp = make_inputs(wl, 7, "cpu")
    kp, vp, table = paged_layout(inp["key_cache"], inp["value_cache"], 64, 7, spare_blocks=4)
    shared = int(table[0, 0])
    table[1, 0] = shared
    inp = {k: v for k, v in inp.items() if k not in ("key_cache", "value_cache")}
    ref = paged_ref(inp, kp, vp, table)
    out = run_paged(inp, kp, vp, table)
    check_step(out, ref, "bf16", "paged shared prefix")
    assert torch.equal(bits_t(out["key_cache"][shared]), bits_t(kp[shared]))


def test_paged_bad_entries_stay_inside_the_pool():
    """Table entries outside the pool: past a row's length + n they are never
    touched (results exact); inside a row's visible range they read as zero
    rows and are never written, and every other row is still exact."""
    wl = WORKLOADS["decode_gqa_bf16"].with_(name="paged_bad", B=4, M=512, len_range=(10, 300))
    inp = make_inputs(wl, 9, "cpu")
    kp, vp, table = paged_layout(inp["key_cache"], inp["value_cache"], 64, 9, spare_blocks=2)
    lens = inp["lengths"].numpy()
    nb = kp.shape[0]
    for b in range(4):  # unused blocks of every row: out of range both ways
        first_unused = (int(lens[b]) + 1 + 63) // 64
        table[b, first_unused:] = torch.tensor([-5, nb, 1 << 30, -1, nb + 7, 12345, -99, nb])[
            :table.shape[1] - first_unused]
    rest = {k: v for k, v in inp.items() if k not in ("key_cache", "value_cache")}
    ref = paged_ref(rest, kp, vp, table)
    out = run_paged(rest, kp, vp, table)
    check_step(out, ref, "bf16", "paged unused bad entries")
    # now a bad entry inside the visible prefix of the longest row (its first
    # block, not the one its new row goes to): the other rows stay exact
    bb = int(np.argmax(lens))
    assert lens[bb] >= 64
    bad = table.clone()
    bad[bb, 0] = nb + 3
    out2 = run_paged(rest, kp, vp, bad)
    for b in [x for x in range(4) if x != bb]:
        np.testing.assert_array_equal(to_f64(out2["attention"][b]), to_f64(out["attention"][b]))
        np.testing.assert_array_equal(to_f64(out2["context"][b]), to_f64(out["context"][b]))
    assert torch.equal(bits_t(out2["key_cache"]), bits_t(out["key_cache"]))
    assert torch.equal(bits_t(out2["value_cache"]), bits_t(out["value_cache"]))


def test_paged_bad_block_size_is_refused():
    """A block size that is not a power of two (and not M) comes back as
    KVC_ERR_SHAPE before anything runs: the pools stay as they were."""
    wl = WORKLOADS["decode_gqa_bf16"].with_(name="paged_refuse", B=2, M=192, len_range=(0, 150))
    inp = make_inputs(wl, 1, "cpu")
    kp, vp, table = paged_layout(inp["key_cache"], inp["value_cache"], 48, 1)
    rest = {k: v for k, v in inp.items() if k not in ("key_cache", "value_cache")}
    with pytest.raises(kvc.KvcError) as e:
        run_paged(rest, kp, vp, table)
    assert e.value.code == -2


# -- capture in a HIP graph (serving loops replay a captured step) ----------
@pytest.mark.parametrize("wl_name,paged", [("decode_gqa_bf16", False), ("chunk_gqa_bf16", False),
                                           ("decode_gqa_bf16", True)])
def test_graph_replays_match_eager(wl_name, paged):
    """The step enqueues only kernels on the caller's stream (no allocation,
    no memset, no synchronisation), so it can be captured in a HIP graph.
    Several replays, with eager work and synchronisations between them, each
    give the eager result bit for bit (in place, lengths_out != lengths, so
    every replay is the same step)."""
    wl = WORKLOADS[wl_name].with_(name="graph", B=4, M=1024, len_range=(0, 1000))
    inp = {k: v.to(DEV) for k, v in make_inputs(wl, 3, "cpu").items()}
    B, Hq, Q, _ = inp["query"].shape
    M, Dv = inp["key_cache"].shape[2], inp["value_cache"].shape[3]
    mask = inp["append_mask"].contiguous().view(torch.uint8)
    if paged:
        kp, vp, table = paged_layout(inp["key_cache"], inp["value_cache"], 64, 3)
        dims = kvc.KvcDims(B, Hq, kp.shape[1], Q, M, inp["query"].shape[3], Dv)
    else:
        dims = kvc.dims_of(inp["query"], inp["key_cache"], inp["value_cache"])
    ws = kvc.workspace_for(dims, kvc.dtype_code(wl.torch_dtype), DEV)
    att = torch.empty(B, Hq, Q, M, dtype=wl.torch_dtype, device=DEV)
    ctx = torch.empty(B, Hq, Q, Dv, dtype=wl.torch_dtype, device=DEV)
    lens_out = torch.empty_like(inp["lengths"])
    status = torch.empty(B, dtype=torch.int32, device=DEV)

    def step(stream=None):
        if paged:
            kvc.kvc_step_paged(inp["query"], inp["new_key"], inp["new_value"], kp, vp, table,
                               inp["lengths"], mask, lens_out, att, ctx, status, workspace=ws,
                               stream=stream)
        else:
            kvc.kvc_step_inplace(inp["query"], inp["new_key"], inp["new_value"],
                                 inp["key_cache"], inp["value_cache"], inp["lengths"], mask,
                                 lens_out, att, ctx, status, workspace=ws, stream=stream)

    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in (att, ctx, lens_out, status)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step(stream=s)
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (att, ctx):
            t.fill_(float("nan"))
        lens_out.fill_(-1)
        status.fill_(-9)
        scratch = torch.randn(1 << 20, device=DEV).sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, exp in zip((att, ctx, lens_out, status), want):
            assert torch.equal(got.view(torch.int16) if got.element_size() == 2 else got,
                               exp.view(torch.int16) if exp.element_size() == 2 else exp), \
                f"replay {rep} differs ({wl_name}, paged={paged})"
        del scratch


# -- read-only re-attention (kvc_attend_over_cache) --------------------------
def reatt_case(dtype: str, B: int, Hq: int, Hk: int, Qmax: int, M: int, D: int, Dv: int,
               seed: int, rows: int | None = None, std: float = 1.0):
    """Packed queries, a continuous cache of ``rows`` rows, per-sequence query
    counts S_b in [0, Qmax] and cached lengths L_b in [S_b, M] (seeded)."""
    rng = np.random.default_rng(seed)
    S = rng.integers(0, Qmax + 1, B)
    S[0] = Qmax
    L = np.array([rng.integers(s, M + 1) for s in S], np.int64)
    L[-1] = M  # a full row
    cu = np.concatenate([[0], np.cumsum(S)]).astype(np.int64)
    g = torch.Generator().manual_seed(seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    rows = B if rows is None else rows
    q = (torch.randn(int(cu[-1]), Hq, D, generator=g) * std).to(tdt)
    kc = (torch.randn(rows, Hk, M, D, generator=g) * std).to(tdt)
    vc = (torch.randn(rows, Hk, M, Dv, generator=g) * std).to(tdt)
    return q, torch.from_numpy(cu), kc, vc, torch.from_numpy(L), S


def run_reatt(q, cu, kc, vc, L, Q, M=None, table=None, slots=None, sink=None, scale=None):
    d = {k: (None if v is None else v.to(DEV)) for k, v in dict(
        q=q, cu=cu, kc=kc, vc=vc, L=L, table=table, slots=slots, sink=sink).items()}
    out = torch.full((q.shape[0], q.shape[1], vc.shape[3]), float("nan"), dtype=kc.dtype,
                     device=DEV)
    status = torch.full((cu.shape[0] - 1,), -9, dtype=torch.int32, device=DEV)
    before = (bits_t(d["kc"]).clone(), bits_t(d["vc"]).clone())
    kvc.kvc_attend_over_cache(d["q"], d["cu"], d["kc"], d["vc"], d["L"], out, Q, M=M,
                              block_table=d["table"], slot_ids=d["slots"], head_sink=d["sink"],
                              row_status=status, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(bits_t(d["kc"]), before[0]) and torch.equal(bits_t(d["vc"]), before[1]), \
        "the cache was written"
    return out.cpu(), status.cpu()


def reatt_ref(q, cu, kc_logical, vc_logical, L, Q, sink=None, scale=None):
    h = host_arrays({"q": q, "k": kc_logical, "v": vc_logical})
    return oracle.default().reattend(h["q"], cu.numpy(), h["k"], h["v"], L.numpy(), Q,
                                     sink=None if sink is None else sink.numpy().astype(np.float64),
                                     scale=scale)


def cumulative(L: torch.Tensor, start: int = 1000) -> torch.Tensor:
    """The [B + 1] cumulative form of per-sequence lengths (any start)."""
    return torch.cat([torch.zeros(1, dtype=torch.int64), torch.cumsum(L, 0)]) + start


def test_reattend_full_size_decode_shape():
    """Re-attention at the full decode size (32 sequences, 32 query heads
    over 8 KV heads, 8192 cached slots, up to one query each): the packed
    output against the oracle, with the cached lengths in both forms."""
    q, cu, kc, vc, L, S = reatt_case("bf16", 32, 32, 8, 1, 8192, 128, 128, 3)
    ref, rst = reatt_ref(q, cu, kc, vc, L, 1)
    for form, Lk in (("lengths", L), ("cumulative", cumulative(L))):
        say(f"[case] reattend full decode size, {form}")
        out, st = run_reatt(q, cu, kc, vc, Lk, 1)
        assert list(st.numpy()) == list(rst)
        check_floats(to_f64(out), ref, "bf16", f"reattend full size ({form})", "context")
    del q, kc, vc
    torch.cuda.empty_cache()


REATT_CASES = [
    # dtype, B, Hq, Hk, Qmax, M, D, Dv (decode-shaped: (Hq/Hk) * Qmax <= 8)
    ("bf16", 6, 16, 4, 2, 700, 128, 128),
    ("bf16", 5, 8, 2, 1, 1024, 64, 64),
    ("f32", 4, 8, 8, 4, 300, 64, 32),
    # head sizes without a decode kernel: the generic kernel
    ("bf16", 4, 6, 2, 3, 200, 96, 80),
    # a small head: the one-slot-per-lane decode kernel, read only
    ("bf16", 4, 8, 2, 2, 300, 32, 32),
]


@pytest.mark.parametrize("kform", ["lengths", "cumulative"])
@pytest.mark.parametrize("case", REATT_CASES, ids=lambda c: "-".join(map(str, c)))
@pytest.mark.parametrize("layout", ["rows", "slot_ids", "paged", "paged16"])
def test_reattend_against_oracle(case, layout, kform):
    dtype, B, Hq, Hk, Qmax, M, D, Dv = case
    for seed in (0, 1):
        say(f"[case] reattend {case} {layout} {kform} seed={seed}")
        rows = B + 3 if layout == "slot_ids" else B
        q, cu, kc, vc, L, S = reatt_case(dtype, B, Hq, Hk, Qmax, M, D, Dv, seed, rows=rows,
                                         std=4.0 if dtype == "f32" else 1.0)
        if kform == "cumulative":  # the oracle takes the same form
            L = cumulative(L, start=seed * 77)
        sink = torch.from_numpy(np.random.default_rng(seed + 9).standard_normal(Hq) * 3
                                ).float() if seed == 1 else None
        scale = 0.25 if dtype == "f32" else None
        if layout == "rows":
            out, st = run_reatt(q, cu, kc, vc, L, Qmax, sink=sink, scale=scale)
            ref, rst = reatt_ref(q, cu, kc, vc, L, Qmax, sink, scale)
        elif layout == "slot_ids":
            slots = torch.from_numpy(np.random.default_rng(seed).permutation(rows)[:B]
                                     .astype(np.int32))
            out, st = run_reatt(q, cu, kc, vc, L, Qmax, slots=slots, sink=sink, scale=scale)
            ref, rst = reatt_ref(q, cu, kc[slots.long()], vc[slots.long()], L, Qmax, sink, scale)
        else:
            Mp = (M + 63) // 64 * 64
            kpad = torch.zeros(B, Hk, Mp, D, dtype=kc.dtype)
            vpad = torch.zeros(B, Hk, Mp, Dv, dtype=vc.dtype)
            kpad[:, :, :M], vpad[:, :, :M] = kc, vc
            # 64-slot blocks, or 16-slot ones (below a chunk: the generic kernel)
            kp, vp, table = paged_layout(kpad, vpad, 16 if layout == "paged16" else 64, seed)
            out, st = run_reatt(q, cu, kp, vp, L, Qmax, M=Mp, table=table, sink=sink,
                                scale=scale)
            ref, rst = reatt_ref(q, cu, kpad, vpad, L, Qmax, sink, scale)
        assert list(st.numpy()) == list(rst), (st, rst)
        check_floats(to_f64(out), ref, dtype, f"reattend {layout} {case}/{seed}", "context")


def test_reattend_chunk_path_with_sink():
    """A prefill-sized re-attention (40 queries x 4 heads per KV head) takes
    the matrix-core chunk kernel, with the sink added in the combine."""
    q, cu, kc, vc, L, S = reatt_case("bf16", 3, 8, 2, 40, 400, 64, 64, 4)
    sink = torch.linspace(-2, 2, 8)
    d = kvc.KvcDims(3, 8, 2, 40, 400, 64, 64)
    assert kvc.kvc_plan_step(d, kvc.KVC_BF16)["path"] == 2
    out, st = run_reatt(q, cu, kc, vc, L, 40, sink=sink)
    ref, rst = reatt_ref(q, cu, kc, vc, L, 40, sink)
    assert list(st.numpy()) == list(rst)
    check_floats(to_f64(out), ref, "bf16", "reattend chunk path", "context")


def test_reattend_rejected_sequences():
    """L > M, more queries than cached positions, more than Q queries: zero
    rows and their codes; the other sequences exact."""
    q, cu, kc, vc, L, S = reatt_case("bf16", 4, 8, 2, 2, 256, 128, 128, 5)
    cu = torch.tensor([0, 1, 3, 4, 7], dtype=torch.int64)  # S = 1, 2, 1, 3 (> Q = 2)
    q = torch.randn(7, 8, 128).to(torch.bfloat16)
    L = torch.tensor([300, 1, 50, 100], dtype=torch.int64)   # L > M; S > L
    for Lk in (L, cumulative(L)):
        out, st = run_reatt(q, cu, kc, vc, Lk, 2)
        ref, rst = reatt_ref(q, cu, kc, vc, Lk, 2)
        assert list(st.numpy()) == [kvc.ROW_BAD_LENGTH, kvc.ROW_BAD_QUERIES, kvc.ROW_OK,
                                    kvc.ROW_BAD_QUERIES] == list(rst)
        got = to_f64(out)
        assert not got[[0, 1, 2, 4, 5, 6]].any()
        check_floats(got, ref, "bf16", "reattend rejected", "context")
    # offsets that go down: a negative length is a bad length
    down = torch.tensor([0, 5, 3, 53, 153], dtype=torch.int64)
    _, st = run_reatt(q, cu, kc, vc, down, 2)
    assert int(st[1]) == kvc.ROW_BAD_LENGTH


# -- backward of the step (kvc_step_backward, fp32) ---------------------------
# |d| <= BWD_TOL (1 + |ref|).  fp32: the gradients are summed in fp64 and
# rounded once to fp32 (relative 2^-24); the largest error seen over every
# backward case is 1.1e-7 (1 + |ref|), so 1e-6 leaves a margin of ~9x.
# bf16: one rounding to bf16 (relative <= 2^-9) of the gradient and of the
# pass-through sum it is added to; the largest seen is 3.7e-3.
BWD_TOL = {"f32": 1e-6,
           "bf16": 4e-3}


def check_grad(got: np.ndarray, want: np.ndarray, dtype: str, what: str):
    """|got - want| <= BWD_TOL (1 + |want|) element-wise; the largest error,
    absolute and relative to (1 + |want|), is printed beside the bar."""
    assert np.all(np.isfinite(got)), f"{what}: not finite"
    diff = np.abs(got - want)
    scaled = diff / (1 + np.abs(want))
    mx = float(diff.max()) if diff.size else 0.0
    ms = float(scaled.max()) if diff.size else 0.0
    say(f"  {what}: max |d| {mx:.3e}, max |d|/(1+|ref|) {ms:.3e}; bar {BWD_TOL[dtype]:g}")
    assert ms <= BWD_TOL[dtype], f"{what}: off by {ms:.3e} (1 + |ref|) > {BWD_TOL[dtype]:g}"

BWD_CASES = [
    WORKLOADS["decode_gqa_bf16"].with_(name="bwd_decode", dtype="f32", B=3, M=300,
                                       len_range=(0, 299), tail_sentinel=None),
    chunk_wl(name="bwd_chunk", dtype="f32", B=3, Hq=8, Hk=2, Q=5, M=200, len_range=(0, 190)),
    WORKLOADS["mha_stress_f32"].with_(name="bwd_stress", B=3, M=160, len_range=(0, 150)),
    # R = 320 packed rows: ten 32-row tiles per chunk, and statistics row
    # groups that take a second tile
    chunk_wl(name="bwd_rows320", dtype="f32", B=2, Hq=16, Hk=2, Q=40, M=160, len_range=(0, 100)),
    # at most 4 packed rows, D = Dv in {64, 128}: the vector-unit kernels
    # for bf16 (runs of 576 slots; capacities that end inside a run and a
    # 64-slot chunk), the fp64 matrix-core ones for fp32
    Workload(name="bwd_vec_q2", B=3, Hq=4, Hk=2, Q=2, M=1100, D=64, Dv=64, dtype="f32",
             len_range=(0, 1090), n_rule="uniform"),
    Workload(name="bwd_vec_r1", B=2, Hq=4, Hk=4, Q=1, M=700, D=128, Dv=128, dtype="f32",
             len_range=(0, 699), n_rule="all"),
    Workload(name="bwd_vec_r3", B=2, Hq=3, Hk=1, Q=1, M=1536, D=64, Dv=64, dtype="f32",
             len_range=(500, 1535), n_rule="all"),
    # 5 to 8 packed rows: the 8-row vector waves in bf16 (the long decode's
    # 8 query heads per KV head; two tokens of three heads)
    Workload(name="bwd_vec_r8", B=3, Hq=16, Hk=2, Q=1, M=1100, D=128, Dv=128, dtype="f32",
             len_range=(0, 1090), n_rule="all"),
    Workload(name="bwd_vec_r6_q2", B=3, Hq=6, Hk=2, Q=2, M=700, D=64, Dv=64, dtype="f32",
             len_range=(0, 690), n_rule="uniform"),
    # head sizes without a tiled kernel: the generic kernels (slot pieces of
    # 64, 32, 8 and 4 slots; ragged row tiles; D != Dv; the tiny step)
    WORKLOADS["tiny_mixed_f32"].with_(name="bwd_gen_tiny"),
    Workload(name="bwd_gen_d96_80", B=2, Hq=6, Hk=2, Q=3, M=300, D=96, Dv=80, dtype="f32",
             len_range=(0, 290), n_rule="uniform"),
    Workload(name="bwd_gen_d256", B=2, Hq=8, Hk=2, Q=1, M=200, D=256, Dv=256, dtype="f32",
             len_range=(0, 199), n_rule="all"),
    Workload(name="bwd_gen_rows40", B=2, Hq=8, Hk=2, Q=10, M=150, D=48, Dv=40, dtype="f32",
             len_range=(0, 130), n_rule="uniform"),
    Workload(name="bwd_gen_d1024", B=2, Hq=2, Hk=1, Q=2, M=70, D=1024, Dv=512, dtype="f32",
             len_range=(0, 60), n_rule="all"),
    # the two backward workloads of bench.py at their full sizes
    WORKLOADS["chunk_gqa_f32"].with_(name="bwd_chunk_gqa_full"),
    WORKLOADS["mha_stress_f32"].with_(name="bwd_stress_full"),
]


@pytest.mark.parametrize("wl", BWD_CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("upstream", ["all", "context_only"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_against_oracle(wl, upstream, dtype):
    wl = wl.with_(dtype=dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    for seed in (0, 1):
        say(f"[case] backward {wl.name} {dtype} {upstream} seed={seed}")
        inp = make_inputs(wl, seed, "cpu")
        if seed == 1:
            # a rejected row, a row that appends nothing (with three rows or
            # more), and a last row that appends at least one
            inp["lengths"][0] = wl.M + 5
            if wl.B > 2:
                inp["append_mask"][-2] = False
            if not inp["append_mask"][-1, 0] and inp["lengths"][-1] < wl.M:
                inp["append_mask"][-1, 0] = True
        dinp = {k: v.to(DEV) for k, v in inp.items()}
        g = torch.Generator().manual_seed(100 + seed)
        B, Hq, Q, D = inp["query"].shape
        Hk, M, Dv = inp["key_cache"].shape[1], inp["key_cache"].shape[2], inp["value_cache"].shape[3]
        ups = {"d_attention": torch.randn(B, Hq, Q, M, generator=g).to(tdt),
               "d_context": torch.randn(B, Hq, Q, Dv, generator=g).to(tdt),
               "d_key_cache_out": torch.randn(B, Hk, M, D, generator=g).to(tdt),
               "d_value_cache_out": torch.randn(B, Hk, M, Dv, generator=g).to(tdt)}
        if upstream == "context_only":
            ups = {k: (v if k == "d_context" else None) for k, v in ups.items()}
        outs = {k: torch.full_like(dinp[src], float("nan")) for k, src in
                (("g_query", "query"), ("g_new_key", "new_key"), ("g_new_value", "new_value"),
                 ("g_key_cache", "key_cache"), ("g_value_cache", "value_cache"))}
        mask = dinp["append_mask"].contiguous().view(torch.uint8)
        kvc.kvc_step_backward(dinp["query"], dinp["new_key"], dinp["new_value"],
                              dinp["key_cache"], dinp["value_cache"], dinp["lengths"], mask,
                              *[None if v is None else v.to(DEV) for v in ups.values()],
                              **outs, scale=wl.scale)
        torch.cuda.synchronize()
        h = host_arrays(inp)
        ref = oracle.step_backward(*(to_f64(inp[k]) for k in ("query", "new_key", "new_value",
                                                              "key_cache", "value_cache")),
                                   h["lengths"], h["append_mask"],
                                   **{k: None if v is None else to_f64(v) for k, v in ups.items()},
                                   scale=wl.scale)
        for name, want in (("g_query", ref.query), ("g_new_key", ref.new_key),
                           ("g_new_value", ref.new_value), ("g_key_cache", ref.key_cache),
                           ("g_value_cache", ref.value_cache)):
            check_grad(to_f64(outs[name]), want, dtype, f"{wl.name}/{dtype}/{upstream}/{seed} {name}")


@pytest.mark.parametrize("which", ["query", "d_key_cache_out", "g_value_cache", "g_new_key"])
@pytest.mark.parametrize("wl", [BWD_CASES[0], BWD_CASES[4]], ids=lambda w: w.name)
def test_backward_misaligned_buffers_take_generic_path(which, wl):
    """A buffer, in or out, that is not 16-byte aligned (2 bytes past a
    boundary) sends the call to the generic kernels: every gradient still
    matches the oracle."""
    wl = wl.with_(dtype="bf16")
    say(f"[case] backward misaligned {wl.name} {which}")
    inp = make_inputs(wl, 0, "cpu")
    dinp = {k: v.to(DEV) for k, v in inp.items()}
    B, Hq, Q, D = inp["query"].shape
    Hk, M, Dv = inp["key_cache"].shape[1], inp["key_cache"].shape[2], inp["value_cache"].shape[3]
    g = torch.Generator().manual_seed(7)
    ups = {"d_attention": torch.randn(B, Hq, Q, M, generator=g).to(torch.bfloat16),
           "d_context": torch.randn(B, Hq, Q, Dv, generator=g).to(torch.bfloat16),
           "d_key_cache_out": torch.randn(B, Hk, M, D, generator=g).to(torch.bfloat16),
           "d_value_cache_out": None}
    dups = {k: None if v is None else v.to(DEV) for k, v in ups.items()}
    outs = {k: torch.full_like(dinp[src], float("nan")) for k, src in
            (("g_query", "query"), ("g_new_key", "new_key"), ("g_new_value", "new_value"),
             ("g_key_cache", "key_cache"), ("g_value_cache", "value_cache"))}
    if which == "query":
        dinp["query"] = misaligned(dinp["query"])
    elif which in dups:
        dups[which] = misaligned(dups[which])
    else:
        outs[which] = misaligned(outs[which])
    mask = dinp["append_mask"].contiguous().view(torch.uint8)
    kvc.kvc_step_backward(dinp["query"], dinp["new_key"], dinp["new_value"],
                          dinp["key_cache"], dinp["value_cache"], dinp["lengths"], mask,
                          *dups.values(), **outs, scale=wl.scale)
    torch.cuda.synchronize()
    h = host_arrays(inp)
    ref = oracle.step_backward(*(to_f64(inp[k]) for k in ("query", "new_key", "new_value",
                                                          "key_cache", "value_cache")),
                               h["lengths"], h["append_mask"],
                               **{k: None if v is None else to_f64(v) for k, v in ups.items()},
                               scale=wl.scale)
    for name, want in (("g_query", ref.query), ("g_new_key", ref.new_key),
                       ("g_new_value", ref.new_value), ("g_key_cache", ref.key_cache),
                       ("g_value_cache", ref.value_cache)):
        check_grad(to_f64(outs[name]), want, "bf16", f"misaligned {which} {name}")


@pytest.mark.parametrize("name", ["decode_gqa_bf16", "long_decode_share8_bf16"])
def test_backward_full_decode_bench_configuration(name):
    """The backward at full size with upstream gradients for all four
    outputs, every gradient element against the oracle: the decode workload
    bench.py --mode backward times (bf16, 32 sequences, 32 query heads over
    8 KV heads, 8192 slots: 4 packed rows; about half a minute of oracle
    time), and one GPU's share of the long decode (4 sequences, 64 query
    heads over 8 KV heads, 16384 slots: the 8-row vector waves)."""
    wl = WORKLOADS[name]
    say(f"[case] backward {wl.name} full size")
    inp = make_inputs(wl, 0, "cpu")
    dinp = {k: v.to(DEV) for k, v in inp.items()}
    g = torch.Generator().manual_seed(100)
    B, Hq, Q, D = inp["query"].shape
    Hk, M, Dv = inp["key_cache"].shape[1], inp["key_cache"].shape[2], inp["value_cache"].shape[3]
    tdt = torch.bfloat16
    ups = {"d_attention": torch.randn(B, Hq, Q, M, generator=g).to(tdt),
           "d_context": torch.randn(B, Hq, Q, Dv, generator=g).to(tdt),
           "d_key_cache_out": torch.randn(B, Hk, M, D, generator=g).to(tdt),
           "d_value_cache_out": torch.randn(B, Hk, M, Dv, generator=g).to(tdt)}
    outs = {k: torch.full_like(dinp[src], float("nan")) for k, src in
            (("g_query", "query"), ("g_new_key", "new_key"), ("g_new_value", "new_value"),
             ("g_key_cache", "key_cache"), ("g_value_cache", "value_cache"))}
    mask = dinp["append_mask"].contiguous().view(torch.uint8)
    kvc.kvc_step_backward(dinp["query"], dinp["new_key"], dinp["new_value"],
                          dinp["key_cache"], dinp["value_cache"], dinp["lengths"], mask,
                          *[v.to(DEV) for v in ups.values()], **outs, scale=wl.scale)
    torch.cuda.synchronize()
    got = {k: to_f64(v) for k, v in outs.items()}
    del dinp, outs
    torch.cuda.empty_cache()
    h = host_arrays(inp)
    ref = oracle.step_backward(*(to_f64(inp[k]) for k in ("query", "new_key", "new_value",
                                                          "key_cache", "value_cache")),
                               h["lengths"], h["append_mask"],
                               **{k: to_f64(v) for k, v in ups.items()}, scale=wl.scale)
    for out_name, want in (("g_query", ref.query), ("g_new_key", ref.new_key),
                           ("g_new_value", ref.new_value), ("g_key_cache", ref.key_cache),
                           ("g_value_cache", ref.value_cache)):
        check_grad(got[out_name], want, "bf16", f"full {wl.name} backward {out_name}")
