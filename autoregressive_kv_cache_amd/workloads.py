"""Seeded synthetic inputs for the KV-cache step.

This module draws inputs and nothing else: it holds none of the step's
arithmetic, so both the GPU library's tests/benchmark and the CPU oracle can
take their inputs from it.

Shapes follow the function contract of "Autoregressive KV-cache append and
causal attention" (biotorch problem kv_cache_attention_step, Starter code):

    query [B,Hq,Q,D]  new_key [B,Hk,Q,D]  new_value [B,Hk,Q,Dv]
    key_cache [B,Hk,M,D]  value_cache [B,Hk,M,Dv]  lengths [B] int64
    append_mask [B,Q] bool (a prefix of Trues per row)

The five named workloads are the ones the library is measured and checked
on; the value distributions, length mixes and mask structure are stated with
each.  No public dataset is involved: every value is drawn from a seeded
generator.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hk: int
    Q: int
    M: int
    D: int
    Dv: int
    dtype: str  # "f32" or "bf16"
    std: float = 1.0  # entries ~ N(0, std^2)
    scale: float | None = None  # None = the default 1/sqrt(D)
    len_range: tuple[int, int] = (0, 0)  # inclusive integer range
    n_rule: str = "all"  # "all" | "uniform" | "choice"
    n_choices: tuple[int, ...] = ()
    force_len0_row: int | None = None  # this row gets length 0
    force_n0_row: int | None = None  # this row gets n = 0
    tail_sentinel: float | None = None  # fill cache slots >= length with this
    notes: str = field(default="", compare=False)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS: dict[str, Workload] = {
    # Tiny mixed step: ragged lengths, one empty cache row, one row with n=0.
    "tiny_mixed_f32": Workload(
        "tiny_mixed_f32", B=2, Hq=4, Hk=2, Q=3, M=16, D=8, Dv=8, dtype="f32",
        len_range=(0, 13), n_rule="uniform", force_len0_row=0, force_n0_row=1),
    # Single-token GQA decode (Llama-style 32/8 heads, head size 128), bf16;
    # unused tail slots hold 1e4 so that any read past a length shows up.
    "decode_gqa_bf16": Workload(
        "decode_gqa_bf16", B=32, Hq=32, Hk=8, Q=1, M=8192, D=128, Dv=128,
        dtype="bf16", len_range=(1024, 8191), n_rule="all", tail_sentinel=1e4),
    # Multi-token chunk append to a filled cache (chunks of 40/32/24 tokens).
    "chunk_gqa_bf16": Workload(
        "chunk_gqa_bf16", B=2, Hq=8, Hk=2, Q=40, M=4096, D=64, Dv=64,
        dtype="bf16", len_range=(512, 2048), n_rule="choice", n_choices=(40, 32, 24)),
    "chunk_gqa_f32": Workload(
        "chunk_gqa_f32", B=2, Hq=8, Hk=2, Q=40, M=4096, D=64, Dv=64,
        dtype="f32", len_range=(512, 2048), n_rule="choice", n_choices=(40, 32, 24)),
    # MHA stress: entries 8*N(0,1) and scale 4 so that scores pass 1000.
    "mha_stress_f32": Workload(
        "mha_stress_f32", B=8, Hq=16, Hk=16, Q=4, M=1024, D=64, Dv=32, dtype="f32",
        std=8.0, scale=4.0, len_range=(0, 1020), n_rule="uniform"),
    # Long-context GQA decode, 131072 slots per sequence.
    "long_decode_bf16": Workload(
        "long_decode_bf16", B=4, Hq=64, Hk=8, Q=1, M=131072, D=128, Dv=128,
        dtype="bf16", len_range=(65536, 131071), n_rule="all"),
    # One GPU's share of long_decode_bf16 when its slot axis is split over 8
    # GPUs (each holding a contiguous 16384-slot range of every sequence):
    # the same heads, an eighth of the capacity and of the lengths.
    "long_decode_share8_bf16": Workload(
        "long_decode_share8_bf16", B=4, Hq=64, Hk=8, Q=1, M=16384, D=128, Dv=128,
        dtype="bf16", len_range=(8192, 16383), n_rule="all"),
}


def draw_lengths_and_counts(wl: Workload, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """Old lengths and prefix counts n, drawn on the CPU (same on any device)."""
    rng = np.random.Generator(np.random.Philox(seed))
    lo, hi = wl.len_range
    lengths = rng.integers(lo, hi + 1, size=wl.B, dtype=np.int64)
    if wl.force_len0_row is not None and wl.force_len0_row < wl.B:
        lengths[wl.force_len0_row] = 0
    lengths = np.minimum(lengths, wl.M)
    n = np.zeros(wl.B, dtype=np.int64)
    for b in range(wl.B):
        room = int(min(wl.Q, wl.M - lengths[b]))
        if wl.n_rule == "all":
            n[b] = room
        elif wl.n_rule == "uniform":
            n[b] = rng.integers(0, room + 1)
        elif wl.n_rule == "choice":
            n[b] = min(room, int(rng.choice(np.asarray(wl.n_choices))))
        else:
            raise ValueError(wl.n_rule)
    if wl.force_n0_row is not None and wl.force_n0_row < wl.B:
        n[wl.force_n0_row] = 0
    return lengths, n


def prefix_mask(n: np.ndarray, Q: int) -> np.ndarray:
    """Row b is n[b] Trues followed by Falses."""
    return np.arange(Q)[None, :] < np.asarray(n)[:, None]


def make_inputs(wl: Workload, seed: int = 0, device: str | torch.device = "cpu",
                lengths: np.ndarray | None = None, n: np.ndarray | None = None
                ) -> dict[str, torch.Tensor]:
    """Draw one step's inputs.  Float tensors come from a torch generator on
    ``device`` (so large caches can be drawn straight into device memory);
    lengths and counts come from a CPU generator."""
    if lengths is None or n is None:
        l0, n0 = draw_lengths_and_counts(wl, seed)
        lengths = l0 if lengths is None else np.asarray(lengths, dtype=np.int64)
        n = n0 if n is None else np.asarray(n, dtype=np.int64)
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)

    def draw(*shape):
        x = torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)
        if wl.std != 1.0:
            x.mul_(wl.std)
        return x.to(wl.torch_dtype)

    B, Hq, Hk, Q, M, D, Dv = wl.B, wl.Hq, wl.Hk, wl.Q, wl.M, wl.D, wl.Dv
    out = {
        "query": draw(B, Hq, Q, D),
        "new_key": draw(B, Hk, Q, D),
        "new_value": draw(B, Hk, Q, Dv),
        "key_cache": draw(B, Hk, M, D),
        "value_cache": draw(B, Hk, M, Dv),
    }
    if wl.tail_sentinel is not None:
        for b in range(B):
            out["key_cache"][b, :, int(lengths[b]):, :] = wl.tail_sentinel
            out["value_cache"][b, :, int(lengths[b]):, :] = wl.tail_sentinel
    out["lengths"] = torch.as_tensor(lengths, dtype=torch.int64).to(device)
    out["append_mask"] = torch.as_tensor(prefix_mask(n, Q)).to(device)
    return out


def host_arrays(inputs: dict[str, torch.Tensor]) -> dict[str, np.ndarray]:
    """Host numpy copies in the layout the oracle reads: float32 stays float32,
    bfloat16 travels as its raw uint16 words, the mask as uint8."""
    out = {}
    for k, v in inputs.items():
        v = v.detach().to("cpu").contiguous()
        if v.dtype == torch.bfloat16:
            out[k] = v.view(torch.int16).numpy().view(np.uint16)
        elif v.dtype == torch.bool:
            out[k] = v.numpy().astype(np.uint8)
        else:
            out[k] = v.numpy()
    return out


def bf16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    """Widen raw bfloat16 words to float64 (exact)."""
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def paged_layout(key_cache: torch.Tensor, value_cache: torch.Tensor, block_size: int,
                 seed: int, spare_blocks: int = 3, fill: float = 7.0
                 ) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """The same caches in the block-pool layout: pools [num_blocks, Hk,
    block_size, D|Dv] and an int32 table [B, M / block_size] that sends row b's
    i-th block to a seeded random pool block.  ``spare_blocks`` extra pool
    blocks belong to no row and hold ``fill`` (so a stray write shows)."""
    B, Hk, M, D = key_cache.shape
    Dv = value_cache.shape[3]
    if M % block_size:
        raise ValueError("block_size must divide M")
    mb = M // block_size
    nb = B * mb + spare_blocks
    perm = np.random.default_rng(seed).permutation(nb)[:B * mb]
    idx = torch.from_numpy(perm.astype(np.int64)).to(key_cache.device)
    kp = torch.full((nb, Hk, block_size, D), fill, dtype=key_cache.dtype, device=key_cache.device)
    vp = torch.full((nb, Hk, block_size, Dv), fill, dtype=value_cache.dtype,
                    device=value_cache.device)
    kp[idx] = key_cache.reshape(B, Hk, mb, block_size, D).permute(0, 2, 1, 3, 4).reshape(
        B * mb, Hk, block_size, D)
    vp[idx] = value_cache.reshape(B, Hk, mb, block_size, Dv).permute(0, 2, 1, 3, 4).reshape(
        B * mb, Hk, block_size, Dv)
    table = torch.from_numpy(perm.reshape(B, mb).astype(np.int32)).to(key_cache.device)
    return kp.contiguous(), vp.contiguous(), table.contiguous()
