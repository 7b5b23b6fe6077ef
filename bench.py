"""Benchmark of the KV-cache append + causal GQA attention step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--mode inplace|oop]

A step is one call of the library's step entry point (kvc_step_inplace by
default) over one batch of seeded synthetic inputs already resident in HBM:
append the new K/V rows, attend every valid query row over its visible
slots, write attention[B,Hq,Q,M] and context[B,Hq,Q,Dv].  The default
workload is single-token GQA decode, bf16, B=32, Hq=32, Hk=8, M=8192,
D=Dv=128, cache lengths uniform in [1024, 8191], tails filled with 1e4.

Prints one JSON line: steps/s (value), ms/step, the step's algorithmic HBM
GB/s and its fraction of the 8 TB/s peak, the attention kernel's roofline
(algorithmic bytes per launch / its average launch time, from HIP events
recorded around that kernel on its stream), the HBM traffic counted by
rocprofv3 for that kernel when a profile of the current kernel source is
committed under profiles/, and the CPU oracle's rate on the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode steps/s + achieved HBM GB/s (% of MI355X peak), GQA Hq32/Hk8 D128 M8192"
PEAK_HBM_GBPS = 8000.0
DOMINANT_KERNEL = "attend"
ENTRY = {"inplace": "kvc_step_inplace", "oop": "kvc_step_out_of_place", "paged": "kvc_step_paged",
         "reattend": "kvc_attend_over_cache", "backward": "kvc_step_backward"}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="decode_gqa_bf16")
    p.add_argument("--mode", choices=["inplace", "oop", "paged", "reattend", "backward"],
                   default="inplace")
    p.add_argument("--block-size", type=int, default=64,
                   help="paged mode: slots per cache block (the pools are block-permuted)")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--copies", type=int, default=4,
                   help="independent input sets the steps rotate over (each step reads data "
                        "the previous steps did not, as the layers of a model would)")
    # events on every step cost ~7 us of stream time per step; every 5th step
    # (coprime with the 4 input copies, so every copy is sampled) costs <1 us
    p.add_argument("--event-every", type=int, default=5,
                   help="record the attend kernel's HIP events on every k-th timed step")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="CPU oracle time budget for the baseline sample")
    return p.parse_args()


class HipEvents:
    """hipEvent_t handles through the HIP runtime torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self) -> int:
        e = ctypes.c_void_p()
        assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def elapsed_ms(self, a: int, b: int) -> float:
        assert self.hip.hipEventSynchronize(ctypes.c_void_p(b)) == 0
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a),
                                            ctypes.c_void_p(b)) == 0
        return float(ms.value)

    def record(self, e: int, stream: int = 0):
        """Record event e on the current (default) stream."""
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        assert self.hip.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream)) == 0

    def destroy(self, e: int):
        self.hip.hipEventDestroy(ctypes.c_void_p(e))


def algorithmic_bytes(wl, lengths, n):
    """What the step must move (per step), and the attention kernel's share.

    Step: read the visible prefix of K and V (length + n rows per KV head,
    the n new rows read from new_key/new_value), write the n new rows into
    the cache, read q, write the full attention rows and the context, plus
    lengths, mask, lengths_out and row_status.

    Attention kernel: the K/V rows it visits (length + n per KV head), q,
    and lengths and mask.  What it writes for the combine kernel (exp values,
    their references, segment partials) is intermediate traffic, not
    algorithmic (see intermediate_bytes); the append itself, the attention
    rows, the normalisation and the context belong to the combine."""
    e = 2 if wl.dtype == "bf16" else 4
    kv = sum(wl.Hk * (int(L) + 2 * int(k)) * (wl.D + wl.Dv) * e for L, k in zip(lengths, n))
    kv_read = sum(wl.Hk * (int(L) + int(k)) * (wl.D + wl.Dv) * e for L, k in zip(lengths, n))
    q = wl.B * wl.Hq * wl.Q * wl.D * e
    att = wl.B * wl.Hq * wl.Q * wl.M * e
    ctx = wl.B * wl.Hq * wl.Q * wl.Dv * e
    small_in = wl.B * (8 + wl.Q)
    small_out = wl.B * (8 + 4)
    step = kv + q + att + ctx + small_in + small_out
    attend = kv_read + q + small_in
    return step, attend, kv


def worker_start(w: int, Nc: int, Pe: int, lead: int) -> int:
    """First chunk of stream worker w, as the kernels split the chunk list:
    even shares for lead 8, else the first half of the workers weigh
    lead / 8 (applied only when Nc >= 2 Pe)."""
    if lead <= 8 or Pe < 2 or Nc < 2 * Pe:
        return w * Nc // Pe
    H = Pe // 2
    S = lead * min(w, H) + 8 * max(w - H, 0)
    return S * Nc // (lead * H + 8 * (Pe - H))


def intermediate_bytes(wl, lengths, n, P: int, C: int = 64, seg_partials: bool = True,
                       lead: int = 8):
    """Bytes the stream attend kernel writes for the combine kernel (bf16
    decode path): per chunk of the flattened list, R rows of C exp values
    (2 B) and R references (4 B); per segment (a worker's run of one KV
    head), R rows of Dv fp32 context partials and (m, l) as two floats.
    Workers own contiguous ranges of the chunk list, split as the kernel
    splits it (worker_start)."""
    R = wl.Hq // wl.Hk * wl.Q
    heads = []  # flattened chunk list: one entry per chunk, its (b, head)
    for b, (L, k) in enumerate(zip(lengths, n)):
        if int(k) == 0:
            continue
        nc = -(-int(L) // C) + 1
        for h in range(wl.Hk):
            heads.extend([(b, h)] * nc)
    Nc = len(heads)
    if Nc == 0:
        return 0
    Pe = min(P, Nc)
    segs = 0
    for w in range(Pe):
        x0, x1 = worker_start(w, Nc, Pe, lead), worker_start(w + 1, Nc, Pe, lead)
        segs += len(set(heads[x0:x1]))
    per_chunk = R * C * 2 + R * 4
    per_seg = R * (wl.Dv * 4 + 8) if seg_partials else 0
    return Nc * per_chunk + segs * per_seg


def reattend_bytes(wl, lengths, n):
    """Read-only re-attention of the last n_b of length_b + n_b cached
    positions: read the visible K/V prefix and q, write the packed output,
    plus the small per-sequence inputs.  Returns (whole call, attention
    kernel share: the K/V rows and q)."""
    e = 2 if wl.dtype == "bf16" else 4
    kv = sum(wl.Hk * (int(L) + int(k)) * (wl.D + wl.Dv) * e for L, k in zip(lengths, n))
    tq = int(sum(int(k) for k in n))
    q = tq * wl.Hq * wl.D * e
    out = tq * wl.Hq * wl.Dv * e
    small = wl.B * (8 + 8 + 4)
    return kv + q + out + small, kv + q


def backward_bytes(wl, lengths, n):
    """Backward of the step: read q, the visible K'/V' rows, the gradients of
    the attention (visible entries), the context and the returned caches;
    write the gradients of q, the new rows and the whole caches.  Returns
    (whole call, the slot-gradient kernel's share: visible K'/V' rows, the
    caches' gradients read and written, q and the context gradient)."""
    e = 2 if wl.dtype == "bf16" else 4
    vis = sum(wl.Hk * (int(L) + int(k)) * (wl.D + wl.Dv) * e for L, k in zip(lengths, n))
    full = wl.B * wl.Hk * wl.M * (wl.D + wl.Dv) * e
    q = wl.B * wl.Hq * wl.Q * wl.D * e
    dctx = wl.B * wl.Hq * wl.Q * wl.Dv * e
    datt = sum(wl.Hq * (int(L) + t + 1) * e for L, k in zip(lengths, n) for t in range(int(k)))
    new = wl.B * wl.Hk * wl.Q * (wl.D + wl.Dv) * e
    step = vis + 2 * full + 2 * q + dctx + datt + new
    return step, vis + 2 * full + q + dctx + new


def oop_extra_bytes(wl, lengths, n):
    """Out of place the whole cache is also returned: per KV head the M - len
    - n slots past the new rows are read and written once and the len cached
    rows are written once more (their read is already counted).  Returns the
    step's extra bytes and the attention kernel's (it writes the rows it
    visits; the rest is copied by the kernels around it)."""
    e = 2 if wl.dtype == "bf16" else 4
    row = (wl.D + wl.Dv) * e
    step = sum(wl.Hk * (2 * wl.M - int(L) - int(k)) * row for L, k in zip(lengths, n))
    attend = sum(wl.Hk * int(L) * row for L in lengths)
    return step, attend


# Sources the attend kernel is compiled from and launched by (the stream
# decode kernels, their row preparation, the host plan and launch code): a change
# to any of them makes a committed counter summary stale.
ATTEND_SOURCES = ("kvc_api.hip", "kvc_common.h", "kvc_decode.h", "kvc_host.h", "kvc_prep.h",
                  "kvc_stream.h")


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "autoregressive_kv_cache_amd", "csrc")
    for f in ATTEND_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def committed_traffic(workload: str, mode: str, digest: str):
    """HBM bytes per attention-kernel dispatch from a committed rocprofv3
    counter summary, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"attend_{workload}_{mode}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_b = re.search(r"traffic_bytes_per_dispatch:\s*([0-9.eE+]+)", text)
    if not m_src or not m_b or m_src.group(1) != digest:
        return None
    return float(m_b.group(1))


def copy_ceiling_gbps(torch, dev, nbytes=2 << 30, reps=10):
    """Device-to-device copy rate (read + write bytes / time) on a 2 GiB buffer."""
    a = torch.empty(nbytes // 2, dtype=torch.int16, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        b.copy_(a)
    e.record()
    e.synchronize()
    ms = s.elapsed_time(e) / reps
    del a, b
    torch.cuda.empty_cache()
    return 2 * nbytes / (ms * 1e-3) / 1e9


def read_ceiling_gbps(torch, kvc, dev, nbytes=2 << 30, reps=10):
    """Streaming read of a 2 GiB buffer with the attend kernels' non-temporal
    16-byte loads (kvc_read_ceiling): bytes / time, the achievable read rate
    next to the 8 TB/s peak."""
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    wgs = cus * 8
    buf = torch.empty(nbytes // 2, dtype=torch.int16, device=dev)
    buf.fill_(3)
    sink = torch.empty(kvc.load().kvc_read_ceiling_sink_bytes(wgs) // 4, dtype=torch.int32,
                       device=dev)
    for _ in range(2):
        kvc.kvc_read_ceiling(buf, wgs, sink)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        kvc.kvc_read_ceiling(buf, wgs, sink)
    e.record()
    e.synchronize()
    ms = s.elapsed_time(e) / reps
    del buf, sink
    torch.cuda.empty_cache()
    return nbytes / (ms * 1e-3) / 1e9


def cpu_baseline(wl, inputs, budget_s: float):
    """The oracle on the same workload, whole steps repeated until each half
    of the time budget is used (at least once): on one thread (step) and on
    every host core (step_threaded: the same row calls over a thread pool)."""
    import oracle
    from autoregressive_kv_cache_amd.workloads import host_arrays
    h = host_arrays(inputs)
    orc = oracle.default()
    args = (h["query"], h["new_key"], h["new_value"], h["key_cache"], h["value_cache"],
            h["lengths"], h["append_mask"])

    def rate(fn):
        reps, t0 = 0, time.perf_counter()
        while True:
            fn()
            reps += 1
            if time.perf_counter() - t0 >= budget_s / 2:
                break
        return reps, time.perf_counter() - t0

    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    threads = max(1, threads or 1)
    r1, t1 = rate(lambda: orc.step(*args, scale=wl.scale))
    rn, tn = rate(lambda: orc.step_threaded(*args, scale=wl.scale, threads=threads))
    return {"value": rn / tn, "unit": "steps/s", "cores": threads, "kind": "oracle",
            "single_thread_value": r1 / t1,
            "sample": f"whole {wl.name} steps of the oracle (double precision) on the same "
                      f"seeded inputs: {rn} in {tn:.1f} s on {threads} threads (rows over a "
                      f"thread pool), {r1} in {t1:.1f} s on one thread"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: this step has no multi-GPU path here "
              "(sharding across GPUs is a design note, not an implementation)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from autoregressive_kv_cache_amd import kvc
    from autoregressive_kv_cache_amd.workloads import (WORKLOADS, draw_lengths_and_counts,
                                                       make_inputs, paged_layout)
    kvc.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = WORKLOADS[args.workload]
    lengths, n = draw_lengths_and_counts(wl, args.seed)
    # `copies` independent input sets with the same lengths and masks (one
    # per "layer"), so that a step never re-reads the previous step's K/V
    # from the 256 MB last-level cache
    sets = []
    for k in range(max(1, args.copies)):
        inp = make_inputs(wl, args.seed + 1000 * k, dev, lengths=lengths, n=n)
        d = {key: inp[key] for key in ("query", "new_key", "new_value", "key_cache",
                                        "value_cache", "lengths")}
        d["mask"] = inp["append_mask"].contiguous().view(torch.uint8)
        d["att"] = torch.empty(wl.B, wl.Hq, wl.Q, wl.M, dtype=inp["key_cache"].dtype, device=dev)
        d["ctx"] = torch.empty(wl.B, wl.Hq, wl.Q, wl.Dv, dtype=inp["key_cache"].dtype, device=dev)
        d["lens_out"] = torch.empty_like(inp["lengths"])
        d["status"] = torch.empty(wl.B, dtype=torch.int32, device=dev)
        if args.mode == "oop":
            d["kc_out"] = torch.empty_like(inp["key_cache"])
            d["vc_out"] = torch.empty_like(inp["value_cache"])
        if args.mode == "backward":
            gen = torch.Generator(device=dev)
            gen.manual_seed(7 + k)
            fdt = inp["key_cache"].dtype
            for name, like in (("d_attention", "att"), ("d_context", "ctx")):
                d[name] = torch.randn(d[like].shape, generator=gen, device=dev).to(fdt)
            d["d_kc"] = torch.randn(inp["key_cache"].shape, generator=gen, device=dev).to(fdt)
            d["d_vc"] = torch.randn(inp["value_cache"].shape, generator=gen, device=dev).to(fdt)
            for name, like in (("g_q", "query"), ("g_nk", "new_key"), ("g_nv", "new_value"),
                               ("g_kc", "key_cache"), ("g_vc", "value_cache")):
                d[name] = torch.empty_like(inp[like])
        if args.mode == "reattend":
            # the cache already holds length + n rows; re-attend the last n
            cnt = torch.from_numpy(np.asarray(n, dtype=np.int64))
            d["cu"] = torch.cat([torch.zeros(1, dtype=torch.int64), cnt.cumsum(0)]).to(dev)
            d["lk"] = (inp["lengths"].cpu() + cnt).to(dev)
            rows = [inp["query"][b, :, :int(n[b])].transpose(0, 1) for b in range(wl.B)]
            d["qp"] = torch.cat(rows).contiguous()
            d["out"] = torch.empty(d["qp"].shape[0], wl.Hq, wl.Dv, dtype=inp["key_cache"].dtype,
                                   device=dev)
        if args.mode == "paged":
            d["kp"], d["vp"], d["table"] = paged_layout(inp["key_cache"], inp["value_cache"],
                                                        args.block_size, args.seed + k)
            if k > 0:  # only the first set's dense caches are kept (for the plan)
                del d["key_cache"], d["value_cache"], inp
        sets.append(d)
        if k == 0:
            first_inputs = inp
    q0, kc0, vc0 = sets[0]["query"], sets[0]["key_cache"], sets[0]["value_cache"]
    dims = kvc.dims_of(q0, kc0, vc0)
    dt = kvc.dtype_code(kc0.dtype)
    plan = kvc.kvc_plan_step(dims, dt)
    if args.mode == "reattend":
        ws = torch.empty(kvc.kvc_attend_workspace_bytes(dims, dt), dtype=torch.uint8, device=dev)
    elif args.mode == "backward":
        ws = torch.empty(int(kvc.load().kvc_backward_workspace_bytes(ctypes.byref(dims), dt)),
                         dtype=torch.uint8, device=dev)
    else:
        ws = kvc.workspace_for(dims, dt, dev)

    ev = HipEvents()
    starts = [ev.create() for _ in range(args.steps)]
    stops = [ev.create() for _ in range(args.steps)]

    # the step entry points with their arguments marshalled once per input
    # copy (as a serving loop would bind its buffers), so a timed step is one
    # foreign call
    bound = []
    for d in sets:
        if args.mode == "paged":
            bound.append(kvc.bind_step_paged(d["query"], d["new_key"], d["new_value"], d["kp"],
                                             d["vp"], d["table"], d["lengths"], d["mask"],
                                             d["lens_out"], d["att"], d["ctx"], d["status"],
                                             workspace=ws, scale=wl.scale))
        elif args.mode == "inplace":
            bound.append(kvc.bind_step_inplace(d["query"], d["new_key"], d["new_value"],
                                               d["key_cache"], d["value_cache"], d["lengths"],
                                               d["mask"], d["lens_out"], d["att"], d["ctx"],
                                               d["status"], workspace=ws, scale=wl.scale))
        elif args.mode == "oop":
            bound.append(kvc.bind_step_out_of_place(d["query"], d["new_key"], d["new_value"],
                                                    d["key_cache"], d["value_cache"],
                                                    d["lengths"], d["mask"], d["kc_out"],
                                                    d["vc_out"], d["lens_out"], d["att"],
                                                    d["ctx"], d["status"], workspace=ws,
                                                    scale=wl.scale))

    def step(i=None, k=0):
        d = sets[k % len(sets)]
        events = None if i is None or i % args.event_every else (starts[i], stops[i])
        if bound:
            bound[k % len(sets)](events)
            return
        if args.mode == "backward":
            if events:
                ev.record(events[0])
            kvc.kvc_step_backward(d["query"], d["new_key"], d["new_value"], d["key_cache"],
                                  d["value_cache"], d["lengths"], d["mask"], d["d_attention"],
                                  d["d_context"], d["d_kc"], d["d_vc"], d["g_q"], d["g_nk"],
                                  d["g_nv"], d["g_kc"], d["g_vc"], workspace=ws, scale=wl.scale)
            if events:
                ev.record(events[1])
        else:  # reattend
            kvc.kvc_attend_over_cache(d["qp"], d["cu"], d["key_cache"], d["value_cache"], d["lk"],
                                      d["out"], wl.Q, row_status=d["status"], workspace=ws,
                                      scale=wl.scale, events=events)

    ceiling = copy_ceiling_gbps(torch, dev)
    read_ceiling = read_ceiling_gbps(torch, kvc, dev)
    for w in range(args.warmup):
        step(None, w)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kernel_ms = [ev.elapsed_ms(a, b) for i, (a, b) in enumerate(zip(starts, stops))
                 if i % args.event_every == 0]
    for e in starts + stops:
        ev.destroy(e)

    step_bytes, attend_bytes, kv_bytes = algorithmic_bytes(wl, lengths, n)
    inter_bytes = None
    if args.mode in ("inplace", "oop", "paged") and plan["path"] == 1 and wl.dtype == "bf16":
        # the workers and their shares as the library's plan states them
        inter_bytes = intermediate_bytes(wl, lengths, n, int(plan["workers"]),
                                         lead=int(plan["lead"]))
    if args.mode == "oop":
        extra_step, extra_attend = oop_extra_bytes(wl, lengths, n)
        step_bytes += extra_step
        attend_bytes += extra_attend
    if args.mode == "reattend":
        step_bytes, attend_bytes = reattend_bytes(wl, lengths, n)
    if args.mode == "backward":
        step_bytes, attend_bytes = backward_bytes(wl, lengths, n)
    ms_per_step = elapsed / args.steps * 1e3
    steps_per_s = args.steps / elapsed
    step_gbps = step_bytes / (ms_per_step * 1e-3) / 1e9
    k_ms = sum(kernel_ms) / len(kernel_ms)
    k_sorted = sorted(kernel_ms)

    def pct(q):  # nearest-rank percentile of the sampled launch durations
        return k_sorted[min(len(k_sorted) - 1, max(0, int(round(q * (len(k_sorted) - 1)))))]
    k_gbps = attend_bytes / (k_ms * 1e-3) / 1e9
    digest = kernel_source_digest()
    traffic = committed_traffic(wl.name, args.mode, digest)
    result = {
        "metric": METRIC,
        "value": steps_per_s,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "entry": ENTRY[args.mode],
                   "B": wl.B, "Hq": wl.Hq, "Hk": wl.Hk, "Q": wl.Q, "M": wl.M, "D": wl.D,
                   "Dv": wl.Dv, "seed": args.seed, "input_copies": len(sets), "plan": plan},
        "achieved_gbps": step_gbps,
        "pct_of_peak_hbm": 100.0 * step_gbps / PEAK_HBM_GBPS,
        "tokens_per_s": steps_per_s * wl.B * wl.Q,
        "step_algorithmic_bytes": step_bytes,
        "copy_ceiling_gbps": ceiling,
        "read_ceiling_gbps": read_ceiling,
        "roofline": {"bound": "hbm",
                     "kernel": "backward (every kernel of the step)" if args.mode == "backward"
                     else DOMINANT_KERNEL, "achieved": k_gbps,
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": k_gbps / PEAK_HBM_GBPS,
                     "traffic": traffic, "bytes_per_launch": attend_bytes,
                     "intermediate_bytes_per_launch": inter_bytes,
                     "avg_launch_ms": k_ms, "launches_sampled": len(kernel_ms),
                     "p10_launch_ms": pct(0.1), "median_launch_ms": pct(0.5),
                     "p90_launch_ms": pct(0.9),
                     "frac_of_copy_ceiling": k_gbps / ceiling,
                     "frac_of_read_ceiling": k_gbps / read_ceiling},
    }
    if args.mode == "paged":
        result["config"]["block_size"] = args.block_size
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, first_inputs, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
