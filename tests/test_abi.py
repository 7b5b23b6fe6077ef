"""The C-ABI library loads, exports what include/kvc.h declares, and rejects
bad arguments on the host before enqueueing anything (no GPU needed: every
call below fails a host-side check)."""
import ctypes
import os
import re

import pytest

from autoregressive_kv_cache_amd import kvc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvc.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvc_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return kvc.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(kvc.EXPORTED), names
    for name in names:
        assert hasattr(lib, name), f"{name} not exported"


def test_status_strings(lib):
    for code in [0, -1, -2, -3, -4, -5, -6, -7, -8, -9, 1, 2, 3, 4]:
        s = kvc.kvc_status_string(code)
        assert s and s != "unknown code"
    assert kvc.kvc_status_string(12345) == "unknown code"


def dims(B=2, Hq=8, Hk=2, Q=3, M=64, D=16, Dv=8):
    return kvc.KvcDims(B, Hq, Hk, Q, M, D, Dv)


def test_workspace_and_plan(lib):
    d = dims()
    ws = kvc.kvc_workspace_bytes(d, kvc.KVC_F32)
    plan = kvc.kvc_plan_step(d, kvc.KVC_F32)
    assert ws == plan["workspace_bytes"] > 0
    assert plan["rows"] == 12
    assert plan["nsplit"] * plan["split"] >= 64
    assert plan["row_tiles"] * plan["rows_per_tile"] >= plan["rows"]
    assert kvc.kvc_workspace_bytes(dims(Hq=3, Hk=2), 0) == 0
    assert kvc.kvc_workspace_bytes(dims(B=0), 0) == 0
    assert kvc.kvc_workspace_bytes(d, 9) == 0
    big = dims(B=32, Hq=32, Hk=8, Q=1, M=8192, D=128, Dv=128)
    assert kvc.kvc_workspace_bytes(big, kvc.KVC_BF16) > 0
    with pytest.raises(kvc.KvcError):
        kvc.kvc_plan_step(dims(Q=-1), 0)


def test_plan_dispatch_rule(lib):
    """Host-only path choice.  The matrix-core chunk kernel (2) only where a
    KV head's packed rows R = (Hq/Hk) Q fill a 16-row tile (R >= 16, D = Dv
    in {64, 128, 256} bf16 or {64, 128} fp32).  Below that the vector decode
    kernels (1): 4 rows a wave up to R = 4, 8 up to 8, and for bf16 with
    D = Dv in {64, 128} two waves of up to 8 rows each up to R = 15
    (rows_per_tile 8, row_tiles 2); small heads (fp32 D = Dv in {8, 16},
    bf16 {16, 32}) up to R = 8 on the one-slot-per-lane kernel.  The rest
    -> the generic kernel (0).
    The workspace covers every path of the shape."""
    cases = [
        (dims(B=32, Hq=32, Hk=8, Q=1, M=8192, D=128, Dv=128), kvc.KVC_BF16, 1, 4, 1),
        (dims(B=4, Hq=64, Hk=8, Q=1, M=131072, D=128, Dv=128), kvc.KVC_BF16, 1, 8, 1),
        (dims(B=8, Hq=16, Hk=16, Q=4, M=1024, D=64, Dv=32), kvc.KVC_F32, 1, 4, 1),
        (dims(B=2, Hq=8, Hk=2, Q=40, M=4096, D=64, Dv=64), kvc.KVC_BF16, 2, None, None),
        (dims(B=2, Hq=8, Hk=2, Q=40, M=4096, D=64, Dv=64), kvc.KVC_F32, 2, None, None),
        (dims(B=2, Hq=8, Hk=2, Q=40, M=4096, D=256, Dv=256), kvc.KVC_F32, 0, None, None),
        (dims(B=2, Hq=4, Hk=1, Q=3, M=100, D=128, Dv=128), kvc.KVC_BF16, 1, 8, 2),   # R = 12
        (dims(B=2, Hq=12, Hk=1, Q=1, M=100, D=64, Dv=64), kvc.KVC_BF16, 1, 8, 2),    # R = 12
        (dims(B=2, Hq=5, Hk=1, Q=3, M=100, D=128, Dv=128), kvc.KVC_BF16, 1, 8, 2),   # R = 15
        (dims(B=2, Hq=9, Hk=1, Q=1, M=100, D=64, Dv=64), kvc.KVC_BF16, 1, 8, 2),     # R = 9
        (dims(B=2, Hq=4, Hk=1, Q=4, M=100, D=128, Dv=128), kvc.KVC_BF16, 2, None, None),  # R = 16
        (dims(B=2, Hq=4, Hk=1, Q=3, M=100, D=128, Dv=128), kvc.KVC_F32, 0, None, None),   # R = 12
        (dims(B=2, Hq=4, Hk=1, Q=3, M=100, D=256, Dv=256), kvc.KVC_BF16, 0, None, None),  # R = 12
        (dims(B=2, Hq=4, Hk=1, Q=3, M=100, D=96, Dv=96), kvc.KVC_BF16, 0, None, None),    # no entry
        # small heads (rows of at most 64 bytes): the one-slot-per-lane decode kernel
        (dims(B=2, Hq=4, Hk=2, Q=3, M=16, D=8, Dv=8), kvc.KVC_F32, 1, 8, 1),
        (dims(B=2, Hq=4, Hk=2, Q=1, M=16, D=8, Dv=8), kvc.KVC_F32, 1, 4, 1),
        (dims(B=2, Hq=8, Hk=2, Q=2, M=99, D=16, Dv=16), kvc.KVC_F32, 1, 8, 1),
        (dims(B=2, Hq=8, Hk=2, Q=1, M=99, D=32, Dv=32), kvc.KVC_BF16, 1, 4, 1),
        (dims(B=2, Hq=8, Hk=2, Q=1, M=99, D=8, Dv=16), kvc.KVC_F32, 0, None, None),
        (dims(B=2, Hq=4, Hk=1, Q=3, M=99, D=8, Dv=8), kvc.KVC_F32, 0, None, None),   # R = 12
    ]
    for d, dt, path, rows, tiles in cases:
        plan = kvc.kvc_plan_step(d, dt)
        assert plan["path"] == path, (d.Q, d.Hq, d.Hk, d.D, dt)
        if path == 1:
            assert (plan["rows_per_tile"], plan["row_tiles"]) == (rows, tiles), plan
        assert plan["nsplit"] * plan["split"] >= d.M
        assert plan["workspace_bytes"] == kvc.kvc_workspace_bytes(d, dt) > 0
        if path != 1:
            assert plan["workers"] == 0 and plan["lead"] == 0


def test_plan_stream_workers():
    """The bf16 stream decode: one workgroup of 4 worker waves per compute
    unit (256 assumed without a device), even shares, two waves per worker
    past 8 rows, and never more workers than the step can have chunks."""
    cases = [
        (dims(B=32, Hq=32, Hk=8, Q=1, M=8192, D=128, Dv=128), 1024),   # 4 rows
        (dims(B=4, Hq=64, Hk=8, Q=1, M=131072, D=128, Dv=128), 1024),  # 8 rows
        (dims(B=4, Hq=96, Hk=8, Q=1, M=8192, D=128, Dv=128), 512),     # 12 rows: row groups
        (dims(B=1, Hq=4, Hk=1, Q=1, M=64, D=64, Dv=64), 4),            # 2 chunks: one workgroup
    ]
    for d, workers in cases:
        plan = kvc.kvc_plan_step(d, kvc.KVC_BF16)
        assert plan["path"] == 1, plan
        assert plan["workers"] == workers, (plan, workers)
        assert plan["lead"] == 8, plan


FAKE = 1 << 40  # never dereferenced: each call below fails a host check first


def call_oop(lib, d, dtype=0, has_scale=0, scale=0.0, ptrs=None, ws_bytes=None):
    e = 4 if dtype == 0 else 2
    B, Hq, Hk, Q, M, D, Dv = d.B, d.Hq, d.Hk, d.Q, d.M, d.D, d.Dv
    sizes = [B * Hq * Q * D * e, B * Hk * Q * D * e, B * Hk * Q * Dv * e, B * Hk * M * D * e,
             B * Hk * M * Dv * e, B * 8, B * Q, B * Hk * M * D * e, B * Hk * M * Dv * e, B * 8,
             B * Hq * Q * M * e, B * Hq * Q * Dv * e, B * 4]
    if ptrs is None:
        ptrs, off = [], FAKE
        for s in sizes:
            ptrs.append(off)
            off += (s + 4095) // 4096 * 4096 + 4096
    ws = kvc.kvc_workspace_bytes(d, dtype) if ws_bytes is None else ws_bytes
    return lib.kvc_step_out_of_place(ctypes.byref(d), dtype, has_scale, scale, *ptrs,
                                     FAKE * 4, ws, None, None), ptrs


def test_host_checks_out_of_place(lib):
    d = dims()
    assert lib.kvc_step_out_of_place(None, 0, 0, 0.0, *([None] * 13), None, 0, None, None) == -1
    assert call_oop(lib, dims(Hq=6, Hk=4))[0] == -2
    assert call_oop(lib, dims(M=0))[0] == -2
    assert call_oop(lib, d, dtype=5)[0] == -3
    assert call_oop(lib, d, has_scale=1, scale=0.0)[0] == -4
    assert call_oop(lib, d, has_scale=1, scale=float("nan"))[0] == -4
    assert call_oop(lib, d, ws_bytes=16)[0] == -5
    _, ptrs = call_oop(lib, d, ws_bytes=16)
    bad = list(ptrs)
    bad[0] = None  # query NULL with Q > 0
    assert call_oop(lib, d, ptrs=bad)[0] == -1
    for out_i, in_i in [(7, 3), (8, 4), (10, 0), (11, 2), (9, 5), (10, 11), (12, 6)]:
        bad = list(ptrs)
        bad[out_i] = bad[in_i]  # an output on top of an input / another output
        assert call_oop(lib, d, ptrs=bad)[0] == -6, (out_i, in_i)


def test_host_checks_inplace(lib):
    d = dims()
    e = 4
    B, Hq, Hk, Q, M, D, Dv = d.B, d.Hq, d.Hk, d.Q, d.M, d.D, d.Dv
    sizes = [B * Hq * Q * D * e, B * Hk * Q * D * e, B * Hk * Q * Dv * e, B * Hk * M * D * e,
             B * Hk * M * Dv * e, B * 8, B * Q, B * 8, B * Hq * Q * M * e, B * Hq * Q * Dv * e,
             B * 4]
    ptrs, off = [], FAKE
    for s in sizes:
        ptrs.append(off)
        off += (s + 4095) // 4096 * 4096 + 4096

    def call(p, ws=16):
        return lib.kvc_step_inplace(ctypes.byref(d), 0, 0, 0.0, *p, FAKE * 4, ws, None, None)

    full = kvc.kvc_workspace_bytes(d, 0)
    assert call(ptrs) == -5  # workspace too small
    for out_i, in_i in [(8, 3), (9, 4), (8, 0), (7, 6), (10, 5)]:
        bad = list(ptrs)
        bad[out_i] = bad[in_i]
        assert call(bad, full) == -6, (out_i, in_i)
    bad = list(ptrs)
    bad[4] = bad[3]  # key and value cache on one buffer
    assert call(bad, full) == -6
    ok = list(ptrs)
    ok[7] = ok[5]  # lengths_out == lengths is allowed; the small workspace still fails
    assert call(ok) == -5


def test_page_face_rejects_cpu_and_options():
    import torch
    q = torch.zeros(1, 1, 1, 2)
    with pytest.raises(ValueError):
        kvc.kv_cache_attention_step(q, q, q, torch.zeros(1, 1, 4, 2), torch.zeros(1, 1, 4, 2),
                                    torch.zeros(1, dtype=torch.int64),
                                    torch.ones(1, 1, dtype=torch.bool), {})
    with pytest.raises(ValueError):
        kvc._options_scale({"scale": 1.0, "dropout": 0.1})
    with pytest.raises(ValueError):
        kvc._options_scale({"scale": -1.0})
    assert kvc._options_scale({}) is None and kvc._options_scale({"scale": 2}) == 2.0


def test_host_checks_paged(lib):
    """kvc_step_paged: block size, workspace and aliasing are checked on the
    host (every call here fails one of those checks; none reaches a launch)."""
    def run(d, block_size=64, num_blocks=64, ptrs=None, ws=1 << 30, dtype=kvc.KVC_BF16):
        e = 2 if dtype == kvc.KVC_BF16 else 4
        B, Hq, Hk, Q, M, D, Dv = d.B, d.Hq, d.Hk, d.Q, d.M, d.D, d.Dv
        mb = max(1, M // block_size)
        sizes = [B * Hq * Q * D * e, B * Hk * Q * D * e, B * Hk * Q * Dv * e,
                 num_blocks * Hk * block_size * D * e, num_blocks * Hk * block_size * Dv * e,
                 B * mb * 4, B * 8, B * Q, B * 8, B * Hq * Q * M * e, B * Hq * Q * Dv * e, B * 4]
        if ptrs is None:
            ptrs, off = [], FAKE
            for sz in sizes:
                ptrs.append(off)
                off += (sz + 4095) // 4096 * 4096 + 4096
        q, nk, nv, kp, vp, tab, ln, mk, lo, at, cx, st = ptrs
        return lib.kvc_step_paged(ctypes.byref(d), dtype, 0, 0.0, q, nk, nv, kp, vp, num_blocks,
                                  block_size, tab, ln, mk, lo, at, cx, st, FAKE * 4, ws, None,
                                  None), ptrs

    d = dims(B=4, Hq=8, Hk=2, Q=1, M=1024, D=128, Dv=128)  # 4 packed rows: the decode path
    assert run(d, block_size=48)[0] == -2       # not a power of two
    assert run(d, block_size=2048)[0] == -2     # does not divide M
    assert run(d, num_blocks=0)[0] == -2
    # blocks smaller than a chunk, and shapes without a decode or chunk
    # kernel, take the generic kernel (the calls then fail the workspace
    # check, before a launch)
    assert run(d, block_size=32, ws=16)[0] == -5
    assert run(d, block_size=1, ws=16)[0] == -5
    assert run(dims(B=4, Hq=8, Hk=2, Q=4, M=1024, D=128, Dv=128), block_size=32, ws=16)[0] == -5
    assert run(dims(B=4, Hq=8, Hk=2, Q=1, M=1024, D=96, Dv=96), ws=16)[0] == -5
    _, ptrs = run(d, ws=16)
    assert run(d, ws=16)[0] == -5
    bad = list(ptrs)
    bad[5] = None  # no block table
    assert run(d, ptrs=bad)[0] == -1
    for out_i, in_i in [(9, 5), (9, 3), (10, 4), (11, 5)]:
        bad = list(ptrs)
        bad[out_i] = bad[in_i]  # attention on the table / pool, row_status on the table
        assert run(d, ptrs=bad)[0] == -6, (out_i, in_i)
    bad = list(ptrs)
    bad[4] = bad[3]  # both pools on one buffer
    assert run(d, ptrs=bad)[0] == -6


def test_host_checks_backward(lib):
    """kvc_step_backward: head sizes beyond the generic kernels' limit
    (D + Dv > 6144), buffers not aligned to their element, and a short
    workspace are refused on the host; any other head size is taken (the
    calls here then fail the workspace check, before a launch)."""
    def run(d, dtype=kvc.KVC_F32, shift=None, ws=16):
        e = 2 if dtype == kvc.KVC_BF16 else 4
        B, Hq, Hk, Q, M, D, Dv = d.B, d.Hq, d.Hk, d.Q, d.M, d.D, d.Dv
        sizes = [B * Hq * Q * D * e, B * Hk * Q * D * e, B * Hk * Q * Dv * e,
                 B * Hk * M * D * e, B * Hk * M * Dv * e, B * 8, B * Q,
                 B * Hq * Q * M * e, B * Hq * Q * Dv * e, B * Hk * M * D * e,
                 B * Hk * M * Dv * e, B * Hq * Q * D * e, B * Hk * Q * D * e,
                 B * Hk * Q * Dv * e, B * Hk * M * D * e, B * Hk * M * Dv * e, ws]
        ptrs, off = [], FAKE
        for sz in sizes:
            ptrs.append(off)
            off += (sz + 4095) // 4096 * 4096 + 4096
        if shift is not None:
            ptrs[shift] += 1
        return lib.kvc_step_backward(ctypes.byref(d), dtype, 0, 0.0, *ptrs, ws, None)

    assert run(dims(D=4096, Dv=2049)) == -8          # D + Dv above 6144
    assert run(dims(D=4096, Dv=2048)) == -5          # at the limit: taken
    for D, Dv in [(8, 8), (96, 80), (256, 256), (1, 3)]:
        assert run(dims(D=D, Dv=Dv)) == -5, (D, Dv)  # no tile: the generic kernels
        assert run(dims(D=D, Dv=Dv), dtype=kvc.KVC_BF16) == -5, (D, Dv)
    for i in (0, 3, 7, 9, 14):  # query, key cache, d_attention, d_key_cache_out, g_key_cache
        assert run(dims(D=64, Dv=64), shift=i) == -8, i
    assert run(dims(D=64, Dv=64), dtype=kvc.KVC_BF16, shift=3) == -8
    assert lib.kvc_backward_workspace_bytes(ctypes.byref(dims(D=96, Dv=80)), kvc.KVC_F32) > 16


def test_host_checks_attend_over_cache(lib):
    """kvc_attend_over_cache: layout, workspace and aliasing are checked on
    the host before anything is enqueued (every call here fails one)."""
    def run(d, Tq=4, num_blocks=8, block_size=None, table=False, slots=False, ptrs=None,
            ws=1 << 34, sink=True, kcount=None):
        e = 2
        B, Hq, Hk, Q, M, D, Dv = d.B, d.Hq, d.Hk, d.Q, d.M, d.D, d.Dv
        bs = M if block_size is None else block_size
        sizes = [Tq * Hq * D * e, (B + 1) * 8, num_blocks * Hk * bs * D * e,
                 num_blocks * Hk * bs * Dv * e, B * max(1, M // bs) * 4, B * 4, B * 8, Hq * 4,
                 Tq * Hq * Dv * e, B * 4]
        if ptrs is None:
            ptrs, off = [], FAKE
            for sz in sizes:
                ptrs.append(off)
                off += (sz + 4095) // 4096 * 4096 + 4096
        qp, cu, kc, vc, tb, sl, lk, sk, out, st = ptrs
        return lib.kvc_attend_over_cache(ctypes.byref(d), kvc.KVC_BF16, 0, 0.0, qp, Tq, cu, kc, vc,
                                         num_blocks, bs, tb if table else None,
                                         sl if slots else None, lk,
                                         d.B if kcount is None else kcount,
                                         sk if sink else None, out, st,
                                         FAKE * 4, ws, None, None), ptrs

    d = dims(B=4, Hq=8, Hk=2, Q=1, M=1024, D=128, Dv=128)
    assert kvc.kvc_attend_workspace_bytes(d, kvc.KVC_BF16) > kvc.kvc_workspace_bytes(d, 1)
    assert run(d, table=True, slots=True, block_size=64)[0] == -2   # two layouts at once
    assert run(d, block_size=64)[0] == -2                           # continuous: block = M
    assert run(d, num_blocks=3)[0] == -2                            # row b needs B rows
    assert run(d, Tq=-1)[0] == -2
    assert run(d, table=True, block_size=48)[0] == -2
    # blocks smaller than a chunk, and shapes of the generic kernel, are taken
    # (the calls then fail the workspace check, before a launch)
    assert run(d, table=True, block_size=32, ws=16)[0] == -5
    assert run(d, table=True, block_size=1, ws=16)[0] == -5
    assert run(dims(B=4, Hq=8, Hk=2, Q=4, M=1024, D=96, Dv=96), slots=True, ws=16)[0] == -5
    assert run(d, ws=16)[0] == -5
    assert run(d, ws=16, kcount=d.B + 1)[0] == -5                   # cumulative form accepted
    for kc in (0, d.B - 1, d.B + 2):                                # [B] or [B + 1] only
        assert run(d, kcount=kc)[0] == -2, kc
    _, ptrs = run(d, ws=16)
    bad = list(ptrs)
    bad[1] = None
    assert run(d, ptrs=bad)[0] == -1
    for out_i, in_i in [(8, 0), (8, 2), (9, 6), (8, 7)]:
        bad = list(ptrs)
        bad[out_i] = bad[in_i]
        assert run(d, ptrs=bad)[0] == -6, (out_i, in_i)


def test_bound_calls_marshal_like_the_plain_calls(lib):
    """A bound step (arguments marshalled once) reaches the same host checks
    as the plain call: with a 16-byte workspace both fail the workspace check
    (KVC_ERR_WORKSPACE) before anything is enqueued, on every call."""
    import torch
    B, Hq, Hk, Q, M, D = 2, 4, 2, 1, 64, 16
    t = {"query": torch.zeros(B, Hq, Q, D), "new_key": torch.zeros(B, Hk, Q, D),
         "new_value": torch.zeros(B, Hk, Q, D), "key_cache": torch.zeros(B, Hk, M, D),
         "value_cache": torch.zeros(B, Hk, M, D), "lengths": torch.zeros(B, dtype=torch.int64),
         "append_mask": torch.ones(B, Q, dtype=torch.uint8)}
    outs = {"lengths_out": torch.zeros(B, dtype=torch.int64),
            "attention": torch.zeros(B, Hq, Q, M), "context": torch.zeros(B, Hq, Q, D)}
    ws = torch.empty(16, dtype=torch.uint8)
    bound = kvc.bind_step_inplace(*t.values(), *outs.values(), workspace=ws, stream=0)
    for _ in range(2):
        with pytest.raises(kvc.KvcError) as e:
            bound()
        assert e.value.code == -5
    with pytest.raises(kvc.KvcError) as e:
        kvc.kvc_step_inplace(*t.values(), *outs.values(), workspace=ws, stream=0)
    assert e.value.code == -5
    kc_out, vc_out = torch.zeros(B, Hk, M, D), torch.zeros(B, Hk, M, D)
    bound = kvc.bind_step_out_of_place(*t.values(), kc_out, vc_out, *outs.values(), workspace=ws,
                                       stream=0)
    with pytest.raises(kvc.KvcError) as e:
        bound()
    assert e.value.code == -5
    pool = torch.zeros(4, Hk, 32, D)
    table = torch.zeros(B, 2, dtype=torch.int32)
    bound = kvc.bind_step_paged(t["query"], t["new_key"], t["new_value"], pool, pool.clone(),
                                table, t["lengths"], t["append_mask"], *outs.values(),
                                workspace=ws, stream=0)
    with pytest.raises(kvc.KvcError) as e:
        bound()
    assert e.value.code == -5


def test_binding_argument_counts_match_the_header(lib):
    """Every ctypes declaration of the binding has as many arguments as the
    C prototype in include/kvc.h (a short list would let ctypes pass the
    trailing ones, such as the stream handle, with the wrong width)."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    protos = dict(re.findall(r"\b(kvc_[a-z_]+)\s*\(([^;{]*?)\)\s*;", text))
    assert set(protos) == set(kvc.EXPORTED)
    for name, params in protos.items():
        count = 0 if params.strip() in ("", "void") else params.count(",") + 1
        assert len(getattr(lib, name).argtypes) == count, (name, count)


def test_noalloc_refuses_steps_beyond_its_scratch(lib):
    """A step whose workspace exceeds the static scratch is refused before
    anything is enqueued (the pointers are never touched); a bad shape is a
    shape error."""
    big = kvc.KvcDims(64, 64, 8, 1, 131072, 128, 128)
    assert kvc.kvc_workspace_bytes(big, kvc.KVC_BF16) > lib.kvc_noalloc_scratch_bytes()
    fake = [16] * 11
    rc = lib.kvc_step_inplace_noalloc(ctypes.byref(big), kvc.KVC_BF16, 0, 0.0, *fake, None, None)
    assert rc == -9, rc
    rc = lib.kvc_step_inplace_noalloc(ctypes.byref(dims(B=0)), kvc.KVC_BF16, 0, 0.0, *fake, None,
                                      None)
    assert rc == -2, rc
    assert lib.kvc_noalloc_scratch_bytes() == 96 << 20
