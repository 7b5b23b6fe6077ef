"""CPU oracle for the KV-cache append + causal GQA attention step.

TEST INFRASTRUCTURE ONLY.  Imported by ``tests/``, by ``__graft_entry__.smoke``
and by the ``cpu_baseline`` leg of ``bench.py``; the product package never
imports it and the GPU library never links it.

The arithmetic lives in ``kvc_oracle.c`` (plain C, double precision); this
module only builds that file with gcc and marshals numpy arrays through
ctypes.  bfloat16 arrays travel as their raw ``uint16`` words.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "kvc_oracle.c")
LIBRARY = os.path.join(HERE, "libkvc_oracle.so")

F32, BF16 = 0, 1
ROW_OK, ROW_BAD_LENGTH, ROW_OVERFLOW, ROW_NOT_PREFIX, ROW_BAD_QUERIES = 0, 1, 2, 3, 4

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle with gcc (IEEE double, no contraction, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", "-I", os.path.dirname(os.path.abspath(source)),
           source, "-o", output + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(output + ".tmp", output)
    return output


def _ptr(a: np.ndarray | None) -> int | None:
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle takes float32 or bfloat16-as-uint16 arrays, got {a.dtype}")


@dataclass
class StepResult:
    key_cache: np.ndarray
    value_cache: np.ndarray
    lengths: np.ndarray
    attention: np.ndarray  # float64 [B, Hq, Q, M]
    context: np.ndarray  # float64 [B, Hq, Q, Dv]
    row_status: np.ndarray  # int32 [B]


class Oracle:
    """ctypes face of ``libkvc_oracle.so`` (or of any library built from a
    variant of ``kvc_oracle.c``, which the mutation tests use)."""

    def __init__(self, path: str = LIBRARY):
        if not os.path.exists(path):
            build(output=path)
        self.path = path
        lib = ctypes.CDLL(path)
        lib.kvc_oracle_append.restype = ctypes.c_int
        lib.kvc_oracle_append.argtypes = [_i64] * 7 + [ctypes.c_int] + [_vp] * 11
        lib.kvc_oracle_attend_row.restype = ctypes.c_int
        lib.kvc_oracle_attend_row.argtypes = ([_i64] * 7 + [ctypes.c_int, ctypes.c_int,
                                              ctypes.c_double] + [_vp] * 3 + [_i64] * 5
                                             + [_vp] * 2)
        lib.kvc_oracle_reattend.restype = ctypes.c_int
        lib.kvc_oracle_reattend.argtypes = ([_i64] * 7 + [ctypes.c_int, ctypes.c_int,
                                            ctypes.c_double, _i64] + [_vp] * 8)
        lib.kvc_oracle_step.restype = ctypes.c_int
        lib.kvc_oracle_step.argtypes = ([_i64] * 7 + [ctypes.c_int, ctypes.c_int,
                                        ctypes.c_double] + [_vp] * 13)
        self.lib = lib

    # -- helpers -----------------------------------------------------------
    @staticmethod
    def _dims(query, new_key, new_value, key_cache, value_cache):
        B, Hq, Q, D = query.shape
        Hk, M = key_cache.shape[1], key_cache.shape[2]
        Dv = value_cache.shape[3]
        return B, Hq, Hk, Q, M, D, Dv

    def step(self, query, new_key, new_value, key_cache, value_cache, lengths,
             append_mask, scale: float | None = None) -> StepResult:
        """The full step over numpy inputs; returns fresh output arrays."""
        args = [np.ascontiguousarray(a) for a in (query, new_key, new_value, key_cache,
                                                   value_cache)]
        query, new_key, new_value, key_cache, value_cache = args
        lengths = np.ascontiguousarray(lengths, dtype=np.int64)
        append_mask = np.ascontiguousarray(append_mask, dtype=np.uint8)
        dt = _dtype_code(query)
        for a in args:
            if _dtype_code(a) != dt:
                raise TypeError("all float inputs must share one dtype")
        B, Hq, Hk, Q, M, D, Dv = self._dims(*args)
        kc_out = np.empty_like(key_cache)
        vc_out = np.empty_like(value_cache)
        len_out = np.empty(B, dtype=np.int64)
        attn = np.empty((B, Hq, Q, M), dtype=np.float64)
        ctx = np.empty((B, Hq, Q, Dv), dtype=np.float64)
        status = np.empty(B, dtype=np.int32)
        rc = self.lib.kvc_oracle_step(
            B, Hq, Hk, Q, M, D, Dv, dt, 0 if scale is None else 1,
            0.0 if scale is None else float(scale), _ptr(query), _ptr(new_key),
            _ptr(new_value), _ptr(key_cache), _ptr(value_cache), _ptr(lengths),
            _ptr(append_mask), _ptr(kc_out), _ptr(vc_out), _ptr(len_out), _ptr(attn),
            _ptr(ctx), _ptr(status))
        if rc != 0:
            raise ValueError(f"oracle rejected the step (code {rc})")
        return StepResult(kc_out, vc_out, len_out, attn, ctx, status)

    def append(self, new_key, new_value, key_cache, value_cache, lengths, append_mask,
               Hq: int | None = None):
        """Append only: returns (key_cache_out, value_cache_out, lengths_out, n, status)."""
        new_key, new_value, key_cache, value_cache = [
            np.ascontiguousarray(a) for a in (new_key, new_value, key_cache, value_cache)]
        lengths = np.ascontiguousarray(lengths, dtype=np.int64)
        append_mask = np.ascontiguousarray(append_mask, dtype=np.uint8)
        dt = _dtype_code(key_cache)
        B, Hk, M, D = key_cache.shape
        Dv = value_cache.shape[3]
        Q = append_mask.shape[1]
        Hq = Hk if Hq is None else Hq
        kc_out = np.empty_like(key_cache)
        vc_out = np.empty_like(value_cache)
        len_out = np.empty(B, dtype=np.int64)
        n = np.empty(B, dtype=np.int64)
        status = np.empty(B, dtype=np.int32)
        rc = self.lib.kvc_oracle_append(
            B, Hq, Hk, Q, M, D, Dv, dt, _ptr(new_key), _ptr(new_value), _ptr(key_cache),
            _ptr(value_cache), _ptr(lengths), _ptr(append_mask), _ptr(kc_out),
            _ptr(vc_out), _ptr(len_out), _ptr(n), _ptr(status))
        if rc != 0:
            raise ValueError(f"oracle rejected the append (code {rc})")
        return kc_out, vc_out, len_out, n, status

    def step_threaded(self, query, new_key, new_value, key_cache, value_cache, lengths,
                      append_mask, scale: float | None = None,
                      threads: int | None = None) -> StepResult:
        """step() with its rows spread over a thread pool: one append, then the
        (b, hq, t) rows of kvc_oracle_attend_row (the calls kvc_oracle_step
        makes, in any order) on `threads` threads; ctypes releases the GIL
        during each call.  The arithmetic is that of step(), row for row."""
        from concurrent.futures import ThreadPoolExecutor
        args = [np.ascontiguousarray(a) for a in (query, new_key, new_value, key_cache,
                                                   value_cache)]
        query, new_key, new_value, key_cache, value_cache = args
        lengths = np.ascontiguousarray(lengths, dtype=np.int64)
        B, Hq, Hk, Q, M, D, Dv = self._dims(*args)
        kc, vc, len_out, n, status = self.append(new_key, new_value, key_cache, value_cache,
                                                 lengths, append_mask, Hq=Hq)
        attn = np.empty((B, Hq, Q, M), dtype=np.float64)
        ctx = np.empty((B, Hq, Q, Dv), dtype=np.float64)
        dt = _dtype_code(query)
        has, sc = (0, 0.0) if scale is None else (1, float(scale))
        qp, kp, vp = _ptr(query), _ptr(kc), _ptr(vc)
        a0, c0 = attn.ctypes.data, ctx.ctypes.data
        rows = [(b, hq, t) for b in range(B) for hq in range(Hq) for t in range(Q)]

        def run(chunk):
            for b, hq, t in chunk:
                row = (b * Hq + hq) * Q + t
                rc = self.lib.kvc_oracle_attend_row(
                    B, Hq, Hk, Q, M, D, Dv, dt, has, sc, qp, kp, vp, int(lengths[b]),
                    int(n[b]), b, hq, t, a0 + row * M * 8, c0 + row * Dv * 8)
                if rc != 0:
                    raise ValueError(f"oracle rejected the row (code {rc})")

        threads = max(1, threads or os.cpu_count() or 1)
        parts = [rows[i::threads] for i in range(threads)]
        with ThreadPoolExecutor(max_workers=threads) as ex:
            for f in [ex.submit(run, part) for part in parts if part]:
                f.result()
        return StepResult(kc, vc, len_out, attn, ctx, status)

    def attend_row(self, query, key_updated, value_updated, old_len: int, n: int, b: int,
                   hq: int, t: int, scale: float | None = None):
        """One (b, hq, t) row over an updated cache: returns (attention[M], context[Dv])."""
        query = np.ascontiguousarray(query)
        key_updated = np.ascontiguousarray(key_updated)
        value_updated = np.ascontiguousarray(value_updated)
        dt = _dtype_code(query)
        B, Hq, Q, D = query.shape
        Hk, M = key_updated.shape[1], key_updated.shape[2]
        Dv = value_updated.shape[3]
        attn = np.empty(M, dtype=np.float64)
        ctx = np.empty(Dv, dtype=np.float64)
        rc = self.lib.kvc_oracle_attend_row(
            B, Hq, Hk, Q, M, D, Dv, dt, 0 if scale is None else 1,
            0.0 if scale is None else float(scale), _ptr(query), _ptr(key_updated),
            _ptr(value_updated), int(old_len), int(n), int(b), int(hq), int(t),
            _ptr(attn), _ptr(ctx))
        if rc != 0:
            raise ValueError(f"oracle rejected the row (code {rc})")
        return attn, ctx

    def raw_step_code(self, B, Hq, Hk, Q, M, D, Dv, dtype=F32, has_scale=0, scale=0.0) -> int:
        """Return code of a step call with NULL buffers (argument checks only)."""
        return self.lib.kvc_oracle_step(B, Hq, Hk, Q, M, D, Dv, dtype, has_scale, scale,
                                        *([None] * 13))


@dataclass
class PagedStepResult:
    key_pool: np.ndarray
    value_pool: np.ndarray
    lengths: np.ndarray
    attention: np.ndarray  # float64 [B, Hq, Q, M]
    context: np.ndarray  # float64 [B, Hq, Q, Dv]
    row_status: np.ndarray  # int32 [B]


def paged_to_dense(pool: np.ndarray, block_table: np.ndarray) -> np.ndarray:
    """The dense cache [B, H, M, D] a block pool [num_blocks, H, block_size, D]
    and a table [B, max_blocks] describe: slot j of row b is row j % block_size
    of block block_table[b, j // block_size] (the block-pool layout of ClikaRT's
    attention_over_cache).  Entries outside the pool (allowed only for slots a
    step never reads) gather block 0."""
    nb, H, bs, D = pool.shape
    B, max_blocks = block_table.shape
    j = np.arange(max_blocks * bs)
    blk = np.clip(block_table[:, j // bs], 0, nb - 1)  # [B, M]
    dense = pool[blk, :, (j % bs)[None, :], :]  # [B, M, H, D]
    return np.ascontiguousarray(dense.transpose(0, 2, 1, 3))


def _oracle_step_paged(oracle: "Oracle", query, new_key, new_value, key_pool, value_pool,
                       block_table, lengths, append_mask, scale=None) -> PagedStepResult:
    """The step over a paged cache, read as the step over the dense cache the
    table describes: gather that cache, run the dense step, and write back
    exactly the slots the step wrote (slot length + t of each accepted row);
    every other pool row keeps its bits."""
    block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    lengths = np.ascontiguousarray(lengths, dtype=np.int64)
    nb, Hk, bs, _ = key_pool.shape
    kc = paged_to_dense(key_pool, block_table)
    vc = paged_to_dense(value_pool, block_table)
    res = oracle.step(query, new_key, new_value, kc, vc, lengths, append_mask, scale=scale)
    kp, vp = key_pool.copy(), value_pool.copy()
    for b in range(block_table.shape[0]):
        if res.row_status[b] != 0:
            continue
        for j in range(int(lengths[b]), int(res.lengths[b])):
            blk = int(block_table[b, j // bs])
            if not 0 <= blk < nb:
                raise ValueError(f"row {b}: slot {j} maps to block {blk} outside the pool")
            kp[blk, :, j % bs] = res.key_cache[b, :, j]
            vp[blk, :, j % bs] = res.value_cache[b, :, j]
    return PagedStepResult(kp, vp, res.lengths, res.attention, res.context, res.row_status)


Oracle.step_paged = _oracle_step_paged


def _oracle_reattend(oracle: "Oracle", q, cu_seqlens_q, key, value, seqlens_k, Q: int,
                     sink=None, scale=None):
    """Read-only re-attention over the logical caches key [B, Hk, M, D] /
    value [B, Hk, M, Dv] (sequence b's cache; paged or row-mapped caches are
    gathered into this form first).  seqlens_k holds each sequence's total
    cached length, per sequence ([B]) or cumulative ([B + 1], the length
    being the difference of neighbours): "ClikaRT::ops::attention_over_cache",
    function description, on cu_seqlens_k.  Returns (out [Tq, Hq, Dv]
    float64, status [B] int32)."""
    q = np.ascontiguousarray(q)
    key = np.ascontiguousarray(key)
    value = np.ascontiguousarray(value)
    cu = np.ascontiguousarray(cu_seqlens_q, dtype=np.int64)
    lk = np.ascontiguousarray(seqlens_k, dtype=np.int64)
    dt = _dtype_code(q)
    Tq, Hq, D = q.shape
    B, Hk, M, _ = key.shape
    if lk.shape == (B + 1,):
        lk = np.ascontiguousarray(lk[1:] - lk[:-1])
    elif lk.shape != (B,):
        raise ValueError(f"seqlens_k has {lk.shape[0]} entries; {B} or {B + 1} expected")
    Dv = value.shape[3]
    sk = None if sink is None else np.ascontiguousarray(sink, dtype=np.float64)
    out = np.empty((Tq, Hq, Dv), dtype=np.float64)
    status = np.empty(B, dtype=np.int32)
    rc = oracle.lib.kvc_oracle_reattend(
        B, Hq, Hk, int(Q), M, D, Dv, dt, 0 if scale is None else 1,
        0.0 if scale is None else float(scale), Tq, _ptr(q), _ptr(cu), _ptr(key), _ptr(value),
        _ptr(lk), _ptr(sk), _ptr(out), _ptr(status))
    if rc != 0:
        raise ValueError(f"oracle rejected the re-attention (code {rc})")
    return out, status


Oracle.reattend = _oracle_reattend

_DEFAULT: Oracle | None = None


def default() -> Oracle:
    """The oracle built from ``kvc_oracle.c`` (built on first use)."""
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle(LIBRARY)
    return _DEFAULT


@dataclass
class StepGrads:
    query: np.ndarray        # [B, Hq, Q, D]
    new_key: np.ndarray      # [B, Hk, Q, D]
    new_value: np.ndarray    # [B, Hk, Q, Dv]
    key_cache: np.ndarray    # [B, Hk, M, D]
    value_cache: np.ndarray  # [B, Hk, M, Dv]


def step_backward(query, new_key, new_value, key_cache, value_cache, lengths, append_mask,
                  d_attention=None, d_context=None, d_key_cache_out=None,
                  d_value_cache_out=None, scale=None) -> StepGrads:
    """Gradients of the step (all in float64, from the definition) given the
    gradients of its outputs: attention, context and the two returned caches
    (each may be None = zero).  The step: the updated caches K', V' are the
    inputs with slots length + t (t < n) replaced by the new rows; valid
    query t (t < n) has scores s_j = scale q.K'_j on j <= length + t,
    P = softmax(s), attention = P, context = P V'.  Backward, per valid row:
    dP_j = dA_j + dO . V'_j, dS_j = P_j (dP_j - sum_k P_k dP_k),
    dq = scale sum_j dS_j K'_j, dK'_j += scale dS_j q, dV'_j += P_j dO;
    then dK' splits into the cache slots that were kept and the new rows
    that were written (an overwritten cache slot gets no gradient).  Rows
    outside the contract are no-ops: only the returned caches pass their
    gradients through."""
    f = lambda a: None if a is None else np.asarray(a, dtype=np.float64)
    q, nk, nv, kc, vc = (np.asarray(a, dtype=np.float64)
                         for a in (query, new_key, new_value, key_cache, value_cache))
    B, Hq, Q, D = q.shape
    Hk, M, Dv = kc.shape[1], kc.shape[2], vc.shape[3]
    G = Hq // Hk
    sc = 1.0 / np.sqrt(D) if scale is None else float(scale)
    dA, dO = f(d_attention), f(d_context)
    dKo, dVo = f(d_key_cache_out), f(d_value_cache_out)
    lengths = np.asarray(lengths, dtype=np.int64)
    mask = np.asarray(append_mask).astype(bool)
    gq = np.zeros_like(q)
    gnk, gnv = np.zeros_like(nk), np.zeros_like(nv)
    dKp = np.zeros_like(kc) if dKo is None else dKo.copy()  # gradient of K' (updated cache)
    dVp = np.zeros_like(vc) if dVo is None else dVo.copy()
    for b in range(B):
        L = int(lengths[b])
        n = 0
        while n < Q and mask[b, n]:
            n += 1
        ok = 0 <= L <= M and not mask[b, n:].any() and L + n <= M
        if not ok:
            continue  # the step leaves this row alone
        Kp, Vp = kc[b].copy(), vc[b].copy()
        Kp[:, L:L + n] = nk[b, :, :n]
        Vp[:, L:L + n] = nv[b, :, :n]
        for h in range(Hq):
            kh = h // G
            for t in range(n):
                vis = L + t + 1
                s = sc * (Kp[kh, :vis] @ q[b, h, t])
                p = np.exp(s - s.max())
                p /= p.sum()
                dP = np.zeros(vis)
                if dA is not None:
                    dP += dA[b, h, t, :vis]
                if dO is not None:
                    dP += Vp[kh, :vis] @ dO[b, h, t]
                dS = p * (dP - p @ dP)
                gq[b, h, t] = sc * (dS @ Kp[kh, :vis])
                dKp[b, kh, :vis] += sc * np.outer(dS, q[b, h, t])
                if dO is not None:
                    dVp[b, kh, :vis] += np.outer(p, dO[b, h, t])
        # K' = cache with slots L .. L+n-1 replaced
        gnk[b, :, :n] = dKp[b, :, L:L + n]
        gnv[b, :, :n] = dVp[b, :, L:L + n]
        dKp[b, :, L:L + n] = 0.0
        dVp[b, :, L:L + n] = 0.0
    return StepGrads(gq, gnk, gnv, dKp, dVp)
