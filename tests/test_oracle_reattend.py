"""The oracle's read-only re-attention (ClikaRT attention_over_cache) against
its pins (no GPU): the step it equals without a sink, closed forms with a
sink, a numpy brute force, and the rejected-row conventions."""
import numpy as np
import pytest

import oracle


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.Oracle()


def draw(rng, B, Hq, Hk, M, D, Dv, S, L):
    cu = np.concatenate([[0], np.cumsum(S)]).astype(np.int64)
    q = rng.standard_normal((int(cu[-1]), Hq, D)).astype(np.float32)
    k = rng.standard_normal((B, Hk, M, D)).astype(np.float32)
    v = rng.standard_normal((B, Hk, M, Dv)).astype(np.float32)
    return q, cu, k, v, np.asarray(L, np.int64)


def test_without_sink_it_is_the_step(orc):
    """Re-attending the last S cached positions equals the step that appended
    them: old length L - S, the rows [L - S, L) as new rows, S valid queries."""
    rng = np.random.default_rng(0)
    B, Hq, Hk, M, D, Dv, Q = 3, 4, 2, 12, 8, 6, 3
    S, L = [1, 3, 2], [5, 12, 2]
    q, cu, k, v, lk = draw(rng, B, Hq, Hk, M, D, Dv, S, L)
    out, st = orc.reattend(q, cu, k, v, lk, Q)
    assert list(st) == [0, 0, 0]
    qs = np.zeros((B, Hq, Q, D), np.float32)
    nk = np.zeros((B, Hk, Q, D), np.float32)
    nv = np.zeros((B, Hk, Q, Dv), np.float32)
    mask = np.zeros((B, Q), np.uint8)
    for b in range(B):
        for t in range(S[b]):
            qs[b, :, t] = q[cu[b] + t]
            nk[b, :, t] = k[b, :, L[b] - S[b] + t]
            nv[b, :, t] = v[b, :, L[b] - S[b] + t]
            mask[b, t] = 1
    ref = orc.step(qs, nk, nv, k, v, lk - np.asarray(S), mask)
    for b in range(B):
        for t in range(S[b]):
            np.testing.assert_allclose(out[cu[b] + t], ref.context[b, :, t], rtol=1e-13,
                                       atol=1e-13)


def test_sink_closed_forms(orc):
    rng = np.random.default_rng(1)
    # one cached key: p = e^s / (e^s + e^sink), out = p v
    q, cu, k, v, lk = draw(rng, 1, 2, 1, 4, 4, 3, [1], [1])
    sink = np.array([0.7, -1.3])
    out, _ = orc.reattend(q, cu, k, v, lk, 1, sink=sink, scale=0.5)
    for h in range(2):
        s = 0.5 * float(q[0, h].astype(np.float64) @ k[0, 0, 0].astype(np.float64))
        p = np.exp(s) / (np.exp(s) + np.exp(sink[h]))
        np.testing.assert_allclose(out[0, h], p * v[0, 0, 0], rtol=1e-13, atol=1e-15)
    # identical keys: every visible slot has the same score s, so
    # out = (sum of the visible values) / (count + e^(sink - s))
    q, cu, k, v, lk = draw(rng, 1, 1, 1, 6, 4, 3, [2], [5])
    k[:] = k[0, 0, 0]
    sink = np.array([2.0])
    out, _ = orc.reattend(q, cu, k, v, lk, 2, sink=sink)
    for t in range(2):
        pos = 5 - 2 + t
        s = float(q[t, 0].astype(np.float64) @ k[0, 0, 0].astype(np.float64)) / 2.0
        want = v[0, 0, :pos + 1].astype(np.float64).sum(0) / (pos + 1 + np.exp(sink[0] - s))
        np.testing.assert_allclose(out[t, 0], want, rtol=1e-12)
    # a sink at -inf is no sink
    q, cu, k, v, lk = draw(rng, 2, 2, 1, 6, 4, 4, [1, 2], [3, 6])
    a, _ = orc.reattend(q, cu, k, v, lk, 2, sink=np.array([-np.inf, -np.inf]))
    b, _ = orc.reattend(q, cu, k, v, lk, 2)
    np.testing.assert_array_equal(a, b)


def test_brute_force(orc):
    """Plain numpy, a different order of the same sums, with GQA and sinks."""
    rng = np.random.default_rng(2)
    B, Hq, Hk, M, D, Dv, Q = 2, 6, 2, 9, 5, 4, 3
    S, L = [3, 2], [7, 2]
    q, cu, k, v, lk = draw(rng, B, Hq, Hk, M, D, Dv, S, L)
    sink = rng.standard_normal(Hq)
    out, _ = orc.reattend(q, cu, k, v, lk, Q, sink=sink, scale=0.3)
    G = Hq // Hk
    for b in range(B):
        for t in range(S[b]):
            pos = L[b] - S[b] + t
            for h in range(Hq):
                kk = k[b, h // G, :pos + 1].astype(np.float64)
                s = 0.3 * (kk @ q[cu[b] + t, h].astype(np.float64))
                w = np.exp(np.append(s, sink[h]) - max(s.max(), sink[h]))
                p = w[:-1] / w.sum()
                np.testing.assert_allclose(out[cu[b] + t, h],
                                           p @ v[b, h // G, :pos + 1].astype(np.float64),
                                           rtol=1e-12, atol=1e-14)


def test_rejected_rows(orc):
    rng = np.random.default_rng(3)
    q, cu, k, v, _ = draw(rng, 3, 2, 1, 4, 4, 4, [1, 3, 1], [0, 0, 0])
    lk = np.array([5, 2, 1], np.int64)  # L > M; S > L; fine
    out, st = orc.reattend(q, cu, k, v, lk, 3)
    assert list(st) == [oracle.ROW_BAD_LENGTH, oracle.ROW_BAD_QUERIES, oracle.ROW_OK]
    assert not out[:4].any() and out[4].any()
    _, st = orc.reattend(q, cu, k, v, np.array([1, 3, 1]), 2)  # S = 3 > Q = 2
    assert st[1] == oracle.ROW_BAD_QUERIES


def test_cumulative_lengths_form(orc):
    """cu_seqlens_k in its cumulative form ([B + 1] offsets, any start):
    sequence b's length is the difference of neighbours, so the outputs and
    codes are those of the per-sequence form; offsets that go down give a
    negative length, which is a bad length; any other count is refused."""
    rng = np.random.default_rng(7)
    B, Hq, Hk, M, D, Dv, Q = 4, 4, 2, 10, 8, 8, 2
    S, L = [1, 2, 0, 2], [3, 10, 4, 2]
    q, cu, k, v, lk = draw(rng, B, Hq, Hk, M, D, Dv, S, L)
    want, wst = orc.reattend(q, cu, k, v, lk, Q)
    cum = 17 + np.concatenate([[0], np.cumsum(lk)]).astype(np.int64)
    got, gst = orc.reattend(q, cu, k, v, cum, Q)
    assert np.array_equal(got, want) and np.array_equal(gst, wst)
    down = cum.copy()
    down[2] = down[1] - 1  # sequence 1 gets length -1, sequence 2 a longer one
    _, st = orc.reattend(q, cu, k, v, down, Q)
    assert st[1] == 1 and st[0] == wst[0] and st[3] == wst[3]
    with pytest.raises(ValueError):
        orc.reattend(q, cu, k, v, cum[:-2], Q)
