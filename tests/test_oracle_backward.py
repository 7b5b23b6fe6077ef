"""The oracle's backward of the step against central finite differences of
the forward oracle (a different implementation: the C forward in double),
plus the structural facts the step fixes (no gradient into overwritten
cache slots, pass-through for rejected rows, rows past n see nothing)."""
import numpy as np
import pytest

import oracle

H = 2.0 ** -10  # inputs are multiples of 2^-8, so x +- H is exact in float32


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.Oracle()


def grid(rng, shape, lim=2.0):
    return (np.round(rng.uniform(-lim, lim, shape) * 256) / 256).astype(np.float32)


def make(rng, B, Hq, Hk, Q, M, D, Dv, lengths, n):
    inp = dict(query=grid(rng, (B, Hq, Q, D)), new_key=grid(rng, (B, Hk, Q, D)),
               new_value=grid(rng, (B, Hk, Q, Dv)), key_cache=grid(rng, (B, Hk, M, D)),
               value_cache=grid(rng, (B, Hk, M, Dv)))
    mask = np.zeros((B, Q), np.uint8)
    for b in range(B):
        mask[b, :n[b]] = 1
    ups = dict(d_attention=rng.standard_normal((B, Hq, Q, M)),
               d_context=rng.standard_normal((B, Hq, Q, Dv)),
               d_key_cache_out=rng.standard_normal((B, Hk, M, D)),
               d_value_cache_out=rng.standard_normal((B, Hk, M, Dv)))
    return inp, np.asarray(lengths, np.int64), mask, ups


def loss(orc, inp, lengths, mask, ups, scale):
    r = orc.step(inp["query"], inp["new_key"], inp["new_value"], inp["key_cache"],
                 inp["value_cache"], lengths, mask, scale=scale)
    return (np.sum(ups["d_attention"] * r.attention) + np.sum(ups["d_context"] * r.context)
            + np.sum(ups["d_key_cache_out"] * r.key_cache.astype(np.float64))
            + np.sum(ups["d_value_cache_out"] * r.value_cache.astype(np.float64)))


@pytest.mark.parametrize("scale", [None, 0.7])
def test_gradients_match_finite_differences(orc, scale):
    rng = np.random.default_rng(0 if scale is None else 1)
    B, Hq, Hk, Q, M, D, Dv = 2, 4, 2, 2, 6, 3, 2
    inp, lengths, mask, ups = make(rng, B, Hq, Hk, Q, M, D, Dv, [2, 3], [2, 1])
    g = oracle.step_backward(**inp, lengths=lengths, append_mask=mask, scale=scale, **ups)
    grads = {"query": g.query, "new_key": g.new_key, "new_value": g.new_value,
             "key_cache": g.key_cache, "value_cache": g.value_cache}
    for name, x in inp.items():
        for idx in np.ndindex(x.shape):
            orig = x[idx]
            x[idx] = orig + np.float32(H)
            lp = loss(orc, inp, lengths, mask, ups, scale)
            x[idx] = orig - np.float32(H)
            lm = loss(orc, inp, lengths, mask, ups, scale)
            x[idx] = orig
            fd = (lp - lm) / (2 * H)
            assert abs(fd - grads[name][idx]) <= 2e-5 + 2e-5 * abs(fd), (name, idx, fd,
                                                                          grads[name][idx])


def test_structure(orc):
    rng = np.random.default_rng(5)
    B, Hq, Hk, Q, M, D, Dv = 3, 2, 1, 3, 8, 4, 4
    # row 0 appends 2 at slot 3; row 1 appends nothing; row 2 overflows (rejected)
    inp, lengths, mask, ups = make(rng, B, Hq, Hk, Q, M, D, Dv, [3, 5, 7], [2, 0, 2])
    g = oracle.step_backward(**inp, lengths=lengths, append_mask=mask, **ups)
    # overwritten slots carry nothing back to the old cache
    assert not g.key_cache[0, :, 3:5].any() and not g.value_cache[0, :, 3:5].any()
    # rows with nothing appended and rejected rows: the cache passes its gradient through
    for b in (1, 2):
        np.testing.assert_array_equal(g.key_cache[b], ups["d_key_cache_out"][b])
        np.testing.assert_array_equal(g.value_cache[b], ups["d_value_cache_out"][b])
        assert not g.query[b].any() and not g.new_key[b].any()
    # masked-out tokens (t >= n) get no gradient; slots past the last visible one
    # see only the pass-through
    assert not g.query[0, :, 2].any() and not g.new_key[0, :, 2].any()
    np.testing.assert_array_equal(g.key_cache[0, :, 5:], ups["d_key_cache_out"][0, :, 5:])


def test_closed_forms():
    """Two cases with a closed form.  One visible slot (length 0, one token):
    P = 1, so dS = P (dP - P dP) = 0; the query gets nothing, the appended
    key only the returned cache's gradient, and the appended value the sum
    of dO over its query heads plus that gradient.  All visible keys equal:
    P is uniform and sum_j dS_j = 0, so dq = scale sum_j dS_j K_j = 0 while
    the keys still get scale dS_j q."""
    rng = np.random.default_rng(11)
    B, Hq, Hk, Q, M, D, Dv = 2, 4, 2, 1, 5, 3, 2
    G = Hq // Hk
    inp, lengths, mask, ups = make(rng, B, Hq, Hk, Q, M, D, Dv, [0, 0], [1, 1])
    g = oracle.step_backward(**inp, lengths=lengths, append_mask=mask, **ups)
    assert np.abs(g.query).max() < 1e-12
    np.testing.assert_allclose(g.new_key[:, :, 0], ups["d_key_cache_out"][:, :, 0], atol=1e-12)
    want_v = ups["d_context"][:, :, 0].reshape(B, Hk, G, Dv).sum(axis=2) \
        + ups["d_value_cache_out"][:, :, 0]
    np.testing.assert_allclose(g.new_value[:, :, 0], want_v, rtol=1e-12, atol=1e-12)
    assert not g.key_cache[:, :, 0].any() and not g.value_cache[:, :, 0].any()

    # equal keys: rows of length 3 plus one appended row, every visible key the same
    inp, lengths, mask, ups = make(rng, B, Hq, Hk, Q, M, D, Dv, [3, 2], [1, 1])
    k = grid(rng, (D,))
    inp["key_cache"][:] = k
    inp["new_key"][:] = k
    g = oracle.step_backward(**inp, lengths=lengths, append_mask=mask, **ups)
    assert np.abs(g.query).max() < 1e-12
    # ... while dS itself is not zero: the keys do get a gradient beyond the pass-through
    assert np.abs(g.key_cache[:, :, :2] - ups["d_key_cache_out"][:, :, :2]).max() > 1e-3
