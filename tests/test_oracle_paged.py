"""The paged step of the oracle against its pins (no GPU).

The oracle reads a block-pool cache as the dense cache its table describes
(the block-pool layout named beside the continuous one for ClikaRT's
attention_over_cache).  Pinned here against the dense oracle (itself pinned
in test_oracle_pins.py) through gathers written out with plain loops, and
against the invariants the layout fixes: pool rows that no appended slot
maps to keep their bits, a shared prefix block reads the same for every row
that maps it.
"""
import numpy as np
import pytest

import oracle


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.Oracle()


def draw(rng, B, Hq, Hk, Q, bs, max_blocks, D, Dv, num_blocks, lengths, n):
    q = rng.standard_normal((B, Hq, Q, D)).astype(np.float32)
    nk = rng.standard_normal((B, Hk, Q, D)).astype(np.float32)
    nv = rng.standard_normal((B, Hk, Q, Dv)).astype(np.float32)
    kp = rng.standard_normal((num_blocks, Hk, bs, D)).astype(np.float32)
    vp = rng.standard_normal((num_blocks, Hk, bs, Dv)).astype(np.float32)
    mask = np.zeros((B, Q), np.uint8)
    for b in range(B):
        mask[b, :n[b]] = 1
    return q, nk, nv, kp, vp, np.asarray(lengths, np.int64), mask


def dense_by_loops(pool, table, M):
    """key_cache[b, h, j] = pool[table[b, j // bs], h, j % bs], slot by slot."""
    nb, H, bs, D = pool.shape
    B = table.shape[0]
    out = np.zeros((B, H, M, D), pool.dtype)
    for b in range(B):
        for h in range(H):
            for j in range(M):
                blk = table[b, j // bs]
                if 0 <= blk < nb:
                    out[b, h, j] = pool[blk, h, j % bs]
    return out


def test_identity_table_is_the_dense_step(orc):
    """Row b owning blocks b*mb .. b*mb+mb-1 in order: the pool is the dense
    cache cut into blocks, and the paged step is the dense step."""
    rng = np.random.default_rng(1)
    B, Hq, Hk, Q, bs, mb, D, Dv = 3, 4, 2, 2, 4, 3, 8, 8
    M = bs * mb
    lengths, n = [0, 5, 9], [2, 1, 2]
    q, nk, nv, kp, vp, ln, mask = draw(rng, B, Hq, Hk, Q, bs, mb, D, Dv, B * mb, lengths, n)
    table = np.arange(B * mb, dtype=np.int32).reshape(B, mb)
    dense_k = kp.reshape(B, mb, Hk, bs, D).transpose(0, 2, 1, 3, 4).reshape(B, Hk, M, D)
    dense_v = vp.reshape(B, mb, Hk, bs, Dv).transpose(0, 2, 1, 3, 4).reshape(B, Hk, M, Dv)
    ref = orc.step(q, nk, nv, dense_k, dense_v, ln, mask)
    got = orc.step_paged(q, nk, nv, kp, vp, table, ln, mask)
    np.testing.assert_array_equal(got.attention, ref.attention)
    np.testing.assert_array_equal(got.context, ref.context)
    np.testing.assert_array_equal(got.lengths, ref.lengths)
    back_k = got.key_pool.reshape(B, mb, Hk, bs, D).transpose(0, 2, 1, 3, 4).reshape(B, Hk, M, D)
    back_v = got.value_pool.reshape(B, mb, Hk, bs, Dv).transpose(0, 2, 1, 3, 4).reshape(B, Hk, M, Dv)
    assert np.array_equal(back_k.view(np.uint32), ref.key_cache.view(np.uint32))
    assert np.array_equal(back_v.view(np.uint32), ref.value_cache.view(np.uint32))


def test_permuted_table_against_loops(orc):
    """Rows own scattered blocks; outputs equal the dense step over the cache
    gathered slot by slot, appended rows land in the mapped pool rows, and
    every other pool row (spare blocks included) keeps its bits."""
    rng = np.random.default_rng(2)
    B, Hq, Hk, Q, bs, mb, D, Dv = 3, 6, 3, 3, 4, 4, 4, 4
    M, nb = bs * mb, B * mb + 5
    lengths, n = [3, 7, 13], [3, 2, 3]
    q, nk, nv, kp, vp, ln, mask = draw(rng, B, Hq, Hk, Q, bs, mb, D, Dv, nb, lengths, n)
    table = rng.permutation(nb)[:B * mb].astype(np.int32).reshape(B, mb)
    dk, dv = dense_by_loops(kp, table, M), dense_by_loops(vp, table, M)
    ref = orc.step(q, nk, nv, dk, dv, ln, mask)
    got = orc.step_paged(q, nk, nv, kp, vp, table, ln, mask)
    np.testing.assert_array_equal(got.attention, ref.attention)
    np.testing.assert_array_equal(got.context, ref.context)
    written = np.zeros((nb, bs), bool)
    for b in range(B):
        for t in range(n[b]):
            j = lengths[b] + t
            blk = table[b, j // bs]
            written[blk, j % bs] = True
            np.testing.assert_array_equal(got.key_pool[blk, :, j % bs], nk[b, :, t])
            np.testing.assert_array_equal(got.value_pool[blk, :, j % bs], nv[b, :, t])
    keep = ~written
    assert np.array_equal(got.key_pool.transpose(0, 2, 1, 3)[keep].view(np.uint32),
                          kp.transpose(0, 2, 1, 3)[keep].view(np.uint32))
    assert np.array_equal(got.value_pool.transpose(0, 2, 1, 3)[keep].view(np.uint32),
                          vp.transpose(0, 2, 1, 3)[keep].view(np.uint32))


def test_shared_prefix_block(orc):
    """Two rows map the same first block (a shared prefix below both lengths):
    each reads it as its own slots 0 .. bs-1."""
    rng = np.random.default_rng(3)
    B, Hq, Hk, Q, bs, mb, D, Dv = 2, 2, 1, 1, 4, 3, 4, 4
    M, nb = bs * mb, 6
    lengths, n = [6, 5], [1, 1]
    q, nk, nv, kp, vp, ln, mask = draw(rng, B, Hq, Hk, Q, bs, mb, D, Dv, nb, lengths, n)
    table = np.array([[0, 1, 2], [0, 3, 4]], np.int32)
    got = orc.step_paged(q, nk, nv, kp, vp, table, ln, mask)
    dk, dv = dense_by_loops(kp, table, M), dense_by_loops(vp, table, M)
    assert np.array_equal(dk[0, :, :bs], dk[1, :, :bs])
    ref = orc.step(q, nk, nv, dk, dv, ln, mask)
    np.testing.assert_array_equal(got.attention, ref.attention)
    np.testing.assert_array_equal(got.context, ref.context)
    assert np.array_equal(got.key_pool[0], kp[0])  # the shared block is only read


def test_rejected_row_writes_nothing(orc):
    """A row outside the contract (overflow) is a no-op in the pool too."""
    rng = np.random.default_rng(4)
    B, Hq, Hk, Q, bs, mb, D, Dv = 2, 2, 1, 2, 4, 2, 4, 4
    lengths, n = [7, 2], [2, 2]  # row 0: 7 + 2 > 8
    q, nk, nv, kp, vp, ln, mask = draw(rng, B, Hq, Hk, Q, bs, mb, D, Dv, 4, lengths, n)
    table = np.array([[0, 1], [2, 3]], np.int32)
    got = orc.step_paged(q, nk, nv, kp, vp, table, ln, mask)
    assert list(got.row_status) == [oracle.ROW_OVERFLOW, oracle.ROW_OK]
    assert np.array_equal(got.key_pool[:2], kp[:2]) and np.array_equal(got.value_pool[:2], vp[:2])
    assert got.lengths[0] == 7 and got.lengths[1] == 4
    assert not got.attention[0].any() and not got.context[0].any()
