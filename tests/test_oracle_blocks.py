"""Pins of the oracle's whole-block moves (copy-on-write copy, swap-out
gather, swap-in scatter) against what the operations must do, on hand-built
pools whose every byte names its block and position.  CPU only.

[P1] "KV Cache 的内存开销与分页机制" and [P2] section 4.1: a sequence that
writes into a shared block first gets a private copy; [P2] section 3:
blocks leave device memory and come back.
"""

import numpy as np
import pytest

import oracle


def _pool(nb=8, per_block=(2, 3, 4)):
    # Block b holds 1000*b + its flat position: every value is unique and a
    # moved block can be recognised anywhere.
    n = int(np.prod(per_block))
    return (1000 * np.arange(nb)[:, None] + np.arange(n)[None, :]).reshape((nb, *per_block)).astype(np.float64)


def test_copy_destination_equals_old_source_and_nothing_else_moves():
    pool = _pool()
    before = pool.copy()
    oracle.copy_blocks(pool, [1, 6], [3, 0])
    assert np.array_equal(pool[3], before[1])
    assert np.array_equal(pool[0], before[6])
    for b in (1, 2, 4, 5, 6, 7):  # sources and bystanders keep their bytes
        assert np.array_equal(pool[b], before[b])


def test_copy_one_source_to_several_destinations():
    pool = _pool()
    before = pool.copy()
    oracle.copy_blocks(pool, [2, 2, 2], [5, 6, 7])
    for b in (5, 6, 7):
        assert np.array_equal(pool[b], before[2])
    assert np.array_equal(pool[:5], before[:5])


def test_copy_works_on_any_per_block_layout():
    # The key pool [NB][H][B][D] and the transposed value pool [NB][H][D][B]
    # move the same way: a block is its whole first-axis slice.
    k, v = _pool(per_block=(2, 4, 3)), _pool(per_block=(2, 3, 4))
    kb, vb = k.copy(), v.copy()
    oracle.copy_blocks(k, [4], [1])
    oracle.copy_blocks(v, [4], [1])
    assert np.array_equal(k[1], kb[4]) and np.array_equal(v[1], vb[4])


@pytest.mark.parametrize("src,dst", [([1, 2], [3, 3]), ([1, 2], [2, 4]), ([3, 1], [1, 5])])
def test_copy_rejects_repeated_or_aliased_destinations(src, dst):
    # Repeated destination, or a destination that is also a source (a chain
    # 1->2, 2->4 would depend on the order of the copies): refused, pool intact.
    pool = _pool()
    before = pool.copy()
    with pytest.raises(ValueError):
        oracle.copy_blocks(pool, src, dst)
    assert np.array_equal(pool, before)


def test_copy_skips_out_of_pool_and_identity_pairs():
    pool = _pool()
    before = pool.copy()
    oracle.copy_blocks(pool, [-1, 3, 8, 5, 2], [4, 3, 1, 100, 6])
    expect = before.copy()
    expect[6] = before[2]  # the only pair inside the pool with src != dst
    assert np.array_equal(pool, expect)


def test_copy_length_mismatch():
    with pytest.raises(ValueError):
        oracle.copy_blocks(_pool(), [1, 2], [3])


def test_gather_rows_in_id_order():
    pool = _pool()
    rows = oracle.gather_blocks(pool, [5, 0, 5, 2])
    assert rows.shape == (4, *pool.shape[1:])
    for i, b in enumerate([5, 0, 5, 2]):
        assert np.array_equal(rows[i], pool[b])


def test_gather_leaves_rows_of_out_of_pool_ids_untouched():
    pool = _pool()
    out = np.full((3, *pool.shape[1:]), -7.0)
    oracle.gather_blocks(pool, [1, 9, -2], out=out)
    assert np.array_equal(out[0], pool[1])
    assert (out[1:] == -7.0).all()
    assert (oracle.gather_blocks(pool, [8])[0] == 0).all()


def test_scatter_writes_only_the_named_blocks():
    pool = np.full((6, 2, 2), -1.0)
    rows = np.arange(3 * 4, dtype=np.float64).reshape(3, 2, 2)
    oracle.scatter_blocks(pool, [4, 0, 6], rows)  # 6 is outside the pool: skipped
    assert np.array_equal(pool[4], rows[0]) and np.array_equal(pool[0], rows[1])
    assert (pool[[1, 2, 3, 5]] == -1.0).all()


def test_scatter_rejects_a_repeated_destination():
    pool = np.zeros((4, 2))
    with pytest.raises(ValueError):
        oracle.scatter_blocks(pool, [1, 1], np.ones((2, 2)))


def test_gather_scatter_round_trip_restores_a_wiped_pool():
    pool = _pool(nb=16)
    rng = np.random.default_rng(0)
    ids = rng.choice(16, 9, replace=False)
    rows = oracle.gather_blocks(pool, ids)
    wiped = pool.copy()
    wiped[ids] = np.nan
    oracle.scatter_blocks(wiped, ids, rows)
    assert np.array_equal(wiped, pool)


def test_swap_to_other_blocks_then_copy_back():
    # Swap out blocks 2, 3, swap them in as 6, 7, then copy-on-write them
    # back over 2, 3 of a pool whose 2, 3 were reused: the round trip through
    # all three moves lands the original bytes.
    pool = _pool()
    before = pool.copy()
    rows = oracle.gather_blocks(pool, [2, 3])
    pool[[2, 3]] = 0.0
    oracle.scatter_blocks(pool, [6, 7], rows)
    oracle.copy_blocks(pool, [6, 7], [2, 3])
    assert np.array_equal(pool[[2, 3]], before[[2, 3]])
    assert np.array_equal(pool[[6, 7]], before[[2, 3]])
