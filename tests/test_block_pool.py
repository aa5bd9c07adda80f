"""Host logic of the paged-cache block pool (mla_block_pool_*): no GPU."""
import ctypes
import os

import numpy as np
import pytest

import mla_latent_kv_02_amd as mla
from mla_latent_kv_02_amd import _binding as bd


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bd.LIB_PATH):
        pytest.skip("libmla.so not built")
    return mla.load_library()


def test_sizes_and_bad_arguments(lib):
    assert lib.mla_block_pool_bytes(10, 2, 3) == 4 * (8 + 10 + 2 + 6)
    assert lib.mla_block_pool_bytes(-1, 2, 3) == -1
    assert lib.mla_block_pool_bytes(4, 2, 0) == -1
    buf = np.zeros(64, np.int32)
    p = buf.ctypes.data_as(ctypes.c_void_p)
    # not initialised: every call refuses it
    assert lib.mla_block_pool_reserve(p, 0, 1) == bd.MLA_ERR_INVALID_ARG
    assert lib.mla_block_pool_release(p, 0) == bd.MLA_ERR_INVALID_ARG
    assert not lib.mla_block_pool_table(p)
    assert lib.mla_block_pool_free_count(p) == -1
    assert lib.mla_block_pool_init(p, 8, 4, 16, 2, 3) == bd.MLA_ERR_INVALID_ARG      # too small
    assert lib.mla_block_pool_init(p, 256, 4, 0, 2, 3) == bd.MLA_ERR_INVALID_ARG     # block size 0
    assert lib.mla_block_pool_init(None, 256, 4, 16, 2, 3) == bd.MLA_ERR_INVALID_ARG
    assert lib.mla_block_pool_init(p, 256, 4, 16, 2, 3) == bd.MLA_OK
    assert lib.mla_block_pool_reserve(p, 2, 1) == bd.MLA_ERR_INVALID_ARG             # b out of range
    assert lib.mla_block_pool_reserve(p, 0, -1) == bd.MLA_ERR_INVALID_ARG
    assert lib.mla_block_pool_reserve(p, 0, 3 * 16 + 1) == bd.MLA_ERR_INVALID_ARG    # > max_blocks
    assert b"free blocks" in lib.mla_status_string(bd.MLA_ERR_OUT_OF_BLOCKS)


def test_growth_order_exhaustion_and_reuse():
    pool = mla.BlockPool(n_blocks=5, block_size=16, B=3, max_blocks=4)
    assert pool.free_count == 5 and (pool.table == -1).all()
    pool.reserve(0, 1)                   # one block
    pool.reserve(1, 16)                  # exactly one block
    pool.reserve(0, 17)                  # crosses into a second block
    np.testing.assert_array_equal(pool.table[0], [0, 2, -1, -1])
    np.testing.assert_array_equal(pool.table[1], [1, -1, -1, -1])
    pool.reserve(0, 5)                   # never shrinks
    np.testing.assert_array_equal(pool.table[0], [0, 2, -1, -1])
    assert pool.free_count == 2
    with pytest.raises(bd.MlaError) as e:
        pool.reserve(2, 3 * 16)          # needs 3, only 2 free: nothing taken
    assert e.value.status == bd.MLA_ERR_OUT_OF_BLOCKS
    assert pool.free_count == 2 and (pool.table[2] == -1).all()
    pool.release(0)                      # blocks 0 and 2 come back on top of the free stack, 0 first
    assert pool.free_count == 4 and (pool.table[0] == -1).all()
    pool.reserve(2, 3 * 16)
    np.testing.assert_array_equal(pool.table[2], [0, 2, 3, -1])
    pool.release(1)
    pool.release(1)                      # releasing an empty sequence is a no-op
    assert pool.free_count == 2


def test_random_workload_keeps_the_pool_consistent():
    """Random grow / release traffic: every block is owned by at most one
    sequence, owned + free = all blocks, each row holds exactly the blocks its
    token count needs, and the outcome of every request matches a plain model
    of the rule (take the most recently freed block first)."""
    rng = np.random.default_rng(7)
    nb, bs, B, mb = 40, 8, 6, 12
    pool = mla.BlockPool(nb, bs, B, mb)
    free = list(range(nb - 1, -1, -1))       # model: a stack, top at the end
    rows = [[] for _ in range(B)]
    toks = [0] * B
    for _ in range(2000):
        b = int(rng.integers(B))
        if rng.random() < 0.15:
            pool.release(b)
            free.extend(reversed(rows[b]))
            rows[b], toks[b] = [], 0
            continue
        n = toks[b] + int(rng.integers(0, 20))
        need = -(-n // bs)
        if need > mb:
            with pytest.raises(bd.MlaError):
                pool.reserve(b, n)
            continue
        extra = max(0, need - len(rows[b]))
        if extra > len(free):
            with pytest.raises(bd.MlaError) as e:
                pool.reserve(b, n)
            assert e.value.status == bd.MLA_ERR_OUT_OF_BLOCKS
            continue
        pool.reserve(b, n)
        for _k in range(extra):
            rows[b].append(free.pop())
        toks[b] = max(toks[b], n)
        owned = [x for r in rows for x in r]
        assert len(owned) == len(set(owned)) and len(owned) + pool.free_count == nb
        for s in range(B):
            np.testing.assert_array_equal(pool.table[s], rows[s] + [-1] * (mb - len(rows[s])))


def test_reserve_all_is_all_or_nothing():
    pool = mla.BlockPool(n_blocks=6, block_size=4, B=3, max_blocks=4)
    pool.reserve_all(np.array([5, -1, 4]))          # 2 + 1 blocks; sequence 1 untouched
    np.testing.assert_array_equal(pool.table[:, :2], [[0, 1], [-1, -1], [2, -1]])
    with pytest.raises(bd.MlaError) as e:
        pool.reserve_all(np.array([16, 8, 4]))      # needs 2 + 2 more, 3 free
    assert e.value.status == bd.MLA_ERR_OUT_OF_BLOCKS
    assert pool.free_count == 3 and (pool.table[1] == -1).all()
    with pytest.raises(bd.MlaError) as e:
        pool.reserve_all(np.array([17, 0, 0]))      # more than max_blocks
    assert e.value.status == bd.MLA_ERR_INVALID_ARG
    pool.reserve_all(np.array([8, 8, 4]))
    assert pool.free_count == 1
    with pytest.raises(ValueError):
        pool.reserve_all(np.array([1, 2]))
