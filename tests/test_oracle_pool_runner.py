"""The multi-process oracle runner (oracle/pool.py) against the oracle itself.

Every full-size parity reference and the benchmark's CPU baseline come from
oracle.pool.run_rows, which splits the requested rows into chunks, evaluates
each chunk in a spawned worker with the oracle function of the call's form,
and concatenates the parts. These CPU tests pin that plumbing: for token
lists over a cached prefix (q_pos0 != 0), micro-block lists and slot-pool
lists, with unsorted and repeated row lists, run_rows with 2 and 3 workers
gives exactly (bit for bit) what one direct oracle call gives. A dropped
argument (q_pos0, block_size, the pool positions), a chunk placed out of
order or a row paired with another row's list fails here.
"""
import numpy as np
import pytest

import oracle
from oracle import pool as oracle_pool
from qsa_inputs import f32_to_bf16_bits


def rand_bf16(rng, shape):
    return f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


def rows_under_test(rng, T):
    """Unsorted rows, with one repeated, that several chunks split."""
    rows = rng.permutation(T)[: max(7, T // 2)]
    return np.concatenate([rows, rows[:1]]).astype(np.int64)


def assert_bitwise(got, ref):
    for g, r in zip(got, ref):
        assert g.dtype == r.dtype and g.shape == r.shape
        np.testing.assert_array_equal(g.view(np.uint64), r.view(np.uint64))


@pytest.mark.parametrize("workers", [2, 3])
def test_token_lists_with_cached_prefix(workers):
    rng = np.random.default_rng(1)
    T, p0, T_kv, Hq, Hkv, K = 40, 57, 120, 6, 2, 30
    q = rand_bf16(rng, (T, Hq, 256))
    k, v = rand_bf16(rng, (T_kv, Hkv, 256)), rand_bf16(rng, (T_kv, Hkv, 256))
    idx = rng.integers(-2, T_kv + 2, size=(T, Hkv, K)).astype(np.int32)
    rows = rows_under_test(rng, T)
    ref = oracle.sparse_prefill(q, k, v, idx[rows], scale=0.07, rows=rows, q_pos0=p0)
    got = oracle_pool.run_rows(q, k, v, idx[rows], rows, 0.07, q_pos0=p0, workers=workers)
    assert_bitwise(got, ref)
    # the prefix matters for these lists: the same call without it differs
    assert not np.array_equal(oracle.sparse_prefill(q, k, v, idx[rows], scale=0.07, rows=rows)[1], ref[1])


@pytest.mark.parametrize("workers", [2, 3])
def test_micro_block_lists(workers):
    rng = np.random.default_rng(2)
    T, p0, T_kv, Hq, Hkv, nb, B = 36, 20, 64, 4, 1, 9, 4
    q = rand_bf16(rng, (T, Hq, 256))
    k, v = rand_bf16(rng, (T_kv, Hkv, 256)), rand_bf16(rng, (T_kv, Hkv, 256))
    bidx = rng.integers(-1, T_kv // B + 1, size=(T, Hkv, nb)).astype(np.int32)
    rows = rows_under_test(rng, T)
    ref = oracle.sparse_prefill_blocks(q, k, v, bidx[rows], B, scale=1 / 16, rows=rows, q_pos0=p0)
    got = oracle_pool.run_rows(q, k, v, bidx[rows], rows, 1 / 16, q_pos0=p0, block_size=B, workers=workers)
    assert_bitwise(got, ref)


@pytest.mark.parametrize("workers", [2, 3])
def test_pool_lists(workers):
    rng = np.random.default_rng(3)
    n_slots, total_q, Hq, Hkv, K = 90, 30, 8, 2, 25
    q = rand_bf16(rng, (total_q, Hq, 256))
    k, v = rand_bf16(rng, (n_slots, Hkv, 256)), rand_bf16(rng, (n_slots, Hkv, 256))
    slot_pos = rng.integers(-1, 60, size=n_slots).astype(np.int32)
    q_pos = rng.integers(0, 60, size=total_q).astype(np.int32)
    idx = rng.integers(-2, n_slots + 2, size=(total_q, Hkv, K)).astype(np.int32)
    rows = rows_under_test(rng, total_q)
    ref = oracle.sparse_prefill_pool(q, k, v, idx[rows], q_pos, slot_pos, scale=1 / 16, rows=rows)
    got = oracle_pool.run_rows(q, k, v, idx[rows], rows, 1 / 16, q_pos=q_pos, slot_pos=slot_pos, workers=workers)
    assert_bitwise(got, ref)


def test_single_worker_and_timing_forms():
    rng = np.random.default_rng(4)
    T, Hq, Hkv, K = 12, 3, 1, 10
    q, k, v = rand_bf16(rng, (T, Hq, 256)), rand_bf16(rng, (T, Hkv, 256)), rand_bf16(rng, (T, Hkv, 256))
    idx = rng.integers(-1, T, size=(T, Hkv, K)).astype(np.int32)
    rows = rng.permutation(T)
    ref = oracle.sparse_prefill(q, k, v, idx[rows], scale=1 / 16, rows=rows)
    assert_bitwise(oracle_pool.run_rows(q, k, v, idx[rows], rows, 1 / 16, workers=1), ref)
    out, lse, secs = oracle_pool.run_rows(q, k, v, idx[rows], rows, 1 / 16, workers=2, return_seconds=True)
    assert_bitwise((out, lse), ref)
    assert secs > 0
