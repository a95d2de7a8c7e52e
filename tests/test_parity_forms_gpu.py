"""GPU parity of the micro-block and slot-pool entry points against the oracle.

Micro-block lists: "Qwen4-Exp QSA llega al Ascend de Huawei" (orcarouter.ai,
Spanish page), section "Por qué QSA es la parte incómoda, en cifras"
(compression ratio 4, 2,048 micro-blocks per query) and section "Nueve
pruebas que pasaron" (causal-tail remainders 0..3). Slot pools: the same
section (unordered physical slots, two requests mapping a shared prefix,
cache-content reuse).

Besides the oracle bar (tests/parity.py), two kernel-to-kernel identities are
checked bit for bit, since the kernel's arithmetic does not depend on where a
row lives: a block list equals the token list it expands to, and a pool batch
equals one extend call per request on that request's gathered cache.
"""
import os
import sys
import time

import numpy as np
import pytest

import oracle
from oracle import pool as oracle_pool
from qsa_inputs import (f32_to_bf16_bits, get_config, make_indices, make_pool_inputs, make_qkv,
                        sample_pool_rows, sample_rows)
from tests.parity import compare, torch_bf16_to_numpy_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import top_sparse_attention_qsa_amd as qsa  # noqa: E402

INT32_MIN = -(2 ** 31)
INT32_MAX = 2 ** 31 - 1


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X: no HIP device visible")
    qsa.load_library()
    return torch.device("cuda", 0)


def dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a)).view(torch.bfloat16).to("cuda")


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda")


def rand_bf16(rng, shape):
    return f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


def progress(msg):
    sys.__stdout__.write(f"    {time.strftime('%H:%M:%S')} {msg}\n")
    sys.__stdout__.flush()


def host(out, lse):
    torch.cuda.synchronize()
    return torch_bf16_to_numpy_bits(out), lse.cpu().numpy()


def run_blocks(q, k, v, bidx, B, q_pos0=0, scale=None):
    return host(*qsa.sparse_prefill_blocks(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_i32(bidx), q_pos0, B,
                                           scale=scale))


def run_tokens(q, k, v, idx, q_pos0=0, scale=None):
    return host(*qsa.sparse_prefill_extend(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_i32(idx), q_pos0,
                                           scale=scale))


def run_pool(q, k, v, idx, q_pos, slot_pos, scale=None):
    return host(*qsa.sparse_prefill_pool(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_i32(idx), dev_i32(q_pos),
                                         dev_i32(slot_pos), scale=scale))


def expand(bidx, B):
    """Token lists named by block lists (entries b*B .. b*B+B-1, in order);
    values that do not fit int32 become -1 (masked either way)."""
    t = bidx.astype(np.int64)[..., None] * B + np.arange(B)
    t = t.reshape(bidx.shape[0], bidx.shape[1], -1)
    t[(t > INT32_MAX) | (t < 0)] = -1
    return t.astype(np.int32)


# ------------------------------------------------------------------ micro-blocks


def test_blocks_small_workload_all_rows():
    cfg = get_config(7)
    q, k, v = make_qkv(cfg)
    bidx = make_indices(cfg)
    out, lse = run_blocks(q, k, v, bidx, cfg.block_size, scale=cfg.scale)
    ref_out, ref_lse = oracle.sparse_prefill_blocks(q, k, v, bidx, cfg.block_size, scale=cfg.scale)
    progress(f"{cfg.name}: {compare(out, lse, ref_out, ref_lse, label=cfg.name)}")


def test_blocks_full_size_sampled_rows():
    cfg = get_config(8)
    t0 = time.perf_counter()
    q, k, v = make_qkv(cfg)
    bidx = make_indices(cfg)
    progress(f"{cfg.name}: inputs in {time.perf_counter() - t0:.1f}s")
    out, lse = run_blocks(q, k, v, bidx, cfg.block_size, scale=cfg.scale)
    rows = sample_rows(cfg)
    progress(f"{cfg.name}: gpu done; oracle on {rows.size} rows")
    ref_out, ref_lse = oracle_pool.run_rows(q, k, v, bidx[rows], rows, cfg.scale, block_size=cfg.block_size)
    stats = compare(out[rows], lse[rows], ref_out, ref_lse, label=cfg.name)
    progress(f"{cfg.name}: {stats} ({time.perf_counter() - t0:.1f}s)")
    assert not np.any((out.view(np.uint16) & 0x7F80) == 0x7F80), "non-finite output"
    assert np.all(np.isfinite(lse))
    assert stats["rel_l2"] < 0.008


@pytest.mark.parametrize("B", [1, 2, 4, 8, 16])
def test_block_causal_tails(B):
    """Every row lists its own block (remainders 0..B-1 all occur) among
    random earlier blocks, a future block and -1 pads, in random order."""
    rng = np.random.default_rng(100 + B)
    T, Hq, Hkv, nb = 8 * B + 3, 6, 2, 11
    q, k, v = rand_bf16(rng, (T, Hq, 256)), rand_bf16(rng, (T + B, Hkv, 256)), rand_bf16(rng, (T + B, Hkv, 256))
    bidx = np.full((T, Hkv, nb), -1, np.int32)
    for t in range(T):
        bt = t // B
        for g in range(Hkv):
            row = [bt] + list(rng.integers(0, bt + 1, size=min(bt, 6))) + [bt + 1]
            row = (row + [-1] * nb)[:nb]
            rng.shuffle(row)
            bidx[t, g] = row
    out, lse = run_blocks(q, k[:T], v[:T], bidx, B)
    ref_out, ref_lse = oracle.sparse_prefill_blocks(q, k[:T], v[:T], bidx, B)
    compare(out, lse, ref_out, ref_lse, label=f"tails B={B}")


@pytest.mark.parametrize("B", [2, 4, 16])
def test_block_lists_equal_their_token_expansion_bitwise(B):
    rng = np.random.default_rng(200 + B)
    T, T_kv, p0 = 301, 420, 119
    q, k, v = rand_bf16(rng, (T, 12, 256)), rand_bf16(rng, (T_kv, 1, 256)), rand_bf16(rng, (T_kv, 1, 256))
    nb = 37
    bidx = rng.integers(-3, (T_kv + B - 1) // B + 2, size=(T, 1, nb)).astype(np.int32)
    a = run_blocks(q, k, v, bidx, B, q_pos0=p0)
    b = run_tokens(q, k, v, expand(bidx, B), q_pos0=p0)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    ref_out, ref_lse = oracle.sparse_prefill_blocks(q, k, v, bidx, B, q_pos0=p0)
    compare(a[0], a[1], ref_out, ref_lse, label=f"blocks extend B={B}")


def test_invalid_blocks_are_masked():
    rng = np.random.default_rng(7)
    T = 40
    q, k, v = rand_bf16(rng, (T, 3, 256)), rand_bf16(rng, (T, 1, 256)), rand_bf16(rng, (T, 1, 256))
    bad = np.array([-1, INT32_MIN, INT32_MAX, 1 << 29, (1 << 29) - 1, 10, -7, 1 << 30], np.int32)
    bidx = np.broadcast_to(bad, (T, 1, bad.size)).copy()
    bidx[:, 0, 5] = np.arange(T) // 4  # the own block, so rows are not empty
    out, lse = run_blocks(q, k, v, bidx, 4)
    ref_out, ref_lse = oracle.sparse_prefill_blocks(q, k, v, bidx, 4)
    compare(out, lse, ref_out, ref_lse, label="invalid blocks")


def test_blocks_empty_and_zero_width():
    rng = np.random.default_rng(8)
    q, k, v = rand_bf16(rng, (5, 2, 256)), rand_bf16(rng, (5, 1, 256)), rand_bf16(rng, (5, 1, 256))
    out, lse = run_blocks(q, k, v, np.zeros((5, 1, 0), np.int32), 4)
    assert np.all(out == 0) and np.all(np.isneginf(lse))
    out, lse = run_blocks(q, k, v, np.full((5, 1, 3), -1, np.int32), 4)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_block_size_is_validated():
    rng = np.random.default_rng(9)
    q, k = rand_bf16(rng, (4, 1, 256)), rand_bf16(rng, (4, 1, 256))
    with pytest.raises(qsa.QsaError):
        qsa.sparse_prefill_blocks(dev_bf16(q), dev_bf16(k), dev_bf16(k), dev_i32(np.zeros((4, 1, 2))), 0, 3)


# ------------------------------------------------------------------ slot pool


def _per_request_extend_bitwise(d, out, lse):
    """Each request's rows equal one extend call over its gathered cache."""
    k, v, idx, slot_pos = d["k"], d["v"], d["idx"], d["slot_pos"]
    for r in d["requests"]:
        a, b = r["rows"]
        table = r["table"]
        lists = idx[a:b]
        pos = np.where(lists >= 0, slot_pos[np.maximum(lists, 0)], -1).astype(np.int32)
        eo, el = run_tokens(d["q"][a:b], k[table], v[table], pos, q_pos0=r["cached"], scale=d["scale"])
        np.testing.assert_array_equal(out[a:b], eo)
        np.testing.assert_array_equal(lse[a:b], el)


def test_pool_small_workload_all_rows():
    d = make_pool_inputs(9)
    out, lse = run_pool(d["q"], d["k"], d["v"], d["idx"], d["q_pos"], d["slot_pos"], scale=d["scale"])
    ref_out, ref_lse = oracle.sparse_prefill_pool(d["q"], d["k"], d["v"], d["idx"], d["q_pos"], d["slot_pos"],
                                                  scale=d["scale"])
    progress(f"{d['cfg'].name}: {compare(out, lse, ref_out, ref_lse, label=d['cfg'].name)}")
    _per_request_extend_bitwise(d, out, lse)


@pytest.mark.parametrize("number", [10, 13])
def test_pool_full_size_sampled_rows(number):
    t0 = time.perf_counter()
    d = make_pool_inputs(number)
    cfg = d["cfg"]
    progress(f"{cfg.name}: inputs in {time.perf_counter() - t0:.1f}s")
    args = (d["q"], d["k"], d["v"], d["idx"], d["q_pos"], d["slot_pos"])
    out, lse = run_pool(*args, scale=cfg.scale)
    rows = sample_pool_rows(cfg)
    progress(f"{cfg.name}: gpu done; oracle on {rows.size} rows")
    ref_out, ref_lse = oracle_pool.run_rows(d["q"], d["k"], d["v"], d["idx"][rows], rows, cfg.scale,
                                            q_pos=d["q_pos"], slot_pos=d["slot_pos"])
    stats = compare(out[rows], lse[rows], ref_out, ref_lse, label=cfg.name)
    progress(f"{cfg.name}: {stats} ({time.perf_counter() - t0:.1f}s)")
    assert not np.any((out.view(np.uint16) & 0x7F80) == 0x7F80), "non-finite output"
    assert np.all(np.isfinite(lse))
    assert stats["rel_l2"] < 0.008
    _per_request_extend_bitwise(d, out, lse)
    progress(f"{cfg.name}: per-request extend identical")


def test_pool_masks_free_outside_and_future_slots():
    """Lists of the small batch with free slots, slots past the pool, negative
    values and the request's own later tokens written over the -1 padding."""
    d = make_pool_inputs(9)
    rng = np.random.default_rng(11)
    idx = d["idx"].copy()
    n_slots = d["slot_pos"].size
    free = np.nonzero(d["slot_pos"] < 0)[0]
    for r in d["requests"]:
        a, b = r["rows"]
        table = r["table"]
        for i in range(a, b):
            p = int(d["q_pos"][i])
            for g in range(idx.shape[1]):
                pad = np.nonzero(idx[i, g] < 0)[0]
                junk = [int(rng.choice(free)), n_slots, n_slots + 77, INT32_MAX, INT32_MIN, -5]
                junk += [int(s) for s in table[p + 1: p + 4]]
                for j, s in zip(pad, junk):
                    idx[i, g, j] = s
    out, lse = run_pool(d["q"], d["k"], d["v"], idx, d["q_pos"], d["slot_pos"])
    ref_out, ref_lse = oracle.sparse_prefill_pool(d["q"], d["k"], d["v"], idx, d["q_pos"], d["slot_pos"])
    compare(out, lse, ref_out, ref_lse, label="pool masking")


# bf16 bit patterns that must never reach an output through a masked slot:
# quiet NaN, NaN with a payload, +Inf, -Inf, negative NaN
NON_FINITE_BF16 = np.array([0x7FC0, 0x7F81, 0x7F80, 0xFF80, 0xFFC0], np.uint16)


def _poison(rng, shape):
    return NON_FINITE_BF16[rng.integers(0, NON_FINITE_BF16.size, size=shape)]


def _poisoned_pool(seed):
    """A pool whose free slots and whose slots holding tokens after every
    query of their request hold NaN / Inf rows in K and V, with lists that
    name those slots among valid ones. Free slots are normal in a reused KV
    pool, and a pool may already hold a request's later tokens (the pages'
    tests of physical slot mappings and cache reuse, "Qwen4-Exp QSA llega al
    Ascend de Huawei", section "Nueve pruebas que pasaron"). Request A holds
    positions 0..199 with queries at 100..149 (positions 150..199 poisoned);
    request B holds positions 0..99 with queries at 60..99; 100 free slots."""
    rng = np.random.default_rng(seed)
    n_a, n_b, n_free, Hkv, Hq, K = 200, 100, 100, 2, 8, 96
    n_slots = n_a + n_b + n_free
    perm = rng.permutation(n_slots)
    table_a, table_b, free = perm[:n_a], perm[n_a:n_a + n_b], perm[n_a + n_b:]
    slot_pos = np.full(n_slots, -1, np.int32)
    slot_pos[table_a] = np.arange(n_a)
    slot_pos[table_b] = np.arange(n_b)
    k, v = rand_bf16(rng, (n_slots, Hkv, 256)), rand_bf16(rng, (n_slots, Hkv, 256))
    bad = np.concatenate([free, table_a[150:]])
    k[bad] = _poison(rng, (bad.size, Hkv, 256))
    v[bad] = _poison(rng, (bad.size, Hkv, 256))
    queries = [(p, table_a) for p in range(100, 150)] + [(p, table_b) for p in range(60, 100)]
    q = rand_bf16(rng, (len(queries), Hq, 256))
    q_pos = np.array([p for p, _ in queries], np.int32)
    idx = np.full((len(queries), Hkv, K), -1, np.int32)
    for i, (p, table) in enumerate(queries):
        for g in range(Hkv):
            own = list(rng.choice(table[: p + 1], size=min(p + 1, 60), replace=False))
            later = list(table[p + 1: p + 12]) + (list(rng.choice(table_a[150:], 6, replace=False))
                                                  if table is table_a else [])
            junk = list(rng.choice(free, 10, replace=False)) + [n_slots, n_slots + 5, -1, INT32_MIN]
            row = own + later + junk
            rng.shuffle(row)
            idx[i, g, : len(row)] = row
    return q, k, v, idx, q_pos, slot_pos


def test_pool_and_decode_never_read_masked_slots():
    """NaN / Inf in slots that the slot rule masks (free slots, tokens after
    the query) leave every output finite and equal to the oracle's, which
    never looks at them: such slots are not gathered at all."""
    q, k, v, idx, q_pos, slot_pos = _poisoned_pool(17)
    ref_out, ref_lse = oracle.sparse_prefill_pool(q, k, v, idx, q_pos, slot_pos)
    assert np.all(np.isfinite(ref_out)) and np.all(np.isfinite(ref_lse))
    out, lse = run_pool(q, k, v, idx, q_pos, slot_pos)
    compare(out, lse, ref_out, ref_lse, label="pool, poisoned masked slots")
    # decode: one query per request (the last one of each), lists cut into ranges
    last = np.array([49, q.shape[0] - 1])
    assert qsa.decode_workspace_bytes(2, q.shape[1], k.shape[1], idx.shape[2]) > 0
    out, lse = run_decode(q[last], k, v, idx[last], q_pos[last], slot_pos)
    compare(out, lse, ref_out[last], ref_lse[last], label="decode, poisoned masked slots")


def test_sequence_forms_never_read_masked_rows():
    """Token and micro-block lists naming cache rows after the query, whose K
    and V hold NaN / Inf: every output finite and equal to the oracle's."""
    rng = np.random.default_rng(18)
    T, p0, T_kv, Hq, Hkv = 64, 100, 300, 6, 2
    q = rand_bf16(rng, (T, Hq, 256))
    k, v = rand_bf16(rng, (T_kv, Hkv, 256)), rand_bf16(rng, (T_kv, Hkv, 256))
    k[p0 + T:] = _poison(rng, (T_kv - p0 - T, Hkv, 256))
    v[p0 + T:] = _poison(rng, (T_kv - p0 - T, Hkv, 256))
    idx = np.full((T, Hkv, 80), -1, np.int32)
    bidx = np.full((T, Hkv, 24), -1, np.int32)
    for t in range(T):
        pos = p0 + t
        for g in range(Hkv):
            row = list(rng.choice(pos + 1, 50, replace=False)) + list(rng.integers(pos + 1, T_kv, 20))
            rng.shuffle(row)
            idx[t, g, : len(row)] = row
            brow = list(rng.choice(pos // 4 + 1, 16, replace=False)) + list(rng.integers(pos // 4 + 1, T_kv // 4, 8))
            rng.shuffle(brow)
            bidx[t, g] = brow
    out, lse = run_tokens(q, k, v, idx, q_pos0=p0)
    ref_out, ref_lse = oracle.sparse_prefill(q, k, v, idx, scale=1 / 16, q_pos0=p0)
    compare(out, lse, ref_out, ref_lse, label="tokens, poisoned later rows")
    out, lse = run_blocks(q, k, v, bidx, 4, q_pos0=p0)
    ref_out, ref_lse = oracle.sparse_prefill_blocks(q, k, v, bidx, 4, scale=1 / 16, q_pos0=p0)
    compare(out, lse, ref_out, ref_lse, label="blocks, poisoned later rows")


def test_pool_cache_reuse_and_inputs_unchanged():
    """The same batch twice over the same pool buffers: identical outputs,
    inputs untouched (cache content reused, never written)."""
    d = make_pool_inputs(9)
    t = [dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"]), dev_i32(d["idx"]), dev_i32(d["q_pos"]),
         dev_i32(d["slot_pos"])]
    before = [x.clone() for x in t]
    o1, l1 = host(*qsa.sparse_prefill_pool(*t))
    o2, l2 = host(*qsa.sparse_prefill_pool(*t))
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    for x, y in zip(t, before):
        assert torch.equal(x, y)


def test_pool_edge_cases():
    rng = np.random.default_rng(12)
    k, v = rand_bf16(rng, (30, 2, 256)), rand_bf16(rng, (30, 2, 256))
    slot_pos = rng.permutation(30).astype(np.int32)
    # no query rows
    o, l = run_pool(np.zeros((0, 4, 256), np.uint16), k, v, np.zeros((0, 2, 5), np.int32),
                    np.zeros(0, np.int32), slot_pos)
    assert o.shape == (0, 4, 256) and l.shape == (0, 4)
    q = rand_bf16(rng, (6, 4, 256))
    q_pos = np.array([0, 5, 29, -1, 100, 3], np.int32)  # a negative position sees nothing
    idx = rng.integers(-2, 33, size=(6, 2, 9)).astype(np.int32)
    out, lse = run_pool(q, k, v, idx, q_pos, slot_pos)
    ref_out, ref_lse = oracle.sparse_prefill_pool(q, k, v, idx, q_pos, slot_pos)
    compare(out, lse, ref_out, ref_lse, label="pool edge")
    assert np.all(np.isneginf(lse[3]))
    # zero selection width
    out, lse = run_pool(q, k, v, np.zeros((6, 2, 0), np.int32), q_pos, slot_pos)
    assert np.all(out == 0) and np.all(np.isneginf(lse))
    # an empty pool: every listed slot is outside it
    empty = np.zeros((0, 2, 256), np.uint16)
    out, lse = run_pool(q, empty, empty, idx, q_pos, np.zeros(0, np.int32))
    assert np.all(out == 0) and np.all(np.isneginf(lse))
    out, lse = run_decode(q, empty, empty, idx, q_pos, np.zeros(0, np.int32))
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_pool_binding_validates():
    rng = np.random.default_rng(13)
    q, k = dev_bf16(rand_bf16(rng, (3, 2, 256))), dev_bf16(rand_bf16(rng, (8, 1, 256)))
    idx = dev_i32(np.zeros((3, 1, 2)))
    with pytest.raises(ValueError):
        qsa.sparse_prefill_pool(q, k, k, idx, dev_i32(np.zeros(2)), dev_i32(np.zeros(8)))
    with pytest.raises(ValueError):
        qsa.sparse_prefill_pool(q, k, k, idx, dev_i32(np.zeros(3)), dev_i32(np.zeros(7)))
    with pytest.raises(TypeError):
        qsa.sparse_prefill_pool(q, k, k, idx, dev_i32(np.zeros(3)).long(), dev_i32(np.zeros(8)))


# ------------------------------------------------------------------ decode


def run_decode(q, k, v, idx, q_pos, slot_pos, scale=None, workspace=None):
    return host(*qsa.sparse_decode(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_i32(idx), dev_i32(q_pos),
                                   dev_i32(slot_pos), scale=scale, workspace=workspace))


@pytest.mark.parametrize("number", [11, 12])
def test_decode_workloads_all_rows(number):
    t0 = time.perf_counter()
    d = make_pool_inputs(number)
    cfg = d["cfg"]
    args = (d["q"], d["k"], d["v"], d["idx"], d["q_pos"], d["slot_pos"])
    n_ws = qsa.decode_workspace_bytes(cfg.total_q, cfg.Hq, cfg.Hkv, cfg.K)
    progress(f"{cfg.name}: inputs in {time.perf_counter() - t0:.1f}s, workspace {n_ws} B")
    assert n_ws > 0  # these batches are small enough to be cut
    out, lse = run_decode(*args, scale=cfg.scale)
    rows = np.arange(cfg.total_q)
    ref_out, ref_lse = oracle_pool.run_rows(d["q"], d["k"], d["v"], d["idx"], rows, cfg.scale, q_pos=d["q_pos"],
                                            slot_pos=d["slot_pos"])
    stats = compare(out, lse, ref_out, ref_lse, label=cfg.name)
    progress(f"{cfg.name}: {stats} ({time.perf_counter() - t0:.1f}s)")
    # the same rows through the unsplit pool kernel agree with it to rounding
    po, pl = run_pool(*args, scale=cfg.scale)
    compare(po, pl, ref_out, ref_lse, label=cfg.name + " pool")
    # deterministic: a second call is identical
    out2, lse2 = run_decode(*args, scale=cfg.scale)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


def test_decode_sparse_and_empty_ranges():
    """Lists of 2,051 slots with only a handful valid: most ranges of the
    split are empty (weight 0 in the merge); one row is empty altogether and
    one has a negative position."""
    rng = np.random.default_rng(30)
    n_slots, K = 5000, 2051
    k, v = rand_bf16(rng, (n_slots, 2, 256)), rand_bf16(rng, (n_slots, 2, 256))
    slot_pos = rng.permutation(n_slots).astype(np.int32)
    q = rand_bf16(rng, (3, 8, 256))
    q_pos = np.array([4000, 4999, -1], np.int32)
    idx = np.full((3, 2, K), -1, np.int32)
    for r in range(3):
        for g in range(2):
            where = rng.choice(K, size=7, replace=False)
            idx[r, g, where] = rng.choice(n_slots, size=7, replace=False)
    idx[1, 1, :] = -1  # KV head 1 of row 1: no slot at all
    out, lse = run_decode(q, k, v, idx, q_pos, slot_pos)
    ref_out, ref_lse = oracle.sparse_prefill_pool(q, k, v, idx, q_pos, slot_pos)
    compare(out, lse, ref_out, ref_lse, label="decode sparse")
    assert np.all(np.isneginf(lse[1, 4:])) and np.all(np.isneginf(lse[2]))


@pytest.mark.parametrize("n_req,K", [(1, 2048), (1, 17), (3, 100), (40, 2048), (700, 64)])
def test_decode_shapes(n_req, K):
    rng = np.random.default_rng(n_req * 7 + K)
    n_slots = 3000
    k, v = rand_bf16(rng, (n_slots, 1, 256)), rand_bf16(rng, (n_slots, 1, 256))
    slot_pos = rng.permutation(n_slots).astype(np.int32)
    q = rand_bf16(rng, (n_req, 12, 256))
    q_pos = rng.integers(0, n_slots, size=n_req).astype(np.int32)
    idx = rng.integers(-5, n_slots + 5, size=(n_req, 1, K)).astype(np.int32)
    out, lse = run_decode(q, k, v, idx, q_pos, slot_pos)
    ref_out, ref_lse = oracle.sparse_prefill_pool(q, k, v, idx, q_pos, slot_pos)
    compare(out, lse, ref_out, ref_lse, label=f"decode n_req={n_req} K={K}")


def test_decode_workspace_reuse_and_checks():
    """One workspace serves consecutive calls of different sizes; a workspace
    below the required size is refused before anything runs."""
    d = make_pool_inputs(11)
    cfg = d["cfg"]
    need = qsa.decode_workspace_bytes(cfg.total_q, cfg.Hq, cfg.Hkv, cfg.K)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    args = (d["q"], d["k"], d["v"], d["idx"], d["q_pos"], d["slot_pos"])
    a = run_decode(*args, workspace=ws)
    b = run_decode(*(x[:2] if i in (0, 3, 4) else x for i, x in enumerate(args)), workspace=ws)
    fresh = run_decode(*(x[:2] if i in (0, 3, 4) else x for i, x in enumerate(args)))
    np.testing.assert_array_equal(b[0], fresh[0])
    np.testing.assert_array_equal(b[1], fresh[1])
    assert a[0].shape[0] == 4
    with pytest.raises(qsa.QsaError):
        run_decode(*args, workspace=ws[: need - 16])


# ------------------------------------------------------------------ largest caches


QSA_MAX_KV_ROWS = 4194303  # include/qsa.h: T_kv * Hkv * 512 bytes must stay below 2^31


def _reference_rows(q, k_rows, v_rows, lists, positions, scale):
    """Oracle outputs from the oracle's own per-row steps, with K/V given only
    for the rows that may be read (dicts position -> bf16 bits [Hkv, 256])."""
    T, Hq = q.shape[0], q.shape[1]
    Hkv = lists.shape[1]
    G = Hq // Hkv
    out = np.zeros((T, Hq, 256))
    lse = np.full((T, Hq), -np.inf)
    for i in range(T):
        q_t = oracle.bf16_to_f64(q[i])
        for g in range(Hkv):
            sel = positions(lists[i, g], i)
            k_sel = np.stack([oracle.bf16_to_f64(k_rows[s][g]) for s in sel]) if sel else np.zeros((0, 256))
            v_sel = np.stack([oracle.bf16_to_f64(v_rows[s][g]) for s in sel]) if sel else np.zeros((0, 256))
            for h in range(g * G, (g + 1) * G):
                o, l, _ = oracle.attend(q_t[h], k_sel, v_sel, scale)
                out[i, h], lse[i, h] = o, l
    return out, lse


def _device_kv(n_rows, Hkv, seed):
    gen = torch.Generator(device="cuda").manual_seed(seed)
    k = torch.randn((n_rows, Hkv, 256), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn((n_rows, Hkv, 256), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    return k, v


def _rows_to_host(t, rows):
    rows = sorted(set(int(r) for r in rows))
    idx = torch.tensor(rows, dtype=torch.int64, device="cuda")
    got = torch_bf16_to_numpy_bits(t.index_select(0, idx))
    return {r: got[i] for i, r in enumerate(rows)}


@pytest.mark.parametrize("Hkv", [1, 2])
def test_extend_at_the_largest_cache(Hkv):
    """T_kv * Hkv = QSA_MAX_KV_ROWS: the last K/V rows sit just below 2^31
    bytes; the lists name them, rows near 2^21 and 2^22, and random ones."""
    T_kv = QSA_MAX_KV_ROWS // Hkv
    T, Hq, K = 48, 6 * Hkv, 320
    p0 = T_kv - T
    progress(f"largest cache: T_kv={T_kv}, Hkv={Hkv} ({2 * T_kv * Hkv * 512 / 2**30:.2f} GiB of K/V)")
    k, v = _device_kv(T_kv, Hkv, seed=900 + Hkv)
    rng = np.random.default_rng(901 + Hkv)
    q = rand_bf16(rng, (T, Hq, 256))
    idx = np.full((T, Hkv, K), -1, np.int32)
    for t in range(T):
        pos = p0 + t
        for g in range(Hkv):
            fixed = [pos, pos - 1, T_kv - 1, T_kv - T - 1, (1 << 22) - 1, 1 << 21, 0, T_kv, T_kv + 5]
            rand = list(rng.integers(0, pos + 1, size=K - len(fixed) - 20))
            row = np.array(fixed + rand + [-1] * 20, np.int64)
            rng.shuffle(row)
            idx[t, g] = row
    out, lse = host(*qsa.sparse_prefill_extend(dev_bf16(q), k, v, dev_i32(idx), p0))
    used = idx[(idx >= 0) & (idx < T_kv)]
    k_rows, v_rows = _rows_to_host(k, used), _rows_to_host(v, used)
    del k, v
    torch.cuda.empty_cache()
    ref_out, ref_lse = _reference_rows(q, k_rows, v_rows, idx,
                                       lambda lst, i: oracle.selected_positions(lst, p0 + i), 1 / 16)
    progress(f"largest cache Hkv={Hkv}: {compare(out, lse, ref_out, ref_lse, label='largest cache')}")


def test_pool_and_decode_at_the_largest_pool():
    """A pool of QSA_MAX_KV_ROWS slots (one KV head): rows in the last slots,
    positions permuted over the whole pool."""
    n_slots, Hq, K = QSA_MAX_KV_ROWS, 8, 260
    k, v = _device_kv(n_slots, 1, seed=910)
    rng = np.random.default_rng(911)
    slot_pos = np.full(n_slots, -1, np.int32)
    live = rng.choice(n_slots, size=100000, replace=False)
    live[:4] = [n_slots - 1, n_slots - 2, n_slots - 3, 0]
    slot_pos[live] = rng.integers(0, 50000, size=live.size)
    T = 24
    q = rand_bf16(rng, (T, Hq, 256))
    q_pos = rng.integers(20000, 50000, size=T).astype(np.int32)
    idx = np.full((T, 1, K), -1, np.int32)
    for t in range(T):
        row = list(live[:4]) + list(rng.choice(live, size=K - 14)) + [n_slots, -3] + [-1] * 8
        idx[t, 0] = np.array(row[:K], np.int64)
    args = (dev_bf16(q), k, v, dev_i32(idx), dev_i32(q_pos), dev_i32(slot_pos))
    out, lse = host(*qsa.sparse_prefill_pool(*args))
    dout, dlse = host(*qsa.sparse_decode(*args))
    used = idx[(idx >= 0) & (idx < n_slots)]
    k_rows, v_rows = _rows_to_host(k, used), _rows_to_host(v, used)
    del k, v, args
    torch.cuda.empty_cache()
    ref_out, ref_lse = _reference_rows(q, k_rows, v_rows, idx,
                                       lambda lst, i: oracle.pool_selected_slots(lst, int(q_pos[i]), slot_pos),
                                       1 / 16)
    compare(out, lse, ref_out, ref_lse, label="largest pool")
    compare(dout, dlse, ref_out, ref_lse, label="largest pool, decode")


@pytest.mark.parametrize("hq,hkv", [(40, 2), (17, 1), (32, 1)])
def test_decode_and_blocks_with_several_head_chunks(hq, hkv):
    """More than 16 query heads per KV head: each list is computed by several
    waves (16 heads each), and in decode each of those by several ranges."""
    rng = np.random.default_rng(hq * 10 + hkv)
    n_slots, K, n_req = 2000, 700, 5
    k, v = rand_bf16(rng, (n_slots, hkv, 256)), rand_bf16(rng, (n_slots, hkv, 256))
    slot_pos = rng.permutation(n_slots).astype(np.int32)
    q = rand_bf16(rng, (n_req, hq, 256))
    q_pos = rng.integers(500, n_slots, size=n_req).astype(np.int32)
    idx = rng.integers(-3, n_slots + 3, size=(n_req, hkv, K)).astype(np.int32)
    assert qsa.decode_workspace_bytes(n_req, hq, hkv, K) > 0
    out, lse = run_decode(q, k, v, idx, q_pos, slot_pos)
    ref_out, ref_lse = oracle.sparse_prefill_pool(q, k, v, idx, q_pos, slot_pos)
    compare(out, lse, ref_out, ref_lse, label=f"decode ({hq},{hkv})")
    # micro-blocks with the same head shape
    T = 70
    qb = rand_bf16(rng, (T, hq, 256))
    kb, vb = rand_bf16(rng, (T, hkv, 256)), rand_bf16(rng, (T, hkv, 256))
    bidx = rng.integers(-1, T // 4 + 2, size=(T, hkv, 9)).astype(np.int32)
    out, lse = run_blocks(qb, kb, vb, bidx, 4)
    ref_out, ref_lse = oracle.sparse_prefill_blocks(qb, kb, vb, bidx, 4)
    compare(out, lse, ref_out, ref_lse, label=f"blocks ({hq},{hkv})")


def test_pool_extreme_positions():
    """Query positions and slot positions at the int32 extremes."""
    rng = np.random.default_rng(77)
    n_slots = 64
    k, v = rand_bf16(rng, (n_slots, 1, 256)), rand_bf16(rng, (n_slots, 1, 256))
    slot_pos = rng.integers(0, 1000, size=n_slots).astype(np.int32)
    slot_pos[:4] = [INT32_MAX, INT32_MIN, INT32_MAX - 1, 0]
    q = rand_bf16(rng, (5, 3, 256))
    q_pos = np.array([INT32_MAX, INT32_MAX - 1, INT32_MIN, 0, 999], np.int32)
    idx = np.tile(np.arange(n_slots, dtype=np.int32), (5, 1, 1))
    out, lse = run_pool(q, k, v, idx, q_pos, slot_pos)
    ref_out, ref_lse = oracle.sparse_prefill_pool(q, k, v, idx, q_pos, slot_pos)
    compare(out, lse, ref_out, ref_lse, label="pool extremes")
    assert np.all(np.isneginf(lse[2]))


QSA_MAX_LIST = 1 << 28  # include/qsa.h: the widest index list accepted


def test_widest_index_list():
    """K = 2^28 entries per list, the widest the ABI accepts: each (row, KV
    head) list is 1 GiB of int32, its entries addressed with byte offsets up to
    2^30. The few usable entries sit at the very end of the lists, at 2^27 and
    near the start, among pads, other negatives and a future position; a wave
    walks all 2^24 tiles of its list. The oracle gets the same entries in the
    same order without the pads (pads change nothing: pinned)."""
    T, Hq, Hkv, K = 2, 4, 1, QSA_MAX_LIST
    rng = np.random.default_rng(930)
    q, k, v = rand_bf16(rng, (T, Hq, 256)), rand_bf16(rng, (T, Hkv, 256)), rand_bf16(rng, (T, Hkv, 256))
    # (list position, entry) per row; every other position holds -1
    entries = [[(12345, 0), (K - 2, 1), (K - 1, 0)],             # 1 is after row 0: masked
               [(5, -7), (1 << 27, 1), (K - 17, 0), (K - 1, 1)]]
    idx = torch.full((T, Hkv, K), -1, dtype=torch.int32, device="cuda")
    short = np.full((T, Hkv, 4), -1, np.int32)
    for t, row in enumerate(entries):
        for i, (at, val) in enumerate(row):
            idx[t, 0, at] = val
            short[t, 0, i] = val
    progress(f"widest list: K = 2^28 ({T * K * 4 / 2**30:.0f} GiB of indices), one wave per row walks 2^24 tiles")
    t0 = time.time()
    out, lse = host(*qsa.sparse_prefill(dev_bf16(q), dev_bf16(k), dev_bf16(v), idx))
    secs = time.time() - t0
    del idx
    torch.cuda.empty_cache()
    ref_out, ref_lse = oracle.sparse_prefill(q, k, v, short)
    progress(f"widest list: {secs:.1f} s; {compare(out, lse, ref_out, ref_lse, label='K = 2^28')}")


# ------------------------------------------------------------------ graph capture


def test_calls_replay_from_a_captured_graph():
    """The entry points allocate nothing and never synchronise, so they can be
    captured in a HIP graph. Every replay (with eager work and a sync between
    replays) must equal the eager results bit for bit."""
    rng = np.random.default_rng(55)
    T, n_slots = 200, 600
    q = dev_bf16(rand_bf16(rng, (T, 6, 256)))
    k, v = dev_bf16(rand_bf16(rng, (T, 2, 256))), dev_bf16(rand_bf16(rng, (T, 2, 256)))
    idx = dev_i32(rng.integers(-2, T + 2, size=(T, 2, 70)))
    kp, vp = dev_bf16(rand_bf16(rng, (n_slots, 2, 256))), dev_bf16(rand_bf16(rng, (n_slots, 2, 256)))
    slot_pos = dev_i32(rng.permutation(n_slots))
    qd = dev_bf16(rand_bf16(rng, (3, 6, 256)))
    q_pos = dev_i32(np.array([500, 20, 599]))
    sidx = dev_i32(rng.integers(-2, n_slots + 2, size=(3, 2, 300)))
    ws = torch.empty(max(qsa.decode_workspace_bytes(3, 6, 2, 300), 16), dtype=torch.uint8, device="cuda")
    outs = [torch.empty((T, 6, 256), dtype=torch.bfloat16, device="cuda"),
            torch.empty((T, 6), dtype=torch.float32, device="cuda"),
            torch.empty((3, 6, 256), dtype=torch.bfloat16, device="cuda"),
            torch.empty((3, 6), dtype=torch.float32, device="cuda")]

    def calls():
        qsa.sparse_prefill(q, k, v, idx, out=outs[0], lse=outs[1])
        qsa.sparse_decode(qd, kp, vp, sidx, q_pos, slot_pos, out=outs[2], lse=outs[3], workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    for rep in range(4):
        for o in outs:
            o.fill_(7.0)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {rep} differs from the eager result"


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_concurrent_calls_on_two_streams():
    """Calls on different streams may run at the same time (the library keeps
    no state): a prefill on one stream and a decode on another, each with its
    own outputs and workspace, launched back to back several times, equal the
    serial results bit for bit."""
    rng = np.random.default_rng(77)
    T, n_slots = 2048, 5000
    q = dev_bf16(rand_bf16(rng, (T, 12, 256)))
    k, v = dev_bf16(rand_bf16(rng, (T, 1, 256))), dev_bf16(rand_bf16(rng, (T, 1, 256)))
    idx = dev_i32(rng.integers(-2, T + 2, size=(T, 1, 256)))
    kp, vp = dev_bf16(rand_bf16(rng, (n_slots, 2, 256))), dev_bf16(rand_bf16(rng, (n_slots, 2, 256)))
    slot_pos = dev_i32(rng.permutation(n_slots))
    qd = dev_bf16(rand_bf16(rng, (8, 6, 256)))
    q_pos = dev_i32(rng.integers(0, n_slots, 8))
    sidx = dev_i32(rng.integers(-2, n_slots + 2, size=(8, 2, 1024)))
    ref = [*qsa.sparse_prefill(q, k, v, idx), *qsa.sparse_decode(qd, kp, vp, sidx, q_pos, slot_pos)]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    results = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            p = qsa.sparse_prefill(q, k, v, idx)
        with torch.cuda.stream(s2):
            d = qsa.sparse_decode(qd, kp, vp, sidx, q_pos, slot_pos)
        results.append([*p, *d])
    torch.cuda.synchronize()
    for rep, res in enumerate(results):
        for got, want in zip(res, ref):
            assert torch.equal(_bits(got), _bits(want)), f"call {rep} on two streams differs from the serial result"
