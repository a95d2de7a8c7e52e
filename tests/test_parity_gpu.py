"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle.

Inputs are the seeded synthetic workloads and hand-built edge cases; the
comparison bar is in tests/parity.py. The cases mirror the operator tests
the pages list for the Ascend path ("Qwen4-Exp QSA llega al Ascend de
Huawei", section "Nueve pruebas que pasaron"): selection widths 1/63/64/65/
2051 with unordered slots, default and explicit scales, fully masked rows,
zero rows, zero selection width, non-contiguous inputs, causal tails with
compression ratio 4, cache-content reuse, the local head shapes at 1 and 257
query rows, and the long prefill against a longer cache.
"""
import json
import os
import sys
import time

import numpy as np
import pytest

import oracle
from oracle import pool as oracle_pool
from qsa_inputs import CONFIGS, EXTEND_CONFIG, f32_to_bf16_bits, get_config, make_indices, make_qkv, sample_rows
from tests.parity import compare, torch_bf16_to_numpy_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import top_sparse_attention_qsa_amd as qsa  # noqa: E402

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_test_matrix.json")))
INT32_MIN = -(2 ** 31)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X: no HIP device visible")
    qsa.load_library()  # fails loudly when libqsa.so is missing
    return torch.device("cuda", 0)


def dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a)).view(torch.bfloat16).to("cuda")


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda")


def run(q, k, v, idx, scale=None, q_pos0=None):
    args = (dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_i32(idx))
    if q_pos0 is None:
        out, lse = qsa.sparse_prefill(*args, scale=scale)
    else:
        out, lse = qsa.sparse_prefill_extend(*args, q_pos0=q_pos0, scale=scale)
    torch.cuda.synchronize()
    return torch_bf16_to_numpy_bits(out), lse.cpu().numpy()


def rand_bf16(rng, shape, sigma=1.0):
    return f32_to_bf16_bits((rng.standard_normal(shape) * sigma).astype(np.float32))


def rand_lists(rng, T, Hkv, K, p0=0, pad_frac=0.15, future_frac=0.05):
    """Unordered lists: distinct positions <= p0 + t, some -1 and some future
    slots mixed in anywhere."""
    idx = np.full((T, Hkv, K), -1, np.int32)
    for t in range(T):
        pos = p0 + t
        for g in range(Hkv):
            n_valid = min(pos + 1, K)
            n_valid = max(1, n_valid - int(rng.binomial(n_valid, pad_frac)))
            row = list(rng.choice(pos + 1, size=n_valid, replace=False))
            n_rest = K - n_valid
            n_future = int(rng.binomial(n_rest, future_frac)) if n_rest else 0
            row += [pos + 1 + int(x) for x in rng.integers(0, 50, n_future)]
            row += [-1] * (n_rest - n_future)
            rng.shuffle(row)
            idx[t, g] = row
    return idx


def progress(msg):
    sys.__stdout__.write(f"    {time.strftime('%H:%M:%S')} {msg}\n")
    sys.__stdout__.flush()


def check(q, k, v, idx, scale=None, rows=None, q_pos0=0, label="", workers=None):
    t0 = time.perf_counter()
    out, lse = run(q, k, v, idx, scale=scale, q_pos0=q_pos0 if q_pos0 else None)
    sc = 1 / 16 if scale is None else scale
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    big = rows.size * q.shape[1] * idx.shape[2] > 2_000_000
    if big:
        progress(f"{label}: gpu done in {time.perf_counter() - t0:.1f}s; oracle on {rows.size} rows")
        ref_out, ref_lse = oracle_pool.run_rows(q, k, v, idx[rows], rows, sc, q_pos0=q_pos0, workers=workers)
    else:
        ref_out, ref_lse = oracle.sparse_prefill(q, k, v, idx[rows], scale=sc, rows=rows, q_pos0=q_pos0)
    stats = compare(out[rows], lse[rows], ref_out, ref_lse, label=label)
    progress(f"{label}: {stats} ({time.perf_counter() - t0:.1f}s)")
    return out, lse, stats


# ------------------------------------------------------------------ workloads


@pytest.mark.parametrize("number", [1, 2])
def test_workload_all_rows(number):
    cfg = get_config(number)
    q, k, v = make_qkv(cfg)
    idx = make_indices(cfg)
    check(q, k, v, idx, scale=cfg.scale, label=cfg.name)


@pytest.mark.parametrize("number", [3, 4, 5, 6])
def test_workload_full_size(number):
    """The full-size workloads, checked on every row (the two T = 32,768
    workloads and the extend workload) or on 4,096 seeded rows plus the
    edge rows (the 235,008-token workload); every output finite."""
    cfg = get_config(number)
    t0 = time.perf_counter()
    progress(f"{cfg.name}: generating inputs ({oracle_pool.default_workers()} workers, "
             f"{os.cpu_count()} cpus)")
    q, k, v = make_qkv(cfg)
    progress(f"{cfg.name}: q/k/v in {time.perf_counter() - t0:.1f}s")
    idx = make_indices(cfg)
    progress(f"{cfg.name}: idx in {time.perf_counter() - t0:.1f}s")
    rows = sample_rows(cfg)
    assert rows.size == (4096 + 6 if number == 5 else cfg.T)
    out, lse, stats = check(q, k, v, idx, scale=cfg.scale, rows=rows, q_pos0=cfg.q_pos0, label=cfg.name)
    g = out.view(np.uint16)
    # every output finite (bf16 exponent not all ones) and every row non-empty
    assert not np.any((g & 0x7F80) == 0x7F80), "non-finite output"
    assert np.all(np.isfinite(lse))
    assert stats["rel_l2"] < GOLDEN["thresholds"]["rel_l2_below"]


# ------------------------------------------------------------------ pages' test matrix


@pytest.mark.parametrize("K", GOLDEN["selection_widths"]["values"])
def test_selection_widths_unordered(K):
    rng = np.random.default_rng(K)
    T = 300 if K < 1000 else 2200
    q, k, v = rand_bf16(rng, (T, 6, 256)), rand_bf16(rng, (T, 2, 256)), rand_bf16(rng, (T, 2, 256))
    idx = rand_lists(rng, T, 2, K)
    rows = None if K < 1000 else np.unique(np.concatenate([np.arange(0, T, 9), [T - 1]]))
    check(q, k, v, idx, rows=rows, label=f"width{K}")


@pytest.mark.parametrize("scale", [None, 0.1, 0.0, -0.07, 1 / 256, 0.25])
def test_default_and_explicit_scales(scale):
    rng = np.random.default_rng(7)
    T = 160
    q, k, v = rand_bf16(rng, (T, 8, 256)), rand_bf16(rng, (T, 2, 256)), rand_bf16(rng, (T, 2, 256))
    idx = rand_lists(rng, T, 2, 70)
    check(q, k, v, idx, scale=scale, label=f"scale{scale}")


@pytest.mark.parametrize("kind", ["all_minus1", "all_future", "int32_min", "width0", "mixed"])
def test_fully_masked_rows(kind):
    rng = np.random.default_rng(3)
    T, K = 96, (0 if kind == "width0" else 40)
    q, k, v = rand_bf16(rng, (T, 3, 256)), rand_bf16(rng, (T, 1, 256)), rand_bf16(rng, (T, 1, 256))
    if kind == "all_minus1":
        idx = np.full((T, 1, K), -1, np.int32)
    elif kind == "int32_min":
        idx = np.full((T, 1, K), INT32_MIN, np.int32)
    elif kind == "all_future":
        idx = (np.arange(T)[:, None, None] + 1 + np.arange(K)[None, None, :]).astype(np.int32)
    elif kind == "width0":
        idx = np.zeros((T, 1, 0), np.int32)
    else:
        idx = rand_lists(rng, T, 1, K)
        idx[::3] = -1
    out, lse, _ = check(q, k, v, idx, label=kind)
    if kind != "mixed":
        assert np.all(out.view(np.uint16) == 0) and np.all(np.isneginf(lse))


def test_zero_tokens():
    q = torch.zeros(0, 4, 256, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(0, 2, 256, dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros(0, 2, 16, dtype=torch.int32, device="cuda")
    out, lse = qsa.sparse_prefill(q, k, k, idx)
    assert out.shape == (0, 4, 256) and lse.shape == (0, 4)


def test_zero_query_rows_give_the_mean():
    rng = np.random.default_rng(4)
    T = 120
    q = rand_bf16(rng, (T, 6, 256))
    q[::2] = 0
    k, v = rand_bf16(rng, (T, 2, 256)), rand_bf16(rng, (T, 2, 256))
    idx = rand_lists(rng, T, 2, 48)
    check(q, k, v, idx, label="zero_q")


def test_non_contiguous_inputs_equal_contiguous():
    rng = np.random.default_rng(5)
    T = 130
    q, k, v = rand_bf16(rng, (T, 6, 256)), rand_bf16(rng, (T, 2, 256)), rand_bf16(rng, (T, 2, 256))
    idx = rand_lists(rng, T, 2, 33)
    out_c, lse_c = run(q, k, v, idx)
    # the same values seen through strided / transposed views
    qt = dev_bf16(np.ascontiguousarray(q.transpose(1, 0, 2))).transpose(0, 1)
    kb = dev_bf16(np.concatenate([k, k], axis=2))[:, :, :256]
    vt = dev_bf16(np.ascontiguousarray(v.transpose(1, 0, 2))).transpose(0, 1)
    it = dev_i32(np.ascontiguousarray(idx.transpose(2, 0, 1))).permute(1, 2, 0)
    assert not (qt.is_contiguous() or kb.is_contiguous() or vt.is_contiguous() or it.is_contiguous())
    out, lse = qsa.sparse_prefill(qt, kb, vt, it)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(torch_bf16_to_numpy_bits(out), out_c)
    np.testing.assert_array_equal(lse.cpu().numpy(), lse_c)


@pytest.mark.parametrize("rem", GOLDEN["causal_tail"]["remainders"])
def test_causal_tail_micro_blocks(rem):
    """Lists of whole 4-token micro-blocks (compression ratio 4): the block
    holding t reaches up to 3 positions past t, which must be masked."""
    rng = np.random.default_rng(40 + rem)
    ratio = GOLDEN["causal_tail"]["compression_ratio"]
    T = 4 * 50 + rem
    q, k, v = rand_bf16(rng, (T, 4, 256)), rand_bf16(rng, (T, 1, 256)), rand_bf16(rng, (T, 1, 256))
    n_blocks = 12
    idx = np.full((T, 1, n_blocks * ratio), -1, np.int32)
    for t in range(T):
        own = t // ratio
        others = rng.choice(own, size=min(own, n_blocks - 1), replace=False) if own else []
        blocks = np.concatenate([[own], others]).astype(np.int64)
        rng.shuffle(blocks)
        pos = (blocks[:, None] * ratio + np.arange(ratio)[None, :]).ravel()
        idx[t, 0, : pos.size] = pos
    check(q, k, v, idx, label=f"tail{rem}")


@pytest.mark.parametrize("hq,hkv", [tuple(p) for p in GOLDEN["head_pairs"]["values"]])
@pytest.mark.parametrize("T", GOLDEN["query_rows"]["values"])
def test_local_head_shapes(hq, hkv, T):
    rng = np.random.default_rng(hq * 1000 + hkv * 10 + T)
    q, k, v = rand_bf16(rng, (T, hq, 256)), rand_bf16(rng, (T, hkv, 256)), rand_bf16(rng, (T, hkv, 256))
    idx = rand_lists(rng, T, hkv, 80)
    check(q, k, v, idx, label=f"heads{hq}x{hkv}_T{T}")


@pytest.mark.parametrize("hq,hkv", [(4, 4), (16, 1), (40, 2), (32, 1), (17, 1), (1, 1)])
def test_other_group_sizes(hq, hkv):
    rng = np.random.default_rng(hq + 100 * hkv)
    T = 70
    q, k, v = rand_bf16(rng, (T, hq, 256)), rand_bf16(rng, (T, hkv, 256)), rand_bf16(rng, (T, hkv, 256))
    idx = rand_lists(rng, T, hkv, 37)
    check(q, k, v, idx, label=f"group{hq}x{hkv}")


def test_repeated_positions_count_per_entry():
    rng = np.random.default_rng(6)
    T = 64
    q, k, v = rand_bf16(rng, (T, 3, 256)), rand_bf16(rng, (T, 1, 256)), rand_bf16(rng, (T, 1, 256))
    idx = np.stack([rng.integers(0, t + 1, 24) for t in range(T)])[:, None, :].astype(np.int32)
    check(q, k, v, idx, label="repeats")


def test_large_logits_and_outlier_rows():
    """Rows scaled x8 (as in the outlier workload) and large explicit scales."""
    rng = np.random.default_rng(8)
    T = 200
    q, k, v = rand_bf16(rng, (T, 8, 256)), rand_bf16(rng, (T, 1, 256), 1.0), rand_bf16(rng, (T, 1, 256))
    sel = rng.choice(T, 20, replace=False)
    k32 = (k.astype(np.uint32) << 16).view(np.float32)
    v32 = (v.astype(np.uint32) << 16).view(np.float32)
    k32[sel] *= 8
    v32[sel] *= 8
    k, v = f32_to_bf16_bits(k32), f32_to_bf16_bits(v32)
    idx = rand_lists(rng, T, 1, 96)
    for scale in (1 / 16, 0.5):
        check(q, k, v, idx, scale=scale, label=f"outliers_scale{scale}")


# ------------------------------------------------------------------ index handling


def test_bit_stable_index_handling():
    """Two runs are bitwise equal, and swapping one masked value for another
    (-1, t+1, T, INT32_MIN, -7) at the same slots changes no bit."""
    rng = np.random.default_rng(9)
    T, K = 250, 70
    q, k, v = rand_bf16(rng, (T, 12, 256)), rand_bf16(rng, (T, 1, 256)), rand_bf16(rng, (T, 1, 256))
    idx = rand_lists(rng, T, 1, K, pad_frac=0.3, future_frac=0.0)
    base_out, base_lse = run(q, k, v, idx)
    again_out, again_lse = run(q, k, v, idx)
    np.testing.assert_array_equal(base_out, again_out)
    np.testing.assert_array_equal(base_lse, again_lse)
    masked = idx < 0
    tt = np.broadcast_to(np.arange(T)[:, None, None], idx.shape)
    for repl in ("next", "T", "min", "neg7"):
        alt = idx.copy()
        alt[masked] = {"next": (tt + 1)[masked], "T": np.full(masked.sum(), T),
                       "min": np.full(masked.sum(), INT32_MIN), "neg7": np.full(masked.sum(), -7)}[repl]
        o, l = run(q, k, v, alt)
        np.testing.assert_array_equal(o, base_out, err_msg=repl)
        np.testing.assert_array_equal(l, base_lse, err_msg=repl)


def test_inputs_unchanged_and_cache_reuse():
    """K/V contents are only read: two calls sharing one cache agree bitwise,
    and every input is bit-identical afterwards."""
    rng = np.random.default_rng(10)
    T = 180
    q1, q2 = rand_bf16(rng, (T, 6, 256)), rand_bf16(rng, (T, 6, 256))
    k, v = rand_bf16(rng, (T, 2, 256)), rand_bf16(rng, (T, 2, 256))
    idx = rand_lists(rng, T, 2, 50)
    dq1, dq2, dk, dv, di = dev_bf16(q1), dev_bf16(q2), dev_bf16(k), dev_bf16(v), dev_i32(idx)
    snap = [t.clone() for t in (dq1, dq2, dk, dv, di)]
    o1, l1 = qsa.sparse_prefill(dq1, dk, dv, di)
    o2, l2 = qsa.sparse_prefill(dq2, dk, dv, di)
    o1b, l1b = qsa.sparse_prefill(dq1, dk, dv, di)
    torch.cuda.synchronize()
    for a, b in zip(snap, (dq1, dq2, dk, dv, di)):
        assert torch.equal(a, b)
    assert torch.equal(o1.view(torch.int16), o1b.view(torch.int16)) and torch.equal(l1, l1b)
    ref_out, ref_lse = oracle.sparse_prefill(q2, k, v, idx, scale=1 / 16)
    compare(torch_bf16_to_numpy_bits(o2), l2.cpu().numpy(), ref_out, ref_lse, label="second request")


# ------------------------------------------------------------------ extend over a cached prefix


@pytest.mark.parametrize("T,T_kv,p0", [(50, 400, 350), (64, 300, 100), (1, 2100, 2099), (257, 1000, 700)])
def test_extend_over_cached_prefix(T, T_kv, p0):
    rng = np.random.default_rng(T + T_kv)
    q = rand_bf16(rng, (T, 6, 256))
    k, v = rand_bf16(rng, (T_kv, 2, 256)), rand_bf16(rng, (T_kv, 2, 256))
    idx = rand_lists(rng, T, 2, 65, p0=p0)
    check(q, k, v, idx, q_pos0=p0, label=f"extend{T}_{T_kv}_{p0}")


def test_extend_equals_rows_of_full_prefill():
    rng = np.random.default_rng(11)
    T, p0 = 300, 211
    q, k, v = rand_bf16(rng, (T, 8, 256)), rand_bf16(rng, (T, 2, 256)), rand_bf16(rng, (T, 2, 256))
    idx = rand_lists(rng, T, 2, 90)
    full_out, full_lse = run(q, k, v, idx)
    ext_out, ext_lse = run(q[p0:], k, v, idx[p0:], q_pos0=p0)
    np.testing.assert_array_equal(ext_out, full_out[p0:])
    np.testing.assert_array_equal(ext_lse, full_lse[p0:])


# ------------------------------------------------------------------ API surface


def test_given_output_buffers_and_side_stream():
    rng = np.random.default_rng(12)
    T = 90
    q, k, v = rand_bf16(rng, (T, 4, 256)), rand_bf16(rng, (T, 1, 256)), rand_bf16(rng, (T, 1, 256))
    idx = rand_lists(rng, T, 1, 40)
    ref_out, ref_lse = run(q, k, v, idx)
    out = torch.full((T, 4, 256), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, 4), 7.0, dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    args = (dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_i32(idx))
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        o, l = qsa.sparse_prefill(*args, out=out, lse=lse)
    s.synchronize()
    assert o.data_ptr() == out.data_ptr() and l.data_ptr() == lse.data_ptr()
    np.testing.assert_array_equal(torch_bf16_to_numpy_bits(out), ref_out)
    np.testing.assert_array_equal(lse.cpu().numpy(), ref_lse)


def test_occupancy_modes_give_identical_bits():
    """The launch runs one or two blocks per CU depending on the cache length
    and the number of items; the arithmetic of every item is the same either
    way. The same queries (positions 32,768..65,535) and lists against a
    98,304-row cache (one block per CU) and against its first 65,536 rows (two
    blocks; no list reaches past them) give identical bits, for token and for
    micro-block lists."""
    rng = np.random.default_rng(91)
    T, p0, Hq, Hkv, K = 32768, 32768, 4, 1, 48
    q, k, v = rand_bf16(rng, (T, Hq, 256)), rand_bf16(rng, (98304, Hkv, 256)), rand_bf16(rng, (98304, Hkv, 256))
    idx = rng.integers(-1, p0 + T, size=(T, Hkv, K)).astype(np.int32)
    bidx = rng.integers(-1, (p0 + T) // 4, size=(T, Hkv, 16)).astype(np.int32)
    dq, dk, dv, didx, dbidx = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_i32(idx), dev_i32(bidx)
    results = {}
    for rows_kv in (98304, 65536):
        kk, vv = dk[:rows_kv], dv[:rows_kv]
        results[rows_kv] = (qsa.sparse_prefill_extend(dq, kk, vv, didx, q_pos0=p0),
                            qsa.sparse_prefill_blocks(dq, kk, vv, dbidx, p0, 4))
    torch.cuda.synchronize()
    for form in (0, 1):
        (o1, l1), (o2, l2) = results[98304][form], results[65536][form]
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), form
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), form
    rows = np.array([0, 1, 777, 20000, T - 1])
    o, l = results[98304][0]
    ref_out, ref_lse = oracle.sparse_prefill(q, k, v, idx[rows], scale=1 / 16, rows=rows, q_pos0=p0)
    compare(torch_bf16_to_numpy_bits(o)[rows], l.cpu().numpy()[rows], ref_out, ref_lse, label="one block per CU")
