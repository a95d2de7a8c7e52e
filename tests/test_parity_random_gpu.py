"""GPU parity on seeded random shapes, every entry point, against the oracle.

Each case draws a form (one sequence, an extend over a cached prefix,
micro-block lists of 2/4/8/16 tokens, a slot-pool batch, a decode step), the
head counts (1-4 KV heads, 1-40 query heads per KV head, so several 16-head
chunks too), the list width (0-300 entries, ragged against the 16-slot
tile), the query count and prefix, the scale, and lists that mix valid
entries with -1 pads, other negatives, positions or blocks after the query,
entries past the cache or pool, repeated entries and free pool slots. Every
row of every case is compared with the oracle at the bar of tests/parity.py.
The operator and its tested cases: "Qwen4-Exp QSA llega al Ascend de Huawei"
(orcarouter.ai, Spanish page), sections "Lo que realmente añade la pull
request" and "Nueve pruebas que pasaron".
"""
import numpy as np
import pytest

import oracle
from qsa_inputs import f32_to_bf16_bits
from tests.parity import compare, torch_bf16_to_numpy_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import top_sparse_attention_qsa_amd as qsa  # noqa: E402

INT32_MIN, INT32_MAX = -(2 ** 31), 2 ** 31 - 1
FORMS = ("tokens", "extend", "blocks", "pool", "decode")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X: no HIP device visible")
    qsa.load_library()


def bf16(rng, shape):
    return f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


def dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a)).view(torch.bfloat16).to("cuda")


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda")


def mixed_lists(rng, n_rows, Hkv, K, limit_of_row, space):
    """Lists of K entries per (row, KV head): valid entries in [0, limit] of
    each row, mixed with pads, other negatives, entries past the limit, past
    the space, INT32 extremes and repeats, in random order."""
    idx = np.empty((n_rows, Hkv, K), np.int64)
    for r in range(n_rows):
        lim = limit_of_row(r)
        for g in range(Hkv):
            kind = rng.integers(0, 9, size=K)
            vals = np.where(kind < 5, rng.integers(0, max(lim, 0) + 1, size=K), -1)
            vals = np.where(kind == 5, rng.integers(lim + 1, lim + 40, size=K), vals)
            vals = np.where(kind == 6, rng.choice([INT32_MIN, -7, INT32_MAX, space, space + 3], size=K), vals)
            if K > 1 and lim >= 0:
                rep = rng.integers(0, K, size=max(1, K // 8))
                vals[rep] = vals[rng.integers(0, K)]  # repeats (each entry counts)
            idx[r, g] = vals
    return np.clip(idx, INT32_MIN, INT32_MAX).astype(np.int32)


def run_case(seed):
    rng = np.random.default_rng(10_000 + seed)
    form = FORMS[seed % len(FORMS)]
    Hkv = int(rng.integers(1, 5))
    G = int(rng.choice([1, 2, 3, 6, 8, 12, 16, 17, 24, 40]))
    Hq = Hkv * G
    K = int(rng.choice([0, 1, 15, 16, 17, 63, 64, 65, int(rng.integers(2, 300))]))
    scale = float(rng.choice([1 / 16, 0.1, 0.03, -0.05]))
    if form in ("tokens", "extend", "blocks"):
        T = int(rng.integers(1, 120))
        p0 = 0 if form == "tokens" else int(rng.integers(0, 400))
        B = int(rng.choice([2, 4, 8, 16])) if form == "blocks" else 1
        T_kv = p0 + T + (0 if form == "tokens" else int(rng.integers(0, 60)))
        q, k, v = bf16(rng, (T, Hq, 256)), bf16(rng, (T_kv, Hkv, 256)), bf16(rng, (T_kv, Hkv, 256))
        idx = mixed_lists(rng, T, Hkv, K, lambda r: (p0 + r) // B, (T_kv + B - 1) // B)
        args = (dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_i32(idx))
        if form == "tokens":
            out, lse = qsa.sparse_prefill(*args, scale=scale)
            ref = oracle.sparse_prefill(q, k, v, idx, scale=scale)
        elif form == "extend":
            out, lse = qsa.sparse_prefill_extend(*args, q_pos0=p0, scale=scale)
            ref = oracle.sparse_prefill(q, k, v, idx, scale=scale, q_pos0=p0)
        else:
            out, lse = qsa.sparse_prefill_blocks(*args, p0, B, scale=scale)
            ref = oracle.sparse_prefill_blocks(q, k, v, idx, B, scale=scale, q_pos0=p0)
        label = f"seed {seed}: {form} T={T} T_kv={T_kv} p0={p0} B={B} ({Hq},{Hkv}) K={K} scale={scale}"
    else:
        n_slots = int(rng.integers(1, 600))
        rows = int(rng.integers(1, 6 if form == "decode" else 120))
        slot_pos = rng.integers(-1, 300, size=n_slots).astype(np.int32)  # -1: a free slot
        q_pos = rng.integers(-1, 320, size=rows).astype(np.int32)
        q, k, v = bf16(rng, (rows, Hq, 256)), bf16(rng, (n_slots, Hkv, 256)), bf16(rng, (n_slots, Hkv, 256))
        idx = mixed_lists(rng, rows, Hkv, K, lambda r: n_slots - 1, n_slots)
        args = (dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_i32(idx), dev_i32(q_pos), dev_i32(slot_pos))
        if form == "pool":
            out, lse = qsa.sparse_prefill_pool(*args, scale=scale)
        else:
            out, lse = qsa.sparse_decode(*args, scale=scale)
        ref = oracle.sparse_prefill_pool(q, k, v, idx, q_pos, slot_pos, scale=scale)
        label = f"seed {seed}: {form} rows={rows} slots={n_slots} ({Hq},{Hkv}) K={K} scale={scale}"
    torch.cuda.synchronize()
    compare(torch_bf16_to_numpy_bits(out), lse.cpu().numpy(), ref[0], ref[1], label=label)


@pytest.mark.parametrize("seed", range(100))
def test_random_shapes_every_form(seed):
    run_case(seed)
