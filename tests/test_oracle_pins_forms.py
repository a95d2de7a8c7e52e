"""Pins of the oracle's micro-block and slot-pool forms.

Micro-block lists: "Qwen4-Exp QSA llega al Ascend de Huawei" (orcarouter.ai,
Spanish page), section "Por qué QSA es la parte incómoda, en cifras" (the
indexer selects micro-blocks at a compression ratio of 4) and section "Nueve
pruebas que pasaron" (causal-tail remainders 0..3 at ratio 4). Slot pools:
the same section (unordered physical slots, two requests mapping a shared
prefix, cache reuse).

As for the token form, nothing here re-types the oracle: full lists reduce to
dense causal attention, which torch's fp64 scaled_dot_product_attention
computes independently; single-block and two-slot cases have closed forms;
tiny block and pool batches are compared with their exact value (50-digit
decimal arithmetic over the rows the form's rule admits, applied by hand);
and planted mistakes in the expansion and slot rules must trip a pin.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.qsa_oracle as qo
from qsa_inputs import f32_to_bf16_bits

D = 256
INT32_MIN = -(2 ** 31)
INT32_MAX = 2 ** 31 - 1


def _rand_bf16(rng, shape):
    return f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


def _sdpa_masked(q, k, v, allowed, scale, G):
    """torch fp64 attention of q [T, Hq, D] over k/v [S, Hkv, D] with a
    boolean [T, S] mask (True = attend); returns (out [T, Hq, D], lse [T, Hq])."""
    Q = torch.from_numpy(qo.bf16_to_f64(q)).permute(1, 0, 2)
    Kr = torch.from_numpy(qo.bf16_to_f64(k)).repeat_interleave(G, dim=1).permute(1, 0, 2)
    Vr = torch.from_numpy(qo.bf16_to_f64(v)).repeat_interleave(G, dim=1).permute(1, 0, 2)
    m = torch.from_numpy(allowed)
    out = F.scaled_dot_product_attention(Q, Kr, Vr, attn_mask=m, scale=scale)
    scores = torch.matmul(Q, Kr.transpose(1, 2).contiguous()) * scale
    lse = torch.logsumexp(scores.masked_fill(~m, float("-inf")), dim=-1)
    return out.permute(1, 0, 2).numpy(), lse.permute(1, 0).numpy()


# ------------------------------------------------------------------ micro-blocks


def _all_block_lists(rng, T, Hkv, n_kv_blocks, p0, extra_pad=3):
    """Every row lists every block of the cache, shuffled, padded with -1."""
    nb = n_kv_blocks + extra_pad
    idx = np.full((T, Hkv, nb), -1, np.int32)
    for t in range(T):
        for g in range(Hkv):
            row = np.full(nb, -1, np.int32)
            row[:n_kv_blocks] = np.arange(n_kv_blocks)
            rng.shuffle(row)
            idx[t, g] = row
    return idx


@pytest.mark.parametrize("B", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("T_kv,T,p0", [(37, 37, 0), (50, 13, 37), (64, 64, 0)])
def test_full_block_lists_match_causal_sdpa(B, T_kv, T, p0):
    """All blocks listed: every token <= the query's position is used once,
    the straddling block included up to the query -- dense causal attention."""
    rng = np.random.default_rng(B * 1000 + T_kv + p0)
    q, k, v = _rand_bf16(rng, (T, 4, D)), _rand_bf16(rng, (T_kv, 2, D)), _rand_bf16(rng, (T_kv, 2, D))
    idx = _all_block_lists(rng, T, 2, (T_kv + B - 1) // B, p0)
    out, lse = oracle.sparse_prefill_blocks(q, k, v, idx, B, scale=1 / 16, q_pos0=p0)
    allowed = np.arange(T_kv)[None, :] <= (p0 + np.arange(T))[:, None]
    ref_out, ref_lse = _sdpa_masked(q, k, v, allowed, 1 / 16, 2)
    np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("B", [2, 4, 8])
def test_own_block_tail_closed_form(B):
    """A row that lists only its own block, with every K row of that block
    equal: weights are uniform over the (t mod B) + 1 tokens up to t, so out
    is their mean V and lse = scale * q.k + ln((t mod B) + 1)."""
    rng = np.random.default_rng(B)
    T = 4 * B
    q, v = _rand_bf16(rng, (T, 2, D)), _rand_bf16(rng, (T, 1, D))
    k = np.broadcast_to(_rand_bf16(rng, (1, 1, D)), (T, 1, D)).copy()
    idx = (np.arange(T) // B).astype(np.int32)[:, None, None]
    out, lse = oracle.sparse_prefill_blocks(q, k, v, idx, B, scale=0.07)
    q64, k64, v64 = (qo.bf16_to_f64(a) for a in (q, k, v))
    for t in range(T):
        b0, n = (t // B) * B, t % B + 1
        mean = np.array([math.fsum(col) / n for col in v64[b0: b0 + n, 0].T])
        for h in range(2):
            np.testing.assert_allclose(out[t, h], mean, rtol=0, atol=1e-13)
            assert abs(lse[t, h] - (0.07 * math.fsum(q64[t, h] * k64[0, 0]) + math.log(n))) < 1e-12


def test_block_remainders_0_to_3_count_tokens():
    """Ratio 4, a query in block b lists b only: it sees remainder + 1 tokens
    (lse with q = 0 is ln(count))."""
    T = 16
    q = np.zeros((T, 1, D), np.uint16)
    rng = np.random.default_rng(2)
    k, v = _rand_bf16(rng, (T, 1, D)), _rand_bf16(rng, (T, 1, D))
    idx = (np.arange(T) // 4).astype(np.int32)[:, None, None]
    _, lse = oracle.sparse_prefill_blocks(q, k, v, idx, 4)
    np.testing.assert_allclose(lse[:, 0], np.log(np.arange(T) % 4 + 1), rtol=0, atol=1e-15)


def test_invalid_blocks_are_masked():
    rng = np.random.default_rng(4)
    T = 12
    q, k, v = _rand_bf16(rng, (T, 2, D)), _rand_bf16(rng, (T, 1, D)), _rand_bf16(rng, (T, 1, D))
    bad = np.array([-1, INT32_MIN, INT32_MAX, 1 << 29, 3, -7], np.int32)  # block 3 = tokens 12..15
    idx = np.broadcast_to(bad, (T, 1, bad.size)).copy()
    out, lse = oracle.sparse_prefill_blocks(q, k, v, idx, 4)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_block_size_one_is_the_token_form():
    rng = np.random.default_rng(6)
    T = 30
    q, k, v = _rand_bf16(rng, (T, 3, D)), _rand_bf16(rng, (T, 1, D)), _rand_bf16(rng, (T, 1, D))
    idx = rng.integers(-2, T + 2, size=(T, 1, 9)).astype(np.int32)
    a = oracle.sparse_prefill_blocks(q, k, v, idx, 1)
    b = oracle.sparse_prefill(q, k, v, idx)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


# ------------------------------------------------------------------ slot pool


def _two_request_pool(seed, n_free=9, G=2):
    """Requests A (0..29) and B (its first 12 tokens shared with A, then 10 of
    its own: positions 12..21), plus C with 8 own tokens; slots permuted, free
    slots hold random garbage. Returns the pool and per-request slot tables."""
    rng = np.random.default_rng(seed)
    lens = {"A": 30, "B_own": 10, "C": 8}
    n_tok = lens["A"] + lens["B_own"] + lens["C"]
    n_slots = n_tok + n_free
    perm = rng.permutation(n_slots)
    tA = perm[:30]
    tB = np.concatenate([tA[:12], perm[30:40]])
    tC = perm[40:48]
    slot_pos = np.full(n_slots, -1, np.int32)
    for t in (tA, tB, tC):
        slot_pos[t] = np.arange(t.size)
    Hkv = 2
    k = _rand_bf16(rng, (n_slots, Hkv, D))
    v = _rand_bf16(rng, (n_slots, Hkv, D))
    return rng, {"A": tA, "B": tB, "C": tC}, slot_pos, k, v, n_free, G


def _pool_batch(rng, tables, slot_pos, Hq, new, K, extra):
    """Query rows: the last `new[r]` positions of each request, concatenated.
    Each row lists the slots of all its request's positions <= its own plus
    `extra` (slots that must be masked), shuffled, -1 padded."""
    rows_q_pos, lists, spans = [], [], {}
    for name, table in tables.items():
        n = new[name]
        a = len(rows_q_pos)
        for p in range(table.size - n, table.size):
            row = list(table[: p + 1]) + list(extra(name, p))
            row += [-1] * (K - len(row))
            row = np.array(row, np.int64)
            rng.shuffle(row)
            lists.append(row)
            rows_q_pos.append(p)
        spans[name] = (a, len(rows_q_pos))
    idx = np.stack(lists)[:, None, :].repeat(2, axis=1).astype(np.int32)
    q = _rand_bf16(rng, (len(rows_q_pos), Hq, D))
    return q, idx, np.array(rows_q_pos, np.int32), spans


def _pool_masked_extra(tables, slot_pos, n_slots):
    free = np.nonzero(slot_pos < 0)[0]

    def extra(name, p):
        t = tables[name]
        future = list(t[p + 1: p + 3])  # the request's own later tokens
        return future + [int(free[p % free.size]), n_slots, n_slots + 5, -1, INT32_MIN]
    return extra


def test_pool_full_lists_match_sdpa_per_request():
    """Each request's rows over the permuted pool give dense causal attention
    over that request's own token sequence (the shared prefix included)."""
    rng, tables, slot_pos, k, v, _, G = _two_request_pool(10)
    Hq = 2 * G
    new = {"A": 30, "B": 10, "C": 8}
    q, idx, q_pos, spans = _pool_batch(rng, tables, slot_pos, Hq, new, K=40,
                                       extra=_pool_masked_extra(tables, slot_pos, k.shape[0]))
    out, lse = oracle.sparse_prefill_pool(q, k, v, idx, q_pos, slot_pos, scale=1 / 16)
    for name, table in tables.items():
        a, b = spans[name]
        L = table.size
        allowed = np.arange(L)[None, :] <= q_pos[a:b][:, None]
        ref_out, ref_lse = _sdpa_masked(q[a:b], k[table], v[table], allowed, 1 / 16, G)
        np.testing.assert_allclose(out[a:b], ref_out, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[a:b], ref_lse, rtol=0, atol=1e-12)


def test_pool_slot_position_closed_form():
    """Two listed slots with equal K: the one holding a later position than
    the query is masked, so out is the other slot's V exactly; free slots and
    slots outside the pool change nothing."""
    rng = np.random.default_rng(12)
    n_slots = 6
    k = np.broadcast_to(_rand_bf16(rng, (1, 1, D)), (n_slots, 1, D)).copy()
    v = _rand_bf16(rng, (n_slots, 1, D))
    slot_pos = np.array([5, 2, -1, 3, 0, 9], np.int32)
    q = _rand_bf16(rng, (3, 1, D))
    q_pos = np.array([3, 2, 8], np.int32)
    idx = np.array([[[3, 5, 2, 6]], [[5, 1, -1, 2]], [[0, 2, 5, 7]]], np.int32)
    out, lse = oracle.sparse_prefill_pool(q, k, v, idx, q_pos, slot_pos, scale=0.05)
    v64 = qo.bf16_to_f64(v)
    np.testing.assert_array_equal(out[0, 0], v64[3, 0])  # slot 5 holds position 9 > 3
    np.testing.assert_array_equal(out[1, 0], v64[1, 0])
    np.testing.assert_allclose(out[2, 0], v64[0, 0], rtol=0, atol=0)
    q64, k64 = qo.bf16_to_f64(q), qo.bf16_to_f64(k)
    for r in range(3):
        assert abs(lse[r, 0] - 0.05 * math.fsum(q64[r, 0] * k64[0, 0])) < 1e-12


def test_pool_identity_mapping_is_the_extend_form():
    """A pool whose slot s holds position s is a contiguous cache."""
    rng = np.random.default_rng(13)
    T_kv, T, p0 = 40, 9, 31
    q, k, v = _rand_bf16(rng, (T, 4, D)), _rand_bf16(rng, (T_kv, 2, D)), _rand_bf16(rng, (T_kv, 2, D))
    idx = rng.integers(-3, T_kv + 3, size=(T, 2, 17)).astype(np.int32)
    a = oracle.sparse_prefill_pool(q, k, v, idx, p0 + np.arange(T, dtype=np.int32),
                                   np.arange(T_kv, dtype=np.int32))
    b = oracle.sparse_prefill(q, k, v, idx, q_pos0=p0)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


# ------------------------------------------------------------------ planted mistakes


def _form_pin_failures():
    failures = []
    rng = np.random.default_rng(40)
    T_kv, T, p0, B = 26, 14, 12, 4
    q, k, v = _rand_bf16(rng, (T, 4, D)), _rand_bf16(rng, (T_kv, 2, D)), _rand_bf16(rng, (T_kv, 2, D))
    idx = _all_block_lists(rng, T, 2, (T_kv + B - 1) // B, p0)
    out, lse = oracle.sparse_prefill_blocks(q, k, v, idx, B, scale=1 / 16, q_pos0=p0)
    allowed = np.arange(T_kv)[None, :] <= (p0 + np.arange(T))[:, None]
    ref_out, ref_lse = _sdpa_masked(q, k, v, allowed, 1 / 16, 2)
    if not (np.allclose(out, ref_out, rtol=0, atol=1e-9) and np.allclose(lse, ref_lse, rtol=0, atol=1e-9)):
        failures.append("blocks_full")
    rng, tables, slot_pos, kp, vp, _, G = _two_request_pool(41)
    new = {"A": 30, "B": 10, "C": 8}
    qq, pidx, q_pos, spans = _pool_batch(rng, tables, slot_pos, 2 * G, new, K=40,
                                         extra=_pool_masked_extra(tables, slot_pos, kp.shape[0]))
    out, lse = oracle.sparse_prefill_pool(qq, kp, vp, pidx, q_pos, slot_pos, scale=1 / 16)
    for name, table in tables.items():
        a, b = spans[name]
        allowed = np.arange(table.size)[None, :] <= q_pos[a:b][:, None]
        ro, rl = _sdpa_masked(qq[a:b], kp[table], vp[table], allowed, 1 / 16, G)
        if not (np.allclose(out[a:b], ro, rtol=0, atol=1e-9) and np.allclose(lse[a:b], rl, rtol=0, atol=1e-9)):
            failures.append("pool_full")
            break
    if not _exact(*_block_decimal_case(), atol=1e-12):
        failures.append("blocks_exact")
    if not _exact(*_pool_decimal_case(), atol=1e-12):
        failures.append("pool_exact")
    return failures


def test_form_pins_pass_on_the_oracle():
    assert _form_pin_failures() == []


def _pool_rule(kind):
    def pool_selected_slots(slot_row, q_pos, slot_pos):
        n = len(slot_pos)
        out = []
        for s in slot_row:
            s = int(s)
            if kind == "slot_number_as_position":
                ok = 0 <= s < n and s <= q_pos
            elif kind == "free_slots_used":
                ok = 0 <= s < n and int(slot_pos[s]) <= q_pos
            elif kind == "strict_causal":
                ok = 0 <= s < n and 0 <= int(slot_pos[s]) < q_pos
            else:
                raise AssertionError(kind)
            if ok:
                out.append(s)
        return out
    return pool_selected_slots


FORM_MUTANTS = {
    "blocks_not_expanded": ("expand_blocks", lambda row, B: [int(b) for b in row]),
    "blocks_shifted": ("expand_blocks",
                       lambda row, B: [(int(b) + 1) * B + i for b in row for i in range(B)]),
    "tail_block_dropped": ("expand_blocks",
                           lambda row, B: [int(b) * B + i for b in row for i in range(B - 1)]),
    "slot_number_as_position": ("pool_selected_slots", _pool_rule("slot_number_as_position")),
    "free_slots_used": ("pool_selected_slots", _pool_rule("free_slots_used")),
    "pool_strict_causal": ("pool_selected_slots", _pool_rule("strict_causal")),
}


@pytest.mark.parametrize("name", sorted(FORM_MUTANTS))
def test_form_pins_catch_planted_mistakes(monkeypatch, name):
    attr, fn = FORM_MUTANTS[name]
    monkeypatch.setattr(qo, attr, fn)
    try:
        failures = _form_pin_failures()
    except (IndexError, ValueError) as e:
        failures = [f"raised {type(e).__name__}"]
    assert failures != [], f"no pin caught the planted mistake {name}"


def test_decode_batch_is_the_last_row_of_each_requests_attention():
    """One query per request at its last position, lists naming every slot of
    the request (plus empty slots): torch fp64 SDPA over the request's own
    sequence, last row."""
    rng, tables, slot_pos, k, v, _, G = _two_request_pool(20)
    Hq = 2 * G
    names = list(tables)
    q = _rand_bf16(rng, (len(names), Hq, D))
    K = 48
    idx = np.full((len(names), 2, K), -1, np.int32)
    q_pos = np.zeros(len(names), np.int32)
    free = np.nonzero(slot_pos < 0)[0]
    for r, name in enumerate(names):
        t = tables[name]
        row = np.array(list(t) + list(free[:3]) + [-1] * (K - t.size - 3), np.int64)
        rng.shuffle(row)
        idx[r] = row
        q_pos[r] = t.size - 1
    out, lse = oracle.sparse_prefill_pool(q, k, v, idx, q_pos, slot_pos, scale=1 / 16)
    for r, name in enumerate(names):
        t = tables[name]
        allowed = np.ones((1, t.size), bool)
        ro, rl = _sdpa_masked(q[r:r + 1], k[t], v[t], allowed, 1 / 16, G)
        np.testing.assert_allclose(out[r:r + 1], ro, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[r:r + 1], rl, rtol=0, atol=1e-12)


# ------------------------------------------------------------------ exact values


def _decimal_over(q, k, v, used, scale, G, digits=50):
    """Exact attention (50-digit decimal, exp of the raw logits, no max shift)
    of each query row t and head h over the K/V rows used[t][h // G]."""
    from decimal import Decimal, localcontext

    T, Hq, _ = q.shape
    q64, k64, v64 = (qo.bf16_to_f64(a) for a in (q, k, v))
    out = np.zeros((T, Hq, D))
    lse = np.full((T, Hq), -np.inf)
    with localcontext() as ctx:
        ctx.prec = digits
        sc = Decimal(float(scale))
        for t in range(T):
            for h in range(Hq):
                sel = used[t][h // G]
                if not sel:
                    continue
                qd = [Decimal(float(x)) for x in q64[t, h]]
                w = [(sc * sum(a * Decimal(float(b)) for a, b in zip(qd, k64[s, h // G]))).exp() for s in sel]
                l = sum(w)
                for d in range(D):
                    out[t, h, d] = float(sum(wi * Decimal(float(v64[s, h // G, d])) for wi, s in zip(w, sel)) / l)
                lse[t, h] = float(l.ln())
    return out, lse


def _block_decimal_case():
    """Micro-block lists (block size 4, a cached prefix, the query's own block
    cut at the query, -1 and out-of-range entries, an empty row) and their
    exact value, the token rule applied by hand: entry b names tokens
    4b..4b+3, each used iff it is at or before the query's position."""
    rng = np.random.default_rng(61)
    T, p0, Hq, Hkv, B = 5, 9, 4, 2, 4
    T_kv = p0 + T
    q, k, v = _rand_bf16(rng, (T, Hq, D)), _rand_bf16(rng, (T_kv, Hkv, D)), _rand_bf16(rng, (T_kv, Hkv, D))
    idx = rng.integers(-1, T_kv // B + 2, size=(T, Hkv, 5)).astype(np.int32)
    idx[2, 1] = -1
    used = [[[b * B + i for b in idx[t, g] if b >= 0 for i in range(B) if b * B + i <= p0 + t]
             for g in range(Hkv)] for t in range(T)]
    out, lse = oracle.sparse_prefill_blocks(q, k, v, idx, B, scale=1 / 16, q_pos0=p0)
    return (out, lse) + _decimal_over(q, k, v, used, 1 / 16, G=Hq // Hkv)


def _pool_decimal_case():
    """A pool batch (permuted slots, a shared prefix, empty slots, slots past
    the pool, a request's own later tokens) and its exact value, the slot
    rule applied by hand: slot s is used iff it is inside the pool, holds a
    token, and that token's position is at or before the query's."""
    rng, tables, slot_pos, k, v, _, G = _two_request_pool(62)
    n_slots = slot_pos.size
    q, idx, q_pos, _ = _pool_batch(rng, tables, slot_pos, 4, {"A": 2, "B": 2, "C": 1}, 48,
                                   _pool_masked_extra(tables, slot_pos, n_slots))
    used = [[[int(s) for s in idx[r, g] if 0 <= s < n_slots and 0 <= slot_pos[s] <= q_pos[r]]
             for g in range(idx.shape[1])] for r in range(q.shape[0])]
    out, lse = oracle.sparse_prefill_pool(q, k, v, idx, q_pos, slot_pos, scale=1 / 16)
    return (out, lse) + _decimal_over(q, k, v, used, 1 / 16, G=G)


def _exact(out, lse, ref_out, ref_lse, atol):
    fin = np.isfinite(ref_lse)
    return (np.allclose(out, ref_out, rtol=0, atol=atol) and np.array_equal(np.isfinite(lse), fin)
            and np.allclose(lse[fin], ref_lse[fin], rtol=0, atol=atol))


def test_block_lists_match_decimal_brute_force():
    assert _exact(*_block_decimal_case(), atol=1e-13)


def test_pool_lists_match_decimal_brute_force():
    assert _exact(*_pool_decimal_case(), atol=1e-13)
