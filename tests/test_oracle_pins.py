"""Pins of the fp64 oracle against facts fixed by the method and by mathematics.

None of these re-types the oracle's own formula: each compares it with an
independent library routine (torch's fp64 scaled_dot_product_attention,
logsumexp, scipy's expit), with a closed form, with an invariant the
definition implies, with the pages' own packed-cache identity, or with the
exact value on tiny inputs (50-digit decimal arithmetic, textbook softmax
without the max shift). The last
test plants plausible mistakes in the oracle and checks that at least one
pin catches each of them.

Definition followed: "Qwen4-Exp QSA llega al Ascend de Huawei" (orcarouter.ai,
Spanish page), section "Lo que realmente añade la pull request" (softmax over
the selected tokens, -1 slots masked, fully masked rows give zero, the packed
[K, V] cache identity) and section "Nueve pruebas que pasaron" (unordered
slots, default and explicit scales, zero selection width, causal tails).
"""
import math

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
import oracle.qsa_oracle as qo
from qsa_inputs import Config, bf16_bits_to_f32, f32_to_bf16_bits, make_inputs

D = 256
INT32_MIN = -(2 ** 31)


def _rand_bf16(rng, shape, sigma=1.0):
    return f32_to_bf16_bits((rng.standard_normal(shape) * sigma).astype(np.float32))


def _small_case(seed, T, Hq, Hkv, sigma=1.0):
    rng = np.random.default_rng(seed)
    q = _rand_bf16(rng, (T, Hq, D), sigma)
    k = _rand_bf16(rng, (T, Hkv, D), sigma)
    v = _rand_bf16(rng, (T, Hkv, D), sigma)
    return rng, q, k, v


def _dense_lists(rng, T, Hkv, K, shuffle):
    """Every row t selects all of 0..t (K >= T), pads -1, optionally shuffled."""
    idx = np.full((T, Hkv, K), -1, np.int32)
    for t in range(T):
        for g in range(Hkv):
            row = np.full(K, -1, np.int32)
            row[: t + 1] = np.arange(t + 1)
            if shuffle:
                rng.shuffle(row)
            idx[t, g] = row
    return idx


def _sdpa_dense_causal(q, k, v, scale, G):
    """torch fp64 causal attention with KV heads repeated G times in place."""
    Q = torch.from_numpy(qo.bf16_to_f64(q)).permute(1, 0, 2)
    Kr = torch.from_numpy(qo.bf16_to_f64(k)).repeat_interleave(G, dim=1).permute(1, 0, 2)
    Vr = torch.from_numpy(qo.bf16_to_f64(v)).repeat_interleave(G, dim=1).permute(1, 0, 2)
    out = F.scaled_dot_product_attention(Q, Kr, Vr, is_causal=True, scale=scale)
    T = Q.shape[1]
    scores = torch.matmul(Q, Kr.transpose(1, 2).contiguous()) * scale
    mask = torch.triu(torch.ones(T, T, dtype=torch.bool), diagonal=1)
    lse = torch.logsumexp(scores.masked_fill(mask, float("-inf")), dim=-1)
    return out.permute(1, 0, 2).numpy(), lse.permute(1, 0).numpy()


# ----------------------------------------------------------------- P-a dense causal


@pytest.mark.parametrize("T,Hq,Hkv", [(40, 6, 2), (33, 2, 2), (24, 8, 1), (20, 12, 1)])
@pytest.mark.parametrize("shuffle", [False, True])
def test_dense_causal_matches_torch_sdpa(T, Hq, Hkv, shuffle):
    rng, q, k, v = _small_case(T * 100 + Hq, T, Hq, Hkv)
    idx = _dense_lists(rng, T, Hkv, K=T + 7, shuffle=shuffle)
    out, lse = oracle.sparse_prefill(q, k, v, idx, scale=1 / 16)
    ref_out, ref_lse = _sdpa_dense_causal(q, k, v, 1 / 16, Hq // Hkv)
    np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("number,n_dense", [(1, 64), (2, 512)])
def test_dense_ramp_of_workloads_matches_torch_sdpa(number, n_dense):
    """Rows t < K of each workload select all of 0..t: dense causal attention."""
    d = make_inputs(number, workers=1)
    cfg = d["cfg"]
    q, k, v = d["q"][:n_dense], d["k"][:n_dense], d["v"][:n_dense]
    rows = np.arange(0, n_dense, 1 if n_dense <= 64 else 7)
    out, lse = oracle.sparse_prefill(q, k, v, d["idx"][:n_dense], scale=cfg.scale, rows=rows)
    ref_out, ref_lse = _sdpa_dense_causal(q, k, v, cfg.scale, cfg.G)
    np.testing.assert_allclose(out, ref_out[rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse[rows], rtol=0, atol=1e-12)


def test_default_scale_is_one_over_sqrt_256():
    rng, q, k, v = _small_case(5, 12, 2, 1)
    idx = _dense_lists(rng, 12, 1, 16, shuffle=False)
    a = oracle.sparse_prefill(q, k, v, idx)
    b = oracle.sparse_prefill(q, k, v, idx, scale=0.0625)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


@pytest.mark.parametrize("scale", [0.1, 0.03125, 1.0])
def test_explicit_scale_matches_torch_sdpa(scale):
    rng, q, k, v = _small_case(11, 18, 4, 2)
    idx = _dense_lists(rng, 18, 2, 18, shuffle=True)
    out, lse = oracle.sparse_prefill(q, k, v, idx, scale=scale)
    ref_out, ref_lse = _sdpa_dense_causal(q, k, v, scale, 2)
    np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("T_kv,T,p0", [(40, 12, 28), (33, 33, 0), (50, 7, 20)])
def test_extend_over_cached_prefix_matches_masked_sdpa(T_kv, T, p0):
    """Queries at positions p0..p0+T-1 against a longer cache, every position
    <= the query's selected: torch fp64 attention with an explicit mask."""
    rng = np.random.default_rng(T_kv * 7 + p0)
    q = _rand_bf16(rng, (T, 4, D))
    k = _rand_bf16(rng, (T_kv, 2, D))
    v = _rand_bf16(rng, (T_kv, 2, D))
    K = T_kv + 3
    idx = np.full((T, 2, K), -1, np.int32)
    for t in range(T):
        for g in range(2):
            row = np.full(K, -1, np.int32)
            row[: p0 + t + 1] = np.arange(p0 + t + 1)
            rng.shuffle(row)
            idx[t, g] = row
    out, lse = oracle.sparse_prefill(q, k, v, idx, scale=1 / 16, q_pos0=p0)
    Q = torch.from_numpy(qo.bf16_to_f64(q)).permute(1, 0, 2)
    Kr = torch.from_numpy(qo.bf16_to_f64(k)).repeat_interleave(2, dim=1).permute(1, 0, 2)
    Vr = torch.from_numpy(qo.bf16_to_f64(v)).repeat_interleave(2, dim=1).permute(1, 0, 2)
    allowed = torch.arange(T_kv)[None, :] <= (p0 + torch.arange(T))[:, None]
    ref = F.scaled_dot_product_attention(Q, Kr, Vr, attn_mask=allowed, scale=1 / 16)
    scores = torch.matmul(Q, Kr.transpose(1, 2).contiguous()) / 16
    ref_lse = torch.logsumexp(scores.masked_fill(~allowed, float("-inf")), dim=-1)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse.permute(1, 0).numpy(), rtol=0, atol=1e-12)


def test_extend_equals_rows_of_full_prefill():
    rng, q, k, v, idx = _sparse_case(seed=31, T=80, Hq=6, Hkv=2, K=30)
    full_out, full_lse = oracle.sparse_prefill(q, k, v, idx, scale=1 / 16)
    p0 = 53
    out, lse = oracle.sparse_prefill(q[p0:], k, v, idx[p0:], scale=1 / 16, q_pos0=p0)
    np.testing.assert_array_equal(out, full_out[p0:])
    np.testing.assert_array_equal(lse, full_lse[p0:])


# ----------------------------------------------------------------- sparse invariants


def _sparse_case(seed=3, T=96, Hq=6, Hkv=2, K=40):
    rng, q, k, v = _small_case(seed, T, Hq, Hkv)
    idx = np.full((T, Hkv, K), -1, np.int32)
    for t in range(T):
        for g in range(Hkv):
            n = min(t + 1, K - 3)
            idx[t, g, :n] = rng.choice(t + 1, size=n, replace=False)
    return rng, q, k, v, idx


def test_order_independence():
    rng, q, k, v, idx = _sparse_case()
    out, lse = oracle.sparse_prefill(q, k, v, idx, scale=1 / 16)
    perm = idx.copy()
    for t in range(perm.shape[0]):
        for g in range(perm.shape[1]):
            rng.shuffle(perm[t, g])
    out2, lse2 = oracle.sparse_prefill(q, k, v, perm, scale=1 / 16)
    np.testing.assert_allclose(out2, out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-12)


def test_constant_values_give_constant_output():
    rng, q, k, v, idx = _sparse_case(seed=4)
    c = np.linspace(-3, 3, D).astype(np.float32)
    v_const = np.broadcast_to(f32_to_bf16_bits(c), v.shape).copy()
    out, lse = oracle.sparse_prefill(q, k, v_const, idx, scale=1 / 16)
    c_exact = bf16_bits_to_f32(f32_to_bf16_bits(c)).astype(np.float64)
    np.testing.assert_allclose(out, np.broadcast_to(c_exact, out.shape), rtol=1e-13, atol=1e-14)


def test_probabilities_sum_to_one():
    rng, q, k, v, idx = _sparse_case(seed=6)
    for t in (0, 1, 17, 60, 95):
        for h in range(q.shape[1]):
            sel, z, p, lse = oracle.row_probabilities(q, k, idx, t, h, scale=1 / 16)
            assert len(sel) == len(p) > 0
            assert abs(p.sum() - 1.0) < 1e-12
            assert abs(math.fsum(np.exp(z - lse)) - 1.0) < 1e-12
            ref = scipy.special.softmax(z)
            np.testing.assert_allclose(p, ref, rtol=0, atol=1e-14)
            assert abs(lse - scipy.special.logsumexp(z)) < 1e-12


@pytest.mark.parametrize("where", ["head", "interior", "tail"])
@pytest.mark.parametrize("bad", ["minus1", "future", "beyond_T", "int32_min", "neg7"])
def test_masked_entries_change_nothing(where, bad):
    rng, q, k, v, idx = _sparse_case(seed=8)
    T, Hkv, K = idx.shape
    out, lse = oracle.sparse_prefill(q, k, v, idx, scale=1 / 16)
    wide = np.full((T, Hkv, K + 3), -1, np.int32)
    for t in range(T):
        for g in range(Hkv):
            vals = {"minus1": -1, "future": t + 1, "beyond_T": T + 5,
                    "int32_min": INT32_MIN, "neg7": -7}[bad]
            row = list(idx[t, g])
            pos = {"head": 0, "interior": len(row) // 2, "tail": len(row)}[where]
            for _ in range(3):
                row.insert(pos, vals)
            wide[t, g] = row
    out2, lse2 = oracle.sparse_prefill(q, k, v, wide, scale=1 / 16)
    np.testing.assert_array_equal(out2, out)
    np.testing.assert_array_equal(lse2, lse)
    # dropping trailing pads (a shorter selection width) changes nothing either
    n_keep = int((idx >= 0).sum(axis=2).max())
    out3, lse3 = oracle.sparse_prefill(q, k, v, idx[:, :, :n_keep], scale=1 / 16)
    np.testing.assert_array_equal(out3, out)
    np.testing.assert_array_equal(lse3, lse)


def test_single_slot_closed_form():
    rng, q, k, v = _small_case(9, 30, 3, 1)
    idx = np.full((30, 1, 5), -1, np.int32)
    picks = [int(rng.integers(0, t + 1)) for t in range(30)]
    for t, s in enumerate(picks):
        idx[t, 0, 2] = s
    out, lse = oracle.sparse_prefill(q, k, v, idx, scale=0.0625)
    q64, k64, v64 = (qo.bf16_to_f64(a) for a in (q, k, v))
    for t, s in enumerate(picks):
        for h in range(3):
            np.testing.assert_array_equal(out[t, h], v64[s, 0])
            exact = 0.0625 * math.fsum(q64[t, h] * k64[s, 0])
            assert abs(lse[t, h] - exact) < 1e-12


def test_two_slots_closed_form():
    rng, q, k, v = _small_case(10, 40, 2, 1)
    q64, k64, v64 = (qo.bf16_to_f64(a) for a in (q, k, v))
    for t in range(1, 40):
        a, b = rng.choice(t + 1, size=2, replace=False)
        idx = np.full((40, 1, 2), -1, np.int32)
        idx[t, 0] = [a, b]
        out, lse = oracle.sparse_prefill(q, k, v, idx, scale=0.1, rows=[t])
        for h in range(2):
            za = 0.1 * math.fsum(q64[t, h] * k64[a, 0])
            zb = 0.1 * math.fsum(q64[t, h] * k64[b, 0])
            pa = scipy.special.expit(za - zb)
            np.testing.assert_allclose(out[0, h], pa * v64[a, 0] + (1 - pa) * v64[b, 0],
                                       rtol=0, atol=1e-13)
            assert abs(lse[0, h] - np.logaddexp(za, zb)) < 1e-12


def test_three_slots_known_logits():
    """Logits 0, 1, 2 built exactly from one-hot q and k: p = (1, e, e^2) / sum."""
    T = 4
    q = np.zeros((T, 1, D), np.float32)
    k = np.zeros((T, 1, D), np.float32)
    v = np.zeros((T, 1, D), np.float32)
    q[3, 0, 5] = 1.0
    k[:3, 0, 5] = [0.0, 1.0, 2.0]
    v[:3, 0, 0] = [1.0, 10.0, 100.0]
    idx = np.array([[[-1, -1, -1, -1]]] * 3 + [[[2, 0, 1, -1]]], np.int32)
    out, lse = oracle.sparse_prefill(f32_to_bf16_bits(q), f32_to_bf16_bits(k),
                                     f32_to_bf16_bits(v), idx, scale=1.0, rows=[3])
    e = math.e
    zsum = 1 + e + e * e
    assert abs(out[0, 0, 0] - (1 + 10 * e + 100 * e * e) / zsum) < 1e-12
    assert abs(lse[0, 0] - math.log(zsum)) < 1e-14
    assert np.all(out[0, 0, 1:] == 0)


@pytest.mark.parametrize("mode", ["zero_q", "zero_scale"])
def test_uniform_weights_give_mean(mode):
    rng, q, k, v, idx = _sparse_case(seed=12)
    scale = 1 / 16
    if mode == "zero_q":
        q = np.zeros_like(q)
    else:
        scale = 0.0
    out, lse = oracle.sparse_prefill(q, k, v, idx, scale=scale)
    v64 = qo.bf16_to_f64(v)
    G = q.shape[1] // k.shape[1]
    for t in range(idx.shape[0]):
        for h in range(q.shape[1]):
            sel = [s for s in idx[t, h // G] if 0 <= s <= t]
            np.testing.assert_allclose(out[t, h], v64[sel, h // G].mean(axis=0), rtol=0, atol=1e-13)
            assert abs(lse[t, h] - math.log(len(sel))) < 1e-13


def test_packed_cache_identity_of_the_ascend_adapter():
    """softmax(scale [Q,0] [K,V]^T) [K,V] = [P K, P V]: its V half is the output."""
    rng, q, k, v, idx = _sparse_case(seed=13, T=50, Hq=4, Hkv=2, K=24)
    out, lse = oracle.sparse_prefill(q, k, v, idx, scale=1 / 16)
    q64, k64, v64 = (qo.bf16_to_f64(a) for a in (q, k, v))
    G = 2
    for t in (0, 7, 30, 49):
        for h in range(4):
            g = h // G
            sel = [s for s in idx[t, g] if 0 <= s <= t]
            C = torch.from_numpy(np.concatenate([k64[sel, g], v64[sel, g]], axis=1))[None]
            Qp = torch.from_numpy(np.concatenate([q64[t, h], np.zeros(D)]))[None, None]
            packed = F.scaled_dot_product_attention(Qp, C, C, scale=1 / 16)[0, 0].numpy()
            np.testing.assert_allclose(packed[D:], out[t, h], rtol=0, atol=1e-12)
            sel_k, z, p, _ = oracle.row_probabilities(q, k, idx, t, h, scale=1 / 16)
            np.testing.assert_allclose(packed[:D], p @ k64[sel_k, g], rtol=0, atol=1e-12)


@pytest.mark.parametrize("kind", ["width0", "all_minus1", "all_future", "int32_min"])
def test_empty_rows_are_zero_with_minus_inf_lse(kind):
    rng, q, k, v = _small_case(14, 16, 3, 1)
    T = 16
    if kind == "width0":
        idx = np.zeros((T, 1, 0), np.int32)
    elif kind == "all_minus1":
        idx = np.full((T, 1, 9), -1, np.int32)
    elif kind == "int32_min":
        idx = np.full((T, 1, 9), INT32_MIN, np.int32)
    else:
        idx = np.stack([np.arange(t + 1, t + 10) for t in range(T)])[:, None, :].astype(np.int32)
    out, lse = oracle.sparse_prefill(q, k, v, idx, scale=1 / 16, Hkv=1)
    assert np.all(out == 0.0) and not np.any(np.signbit(out))
    assert np.all(np.isneginf(lse))


def test_repeated_position_counts_per_entry():
    """A position listed twice is two softmax terms (the gather's multiset)."""
    rng, q, k, v = _small_case(15, 8, 1, 1)
    idx = np.full((8, 1, 3), -1, np.int32)
    idx[7, 0] = [2, 2, 5]
    out, _ = oracle.sparse_prefill(q, k, v, idx, scale=0.5, rows=[7])
    q64, k64, v64 = (qo.bf16_to_f64(a) for a in (q, k, v))
    z2 = 0.5 * math.fsum(q64[7, 0] * k64[2, 0])
    z5 = 0.5 * math.fsum(q64[7, 0] * k64[5, 0])
    p2 = 2 * math.exp(z2) / (2 * math.exp(z2) + math.exp(z5))
    np.testing.assert_allclose(out[0, 0], p2 * v64[2, 0] + (1 - p2) * v64[5, 0], rtol=0, atol=1e-13)


def _decimal_attention(q, k, v, idx, scale, G, digits=50):
    """Brute force in 50-digit decimal arithmetic, straight from the definition:
    w_j = exp(z_j) (no max subtracted), out = sum_j w_j v_j / sum_j w_j, lse =
    ln sum_j w_j. bf16 values and the scale convert to decimal exactly, the
    products and sums are exact at this precision, and exp / ln are correctly
    rounded, so the result is the exact value to ~1e-45."""
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
                g = h // G
                sel = [int(s) for s in idx[t, g] if 0 <= int(s) <= t]
                if not sel:
                    continue
                qd = [Decimal(float(x)) for x in q64[t, h]]
                w = [(sc * sum(a * Decimal(float(b)) for a, b in zip(qd, k64[s, g]))).exp() for s in sel]
                l = sum(w)
                for d in range(D):
                    out[t, h, d] = float(sum(wi * Decimal(float(v64[s, g, d])) for wi, s in zip(w, sel)) / l)
                lse[t, h] = float(l.ln())
    return out, lse


def _decimal_case(seed=31):
    """Tiny rows with shuffled positions, -1 pads, a future position and one
    repeated position."""
    rng, q, k, v = _small_case(seed, 7, 4, 2)
    idx = np.full((7, 2, 6), -1, np.int32)
    for t in range(7):
        for g in range(2):
            row = [int(s) for s in rng.choice(t + 1, size=min(t + 1, 3), replace=False)]
            row += [row[0], t + 1 + int(rng.integers(0, 4))]
            row += [-1] * (6 - len(row))
            rng.shuffle(row)
            idx[t, g] = row
    idx[0, 1] = -1  # one empty row
    return q, k, v, idx


def test_tiny_cases_match_decimal_brute_force():
    q, k, v, idx = _decimal_case()
    for scale in (1 / 16, 0.3):
        out, lse = oracle.sparse_prefill(q, k, v, idx, scale=scale)
        ref_out, ref_lse = _decimal_attention(q, k, v, idx, scale, G=2)
        np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-13)
        np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(ref_lse))
        fin = np.isfinite(ref_lse)
        np.testing.assert_allclose(lse[fin], ref_lse[fin], rtol=0, atol=1e-13)


def test_bf16_widening_is_exact():
    vals = np.array([0.0, -0.0, 1.0, -2.5, 3.0e38, 1.0e-38, 0.1], np.float32)
    bits = f32_to_bf16_bits(vals)
    got = qo.bf16_to_f64(bits)
    np.testing.assert_array_equal(got, bf16_bits_to_f32(bits).astype(np.float64))
    t = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(got, t)


# ----------------------------------------------------------------- planted mistakes


def _pin_failures():
    """Run a compact set of the pins above; return the names of those that fail."""
    failures = []
    rng, q, k, v = _small_case(21, 26, 6, 2)
    idx = _dense_lists(rng, 26, 2, 30, shuffle=True)
    out, lse = oracle.sparse_prefill(q, k, v, idx, scale=1 / 16)
    ref_out, ref_lse = _sdpa_dense_causal(q, k, v, 1 / 16, 3)
    if not (np.allclose(out, ref_out, rtol=0, atol=1e-9) and np.allclose(lse, ref_lse, rtol=0, atol=1e-9)):
        failures.append("dense_causal")
    rng, q, k, v, sp = _sparse_case(seed=22, T=40, Hq=4, Hkv=2, K=20)
    o1, l1 = oracle.sparse_prefill(q, k, v, sp, scale=1 / 16)
    wide = np.concatenate([sp, np.stack([np.full((2,), t + 1) for t in range(40)])[:, None, :]
                           .repeat(2, axis=1).astype(np.int32), np.full((40, 2, 2), -1, np.int32)], axis=2)
    o2, l2 = oracle.sparse_prefill(q, k, v, wide, scale=1 / 16)
    if not (np.array_equal(o1, o2) and np.array_equal(l1, l2)):
        failures.append("masking")
    c = f32_to_bf16_bits(np.full(D, 1.5, np.float32))
    oc, _ = oracle.sparse_prefill(q, k, np.broadcast_to(c, v.shape).copy(), sp, scale=1 / 16)
    nonempty = (sp >= 0).any(axis=2).repeat(2, axis=1)
    if not np.allclose(oc[nonempty], 1.5, rtol=0, atol=1e-12):
        failures.append("constant_v")
    single = np.full((40, 2, 3), -1, np.int32)
    single[:, :, 1] = np.arange(40)[:, None] // 2
    os_, ls_ = oracle.sparse_prefill(q, k, v, single, scale=1 / 16)
    q64, k64, v64 = (qo.bf16_to_f64(a) for a in (q, k, v))
    for t in (5, 39):
        for h in range(4):
            s = t // 2
            if not np.array_equal(os_[t, h], v64[s, h // 2]) or \
                    abs(ls_[t, h] - math.fsum(q64[t, h] * k64[s, h // 2]) / 16) > 1e-12:
                failures.append("single_slot")
                break
    empty = np.full((40, 2, 4), -1, np.int32)
    oe, le = oracle.sparse_prefill(q, k, v, empty, scale=1 / 16)
    if not (np.all(oe == 0) and np.all(np.isneginf(le))):
        failures.append("empty_rows")
    q, k, v, idx = _decimal_case()
    od, ld = oracle.sparse_prefill(q, k, v, idx, scale=1 / 16)
    rd, rl = _decimal_attention(q, k, v, idx, 1 / 16, G=2)
    fin = np.isfinite(rl)
    if not (np.allclose(od, rd, rtol=0, atol=1e-12) and np.array_equal(np.isfinite(ld), fin)
            and np.allclose(ld[fin], rl[fin], rtol=0, atol=1e-12)):
        failures.append("exact_decimal")
    return failures


def test_pins_pass_on_the_oracle():
    assert _pin_failures() == []


def _attend_variant(kind):
    def attend(q_h, k_sel, v_sel, scale):
        n = k_sel.shape[0]
        if n == 0:
            return np.zeros(q_h.shape[-1]), -np.inf, np.zeros(0)
        s = {"no_scale": 1.0, "neg_sign": -scale}.get(kind, scale)
        z = s * (k_sel @ q_h)
        m = z.max()
        w = np.exp(z - m)
        l = w.sum()
        p = w if kind == "unnormalised" else w / l
        vals = k_sel if kind == "k_for_v" else v_sel
        out = p @ vals
        lse = np.log(l) if kind == "lse_drops_max" else m + np.log(l)
        return out, lse, p
    return attend


MUTANTS = {
    "gqa_interleaved": ("kv_head_of", lambda h, G: h % 2),
    "causal_drops_diagonal": ("selected_positions",
                              lambda row, t: [int(s) for s in row if 0 <= int(s) < t]),
    "causal_leaks_next": ("selected_positions",
                          lambda row, t: [int(s) for s in row if 0 <= int(s) <= t + 1]),
    "negatives_not_masked": ("selected_positions",
                             lambda row, t: [int(s) for s in row if int(s) <= t]),
    "no_scale": ("attend", _attend_variant("no_scale")),
    "neg_sign": ("attend", _attend_variant("neg_sign")),
    "unnormalised": ("attend", _attend_variant("unnormalised")),
    "k_for_v": ("attend", _attend_variant("k_for_v")),
    "lse_drops_max": ("attend", _attend_variant("lse_drops_max")),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(monkeypatch, name):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(qo, attr, fn)
    try:
        failures = _pin_failures()
    except (IndexError, ValueError) as e:  # an out-of-range gather also exposes it
        failures = [f"raised {type(e).__name__}"]
    assert failures != [], f"no pin caught the planted mistake {name}"
