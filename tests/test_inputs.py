"""Checks of the seeded input generators: index structure, seeding, samplers."""
import dataclasses
import itertools

import numpy as np
import pytest

from qsa_inputs import CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, get_config, make_indices, make_qkv
from qsa_inputs import generate as gen


def _check_rows(cfg, idx, rows):
    K, W = cfg.K, cfg.window
    for i, t in enumerate(rows):
        for g in range(cfg.Hkv):
            row = idx[i, g]
            valid = row[row >= 0]
            assert np.all(row[len(valid):] == -1), "pads only at the end"
            assert np.all(np.diff(valid) > 0), "ascending and distinct"
            assert valid.size == min(t + 1, K)
            assert valid.max() == t and valid.min() >= 0
            if t + 1 <= K:
                np.testing.assert_array_equal(valid, np.arange(t + 1))
                continue
            window = np.arange(t - W + 1, t + 1)
            assert np.all(np.isin(window, valid)), "whole local window selected"
            if cfg.sink:
                assert valid[0] == 0
            rest = np.setdiff1d(valid, window)
            if cfg.sink:
                rest = rest[1:]
            assert rest.size == cfg.n_rest
            lo = 1 if cfg.sink else 0
            assert rest.min() >= lo and rest.max() <= t - W - cfg.gap


@pytest.mark.parametrize("number", [1, 2])
def test_full_index_structure_small_workloads(number):
    cfg = get_config(number)
    idx = make_indices(cfg, workers=1)
    assert idx.shape == (cfg.T, cfg.Hkv, cfg.K) and idx.dtype == np.int32
    _check_rows(cfg, idx, range(cfg.T))


@pytest.mark.parametrize("number", [3, 4, 5])
def test_sampled_index_structure_large_workloads(number):
    cfg = get_config(number)
    rows = [0, 1, cfg.K - 2, cfg.K - 1, cfg.K, cfg.K + 1, 5000, cfg.T - 1]
    idx = make_indices(cfg, rows=rows, workers=1)
    _check_rows(cfg, idx, rows)


def test_row_subsets_match_full_generation_and_workers():
    cfg = get_config(2)
    full = make_indices(cfg, workers=1)
    rows = [0, 511, 512, 1500, 4095]
    np.testing.assert_array_equal(make_indices(cfg, rows=rows, workers=1), full[rows])
    np.testing.assert_array_equal(make_indices(cfg, workers=2), full)
    q1, k1, v1 = make_qkv(cfg, workers=1)
    q2, k2, v2 = make_qkv(cfg, workers=2)
    for a, b in ((q1, q2), (k1, k2), (v1, v2)):
        np.testing.assert_array_equal(a, b)


def test_kv_heads_draw_independently():
    cfg = get_config(4)
    idx = make_indices(cfg, rows=[20000], workers=1)
    assert not np.array_equal(idx[0, 0], idx[0, 1])


def test_outlier_rows_are_scaled_by_eight():
    cfg = get_config(3)
    small = dataclasses.replace(cfg, T=2048, oracle_rows=0)
    plain = dataclasses.replace(small, outlier_frac=0.0)
    q, k, v = make_qkv(small, workers=1)
    q0, k0, v0 = make_qkv(plain, workers=1)
    pos = gen.outlier_positions(small)
    assert pos.size == round(0.01 * 2048) and np.unique(pos).size == pos.size
    np.testing.assert_array_equal(q, q0)
    for a, a0 in ((k, k0), (v, v0)):
        np.testing.assert_array_equal(bf16_bits_to_f32(a[pos]), 8 * bf16_bits_to_f32(a0[pos]))
        keep = np.setdiff1d(np.arange(2048), pos)
        np.testing.assert_array_equal(a[keep], a0[keep])
    assert gen.outlier_positions(cfg).size == 328


def test_bf16_rounding_is_nearest_even():
    import torch
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 3.0e-39]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(f32_to_bf16_bits(x), ref)


def test_uniform_sampler_is_uniform_over_subsets():
    rng = np.random.default_rng(1)
    n_rows = 30000
    picks = gen._uniform_distinct(rng, np.full(n_rows, 5), 3)  # small-population path
    picks.sort(axis=1)
    subsets = {s: 0 for s in itertools.combinations(range(5), 3)}
    for row in map(tuple, picks):
        subsets[row] += 1
    freq = np.array(list(subsets.values())) / n_rows
    assert np.all(np.abs(freq - 0.1) < 0.012)
    big = gen._uniform_distinct(rng, np.full(20000, 40), 3)  # redraw path (40 > 4*3)
    assert all(len(set(r)) == 3 for r in big.tolist())
    counts = np.bincount(big.ravel(), minlength=40) / big.size
    assert np.all(np.abs(counts - 1 / 40) < 0.004)


def test_weighted_sampler_matches_successive_sampling():
    rng = np.random.default_rng(2)
    n_rows, t, lo, hi = 40000, 30, 1, 6
    w = 1.0 / (1.0 + (t - np.arange(lo, hi + 1)) / 1024.0)
    w_strong = np.array([1.0, 2.0, 4.0, 8.0, 16.0, 32.0])
    p = w / w.sum()
    picks = gen._weighted_distinct(rng, np.full(n_rows, t), lo, np.full(n_rows, hi), 2)
    assert all(a != b for a, b in picks.tolist())
    incl = np.array([(picks == s).any(axis=1).mean() for s in range(lo, hi + 1)])
    exact = np.array([p[i] + sum(p[j] * p[i] / (1 - p[j]) for j in range(len(p)) if j != i)
                      for i in range(len(p))])
    assert np.all(np.abs(incl - exact) < 0.01)
    # a steep weight (t close to the population) is visibly non-uniform
    steep = gen._weighted_distinct(rng, np.full(n_rows, 3000), 1, np.full(n_rows, 2990), 1)
    far, near = (steep < 100).mean(), (steep > 2890).mean()
    assert near > 1.5 * far
    del w_strong


def test_workload_table():
    assert [c.G for c in CONFIGS] == [3, 6, 8, 12, 12]
    assert [c.valid_slots() for c in CONFIGS] == [14368, 1966336, 130025472, 130025472, 479200256]
    assert CONFIGS[4].T == 918 * 256
