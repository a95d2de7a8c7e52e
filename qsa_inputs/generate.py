"""Seeded generators for Q/K/V and top-K index lists (host, NumPy).

Every random draw comes from a PCG64 stream keyed by
(workload seed, stream id, head, chunk of 1024 rows), so any subset of rows
can be regenerated bit-for-bit without drawing the rest, and a process pool
gives the same arrays as a single process.

Index lists follow the workload recipe in `configs.py`. Distinct draws use
exact samplers:
  uniform   draw with replacement, then redraw every repeated value until
            all are distinct (the law of the resulting set is invariant under
            relabelling the population, hence uniform over subsets); rows
            whose population is at most 4x the draw count use the m smallest
            of i.i.d. uniform keys instead, so no row needs many redraws;
  weighted  Gumbel-top-k: the m largest of log w(s) + Gumbel noise, which is
            successive sampling without replacement with probability
            proportional to w (Efraimidis and Spirakis, 2006).
"""
import os
from concurrent.futures import ProcessPoolExecutor
import multiprocessing as mp

import numpy as np

from .configs import Config, D, get_config

STREAM_Q, STREAM_K, STREAM_V, STREAM_OUTLIERS, STREAM_IDX, STREAM_ROWS = range(6)
CHUNK = 1024  # rows per independently seeded chunk
_WEIGHTED_SUB = 128  # rows per key matrix inside a weighted chunk (bounds memory)


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


# --------------------------------------------------------------------------- bf16


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); returns uint16 bits.

    Inputs are finite by construction (no NaN handling).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------- pools


def _default_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _map(fn, jobs, workers):
    if workers is None:
        workers = _default_workers()
    if workers <= 1 or len(jobs) <= 1:
        return [fn(j) for j in jobs]
    # spawn: the children never inherit a GPU context from the parent
    with ProcessPoolExecutor(max_workers=min(workers, len(jobs)),
                             mp_context=mp.get_context("spawn")) as ex:
        return list(ex.map(fn, jobs))


# --------------------------------------------------------------------------- Q, K, V


def _normal_chunk(job):
    seed, stream, head_key, c, n = job
    rng = _rng(seed, stream, head_key, c)
    return f32_to_bf16_bits(rng.standard_normal(n, dtype=np.float32))


def _normal_bf16(seed: int, stream: int, rows: int, row_elems: int, workers) -> np.ndarray:
    jobs = []
    for c in range((rows + CHUNK - 1) // CHUNK):
        n = (min(rows, (c + 1) * CHUNK) - c * CHUNK) * row_elems
        jobs.append((seed, stream, 0, c, n))
    parts = _map(_normal_chunk, jobs, workers)
    if not parts:
        return np.zeros(0, np.uint16)
    return np.concatenate(parts)


def make_qkv(cfg: Config, seed: int = None, workers=None):
    """bf16 Q [T,Hq,256], K and V [T,Hkv,256] as uint16 bit arrays, N(0,1) values.

    When the workload has outliers, one seeded set of round(frac*T) positions
    has its K and V rows multiplied by `outlier_scale` at every KV head (a
    power of two, so the bf16 values stay exact).
    """
    cfg = get_config(cfg)
    seed = cfg.number if seed is None else seed
    T, Hq, Hkv, Tk = cfg.T, cfg.Hq, cfg.Hkv, cfg.kv_len
    q = _normal_bf16(seed, STREAM_Q, T, Hq * D, workers).reshape(T, Hq, D)
    k = _normal_bf16(seed, STREAM_K, Tk, Hkv * D, workers).reshape(Tk, Hkv, D)
    v = _normal_bf16(seed, STREAM_V, Tk, Hkv * D, workers).reshape(Tk, Hkv, D)
    if cfg.outlier_frac > 0.0 and Tk > 0:
        pos = outlier_positions(cfg, seed)
        for a in (k, v):
            a[pos] = f32_to_bf16_bits(bf16_bits_to_f32(a[pos]) * np.float32(cfg.outlier_scale))
    return q, k, v


def outlier_positions(cfg: Config, seed: int = None) -> np.ndarray:
    cfg = get_config(cfg)
    seed = cfg.number if seed is None else seed
    Tk = cfg.kv_len
    if cfg.outlier_frac <= 0.0 or Tk == 0:
        return np.zeros(0, np.int64)
    n_out = int(round(cfg.outlier_frac * Tk))
    return np.sort(_rng(seed, STREAM_OUTLIERS).choice(Tk, size=n_out, replace=False))


# --------------------------------------------------------------------------- indices


def _uniform_distinct(rng, npop: np.ndarray, m: int) -> np.ndarray:
    """For each row i, m distinct offsets drawn uniformly from [0, npop[i])."""
    n = npop.shape[0]
    out = np.empty((n, m), np.int64)
    if n == 0 or m == 0:
        return out
    small = npop <= 4 * m
    if small.any():
        rows = np.nonzero(small)[0]
        width = int(npop[rows].max())
        keys = rng.random((rows.size, width))
        keys[np.arange(width)[None, :] >= npop[rows][:, None]] = 2.0
        out[rows] = np.argpartition(keys, m - 1, axis=1)[:, :m] if m < width else \
            np.argsort(keys, axis=1)[:, :m]
    if (~small).any():
        rows = np.nonzero(~small)[0]
        hi = npop[rows][:, None]
        x = rng.integers(0, hi, size=(rows.size, m))
        while True:
            x.sort(axis=1)
            dup = np.zeros(x.shape, bool)
            dup[:, 1:] = x[:, 1:] == x[:, :-1]
            if not dup.any():
                break
            r = np.nonzero(dup)[0]
            x[dup] = rng.integers(0, npop[rows][r])
        out[rows] = x
    return out


def _weighted_distinct(rng, tt: np.ndarray, lo: int, hi: np.ndarray, m: int) -> np.ndarray:
    """For each row i, m distinct positions in [lo, hi[i]] drawn without replacement
    with probability proportional to w(s) = 1 / (1 + (t_i - s) / 1024)."""
    n = tt.shape[0]
    out = np.empty((n, m), np.int64)
    for a in range(0, n, _WEIGHTED_SUB):
        b = min(n, a + _WEIGHTED_SUB)
        t = tt[a:b][:, None].astype(np.float64)
        width = int(hi[a:b].max()) - lo + 1
        s = lo + np.arange(width, dtype=np.float64)[None, :]
        logw = -np.log1p((t - s) / 1024.0)
        u = rng.random((b - a, width))
        keys = logw - np.log(-np.log(u))
        keys[s > hi[a:b][:, None]] = -np.inf
        if m < width:
            sel = np.argpartition(-keys, m - 1, axis=1)[:, :m]
        else:
            sel = np.argsort(-keys, axis=1)[:, :m]
        out[a:b] = sel + lo
    return out


def _position_lists(rng, pos: np.ndarray, K: int, window: int, sink: bool, gap: int,
                    sampler: str) -> np.ndarray:
    """Index lists [n, K] (int64, -1 padded) for queries at positions `pos`
    (in units of the list entries: tokens, or blocks for block lists)."""
    out = np.full((pos.size, K), -1, np.int64)
    if K == 0:
        return out
    dense = pos + 1 <= K
    for r in np.nonzero(dense)[0]:
        t = pos[r]
        out[r, : t + 1] = np.arange(t + 1)
    sparse_rows = np.nonzero(~dense)[0]
    if sparse_rows.size == 0:
        return out
    tt = pos[sparse_rows]
    lo = 1 if sink else 0
    hi = tt - window - gap
    m = K - window - (1 if sink else 0)
    if m > 0:
        if sampler == "uniform":
            rest = _uniform_distinct(rng, hi - lo + 1, m) + lo
        elif sampler == "weighted":
            rest = _weighted_distinct(rng, tt, lo, hi, m)
        else:
            raise ValueError(sampler)
    else:
        rest = np.zeros((tt.size, 0), np.int64)
    win = tt[:, None] - window + 1 + np.arange(window, dtype=np.int64)[None, :]
    parts = [rest, win]
    if sink:
        parts.insert(0, np.zeros((tt.size, 1), np.int64))
    full = np.concatenate(parts, axis=1)
    full.sort(axis=1)
    out[sparse_rows] = full
    return out


def _idx_chunk(job):
    (seed, c, g, T, K, window, sink, gap, sampler, q_pos0, shift) = job
    t0, t1 = c * CHUNK, min(T, (c + 1) * CHUNK)
    # absolute positions, in entry units (block number for block lists)
    pos = (np.arange(t0, t1, dtype=np.int64) + q_pos0) >> shift
    rng = _rng(seed, STREAM_IDX, g, c)
    return _position_lists(rng, pos, K, window, sink, gap, sampler).astype(np.int32)


def make_indices(cfg: Config, seed: int = None, rows=None, workers=None) -> np.ndarray:
    """int32 [T, Hkv, K] index lists (or [len(rows), Hkv, K] for a row subset).

    Entries are token positions, or micro-block numbers when the workload's
    block_size > 1 (row t then sits in block (q_pos0 + t) // block_size)."""
    cfg = get_config(cfg)
    seed = cfg.number if seed is None else seed
    T, Hkv, K = cfg.T, cfg.Hkv, cfg.K
    if cfg.window + (1 if cfg.sink else 0) > K:
        raise ValueError("window + sink exceed the selection width")
    n_chunks = (T + CHUNK - 1) // CHUNK
    chunks = range(n_chunks) if rows is None else sorted(set(int(r) // CHUNK for r in rows))
    shift = cfg.block_size.bit_length() - 1
    assert cfg.block_size == 1 << shift
    jobs = [(seed, c, g, T, K, cfg.window, cfg.sink, cfg.gap, cfg.sampler, cfg.q_pos0, shift)
            for c in chunks for g in range(Hkv)]
    parts = _map(_idx_chunk, jobs, workers)
    by_key = {(j[1], j[2]): p for j, p in zip(jobs, parts)}
    if rows is None:
        out = np.empty((T, Hkv, K), np.int32)
        for (c, g), p in by_key.items():
            out[c * CHUNK: c * CHUNK + p.shape[0], g, :] = p
        return out
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, Hkv, K), np.int32)
    for i, r in enumerate(rows):
        c = int(r) // CHUNK
        for g in range(Hkv):
            out[i, g, :] = by_key[(c, g)][int(r) - c * CHUNK]
    return out


def sample_rows(cfg: Config, n: int = None, seed: int = None) -> np.ndarray:
    """Sorted query rows for sampled parity checks: n seeded rows drawn without
    replacement plus the forced edge rows {0, 1, K-2, K-1, K, T-1}."""
    cfg = get_config(cfg)
    seed = cfg.number if seed is None else seed
    n = cfg.oracle_rows if n is None else n
    T, K = cfg.T, cfg.K
    if n <= 0 or n >= T:
        return np.arange(T, dtype=np.int64)
    picked = _rng(seed, STREAM_ROWS).choice(T, size=n, replace=False)
    forced = [r for r in (0, 1, K - 2, K - 1, K, T - 1) if 0 <= r < T]
    return np.unique(np.concatenate([picked, np.asarray(forced, np.int64)]))


def make_inputs(cfg, seed: int = None, workers=None) -> dict:
    """All operator inputs of a workload: dict(q, k, v, idx, scale, cfg)."""
    cfg = get_config(cfg)
    q, k, v = make_qkv(cfg, seed, workers)
    idx = make_indices(cfg, seed, workers=workers)
    return {"q": q, "k": k, "v": v, "idx": idx, "scale": cfg.scale, "cfg": cfg}
