"""Seeded ragged batches over one K/V slot pool (host, NumPy).

A batch is a list of requests (see `configs.Request`). Every token of every
request is held by one pool slot; a request that shares a prefix with an
earlier one uses that request's slots for the shared tokens. The slots of all
distinct tokens, plus `free_slots` slots that hold no token, are a seeded
random permutation of 0 .. n_slots - 1, so a request's tokens sit in the pool
in no particular order.

Returned arrays:
  q         uint16 [total_q, Hq, 256]   bf16 bits, query rows of all requests
  k, v      uint16 [n_slots, Hkv, 256]  bf16 bits, the pool (free slots too)
  idx       int32  [total_q, Hkv, K]    pool slots, -1 padded
  q_pos     int32  [total_q]            position of each row in its request
  slot_pos  int32  [n_slots]            position of the token in each slot,
                                        -1 for a free slot
  requests  list of dict(rows=(a, b), cached, new, table) where table is the
            int64 [cached + new] slot of each of the request's positions

Per-query lists use the token recipe of `generate` over the query's own
request positions, then name the slots of the chosen positions. Like the
rest of this package it holds none of the operator's arithmetic.
"""
import numpy as np

from .configs import D, PoolConfig, get_config
from .generate import CHUNK, _map, _normal_bf16, _position_lists, _rng

STREAM_POOL_Q, STREAM_POOL_K, STREAM_POOL_V, STREAM_POOL_SLOTS, STREAM_POOL_IDX = range(16, 21)


def slot_tables(cfg: PoolConfig, seed: int = None):
    """(tables, slot_pos): tables[r] int64 [cached + new] slots of request r's
    positions; slot_pos int32 [n_slots] (-1: free)."""
    cfg = get_config(cfg)
    seed = cfg.number if seed is None else seed
    perm = _rng(seed, STREAM_POOL_SLOTS).permutation(cfg.n_slots).astype(np.int64)
    tables = []
    nxt = 0  # next unused entry of the permutation
    for i, r in enumerate(cfg.requests):
        if r.share_from >= 0:
            if r.share_from >= i:
                raise ValueError("a shared prefix must come from an earlier request")
            src = tables[r.share_from]
            if src.size < r.cached:
                raise ValueError("shared prefix longer than its source request")
            prefix = src[: r.cached]
            own = perm[nxt: nxt + r.new]
            nxt += r.new
        else:
            prefix = perm[nxt: nxt + r.cached]
            own = perm[nxt + r.cached: nxt + r.cached + r.new]
            nxt += r.cached + r.new
        tables.append(np.concatenate([prefix, own]))
    assert nxt == cfg.n_tokens
    slot_pos = np.full(cfg.n_slots, -1, np.int32)
    for t in tables:
        slot_pos[t] = np.arange(t.size, dtype=np.int32)
    return tables, slot_pos


def _pool_idx_chunk(job):
    seed, r, g, c, cached, new, K, window, sink, gap, sampler = job
    t0, t1 = c * CHUNK, min(new, (c + 1) * CHUNK)
    pos = cached + np.arange(t0, t1, dtype=np.int64)
    rng = _rng(seed, STREAM_POOL_IDX, r, g, c)
    return _position_lists(rng, pos, K, window, sink, gap, sampler)


def make_pool_inputs(cfg, seed: int = None, workers=None) -> dict:
    """All operator inputs of a ragged pool batch (see the module docstring)."""
    cfg = get_config(cfg)
    if not isinstance(cfg, PoolConfig):
        raise TypeError(f"{cfg.name} is not a pool workload")
    seed = cfg.number if seed is None else seed
    tables, slot_pos = slot_tables(cfg, seed)
    total_q, Hq, Hkv, K = cfg.total_q, cfg.Hq, cfg.Hkv, cfg.K
    q = _normal_bf16(seed, STREAM_POOL_Q, total_q, Hq * D, workers).reshape(total_q, Hq, D)
    k = _normal_bf16(seed, STREAM_POOL_K, cfg.n_slots, Hkv * D, workers).reshape(cfg.n_slots, Hkv, D)
    v = _normal_bf16(seed, STREAM_POOL_V, cfg.n_slots, Hkv * D, workers).reshape(cfg.n_slots, Hkv, D)
    jobs = []
    for r, req in enumerate(cfg.requests):
        for g in range(Hkv):
            for c in range((req.new + CHUNK - 1) // CHUNK):
                jobs.append((seed, r, g, c, req.cached, req.new, K, cfg.window, cfg.sink, cfg.gap,
                             cfg.sampler))
    parts = _map(_pool_idx_chunk, jobs, workers)
    idx = np.full((total_q, Hkv, K), -1, np.int32)
    q_pos = np.empty(total_q, np.int32)
    starts = np.cumsum([0] + [r.new for r in cfg.requests])
    requests = []
    for r, req in enumerate(cfg.requests):
        a = int(starts[r])
        q_pos[a: a + req.new] = req.cached + np.arange(req.new, dtype=np.int32)
        requests.append({"rows": (a, a + req.new), "cached": req.cached, "new": req.new,
                         "table": tables[r]})
    for job, pos_lists in zip(jobs, parts):
        _, r, g, c = job[:4]
        a = int(starts[r]) + c * CHUNK
        table = tables[r]
        slots = np.where(pos_lists >= 0, table[np.maximum(pos_lists, 0)], -1)
        idx[a: a + pos_lists.shape[0], g, :] = slots.astype(np.int32)
    return {"q": q, "k": k, "v": v, "idx": idx, "q_pos": q_pos, "slot_pos": slot_pos,
            "requests": requests, "scale": cfg.scale, "cfg": cfg}


def sample_pool_rows(cfg, n: int = None, seed: int = None) -> np.ndarray:
    """Sorted query rows for sampled parity checks: n seeded rows plus the
    first and last row of every request."""
    cfg = get_config(cfg)
    seed = cfg.number if seed is None else seed
    n = cfg.oracle_rows if n is None else n
    T = cfg.total_q
    if n <= 0 or n >= T:
        return np.arange(T, dtype=np.int64)
    picked = _rng(seed, STREAM_POOL_SLOTS + 100).choice(T, size=n, replace=False)
    starts = np.cumsum([0] + [r.new for r in cfg.requests])
    forced = [int(s) for s in starts[:-1]] + [int(s) - 1 for s in starts[1:]]
    return np.unique(np.concatenate([picked, np.asarray(forced, np.int64)]))
