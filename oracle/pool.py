"""Run the fp64 oracle over many query rows in a process pool.

TEST INFRASTRUCTURE ONLY (test suite, smoke check, benchmark CPU baseline).
The arrays are written once to a temporary directory as .npy files and
memory-mapped by each worker; workers are started with the "spawn" method so
they never inherit a GPU context. Each worker evaluates a contiguous chunk of
the requested rows with the oracle function of the call's form, unchanged:
`sparse_prefill` (token lists), `sparse_prefill_blocks` (micro-block lists)
or `sparse_prefill_pool` (slot lists over a K/V pool).
"""
import os
import shutil
import tempfile
import time
from concurrent.futures import ProcessPoolExecutor
import multiprocessing as mp

import numpy as np

from . import qsa_oracle

_ARRAYS = {}


# Worker processes are capped at 16: one GPU's share of a multi-GPU host's
# cores, whatever the process's affinity set shows.
MAX_WORKERS = 16


def affinity_cpus() -> int:
    """CPUs in this process's affinity set."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def default_workers() -> int:
    return max(1, min(MAX_WORKERS, affinity_cpus()))


def _init(paths):
    # one process per core: keep each worker's BLAS single-threaded
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:  # pragma: no cover
        pass
    for name, path in paths.items():
        _ARRAYS[name] = np.load(path, mmap_mode="r")


def _evaluate(arrays, rows, idx_rows, scale, q_pos0, block_size):
    q, k, v = arrays["q"], arrays["k"], arrays["v"]
    if "slot_pos" in arrays:
        return qsa_oracle.sparse_prefill_pool(q, k, v, idx_rows, arrays["q_pos"], arrays["slot_pos"],
                                              scale=scale, rows=rows)
    if block_size is not None:
        return qsa_oracle.sparse_prefill_blocks(q, k, v, idx_rows, block_size, scale=scale, rows=rows,
                                                q_pos0=q_pos0)
    return qsa_oracle.sparse_prefill(q, k, v, idx_rows, scale=scale, rows=rows, q_pos0=q_pos0)


def _chunk(args):
    rows, idx_rows, scale, q_pos0, block_size = args
    return _evaluate(_ARRAYS, rows, idx_rows, scale, q_pos0, block_size)


def run_rows(q, k, v, idx_rows, rows, scale, q_pos0: int = 0, workers: int = None,
             return_seconds: bool = False, block_size: int = None, q_pos=None, slot_pos=None):
    """Oracle outputs for query `rows`; idx_rows holds those rows' index lists.

    Token lists by default; micro-block lists when `block_size` is given;
    pool slot lists when `q_pos` and `slot_pos` are given (k and v are then
    the pool). Returns (out [R, Hq, 256] float64, lse [R, Hq] float64), plus
    the wall time of the evaluation itself (excluding worker start-up) when
    asked.
    """
    rows = np.asarray(rows, dtype=np.int64)
    idx_rows = np.asarray(idx_rows)
    assert idx_rows.shape[0] == rows.size
    assert (q_pos is None) == (slot_pos is None)
    arrays = {"q": q, "k": k, "v": v}
    if slot_pos is not None:
        arrays.update(q_pos=np.asarray(q_pos), slot_pos=np.asarray(slot_pos))
    workers = default_workers() if workers is None else workers
    if workers <= 1 or rows.size < 2:
        t0 = time.perf_counter()
        res = _evaluate(arrays, rows, idx_rows, scale, q_pos0, block_size)
        dt = time.perf_counter() - t0
        return (res + (dt,)) if return_seconds else res
    tmp = tempfile.mkdtemp(prefix="qsa_oracle_", dir="/dev/shm" if os.path.isdir("/dev/shm") else None)
    try:
        paths = {}
        for name, a in arrays.items():
            paths[name] = os.path.join(tmp, name + ".npy")
            np.save(paths[name], np.ascontiguousarray(a))
        n_chunks = min(rows.size, workers * 4)
        bounds = np.linspace(0, rows.size, n_chunks + 1).astype(int)
        jobs = [(rows[a:b], idx_rows[a:b], scale, q_pos0, block_size)
                for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
        with ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn"),
                                 initializer=_init, initargs=(paths,)) as ex:
            list(ex.map(_init_probe, range(workers)))  # start every worker before timing
            t0 = time.perf_counter()
            parts = list(ex.map(_chunk, jobs))
            dt = time.perf_counter() - t0
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    out = np.concatenate([p[0] for p in parts])
    lse = np.concatenate([p[1] for p in parts])
    return (out, lse, dt) if return_seconds else (out, lse)


def _init_probe(_):
    return len(_ARRAYS)
