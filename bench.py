#!/usr/bin/env python3
"""Benchmark of the QSA sparse-prefill operator on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload c4]

A step is one call of the operator over the whole workload (all query tokens,
all heads): gather the selected K/V rows, scores, softmax, weighted values,
outputs. Inputs are generated on the host (seeded, synthetic), copied to HBM
once, and resident before the timed region starts. Prints one JSON line.

Default workload: T = 32768 query tokens, (Hq, Hkv) = (24, 2) -- the
24-query / 2-KV-head model of "Qwen4-Exp QSA llega al Ascend de Huawei",
section "Por qué QSA es la parte incómoda, en cifras" -- K = 2048 selected
slots per (token, KV head) (the page's 2,048 budget), head dim 256, bf16.

Roofline: the kernel is bound by HBM bandwidth on the gathered rows. Per
valid slot it must gather 512 B of K and 512 B of V; `achieved` is those
algorithmic bytes per launch divided by the mean kernel duration, measured
with a HIP event pair around the K timed steps on the stream the kernel runs
on, against MI355X's 8 TB/s. A second pass of K steps, each between its own
events, gives the minimum and median launch durations.
`traffic` comes from committed rocprofv3 FETCH_SIZE / WRITE_SIZE counter runs
of this same command, scaled by the counters' reading on a copy kernel of
known size, and is reported only while the built library is byte-identical
to the one the counters were taken on.

Other workloads (--workload): any of the token workloads c1..c6, the
micro-block workloads c7/c8 (entries name 4-token blocks, the model's
compression ratio), the ragged slot-pool batches c9/c10/c13 and the decode
batches c11/c12 (one query per request; the step includes the merge of the
split lists). Each is timed the same way through its own entry point.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
LIBRARY = "top_sparse_attention_qsa_amd/lib/libqsa.so"
METRIC = "QSA sparse prefill query-tokens/s and gathered-KV GB/s (% HBM roofline), 1 GPU"


def kernel_sha() -> str:
    """First 16 hex digits of the sha256 of the built library: the code that
    runs (the build is deterministic, so comment-only edits keep it)."""
    h = hashlib.sha256()
    with open(os.path.join(ROOT, LIBRARY), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def measured_traffic(workload: str, sha: str):
    """Bytes per launch moved past L2 (FETCH_SIZE + WRITE_SIZE, calibrated), from the
    committed counter summary of this workload, or None when absent or stale."""
    path = os.path.join(ROOT, "profiles", f"qsa_prefill_kernel_{workload}_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_sha") != sha:
        return None
    return int(round(rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]))


def load_inputs(cfg):
    """Host arrays of a workload: dict(q, k, v, idx[, q_pos, slot_pos])."""
    from qsa_inputs import PoolConfig, make_indices, make_pool_inputs, make_qkv

    if isinstance(cfg, PoolConfig):
        d = make_pool_inputs(cfg)
        return {n: d[n] for n in ("q", "k", "v", "idx", "q_pos", "slot_pos")}
    q, k, v = make_qkv(cfg)
    return {"q": q, "k": k, "v": v, "idx": make_indices(cfg)}


def cpu_baseline(cfg, d, n_rows: int):
    """The fp64 oracle, as it is, on a seeded sample of the workload's rows."""
    from oracle import pool
    from qsa_inputs import PoolConfig, sample_pool_rows, sample_rows

    if isinstance(cfg, PoolConfig):
        rows = sample_pool_rows(cfg, n=n_rows, seed=cfg.number + 1000)
        kw = {"q_pos": d["q_pos"], "slot_pos": d["slot_pos"]}
    else:
        rows = sample_rows(cfg, n=n_rows, seed=cfg.number + 1000)
        kw = {"q_pos0": cfg.q_pos0, "block_size": cfg.block_size if cfg.block_size > 1 else None}
    rows = rows[:n_rows]
    workers = pool.default_workers()
    _, _, secs = pool.run_rows(d["q"], d["k"], d["v"], d["idx"][rows], rows, cfg.scale, workers=workers,
                               return_seconds=True, **kw)
    return {
        "value": round(float(rows.size / secs), 3),
        "unit": "query-tokens/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"{rows.size} seeded rows of {cfg.name} (all {cfg.Hq} heads each), fp64 NumPy, "
                  f"one process per core, BLAS single-threaded; {secs:.2f} s wall",
    }


def workload_config(cfg) -> dict:
    from qsa_inputs import PoolConfig

    c = {"workload": cfg.name, "T": cfg.T, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "head_dim": 256, "K": cfg.K,
         "scale": cfg.scale}
    if isinstance(cfg, PoolConfig):
        c.update(requests=[{"new": r.new, "cached": r.cached, "share_from": r.share_from} for r in cfg.requests],
                 n_slots=cfg.n_slots, free_slots=cfg.free_slots)
    else:
        c.update(q_pos0=cfg.q_pos0, T_kv=cfg.kv_len, block_size=cfg.block_size)
    c.update(index_lists=cfg.description, valid_slots=cfg.valid_slots(), parallelism="single GPU")
    return c


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c4", help="c1..c13 or a workload name (default c4)")
    ap.add_argument("--cpu-rows", type=int, default=32768,
                    help="rows for the oracle CPU baseline (all 32,768 rows of the default workload: about 9 s on 16 cores)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (the operator "
              "would shard over query rows or KV heads with no exchange after the kernel). "
              "Run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        ap.error("--steps must be >= 1 and --warmup >= 0")

    import numpy as np
    import torch

    import top_sparse_attention_qsa_amd as qsa
    from qsa_inputs import PoolConfig, get_config

    cfg = get_config(args.workload)
    t0 = time.perf_counter()
    d = load_inputs(cfg)
    log(f"{cfg.name}: inputs generated in {time.perf_counter() - t0:.1f}s")

    cpu = None
    if not args.no_cpu_baseline and args.cpu_rows > 0:
        t0 = time.perf_counter()
        cpu = cpu_baseline(cfg, d, args.cpu_rows)
        log(f"cpu baseline {cpu['value']} q-tok/s on {cpu['cores']} cores ({time.perf_counter() - t0:.1f}s)")

    if not torch.cuda.is_available():
        print("bench.py needs a GPU (no HIP device visible)", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    qsa.load_library()
    to_bf16 = lambda a: torch.from_numpy(a).view(torch.bfloat16).to(dev)
    dq, dk, dv = to_bf16(d["q"]), to_bf16(d["k"]), to_bf16(d["v"])
    didx = torch.from_numpy(d["idx"]).to(dev)
    out = torch.empty((cfg.T, cfg.Hq, 256), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((cfg.T, cfg.Hq), dtype=torch.float32, device=dev)
    if isinstance(cfg, PoolConfig):
        dqp, dsp = torch.from_numpy(d["q_pos"]).to(dev), torch.from_numpy(d["slot_pos"]).to(dev)
    del d

    if isinstance(cfg, PoolConfig) and cfg.decode:
        n_ws = qsa.decode_workspace_bytes(cfg.T, cfg.Hq, cfg.Hkv, cfg.K)
        ws = torch.empty(max(n_ws, 1), dtype=torch.uint8, device=dev)

    def step():
        if isinstance(cfg, PoolConfig) and cfg.decode:
            qsa.sparse_decode(dq, dk, dv, didx, dqp, dsp, scale=cfg.scale, out=out, lse=lse, workspace=ws)
        elif isinstance(cfg, PoolConfig):
            qsa.sparse_prefill_pool(dq, dk, dv, didx, dqp, dsp, scale=cfg.scale, out=out, lse=lse)
        elif cfg.block_size > 1:
            qsa.sparse_prefill_blocks(dq, dk, dv, didx, cfg.q_pos0, cfg.block_size, scale=cfg.scale, out=out,
                                      lse=lse)
        elif cfg.q_pos0:
            qsa.sparse_prefill_extend(dq, dk, dv, didx, cfg.q_pos0, scale=cfg.scale, out=out, lse=lse)
        else:
            qsa.sparse_prefill(dq, dk, dv, didx, scale=cfg.scale, out=out, lse=lse)

    # a plain copy of known size: context for the bandwidth and the counters' scale
    copy_bytes = 1 << 30
    src = torch.empty(copy_bytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(2):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)
    c1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * copy_bytes * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst

    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()
    cold0, cold1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cold0.record(stream)
    step()
    cold1.record(stream)
    for _ in range(max(0, args.warmup - 1)):
        step()
    torch.cuda.synchronize()
    first_ms = cold0.elapsed_time(cold1)

    # the timed region: K steps back to back, one HIP event pair around them
    # (an event pair per step costs host time that a microsecond decode step
    # would show)
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    r0.record(stream)
    for _ in range(args.steps):
        step()
    r1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    region_ms = r0.elapsed_time(r1) / args.steps

    # then K more steps, each between its own events: the spread of launch durations
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    kms = np.array([e0.elapsed_time(e1) for e0, e1 in evs])

    ms_per_step = wall * 1e3 / args.steps
    gathered = cfg.gathered_bytes()
    kernel_s = region_ms * 1e-3
    achieved = gathered / kernel_s / 1e9
    sha = kernel_sha()
    traffic = measured_traffic(cfg.name, sha)
    qtok_s = cfg.T / (ms_per_step * 1e-3)

    res = {
        "metric": METRIC,
        "value": round(qtok_s, 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": workload_config(cfg),
        "gathered_kv_GBps": round(gathered / (ms_per_step * 1e-3) / 1e9, 1),
        "hbm_roofline_frac": round(gathered / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "copy_roofline_frac": round(gathered / (ms_per_step * 1e-3) / 1e9 / copy_gbps, 4),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "kernel": "qsa_prefill_kernel",
            "algorithmic_bytes_per_launch": gathered,
            "kernel_ms_mean": round(region_ms, 4),
            "kernel_ms_min": round(float(kms.min()), 4),
            "kernel_ms_median": round(float(np.median(kms)), 4),
            "kernel_ms_mean_per_launch_pass": round(float(kms.mean()), 4),
            "kernel_sha": sha,
        },
        "first_call_ms": round(first_ms, 3),
        "copy_GBps": round(copy_gbps, 1),
        "useful_tflops": round(cfg.useful_flops() / kernel_s / 1e12, 2),
        "cpu_baseline": cpu,
        "gpu_over_cpu": round(qtok_s / cpu["value"], 1) if cpu else None,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
