#!/usr/bin/env python3
"""Benchmark of the QSA sparse-prefill operator on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload c4] [--graph]

A step is one call of the operator over the whole workload (all query tokens,
all heads): gather the selected K/V rows, scores, softmax, weighted values,
outputs. Inputs are generated on the host (seeded, synthetic), copied to HBM
once, and resident before the timed region starts. Prints one JSON line.

Default workload: T = 32768 query tokens, (Hq, Hkv) = (24, 2) -- the
24-query / 2-KV-head model of "Qwen4-Exp QSA llega al Ascend de Huawei",
section "Por qué QSA es la parte incómoda, en cifras" -- K = 2048 selected
slots per (token, KV head) (the page's 2,048 budget), head dim 256, bf16.

Roofline: the operator is a gather (G <= 12 flop per gathered byte against a
ridge of ~310), and every gathered byte reaches the waves through the
vector-memory return path: L2 (16 channels x 128 B/clk per XCD, 8 XCDs) to
the vector L1 and the texture-data unit of each CU (64 B/clk, 256 CUs), both
16 KiB per clock chip-wide, 39.3 TB/s at the 2.4 GHz peak clock. Most
gathered rows repeat across neighbouring queries and are served from L2, so
that path, not HBM, binds the cache-resident workloads. `achieved` is the
algorithmic bytes per launch (512 B of K + 512 B of V per valid slot) over
the mean kernel duration, measured with a HIP event pair around the K timed
steps on the stream the kernel runs on. A second pass of K steps, each
between its own events, gives the minimum and median launch durations.
`traffic` is what crosses L2 to the fabric per launch (Infinity Cache hits
and HBM), from committed rocprofv3 counter runs of this same command: reads
from the L2's own request counts by size (32, 64 and 128 B), writes from
WRITE_SIZE; `past_l2` sets it against the 8 TB/s HBM peak. Both are reported
only while the built library is byte-identical to the one the counters were
taken on. `hbm_roofline_frac` is the metric's logical figure (gathered bytes
over 8 TB/s): above 1 whenever caches serve the gather, so not a roofline.

Other workloads (--workload): any of the token workloads c1..c6, the
micro-block workloads c7/c8 (entries name 4-token blocks, the model's
compression ratio), the ragged slot-pool batches c9/c10/c13 and the decode
batches c11/c12 (one query per request; the step includes the merge of the
split lists). Each is timed the same way through its own entry point.

With --graph the timed calls are replayed from a captured HIP graph rather
than launched one host call at a time; the microsecond workloads are
otherwise bound by the host's per-call work. The line's `launch` field says
which.
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
# L2 -> CU return path: 8 XCDs x 16 L2 channels x 128 B per clock (= 256 CUs x
# 64 B per clock into the texture-data units) at the 2.4 GHz peak clock
L2_CU_BYTES_PER_CLK = 8 * 16 * 128
PEAK_CLOCK_HZ = 2.4e9
L2_CU_PEAK_GBPS = L2_CU_BYTES_PER_CLK * PEAK_CLOCK_HZ / 1e9
LIBRARY = "top_sparse_attention_qsa_amd/lib/libqsa.so"
PROBE = "top_sparse_attention_qsa_amd/lib/qsa_gather_probe"
# the library's occupancy rule: one 4-wave block per CU for caches of 81,920
# rows or more with 32,768 work items or more, two blocks otherwise
ONE_BLOCK_ROWS, ONE_BLOCK_ITEMS = 81920, 32768
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
    """Counter record of this workload's kernel (bytes per launch past L2, the
    clock under load) from its committed summary, or None when absent or
    taken on another build of the library."""
    path = os.path.join(ROOT, "profiles", f"qsa_prefill_kernel_{workload}_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_sha") != sha or "read_bytes_per_launch" not in rec:
        return None
    return rec


def roofline_records(gathered: int, kernel_s: float, counters):
    """The `roofline` and `past_l2` objects for `gathered` algorithmic bytes
    per launch and a mean launch of `kernel_s` seconds; `counters` is the
    workload's counter record (measured_traffic) or None."""
    achieved = gathered / kernel_s / 1e9
    traffic = None if counters is None else int(round(counters["read_bytes_per_launch"]
                                                      + counters["write_bytes_per_launch"]))
    roofline = {
        "bound": "l2",
        "bound_detail": "vector-memory return path: L2 (8 XCDs x 16 channels x 128 B/clk) to the CUs' "
                        "vector L1 / texture-data units (256 x 64 B/clk) = 16 KiB/clk at 2.4 GHz; every "
                        "gathered K/V byte crosses it",
        "achieved": round(achieved, 1),
        "peak": round(L2_CU_PEAK_GBPS, 1),
        "unit": "GB/s",
        "frac": round(achieved / L2_CU_PEAK_GBPS, 4),
        "traffic": traffic,
        "traffic_kind": "bytes per launch from L2 to the fabric (Infinity Cache hits and HBM), reads from "
                        "the L2's 32/64/128-B request counts, writes from WRITE_SIZE",
        "kernel": "qsa_prefill_kernel",
        "algorithmic_bytes_per_launch": gathered,
    }
    if counters is not None and counters.get("clock_hz"):
        # the same fraction at the clock the counters measured under this load
        clk = counters["clock_hz"]
        roofline["profiled_clock_GHz"] = round(clk / 1e9, 3)
        roofline["frac_at_profiled_clock"] = round(achieved / (L2_CU_BYTES_PER_CLK * clk / 1e9), 4)
    past_l2 = None
    if traffic is not None:
        past_l2 = {"bytes_per_launch": traffic, "GBps": round(traffic / kernel_s / 1e9, 1),
                   "frac_of_hbm_peak": round(traffic / kernel_s / 1e9 / HBM_PEAK_GBPS, 4),
                   "gathered_bytes_from_l2_frac": round(1 - counters["read_bytes_per_launch"] / gathered, 4)}
    return roofline, past_l2


def kernel_waves_per_cu(cfg):
    """Waves per CU the gather kernel runs this workload with (None for the
    decode batches, whose split ranges run in one-wave blocks)."""
    from qsa_inputs import PoolConfig

    if isinstance(cfg, PoolConfig):
        if cfg.decode:
            return None
        n_rows = cfg.n_slots
    else:
        n_rows = cfg.kv_len
    items = cfg.T * cfg.Hkv * ((cfg.Hq // cfg.Hkv + 15) // 16)
    return 4 if n_rows >= ONE_BLOCK_ROWS and items >= ONE_BLOCK_ITEMS else 8


def parse_probe(text: str):
    """GB/s from the gather probe's output line, or None."""
    import re

    m = re.search(r"([\d.]+) TB/s", text)
    return float(m.group(1)) * 1000.0 if m else None


def measure_gather_ceiling(waves_per_cu: int):
    """The gather probe on L2-resident rows (8,192 rows of 512 B) at the
    kernel's waves per CU, 16 loads in flight per wave (16 KB, as the kernel
    holds): GB/s received by the waves, median of 5 launches; None when the
    probe is not built or fails."""
    import subprocess

    path = os.path.join(ROOT, PROBE)
    if waves_per_cu is None or not os.path.exists(path):
        return None
    try:
        res = subprocess.run([path, "8192", str(waves_per_cu), "200", "16", "5"], capture_output=True, text=True,
                             timeout=120)
    except (OSError, subprocess.TimeoutExpired):
        return None
    return parse_probe(res.stdout) if res.returncode == 0 else None


def load_inputs(cfg):
    """Host arrays of a workload: dict(q, k, v, idx[, q_pos, slot_pos])."""
    from qsa_inputs import PoolConfig, make_indices, make_pool_inputs, make_qkv

    if isinstance(cfg, PoolConfig):
        d = make_pool_inputs(cfg)
        return {n: d[n] for n in ("q", "k", "v", "idx", "q_pos", "slot_pos")}
    q, k, v = make_qkv(cfg)
    return {"q": q, "k": k, "v": v, "idx": make_indices(cfg)}


def cpu_baseline(cfg, d, n_rows: int):
    """The fp64 oracle, as it is, on a seeded sample of the workload's rows:
    ((rows, out, lse) it computed, the timing record)."""
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
    affinity = pool.affinity_cpus()
    ref_out, ref_lse, secs = pool.run_rows(d["q"], d["k"], d["v"], d["idx"][rows], rows, cfg.scale,
                                           workers=workers, return_seconds=True, **kw)
    reference = (rows, ref_out, ref_lse)
    return reference, {
        "value": round(float(rows.size / secs), 3),
        "unit": "query-tokens/s",
        "cores": workers,
        "affinity_cpus": affinity,
        "kind": "oracle",
        "sample": f"{rows.size} seeded rows of {cfg.name} (all {cfg.Hq} heads each), fp64 NumPy, "
                  f"{workers} processes (one per core; {affinity} CPUs in this process's affinity set, "
                  f"at most {pool.MAX_WORKERS} used), BLAS single-threaded; {secs:.2f} s wall",
    }


def parity_record(rows, ref_out, ref_lse, out_bits, lse):
    """The GPU's outputs on the rows the CPU baseline computed, against the
    oracle's: max |out| and |lse| errors, rel-L2, and whether every element
    is within 1e-2 plus half a bf16 ulp of the oracle (every finite lse within
    1e-3, every empty row +0.0 with lse -inf on both sides)."""
    import numpy as np

    g = (np.asarray(out_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    g = g.astype(np.float64)
    err = np.abs(g - ref_out)
    _, ex = np.frexp(np.abs(ref_out))
    bound = 1e-2 + np.ldexp(1.0, np.maximum(ex, -125) - 9)
    fin = np.isfinite(ref_lse)
    lse = np.asarray(lse, dtype=np.float64)
    lerr = np.abs(lse[fin] - ref_lse[fin])
    same_empty = bool(np.array_equal(np.isfinite(lse), fin) and np.all(lse[~fin] == ref_lse[~fin]))
    outside = int(np.count_nonzero(err > bound))
    max_lse = float(lerr.max()) if lerr.size else 0.0
    return {
        "rows_checked": int(np.asarray(rows).size),
        "max_abs_out": float(err.max()) if err.size else 0.0,
        "max_abs_lse": max_lse,
        "rel_l2": float(np.linalg.norm(g - ref_out) / max(np.linalg.norm(ref_out), 1e-300)) if err.size else 0.0,
        "outside_bar": outside,
        "within_bar": bool(outside == 0 and max_lse <= 1e-3 and same_empty),
        "bar": "|out - oracle| <= 1e-2 + half a bf16 ulp of the oracle; |lse - oracle| <= 1e-3 on finite lse",
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
    ap.add_argument("--graph", action="store_true",
                    help="launch the timed calls from a captured HIP graph (the timed region replays one graph of "
                         "--steps calls) instead of one host call each: the same kernels without the host's "
                         "per-call work, as a serving loop would run them (the per-launch pass stays eager: "
                         "a one-call graph adds the graph's own launch time)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the operator "
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

    cpu = reference = None
    if not args.no_cpu_baseline and args.cpu_rows > 0:
        t0 = time.perf_counter()
        reference, cpu = cpu_baseline(cfg, d, args.cpu_rows)
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
    # what this GPU delivers to the waves for random 512-B rows held in L2, at
    # the kernel's occupancy (a separate process, before the timed region)
    wpc = kernel_waves_per_cu(cfg)
    ceiling = measure_gather_ceiling(wpc)

    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    cold0, cold1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cold0.record(stream)
    step()
    cold1.record(stream)
    for _ in range(max(0, args.warmup - 1)):
        step()
    torch.cuda.synchronize()
    first_ms = cold0.elapsed_time(cold1)

    if args.graph:
        # the same calls, captured after the warm-up (the library allocates
        # nothing and never synchronises, so every call is capturable)
        graph_all = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph_all):
            for _ in range(args.steps):
                step()
        torch.cuda.synchronize()
        timed_calls = graph_all.replay
    else:
        def timed_calls():
            for _ in range(args.steps):
                step()

    # the timed region: K steps back to back, one HIP event pair around them
    # (an event pair per step costs host time that a microsecond decode step
    # would show)
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    r0.record(stream)
    timed_calls()
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
    # the allocator's peak over the calls (read before the parity check below,
    # whose row gathers allocate copies of the outputs)
    peak_bytes = int(torch.cuda.max_memory_allocated(dev))

    ms_per_step = wall * 1e3 / args.steps
    gathered = cfg.gathered_bytes()
    kernel_s = region_ms * 1e-3
    achieved = gathered / kernel_s / 1e9
    sha = kernel_sha()
    counters = measured_traffic(cfg.name, sha)
    qtok_s = cfg.T / (ms_per_step * 1e-3)
    logical_gbps = gathered / (ms_per_step * 1e-3) / 1e9

    # the outputs of the last timed call, on the rows the oracle computed
    parity = None
    if reference is not None:
        rows_chk, ref_out, ref_lse = reference
        sel = torch.from_numpy(np.asarray(rows_chk, dtype=np.int64)).to(dev)
        got = out.index_select(0, sel).view(torch.int16).cpu().numpy().view(np.uint16)
        got_lse = lse.index_select(0, sel).cpu().numpy()
        parity = parity_record(rows_chk, ref_out, ref_lse, got, got_lse)
        del ref_out, ref_lse, reference

    roofline, past_l2 = roofline_records(gathered, kernel_s, counters)
    if ceiling:
        roofline["measured_ceiling"] = {
            "GBps": round(ceiling, 1), "waves_per_cu": wpc, "frac": round(achieved / ceiling, 4),
            "what": "qsa_gather_probe in this run: random 512-B row pairs from an L2-resident 4 MB buffer, the "
                    "kernel's load shape and waves per CU, 16 loads in flight per wave, no other work"}
    roofline.update(kernel_ms_mean=round(region_ms, 4), kernel_ms_min=round(float(kms.min()), 4),
                    kernel_ms_median=round(float(np.median(kms)), 4),
                    kernel_ms_mean_per_launch_pass=round(float(kms.mean()), 4), kernel_sha=sha)

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
        "launch": "hip_graph" if args.graph else "eager",
        "gathered_kv_GBps": round(logical_gbps, 1),
        "hbm_roofline_frac": round(logical_gbps / HBM_PEAK_GBPS, 4),
        "copy_roofline_frac": round(logical_gbps / copy_gbps, 4),
        "roofline": roofline,
        "past_l2": past_l2,
        "first_call_ms": round(first_ms, 3),
        "copy_GBps": round(copy_gbps, 1),
        "useful_tflops": round(cfg.useful_flops() / kernel_s / 1e12, 2),
        "device_memory": {"max_allocated_bytes": peak_bytes,
                          "max_allocated_MiB": round(peak_bytes / 2 ** 20, 1),
                          "note": "PyTorch allocator peak over the timed calls: resident inputs, outputs "
                                  "and any decode workspace; the library itself allocates nothing"},
        "cpu_baseline": cpu,
        "parity": parity,
        "device": {"name": torch.cuda.get_device_name(dev),
                   "arch": getattr(torch.cuda.get_device_properties(dev), "gcnArchName", None),
                   "hip": torch.version.hip, "torch": torch.__version__},
        "gpu_over_cpu": round(qtok_s / cpu["value"], 1) if cpu else None,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
