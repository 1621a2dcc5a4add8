"""Benchmark: one decode step of paged attention on one MI355X.

A step is the whole hot path over one batch: the copy-on-write block copies
(none for workloads without shared partial blocks), the cache write of every
sequence's newest token, and paged decode attention (partition kernel plus
split-K reduce when contexts span several partitions).  Inputs are synthetic
and seeded and already resident in HBM when timing starts.

Prints ONE JSON line.  ``value`` is KV-read GB/s over the whole step:
algorithmic K+V bytes (sum of context lengths x KV heads x head dim x 2 x
element bytes) divided by the step time.  ``roofline`` reports the decode
partition kernel alone (HIP events recorded around that kernel on its
stream) against the MI355X HBM peak of 8 TB/s.  ``cpu_baseline`` times the
fp64 CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "pa_decode KV-read GB/s (% of HBM peak) + decode seqs/s at 1 MI355X"
WORKLOAD_TEXT = {
    "gqa70b": "70B-like GQA layer: 256 seqs x 4096 tokens, 64 q heads / 8 KV heads, head_dim 128, "
              "bf16 KV, 16-token blocks scattered over a 65536-block pool",
    "mha13b": "13B-like MHA layer: 32 seqs, contexts uniform in [1, 2048], 40 heads, head_dim 128, "
              "bf16 KV, 16-token blocks scattered",
    "fp8": "FP8 KV cache, long tail: 128 seqs, lognormal contexts (median 2048, clipped "
           "[16, 32768]), 64 q / 8 KV heads, head_dim 128, e4m3 K/V, bf16 q, 512-token partitions",
    "sampling_a": "parallel sampling: 64 prompts x 3 samples, 1024-token shared prompts + 0..512 "
                  "private tokens, 40 q / 8 KV heads, head_dim 128, bf16",
    "sampling_b": "parallel sampling with copy-on-write: 64 prompts x 3 samples, 1016-token shared "
                  "prompts + 0..512 private tokens, 40 q / 8 KV heads, head_dim 128, bf16",
    "tiny": "worked example: 1 seq x 40 tokens, 1 head, head_dim 64, fp32, 3 random blocks of 64",
}
DTYPE_NAME = {0: "f32", 1: "bf16", 2: "fp8e4m3"}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gqa70b", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--partition-tokens", type=int, default=None,
                    help="split-K partition length (default: the workload's, else auto)")
    ap.add_argument("--cpu-seqs", type=int, default=None,
                    help="sequences in the CPU-oracle sample (default: ~10-30 s of CPU work)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="instead of the benchmark, run a plain device copy of BYTES bytes "
                         "--steps times (reference for hardware byte counters)")
    return ap.parse_args()


def copy_probe(nbytes: int, steps: int) -> None:
    """A plain copy kernel of known size: reads and writes `nbytes` per launch."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"copy_probe_bytes": src.numel() * 4, "launches": steps,
                      "ms_per_copy": round(dt * 1e3, 4),
                      "read_plus_write_GBps": round(2 * src.numel() * 4 / dt / 1e9, 1)}), flush=True)


def source_digest() -> str:
    h = hashlib.sha256()
    for f in ("pa_decode.hip", "pa_decode_mfma.hip", "pa_internal.h"):
        h.update(open(os.path.join(ROOT, "paged_kv_cache_401_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def traffic_for(workload: str, kernel: str, launches_bytes: float):
    """HBM bytes per launch from committed rocprofv3 counter summaries, when
    they were taken on the current decode sources; else None."""
    path = os.path.join(ROOT, "profiles", "pmc_%s.json" % workload)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_digest") != source_digest() or rec.get("kernel") != kernel:
        return None
    return float(rec["hbm_bytes_per_launch"])


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args.copy_probe, args.steps)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(the decode hot path shards by sequence or KV head with no exchange; "
              "see the design notes).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from paged_kv_cache_401_amd import ops
    from paged_kv_cache_401_amd import workloads as wl

    dev = "cuda:0"
    torch.cuda.set_device(0)
    t0 = time.time()
    w = wl.make_workload(args.workload, small=False, device=dev)
    ptok = w.partition_tokens if args.partition_tokens is None else args.partition_tokens
    pool = ops.KVPool(w.num_blocks, w.Hkv, w.D, w.pool_dtype, device=dev, k_scale=w.k_scale,
                      v_scale=w.v_scale, fill=0)
    for op in w.ops:
        if op[0] == "write":
            ops.reshape_and_cache(pool, op[1], op[2],
                                  torch.as_tensor(op[3], dtype=torch.int32, device=dev))
        else:
            ops.copy_blocks(pool, torch.as_tensor(op[1], dtype=torch.int32, device=dev))
    q = w.q.to(dev)
    tables = torch.as_tensor(w.block_tables, dtype=torch.int32, device=dev)
    ctx = torch.as_tensor(w.context_lens, dtype=torch.int32, device=dev)
    out = torch.empty((w.S, w.Hq, w.D), dtype=torch.float32, device=dev)
    ptok_used = ops.decode_partition_tokens(pool, w.S, w.Hq, w.max_blocks_per_seq, ptok)
    ws_bytes = ops.decode_workspace_size(pool, w.S, w.Hq, w.max_blocks_per_seq, ptok)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    # the step's new tokens: each sequence's newest token, rewritten in place
    if w.step_slots is not None:
        step_k, step_v = w.step_k.to(dev), w.step_v.to(dev)
        step_slots = torch.as_tensor(w.step_slots, dtype=torch.int32, device=dev)
    else:
        step_k = step_v = step_slots = None
    no_pairs = torch.zeros((0, 2), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    def step():
        ops.copy_blocks(pool, no_pairs)
        if step_slots is not None:
            ops.reshape_and_cache(pool, step_k, step_v, step_slots)
        ops.decode(pool, q, tables, ctx, w.scale, out=out, partition_tokens=ptok,
                   workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps, HIP events on the stream around the
    # decode partition kernel of every step, wall clock around the whole
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps)]
    for e in evs:  # materialise the HIP events before handing them to the library
        e.record(stream)
    step_begin = torch.cuda.Event(enable_timing=True)
    step_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    step_begin.record(stream)
    for i in range(args.steps):
        ops.copy_blocks(pool, no_pairs)
        if step_slots is not None:
            ops.reshape_and_cache(pool, step_k, step_v, step_slots)
        ops.set_profile_events(evs[2 * i], evs[2 * i + 1])
        ops.decode(pool, q, tables, ctx, w.scale, out=out, partition_tokens=ptok, workspace=ws)
    step_end.record(stream)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - wall0
    gpu_ms = step_begin.elapsed_time(step_end)
    kern_ms = [evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(args.steps)]

    ms_per_step = gpu_ms / args.steps
    kv_bytes = w.kv_bytes()
    kern_avg_ms = float(np.mean(kern_ms))
    achieved = kv_bytes / (kern_avg_ms * 1e-3) / 1e9
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    kernel_name = ops.decode_variant(pool, w.Hq)
    traffic = traffic_for(args.workload, kernel_name, kv_bytes)

    # the read bandwidth this GPU sustains on a plain streaming read of the K pool
    sink = torch.zeros(16, dtype=torch.uint8, device=dev)
    for _ in range(3):
        ops.probe_read(pool.k, sink)
    pb, pe = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pb.record(stream)
    for _ in range(10):
        ops.probe_read(pool.k, sink)
    pe.record(stream)
    torch.cuda.synchronize()
    probe_gbps = pool.k.numel() / (pb.elapsed_time(pe) / 10 * 1e-3) / 1e9

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAME[w.pool_dtype],
        "data": "synthetic (seeded N(0,1) q/K/V, scattered 16-token blocks)",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "num_seqs": w.S,
                   "num_q_heads": w.Hq, "num_kv_heads": w.Hkv, "head_dim": w.D,
                   "total_context_tokens": int(w.context_lens.sum()),
                   "partition_tokens": ptok_used, "kv_bytes": kv_bytes,
                   "parallelism": "single GPU"},
        "pct_hbm_peak_step": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "decode_seqs_per_s": round(w.S / (ms_per_step * 1e-3), 1),
        "decode_kernel_ms": round(kern_avg_ms, 5),
        "decode_kernel_ms_min": round(float(np.min(kern_ms)), 5),
        "wall_ms_per_step": round(1e3 * wall_s / args.steps, 5),
        "unique_kv_bytes": w.unique_kv_bytes(),
        "decode_unique_GBps": round(w.unique_kv_bytes() / (kern_avg_ms * 1e-3) / 1e9, 2),
        "read_probe_GBps": round(probe_gbps, 1),
        "decode_pct_of_read_probe": round(100.0 * achieved / probe_gbps, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "kernel": kernel_name,
                     "algorithmic_bytes_per_launch": kv_bytes},
        "setup_s": round(setup_s, 2),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"], rec["max_abs_err_vs_oracle_sample"] = cpu_baseline(
            w, args, out, pool)
    print(json.dumps(rec), flush=True)


def cpu_baseline(w, args, gpu_out, pool):
    """Time the fp64 oracle (as it stands) on the first sequences of the same
    workload, on this host's cores; also compare those rows with the GPU."""
    import numpy as np

    import oracle
    from paged_kv_cache_401_amd.workloads import raw_numpy

    threads = len(os.sched_getaffinity(0))
    # the oracle takes ~9 ns per (query head, token, head dim) on one core
    per_seq_cpu_s = w.Hq * float(np.mean(w.context_lens)) * w.D * 9e-9
    n = args.cpu_seqs or max(1, min(w.S, int(20.0 / max(per_seq_cpu_s, 1e-6))))
    seqs = list(range(n))
    kp = oracle.new_pool(w.num_blocks, w.Hkv, w.D, w.pool_dtype)
    vp = oracle.new_pool(w.num_blocks, w.Hkv, w.D, w.pool_dtype)
    if w.name.startswith("sampling"):
        for op in w.ops:
            if op[0] == "write":
                oracle.reshape_and_cache(kp, vp, w.pool_dtype, w.num_blocks, w.Hkv, w.D,
                                         raw_numpy(op[1]), raw_numpy(op[2]), w.kv_in_dtype, op[3],
                                         w.k_scale, w.v_scale)
            else:
                oracle.copy_blocks(kp, vp, w.pool_dtype, w.Hkv, w.D, op[1])
    else:
        import torch
        _, k, v, slots = w.ops[0]
        off = np.concatenate([[0], np.cumsum(w.context_lens.astype(np.int64))])
        idx = np.arange(off[0], off[n])
        it = torch.as_tensor(idx, device=k.device)
        oracle.reshape_and_cache(kp, vp, w.pool_dtype, w.num_blocks, w.Hkv, w.D,
                                 raw_numpy(k.index_select(0, it)), raw_numpy(v.index_select(0, it)),
                                 w.kv_in_dtype, slots[idx], w.k_scale, w.v_scale)
    rows = [(s, h) for s in seqs for h in range(w.Hq)]
    t0 = time.perf_counter()
    ref = oracle.paged_attention(kp, vp, w.pool_dtype, w.Hkv, w.D, raw_numpy(w.q), w.q_dtype,
                                 w.S, w.Hq, w.block_tables, w.context_lens, w.scale, w.k_scale,
                                 w.v_scale, rows=rows, threads=threads)
    dt = time.perf_counter() - t0
    got = gpu_out.cpu().numpy()[seqs].reshape(-1, w.D).astype(np.float64)
    err = float(np.max(np.abs(got - ref)))
    eb = {0: 4, 1: 2, 2: 1}[w.pool_dtype]
    sample_bytes = int(w.context_lens[:n].astype(np.int64).sum()) * w.Hkv * w.D * 2 * eb
    cpu_model = platform.processor() or ""
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                cpu_model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return ({"value": round(sample_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
             "kind": "oracle",
             "sample": "first %d of %d sequences, all %d query heads (%d KV bytes), fp64 C oracle"
                       % (n, w.S, w.Hq, sample_bytes),
             "seconds": round(dt, 3), "seqs_per_s": round(n / dt, 3), "cpu_model": cpu_model},
            err)


if __name__ == "__main__":
    main()
