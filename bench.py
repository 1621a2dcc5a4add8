"""Benchmark: one decode step of paged attention on one MI355X.

A step is the whole hot path over one batch: the copy-on-write block copies
(none for workloads without shared partial blocks), the cache write of every
sequence's newest token, and paged decode attention (partition kernel plus
split-K reduce when contexts span several partitions).  The newest tokens are
written by the cache-write kernel before the decode call (default), or by the
decode call itself with ``--append fused`` (pa_decode_append).  Inputs are
synthetic and seeded and already resident in HBM when timing starts.

Prints ONE JSON line.  ``value`` is KV-read GB/s over the whole step:
algorithmic K+V bytes divided by the step time.  The algorithmic bytes are
those of the distinct token slots the step reads (context tokens x KV heads x
head dim x 2 x element bytes, a block shared by several sequences counted
once); without shared blocks that is the sum over sequences.  ``roofline``
reports the decode partition kernel alone (HIP events recorded around that
kernel on its stream) against the MI355X HBM peak of 8 TB/s.
``cpu_baseline`` times the fp64 CPU oracle on a bounded sample of the same
workload.  The default run (the 70B-like layer) also times and checks the
other decode configurations against the oracle (``configs``).
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
    "prefill_gqa70b": "causal prefill of 8 whole 4096-token prompts, 64 q / 8 KV heads, head_dim 128, "
                      "bf16 KV in scattered 16-token blocks",
    "prefill_mha13b": "causal prefill of 8 whole 2048-token prompts, 40 heads, head_dim 128, bf16 KV",
    "chunked_gqa70b": "chunked prefill: 32 seqs, cached prefix uniform [0, 3584] + 512-token chunk, "
                      "64 q / 8 KV heads, head_dim 128, bf16 KV",
    "chunked_fp8": "chunked prefill: 32 seqs, cached prefix uniform [0, 3584] + 512-token chunk, "
                   "64 q / 8 KV heads, head_dim 128, e4m3 KV, bf16 q",
}
WORKLOAD_TEXT["beam"] = ("beam search: 64 requests x 8 beams over shared 1000-token prompts after 40 "
                         "steps of forks and copy-on-write, 64 q / 8 KV heads, head_dim 128, bf16; "
                         "a step copies the last step's ~176 shared partial blocks")
WORKLOAD_TEXT["swap"] = ("block swap: 16 of 64 sequences x 4096 tokens (70B-like: 8 KV heads, head_dim "
                         "128, bf16) moved block by block to pinned host memory and back: 4096 "
                         "blocks x 32 KiB for K and for V")
WORKLOAD_TEXT["prefix"] = ("prefix caching by full-block hashing: 128 requests over 8 system prompts "
                           "(64..2048 tokens) + 16..512 private tokens, 64 q / 8 KV heads, head_dim "
                           "128, bf16; prompt processing = cache write + causal prefill of each "
                           "request's uncached tokens over its (partly cached) context")
WORKLOAD_TEXT["fill_gqa70b"] = ("bulk cache write: the 70B-like layer's 1,048,576 prompt tokens (256 "
                                "seqs x 4096, 8 KV heads, head_dim 128, bf16) into scattered 16-token "
                                "blocks of a 65536-block pool")
WORKLOAD_TEXT["fill_fp8"] = ("bulk cache write with fp8 encoding: the long-tail workload's prompt tokens "
                             "(128 seqs, lognormal contexts, 8 KV heads, head_dim 128) from bf16 into "
                             "an e4m3 pool")
PREFILL = ("prefill_gqa70b", "prefill_mha13b", "chunked_gqa70b", "chunked_fp8")
FILL = {"fill_gqa70b": "gqa70b", "fill_fp8": "fp8"}
MFMA_BF16_PEAK_TFLOPS = 2500.0
DTYPE_NAME = {0: "f32", 1: "bf16", 2: "fp8e4m3"}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gqa70b", choices=sorted(WORKLOAD_TEXT),
                    help="decode workload (default: the 70B-like GQA layer) or a prefill one")
    ap.add_argument("--partition-tokens", type=int, default=None,
                    help="split-K partition length (default: the workload's, else auto)")
    ap.add_argument("--cpu-seqs", type=int, default=None,
                    help="sequences in the CPU-oracle sample (default: ~10-30 s of CPU work)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode", choices=("auto", "plain", "prefix-shared"), default="auto",
                    help="decode entry point: pa_decode_ex per sequence (plain), or "
                         "pa_decode_prefix_shared over the groups of sequences forked from shared "
                         "prompts (auto: prefix-shared for workloads with such groups)")
    ap.add_argument("--no-configs", action="store_true",
                    help="default workload: skip timing and checking the other decode "
                         "configurations (the 'configs' record)")
    ap.add_argument("--graph", action="store_true",
                    help="decode workloads: also capture one step into a HIP graph and time its "
                         "replays (reported as graph_ms_per_step)")
    ap.add_argument("--append", choices=("separate", "fused"), default="separate",
                    help="decode workloads: write the step's new tokens with the cache-write "
                         "kernel before decoding (separate) or inside the decode call (fused)")
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


class KernelTimer:
    """HIP timing events for the partition kernel of every timed step, created
    with a device-scope release (hipEventReleaseToDevice, the form HIP offers
    for timing commands between events; timing needs no system-scope release
    and its cache write-back).  The library has the kernel's dispatch record
    them (pa_set_profile_events).  The events come from the HIP runtime this
    process already runs (loaded by torch, shared with libpa.so)."""

    RELEASE_TO_DEVICE = 0x40000000

    def __init__(self, n: int):
        import ctypes
        path = None
        for ln in open("/proc/self/maps"):
            if "libamdhip64.so" in ln:
                path = ln.split()[-1]
                break
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded")
        self.hip = ctypes.CDLL(path)
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.events = []
        for _ in range(2 * n):
            ev = ctypes.c_void_p()
            rc = self.hip.hipEventCreateWithFlags(ctypes.byref(ev), self.RELEASE_TO_DEVICE)
            if rc != 0:
                raise RuntimeError("hipEventCreateWithFlags failed (%d)" % rc)
            self.events.append(ev.value)

    def pair(self, i):
        return self.events[2 * i], self.events[2 * i + 1]

    def record(self, k, stream):
        """Record event k (of 2 n) on `stream` (a torch stream)."""
        rc = self.hip.hipEventRecord(self.events[k], stream.cuda_stream)
        if rc != 0:
            raise RuntimeError("hipEventRecord failed (%d)" % rc)

    def elapsed_ms(self, i) -> float:
        import ctypes
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), *self.pair(i))
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed (%d)" % rc)
        return float(ms.value)

    def close(self):
        for ev in self.events:
            self.hip.hipEventDestroy(ev)
        self.events = []


def source_digest() -> str:
    """Digest of the code (comments and blank lines dropped) and compile flags
    the matrix-core decode kernel is built from."""
    from paged_kv_cache_401_amd import build as pa_build
    h = hashlib.sha256()
    for f in ("pa_decode_mfma.hip", "pa_mfma_util.h", "pa_internal.h", "pa_store.h"):
        for ln in open(os.path.join(ROOT, "paged_kv_cache_401_amd", "csrc", f)).read().splitlines():
            code = ln.split("//", 1)[0].rstrip()
            if code:
                h.update(code.encode() + b"\n")
    h.update(" ".join(pa_build.common_flags()).replace(ROOT, "").encode())
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
    if args.workload in PREFILL:
        run_prefill(args)
        return
    if args.workload == "swap":
        run_swap(args)
        return
    if args.workload in FILL:
        run_fill(args)
        return
    if args.workload == "prefix":
        run_prefix(args)
        return

    import numpy as np
    import torch

    from paged_kv_cache_401_amd import workloads as wl

    torch.cuda.set_device(0)
    t0 = time.time()
    w = wl.make_workload(args.workload, small=False, device="cuda:0")
    setup_s = time.time() - t0
    ptok = w.partition_tokens if args.partition_tokens is None else args.partition_tokens
    prefix_shared = (args.decode == "prefix-shared" or
                     (args.decode == "auto" and "group_sizes" in w.info and args.append == "separate"))
    r = decode_run(w, args.steps, args.warmup, ptok, args.append, graph=args.graph,
                   flush_and_probe=True, prefix_shared=prefix_shared)
    kv_bytes, uniq = w.kv_bytes(), w.unique_kv_bytes()
    traffic = traffic_for(args.workload, r["kernel"], uniq)
    rec = {
        "metric": METRIC,
        "value": round(uniq / (r["ms_per_step"] * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAME[w.pool_dtype],
        "data": "synthetic (seeded N(0,1) q/K/V, scattered 16-token blocks)",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "num_seqs": w.S,
                   "num_q_heads": w.Hq, "num_kv_heads": w.Hkv, "head_dim": w.D,
                   "total_context_tokens": int(w.context_lens.sum()),
                   "partition_tokens": r["partition_tokens"], "kv_bytes": kv_bytes,
                   "unique_kv_bytes": uniq, "kv_loads": r["kv_loads"],
                   "cache_write": r["cache_write"], "parallelism": "single GPU"},
        "pct_hbm_peak_step": round(100.0 * uniq / (r["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
        "decode_seqs_per_s": round(w.S / (r["ms_per_step"] * 1e-3), 1),
        "decode_kernel_ms": round(r["kernel_ms"], 5),
        "decode_kernel_ms_min": round(float(np.min(r["kernel_ms_all"])), 5),
        "decode_kernel_ms_p10_median_p90": [round(float(x), 5) for x in
                                            np.percentile(r["kernel_ms_all"], [10, 50, 90])],
        "wall_ms_per_step": round(r["wall_ms_per_step"], 5),
        "logical_kv_GBps": round(kv_bytes / (r["kernel_ms"] * 1e-3) / 1e9, 2),
    }
    rec.update(r["extra"])
    if "read_probe_GBps" in rec:
        rec["decode_pct_of_read_probe"] = round(
            100.0 * uniq / (r["kernel_ms"] * 1e-3) / 1e9 / rec["read_probe_GBps"], 2)
    rec["roofline"] = {"bound": "hbm", "achieved": round(uniq / (r["kernel_ms"] * 1e-3) / 1e9, 2),
                       "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                       "frac": round(uniq / (r["kernel_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                       "traffic": traffic, "kernel": r["kernel"],
                       "algorithmic_bytes_per_launch": uniq,
                       "bytes_note": "K+V bytes of the distinct token slots one launch reads "
                                     "(blocks shared by several sequences counted once)"}
    rec["setup_s"] = round(setup_s, 2)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"], rec["max_abs_err_vs_oracle_sample"] = cpu_baseline(
            w, args, r["out"], r["pool"])
    if args.workload == "gqa70b" and not args.no_configs:
        del r
        torch.cuda.empty_cache()
        rec["configs"] = other_configs(args)
    print(json.dumps(rec), flush=True)


def decode_run(w, steps, warmup, ptok, append="separate", graph=False, flush_and_probe=False,
               prefix_shared=False):
    """Time `steps` decode steps of workload `w` after `warmup` untimed ones.
    A step: the copy-on-write copies of the workload's last step (beam search;
    none otherwise), the cache write of every sequence's newest token (before
    the decode call, or inside it with append="fused"), and the decode call
    (partition kernel + split-K reduce).  With `prefix_shared` (workloads
    whose sequences come in groups forked from shared prompts) the decode
    call is pa_decode_prefix_shared over those groups, and the plain decode
    kernel is timed on the same pool for comparison.  HIP events on the
    launch stream bracket the whole timed region and, every step, the
    partition kernel."""
    import numpy as np
    import torch

    from paged_kv_cache_401_amd import ops

    dev = "cuda:0"
    pool = ops.KVPool(w.num_blocks, w.Hkv, w.D, w.pool_dtype, device=dev, k_scale=w.k_scale,
                      v_scale=w.v_scale, fill=0)
    cow_pairs = None
    for op in w.ops:
        if op[0] == "write":
            ops.reshape_and_cache(pool, op[1].to(dev), op[2].to(dev),
                                  torch.as_tensor(op[3], dtype=torch.int32, device=dev))
        else:
            cow_pairs = torch.as_tensor(op[1], dtype=torch.int32, device=dev)
            ops.copy_blocks(pool, cow_pairs)
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
    # the step's copy-on-write pairs (beam search: the last step's; else none)
    sp = w.info.get("step_pairs")
    step_pairs = torch.as_tensor(np.zeros((0, 2), np.int32) if sp is None else sp,
                                 dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    # blocks shared across sequences (prompts, beams): cached rather than streaming loads
    shared = bool(w.info.get("shared_kv", False))
    # The step's new tokens are each sequence's last position: with fused
    # appends the decode call writes them itself (pa_decode_append).
    fused = append == "fused" and step_slots is not None
    if fused:
        last = np.array([int(w.block_tables[s][(c - 1) // 16]) * 16 + (c - 1) % 16
                         for s, c in enumerate(w.context_lens)], np.int32)
        if not np.array_equal(last, w.step_slots):
            raise SystemExit("--append fused needs every sequence's newest token at its last "
                             "position, in a block of its own")
    new_kv = dict(k_new=step_k, v_new=step_v) if fused else {}
    write_first = step_slots is not None and not fused
    groups = None
    if prefix_shared:
        from paged_kv_cache_401_amd.blocks import prefix_groups
        if fused:
            raise SystemExit("the prefix-shared decode takes its new tokens from the cache write")
        mg = max(1, 16 // w.group)
        st, pb = prefix_groups(w.block_tables, w.context_lens, w.info["group_sizes"], mg)
        groups = (torch.as_tensor(np.asarray(st, np.int32), device=dev),
                  torch.as_tensor(np.asarray(pb, np.int32), device=dev), mg)
        sws = ops.decode_prefix_shared_workspace_size(pool, w.S, w.Hq, w.max_blocks_per_seq,
                                                      len(pb), mg, ptok)
        ptok_used = ops.decode_prefix_shared_plan(pool, w.S, w.Hq, w.max_blocks_per_seq, len(pb), mg,
                                                  ptok)["partition_tokens"]
        sws_t = torch.empty(max(sws, 16), dtype=torch.uint8, device=dev)

    def decode_call():
        if groups is None:
            ops.decode(pool, q, tables, ctx, w.scale, out=out, partition_tokens=ptok,
                       workspace=ws, shared_kv=shared, **new_kv)
        else:
            ops.decode_prefix_shared(pool, q, tables, ctx, groups[0], groups[1], groups[2], w.scale,
                                     out=out, partition_tokens=ptok, workspace=sws_t)

    def step():
        ops.copy_blocks(pool, step_pairs)
        if write_first:
            ops.reshape_and_cache(pool, step_k, step_v, step_slots)
        decode_call()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps, HIP events on the stream timing the
    # decode partition kernel of every step, wall clock around the whole
    stream = torch.cuda.current_stream()
    timer = KernelTimer(steps)
    step_begin = torch.cuda.Event(enable_timing=True)
    step_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    step_begin.record(stream)
    for i in range(steps):
        ops.copy_blocks(pool, step_pairs)
        if write_first:
            ops.reshape_and_cache(pool, step_k, step_v, step_slots)
        ops.set_profile_events(*timer.pair(i))
        decode_call()
    step_end.record(stream)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - wall0
    kern_ms = [timer.elapsed_ms(i) for i in range(steps)]
    timer.close()
    plan = ops.decode_plan(pool, w.S, w.Hq, w.max_blocks_per_seq, ptok)
    res = {"pool": pool, "out": out,
           "kernel": "decode_shared_kernel" if groups is not None else plan["kernel"],
           "partition_tokens": ptok_used, "ms_per_step": step_begin.elapsed_time(step_end) / steps,
           "wall_ms_per_step": 1e3 * wall_s / steps, "kernel_ms": float(np.mean(kern_ms)),
           "kernel_ms_all": kern_ms,
           "kv_loads": ("non-temporal, shared blocks read once per group" if groups is not None
                        else "cached (shared blocks)" if shared else "non-temporal"),
           "cache_write": ("none" if step_slots is None else
                           "in the decode call" if fused else "separate kernel"),
           "extra": {}}

    def time_copies(pairs, label, target):
        """The copy-on-write kernel alone on `pairs` in pool `target`: read +
        write bytes of K and V blocks."""
        cb, ce = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ops.copy_blocks(target, pairs)
        cb.record(stream)
        for _ in range(steps):
            ops.copy_blocks(target, pairs)
        ce.record(stream)
        torch.cuda.synchronize()
        copy_ms = cb.elapsed_time(ce) / steps
        block_bytes = pool.nbytes // w.num_blocks
        moved = 2 * 2 * int(pairs.shape[0]) * block_bytes
        return {"pairs": int(pairs.shape[0]), "what": label, "block_bytes_per_pool": block_bytes,
                "ms": round(copy_ms, 5), "read_plus_write_GBps": round(moved / copy_ms / 1e6, 1)}

    # The copy-on-write pairs alone, timed on a scratch pool of the same
    # shape: in the real pool each copy's destination has since received its
    # sequence's own token, which copying again without that write would
    # overwrite (and the decode calls after this point read the real pool).
    timed_pairs = None
    if step_pairs.shape[0]:
        timed_pairs = (step_pairs, "the step's copy-on-write pairs")
    elif cow_pairs is not None and cow_pairs.shape[0]:
        timed_pairs = (cow_pairs, "the fork's copy-on-write pairs (shared partial prompt blocks)")
    if timed_pairs is not None:
        scratch = ops.KVPool(w.num_blocks, w.Hkv, w.D, w.pool_dtype, device=dev, k_scale=w.k_scale,
                             v_scale=w.v_scale, fill=0)
        res["extra"]["copy_blocks"] = time_copies(timed_pairs[0], timed_pairs[1], scratch)
        del scratch
    if groups is not None:
        # the plain decode (one workgroup per sequence and KV head) on the same
        # pool, its partition kernel timed the same way
        res["extra"]["prefix_groups"] = {"groups": int(groups[1].numel()), "max_group_size": groups[2],
                                         "shared_blocks_per_group": sorted(set(groups[1].tolist()))[:4]}
        plain_out = torch.empty_like(out)
        for _ in range(3):
            ops.decode(pool, q, tables, ctx, w.scale, out=plain_out, partition_tokens=0, shared_kv=True)
        timer = KernelTimer(steps)
        for i in range(steps):
            ops.set_profile_events(*timer.pair(i))
            ops.decode(pool, q, tables, ctx, w.scale, out=plain_out, partition_tokens=0, shared_kv=True)
        torch.cuda.synchronize()
        res["extra"]["plain_decode_kernel_ms"] = round(float(np.mean([timer.elapsed_ms(i)
                                                                      for i in range(steps)])), 5)
        timer.close()
        res["extra"]["plain_vs_prefix_shared_max_abs_diff"] = float(
            (plain_out - out).abs().max().item())
    if graph:
        res["extra"]["graph"] = graph_step_time(step, steps, w.S)
    if flush_and_probe:
        res["extra"].update(flushed_and_probe(w, pool, decode_call, steps))
    return res


def flushed_and_probe(w, pool, decode_call, steps):
    """The same decode call once more per step with a 1 GiB read before each
    launch (untimed, outside the timed steps): afterwards the 256 MB MALL
    holds clean lines of another buffer and nothing of the pool, so the
    kernel reads every byte from HBM.  (A 1 GiB write instead leaves dirty
    lines whose write-back then slows the decode itself.)  Back-to-back steps
    let a pool not much larger than the MALL, or blocks shared across steps,
    find part of themselves there.  Then the read bandwidth this GPU
    sustains on a plain streaming read of the K pool."""
    import numpy as np
    import torch

    from paged_kv_cache_401_amd import ops

    dev = "cuda:0"
    stream = torch.cuda.current_stream()
    flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    flush.sum()
    flush.sum()
    timer = KernelTimer(steps)
    for i in range(steps):
        flush.sum()
        ops.set_profile_events(*timer.pair(i))
        decode_call()
    torch.cuda.synchronize()
    flushed_ms = [timer.elapsed_ms(i) for i in range(steps)]
    timer.close()
    del flush
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
    med = float(np.median(flushed_ms))
    uniq = w.unique_kv_bytes()
    return {"decode_kernel_ms_after_1GiB_read_p10_median_p90":
                [round(float(x), 5) for x in np.percentile(flushed_ms, [10, 50, 90])],
            "pct_hbm_peak_after_1GiB_read": round(100.0 * uniq / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
            "read_probe_GBps": round(probe_gbps, 1)}


# The other decode configurations, timed and checked in the default run.
CONFIG_RUNS = ("tiny", "mha13b", "sampling_a", "sampling_b", "fp8")


def other_configs(args):
    """Each other decode configuration once more, at full size: step and
    partition-kernel times, GB/s on logical and on unique KV bytes (the
    roofline fraction on unique bytes), and the max abs error against the
    fp64 oracle over the whole output tensor (a sample of sequences for the
    fp8 pool)."""
    import numpy as np
    import torch

    from paged_kv_cache_401_amd import workloads as wl

    recs = {}
    steps, warmup = args.steps, args.warmup
    for name in CONFIG_RUNS:
        t0 = time.time()
        w = wl.make_workload(name, small=False, device="cuda:0")
        r = decode_run(w, steps, warmup, w.partition_tokens, "separate",
                       prefix_shared="group_sizes" in w.info)
        kv, uniq = w.kv_bytes(), w.unique_kv_bytes()
        # the whole output tensor; for the fp8 pool every 8th sequence and the
        # longest and shortest (the oracle's fp8 encoder takes ~40 ns per
        # element, single-threaded: ~36 s for the whole pool)
        if DTYPE_NAME[w.pool_dtype] == "fp8e4m3":
            ctxs = w.context_lens
            seqs = sorted(set(range(0, w.S, 8)) | {w.S - 1, int(np.argmax(ctxs)), int(np.argmin(ctxs))})
        else:
            seqs = list(range(w.S))
        err = sampled_error(w, r["out"], seqs)
        rec = {"workload": WORKLOAD_TEXT[name], "dtype": DTYPE_NAME[w.pool_dtype],
               "num_seqs": w.S, "steps": steps, "warmup": warmup,
               "partition_tokens": r["partition_tokens"], "kernel": r["kernel"],
               "kv_loads": r["kv_loads"], "cache_write": r["cache_write"],
               "ms_per_step": round(r["ms_per_step"], 5),
               "decode_kernel_ms": round(r["kernel_ms"], 5),
               "decode_seqs_per_s": round(w.S / (r["ms_per_step"] * 1e-3), 1),
               "kv_bytes": kv, "unique_kv_bytes": uniq,
               "logical_kv_GBps": round(kv / (r["kernel_ms"] * 1e-3) / 1e9, 2),
               "unique_kv_GBps": round(uniq / (r["kernel_ms"] * 1e-3) / 1e9, 2),
               "roofline_frac": round(uniq / (r["kernel_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
               "step_unique_GBps": round(uniq / (r["ms_per_step"] * 1e-3) / 1e9, 2),
               "max_abs_err_vs_oracle": err,
               "oracle_rows": ("all %d sequences" % w.S if len(seqs) == w.S
                               else "%d of %d sequences" % (len(seqs), w.S)) + ", every query head",
               "setup_s": round(time.time() - t0, 2)}
        rec.update(r["extra"])
        recs[name] = rec
        del r, w
        torch.cuda.empty_cache()
    return recs


def sampled_error(w, gpu_out, seqs):
    """Max abs error of the GPU rows of `seqs` (every query head) against the
    fp64 oracle, on an oracle pool holding what those rows read; the time the
    oracle took is printed to stderr."""
    import numpy as np
    import torch

    import oracle
    from paged_kv_cache_401_amd.workloads import raw_numpy

    kp = oracle.new_pool(w.num_blocks, w.Hkv, w.D, w.pool_dtype)
    vp = oracle.new_pool(w.num_blocks, w.Hkv, w.D, w.pool_dtype)
    if len(w.ops) > 1:      # shared prompts: the whole cache history
        for op in w.ops:
            if op[0] == "write":
                oracle.reshape_and_cache(kp, vp, w.pool_dtype, w.num_blocks, w.Hkv, w.D,
                                         raw_numpy(op[1]), raw_numpy(op[2]), w.kv_in_dtype, op[3],
                                         w.k_scale, w.v_scale)
            else:
                oracle.copy_blocks(kp, vp, w.pool_dtype, w.Hkv, w.D, op[1])
    else:                   # independent sequences: only theirs
        _, k, v, slots = w.ops[0]
        off = np.concatenate([[0], np.cumsum(w.context_lens.astype(np.int64))])
        idx = np.concatenate([np.arange(off[s], off[s + 1]) for s in seqs])
        it = torch.as_tensor(idx, device=k.device)
        oracle.reshape_and_cache(kp, vp, w.pool_dtype, w.num_blocks, w.Hkv, w.D,
                                 raw_numpy(k.index_select(0, it)), raw_numpy(v.index_select(0, it)),
                                 w.kv_in_dtype, slots[idx], w.k_scale, w.v_scale)
    rows = [(s, h) for s in seqs for h in range(w.Hq)]
    t0 = time.perf_counter()
    ref = oracle.paged_attention(kp, vp, w.pool_dtype, w.Hkv, w.D, raw_numpy(w.q), w.q_dtype,
                                 w.S, w.Hq, w.block_tables, w.context_lens, w.scale, w.k_scale,
                                 w.v_scale, rows=rows, threads=len(os.sched_getaffinity(0)))
    print("oracle: %s, %d rows in %.1f s" % (w.name, len(rows), time.perf_counter() - t0),
          file=sys.stderr, flush=True)
    got = gpu_out.cpu().numpy()[seqs].reshape(-1, w.D).astype(np.float64)
    return float(np.max(np.abs(got - ref)))


def graph_step_time(step, steps, num_seqs):
    """The same step captured once into a HIP graph and replayed: the launch
    cost of its kernels is paid once at capture."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for _ in range(steps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    ms = a.elapsed_time(b) / steps
    return {"ms_per_step": round(ms, 5), "wall_ms_per_step": round(1e3 * wall, 5),
            "decode_seqs_per_s": round(num_seqs / (ms * 1e-3), 1)}


def run_prefill(args):
    """One prefill step: write every sequence's chunk of new tokens into its
    slots, then causal prefill attention of the chunks over their contexts.
    ``value`` is algorithmic TFLOP/s of the step (sum over chunk rows and
    heads of 4 D flops per token seen); ``roofline`` is the prefill kernel
    alone against the bf16 matrix-core peak."""
    import numpy as np
    import torch

    from paged_kv_cache_401_amd import ops
    from paged_kv_cache_401_amd import workloads as wl

    dev = "cuda:0"
    torch.cuda.set_device(0)
    t0 = time.time()
    w = wl.make_prefill_workload(args.workload, small=False, device=dev)
    pool = ops.KVPool(w.num_blocks, w.Hkv, w.D, w.pool_dtype, device=dev, k_scale=w.k_scale,
                      v_scale=w.v_scale, fill=0)
    _, k, v, slots = w.ops[0]
    slots_t = torch.as_tensor(slots, dtype=torch.int32, device=dev)
    ops.reshape_and_cache(pool, k, v, slots_t)          # the cached prefixes (and chunks)
    # the step's cache write: the chunk tokens, the last n of each context
    off = np.concatenate([[0], np.cumsum(w.context_lens.astype(np.int64))])
    n_new = np.diff(w.query_start)
    idx = np.concatenate([np.arange(off[s + 1] - n_new[s], off[s + 1]) for s in range(w.S)])
    it = torch.as_tensor(idx, device=dev)
    ck, cv = k.index_select(0, it), v.index_select(0, it)
    cslots = slots_t.index_select(0, it)
    q = w.prefill_q
    qs = torch.as_tensor(w.query_start, dtype=torch.int32, device=dev)
    bt = torch.as_tensor(w.block_tables, dtype=torch.int32, device=dev)
    ctx = torch.as_tensor(w.context_lens, dtype=torch.int32, device=dev)
    mql = int(n_new.max())
    out = torch.empty((q.shape[0], w.Hq, w.D), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    for _ in range(args.warmup):
        ops.reshape_and_cache(pool, ck, cv, cslots)
        ops.prefill(pool, q, qs, mql, bt, ctx, w.scale, out=out)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    timer = KernelTimer(args.steps)
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    b0.record(stream)
    for i in range(args.steps):
        ops.reshape_and_cache(pool, ck, cv, cslots)
        ops.set_profile_events(*timer.pair(i))
        ops.prefill(pool, q, qs, mql, bt, ctx, w.scale, out=out)
    b1.record(stream)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - wall0
    ms_step = b0.elapsed_time(b1) / args.steps
    kern = [timer.elapsed_ms(i) for i in range(args.steps)]
    timer.close()
    kern_ms = float(np.mean(kern))
    flops = w.prefill_flops()
    achieved = flops / (kern_ms * 1e-3) / 1e12
    value = flops / (ms_step * 1e-3) / 1e12
    tokens = int(w.query_start[-1])
    rec = {
        "metric": "pa_prefill TFLOP/s (algorithmic, causal) at 1 MI355X",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAME[w.pool_dtype],
        "data": "synthetic (seeded N(0,1) q/K/V, scattered 16-token blocks)",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "num_seqs": w.S,
                   "num_q_heads": w.Hq, "num_kv_heads": w.Hkv, "head_dim": w.D,
                   "chunk_tokens": tokens, "total_context_tokens": int(w.context_lens.sum()),
                   "algorithmic_flops": flops, "parallelism": "single GPU"},
        "prefill_tokens_per_s": round(tokens / (ms_step * 1e-3), 1),
        "prefill_kernel_ms": round(kern_ms, 5),
        "prefill_kernel_ms_min": round(float(np.min(kern)), 5),
        "wall_ms_per_step": round(1e3 * wall_s / args.steps, 5),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "prefill_mfma_kernel", "algorithmic_flops_per_launch": flops},
        "setup_s": round(setup_s, 2),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"], rec["max_abs_err_vs_oracle_sample"] = prefill_cpu_baseline(
            w, args, out)
    print(json.dumps(rec), flush=True)


def run_prefix(args):
    """Prompt processing of the request stream with prefix caching (only the
    uncached tokens are written and prefilled, over contexts whose cached
    prefixes are shared blocks) against the same requests without caching
    (every token written and prefilled).  ``value`` is prompt tokens per
    second with caching."""
    import numpy as np
    import torch

    from paged_kv_cache_401_amd import ops
    from paged_kv_cache_401_amd import workloads as wl

    dev = "cuda:0"
    torch.cuda.set_device(0)
    runs = {}
    for caching in (True, False):
        w = wl.make_prefix_workload(small=False, device=dev, caching=caching)
        pool = ops.KVPool(w.num_blocks, w.Hkv, w.D, w.pool_dtype, device=dev, fill=0)
        _, k, v, slots = w.ops[0]
        slots_t = torch.as_tensor(slots, dtype=torch.int32, device=dev)
        qs = torch.as_tensor(w.query_start, dtype=torch.int32, device=dev)
        bt = torch.as_tensor(w.block_tables, dtype=torch.int32, device=dev)
        ctx = torch.as_tensor(w.context_lens, dtype=torch.int32, device=dev)
        mql = int(np.diff(w.query_start).max())
        out = torch.empty((w.prefill_q.shape[0], w.Hq, w.D), dtype=torch.float32, device=dev)

        def step():
            ops.reshape_and_cache(pool, k, v, slots_t)
            ops.prefill(pool, w.prefill_q, qs, mql, bt, ctx, w.scale, out=out)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        timer = KernelTimer(args.steps)
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        b0.record(stream)
        for i in range(args.steps):
            ops.reshape_and_cache(pool, k, v, slots_t)
            ops.set_profile_events(*timer.pair(i))
            ops.prefill(pool, w.prefill_q, qs, mql, bt, ctx, w.scale, out=out)
        b1.record(stream)
        torch.cuda.synchronize()
        kern = float(np.mean([timer.elapsed_ms(i) for i in range(args.steps)]))
        timer.close()
        runs[caching] = (w, b0.elapsed_time(b1) / args.steps, kern)
    w, ms, kern = runs[True]
    w0, ms0, _ = runs[False]
    prompt_tokens = int(w.context_lens.sum())
    flops = w.prefill_flops()
    rec = {
        "metric": "prefix-cached prompt processing: prompt tokens/s at 1 MI355X",
        "value": round(prompt_tokens / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded token ids and N(0,1) K/V; K/V of a system prompt depends "
                "only on (prompt, position))",
        "config": {"workload": WORKLOAD_TEXT["prefix"], "requests": w.S,
                   "prompt_tokens": prompt_tokens,
                   "cached_tokens": int(w.info["cached_tokens"].sum()),
                   "physical_blocks": w.info["physical_blocks"],
                   "logical_blocks": w.info["logical_blocks"], "parallelism": "single GPU"},
        "no_cache_ms_per_step": round(ms0, 5),
        "speedup_vs_no_cache": round(ms0 / ms, 3),
        "blocks_saved_frac": round(1 - w.info["physical_blocks"] / w0.info["physical_blocks"], 4),
        "roofline": {"bound": "mfma", "achieved": round(flops / (kern * 1e-3) / 1e12, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(flops / (kern * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "kernel": "prefill_mfma_kernel",
                     "algorithmic_flops_per_launch": flops},
    }
    print(json.dumps(rec), flush=True)


def run_fill(args):
    """The cache write of a whole workload's tokens per step (the bulk fill of
    the pool when prompts are stored); ``value`` is algorithmic bytes (K and V
    inputs read + pool tiles written) per second, against the HBM peak."""
    import numpy as np
    import torch

    import oracle
    from paged_kv_cache_401_amd import ops
    from paged_kv_cache_401_amd import workloads as wl

    dev = "cuda:0"
    torch.cuda.set_device(0)
    w = wl.make_workload(FILL[args.workload], small=False, device=dev)
    pool = ops.KVPool(w.num_blocks, w.Hkv, w.D, w.pool_dtype, device=dev, k_scale=w.k_scale,
                      v_scale=w.v_scale, fill=0)
    _, k, v, slots = w.ops[0]
    st = torch.as_tensor(slots, dtype=torch.int32, device=dev)
    n = int(slots.size)
    nbytes = 2 * k.numel() * k.element_size() + 2 * k.numel() * ops.ELEM_BYTES[w.pool_dtype]
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        ops.reshape_and_cache(pool, k, v, st)
    torch.cuda.synchronize()
    timer = KernelTimer(args.steps)
    t0 = time.perf_counter()
    for i in range(args.steps):
        timer.record(2 * i, stream)
        ops.reshape_and_cache(pool, k, v, st)
        timer.record(2 * i + 1, stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    ms = float(np.mean([timer.elapsed_ms(i) for i in range(args.steps)]))
    timer.close()
    gbps = nbytes / ms / 1e6
    rec = {
        "metric": "pa_reshape_and_cache bulk GB/s (K/V read + pool written) at 1 MI355X",
        "value": round(gbps, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": DTYPE_NAME[w.pool_dtype],
        "data": "synthetic (seeded N(0,1) K/V, scattered 16-token blocks)",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "tokens": n, "num_kv_heads": w.Hkv,
                   "head_dim": w.D, "algorithmic_bytes": nbytes, "parallelism": "single GPU"},
        "wall_ms_per_step": round(1e3 * wall, 4),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "reshape_and_cache_kernel", "algorithmic_bytes_per_launch": nbytes},
    }
    if not args.no_cpu_baseline:
        # the oracle's cache write of the first tokens (about a tenth), scaled to GB/s
        m = max(16, n // 10)
        kn = k[:m].cpu().contiguous()
        vn = v[:m].cpu().contiguous()
        from paged_kv_cache_401_amd.workloads import raw_numpy
        kr, vr = raw_numpy(kn), raw_numpy(vn)
        kp = oracle.new_pool(w.num_blocks, w.Hkv, w.D, w.pool_dtype)
        vp = oracle.new_pool(w.num_blocks, w.Hkv, w.D, w.pool_dtype)
        c0 = time.perf_counter()
        oracle.reshape_and_cache(kp, vp, w.pool_dtype, w.num_blocks, w.Hkv, w.D, kr, vr, w.kv_in_dtype,
                                 slots[:m], w.k_scale, w.v_scale)
        cpu_s = time.perf_counter() - c0
        rec["cpu_baseline"] = {"value": round(nbytes * m / n / cpu_s / 1e9, 4), "unit": "GB/s",
                               "cores": 1, "kind": "oracle",  # the oracle's write loop is serial
                               "sample": "first %d of %d tokens through the C oracle's cache write"
                                         % (m, n), "seconds": round(cpu_s, 3)}
    print(json.dumps(rec), flush=True)


def run_swap(args):
    """Swap-out then swap-in of the same 4096 blocks per step; ``value`` is the
    bytes moved over the host link per second (both directions); a plain
    pinned-host DMA copy of the same byte count is timed as the reference."""
    import numpy as np
    import torch

    import oracle
    from paged_kv_cache_401_amd import ops
    from paged_kv_cache_401_amd import workloads as wl

    dev = "cuda:0"
    torch.cuda.set_device(0)
    w = wl.make_workload("gqa70b", small=False, num_seqs=64, device=dev)
    pool = ops.KVPool(w.num_blocks, w.Hkv, w.D, w.pool_dtype, device=dev, fill=0)
    _, k, v, slots = w.ops[0]
    ops.reshape_and_cache(pool, k, v, torch.as_tensor(slots, dtype=torch.int32, device=dev))
    mgr = w.info["manager"]
    blocks = [b for s in range(16) for b in mgr.block_table(s)]
    host = ops.HostPool(pool, len(blocks))
    pairs = torch.as_tensor(np.stack([blocks, np.arange(len(blocks))], 1), dtype=torch.int32,
                            device=dev)
    moved = 2 * len(blocks) * host.slot_bytes           # K and V, one direction
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        ops.swap_blocks(pool, host, pairs, ops.SWAP_OUT)
        ops.swap_blocks(pool, host, pairs, ops.SWAP_IN)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[3 * i].record(stream)
        ops.swap_blocks(pool, host, pairs, ops.SWAP_OUT)
        ev[3 * i + 1].record(stream)
        ops.swap_blocks(pool, host, pairs, ops.SWAP_IN)
        ev[3 * i + 2].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    out_ms = float(np.mean([ev[3 * i].elapsed_time(ev[3 * i + 1]) for i in range(args.steps)]))
    in_ms = float(np.mean([ev[3 * i + 1].elapsed_time(ev[3 * i + 2]) for i in range(args.steps)]))
    # reference: DMA copies of the same byte count between HBM and pinned host memory
    dbuf = torch.empty(moved // 2, dtype=torch.uint8, device=dev)
    hbuf = torch.empty(moved // 2, dtype=torch.uint8, pin_memory=True)
    hbuf.copy_(dbuf, non_blocking=True)
    torch.cuda.synchronize()
    a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    a.record(stream)
    for _ in range(args.steps):
        hbuf.copy_(dbuf, non_blocking=True)
        hbuf.copy_(dbuf, non_blocking=True)
    b.record(stream)
    for _ in range(args.steps):
        dbuf.copy_(hbuf, non_blocking=True)
        dbuf.copy_(hbuf, non_blocking=True)
    c.record(stream)
    torch.cuda.synchronize()
    dma_d2h = moved / (a.elapsed_time(b) / args.steps) / 1e6
    dma_h2d = moved / (b.elapsed_time(c) / args.steps) / 1e6
    step_ms = out_ms + in_ms
    # CPU baseline: the oracle's swap (memcpy of the same blocks) on host pools
    kp = np.zeros(pool.nbytes, np.uint8)
    vp = np.zeros(pool.nbytes, np.uint8)
    hk = np.zeros(host.k.numel(), np.uint8)
    hv = np.zeros(host.v.numel(), np.uint8)
    pr = pairs.cpu().numpy()
    c0 = time.perf_counter()
    reps = 5
    for _ in range(reps):
        oracle.swap_blocks(kp, vp, hk, hv, w.pool_dtype, w.Hkv, w.D, w.num_blocks, len(blocks),
                           pr, 0)
        oracle.swap_blocks(kp, vp, hk, hv, w.pool_dtype, w.Hkv, w.D, w.num_blocks, len(blocks),
                           pr, 1)
    cpu_s = (time.perf_counter() - c0) / reps
    rec = {
        "metric": "pa_swap_blocks host-link GB/s (swap-out + swap-in) at 1 MI355X",
        "value": round(2 * moved / step_ms / 1e6, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAME[w.pool_dtype],
        "data": "synthetic (seeded N(0,1) K/V, scattered 16-token blocks)",
        "config": {"workload": WORKLOAD_TEXT["swap"], "blocks": len(blocks),
                   "block_bytes_per_pool": host.slot_bytes, "bytes_each_direction": moved,
                   "parallelism": "single GPU"},
        "swap_out_ms": round(out_ms, 4), "swap_out_GBps": round(moved / out_ms / 1e6, 2),
        "swap_in_ms": round(in_ms, 4), "swap_in_GBps": round(moved / in_ms / 1e6, 2),
        "dma_copy_d2h_GBps": round(dma_d2h, 2), "dma_copy_h2d_GBps": round(dma_h2d, 2),
        "wall_ms_per_step": round(1e3 * wall, 4),
        "roofline": {"bound": "host-link", "achieved": round(2 * moved / step_ms / 1e6, 2),
                     "peak": round((dma_d2h + dma_h2d) / 2, 2), "unit": "GB/s",
                     "frac": round((2 * moved / step_ms / 1e6) / ((dma_d2h + dma_h2d) / 2), 4),
                     "traffic": None, "kernel": "swap_blocks_kernel",
                     "peak_note": "measured pinned-host DMA copy rate of the same bytes"},
        "cpu_baseline": {"value": round(2 * moved / cpu_s / 1e9, 3), "unit": "GB/s", "cores": 1,
                         "kind": "oracle",
                         "sample": "the same 4096-block swap-out + swap-in as host memcpy"},
    }
    print(json.dumps(rec), flush=True)


def prefill_cpu_baseline(w, args, gpu_out):
    """Time the fp64 oracle on a bounded sample of chunk rows (all heads of
    every n-th chunk token of every sequence) and compare them with the GPU."""
    import numpy as np

    import oracle
    from paged_kv_cache_401_amd.workloads import raw_numpy

    threads = len(os.sched_getaffinity(0))
    _, k, v, slots = w.ops[0]
    kp = oracle.new_pool(w.num_blocks, w.Hkv, w.D, w.pool_dtype)
    vp = oracle.new_pool(w.num_blocks, w.Hkv, w.D, w.pool_dtype)
    oracle.reshape_and_cache(kp, vp, w.pool_dtype, w.num_blocks, w.Hkv, w.D, raw_numpy(k),
                             raw_numpy(v), w.kv_in_dtype, slots, w.k_scale, w.v_scale)
    # ~9 ns per (row, token seen, head dim) on one core; aim at ~15 s of CPU work
    per_row_s = float(np.mean(w.context_lens)) * w.D * 9e-9
    want_rows = max(w.Hq, int(15.0 * threads / max(per_row_s, 1e-9)))
    total = int(w.query_start[-1])
    stride = max(1, total * w.Hq // want_rows)
    toks = np.arange(0, total, stride)
    rows = np.array([(t, h) for t in toks for h in range(w.Hq)], np.int32)
    t0 = time.perf_counter()
    ref = oracle.prefill_attention(kp, vp, w.pool_dtype, w.Hkv, w.D, raw_numpy(w.prefill_q),
                                   w.q_dtype, w.S, w.Hq, w.query_start, w.block_tables,
                                   w.context_lens, w.scale, w.k_scale, w.v_scale, rows=rows,
                                   threads=threads)
    dt = time.perf_counter() - t0
    got = gpu_out.cpu().numpy()[rows[:, 0], rows[:, 1]].astype(np.float64)
    err = float(np.max(np.abs(got - ref)))
    # algorithmic flops of the sampled rows
    seq = np.searchsorted(w.query_start, rows[:, 0], side="right") - 1
    pos = w.context_lens[seq] - np.diff(w.query_start)[seq] + (rows[:, 0] - w.query_start[seq])
    flops = float(np.sum(pos + 1)) * 4 * w.D
    return ({"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
             "kind": "oracle",
             "sample": "%d chunk rows (every %d-th chunk token, all %d heads), fp64 C oracle"
                       % (rows.shape[0], stride, w.Hq),
             "seconds": round(dt, 3)}, err)


def cpu_baseline(w, args, gpu_out, pool):
    """Time the fp64 oracle (as it stands) on the first sequences of the same
    workload, on this host's cores; also compare those rows with the GPU."""
    import numpy as np

    import oracle
    from paged_kv_cache_401_amd.workloads import raw_numpy

    threads = len(os.sched_getaffinity(0))
    # the oracle takes ~9 ns per (query head, token, head dim) on one core;
    # aim at ~15 s of CPU work over `threads` cores, at most the whole batch
    per_seq_cpu_s = w.Hq * float(np.mean(w.context_lens)) * w.D * 9e-9
    n = args.cpu_seqs or max(1, min(w.S, int(15.0 * threads / max(per_seq_cpu_s, 1e-6))))
    seqs = list(range(n))
    kp = oracle.new_pool(w.num_blocks, w.Hkv, w.D, w.pool_dtype)
    vp = oracle.new_pool(w.num_blocks, w.Hkv, w.D, w.pool_dtype)
    if w.name.startswith("sampling") or w.name == "beam":
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
