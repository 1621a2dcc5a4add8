"""Helpers that drive the CPU oracle over a seeded workload (tests only)."""
import numpy as np

import oracle
from paged_kv_cache_401_amd.workloads import raw_numpy


def oracle_pools(w, fill=0):
    """Apply the workload's cache operations, in order, to fresh oracle pools."""
    kp = oracle.new_pool(w.num_blocks, w.Hkv, w.D, w.pool_dtype, fill)
    vp = oracle.new_pool(w.num_blocks, w.Hkv, w.D, w.pool_dtype, fill)
    for op in w.ops:
        if op[0] == "write":
            _, k, v, slots = op
            oracle.reshape_and_cache(kp, vp, w.pool_dtype, w.num_blocks, w.Hkv, w.D,
                                     raw_numpy(k), raw_numpy(v), w.kv_in_dtype, slots,
                                     w.k_scale, w.v_scale)
        else:
            oracle.copy_blocks(kp, vp, w.pool_dtype, w.Hkv, w.D, op[1])
    return kp, vp


def oracle_decode(w, kp, vp, rows=None, q=None, ctx=None, tables=None, threads=0):
    return oracle.paged_attention(
        kp, vp, w.pool_dtype, w.Hkv, w.D, raw_numpy(w.q if q is None else q), w.q_dtype,
        w.S, w.Hq, w.block_tables if tables is None else tables,
        w.context_lens if ctx is None else ctx, w.scale, w.k_scale, w.v_scale,
        rows=rows, threads=threads)


def as_f64(raw, dtype):
    """Real values of raw elements (fp32 array, bf16 bits as uint16)."""
    raw = np.asarray(raw)
    if dtype == oracle.F32:
        return raw.view(np.float32).astype(np.float64)
    if dtype == oracle.BF16:
        return (raw.view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(dtype)
