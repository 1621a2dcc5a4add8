"""GPU: pa_decode_append -- a decode step that writes every sequence's newest
token (position context_len - 1, slot through the block table) and attends
-- leaves the same pool bytes and gives the same outputs, bit for bit, as
pa_reshape_and_cache of those tokens followed by pa_decode_ex, on every
kernel path: the matrix-core kernel (written inside the attention kernel),
one query head per KV head on the vector-ALU kernel (likewise), and grouped
heads on the vector-ALU kernel (a write kernel of its own first); with and
without split-K partitions, and with empty contexts and out-of-pool table
entries (the kernels skip those).  Where every table entry is in the pool,
the result also equals the oracle on its own updated cache.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from bitwise import assert_same_bytes
from gpu_helpers import gpu_pool, tolerance
from oracle_helpers import oracle_decode, oracle_pools
from paged_kv_cache_401_amd import ops
from paged_kv_cache_401_amd import workloads as wl
from paged_kv_cache_401_amd.workloads import raw_numpy

pytestmark = pytest.mark.gpu
DEV = "cuda"


def i32(a):
    return torch.as_tensor(np.asarray(a, dtype=np.int32), device=DEV)


def last_slots(w, ctx, tables):
    return np.array([int(tables[s][(c - 1) // 16]) * 16 + (c - 1) % 16 if c > 0 else -1
                     for s, c in enumerate(ctx)], np.int32)


def group_workload(group):
    rng = np.random.default_rng(40 + group)
    return wl._simple("groups", 4, 2 * group, 2, 128, [33, 1, 300, 64], oracle.BF16, oracle.BF16,
                      oracle.BF16, float(np.float32(1 / math.sqrt(128))), 23, "cpu", rng)


def many_rows_workload(D, dt):
    """2048 (sequence, KV head) rows: the grouped kernel runs one wavefront
    per workgroup."""
    rng = np.random.default_rng(60 + D + dt)
    ctx = rng.integers(1, 201, 256)
    return wl._simple("many_rows", 256, 32, 8, D, ctx, dt, oracle.BF16, oracle.BF16,
                      float(np.float32(1 / math.sqrt(D))), 29, "cpu", rng, fp8_scales=dt == oracle.FP8)


CASES = {
    "gqa70b": lambda: wl.make_workload("gqa70b", small=True),      # matrix-core, bf16
    "rows_d64": lambda: many_rows_workload(64, oracle.BF16),        # matrix-core, one wavefront
    "rows_fp8": lambda: many_rows_workload(128, oracle.FP8),        # the same over an fp8 pool
    "fp8": lambda: wl.make_workload("fp8", small=True),            # matrix-core, fp8 from bf16
    "mha13b": lambda: wl.make_workload("mha13b", small=True),      # vector ALU, one head per KV head
    "tiny": lambda: wl.make_workload("tiny", small=True),          # vector ALU, fp32
    "group32": lambda: group_workload(32),                          # vector ALU, grouped: own kernel
    "beam": lambda: wl.make_workload("beam", small=True),           # shared prompts, private tails
}


@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("ptok", [0, 16, 64])
def test_append_equals_write_then_decode(case, ptok):
    w = CASES[case]()
    ctx = w.context_lens.copy()
    tables = w.block_tables.copy()
    if case in ("gqa70b", "mha13b", "fp8", "rows_d64", "rows_fp8"):
        ctx[1] = 0                        # an empty context writes nothing
    if case == "fp8":
        tables[2, (ctx[2] - 1) // 16] = w.num_blocks + 5   # an out-of-pool last block: skipped
    gen = torch.Generator().manual_seed(7)
    in_dt = torch.float32 if w.kv_in_dtype == oracle.F32 else torch.bfloat16
    k_new = (torch.randn((w.S, w.Hkv, w.D), generator=gen) * 2).to(in_dt)
    v_new = (torch.randn((w.S, w.Hkv, w.D), generator=gen) * 2).to(in_dt)
    q = w.q.to(DEV)
    shared = bool(w.info.get("shared_kv", False))
    pt = ptok or w.partition_tokens

    ref_pool = gpu_pool(w, fill=0xFF)
    ops.reshape_and_cache(ref_pool, k_new.to(DEV), v_new.to(DEV), i32(last_slots(w, ctx, tables)))
    ref = ops.decode(ref_pool, q, i32(tables), i32(ctx), w.scale, partition_tokens=pt, shared_kv=shared)

    pool = gpu_pool(w, fill=0xFF)
    got = ops.decode(pool, q, i32(tables), i32(ctx), w.scale, partition_tokens=pt, shared_kv=shared,
                     k_new=k_new.to(DEV), v_new=v_new.to(DEV))
    torch.cuda.synchronize()
    assert_same_bytes(pool.k.cpu().numpy(), ref_pool.k.cpu().numpy(), what="K pool")
    assert_same_bytes(pool.v.cpu().numpy(), ref_pool.v.cpu().numpy(), what="V pool")
    assert_same_bytes(got.cpu().numpy(), ref.cpu().numpy(), what="outputs")

    if case == "fp8":
        return  # the oracle defines attention over in-pool block ids only
    # and the oracle, on its own cache updated by its own write
    kp, vp = oracle_pools(w, fill=0xFF)
    oracle.reshape_and_cache(kp, vp, w.pool_dtype, w.num_blocks, w.Hkv, w.D, raw_numpy(k_new),
                             raw_numpy(v_new), w.kv_in_dtype, last_slots(w, ctx, tables), w.k_scale,
                             w.v_scale)
    want = oracle_decode(w, kp, vp, ctx=ctx, tables=tables)
    err = float(np.max(np.abs(got.cpu().numpy().astype(np.float64) - want)))
    assert err <= tolerance(w), "max abs error %.3e" % err


def test_append_full_size_step_and_graph():
    """The 70B-like decode step at full size as one fused call, eager and
    replayed from a HIP graph, against a separate write and decode."""
    w = wl.make_workload("gqa70b", small=False, device=DEV)
    pool = gpu_pool(w)
    ref_pool = ops.KVPool(w.num_blocks, w.Hkv, w.D, w.pool_dtype, device=DEV)
    ref_pool.k.copy_(pool.k)
    ref_pool.v.copy_(pool.v)
    tables, ctx = i32(w.block_tables), i32(w.context_lens)
    gen = torch.Generator(device=DEV).manual_seed(8)
    k_new = torch.randn((w.S, w.Hkv, w.D), generator=gen, device=DEV).to(torch.bfloat16)
    v_new = torch.randn((w.S, w.Hkv, w.D), generator=gen, device=DEV).to(torch.bfloat16)
    ops.reshape_and_cache(ref_pool, k_new, v_new, i32(w.step_slots))
    ref = ops.decode(ref_pool, w.q, tables, ctx, w.scale)
    out = torch.empty_like(ref)
    ops.decode(pool, w.q, tables, ctx, w.scale, out=out, k_new=k_new, v_new=v_new)
    torch.cuda.synchronize()
    assert_same_bytes(out.cpu().numpy(), ref.cpu().numpy(), what="eager")
    assert bool((pool.k == ref_pool.k).all()) and bool((pool.v == ref_pool.v).all())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ops.decode(pool, w.q, tables, ctx, w.scale, out=out, k_new=k_new, v_new=v_new)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ops.decode(pool, w.q, tables, ctx, w.scale, out=out, k_new=k_new, v_new=v_new)
    for rep in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert_same_bytes(out.cpu().numpy(), ref.cpu().numpy(), what="replay %d" % rep)


@pytest.mark.parametrize("Hq,Hkv", [(16, 2), (2, 2), (64, 2)])
@pytest.mark.parametrize("ptok", [0, 32])
def test_append_overlong_context_writes_nothing(Hq, Hkv, ptok):
    """A context longer than its table row (max_blocks_per_seq * 16) is
    attended as that many tokens and has no slot for a newest token: the step
    writes nothing for it -- no cached token is overwritten -- and writes the
    other sequences' tokens as usual.  Matrix-core kernel (16 / 2 heads),
    vector-ALU kernel with one head per KV head (2 / 2), and grouped heads on
    the vector-ALU kernel with its separate write kernel (64 / 2)."""
    rng = np.random.default_rng(77 + Hq)
    w = wl._simple("overlong", 3, Hq, Hkv, 128, [64, 33, 128], oracle.BF16, oracle.BF16, oracle.BF16,
                   float(np.float32(1 / math.sqrt(128))), 31, "cpu", rng)
    tables = w.block_tables.copy()
    assert tables.shape[1] * 16 == 128
    ctx = w.context_lens.copy()
    ctx[2] = 128 + 7                           # clamped to the row's 128 tokens, all written
    gen = torch.Generator().manual_seed(9)
    k_new = (torch.randn((w.S, w.Hkv, w.D), generator=gen) * 2).to(torch.bfloat16)
    v_new = (torch.randn((w.S, w.Hkv, w.D), generator=gen) * 2).to(torch.bfloat16)
    slots = last_slots(w, np.minimum(ctx, 128), tables)
    slots[2] = -1                              # nothing is written for the over-long context

    ref_pool = gpu_pool(w, fill=0xFF)
    before_k, before_v = ref_pool.k.cpu().numpy(), ref_pool.v.cpu().numpy()
    ops.reshape_and_cache(ref_pool, k_new.to(DEV), v_new.to(DEV), i32(slots))
    ref = ops.decode(ref_pool, w.q.to(DEV), i32(tables), i32(ctx), w.scale, partition_tokens=ptok)

    pool = gpu_pool(w, fill=0xFF)
    got = ops.decode(pool, w.q.to(DEV), i32(tables), i32(ctx), w.scale, partition_tokens=ptok,
                     k_new=k_new.to(DEV), v_new=v_new.to(DEV))
    torch.cuda.synchronize()
    gk, gv = pool.k.cpu().numpy(), pool.v.cpu().numpy()
    assert_same_bytes(gk, ref_pool.k.cpu().numpy(), what="K pool")
    assert_same_bytes(gv, ref_pool.v.cpu().numpy(), what="V pool")
    assert_same_bytes(got.cpu().numpy(), ref.cpu().numpy(), what="outputs")
    # the over-long sequence's blocks are unchanged; the others' last blocks changed
    tile = Hkv * 16 * w.D * 2
    for b in tables[2]:
        sl = slice(int(b) * tile, (int(b) + 1) * tile)
        assert np.array_equal(gk[sl], before_k[sl]) and np.array_equal(gv[sl], before_v[sl])
    for s in (0, 1):
        b = int(tables[s][(ctx[s] - 1) // 16])
        assert not np.array_equal(gk[b * tile:(b + 1) * tile], before_k[b * tile:(b + 1) * tile])
