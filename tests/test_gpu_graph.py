"""GPU: the operations captured into a HIP graph (torch.cuda.CUDAGraph) and
replayed give exactly what the same calls give eagerly.

Every entry point only enqueues kernels on the caller's stream (no
allocation, no memset, no host synchronisation), so a decode step -- the
copy-on-write copies, the cache write of the new tokens and the partition and
split-K reduce kernels -- can be captured once and replayed.  Each test
replays several times with eager work and synchronisations in between, feeds
new inputs into the captured buffers between replays, and checks every replay
against an eager run on the same inputs.
"""
import numpy as np
import pytest
import torch

from bitwise import assert_same_bytes
from gpu_helpers import gpu_pool
from paged_kv_cache_401_amd import ops
from paged_kv_cache_401_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"


def capture(fn):
    """Warm fn up on a side stream, then capture one call of it."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def i32(a):
    return torch.as_tensor(np.asarray(a, dtype=np.int32), device=DEV)


@pytest.mark.parametrize("name,ptok", [("gqa70b", 0), ("fp8", 512), ("mha13b", 256),
                                       ("tiny", 0), ("sampling_b", 0)])
def test_decode_graph_replays_match_eager(name, ptok):
    w = wl.make_workload(name, small=True, device=DEV)
    pool = gpu_pool(w)
    ptok = ptok or w.partition_tokens
    q = w.q.to(DEV).clone()
    tables, ctx = i32(w.block_tables), i32(w.context_lens)
    out_g = torch.full((w.S, w.Hq, w.D), 7.0, device=DEV)
    need = ops.decode_workspace_size(pool, w.S, w.Hq, w.max_blocks_per_seq, ptok)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
    shared = bool(w.info.get("shared_kv", False))

    def step():
        ops.decode(pool, q, tables, ctx, w.scale, out=out_g, partition_tokens=ptok, workspace=ws,
                   shared_kv=shared)

    g = capture(step)
    gen = torch.Generator(device=DEV).manual_seed(3)
    for rep in range(4):
        if rep:  # new queries in the captured buffer
            q.copy_(torch.randn(q.shape, generator=gen, device=DEV).to(q.dtype))
        out_g.fill_(7.0)
        g.replay()
        # eager work between replays, on its own output and workspace
        ref = ops.decode(pool, q, tables, ctx, w.scale, partition_tokens=ptok, shared_kv=shared)
        torch.cuda.synchronize()
        assert_same_bytes(out_g.cpu().numpy(), ref.cpu().numpy(), what="replay %d" % rep)


def test_decode_step_with_cache_write_and_copies_graph():
    """The whole beam-search step (copy-on-write pairs, one new token per
    beam, decode) captured once: each replay's pool bytes and outputs equal
    an eager step run on a clone of the pool."""
    w = wl.make_workload("beam", small=True, device=DEV)
    pool = gpu_pool(w)
    pairs = i32(np.asarray(w.info["step_pairs"]).reshape(-1, 2))
    step_k, step_v = w.step_k.to(DEV).clone(), w.step_v.to(DEV).clone()
    slots = i32(w.step_slots)
    q = w.q.to(DEV).clone()
    tables, ctx = i32(w.block_tables), i32(w.context_lens)
    out_g = torch.empty((w.S, w.Hq, w.D), device=DEV)
    need = ops.decode_workspace_size(pool, w.S, w.Hq, w.max_blocks_per_seq, w.partition_tokens)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)

    def step(pl, out):
        ops.copy_blocks(pl, pairs)
        ops.reshape_and_cache(pl, step_k, step_v, slots)
        ops.decode(pl, q, tables, ctx, w.scale, out=out, partition_tokens=w.partition_tokens,
                   workspace=ws, shared_kv=True)

    g = capture(lambda: step(pool, out_g))
    twin = ops.KVPool(w.num_blocks, w.Hkv, w.D, w.pool_dtype, device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(4)
    for rep in range(3):
        if rep:  # new token values in the captured buffers
            step_k.copy_(torch.randn(step_k.shape, generator=gen, device=DEV).to(step_k.dtype))
            step_v.copy_(torch.randn(step_v.shape, generator=gen, device=DEV).to(step_v.dtype))
        twin.k.copy_(pool.k)
        twin.v.copy_(pool.v)
        g.replay()
        out_e = torch.empty_like(out_g)
        step(twin, out_e)
        torch.cuda.synchronize()
        assert_same_bytes(pool.k.cpu().numpy(), twin.k.cpu().numpy(), what="K pool, replay %d" % rep)
        assert_same_bytes(pool.v.cpu().numpy(), twin.v.cpu().numpy(), what="V pool, replay %d" % rep)
        assert_same_bytes(out_g.cpu().numpy(), out_e.cpu().numpy(), what="out, replay %d" % rep)


@pytest.mark.parametrize("name", ["chunked_gqa70b", "chunked_fp8"])
def test_prefill_graph_replays_match_eager(name):
    w = wl.make_prefill_workload(name, small=True, device=DEV)
    pool = gpu_pool(w)
    q = w.prefill_q.to(DEV).clone()
    qs, tables, ctx = i32(w.query_start), i32(w.block_tables), i32(w.context_lens)
    mql = int(np.diff(w.query_start).max())
    out_g = torch.empty((q.shape[0], w.Hq, w.D), device=DEV)

    def step():
        ops.prefill(pool, q, qs, mql, tables, ctx, w.scale, out=out_g)

    g = capture(step)
    gen = torch.Generator(device=DEV).manual_seed(5)
    for rep in range(3):
        if rep:
            q.copy_(torch.randn(q.shape, generator=gen, device=DEV).to(q.dtype))
        g.replay()
        ref = ops.prefill(pool, q, qs, mql, tables, ctx, w.scale)
        torch.cuda.synchronize()
        assert_same_bytes(out_g.cpu().numpy(), ref.cpu().numpy(), what="replay %d" % rep)
