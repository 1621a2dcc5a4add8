"""Pins of the oracle's causal (chunked) prefill against what the pages and
the mathematics fix.

The French page's KV-cache article: producing token n+1 needs the K and V of
tokens 1..n, so a token of a prompt attends to itself and everything before
it.  The glossary page's related-techniques section: engines run
FlashAttention-style kernels that read the paged blocks.  Paging only moves
bytes, so a chunk row at position p must equal the decode result over the
first p + 1 tokens, and scipy's softmax with a causal mask on the contiguous
K/V.
"""
import numpy as np
import pytest
import torch

import fp8_torch
import oracle
from oracle_helpers import as_f64, oracle_pools
from paged_kv_cache_401_amd import workloads as wl
from paged_kv_cache_401_amd.blocks import BlockManager, blocks_for
from paged_kv_cache_401_amd.workloads import raw_numpy
from bitwise import assert_same_bytes


def _prefill(w, kp, vp, q=None, ctx=None, qs=None, rows=None):
    return oracle.prefill_attention(
        kp, vp, w.pool_dtype, w.Hkv, w.D, raw_numpy(w.prefill_q if q is None else q), w.q_dtype,
        w.S, w.Hq, w.query_start if qs is None else qs, w.block_tables,
        w.context_lens if ctx is None else ctx, w.scale, w.k_scale, w.v_scale, rows=rows)


def _logical(w):
    """Per sequence, its K and V tokens in logical order (bulk-write order)."""
    _, k, v, _ = w.ops[0]
    out, off = [], 0
    for n in w.context_lens:
        out.append((k[off:off + n], v[off:off + n]))
        off += int(n)
    return out


@pytest.mark.parametrize("name", ["prefill_gqa70b", "prefill_mha13b", "chunked_gqa70b",
                                  "chunked_fp8"])
def test_prefill_equals_dense_causal_library_softmax(name):
    """Rows of a chunk at positions ctx-n .. ctx-1 equal scipy's softmax of the
    causally masked scores times V on the contiguous logical K/V (for the fp8
    cache: torch's E4M3FN codes of the scaled inputs, widened, times k_scale
    for K and v_scale for V)."""
    w = wl.make_prefill_workload(name, small=True)
    kp, vp = oracle_pools(w)
    out = _prefill(w, kp, vp)
    q = as_f64(raw_numpy(w.prefill_q), w.q_dtype)
    logical = _logical(w)
    for s in range(w.S):
        a, b = int(w.query_start[s]), int(w.query_start[s + 1])
        first = int(w.context_lens[s]) - (b - a)
        if w.pool_dtype == oracle.FP8:
            K = fp8_torch.dequant(logical[s][0], w.k_scale)
            V = fp8_torch.dequant(logical[s][1], w.v_scale)
        else:
            K = as_f64(raw_numpy(logical[s][0]), w.pool_dtype)
            V = as_f64(raw_numpy(logical[s][1]), w.pool_dtype)
        for h in range(w.Hq):
            g = h // w.group
            ref = oracle.dense_causal_attention(q[a:b, h], K[:, g], V[:, g], w.scale, first)
            np.testing.assert_allclose(out[a:b, h], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("name", ["chunked_gqa70b", "chunked_fp8", "prefill_mha13b"])
def test_each_chunk_row_equals_decode_at_its_position(name):
    """A chunk row at position p is the decode step of that token over the first
    p + 1 tokens (the decode oracle is pinned separately), bit for bit."""
    w = wl.make_prefill_workload(name, small=True)
    kp, vp = oracle_pools(w)
    out = _prefill(w, kp, vp)
    rng = np.random.default_rng(1)
    for s in range(w.S):
        a, b = int(w.query_start[s]), int(w.query_start[s + 1])
        for i in sorted({0, b - a - 1, int(rng.integers(0, b - a))}):
            pos = int(w.context_lens[s]) - (b - a) + i
            qd = w.prefill_q[a + i:a + i + 1]
            dec = oracle.paged_attention(kp, vp, w.pool_dtype, w.Hkv, w.D, raw_numpy(qd),
                                         w.q_dtype, 1, w.Hq, w.block_tables[s:s + 1],
                                         np.array([pos + 1], np.int32), w.scale, w.k_scale,
                                         w.v_scale)
            assert_same_bytes(dec[0], out[a + i], what=str((s, i)))


def test_causality_future_tokens_do_not_matter():
    """Changing the K/V of the token after position p leaves row p unchanged,
    bit for bit; changing the token at p itself changes it."""
    w = wl.make_prefill_workload("prefill_mha13b", small=True)
    kp, vp = oracle_pools(w)
    base = _prefill(w, kp, vp)
    s, i = 0, 70  # row at position 70 of sequence 0 (prefix 0)
    for t, expect_same in ((i + 1, True), (i, False)):
        kp2, vp2 = kp.copy(), vp.copy()
        b = int(w.block_tables[s][t // 16])
        k = raw_numpy(torch.full((1, w.Hkv, w.D), 3.0, dtype=torch.bfloat16))
        oracle.reshape_and_cache(kp2, vp2, w.pool_dtype, w.num_blocks, w.Hkv, w.D, k, k,
                                 w.kv_in_dtype, np.array([b * 16 + t % 16], np.int32))
        out = _prefill(w, kp2, vp2)
        same = out[i].tobytes() == base[i].tobytes()
        assert same == expect_same, (t, expect_same)
        # rows before the changed token never change
        assert_same_bytes(out[:t], base[:t])


def test_first_prompt_row_returns_first_value_exactly():
    """A whole-prompt chunk's first row sees one token: its value row, exactly."""
    w = wl.make_prefill_workload("prefill_gqa70b", small=True)
    kp, vp = oracle_pools(w)
    out = _prefill(w, kp, vp)
    logical = _logical(w)
    for s in range(w.S):
        a = int(w.query_start[s])
        V = as_f64(raw_numpy(logical[s][1]), w.pool_dtype)
        for h in range(w.Hq):
            assert (out[a, h] == V[0, h // w.group]).all()


def test_gqa_prefill_equals_mha_with_replicated_kv_heads():
    ctx, D, Hq, Hkv, n = 45, 64, 6, 2, 20
    gen = torch.Generator().manual_seed(8)
    K = torch.randn(ctx, Hkv, D, generator=gen)
    V = torch.randn(ctx, Hkv, D, generator=gen)
    q = torch.randn(n, Hq, D, generator=gen)

    def run(Kx, Vx, H):
        nb = blocks_for(ctx) + 2
        mgr = BlockManager(nb, free_list=np.random.default_rng(0).permutation(nb))
        mgr.add_sequence(0)
        slots, _ = mgr.append_tokens(0, ctx)
        kp = oracle.new_pool(nb, H, D, oracle.F32)
        vp = oracle.new_pool(nb, H, D, oracle.F32)
        oracle.reshape_and_cache(kp, vp, oracle.F32, nb, H, D, Kx.numpy(), Vx.numpy(),
                                 oracle.F32, np.asarray(slots, np.int32))
        t = np.asarray([mgr.block_table(0)], np.int32)
        return oracle.prefill_attention(kp, vp, oracle.F32, H, D, q.numpy(), oracle.F32, 1, Hq,
                                        [0, n], t, [ctx], 0.125)

    gqa = run(K, V, Hkv)
    mha = run(K.repeat_interleave(Hq // Hkv, 1).contiguous(),
              V.repeat_interleave(Hq // Hkv, 1).contiguous(), Hq)
    assert_same_bytes(gqa, mha)


def test_empty_chunks_and_overlong_chunk():
    """Sequences with an empty chunk produce no rows; a chunk longer than its
    context has rows at negative positions, which are zero."""
    w = wl.make_prefill_workload("chunked_gqa70b", small=True)
    kp, vp = oracle_pools(w)
    qs = np.array([0, 0, 40, 40], np.int32)          # only sequence 1 has a chunk
    q = w.prefill_q[40:80].contiguous()
    out = _prefill(w, kp, vp, q=q, qs=qs)
    ref = _prefill(w, kp, vp)
    assert_same_bytes(out, ref[40:80])
    ctx = w.context_lens.copy()
    ctx[0] = 30                                        # chunk of 40 in a 30-token context
    out = _prefill(w, kp, vp, ctx=ctx)
    assert (out[:10] == 0).all()
    assert not (out[10:40] == 0).all()


def test_sampled_rows_equal_full_run():
    w = wl.make_prefill_workload("chunked_gqa70b", small=True)
    kp, vp = oracle_pools(w)
    full = _prefill(w, kp, vp)
    rows = np.array([[0, 0], [119, 63], [57, 17], [80, 8]], np.int32)
    part = _prefill(w, kp, vp, rows=rows)
    for r, (i, h) in enumerate(rows):
        assert_same_bytes(part[r], full[i, h])
