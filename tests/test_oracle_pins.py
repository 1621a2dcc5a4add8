"""Pins of the CPU oracle against what the source pages and mathematics fix.

Each test names the fact it checks.  None of them re-derives the oracle's
formula: they use the pages' worked example, library routines (scipy softmax,
torch's float8_e4m3fn cast), closed forms, invariants and exact integers.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import fp8_torch
import oracle
from oracle_helpers import as_f64, oracle_decode, oracle_pools
from paged_kv_cache_401_amd import workloads as wl
from paged_kv_cache_401_amd.blocks import BlockManager, blocks_for, unused_slots
from paged_kv_cache_401_amd.workloads import raw_numpy
from bitwise import assert_same_bytes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- worked example
def test_worked_example_table_readback_and_waste():
    """Glossary page, how paging works: 40 keys of dim 64 in a 64-block pool with
    free list [41, 7, 19, 2, 33] take ceil(40/16) = 3 blocks -> table [41, 7, 19];
    reading back through the table returns the keys bit for bit; 8 slots stay
    unused against 2008 for a 2048-token reservation."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    n, D, NB = g["num_tokens"], g["head_dim"], g["pool_blocks"]
    mgr = BlockManager(NB, free_list=g["free_list"])
    mgr.add_sequence(0)
    slots, pairs = mgr.append_tokens(0, n)
    table = mgr.block_table(0)
    assert pairs == []
    assert blocks_for(n) == g["expected_blocks_needed"]
    assert table == g["expected_block_table"]
    assert mgr.free == g["free_list"][len(table):]
    # token pos lives in block table[pos // 16] at slot pos % 16
    for pos, s in enumerate(slots):
        assert s // 16 == table[pos // 16] and s % 16 == pos % 16
    gen = torch.Generator().manual_seed(0)
    keys = torch.randn(n, D, generator=gen)
    kp = oracle.new_pool(NB, 1, D, oracle.F32)
    vp = oracle.new_pool(NB, 1, D, oracle.F32)
    k3 = keys.reshape(n, 1, D).numpy()
    oracle.reshape_and_cache(kp, vp, oracle.F32, NB, 1, D, k3, k3, oracle.F32, slots)
    got = oracle.gather(kp, False, oracle.F32, 1, D, table, n, 0)
    intact = got.tobytes() == keys.numpy().tobytes()
    assert intact == g["expected_keys_intact"]
    assert unused_slots(n) == g["expected_unused_slots_paged"]
    assert g["reservation_tokens"] - n == g["expected_unused_slots_reserved"]
    # only the three table blocks changed (the pool starts zeroed)
    tile = 16 * D * 4
    touched = {b for b in range(NB) if kp[b * tile:(b + 1) * tile].any()}
    assert touched == set(table)


def test_scatter_sentinel_and_negative_slots():
    """Slots outside the write set keep their bytes; a negative slot is skipped."""
    NB, Hkv, D = 6, 2, 64
    for dt in (oracle.F32, oracle.BF16):
        kp = oracle.new_pool(NB, Hkv, D, dt, fill=0xFF)
        vp = oracle.new_pool(NB, Hkv, D, dt, fill=0xFF)
        npdt = np.float32 if dt == oracle.F32 else np.uint16
        k = np.arange(3 * Hkv * D).astype(npdt).reshape(3, Hkv, D)
        slots = np.array([17, -1, 95], dtype=np.int32)
        oracle.reshape_and_cache(kp, vp, dt, NB, Hkv, D, k, k, dt, slots)
        eb = oracle.ELEM_BYTES[dt]
        changed = (kp != 0xFF).sum()
        # two tokens x Hkv heads x D elements, each eb bytes (none of them 0xFF-only)
        assert changed <= 2 * Hkv * D * eb and changed >= 2 * Hkv * D
        got = oracle.gather(kp, False, dt, Hkv, D, [1], 2, 1)
        assert_same_bytes(got[1], k[0, 1])
        got = oracle.gather(vp, True, dt, Hkv, D, [0, 5], 32, 0)
        assert_same_bytes(got[31], k[2, 0])


def test_copy_blocks_copies_whole_blocks_only():
    NB, Hkv, D = 5, 2, 64
    rng = np.random.default_rng(3)
    kp = rng.integers(0, 256, NB * Hkv * 16 * D * 2, dtype=np.uint8)
    vp = rng.integers(0, 256, NB * Hkv * 16 * D * 2, dtype=np.uint8)
    k0, v0 = kp.copy(), vp.copy()
    oracle.copy_blocks(kp, vp, oracle.BF16, Hkv, D, [[3, 1], [0, 4]])
    t = Hkv * 16 * D * 2
    blk = lambda a, b: a[b * t:(b + 1) * t]
    assert (blk(kp, 1) == blk(k0, 3)).all() and (blk(vp, 4) == blk(v0, 0)).all()
    for b in (0, 2, 3):
        assert (blk(kp, b) == blk(k0, b)).all() and (blk(vp, b) == blk(v0, b)).all()
    oracle.copy_blocks(kp, vp, oracle.BF16, Hkv, D, np.zeros((0, 2), np.int32))


@pytest.mark.parametrize("name", ["tiny", "mha13b", "gqa70b", "sampling_b", "fp8"])
def test_workload_readback_through_tables(name):
    """Every sequence's tokens read back through its table in logical order
    (the Russian page: attention reads through the table keeping the order).
    An fp8 pool holds the E4M3FN codes of the inputs scaled by fp32(1/scale):
    they read back as torch's float8_e4m3fn cast of those products (glossary
    page, related techniques: the 8-bit cache)."""
    w = wl.make_workload(name, small=True)
    kp, vp = oracle_pools(w)
    logical = _logical_tokens(w)
    for s in range(w.S):
        n = int(w.context_lens[s])
        for g in range(w.Hkv):
            for pool, is_v, idx in ((kp, False, 0), (vp, True, 1)):
                got = oracle.gather(pool, is_v, w.pool_dtype, w.Hkv, w.D, w.block_tables[s], n, g)
                x = logical[s][idx][:, g, :]
                if w.pool_dtype == oracle.FP8:
                    want = fp8_torch.codes(x, w.v_scale if is_v else w.k_scale)
                else:
                    want = raw_numpy(x)
                assert_same_bytes(got, want, what=str((s, g, is_v)))


def _logical_tokens(w):
    """Per sequence, its K and V tokens in logical order, from the draw order."""
    if not w.name.startswith("sampling"):
        _, k, v, _ = w.ops[0]
        out, off = [], 0
        for n in w.context_lens:
            out.append((k[off:off + n], v[off:off + n]))
            off += int(n)
        return out
    P, L = w.S // 3, w.info["prompt_len"]
    kp_, vp_ = w.ops[0][1], w.ops[0][2]
    kc, vc = w.ops[-1][1], w.ops[-1][2]
    out, off = [], 0
    for p in range(P):
        for j in range(3):
            c = int(w.info["continuation"][p, j])
            out.append((torch.cat([kp_[p * L:(p + 1) * L], kc[off:off + c]]),
                        torch.cat([vp_[p * L:(p + 1) * L], vc[off:off + c]])))
            off += c
    return out


# ------------------------------------------------------------- dense equivalence
@pytest.mark.parametrize("name", ["tiny", "mha13b", "gqa70b", "sampling_b", "fp8"])
def test_paged_equals_dense_library_softmax(name):
    """Paging changes where bytes live, not the result: the paged oracle equals
    scipy softmax(scale q K^T) V on the contiguous logical K/V.  For the fp8
    cache the contiguous K and V are what the pool holds, built without the
    oracle: torch's E4M3FN codes of the scaled inputs, widened by torch, times
    k_scale for K and v_scale for V (the workload's two scales differ)."""
    w = wl.make_workload(name, small=True)
    kp, vp = oracle_pools(w)
    out = oracle_decode(w, kp, vp)
    logical = _logical_tokens(w)
    q = as_f64(raw_numpy(w.q), w.q_dtype)
    if w.pool_dtype == oracle.FP8:
        assert w.k_scale != w.v_scale
    for s in range(w.S):
        if w.pool_dtype == oracle.FP8:
            K = fp8_torch.dequant(logical[s][0], w.k_scale)
            V = fp8_torch.dequant(logical[s][1], w.v_scale)
        else:
            K = as_f64(raw_numpy(logical[s][0]), w.pool_dtype)
            V = as_f64(raw_numpy(logical[s][1]), w.pool_dtype)
        for h in range(w.Hq):
            g = h // w.group
            ref = oracle.dense_attention(q[s, h], K[:, g, :], V[:, g, :], w.scale)
            np.testing.assert_allclose(out[s, h], ref, rtol=0, atol=1e-12)


def test_fp8_scales_two_tokens_closed_form():
    """Two tokens in an fp8 pool with distinct power-of-two scales (inputs on
    the E4M3FN grid times the scale, so every code is exact): the scores use
    K = code * k_scale and the output mixes V = code * v_scale with logistic
    weights -- a swapped, dropped or inverted scale changes the result."""
    from scipy.special import expit
    D, k_scale, v_scale, scale = 64, 2.0 ** -5, 2.0 ** -1, 0.75   # all exact in fp32
    rng = np.random.default_rng(12)
    grid = oracle.fp8_decode(np.arange(0, 0x78, dtype=np.uint8))    # 0 .. 240, exact codes
    kc = rng.choice(grid, (2, D)) * rng.choice([-1.0, 1.0], (2, D))
    vc = rng.choice(grid, (2, D)) * rng.choice([-1.0, 1.0], (2, D))
    K = torch.from_numpy(kc * k_scale).float().reshape(2, 1, D)
    V = torch.from_numpy(vc * v_scale).float().reshape(2, 1, D)
    nb = 3
    kp = oracle.new_pool(nb, 1, D, oracle.FP8)
    vp = oracle.new_pool(nb, 1, D, oracle.FP8)
    oracle.reshape_and_cache(kp, vp, oracle.FP8, nb, 1, D, K.numpy(), V.numpy(), oracle.F32,
                             np.array([32, 33], np.int32), k_scale, v_scale)
    q = (torch.randn(1, 1, D, generator=torch.Generator().manual_seed(3)) / 16).to(torch.bfloat16)
    out = oracle.paged_attention(kp, vp, oracle.FP8, 1, D, raw_numpy(q), oracle.BF16, 1, 1,
                                 np.array([[2]], np.int32), np.array([2], np.int32), scale,
                                 k_scale, v_scale)
    qd = q[0, 0].double().numpy()
    s0, s1 = scale * float(qd @ (kc[0] * k_scale)), scale * float(qd @ (kc[1] * k_scale))
    ref = expit(s0 - s1) * vc[0] * v_scale + expit(s1 - s0) * vc[1] * v_scale
    assert abs(s0 - s1) > 0.5      # the weights are far from 1/2
    np.testing.assert_allclose(out[0, 0], ref, rtol=0, atol=1e-14)


# ----------------------------------------------------------------- invariants
def test_block_placement_invariance_bit_exact():
    """Relabelling physical blocks (pool and tables together) leaves every
    output bit unchanged (the table, not placement, defines the order)."""
    w = wl.make_workload("mha13b", small=True)
    kp, vp = oracle_pools(w)
    ref = oracle_decode(w, kp, vp)
    perm = np.random.default_rng(11).permutation(w.num_blocks).astype(np.int32)
    kp2 = oracle.new_pool(w.num_blocks, w.Hkv, w.D, w.pool_dtype)
    vp2 = oracle.new_pool(w.num_blocks, w.Hkv, w.D, w.pool_dtype)
    _, k, v, slots = w.ops[0]
    slots2 = perm[slots // 16] * 16 + slots % 16
    oracle.reshape_and_cache(kp2, vp2, w.pool_dtype, w.num_blocks, w.Hkv, w.D, raw_numpy(k),
                             raw_numpy(v), w.kv_in_dtype, slots2.astype(np.int32))
    tables2 = np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)], -1)
    out = oracle_decode(w, kp2, vp2, tables=tables2.astype(np.int32))
    assert_same_bytes(out, ref)


@pytest.mark.parametrize("name", ["sampling_a", "sampling_b"])
def test_shared_prefix_equals_private_copies(name):
    """Glossary page, sharing blocks: samples pointing at shared, refcounted
    prompt blocks (with copy-on-write of the partial block) give the same
    outputs, bit for bit, as samples holding private copies."""
    w = wl.make_workload(name, small=True)
    kp, vp = oracle_pools(w)
    shared = oracle_decode(w, kp, vp)
    if name == "sampling_b":
        assert w.info["cow_pairs"] > 0
        assert w.info["physical_blocks"] < w.info["logical_blocks"]
    logical = _logical_tokens(w)
    mgr = BlockManager(sum(blocks_for(n) for n in w.context_lens))
    kp2 = oracle.new_pool(mgr.num_blocks, w.Hkv, w.D, w.pool_dtype)
    vp2 = oracle.new_pool(mgr.num_blocks, w.Hkv, w.D, w.pool_dtype)
    for s in range(w.S):
        mgr.add_sequence(s)
        slots, _ = mgr.append_tokens(s, int(w.context_lens[s]))
        oracle.reshape_and_cache(kp2, vp2, w.pool_dtype, mgr.num_blocks, w.Hkv, w.D,
                                 raw_numpy(logical[s][0]), raw_numpy(logical[s][1]),
                                 w.kv_in_dtype, np.asarray(slots, np.int32))
    tables = np.full((w.S, max(blocks_for(n) for n in w.context_lens)), -1, np.int32)
    for s in range(w.S):
        t = mgr.block_table(s)
        tables[s, :len(t)] = t
    private = oracle_decode(w, kp2, vp2, tables=tables)
    assert_same_bytes(private, shared)


def _tiny_pool(ctx, Hkv=1, D=64, seed=0, dt=oracle.F32, K=None, V=None):
    """A pool holding one sequence of ctx tokens in scattered blocks."""
    rng = np.random.default_rng(seed)
    nb = max(1, blocks_for(ctx)) + 3
    mgr = BlockManager(nb, free_list=rng.permutation(nb))
    mgr.add_sequence(0)
    slots, _ = mgr.append_tokens(0, ctx)
    gen = torch.Generator().manual_seed(seed)
    K = torch.randn(ctx, Hkv, D, generator=gen) if K is None else K
    V = torch.randn(ctx, Hkv, D, generator=gen) if V is None else V
    tdt = torch.float32 if dt == oracle.F32 else torch.bfloat16
    K, V = K.to(tdt), V.to(tdt)
    kp = oracle.new_pool(nb, Hkv, D, dt)
    vp = oracle.new_pool(nb, Hkv, D, dt)
    oracle.reshape_and_cache(kp, vp, dt, nb, Hkv, D, raw_numpy(K), raw_numpy(V), dt,
                             np.asarray(slots, np.int32))
    table = np.full((1, max(1, blocks_for(ctx))), -1, np.int32)
    table[0, :len(mgr.block_table(0))] = mgr.block_table(0)
    return kp, vp, table, K, V


def _attend(kp, vp, table, ctx, q, scale, Hkv=1, D=64, dt=oracle.F32):
    Hq = q.shape[1]
    return oracle.paged_attention(kp, vp, dt, Hkv, D, raw_numpy(q), dt, 1, Hq, table,
                                  np.array([ctx], np.int32), scale)


def test_single_token_returns_its_value_exactly():
    kp, vp, table, K, V = _tiny_pool(1)
    q = torch.randn(1, 1, 64)
    out = _attend(kp, vp, table, 1, q, 0.125)
    assert (out[0, 0] == V[0, 0].double().numpy()).all()


def test_zero_query_gives_mean_of_values():
    kp, vp, table, K, V = _tiny_pool(37)
    out = _attend(kp, vp, table, 37, torch.zeros(1, 1, 64), 0.125)
    np.testing.assert_allclose(out[0, 0], V[:, 0].double().mean(0).numpy(), rtol=0, atol=1e-15)


def test_two_tokens_logistic_closed_form():
    """With two tokens the weights are logistic functions of the score gap."""
    from scipy.special import expit
    kp, vp, table, K, V = _tiny_pool(2, seed=5)
    q = torch.randn(1, 1, 64, generator=torch.Generator().manual_seed(9))
    scale = 0.125
    out = _attend(kp, vp, table, 2, q, scale)
    s0 = scale * float(np.dot(q[0, 0].double().numpy(), K[0, 0].double().numpy()))
    s1 = scale * float(np.dot(q[0, 0].double().numpy(), K[1, 0].double().numpy()))
    ref = expit(s0 - s1) * V[0, 0].double().numpy() + expit(s1 - s0) * V[1, 0].double().numpy()
    np.testing.assert_allclose(out[0, 0], ref, rtol=0, atol=1e-14)


def test_gqa_equals_mha_with_replicated_kv_heads():
    """Grouped-query attention (glossary page, related techniques) is MHA in
    which each KV head is repeated for its group of query heads."""
    ctx, D, Hq, Hkv = 53, 64, 6, 2
    gen = torch.Generator().manual_seed(2)
    K = torch.randn(ctx, Hkv, D, generator=gen)
    V = torch.randn(ctx, Hkv, D, generator=gen)
    q = torch.randn(1, Hq, D, generator=gen)
    kp, vp, table, _, _ = _tiny_pool(ctx, Hkv=Hkv, K=K, V=V)
    gqa = oracle.paged_attention(kp, vp, oracle.F32, Hkv, D, q.numpy(), oracle.F32, 1, Hq,
                                 table, np.array([ctx], np.int32), 0.125)
    Kr = K.repeat_interleave(Hq // Hkv, dim=1)
    Vr = V.repeat_interleave(Hq // Hkv, dim=1)
    kp2, vp2, table2, _, _ = _tiny_pool(ctx, Hkv=Hq, K=Kr, V=Vr)
    mha = oracle.paged_attention(kp2, vp2, oracle.F32, Hq, D, q.numpy(), oracle.F32, 1, Hq,
                                 table2, np.array([ctx], np.int32), 0.125)
    assert_same_bytes(gqa, mha)


def test_linear_in_values_and_inside_their_hull():
    ctx = 70
    gen = torch.Generator().manual_seed(4)
    K = torch.randn(ctx, 1, 64, generator=gen)
    # values on a 1/16 grid, so that 2*V1 - 3*V2 is exact in fp32
    V1 = torch.randint(-64, 65, (ctx, 1, 64), generator=gen).float() / 16
    V2 = torch.randint(-64, 65, (ctx, 1, 64), generator=gen).float() / 16
    q = torch.randn(1, 1, 64, generator=gen)
    outs = []
    for V in (V1, V2, 2.0 * V1 - 3.0 * V2):
        kp, vp, table, _, _ = _tiny_pool(ctx, K=K, V=V)
        outs.append(_attend(kp, vp, table, ctx, q, 0.3)[0, 0])
    np.testing.assert_allclose(outs[2], 2.0 * outs[0] - 3.0 * outs[1], rtol=0, atol=1e-13)
    lo, hi = V1[:, 0].double().min(0).values.numpy(), V1[:, 0].double().max(0).values.numpy()
    assert (outs[0] >= lo).all() and (outs[0] <= hi).all()


@pytest.mark.parametrize("target", [0, 15, 16, 40, 77])
def test_one_hot_probe_selects_exactly_one_value(target):
    """Score c*scale >= 200 on one token and 0 elsewhere: every other weight is
    below 1e-86, so the output equals that token's value row exactly."""
    ctx, D = 78, 64
    K = torch.zeros(ctx, 1, D)
    K[target, 0, 0] = 1000.0
    V = torch.randn(ctx, 1, D, generator=torch.Generator().manual_seed(target))
    q = torch.zeros(1, 1, D)
    q[0, 0, 0] = 1.0
    kp, vp, table, _, _ = _tiny_pool(ctx, K=K, V=V)
    out = _attend(kp, vp, table, ctx, q, 0.25)
    assert (out[0, 0] == V[target, 0].double().numpy()).all()


def test_empty_context_gives_zeros():
    kp, vp, table, _, _ = _tiny_pool(5)
    out = oracle.paged_attention(kp, vp, oracle.F32, 1, 64, np.ones((1, 1, 64), np.float32),
                                 oracle.F32, 1, 1, table, np.array([0], np.int32), 0.125)
    assert (out == 0).all()


# ------------------------------------------------------------------ fp8 codec
def test_fp8_decode_matches_torch_float8_e4m3fn():
    """The 256-code E4M3FN table equals torch's float8_e4m3fn widening."""
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.fp8_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert (mine[ok] == ref[ok]).all()
    assert np.isnan(mine[[0x7F, 0xFF]]).all() and np.isnan(mine).sum() == 2
    assert mine[0x7E] == 448.0 and mine[0x08] == 2.0 ** -6 and mine[0x01] == 2.0 ** -9
    assert mine[0x38] == 1.0 and mine[0x80] == 0.0 and np.signbit(mine[0x80])


def test_fp8_encode_matches_torch_cast_below_overflow():
    """Round-to-nearest-even agrees with torch's cast wherever torch does not
    overflow to NaN (|x| < 464, the midpoint above 448)."""
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(2.0) ** rng.integers(
            -14, 9, 200000).astype(np.float32),
        oracle.fp8_decode(np.arange(127, dtype=np.uint8)).astype(np.float32),
    ])
    vals = oracle.fp8_decode(np.arange(127, dtype=np.uint8))
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)  # exact in fp32
    x = np.concatenate([x, mids, -mids, np.nextafter(mids, np.float32(0)),
                        np.nextafter(mids, np.float32(1e9))]).astype(np.float32)
    x = x[np.abs(x) < 464]
    mine = oracle.fp8_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)


def test_fp8_encode_saturates_and_keeps_nan():
    x = np.array([448.0, 463.9, 464.0, 1000.0, 1e30, np.inf, -np.inf, -500.0, np.nan, -0.0],
                 dtype=np.float32)
    got = oracle.fp8_encode(x)
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F, 0x80]


def test_fp8_pool_is_half_of_bf16_pool():
    """Glossary page, related techniques: an 8-bit cache takes about half the
    memory of a 16-bit one (exactly half for the same block count)."""
    a = oracle.new_pool(100, 8, 128, oracle.FP8).nbytes
    b = oracle.new_pool(100, 8, 128, oracle.BF16).nbytes
    assert 2 * a == b


def test_fp8_scatter_encodes_scaled_values():
    """An fp8 pool stores encode(x * fp32(1/scale)); decoding times the scale
    recovers x within half an fp8 step."""
    gen = torch.Generator().manual_seed(1)
    x = torch.randn(40, 1, 128, generator=gen).to(torch.bfloat16)
    scale = float((x.abs().max().float() / 448.0).item())
    kp, vp, table, _, _ = (None,) * 5
    nb = 3
    kp = oracle.new_pool(nb, 1, 128, oracle.FP8)
    vp = oracle.new_pool(nb, 1, 128, oracle.FP8)
    slots = np.arange(40, dtype=np.int32)
    oracle.reshape_and_cache(kp, vp, oracle.FP8, nb, 1, 128, raw_numpy(x), raw_numpy(x),
                             oracle.BF16, slots, scale, scale)
    codes = oracle.gather(kp, False, oracle.FP8, 1, 128, [0, 1, 2], 40, 0)
    xf = x.float().numpy().reshape(40, 128)
    inv = np.float32(1.0) / np.float32(scale)
    want = oracle.fp8_encode((xf * inv).astype(np.float32))
    assert np.array_equal(codes, want)
    back = oracle.fp8_decode(codes.ravel()).reshape(40, 128) * scale
    rel = np.abs(back - xf) / np.maximum(np.abs(xf), 2.0 ** -6 * scale)
    assert rel.max() <= 2.0 ** -4 + 1e-6


# --------------------------------------------------------------- accounting
def test_waste_is_only_the_last_block_tail():
    """Glossary page: waste is bounded by the unfilled part of the last block."""
    for n in range(1, 200):
        assert unused_slots(n) == 16 * math.ceil(n / 16) - n
        assert 0 <= unused_slots(n) < 16
    # contexts uniform in [1, 2048]: mean waste is exactly 7.5 slots
    assert np.mean([unused_slots(n) for n in range(1, 2049)]) == 7.5


def test_sampling_accounting():
    w = wl.make_workload("sampling_a", small=True)
    P = w.S // 3
    assert w.info["shared_prompt_blocks"] == P * 64
    assert w.info["cow_pairs"] == 0
    cont = w.info["continuation"]
    logical = sum(blocks_for(1024 + c) for c in cont.ravel())
    private = sum(blocks_for(c) for c in cont.ravel())
    assert w.info["logical_blocks"] == logical
    assert w.info["physical_blocks"] == P * 64 + private
    wb = wl.make_workload("sampling_b", small=True)
    # three holders of each half-full prompt block: every writer but the last
    # holder copies, so a prompt with k writing samples makes min(k, 2) copies
    writers = (wb.info["continuation"] > 0).sum(axis=1)
    assert wb.info["cow_pairs"] == int(np.minimum(writers, 2).sum())
