"""Seeded synthetic workloads for paged decode attention.

This module draws inputs only: context lengths, block placement (through the
host block manager), q/K/V values and the order of cache operations.  It holds
no attention, scatter or gather arithmetic, and both the GPU path and the CPU
oracle consume what it returns.

The five workload shapes come from the source pages' scenarios:
- ``tiny``: the worked example of the "PagedAttention" glossary page
  (Ultralytics), section on how paging works: one 40-token request, head
  dim 64, blocks of 16 drawn at random from a pool of 64, fp32.
- ``mha13b``: a LLaMA-13B-shaped layer (40 heads of 128, the model whose
  per-sequence KV cache the same page's memory-problem section sizes at
  1.7 GB): batch 32, bf16, contexts uniform in [1, 2048].
- ``gqa70b``: one layer of the French page's Llama 3.1 70B scenario (memory
  problem section: 256 users x 4096 tokens): 64 query heads over 8 KV heads,
  every context 4096 tokens, blocks scattered.
- ``sampling``: parallel sampling over shared prompts (glossary page, section
  on sharing blocks): 64 prompts x 3 samples, 40 query / 8 KV heads; each
  prompt's blocks are shared by its samples; each sample then appends
  0..512 private tokens.  Variant "a" uses 1024-token prompts (no partial
  shared block, so no copy-on-write); variant "b" uses 1016-token prompts so
  the shared last block is half full and the first writers copy it.
- ``fp8``: FP8 cache (glossary page, related techniques): 128 sequences,
  64 / 8 heads, K/V stored as E4M3 with one fp32 scale per pool
  (max |x| / 448), q in bf16, lognormal context lengths (median 2048,
  sigma 1, clipped to [16, 32768]), split-K partitions of 512 tokens.

Random draws: numpy ``default_rng(seed)`` for lengths and block placement;
``torch.Generator`` seeded with the same seed for N(0, 1) values drawn in
fp32 and rounded to the storage dtype (round-to-nearest-even).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

from .blocks import BlockManager, blocks_for

F32, BF16, FP8 = 0, 1, 2
TORCH_DTYPE = {F32: torch.float32, BF16: torch.bfloat16}
CONFIG_IDS = ("tiny", "mha13b", "gqa70b", "sampling_a", "sampling_b", "fp8")
PREFILL_IDS = ("prefill_gqa70b", "prefill_mha13b", "chunked_gqa70b", "chunked_fp8")
BEAM_IDS = ("beam",)
PREFIX_IDS = ("prefix",)
SEEDS = {"tiny": 0, "mha13b": 1, "gqa70b": 2, "sampling_a": 3, "sampling_b": 3, "fp8": 4,
         "prefill_gqa70b": 5, "prefill_mha13b": 6, "chunked_gqa70b": 7, "chunked_fp8": 8,
         "beam": 9, "prefix": 10}


@dataclass
class Workload:
    name: str
    S: int
    Hq: int
    Hkv: int
    D: int
    pool_dtype: int
    q_dtype: int
    kv_in_dtype: int
    num_blocks: int
    context_lens: np.ndarray          # int32 [S]
    block_tables: np.ndarray          # int32 [S][MBS]; unused entries are -1
    q: torch.Tensor                   # [S][Hq][D]
    scale: float
    k_scale: float = 1.0
    v_scale: float = 1.0
    partition_tokens: int = 0
    # cache operations that build the pool, in order:
    #   ("write", k [N][Hkv][D], v [N][Hkv][D], slots int32 [N]) or ("copy", pairs int32 [P][2])
    ops: list = field(default_factory=list)
    # the newest token of every sequence (what one decode step writes)
    step_k: torch.Tensor | None = None
    step_v: torch.Tensor | None = None
    step_slots: np.ndarray | None = None
    # prefill: each sequence's chunk of new tokens is the last
    # query_start[s+1] - query_start[s] tokens of its context; prefill_q holds
    # their queries, [query_start[S]][Hq][D]
    query_start: np.ndarray | None = None
    prefill_q: torch.Tensor | None = None
    info: dict = field(default_factory=dict)

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes one decode pass reads: sum ctx * Hkv * D * 2 * elem."""
        eb = {F32: 4, BF16: 2, FP8: 1}[self.pool_dtype]
        return int(self.context_lens.astype(np.int64).sum()) * self.Hkv * self.D * 2 * eb

    def prefill_flops(self) -> int:
        """Algorithmic flops of one causal prefill pass: every (chunk token,
        query head) row does 2 D flops for q.K and 2 D for P.V per token it
        sees (positions 0..p)."""
        total = 0
        for s in range(self.S):
            n = int(self.query_start[s + 1] - self.query_start[s])
            c = int(self.context_lens[s])
            first = c - n + 1   # tokens seen by the chunk's first row
            total += n * first + n * (n - 1) // 2
        return total * self.Hq * 4 * self.D

    def prefill_kv_bytes(self) -> int:
        """K+V bytes of every context token of every sequence (each read at
        least once by a prefill pass)."""
        return self.kv_bytes()

    def unique_kv_bytes(self) -> int:
        """K+V bytes of distinct physical token slots one decode pass reads (shared
        prompt blocks counted once)."""
        eb = {F32: 4, BF16: 2, FP8: 1}[self.pool_dtype]
        used = {}
        for s in range(self.S):
            n = int(self.context_lens[s])
            for i in range(-(-n // 16)):
                b = int(self.block_tables[s, i])
                used[b] = max(used.get(b, 0), min(16, n - 16 * i))
        return sum(used.values()) * self.Hkv * self.D * 2 * eb


def _f32(x: float) -> float:
    """The nearest fp32 value: the entry points take the softmax scale as fp32."""
    return float(np.float32(x))


def _randn(gen, shape, dtype, device):
    x = torch.randn(shape, generator=gen, dtype=torch.float32, device=device)
    return x.to(dtype)


def _tables_from(mgr: BlockManager, seq_ids, mbs=None) -> np.ndarray:
    rows = [mgr.block_table(s) for s in seq_ids]
    mbs = mbs or max(1, max(len(r) for r in rows))
    t = np.full((len(rows), mbs), -1, dtype=np.int32)
    for i, r in enumerate(rows):
        t[i, :len(r)] = r
    return t


def _simple(name, S, Hq, Hkv, D, ctx, pool_dt, q_dt, in_dt, scale, seed, device,
            rng, num_blocks=None, free_list=None, partition_tokens=0, fp8_scales=False):
    """Independent sequences, each filled by one bulk write."""
    ctx = np.asarray(ctx, dtype=np.int32)
    need = int(sum(blocks_for(c) for c in ctx))
    nb = need if num_blocks is None else num_blocks
    if free_list is None:
        free_list = rng.permutation(nb)
    mgr = BlockManager(nb, free_list=free_list)
    slots = []
    for s in range(S):
        mgr.add_sequence(s)
        sl, pairs = mgr.append_tokens(s, int(ctx[s]))
        assert not pairs
        slots.extend(sl)
    tables = _tables_from(mgr, range(S))
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    tdt = TORCH_DTYPE[in_dt]
    N = int(ctx.sum())
    q = _randn(gen, (S, Hq, D), TORCH_DTYPE[q_dt], device)
    k = _randn(gen, (N, Hkv, D), tdt, device)
    v = _randn(gen, (N, Hkv, D), tdt, device)
    slots = np.asarray(slots, dtype=np.int32)
    k_scale = v_scale = 1.0
    if fp8_scales:
        k_scale = float((k.abs().max().float() / 448.0).item())
        v_scale = float((v.abs().max().float() / 448.0).item())
    last = np.cumsum(ctx.astype(np.int64)) - 1
    lt = torch.as_tensor(last, device=device)
    w = Workload(name=name, S=S, Hq=Hq, Hkv=Hkv, D=D, pool_dtype=pool_dt, q_dtype=q_dt,
                 kv_in_dtype=in_dt, num_blocks=nb, context_lens=ctx, block_tables=tables,
                 q=q, scale=scale, k_scale=k_scale, v_scale=v_scale,
                 partition_tokens=partition_tokens, ops=[("write", k, v, slots)],
                 step_k=k.index_select(0, lt), step_v=v.index_select(0, lt),
                 step_slots=slots[last])
    w.info["manager"] = mgr
    return w


def make_workload(name: str, small: bool = False, device="cpu", seed: int | None = None,
                  num_seqs: int | None = None) -> Workload:
    """Build one of the named workloads.  ``small`` keeps every per-sequence
    shape but uses a few sequences, so the oracle finishes in seconds."""
    if seed is None:
        seed = SEEDS[name]
    rng = np.random.default_rng(seed)
    if name == "tiny":
        table = rng.choice(64, 3, replace=False)
        free = list(table) + [b for b in range(64) if b not in set(table.tolist())]
        return _simple("tiny", 1, 1, 1, 64, [40], F32, F32, F32, 1.0 / 8.0, seed, device,
                       rng, num_blocks=64, free_list=free)
    if name == "mha13b":
        S = num_seqs or (5 if small else 32)
        ctx = rng.integers(1, 2049, size=S)
        return _simple("mha13b", S, 40, 40, 128, ctx, BF16, BF16, BF16,
                       _f32(1.0 / math.sqrt(128)), seed, device, rng)
    if name == "gqa70b":
        S = num_seqs or (3 if small else 256)
        ctx = np.full(S, 4096)
        return _simple("gqa70b", S, 64, 8, 128, ctx, BF16, BF16, BF16,
                       _f32(1.0 / math.sqrt(128)), seed, device, rng)
    if name == "fp8":
        S = num_seqs or (5 if small else 128)
        z = rng.standard_normal(S)
        ctx = np.clip(np.rint(np.exp(math.log(2048.0) + 1.0 * z)), 16, 32768).astype(np.int64)
        return _simple("fp8", S, 64, 8, 128, ctx, FP8, BF16, BF16, _f32(1.0 / math.sqrt(128)),
                       seed, device, rng, partition_tokens=512, fp8_scales=True)
    if name in ("sampling_a", "sampling_b"):
        return _sampling(name, small, device, seed, rng, num_seqs)
    if name == "beam":
        return make_beam_workload(small, device, seed)
    if name == "prefix":
        return make_prefix_workload(small, device, seed)
    if name in PREFILL_IDS:
        return make_prefill_workload(name, small, device, seed)
    raise KeyError(name)


def make_prefill_workload(name: str, small: bool = False, device="cpu",
                          seed: int | None = None) -> Workload:
    """Prefill workloads: every sequence's context is in the pool (one bulk
    write) and its last ``n_new`` tokens form the chunk whose queries attend
    causally over the context.

    - ``prefill_gqa70b``: whole prompts (chunk = context) with the 70B-like
      heads (64 q / 8 KV, head dim 128, bf16): 8 prompts of 4096 tokens,
      the French page's per-user sequence length.
    - ``prefill_mha13b``: whole prompts with LLaMA-13B heads (40 / 40): 8
      prompts of 2048 tokens.
    - ``chunked_gqa70b``: chunked prefill, 70B-like heads: 32 sequences with
      a cached prefix uniform in [0, 3584] tokens and a 512-token chunk.
    - ``chunked_fp8``: the same with an E4M3 cache (per-pool scales).
    ``small`` keeps the heads but uses 2-3 short, ragged sequences.
    """
    if seed is None:
        seed = SEEDS[name]
    rng = np.random.default_rng(seed)
    scale = _f32(1.0 / math.sqrt(128))
    if name == "prefill_gqa70b":
        Hq, Hkv, pool_dt = 64, 8, BF16
        n_new = np.array([77, 300, 16]) if small else np.full(8, 4096)
        prefix = np.zeros_like(n_new)
    elif name == "prefill_mha13b":
        Hq, Hkv, pool_dt = 40, 40, BF16
        n_new = np.array([150, 33]) if small else np.full(8, 2048)
        prefix = np.zeros_like(n_new)
    elif name in ("chunked_gqa70b", "chunked_fp8"):
        Hq, Hkv = 64, 8
        pool_dt = FP8 if name == "chunked_fp8" else BF16
        S = 3 if small else 32
        n_new = np.full(S, 40 if small else 512)
        prefix = rng.integers(0, 200 if small else 3585, size=S)
        if small:
            prefix[0] = 0
    else:
        raise KeyError(name)
    ctx = (prefix + n_new).astype(np.int32)
    w = _simple(name, len(ctx), Hq, Hkv, 128, ctx, pool_dt, BF16, BF16, scale, seed, device,
                rng, fp8_scales=pool_dt == FP8)
    qs = np.zeros(len(ctx) + 1, dtype=np.int32)
    qs[1:] = np.cumsum(n_new)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed + 1000)
    w.query_start = qs
    w.prefill_q = _randn(gen, (int(qs[-1]), Hq, 128), torch.bfloat16, device)
    return w


def make_beam_workload(small: bool = False, device="cpu", seed: int | None = None,
                       steps: int | None = None) -> Workload:
    """Beam search over shared prompts (glossary page, sharing blocks: beam
    search reuses one copy of the shared prefix; a sequence about to write
    into a block others still use copies it first).

    R requests x W beams with the 70B-like heads (64 q / 8 KV, head dim 128,
    bf16).  Each prompt (1000 tokens, so its last block is partial) is written
    once and shared by its W beams.  Every step then re-selects W parents per
    request with replacement (seeded): beams chosen by no one are freed, a
    beam chosen c times keeps its table for one child and is forked for the
    other c - 1, and every new beam appends one token; writers into a shared
    partial last block copy it first (copy-on-write), in beam order.  The last
    step's copies and writes are the benchmarked step; ``beam_tokens`` holds
    each beam's logical token history (indices into the concatenated writes).
    Full size: 64 requests x 8 beams, 40 steps; small: 2 x 4, 6 steps.
    """
    if seed is None:
        seed = SEEDS["beam"]
    rng = np.random.default_rng(seed)
    R, W = (2, 4) if small else (64, 8)
    T = steps if steps is not None else (6 if small else 40)
    prompt = 37 if small else 1000
    Hq, Hkv, D = 64, 8, 128
    nb = R * (blocks_for(prompt) + W * (T + 2))
    mgr = BlockManager(nb, free_list=rng.permutation(nb))
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    ops, hist, ntok = [], {}, 0
    slots = []
    for r in range(R):
        mgr.add_sequence(("prompt", r))
        sl, _ = mgr.append_tokens(("prompt", r), prompt)
        slots.extend(sl)
        hist[("prompt", r)] = list(range(ntok, ntok + prompt))
        ntok += prompt
    k = _randn(gen, (R * prompt, Hkv, D), torch.bfloat16, device)
    v = _randn(gen, (R * prompt, Hkv, D), torch.bfloat16, device)
    ops.append(("write", k, v, np.asarray(slots, dtype=np.int32)))
    beams = []
    for r in range(R):
        for b in range(W):
            mgr.fork(("prompt", r), (r, b, 0))
            hist[(r, b, 0)] = list(hist[("prompt", r)])
        mgr.free_sequence(("prompt", r))
        beams.append([(r, b, 0) for b in range(W)])
    step_pairs = np.zeros((0, 2), np.int32)
    for t in range(1, T + 1):
        new_beams = []
        for r in range(R):
            parents = np.sort(rng.integers(0, W, size=W))
            counts = np.bincount(parents, minlength=W)
            for b in range(W):                      # drop beams nobody continues
                if counts[b] == 0:
                    mgr.free_sequence(beams[r][b])
                    del hist[beams[r][b]]
            kids = []
            for b in range(W):
                for c in range(int(counts[b])):
                    child = (r, len(kids), t)
                    if c == 0:                      # the first child takes the parent's table
                        mgr.seqs[child] = mgr.seqs.pop(beams[r][b])
                        hist[child] = hist.pop(beams[r][b])
                    else:
                        mgr.fork(kids[-c], child)
                        hist[child] = list(hist[kids[-c]])
                    kids.append(child)
            new_beams.append(kids)
        beams = new_beams
        slots, pairs = [], []
        for r in range(R):
            for sid in beams[r]:
                sl, pr = mgr.append_tokens(sid, 1)
                slots.extend(sl)
                pairs.extend(pr)
                hist[sid].append(ntok)
                ntok += 1
        n = len(slots)
        kn = _randn(gen, (n, Hkv, D), torch.bfloat16, device)
        vn = _randn(gen, (n, Hkv, D), torch.bfloat16, device)
        step_pairs = np.asarray(pairs, dtype=np.int32).reshape(-1, 2)
        if len(pairs):
            ops.append(("copy", step_pairs))
        ops.append(("write", kn, vn, np.asarray(slots, dtype=np.int32)))
    seqs = [sid for r in range(R) for sid in beams[r]]
    ctx = np.asarray([mgr.length(sq) for sq in seqs], dtype=np.int32)
    tables = _tables_from(mgr, seqs)
    q = _randn(gen, (len(seqs), Hq, D), torch.bfloat16, device)
    last = ops[-1]
    w = Workload(name="beam", S=len(seqs), Hq=Hq, Hkv=Hkv, D=D, pool_dtype=BF16, q_dtype=BF16,
                 kv_in_dtype=BF16, num_blocks=nb, context_lens=ctx, block_tables=tables, q=q,
                 scale=_f32(1.0 / math.sqrt(D)), ops=ops, step_k=last[1], step_v=last[2],
                 step_slots=last[3])
    w.info.update(shared_kv=True, manager=mgr, requests=R, beams=W, steps=T, prompt_len=prompt,
                  step_pairs=step_pairs, beam_tokens=[hist[sq] for sq in seqs],
                  cow_copies=mgr.n_cow, physical_blocks=mgr.physical_blocks_in_use(),
                  logical_blocks=mgr.logical_blocks())
    return w


def make_prefix_workload(small: bool = False, device="cpu", seed: int | None = None,
                         caching: bool = True, num_blocks: int | None = None) -> Workload:
    """Requests that start with shared system prompts, served with prefix
    caching by full-block hashing (glossary page, sharing blocks: hashing
    complete blocks extends sharing across requests).

    P system prompts (lengths uniform in [64, 2048]) and R requests, each a
    seeded choice of system prompt plus a private user part of 16..512
    tokens; 70B-like heads (64 q / 8 KV, head dim 128, bf16).  A system
    prompt's K/V depends only on (prompt, position) and user tokens are
    private, so equal prefixes hold equal K/V, as in a model.  Requests
    arrive in order; each reuses the cached full blocks of its prefix and
    writes only the rest (``caching=False`` writes every token into private
    blocks: the reference).  ``query_start`` counts each request's uncached
    tokens, the chunk a chunked prefill computes.  Full size: 8 prompts, 128
    requests; small: 3 prompts, 8 requests.
    """
    from .prefix_cache import PrefixCache
    if seed is None:
        seed = SEEDS["prefix"]
    rng = np.random.default_rng(seed)
    P, R = (3, 8) if small else (8, 128)
    Hq, Hkv, D = 64, 8, 128
    sys_len = rng.integers(64, (300 if small else 2049), size=P)
    sys_ids = [rng.integers(0, 32000, size=int(n)) for n in sys_len]
    choice = rng.integers(0, P, size=R)
    user_len = rng.integers(16, (60 if small else 513), size=R)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    sys_k = [_randn(gen, (int(n), Hkv, D), torch.bfloat16, device) for n in sys_len]
    sys_v = [_randn(gen, (int(n), Hkv, D), torch.bfloat16, device) for n in sys_len]
    user_k = _randn(gen, (int(user_len.sum()), Hkv, D), torch.bfloat16, device)
    user_v = _randn(gen, (int(user_len.sum()), Hkv, D), torch.bfloat16, device)
    user_off = np.concatenate([[0], np.cumsum(user_len)])
    lens = sys_len[choice] + user_len
    nb = num_blocks or int(sum(blocks_for(n) for n in lens))
    mgr = BlockManager(nb, free_list=rng.permutation(nb))
    cache = PrefixCache(mgr) if caching else None
    ks, vs, slots, cached, history = [], [], [], [], []
    for r in range(R):
        s_ = int(choice[r])
        ids = np.concatenate([sys_ids[s_], rng.integers(32000, 64000, size=int(user_len[r]))])
        if cache is not None:
            c, sl = cache.add_request(r, ids)
        else:
            mgr.add_sequence(r)
            c = 0
            sl, _ = mgr.append_tokens(r, len(ids))
        cached.append(c)
        # K/V of tokens c.. of this request, in order
        a, b = user_off[r], user_off[r + 1]
        k_full = torch.cat([sys_k[s_], user_k[a:b]])
        v_full = torch.cat([sys_v[s_], user_v[a:b]])
        ks.append(k_full[c:])
        vs.append(v_full[c:])
        slots.extend(sl)
        history.append((s_, int(a), int(b)))
    cached = np.asarray(cached, dtype=np.int64)
    ctx = lens.astype(np.int32)
    tables = _tables_from(mgr, range(R))
    qs = np.zeros(R + 1, dtype=np.int32)
    qs[1:] = np.cumsum(ctx - cached)
    q = _randn(gen, (R, Hq, D), torch.bfloat16, device)
    w = Workload(name="prefix", S=R, Hq=Hq, Hkv=Hkv, D=D, pool_dtype=BF16, q_dtype=BF16,
                 kv_in_dtype=BF16, num_blocks=nb, context_lens=ctx, block_tables=tables, q=q,
                 scale=_f32(1.0 / math.sqrt(D)),
                 ops=[("write", torch.cat(ks), torch.cat(vs), np.asarray(slots, dtype=np.int32))])
    w.query_start = qs
    w.prefill_q = _randn(gen, (int(qs[-1]), Hq, D), torch.bfloat16, device)
    w.info.update(shared_kv=caching, manager=mgr, cache=cache, cached_tokens=cached,
                  system_len=sys_len,
                  system_choice=choice, user_len=user_len, history=history,
                  physical_blocks=mgr.physical_blocks_in_use(),
                  logical_blocks=mgr.logical_blocks(),
                  system_kv=(sys_k, sys_v), user_kv=(user_k, user_v))
    return w


def _sampling(name, small, device, seed, rng, num_prompts=None) -> Workload:
    P = num_prompts or (2 if small else 64)
    n = 3
    Hq, Hkv, D = 40, 8, 128
    prompt = 1024 if name == "sampling_a" else 1016
    cont = rng.integers(0, 513, size=(P, n))
    # pool: prompt blocks + worst-case private blocks per sample (+1 copy each)
    nb = P * blocks_for(prompt) + int(sum(blocks_for(prompt + c) + 1 for c in cont.ravel()))
    mgr = BlockManager(nb, free_list=rng.permutation(nb))
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    ops = []
    # 1. prompts, written once
    pslots = []
    for p in range(P):
        mgr.add_sequence(("prompt", p))
        sl, pairs = mgr.append_tokens(("prompt", p), prompt)
        assert not pairs
        pslots.extend(sl)
    q = _randn(gen, (P * n, Hq, D), torch.bfloat16, device)
    kp = _randn(gen, (P * prompt, Hkv, D), torch.bfloat16, device)
    vp = _randn(gen, (P * prompt, Hkv, D), torch.bfloat16, device)
    ops.append(("write", kp, vp, np.asarray(pslots, dtype=np.int32)))
    shared_blocks = mgr.physical_blocks_in_use()
    # 2. fork n samples per prompt; the prompt's own handle is then released
    for p in range(P):
        for j in range(n):
            mgr.fork(("prompt", p), (p, j))
        mgr.free_sequence(("prompt", p))
    # 3. each sample appends its private tokens; first writers into a shared
    #    partial block copy it (copy-on-write), in sample order
    cslots, cow = [], []
    for p in range(P):
        for j in range(n):
            sl, pairs = mgr.append_tokens((p, j), int(cont[p, j]))
            cslots.extend(sl)
            cow.extend(pairs)
    if cow:
        ops.append(("copy", np.asarray(cow, dtype=np.int32).reshape(-1, 2)))
    Nc = len(cslots)
    kc = _randn(gen, (Nc, Hkv, D), torch.bfloat16, device)
    vc = _randn(gen, (Nc, Hkv, D), torch.bfloat16, device)
    ops.append(("write", kc, vc, np.asarray(cslots, dtype=np.int32)))
    seqs = [(p, j) for p in range(P) for j in range(n)]
    ctx = np.asarray([mgr.length(s) for s in seqs], dtype=np.int32)
    tables = _tables_from(mgr, seqs)
    # a decode step's cache write: each sample's newest token, where it is a
    # private one (a sample with no private token yet would write into the
    # shared prompt block, which its next step copies first: slot -1 here)
    last = np.cumsum(cont.ravel()) - 1
    has = cont.ravel() > 0
    step_slots = np.where(has, np.asarray(cslots + [-1], np.int32)[np.where(has, last, Nc)], -1)
    li = torch.as_tensor(np.where(has, last, 0), device=kc.device)
    step_k, step_v = (kc.index_select(0, li), vc.index_select(0, li)) if Nc else (None, None)
    w = Workload(name=name, S=P * n, Hq=Hq, Hkv=Hkv, D=D, pool_dtype=BF16, q_dtype=BF16,
                 kv_in_dtype=BF16, num_blocks=nb, context_lens=ctx, block_tables=tables, q=q,
                 scale=_f32(1.0 / math.sqrt(D)), ops=ops, step_k=step_k, step_v=step_v,
                 step_slots=step_slots.astype(np.int32) if Nc else None)
    w.info.update(shared_kv=True, manager=mgr, prompt_len=prompt, continuation=cont,
                  shared_prompt_blocks=shared_blocks, group_sizes=[n] * P,
                  physical_blocks=mgr.physical_blocks_in_use(),
                  logical_blocks=mgr.logical_blocks(), cow_pairs=len(cow))
    return w


def make_groups_workload(groups, Hq: int, Hkv: int, D: int = 128, pool_dtype: int = BF16,
                         seed: int = 0, device="cpu", name: str = "groups") -> Workload:
    """Groups of sequences forked from shared prompts: ``groups`` lists
    (prompt tokens, [continuation tokens of each member]).  Each prompt is
    written once; its members fork it (sharing its blocks, with reference
    counts) and append their continuations, the first writers into a shared
    partly filled block copying it first (glossary page, sharing blocks
    between sequences).  Sequences are numbered group by group;
    ``info["group_sizes"]`` holds the member counts.  bf16 inputs; an fp8
    pool gets per-pool scales (max |x| / 448)."""
    rng = np.random.default_rng(seed)
    nb = int(sum(blocks_for(pl) + sum(blocks_for(pl + c) + 1 for c in cs) for pl, cs in groups))
    mgr = BlockManager(nb, free_list=rng.permutation(nb))
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    pslots = []
    for gi, (pl, _) in enumerate(groups):
        mgr.add_sequence(("prompt", gi))
        sl, _ = mgr.append_tokens(("prompt", gi), int(pl))
        pslots.extend(sl)
    seqs = [(gi, j) for gi, (_, cs) in enumerate(groups) for j in range(len(cs))]
    q = _randn(gen, (len(seqs), Hq, D), torch.bfloat16, device)
    kp = _randn(gen, (len(pslots), Hkv, D), torch.bfloat16, device)
    vp = _randn(gen, (len(pslots), Hkv, D), torch.bfloat16, device)
    ops = [("write", kp, vp, np.asarray(pslots, dtype=np.int32))]
    for gi, (_, cs) in enumerate(groups):
        for j in range(len(cs)):
            mgr.fork(("prompt", gi), (gi, j))
        mgr.free_sequence(("prompt", gi))
    cslots, cow = [], []
    for gi, (_, cs) in enumerate(groups):
        for j, c in enumerate(cs):
            sl, pairs = mgr.append_tokens((gi, j), int(c))
            cslots.extend(sl)
            cow.extend(pairs)
    if cow:
        ops.append(("copy", np.asarray(cow, dtype=np.int32).reshape(-1, 2)))
    kc = _randn(gen, (len(cslots), Hkv, D), torch.bfloat16, device)
    vc = _randn(gen, (len(cslots), Hkv, D), torch.bfloat16, device)
    if cslots:
        ops.append(("write", kc, vc, np.asarray(cslots, dtype=np.int32)))
    k_scale = v_scale = 1.0
    if pool_dtype == FP8:
        k_scale = float((torch.cat([kp, kc]).abs().max().float() / 448.0).item())
        v_scale = float((torch.cat([vp, vc]).abs().max().float() / 448.0).item())
    ctx = np.asarray([mgr.length(sq) for sq in seqs], dtype=np.int32)
    w = Workload(name=name, S=len(seqs), Hq=Hq, Hkv=Hkv, D=D, pool_dtype=pool_dtype, q_dtype=BF16,
                 kv_in_dtype=BF16, num_blocks=nb, context_lens=ctx,
                 block_tables=_tables_from(mgr, seqs), q=q, scale=_f32(1.0 / math.sqrt(D)),
                 k_scale=k_scale, v_scale=v_scale, ops=ops)
    w.info.update(manager=mgr, group_sizes=[len(cs) for _, cs in groups], cow_pairs=len(cow))
    return w


def raw_numpy(t: torch.Tensor) -> np.ndarray:
    """The raw element bits of a CPU/GPU tensor as a numpy array (bf16 as uint16)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
