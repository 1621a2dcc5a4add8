"""Prefix caching by full-block hashing, on the host.

The glossary page's section on sharing blocks between sequences: hashing
complete blocks extends block sharing across requests, which is how vLLM
caches prompts.  Here a full block of 16 tokens is named by a chained hash of
its parent block's hash and its own token ids, so two equal hashes stand for
two equal prefixes, and a request whose prompt starts with a cached prefix
reuses those physical blocks (with a reference each) instead of computing and
writing their K/V again.  Only full blocks enter the cache: a partial block
may still receive tokens.

A cached block whose reference count drops to zero stays in the table, its
K/V still valid, and waits on the free list; a later hit takes it back off
the free list, and when the allocator hands it to new content its entry is
dropped.  The kernels are unchanged: cached prefixes are just blocks in the
requests' block tables, read by pa_decode and by pa_prefill for the uncached
rest of each prompt.
"""
from __future__ import annotations

import hashlib

import numpy as np

from .blocks import BLOCK_SIZE, BlockManager


def block_hash(parent: bytes, tokens) -> bytes:
    """Chained hash of one full block: its parent's hash and its token ids."""
    h = hashlib.sha256()
    h.update(parent)
    h.update(np.asarray(tokens, dtype=np.int64).tobytes())
    return h.digest()


class PrefixCache:
    """Full-block hash -> physical block map on top of a BlockManager."""

    def __init__(self, manager: BlockManager):
        self.mgr = manager
        self.block_of: dict = {}   # hash -> block id
        self.hash_of: dict = {}    # block id -> hash
        self.hit_blocks = 0
        self.new_blocks = 0
        self.evicted = 0
        allocate = manager._allocate

        def allocate_dropping_stale_entry() -> int:
            b = allocate()
            h = self.hash_of.pop(b, None)
            if h is not None:      # the block now gets new content
                del self.block_of[h]
                self.evicted += 1
            return b

        manager._allocate = allocate_dropping_stale_entry

    def add_request(self, seq_id, token_ids):
        """Start sequence ``seq_id`` for the prompt ``token_ids``.

        Reuses the cached blocks of the prompt's longest cached run of full
        blocks and reserves slots for the rest.  Returns ``(cached, slots)``:
        the number of leading tokens whose K/V is already in the pool, and
        the slots of the remaining tokens, which the caller writes
        (pa_reshape_and_cache) and attends (pa_prefill) before any other
        request can hit their blocks.
        """
        mgr = self.mgr
        token_ids = np.asarray(token_ids, dtype=np.int64)
        n = len(token_ids)
        mgr.add_sequence(seq_id)
        seq = mgr.seqs[seq_id]
        parent = b""
        cached = 0
        for i in range(n // BLOCK_SIZE):
            h = block_hash(parent, token_ids[BLOCK_SIZE * i:BLOCK_SIZE * (i + 1)])
            b = self.block_of.get(h)
            if b is None:
                break
            if mgr.refcount[b] == 0:
                mgr.free.remove(b)             # a cached block back in use
            mgr.refcount[b] += 1
            seq.table.append(b)
            seq.length += BLOCK_SIZE
            parent = h
            cached += BLOCK_SIZE
        self.hit_blocks += cached // BLOCK_SIZE
        slots, pairs = mgr.append_tokens(seq_id, n - cached)
        assert not pairs, "a request's own new blocks are never shared"
        for i in range(cached // BLOCK_SIZE, n // BLOCK_SIZE):
            h = block_hash(parent, token_ids[BLOCK_SIZE * i:BLOCK_SIZE * (i + 1)])
            b = seq.table[i]
            self.block_of[h] = b
            self.hash_of[b] = h
            parent = h
            self.new_blocks += 1
        return cached, slots
