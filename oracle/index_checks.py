"""Plain-Python statement of the index preconditions that the paged-cache
operations trust, used to check the library's device-side index checks.

TEST INFRASTRUCTURE ONLY (same rules as the rest of ``oracle/``).

The pages fix how indices are formed -- token ``pos`` of a request lives in
slot ``pos % 16`` of block ``table[pos // 16]`` (glossary page, how paging
works; Russian page, logical order vs physical placement), a copy-on-write
copies one shared block to a fresh one (glossary page, sharing blocks) and
eviction moves whole blocks to host memory (French page, how PagedAttention
solves this) -- but not what an operation does when the indices break those
rules.  The reading taken here: every id must name an existing block, slot
or host slot; a context never exceeds its table; one call never writes the
same slot or block twice; a copy never reads a block it also writes; chunk
offsets start at 0 and never decrease.

Each check returns (faults, kinds, first): one fault per (element, kind) at
fault, the OR of the kinds, and the smallest element index at fault (-1 if
none).  A repeated id is a fault of every element that names it.
"""
from __future__ import annotations

from collections import Counter

# fault kinds: the bit values of the library's report (a stated interface)
CONTEXT_LEN, BLOCK_ID, SLOT_RANGE, SLOT_REPEATED = 1, 2, 4, 8
PAIR_RANGE, DST_REPEATED, DST_IS_SRC, HOST_SLOT_REPEATED, QUERY_START = 16, 32, 64, 128, 256
BLOCK = 16


def _report(faults):
    """faults: list of (element index, kind)."""
    if not faults:
        return 0, 0, -1
    kinds = 0
    for _, k in faults:
        kinds |= k
    return len(faults), kinds, min(i for i, _ in faults)


def check_tables(num_blocks, block_tables, context_lens):
    """Sequence s reads the first ceil(ctx / 16) entries of its table row,
    ctx clamped to the row's capacity; its length must fit the row."""
    faults = []
    for s, row in enumerate(block_tables):
        row = [int(b) for b in row]
        cap = len(row) * BLOCK
        c = int(context_lens[s])
        if c < 0 or c > cap:
            faults.append((s, CONTEXT_LEN))
        c = min(max(c, 0), cap)
        used = row[:(c + BLOCK - 1) // BLOCK]
        if any(b < 0 or b >= num_blocks for b in used):
            faults.append((s, BLOCK_ID))
    return _report(faults)


def check_query_start(query_start):
    qs = [int(x) for x in query_start]
    faults = [(0, QUERY_START)] if qs[0] != 0 else []
    for s in range(1, len(qs)):
        if qs[s] < qs[s - 1]:
            faults.append((s, QUERY_START))
    return _report(faults)


def check_slots(num_blocks, slot_mapping):
    """Negative slots are skipped tokens; the others must exist and be
    written by one token only."""
    slots = [int(x) for x in slot_mapping]
    n_slots = num_blocks * BLOCK
    count = Counter(x for x in slots if 0 <= x < n_slots)
    faults = []
    for i, x in enumerate(slots):
        if x >= n_slots:
            faults.append((i, SLOT_RANGE))
        elif x >= 0 and count[x] > 1:
            faults.append((i, SLOT_REPEATED))
    return _report(faults)


def check_copy_pairs(num_blocks, pairs):
    pairs = [(int(a), int(b)) for a, b in pairs]
    ok = [0 <= a < num_blocks and 0 <= b < num_blocks for a, b in pairs]
    dsts = Counter(b for (a, b), good in zip(pairs, ok) if good)
    srcs = {a for (a, b), good in zip(pairs, ok) if good}
    faults = []
    for i, ((a, b), good) in enumerate(zip(pairs, ok)):
        if not good:
            faults.append((i, PAIR_RANGE))
            continue
        if dsts[b] > 1:
            faults.append((i, DST_REPEATED))
        if b in srcs:
            faults.append((i, DST_IS_SRC))
    return _report(faults)


def check_swap_pairs(num_blocks, num_host_slots, pairs):
    pairs = [(int(a), int(b)) for a, b in pairs]
    ok = [0 <= a < num_blocks and 0 <= b < num_host_slots for a, b in pairs]
    blocks = Counter(a for (a, b), good in zip(pairs, ok) if good)
    slots = Counter(b for (a, b), good in zip(pairs, ok) if good)
    faults = []
    for i, ((a, b), good) in enumerate(zip(pairs, ok)):
        if not good:
            faults.append((i, PAIR_RANGE))
            continue
        if blocks[a] > 1:
            faults.append((i, DST_REPEATED))
        if slots[b] > 1:
            faults.append((i, HOST_SLOT_REPEATED))
    return _report(faults)
