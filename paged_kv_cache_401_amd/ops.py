"""Python binding of libpa.so (the C ABI in include/pa.h).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every computation runs in the library's HIP kernels.  There is no
fallback: if libpa.so is missing or a call fails, an exception is raised.

torch is imported before the library is loaded so that libpa.so binds to the
HIP runtime torch already holds (one runtime per process).
"""
from __future__ import annotations

import ctypes
import os

import torch

F32, BF16, FP8 = 0, 1, 2
ELEM_BYTES = {F32: 4, BF16: 2, FP8: 1}
BLOCK_SIZE = 16
TORCH_TO_PA = {torch.float32: F32, torch.bfloat16: BF16}

# PA_LIBPA: load another build of the library (the host-sanitizer build)
LIB_PATH = os.environ.get("PA_LIBPA") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")

# every symbol include/pa.h declares
EXPORTS = ("pa_pool_bytes", "pa_decode_partition_tokens", "pa_decode_workspace_size", "pa_decode",
           "pa_decode_ex", "pa_decode_noalloc", "pa_decode_append", "pa_decode_prefix_shared",
           "pa_decode_prefix_shared_workspace_size", "pa_decode_prefix_shared_plan",
           "pa_prefill", "pa_reshape_and_cache", "pa_swap_blocks", "pa_copy_blocks",
           "pa_check_workspace_size", "pa_check_tables", "pa_check_query_start", "pa_check_slots",
           "pa_check_copy_pairs", "pa_check_swap_pairs", "pa_set_debug",
           "pa_decode_variant", "pa_decode_plan", "pa_set_profile_events",
           "pa_probe_read", "pa_strerror", "pa_last_error", "pa_build_info")

# index fault kinds of the pa_check_* reports (PA_FAULT_* in pa.h)
FAULT_CONTEXT_LEN, FAULT_BLOCK_ID, FAULT_SLOT_RANGE, FAULT_SLOT_REPEATED = 1, 2, 4, 8
FAULT_PAIR_RANGE, FAULT_DST_REPEATED, FAULT_DST_IS_SRC = 16, 32, 64
FAULT_HOST_SLOT_REPEATED, FAULT_QUERY_START = 128, 256
ERR_INDEX = -9


class PAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("libpa error %d: %s" % (status, message))
        self.status = status


class PoolDesc(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("num_blocks", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("k_scale", ctypes.c_float),
                ("v_scale", ctypes.c_float)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libpa.so (built by ``__graft_entry__.build()``); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise PAError(-7, "%s is not built; run __graft_entry__.build()" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    P, I32, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    PD = ctypes.POINTER(PoolDesc)
    L.pa_pool_bytes.argtypes = [PD]
    L.pa_pool_bytes.restype = SZ
    L.pa_decode_partition_tokens.argtypes = [PD, I32, I32, I32, I32]
    L.pa_decode_partition_tokens.restype = I32
    L.pa_decode_workspace_size.argtypes = [PD, I32, I32, I32, I32]
    L.pa_decode_workspace_size.restype = SZ
    L.pa_decode.argtypes = [PD, P, I32, I32, I32, P, I32, P, F, P, I32, P, SZ, P]
    L.pa_decode.restype = ctypes.c_int
    L.pa_decode_ex.argtypes = [PD, P, I32, I32, I32, P, I32, P, F, P, I32, P, SZ, ctypes.c_uint32, P]
    L.pa_decode_ex.restype = ctypes.c_int
    L.pa_decode_noalloc.argtypes = [PD, P, I32, I32, I32, P, I32, P, F, P, I32, ctypes.c_uint32, P]
    L.pa_decode_noalloc.restype = ctypes.c_int
    L.pa_decode_prefix_shared.argtypes = [PD, P, I32, I32, I32, P, I32, P, P, P, I32, I32, F, P, I32, P,
                                          SZ, ctypes.c_uint32, P]
    L.pa_decode_prefix_shared.restype = ctypes.c_int
    L.pa_decode_prefix_shared_workspace_size.argtypes = [PD, I32, I32, I32, I32, I32, I32]
    L.pa_decode_prefix_shared_workspace_size.restype = SZ
    L.pa_decode_prefix_shared_plan.argtypes = [PD, I32, I32, I32, I32, I32, I32, P]
    L.pa_decode_prefix_shared_plan.restype = ctypes.c_int
    L.pa_decode_append.argtypes = [PD, P, I32, I32, I32, P, I32, P, F, P, I32, P, SZ, ctypes.c_uint32,
                                   P, P, I32, P]
    L.pa_decode_append.restype = ctypes.c_int
    L.pa_prefill.argtypes = [PD, P, I32, I32, I32, P, I32, P, I32, P, F, P, P]
    L.pa_prefill.restype = ctypes.c_int
    L.pa_reshape_and_cache.argtypes = [PD, P, P, I32, P, I32, P]
    L.pa_reshape_and_cache.restype = ctypes.c_int
    L.pa_swap_blocks.argtypes = [PD, P, P, I32, P, I32, I32, P]
    L.pa_swap_blocks.restype = ctypes.c_int
    L.pa_copy_blocks.argtypes = [PD, P, I32, P]
    L.pa_copy_blocks.restype = ctypes.c_int
    L.pa_check_workspace_size.argtypes = [PD, I32]
    L.pa_check_workspace_size.restype = SZ
    L.pa_check_tables.argtypes = [PD, I32, P, I32, P, P, P]
    L.pa_check_tables.restype = ctypes.c_int
    L.pa_check_query_start.argtypes = [I32, P, P, P]
    L.pa_check_query_start.restype = ctypes.c_int
    L.pa_check_slots.argtypes = [PD, P, I32, P, SZ, P, P]
    L.pa_check_slots.restype = ctypes.c_int
    L.pa_check_copy_pairs.argtypes = [PD, P, I32, P, SZ, P, P]
    L.pa_check_copy_pairs.restype = ctypes.c_int
    L.pa_check_swap_pairs.argtypes = [PD, I32, P, I32, P, SZ, P, P]
    L.pa_check_swap_pairs.restype = ctypes.c_int
    L.pa_set_debug.argtypes = [ctypes.c_int]
    L.pa_set_debug.restype = ctypes.c_int
    L.pa_decode_variant.argtypes = [PD, I32]
    L.pa_decode_variant.restype = ctypes.c_int
    L.pa_decode_plan.argtypes = [PD, I32, I32, I32, I32, P]
    L.pa_decode_plan.restype = ctypes.c_int
    L.pa_set_profile_events.argtypes = [P, P]
    L.pa_set_profile_events.restype = ctypes.c_int
    L.pa_probe_read.argtypes = [P, SZ, P, P]
    L.pa_probe_read.restype = ctypes.c_int
    L.pa_strerror.argtypes = [ctypes.c_int]
    L.pa_strerror.restype = ctypes.c_char_p
    L.pa_last_error.argtypes = []
    L.pa_last_error.restype = ctypes.c_char_p
    L.pa_build_info.argtypes = []
    L.pa_build_info.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(rc: int) -> None:
    if rc != 0:
        raise PAError(rc, lib().pa_last_error().decode())


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    return t.data_ptr()


class KVPool:
    """Device K and V pools: num_blocks x num_kv_heads tiles of 16 x head_dim
    elements of ``dtype`` each, held as raw byte tensors."""

    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int, dtype: int,
                 device="cuda", k_scale: float = 1.0, v_scale: float = 1.0, fill: int | None = None):
        self.num_blocks, self.num_kv_heads, self.head_dim, self.dtype = (
            int(num_blocks), int(num_kv_heads), int(head_dim), int(dtype))
        self.k_scale, self.v_scale = float(k_scale), float(v_scale)
        nbytes = self.num_blocks * self.num_kv_heads * BLOCK_SIZE * self.head_dim * ELEM_BYTES[dtype]
        alloc = torch.empty if fill is None else (lambda n, **kw: torch.full((n,), fill, **kw))
        self.k = alloc(nbytes, dtype=torch.uint8, device=device)
        self.v = alloc(nbytes, dtype=torch.uint8, device=device)
        got = lib().pa_pool_bytes(ctypes.byref(self.desc()))
        if got != nbytes:
            raise PAError(-3, "pool descriptor rejected: %s" % lib().pa_last_error().decode())

    def desc(self) -> PoolDesc:
        return PoolDesc(self.k.data_ptr(), self.v.data_ptr(), self.num_blocks, self.num_kv_heads,
                        BLOCK_SIZE, self.head_dim, self.dtype, self.k_scale, self.v_scale)

    @property
    def nbytes(self) -> int:
        return self.k.numel()


def reshape_and_cache(pool: KVPool, k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                      stream=None) -> None:
    n = slot_mapping.numel()
    if k.shape != (n, pool.num_kv_heads, pool.head_dim) or v.shape != k.shape:
        raise ValueError("k/v must be [num_tokens][num_kv_heads][head_dim]")
    if k.dtype != v.dtype or k.dtype not in TORCH_TO_PA:
        raise TypeError("k/v must both be float32 or bfloat16")
    d = pool.desc()
    _check(lib().pa_reshape_and_cache(ctypes.byref(d), _dev(k, "k"), _dev(v, "v"),
                                      TORCH_TO_PA[k.dtype], _dev(slot_mapping, "slot_mapping",
                                                                 torch.int32), n, _stream(stream)))


def copy_blocks(pool: KVPool, pairs: torch.Tensor, stream=None) -> None:
    n = pairs.numel() // 2
    ptr = _dev(pairs, "pairs", torch.int32) if n else None
    d = pool.desc()
    _check(lib().pa_copy_blocks(ctypes.byref(d), ptr, n, _stream(stream)))


SWAP_OUT, SWAP_IN = 0, 1


class HostPool:
    """Pinned host memory for swapped-out blocks: num_slots slots, each one
    whole block of the device pool (every KV head) for K and for V."""

    def __init__(self, pool: KVPool, num_slots: int):
        self.num_slots = int(num_slots)
        self.slot_bytes = pool.nbytes // pool.num_blocks
        n = max(1, self.num_slots) * self.slot_bytes
        self.k = torch.empty(n, dtype=torch.uint8, pin_memory=True)
        self.v = torch.empty(n, dtype=torch.uint8, pin_memory=True)


def swap_blocks(pool: KVPool, host: HostPool, pairs: torch.Tensor, direction: int,
                stream=None) -> None:
    """Move whole blocks: pairs is int32 [P][2] (device block, host slot) on the
    GPU; direction SWAP_OUT (device -> host) or SWAP_IN (host -> device)."""
    n = pairs.numel() // 2
    ptr = _dev(pairs, "pairs", torch.int32) if n else None
    if not host.k.is_pinned() or not host.v.is_pinned():
        raise ValueError("host pools must be pinned")
    d = pool.desc()
    _check(lib().pa_swap_blocks(ctypes.byref(d), host.k.data_ptr(), host.v.data_ptr(),
                                host.num_slots, ptr, n, int(direction), _stream(stream)))


def decode_partition_tokens(pool: KVPool, num_seqs, num_q_heads, max_blocks_per_seq,
                            partition_tokens=0) -> int:
    d = pool.desc()
    r = lib().pa_decode_partition_tokens(ctypes.byref(d), num_seqs, num_q_heads,
                                         max_blocks_per_seq, partition_tokens)
    if r < 0:
        raise PAError(r, lib().pa_last_error().decode())
    return r


def decode_workspace_size(pool: KVPool, num_seqs, num_q_heads, max_blocks_per_seq,
                          partition_tokens=0) -> int:
    decode_partition_tokens(pool, num_seqs, num_q_heads, max_blocks_per_seq, partition_tokens)
    d = pool.desc()
    return int(lib().pa_decode_workspace_size(ctypes.byref(d), num_seqs, num_q_heads,
                                              max_blocks_per_seq, partition_tokens))


DECODE_STREAM_KV, DECODE_SHARED_KV = 0, 1


def decode(pool: KVPool, q: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
           scale: float, out: torch.Tensor | None = None, partition_tokens: int = 0,
           workspace: torch.Tensor | None = None, stream=None,
           shared_kv: bool = False, k_new: torch.Tensor | None = None,
           v_new: torch.Tensor | None = None) -> torch.Tensor:
    """Paged decode attention; ``shared_kv`` marks batches whose sequences
    share blocks (cached rather than streaming K/V loads; same result).
    With ``k_new``/``v_new`` ([num_seqs][num_kv_heads][head_dim]) each
    sequence's newest token, at position context_len - 1, is written to the
    pool first, in the same step (pa_decode_append)."""
    S, Hq, D = q.shape
    if D != pool.head_dim:
        raise ValueError("q head dim %d differs from the pool's %d" % (D, pool.head_dim))
    if q.dtype not in TORCH_TO_PA:
        raise TypeError("q must be float32 or bfloat16")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables must be [num_seqs][max_blocks]; context_lens [num_seqs]")
    mbs = block_tables.shape[1]
    if out is None:
        out = torch.empty((S, Hq, D), dtype=torch.float32, device=q.device)
    elif tuple(out.shape) != (S, Hq, D):
        raise ValueError("out must be [num_seqs][num_q_heads][head_dim] = %s, got %s"
                         % ((S, Hq, D), tuple(out.shape)))
    need = decode_workspace_size(pool, S, Hq, mbs, partition_tokens)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wptr = workspace.data_ptr() if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    d = pool.desc()
    flags = DECODE_SHARED_KV if shared_kv else DECODE_STREAM_KV
    common = (ctypes.byref(d), _dev(q, "q"), TORCH_TO_PA[q.dtype], S, Hq,
              _dev(block_tables, "block_tables", torch.int32), mbs,
              _dev(context_lens, "context_lens", torch.int32), float(scale),
              _dev(out, "out", torch.float32), int(partition_tokens), wptr, wbytes, flags)
    if k_new is None and v_new is None:
        _check(lib().pa_decode_ex(*common, _stream(stream)))
        return out
    shape = (S, pool.num_kv_heads, pool.head_dim)
    if k_new is None or v_new is None or k_new.shape != shape or v_new.shape != shape:
        raise ValueError("k_new and v_new must both be [num_seqs][num_kv_heads][head_dim]")
    if k_new.dtype != v_new.dtype or k_new.dtype not in TORCH_TO_PA:
        raise TypeError("k_new/v_new must both be float32 or bfloat16")
    _check(lib().pa_decode_append(*common, _dev(k_new, "k_new"), _dev(v_new, "v_new"),
                                  TORCH_TO_PA[k_new.dtype], _stream(stream)))
    return out


def decode_prefix_shared_workspace_size(pool: KVPool, num_seqs, num_q_heads, max_blocks_per_seq,
                                        num_groups, max_group_size, partition_tokens=0) -> int:
    d = pool.desc()
    return int(lib().pa_decode_prefix_shared_workspace_size(
        ctypes.byref(d), int(num_seqs), int(num_q_heads), int(max_blocks_per_seq), int(num_groups),
        int(max_group_size), int(partition_tokens)))


def decode_prefix_shared(pool: KVPool, q: torch.Tensor, block_tables: torch.Tensor,
                         context_lens: torch.Tensor, group_start: torch.Tensor,
                         prefix_blocks: torch.Tensor, max_group_size: int, scale: float,
                         out: torch.Tensor | None = None, partition_tokens: int = 0,
                         workspace: torch.Tensor | None = None, stream=None,
                         shared_kv: bool = False) -> torch.Tensor:
    """pa_decode_prefix_shared: decode of a batch in groups of consecutive
    sequences that share their first ``prefix_blocks[i]`` table entries
    (``group_start`` int32 [G + 1] and ``prefix_blocks`` int32 [G] on the GPU,
    e.g. from ``blocks.prefix_groups``)."""
    S, Hq, D = q.shape
    if D != pool.head_dim:
        raise ValueError("q head dim %d differs from the pool's %d" % (D, pool.head_dim))
    if q.dtype != torch.bfloat16:
        raise TypeError("q must be bfloat16")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables must be [num_seqs][max_blocks]; context_lens [num_seqs]")
    G = prefix_blocks.numel()
    if group_start.numel() != G + 1:
        raise ValueError("group_start must hold num_groups + 1 offsets")
    mbs = block_tables.shape[1]
    if out is None:
        out = torch.empty((S, Hq, D), dtype=torch.float32, device=q.device)
    elif tuple(out.shape) != (S, Hq, D):
        raise ValueError("out must be [num_seqs][num_q_heads][head_dim] = %s, got %s"
                         % ((S, Hq, D), tuple(out.shape)))
    d = pool.desc()
    need = decode_prefix_shared_workspace_size(pool, S, Hq, mbs, G, max_group_size, partition_tokens)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wptr = workspace.data_ptr() if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    flags = DECODE_SHARED_KV if shared_kv else DECODE_STREAM_KV
    _check(lib().pa_decode_prefix_shared(
        ctypes.byref(d), _dev(q, "q"), BF16, S, Hq, _dev(block_tables, "block_tables", torch.int32), mbs,
        _dev(context_lens, "context_lens", torch.int32), _dev(group_start, "group_start", torch.int32),
        _dev(prefix_blocks, "prefix_blocks", torch.int32), G, int(max_group_size), float(scale),
        _dev(out, "out", torch.float32), int(partition_tokens), wptr, wbytes, flags, _stream(stream)))
    return out


def decode_noalloc(pool: KVPool, q: torch.Tensor, block_tables: torch.Tensor,
                   context_lens: torch.Tensor, scale: float, out: torch.Tensor,
                   partition_tokens: int = 0, stream=None, shared_kv: bool = False) -> torch.Tensor:
    """pa_decode_noalloc: decode whose split-K partials go to the library's
    static per-device scratch; ``out`` must be given ([num_seqs][num_q_heads]
    [head_dim] fp32), as the call allocates nothing."""
    S, Hq, D = q.shape
    if D != pool.head_dim:
        raise ValueError("q head dim %d differs from the pool's %d" % (D, pool.head_dim))
    if q.dtype not in TORCH_TO_PA:
        raise TypeError("q must be float32 or bfloat16")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables must be [num_seqs][max_blocks]; context_lens [num_seqs]")
    if tuple(out.shape) != (S, Hq, D):
        raise ValueError("out must be [num_seqs][num_q_heads][head_dim] = %s, got %s"
                         % ((S, Hq, D), tuple(out.shape)))
    d = pool.desc()
    flags = DECODE_SHARED_KV if shared_kv else DECODE_STREAM_KV
    _check(lib().pa_decode_noalloc(ctypes.byref(d), _dev(q, "q"), TORCH_TO_PA[q.dtype], S, Hq,
                                   _dev(block_tables, "block_tables", torch.int32),
                                   block_tables.shape[1],
                                   _dev(context_lens, "context_lens", torch.int32), float(scale),
                                   _dev(out, "out", torch.float32), int(partition_tokens), flags,
                                   _stream(stream)))
    return out


def prefill(pool: KVPool, q: torch.Tensor, query_start: torch.Tensor, max_query_len: int,
            block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
            out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Causal prefill of each sequence's chunk (its last query_start[s+1] -
    query_start[s] context tokens); q is bf16 [total][Hq][D]."""
    T, Hq, D = q.shape
    if D != pool.head_dim:
        raise ValueError("q head dim %d differs from the pool's %d" % (D, pool.head_dim))
    S = context_lens.numel()
    if query_start.numel() != S + 1:
        raise ValueError("query_start must hold num_seqs + 1 offsets")
    if block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must be [num_seqs][max_blocks]")
    if q.dtype != torch.bfloat16:
        raise TypeError("prefill q must be bfloat16")
    if out is None:
        out = torch.empty((T, Hq, D), dtype=torch.float32, device=q.device)
    elif tuple(out.shape) != (T, Hq, D):
        raise ValueError("out must be [total chunk tokens][num_q_heads][head_dim] = %s, got %s"
                         % ((T, Hq, D), tuple(out.shape)))
    d = pool.desc()
    _check(lib().pa_prefill(ctypes.byref(d), _dev(q, "q"), BF16, S, Hq,
                            _dev(query_start, "query_start", torch.int32), int(max_query_len),
                            _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
                            _dev(context_lens, "context_lens", torch.int32), float(scale),
                            _dev(out, "out", torch.float32), _stream(stream)))
    return out


class IndexChecker:
    """Runs the library's device-side index checks for one pool.  Each check
    returns (faults, kinds, first): the number of faults, the OR of their
    FAULT_* kinds and the smallest element index at fault (-1 if none).  It
    waits for the check's stream to read the report."""

    def __init__(self, pool: KVPool, num_host_slots: int = 0):
        self.pool = pool
        self.num_host_slots = int(num_host_slots)
        d = pool.desc()
        n = int(lib().pa_check_workspace_size(ctypes.byref(d), self.num_host_slots))
        if n == 0:
            raise PAError(-3, "pa_check_workspace_size rejected the pool")
        self.workspace = torch.empty(n, dtype=torch.uint8, device=pool.k.device)
        self.report = torch.empty(3, dtype=torch.int32, device=pool.k.device)

    def _result(self, rc, stream):
        _check(rc)
        if stream is not None and hasattr(stream, "synchronize"):
            stream.synchronize()
        elif stream is not None:
            torch.cuda.synchronize()
        return tuple(int(x) for x in self.report.cpu().tolist())

    def tables(self, block_tables: torch.Tensor, context_lens: torch.Tensor, stream=None):
        d = self.pool.desc()
        S = context_lens.numel()
        return self._result(lib().pa_check_tables(
            ctypes.byref(d), S, _dev(block_tables, "block_tables", torch.int32),
            block_tables.shape[1], _dev(context_lens, "context_lens", torch.int32),
            self.report.data_ptr(), _stream(stream)), stream)

    def query_start(self, query_start: torch.Tensor, stream=None):
        return self._result(lib().pa_check_query_start(
            query_start.numel() - 1, _dev(query_start, "query_start", torch.int32),
            self.report.data_ptr(), _stream(stream)), stream)

    def slots(self, slot_mapping: torch.Tensor, stream=None):
        d = self.pool.desc()
        n = slot_mapping.numel()
        ptr = _dev(slot_mapping, "slot_mapping", torch.int32) if n else None
        return self._result(lib().pa_check_slots(
            ctypes.byref(d), ptr, n, self.workspace.data_ptr(), self.workspace.numel(),
            self.report.data_ptr(), _stream(stream)), stream)

    def copy_pairs(self, pairs: torch.Tensor, stream=None):
        d = self.pool.desc()
        n = pairs.numel() // 2
        ptr = _dev(pairs, "pairs", torch.int32) if n else None
        return self._result(lib().pa_check_copy_pairs(
            ctypes.byref(d), ptr, n, self.workspace.data_ptr(), self.workspace.numel(),
            self.report.data_ptr(), _stream(stream)), stream)

    def swap_pairs(self, pairs: torch.Tensor, stream=None):
        d = self.pool.desc()
        n = pairs.numel() // 2
        ptr = _dev(pairs, "pairs", torch.int32) if n else None
        return self._result(lib().pa_check_swap_pairs(
            ctypes.byref(d), self.num_host_slots, ptr, n, self.workspace.data_ptr(),
            self.workspace.numel(), self.report.data_ptr(), _stream(stream)), stream)


def set_debug(on: bool) -> bool:
    """Debug mode: every operation first checks its index data and raises
    PAError(ERR_INDEX) instead of running when a check finds a fault.
    Returns the previous setting."""
    return bool(lib().pa_set_debug(1 if on else 0))


def decode_variant(pool: KVPool, num_q_heads: int) -> str:
    """Name of the partition kernel pa_decode launches for this pool."""
    d = pool.desc()
    r = lib().pa_decode_variant(ctypes.byref(d), num_q_heads)
    if r < 0:
        raise PAError(r, lib().pa_last_error().decode())
    return "decode_mfma_kernel" if r == 1 else "decode_valu_kernel"


DECODE_KERNELS = ("decode_valu_kernel", "decode_mfma_kernel", "decode_group_kernel")


def decode_plan(pool: KVPool, num_seqs, num_q_heads, max_blocks_per_seq, partition_tokens=0) -> dict:
    """The launch pa_decode_ex makes: its partition kernel, partition tokens,
    partial results per row and partitions merged into each."""
    plan = (ctypes.c_int32 * 4)()
    d = pool.desc()
    _check(lib().pa_decode_plan(ctypes.byref(d), int(num_seqs), int(num_q_heads),
                                int(max_blocks_per_seq), int(partition_tokens), plan))
    return {"kernel": DECODE_KERNELS[plan[0]], "partition_tokens": plan[1],
            "partials_per_row": plan[2], "partitions_per_partial": plan[3]}


def decode_prefix_shared_plan(pool: KVPool, num_seqs, num_q_heads, max_blocks_per_seq, num_groups,
                              max_group_size, partition_tokens=0) -> dict:
    """The launch pa_decode_prefix_shared makes: its partition tokens and the
    partitions at most per group and KV head."""
    plan = (ctypes.c_int32 * 2)()
    d = pool.desc()
    _check(lib().pa_decode_prefix_shared_plan(ctypes.byref(d), int(num_seqs), int(num_q_heads),
                                              int(max_blocks_per_seq), int(num_groups),
                                              int(max_group_size), int(partition_tokens), plan))
    return {"partition_tokens": plan[0], "max_partitions": plan[1]}


def set_profile_events(before, after) -> None:
    """Have the next decode's (or prefill's) partition kernel store its start
    and end times in ``before``/``after``: torch.cuda.Event objects or raw
    hipEvent_t handles (pass None, None to clear)."""
    raw = lambda e: None if e is None else (e.cuda_event if hasattr(e, "cuda_event") else int(e))
    _check(lib().pa_set_profile_events(raw(before), raw(after)))


def probe_read(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Enqueue one streaming read of ``buf`` (measurement aid)."""
    rc = lib().pa_probe_read(_dev(buf, "buf"), buf.numel() * buf.element_size(),
                             _dev(sink, "sink"), _stream(stream))
    if rc != 0:
        raise PAError(rc, lib().pa_strerror(rc).decode())


def build_info() -> str:
    return lib().pa_build_info().decode()
