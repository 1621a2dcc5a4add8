"""fp64 CPU oracle for paged decode attention, paged (chunked) prefill
attention, the paged cache write and the copy-on-write block copy.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the GPU library (``paged_kv_cache_401_amd``) and never imports it.

The arithmetic lives in ``pa_oracle.c`` (plain C, fp64, built with
``-O2 -ffp-contract=off`` and OpenMP over independent output rows).  This
module only marshals numpy arrays.  ``dense_attention`` is a numpy/scipy
restatement used to pin the C code against a library softmax.

Every function cites the page section it follows in ``pa_oracle.c``.
``index_checks.py`` states, as plain loops, the index preconditions the
library's device-side checks enforce.
Parity status: every entry point here is pinned by CPU tests
(``tests/test_oracle_pins.py``, ``tests/test_oracle_prefill_pins.py``,
``tests/test_index_checks_host.py``); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

F32, BF16, FP8 = 0, 1, 2
ELEM_BYTES = {F32: 4, BF16: 2, FP8: 1}
BLOCK = 16

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_BUILT = os.path.join(_HERE, "liboracle.so")
# PA_ORACLE_LIB: load another build of the same source (the sanitizer build)
_LIB = os.environ.get("PA_ORACLE_LIB") or _BUILT
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_BUILT):
        tmp = _BUILT + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
             "-fPIC", "-shared", "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _BUILT)
    return _BUILT


def build_sanitized(out: str) -> str:
    """The same source built with AddressSanitizer and UndefinedBehaviorSanitizer
    (gcc; any finding aborts), for host-side checks of the oracle.  Load it by
    setting PA_ORACLE_LIB, with gcc's libasan and libubsan preloaded."""
    subprocess.check_call(
        ["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
         "-shared", "-std=c11", "-o", out, _SRC, "-lm"])
    return out


def bind(L: ctypes.CDLL) -> ctypes.CDLL:
    """Declare the argument types of the oracle's C entry points on ``L``."""
    P, I, I64, F, D = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                       ctypes.c_float, ctypes.c_double)
    L.orc_fp8_decode.argtypes = [ctypes.c_uint8]
    L.orc_fp8_decode.restype = D
    L.orc_fp8_encode.argtypes = [F]
    L.orc_fp8_encode.restype = ctypes.c_uint8
    L.orc_fp8_encode_array.argtypes = [P, P, I64]
    L.orc_fp8_encode_array.restype = None
    L.orc_reshape_and_cache.argtypes = [P, P, I, I64, I, I, P, P, I, P, I64, F, F]
    L.orc_reshape_and_cache.restype = None
    L.orc_copy_blocks.argtypes = [P, P, I, I, I, P, I64]
    L.orc_copy_blocks.restype = None
    L.orc_swap_blocks.argtypes = [P, P, P, P, I, I, I, I64, I64, P, I64, I]
    L.orc_swap_blocks.restype = None
    L.orc_gather.argtypes = [P, I, I, I, I, P, I64, I, P]
    L.orc_gather.restype = None
    L.orc_paged_attention.argtypes = [P, P, I, F, F, I, I, P, I, I, I, P, I, P, F,
                                      P, P, I64, I]
    L.orc_paged_attention.restype = I
    L.orc_prefill_attention.argtypes = [P, P, I, F, F, I, I, P, I, I, I, P, P, I, P, F,
                                        P, P, I64, I]
    L.orc_prefill_attention.restype = I
    L.orc_max_threads.argtypes = []
    L.orc_max_threads.restype = I
    return L


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = bind(ctypes.CDLL(_LIB))
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _bytes(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    return a.reshape(-1).view(np.uint8)


def max_threads() -> int:
    return int(lib().orc_max_threads())


# ------------------------------------------------------------------ fp8 codec
def fp8_decode(codes) -> np.ndarray:
    """Value of each OCP E4M3FN code (fp64), from the format definition."""
    codes = np.asarray(codes, dtype=np.uint8).reshape(-1)
    f = lib().orc_fp8_decode
    return np.array([f(int(c)) for c in codes], dtype=np.float64)


def fp8_encode(x) -> np.ndarray:
    """Nearest E4M3FN code to each fp32 value, ties to even, saturating at 448."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    out = np.empty(x.shape, dtype=np.uint8)
    lib().orc_fp8_encode_array(_ptr(x), _ptr(out), x.size)
    return out


# ----------------------------------------------------------------- the pool
def tile_elems(D: int) -> int:
    return BLOCK * D


def new_pool(num_blocks: int, Hkv: int, D: int, dtype: int, fill: int = 0) -> np.ndarray:
    """A byte array holding one K or V pool: num_blocks x Hkv tiles of 16 x D."""
    n = num_blocks * Hkv * BLOCK * D * ELEM_BYTES[dtype]
    return np.full(n, fill, dtype=np.uint8)


def reshape_and_cache(k_pool, v_pool, pool_dt, num_blocks, Hkv, D, k, v, in_dt,
                      slot_mapping, k_scale=1.0, v_scale=1.0):
    """Scatter k/v [N][Hkv][D] (raw elements of ``in_dt``) into the pools."""
    kb, vb = _bytes(k), _bytes(v)
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int32)
    n = slots.size
    assert kb.size == n * Hkv * D * ELEM_BYTES[in_dt] == vb.size
    lib().orc_reshape_and_cache(_ptr(k_pool), _ptr(v_pool), pool_dt, num_blocks, Hkv, D,
                                _ptr(kb), _ptr(vb), in_dt, _ptr(slots), n,
                                float(k_scale), float(v_scale))


def copy_blocks(k_pool, v_pool, pool_dt, Hkv, D, pairs):
    pairs = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
    lib().orc_copy_blocks(_ptr(k_pool), _ptr(v_pool), pool_dt, Hkv, D, _ptr(pairs),
                          pairs.shape[0])


def swap_blocks(k_pool, v_pool, host_k, host_v, pool_dt, Hkv, D, num_blocks, num_slots, pairs,
                direction):
    """Copy whole blocks between the pools and host slots: direction 0 =
    device block -> host slot, 1 = host slot -> device block; pairs are
    (device block, host slot)."""
    pairs = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
    lib().orc_swap_blocks(_ptr(k_pool), _ptr(v_pool), _ptr(host_k), _ptr(host_v), pool_dt, Hkv,
                          D, num_blocks, num_slots, _ptr(pairs), pairs.shape[0], int(direction))


def gather(pool, is_v, pool_dt, Hkv, D, table, n, g) -> np.ndarray:
    """Raw elements of the first n tokens of KV head g read through `table`,
    as a byte array of shape [n][D * elem_bytes]."""
    table = np.ascontiguousarray(table, dtype=np.int32)
    out = np.zeros((n, D * ELEM_BYTES[pool_dt]), dtype=np.uint8)
    lib().orc_gather(_ptr(pool), int(bool(is_v)), pool_dt, Hkv, D, _ptr(table), n, g,
                     _ptr(out))
    return out


def paged_attention(k_pool, v_pool, pool_dt, Hkv, D, q, q_dt, S, Hq, block_tables,
                    context_lens, scale, k_scale=1.0, v_scale=1.0, rows=None,
                    threads=0) -> np.ndarray:
    """fp64 decode attention.  Returns [S][Hq][D], or [len(rows)][D] when
    ``rows`` lists (s, h) pairs."""
    qb = _bytes(q)
    tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    MBS = tables.shape[1] if tables.ndim == 2 else tables.size // max(S, 1)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    if rows is not None:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 2))
        out = np.zeros((rows.shape[0], D), dtype=np.float64)
        nrows = rows.shape[0]
    else:
        out = np.zeros((S, Hq, D), dtype=np.float64)
        nrows = 0
    rc = lib().orc_paged_attention(_ptr(k_pool), _ptr(v_pool), pool_dt, float(k_scale),
                                   float(v_scale), Hkv, D, _ptr(qb), q_dt, S, Hq,
                                   _ptr(tables), MBS, _ptr(ctx), float(scale), _ptr(out),
                                   _ptr(rows), nrows, int(threads))
    if rc != 0:
        raise ValueError("oracle rejected the arguments (rc=%d)" % rc)
    return out


def prefill_attention(k_pool, v_pool, pool_dt, Hkv, D, q, q_dt, S, Hq, query_start, block_tables,
                      context_lens, scale, k_scale=1.0, v_scale=1.0, rows=None,
                      threads=0) -> np.ndarray:
    """fp64 causal attention of each sequence's chunk of new tokens (the last
    ``query_start[s+1] - query_start[s]`` tokens of its context) over its
    paged context.  q is [total][Hq][D]; returns [total][Hq][D], or
    [len(rows)][D] when ``rows`` lists (chunk token, head) pairs."""
    qb = _bytes(q)
    qs = np.ascontiguousarray(query_start, dtype=np.int32)
    assert qs.size == S + 1
    tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    MBS = tables.shape[1] if tables.ndim == 2 else tables.size // max(S, 1)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    if rows is not None:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 2))
        out = np.zeros((rows.shape[0], D), dtype=np.float64)
        nrows = rows.shape[0]
    else:
        out = np.zeros((int(qs[-1]), Hq, D), dtype=np.float64)
        nrows = 0
    rc = lib().orc_prefill_attention(_ptr(k_pool), _ptr(v_pool), pool_dt, float(k_scale),
                                     float(v_scale), Hkv, D, _ptr(qb), q_dt, S, Hq, _ptr(qs),
                                     _ptr(tables), MBS, _ptr(ctx), float(scale), _ptr(out),
                                     _ptr(rows), nrows, int(threads))
    if rc != 0:
        raise ValueError("oracle rejected the arguments (rc=%d)" % rc)
    return out


# ------------------------------------------------------- library restatement
def dense_attention(q, K, V, scale) -> np.ndarray:
    """softmax(scale * q K^T) V for contiguous K/V, via scipy's softmax and
    numpy matmul in fp64 (a library routine, used to pin the C oracle)."""
    from scipy.special import softmax
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    w = softmax(np.float64(scale) * (K @ q), axis=-1)
    return w @ V


def dense_causal_attention(Q, K, V, scale, first_pos) -> np.ndarray:
    """Rows of Q [n][D] at positions first_pos .. first_pos + n - 1 over K/V
    [ctx][D]: scipy softmax of scale * Q K^T with every key after a row's
    position masked to -inf, then times V (fp64 library restatement)."""
    from scipy.special import softmax
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    s = np.float64(scale) * (Q @ K.T)
    pos = first_pos + np.arange(Q.shape[0])[:, None]
    s = np.where(np.arange(K.shape[0])[None, :] <= pos, s, -np.inf)
    return softmax(s, axis=-1) @ V
