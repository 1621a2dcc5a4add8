/*
 * pa.h -- C ABI of the MI355X (gfx950) paged KV cache library (libpa.so).
 *
 * Operations on a pool of fixed-size KV blocks, as the source pages state
 * the problem:
 *   - pa_reshape_and_cache: write new tokens' K/V into their slots
 *     ("PagedAttention" glossary page (Ultralytics), how paging works, and the
 *     French page's second article, "what is the KV cache": only the new
 *     token's K and V are computed and appended to the cache; token `pos` of
 *     a request lives at slot `pos % 16` of block `table[pos / 16]`).
 *   - pa_copy_blocks: copy whole blocks before a sequence writes into a block
 *     others still use (glossary page, sharing blocks between sequences:
 *     copy-on-write; Russian page, "two answers to one request": only the
 *     block that has to split is copied).
 *   - pa_decode: single-query attention of every sequence over its context,
 *     read block by block through its block table in logical order (glossary
 *     page, how paging works; Russian page, logical order vs physical
 *     placement), with query heads grouped over shared KV heads (glossary
 *     page, related techniques: grouped-query attention).  The pages print no
 *     formula; the operation is softmax(scale * q K^T) V over the ctx tokens.
 *   - pa_prefill: the same attention for a chunk of new tokens per sequence,
 *     each attending causally to itself and every earlier token (glossary
 *     page, related techniques: FlashAttention-style kernels that read paged
 *     blocks).
 *   - pa_swap_blocks: move whole blocks between the device pool and pinned
 *     host memory (French page: fine-grained eviction of small pages to the
 *     CPU instead of whole sequences).
 *
 * Conventions for every entry point
 *   - Pointers are device pointers unless stated; the caller owns every
 *     buffer and keeps it alive until the enqueued work completes.  The
 *     library allocates no device memory (debug mode aside, see pa_set_debug)
 *     and keeps no pointer after return.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *     work on it and never synchronise the host.
 *   - Return value: PA_OK (0) or a negative pa_status.  On error nothing is
 *     enqueued and pa_last_error() describes the cause (thread-local).
 *     Host-visible scalars and pointer alignment are checked; index data in
 *     device memory (tables, slots, pairs, lengths) is not read by the host.
 *     Kernels skip block ids outside [0, num_blocks) and clamp context lengths
 *     to [0, max_blocks_per_seq * 16] instead of faulting.
 *
 * Pool layout (pa_pool_t.k_pool / v_pool, each num_blocks * num_kv_heads
 * tiles of 16 * head_dim elements of kv_dtype).  Tile (b, g) -- block b,
 * KV head g -- starts at element (b * num_kv_heads + g) * 16 * head_dim.
 *   K tile: element (t, d) at ((d / X) * 16 + t) * X + d % X, X = 16 / elem_bytes
 *           (each token's head vector in 16-byte runs, token-major per run).
 *   V tile: element (t, d) at ((t / 4) * (D / W) + d / W) * 4W + (d % W) * 4 + t % 4,
 *           W = 4 / elem_bytes (16-byte cells of 4 tokens x W dims, tokens fastest).
 * Both orders make each 16-lane quarter of a wavefront load 256 contiguous
 * bytes straight into matrix-core operand registers.
 *
 * This is NOT the plain row-major tile [16 slots][head_dim] (each token's head
 * vector contiguous) of the glossary page's schematic pool [block][slot][dim]:
 * the pages fix which block and slot a token occupies, not the byte order
 * inside a block, and the order above lets the decode kernel take K and V
 * from memory into matrix-core operands with no transpose (the plain order
 * would need a transpose through LDS or registers per block).  Tiles written
 * by pa_reshape_and_cache, pa_decode_append, pa_copy_blocks and
 * pa_swap_blocks are always in this order; a caller that fills pool memory
 * itself in the row-major order gets wrong results and must write through
 * pa_reshape_and_cache instead.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_BLOCK_SIZE 16

typedef enum pa_dtype {
    PA_F32 = 0,      /* IEEE binary32 */
    PA_BF16 = 1,     /* bfloat16 */
    PA_FP8_E4M3 = 2  /* OCP FP8 E4M3FN: bias 7, max 448, no infinities, NaN = S.1111.111 */
} pa_dtype;

typedef enum pa_status {
    PA_OK = 0,
    PA_ERR_NULL = -1,        /* a required pointer is NULL */
    PA_ERR_DTYPE = -2,       /* unknown dtype or unsupported dtype pairing */
    PA_ERR_SHAPE = -3,       /* negative/zero size, Hq % Hkv != 0, bad partition size */
    PA_ERR_UNSUPPORTED = -4, /* block_size != 16 or head_dim not 64 / 128 */
    PA_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required */
    PA_ERR_ALIGN = -6,       /* a pointer is not 16-byte aligned */
    PA_ERR_HIP = -7,         /* the HIP runtime reported an error */
    PA_ERR_RANGE = -8,       /* a scale is not finite and positive */
    PA_ERR_INDEX = -9        /* debug mode only: the index data in device memory breaks
                                the entry point's preconditions (see pa_set_debug) */
} pa_status;

/* The shared KV block pool.  k_scale / v_scale: per-pool dequantisation
 * scales of an FP8 pool (stored code * scale = value); ignored (use 1) for
 * 16/32-bit pools. */
typedef struct pa_pool {
    void *k_pool;
    void *v_pool;
    int32_t num_blocks;   /* 1 .. 2^27 - 1, so that every slot (block * 16 + position) is an int32 */
    int32_t num_kv_heads;
    int32_t block_size; /* must be 16 */
    int32_t head_dim;   /* 64 or 128 */
    int32_t kv_dtype;   /* pa_dtype */
    float k_scale;
    float v_scale;
} pa_pool_t;

/* Bytes of ONE pool (K or V): num_blocks * num_kv_heads * 16 * head_dim * elem. */
size_t pa_pool_bytes(const pa_pool_t *pool);

/* Partition size (tokens, multiple of 16) that pa_decode uses for these
 * arguments; `partition_tokens` = 0 asks for the library's choice.  Returns a
 * negative pa_status on invalid arguments. */
int32_t pa_decode_partition_tokens(const pa_pool_t *pool, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t max_blocks_per_seq,
                                   int32_t partition_tokens);

/* Workspace bytes pa_decode needs for these arguments (0 when every context
 * fits one partition).  Holds fp32 partial results of the split-K passes.
 * The context bound is given as max_blocks_per_seq, the capacity of one
 * block-table row (pa_decode's argument of the same name), rather than as a
 * longest context length: pa_decode sizes its grid from the table's
 * capacity, max_blocks_per_seq * 16 tokens, so that is the bound the
 * workspace must cover.  A caller that knows only its longest context n
 * passes ceil(n / 16) and must then call pa_decode with block tables of that
 * many columns. */
size_t pa_decode_workspace_size(const pa_pool_t *pool, int32_t num_seqs, int32_t num_q_heads,
                                int32_t max_blocks_per_seq, int32_t partition_tokens);

/*
 * pa_decode -- paged single-query decode attention.
 *   q              [num_seqs][num_q_heads][head_dim], q_dtype: PA_F32 with an
 *                  fp32 pool, PA_BF16 with a bf16 or fp8 pool.
 *   block_tables   int32 [num_seqs][max_blocks_per_seq]: physical block of each
 *                  logical block; entries past ceil(ctx / 16) are never read.
 *   context_lens   int32 [num_seqs]: tokens attended (0 gives a zero row).
 *   scale          softmax scale applied to q . k.
 *   out            fp32 [num_seqs][num_q_heads][head_dim] (16-byte aligned;
 *                  q too).
 *   partition_tokens  split-K partition length in tokens (multiple of 16),
 *                  0 = library's choice.  Contexts longer than one partition
 *                  are processed as independent partitions merged by a
 *                  second kernel; the result does not depend on the split
 *                  beyond fp32 rounding.
 *   workspace      device buffer of >= pa_decode_workspace_size(...) bytes
 *                  (may be NULL when that size is 0).
 * Query head h attends with KV head h / (num_q_heads / num_kv_heads).
 * Precision: scores, softmax and accumulation in fp32.  The probabilities
 * enter the P.V product in fp32 (fp32 pools) or to 16 significant bits as
 * bf16 hi + lo pairs, except with an fp8 pool and several query heads per KV
 * head, where they are rounded to fp16 (relative error <= 2^-11; the row sum
 * adds the same rounded values) against V widened exactly to fp16.
 */
int pa_decode(const pa_pool_t *pool, const void *q, int32_t q_dtype, int32_t num_seqs,
              int32_t num_q_heads, const int32_t *block_tables, int32_t max_blocks_per_seq,
              const int32_t *context_lens, float scale, float *out, int32_t partition_tokens,
              void *workspace, size_t workspace_bytes, void *stream);

/* Flags of pa_decode_ex: how the kernels load K/V. */
#define PA_DECODE_STREAM_KV 0u /* every block is read once per call: non-temporal loads (default) */
#define PA_DECODE_SHARED_KV 1u /* blocks are shared by several sequences of the batch (shared
                                  prompts, parallel sampling, beams): ordinary cached loads, so
                                  sequences read later find them in cache */

/* pa_decode with flags (PA_DECODE_* above); pa_decode is pa_decode_ex with
 * PA_DECODE_STREAM_KV.  The flags change only the cache policy of the K/V
 * loads, never the result.  Unknown flags give PA_ERR_SHAPE. */
int pa_decode_ex(const pa_pool_t *pool, const void *q, int32_t q_dtype, int32_t num_seqs,
                 int32_t num_q_heads, const int32_t *block_tables, int32_t max_blocks_per_seq,
                 const int32_t *context_lens, float scale, float *out, int32_t partition_tokens,
                 void *workspace, size_t workspace_bytes, uint32_t flags, void *stream);

/* Largest split-K scratch, in bytes, that pa_decode_noalloc keeps per device. */
#define PA_DECODE_NOALLOC_MAX_SCRATCH ((size_t)64 << 20)

/*
 * pa_decode_noalloc -- pa_decode_ex for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, and harnesses
 * that forbid hipMalloc.  Same arguments, flags, result and errors as
 * pa_decode_ex, without the workspace: the split-K partial results go to a
 * static array of PA_DECODE_NOALLOC_MAX_SCRATCH bytes in device memory, one
 * per device, which the library takes on its first call on that device and
 * holds until the process ends.  Calls needing more than that
 * (pa_decode_workspace_size of the same arguments) return PA_ERR_WORKSPACE
 * and enqueue nothing.  The call allocates nothing: no hipMalloc or hipFree,
 * and debug mode's index checks, which allocate, are not run by it.  Every
 * call on one device shares that device's array (nothing in it needs to
 * start cleared): calls that overlap on one device -- on different streams,
 * or from different host threads -- race and give undefined results.
 */
int pa_decode_noalloc(const pa_pool_t *pool, const void *q, int32_t q_dtype, int32_t num_seqs,
                      int32_t num_q_heads, const int32_t *block_tables, int32_t max_blocks_per_seq,
                      const int32_t *context_lens, float scale, float *out, int32_t partition_tokens,
                      uint32_t flags, void *stream);

/*
 * pa_decode_prefix_shared -- pa_decode_ex for a batch whose sequences come in
 * groups that hold the same first blocks in their block tables: the samples
 * of one prompt (parallel sampling), the beams of one request, requests over
 * one cached system prompt ("PagedAttention" glossary page, sharing blocks
 * between sequences: several tables name the same physical blocks of a
 * shared prefix).  The result is that of pa_decode_ex for every sequence, up
 * to fp32 rounding order; the shared blocks are read once per group and KV
 * head instead of once per sequence, every query head of every member of a
 * group being a column of one 16-column matrix-core tile.
 *   group_start    int32 [num_groups + 1] (device): group i is sequences
 *                  group_start[i] .. group_start[i+1] - 1; group_start[0] = 0,
 *                  non-decreasing, group_start[num_groups] = num_seqs.  A
 *                  sequence that shares nothing is a group of its own.
 *   prefix_blocks  int32 [num_groups] (device): leading table entries every
 *                  member of group i holds in common.  Only whole blocks
 *                  inside every member's context count (the kernel takes at
 *                  most min over members of floor(context_len / 16)).
 *   max_group_size host-side bound on the members of any group (larger
 *                  groups are cut to it); max_group_size * (num_q_heads /
 *                  num_kv_heads) must be at most 16 (PA_ERR_SHAPE).
 *   partition_tokens  0 = library's choice, else a multiple of 16 up to
 *                  8192: a group's blocks (shared ones, then each member's
 *                  own) are cut into partitions of this many tokens.
 *   workspace      device buffer of >= pa_decode_prefix_shared_workspace_size
 *                  bytes (may be NULL when that is 0).
 * Pools: PA_BF16 or PA_FP8_E4M3 (PA_ERR_UNSUPPORTED for fp32); q_dtype
 * PA_BF16.  Other arguments, flags and errors as pa_decode_ex.  The group
 * arrays are device data the host does not read: members beyond the batch
 * or max_group_size are left out.
 */
int pa_decode_prefix_shared(const pa_pool_t *pool, const void *q, int32_t q_dtype, int32_t num_seqs,
                            int32_t num_q_heads, const int32_t *block_tables, int32_t max_blocks_per_seq,
                            const int32_t *context_lens, const int32_t *group_start,
                            const int32_t *prefix_blocks, int32_t num_groups, int32_t max_group_size,
                            float scale, float *out, int32_t partition_tokens, void *workspace,
                            size_t workspace_bytes, uint32_t flags, void *stream);

/* Workspace bytes pa_decode_prefix_shared needs for these arguments (0 when
 * every group's blocks fit one partition; 0 also on invalid arguments). */
size_t pa_decode_prefix_shared_workspace_size(const pa_pool_t *pool, int32_t num_seqs,
                                              int32_t num_q_heads, int32_t max_blocks_per_seq,
                                              int32_t num_groups, int32_t max_group_size,
                                              int32_t partition_tokens);

/* The launch pa_decode_prefix_shared makes for these arguments (for tooling
 * and profiles): plan[0] = partition tokens (the library's choice when
 * partition_tokens is 0), plan[1] = partitions at most per group and KV head
 * (1: outputs written at once, no merge kernel).  Returns a pa_status. */
int pa_decode_prefix_shared_plan(const pa_pool_t *pool, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t max_blocks_per_seq, int32_t num_groups, int32_t max_group_size,
                                 int32_t partition_tokens, int32_t plan[2]);

/*
 * pa_decode_append -- one decode step: write every sequence's newest token,
 * then attend as pa_decode_ex.  The newest token of sequence s sits at
 * position context_lens[s] - 1 (its context includes it, as the step
 * appends the token's K and V before attending: French page, second
 * article, "what is the KV cache"); its slot follows from the block table
 * (slot = block_tables[s][p / 16] * 16 + p % 16).  The result, pool bytes
 * included, equals pa_reshape_and_cache of these tokens followed by
 * pa_decode_ex.  The write is done by the attention kernel itself (one
 * launch, no gap between a write kernel and the decode kernel) when one
 * workgroup alone reads each sequence's last block per KV head -- the
 * matrix-core kernel, or one query head per KV head -- and by a small
 * kernel of its own just before otherwise.
 *   k_new, v_new   [num_seqs][num_kv_heads][head_dim] of kv_dtype: the pool's
 *                  dtype for 16/32-bit pools, PA_BF16 or PA_F32 for an FP8 pool
 *                  (encoded as pa_reshape_and_cache does).  Sequences with
 *                  context length 0, a context longer than its table row
 *                  (max_blocks_per_seq * 16; attended as that many tokens),
 *                  or whose last table entry is outside the pool, write
 *                  nothing.
 * Other arguments, flags and errors as pa_decode_ex.
 */
int pa_decode_append(const pa_pool_t *pool, const void *q, int32_t q_dtype, int32_t num_seqs,
                     int32_t num_q_heads, const int32_t *block_tables, int32_t max_blocks_per_seq,
                     const int32_t *context_lens, float scale, float *out, int32_t partition_tokens,
                     void *workspace, size_t workspace_bytes, uint32_t flags, const void *k_new,
                     const void *v_new, int32_t kv_dtype, void *stream);

/*
 * pa_prefill -- causal (chunked) prefill attention over the paged pool.
 * Each sequence's chunk of new tokens is the last
 * n_s = query_start[s+1] - query_start[s] tokens of its context; their K/V
 * must already be in the pool (pa_reshape_and_cache), as the pages describe
 * the prompt's K/V being stored before generation continues (French page,
 * second article, "what is the KV cache"; Russian page: memory for the input
 * is allocated first).  Chunk token i of sequence s sits at position
 * p = context_lens[s] - n_s + i and attends to tokens 0..p of its context,
 * read through its block table -- the FlashAttention-style kernel reading
 * paged blocks of the glossary page's related techniques.  Row (token, h)
 * equals what pa_decode computes for that token's query over a context of
 * p + 1 tokens.
 *   q              bf16 [query_start[num_seqs]][num_q_heads][head_dim]
 *                  (16-byte aligned).
 *   query_start    int32 [num_seqs + 1], non-decreasing, query_start[0] = 0.
 *   max_query_len  host-side upper bound of every n_s (sizes the grid);
 *                  chunk tokens beyond it are not computed (their rows of out
 *                  are left as they were), and those below it keep their
 *                  positions context_len - n_s + i.  0 is a no-op.
 *   block_tables, max_blocks_per_seq, context_lens, scale: as for pa_decode.
 *   out            fp32 [query_start[num_seqs]][num_q_heads][head_dim]
 *                  (16-byte aligned).  A row whose position is negative (a
 *                  chunk longer than its context) is written as zeros.
 * Pools: PA_BF16 or PA_FP8_E4M3 (PA_ERR_UNSUPPORTED for fp32); q_dtype must
 * be PA_BF16.  Cache entries inside each context must be finite.
 * Precision: scores and the softmax in fp32; the probabilities enter the P.V
 * product rounded to fp16 (relative error <= 2^-11; the row sum adds the
 * same rounded values), against V widened to fp16 -- exact for E4M3 codes and
 * for bf16 magnitudes in [2^-14, 2^16) (within 2^-25 below), so a bf16 pool's
 * V entries inside each context must also be below 2^16 in magnitude (larger
 * ones become infinite); accumulation in fp32.
 */
int pa_prefill(const pa_pool_t *pool, const void *q, int32_t q_dtype, int32_t num_seqs,
               int32_t num_q_heads, const int32_t *query_start, int32_t max_query_len,
               const int32_t *block_tables, int32_t max_blocks_per_seq,
               const int32_t *context_lens, float scale, float *out, void *stream);

/*
 * pa_reshape_and_cache -- write num_tokens new tokens into the pool.
 *   k, v           [num_tokens][num_kv_heads][head_dim] of kv_dtype: the pool's
 *                  dtype for 16/32-bit pools; PA_BF16 or PA_F32 for an FP8 pool.
 *                  16-byte aligned.
 *   slot_mapping   int32 [num_tokens]: slot = block * 16 + position in block;
 *                  a negative slot skips the token.
 * FP8 pools store the E4M3FN code nearest to fp32(x) * fp32(1 / scale)
 * (round to nearest even, saturating to +-448); other pools store the input
 * bits unchanged.  Slots must be distinct within one call.
 */
int pa_reshape_and_cache(const pa_pool_t *pool, const void *k, const void *v, int32_t kv_dtype,
                         const int32_t *slot_mapping, int32_t num_tokens, void *stream);

/*
 * pa_copy_blocks -- copy-on-write block copy.
 *   src_dst_pairs  int32 [num_pairs][2]: copy every KV head's K and V tile of
 *                  block src over block dst.  Destinations must be distinct
 *                  and none may also be a source.  num_pairs = 0 is a no-op.
 */
int pa_copy_blocks(const pa_pool_t *pool, const int32_t *src_dst_pairs, int32_t num_pairs,
                   void *stream);

/* Directions of pa_swap_blocks. */
#define PA_SWAP_OUT 0 /* device pool -> host pool */
#define PA_SWAP_IN 1  /* host pool -> device pool */

/*
 * pa_swap_blocks -- move whole blocks between the device pool and a host
 * pool: the fine-grained eviction of the French page ("how PagedAttention
 * solves this problem": when memory is full, small pages move to the CPU
 * instead of whole sequences).
 *   host_k, host_v  the host pool: num_host_slots slots, each holding one
 *                   whole block's K (resp. V) bytes for every KV head in the
 *                   device pool's tile order (num_kv_heads * 16 * head_dim
 *                   elements of kv_dtype).  Must be pinned host memory
 *                   (hipHostMalloc, or a pinned torch tensor) that the
 *                   device can map; PA_ERR_HIP otherwise.  16-byte aligned.
 *                   Owned by the caller.
 *   block_slot_pairs  int32 [num_pairs][2] in device memory: (device block,
 *                   host slot).  PA_SWAP_OUT copies each block's bytes into
 *                   its slot; PA_SWAP_IN copies each slot's bytes into its
 *                   block.  Blocks must be distinct, slots must be distinct.
 *                   Pairs with an id out of range are skipped.
 * The copy is asynchronous on `stream`: host memory may be read only after
 * the stream reaches this point (swap-out), and a swapped-in block may be
 * attended by work enqueued after it.  num_pairs = 0 is a no-op.
 */
int pa_swap_blocks(const pa_pool_t *pool, void *host_k, void *host_v, int32_t num_host_slots,
                   const int32_t *block_slot_pairs, int32_t num_pairs, int32_t direction,
                   void *stream);

/*
 * Index checks.  The entry points above read their index data (context
 * lengths, block tables, chunk offsets, slots, block pairs) from device
 * memory and trust it: they skip out-of-range ids and clamp lengths instead
 * of faulting, and leave repeated slots or destinations as a race.  These
 * calls check that data on the device against each entry point's stated
 * preconditions.  Each enqueues its kernels on `stream` and fills `report`,
 * device int32[3]:
 *   report[0]  number of faults: one per (element, kind) at fault, where an
 *              element is a sequence, a chunk offset, a token or a pair;
 *   report[1]  OR of the PA_FAULT_* kinds found;
 *   report[2]  smallest index of an element at fault, -1 if none.
 * A repeated slot or block is a fault of every element that names it.  The
 * report does not depend on thread timing.  `workspace` (device memory of
 * pa_check_workspace_size bytes, 4-byte aligned) holds the bitmaps that
 * find repeats; its contents on entry do not matter.
 */
#define PA_FAULT_CONTEXT_LEN 1         /* context_lens[s] < 0 or > max_blocks_per_seq * 16 */
#define PA_FAULT_BLOCK_ID 2            /* a table entry read for sequence s is outside [0, num_blocks) */
#define PA_FAULT_SLOT_RANGE 4          /* slot >= num_blocks * 16 (negative slots are skips) */
#define PA_FAULT_SLOT_REPEATED 8       /* a slot written by two tokens of one call */
#define PA_FAULT_PAIR_RANGE 16         /* a pair's block (or host slot) outside its range */
#define PA_FAULT_DST_REPEATED 32       /* copy: destination named twice; swap: block named twice */
#define PA_FAULT_DST_IS_SRC 64         /* copy: a destination that is also a source */
#define PA_FAULT_HOST_SLOT_REPEATED 128 /* swap: host slot named twice */
#define PA_FAULT_QUERY_START 256       /* query_start[0] != 0, or query_start decreases at s */

/* Workspace bytes the checks need for this pool and host pool size. */
size_t pa_check_workspace_size(const pa_pool_t *pool, int32_t num_host_slots);

/* pa_decode / pa_prefill preconditions on context_lens and block_tables
 * (elements: sequences). */
int pa_check_tables(const pa_pool_t *pool, int32_t num_seqs, const int32_t *block_tables,
                    int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t *report,
                    void *stream);

/* pa_prefill precondition on query_start[0..num_seqs] (elements: offsets). */
int pa_check_query_start(int32_t num_seqs, const int32_t *query_start, int32_t *report,
                         void *stream);

/* pa_reshape_and_cache preconditions on slot_mapping (elements: tokens). */
int pa_check_slots(const pa_pool_t *pool, const int32_t *slot_mapping, int32_t num_tokens,
                   void *workspace, size_t workspace_bytes, int32_t *report, void *stream);

/* pa_copy_blocks preconditions on src_dst_pairs (elements: pairs). */
int pa_check_copy_pairs(const pa_pool_t *pool, const int32_t *src_dst_pairs, int32_t num_pairs,
                        void *workspace, size_t workspace_bytes, int32_t *report, void *stream);

/* pa_swap_blocks preconditions on block_slot_pairs (elements: pairs). */
int pa_check_swap_pairs(const pa_pool_t *pool, int32_t num_host_slots,
                        const int32_t *block_slot_pairs, int32_t num_pairs, void *workspace,
                        size_t workspace_bytes, int32_t *report, void *stream);

/*
 * Debug mode (off by default; on at load when the environment variable
 * PA_DEBUG is 1, or after pa_set_debug(1)).  In it every operation first
 * runs the matching checks on its stream, waits for them, and returns
 * PA_ERR_INDEX without enqueueing the operation when any fault is found
 * (pa_last_error names the kinds and the first index).  Debug mode gives up
 * two conventions of this header for that: it allocates a device buffer
 * (kept per device until the process ends) and it synchronises the stream.
 * Returns the previous setting.
 */
int pa_set_debug(int on);

/* Which partition kernel pa_decode launches for this pool and head count:
 * 0 = vector-ALU kernel (one workgroup per query head), 1 = matrix-core
 * kernel (one workgroup per KV head and its group of query heads).  Returns a
 * negative pa_status on invalid arguments. */
int pa_decode_variant(const pa_pool_t *pool, int32_t num_q_heads);

/* The launch pa_decode_ex makes for these arguments (for tooling and
 * profiles): plan[0] = partition kernel (0 vector-ALU, one workgroup per
 * query head; 1 matrix-core, one partition per workgroup; 2 matrix-core,
 * four partitions per workgroup merged on chip), plan[1] = partition
 * tokens, plan[2] = partial results per (sequence, query head) row (1: none,
 * no merge kernel), plan[3] = partitions merged into each partial result.
 * Returns a pa_status. */
int pa_decode_plan(const pa_pool_t *pool, int32_t num_seqs, int32_t num_q_heads,
                   int32_t max_blocks_per_seq, int32_t partition_tokens, int32_t plan[4]);

/* Measurement aid: the next pa_decode or pa_prefill call on this host
 * thread stores its partition (or prefill) kernel's start time in `before`
 * and its end time in `after` (hipEvent_t; hipEventElapsedTime gives the
 * kernel's duration).  The kernel is launched with hipExtLaunchKernel, whose
 * dispatch records the two events itself.  Pass NULLs to clear. */
int pa_set_profile_events(void *before, void *after);

/* Measurement aid: enqueue one streaming read of `bytes` bytes (rounded down
 * to 16) of device buffer `buf` (16-byte aligned) by a grid-stride kernel, to
 * time the read bandwidth the GPU sustains.  `sink` is a device buffer of at
 * least 16 bytes that the kernel may write.  Returns a pa_status. */
int pa_probe_read(const void *buf, size_t bytes, void *sink, void *stream);

/* Static description of a status code. */
const char *pa_strerror(int status);

/* Description of the last error on this host thread ("" if none). */
const char *pa_last_error(void);

/* Build description: target architecture and kernel variants. */
const char *pa_build_info(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
