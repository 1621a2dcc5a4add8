// pa_api.hip -- the C ABI declared in include/pa.h: argument checks,
// partition and workspace sizing, kernel dispatch and error reporting.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

namespace {

thread_local char g_last_error[512] = "";
thread_local hipEvent_t g_ev_before = nullptr;
thread_local hipEvent_t g_ev_after = nullptr;

int fail(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_last_error[0] = '\0';
    return PA_OK;
}

bool aligned16(const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

int check_pool(const pa_pool_t *pool) {
    if (!pool) return fail(PA_ERR_NULL, "pool descriptor is NULL");
    if (!pool->k_pool || !pool->v_pool) return fail(PA_ERR_NULL, "k_pool or v_pool is NULL");
    if (pool->kv_dtype < PA_F32 || pool->kv_dtype > PA_FP8_E4M3)
        return fail(PA_ERR_DTYPE, "unknown kv_dtype %d", pool->kv_dtype);
    if (pool->block_size != PA_BLOCK_SIZE)
        return fail(PA_ERR_UNSUPPORTED, "block_size %d: only 16 is supported", pool->block_size);
    if (pool->head_dim != 64 && pool->head_dim != 128)
        return fail(PA_ERR_UNSUPPORTED, "head_dim %d: only 64 and 128 are supported", pool->head_dim);
    if (pool->num_blocks <= 0 || pool->num_kv_heads <= 0)
        return fail(PA_ERR_SHAPE, "num_blocks %d and num_kv_heads %d must be positive",
                    pool->num_blocks, pool->num_kv_heads);
    if (pool->num_blocks > INT32_MAX / PA_BLOCK_SIZE)
        return fail(PA_ERR_SHAPE, "num_blocks %d: slots (block * 16 + position) must fit int32",
                    pool->num_blocks);
    if (!aligned16(pool->k_pool) || !aligned16(pool->v_pool))
        return fail(PA_ERR_ALIGN, "k_pool and v_pool must be 16-byte aligned");
    if (pool->kv_dtype == PA_FP8_E4M3) {
        if (!(isfinite(pool->k_scale) && pool->k_scale > 0.f && isfinite(pool->v_scale) &&
              pool->v_scale > 0.f))
            return fail(PA_ERR_RANGE, "fp8 pool scales must be finite and positive (k %g, v %g)",
                        (double)pool->k_scale, (double)pool->v_scale);
        if (!isfinite(1.0f / pool->k_scale) || !isfinite(1.0f / pool->v_scale))
            return fail(PA_ERR_RANGE, "fp8 pool scale too small to invert in fp32");
    }
    return PA_OK;
}

int64_t tile_bytes(const pa_pool_t *pool) {
    return (int64_t)PA_BLOCK_SIZE * pool->head_dim * pa::elem_bytes(pool->kv_dtype);
}

// Library's partition size.  Measured on MI355X: splitting a context costs a
// partial-result write and read plus a second launch, and does not pay for
// contexts up to 4096 tokens; longer contexts are cut into 2048-token
// partitions so that no workgroup walks an unbounded chain of blocks.  Small
// batches split further (down to 256 tokens) until ~1024 workgroups exist.
// SIMDs of the current device (four per compute unit), read once per device.
int32_t simd_count() {
    static std::atomic<int32_t> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1024;
    int32_t v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return 1024;
    v = 4 * cus;
    cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

// How the grouped (matrix-core) kernel maps work to wavefronts (unused by
// the vector-ALU kernel).  Short split-K partitions (<= 512 tokens) go to
// partition groups: one wavefront per partition, kGroupParts partitions of
// a row per workgroup merged on chip, so a partial result per group instead
// of one per partition reaches memory (the stores that end a work item cost
// far more than their bytes while the chip streams K/V).  Otherwise one
// wavefront walks all of a partition's blocks and needs no merge; it is
// faster when the batch alone has at least two rows per SIMD, so that one
// wavefront per row still fills the chip (70B-like batch, 2048 rows: 0.660
// -> 0.653 ms; beam search 0.141 -> 0.135 ms); with fewer rows four
// wavefronts per partition keep more loads in flight (parallel sampling,
// 1536 rows: 0.105 against 0.115).
int wave_mode(const pa_pool_t *pool, int32_t num_seqs, int32_t num_q_heads, int32_t raw_partitions,
              int32_t ptok) {
    if (raw_partitions > 1 && ptok <= 512) return pa::kPartGroups;
    const int64_t rows = (int64_t)num_seqs * pool->num_kv_heads;
    const int64_t simds = simd_count();
    if (rows < 2 * simds) return pa::kFourWaves;
    // With a bf16 pool and exactly one row per slot at two wavefronts per
    // SIMD, three blocks in flight per wavefront (200 VGPRs): the 70B-like
    // batch (2048 rows) after a 1 GiB read 0.666 -> 0.647 ms, back to back
    // 0.643 -> 0.645 ms; with more rows the second round costs more (beam
    // search, 4096 rows: 0.123 -> 0.131 ms), so they keep two.
    if (pool->kv_dtype == PA_BF16 && rows <= 2 * simds) return pa::kOneWaveDeep;
    return pa::kOneWave;
}

bool grouped_kernel(const pa_pool_t *pool, int32_t num_q_heads) {
    return pa::mfma_path_supported(pool->kv_dtype, pool->head_dim, num_q_heads / pool->num_kv_heads);
}

int32_t auto_partition(const pa_pool_t *pool, int32_t num_seqs, int32_t num_q_heads,
                       int32_t max_blocks_per_seq) {
    const bool mfma = pa::mfma_path_supported(pool->kv_dtype, pool->head_dim,
                                              num_q_heads / pool->num_kv_heads);
    const int64_t rows = (int64_t)num_seqs * (mfma ? pool->num_kv_heads : num_q_heads);
    const int64_t max_tokens = (int64_t)max_blocks_per_seq * PA_BLOCK_SIZE;
    int64_t ptok = max_tokens <= 4096 ? max_tokens : 2048;
    while (ptok > 256 && rows * ((max_tokens + ptok - 1) / ptok) < 1024)
        ptok = ((ptok / 2 + 15) / 16) * 16;
    return (int32_t)(ptok < 16 ? 16 : ptok);
}

int resolve_partition(const pa_pool_t *pool, int32_t num_seqs, int32_t num_q_heads,
                      int32_t max_blocks_per_seq, int32_t partition_tokens, int32_t *out) {
    if (partition_tokens < 0 || partition_tokens % PA_BLOCK_SIZE != 0)
        return fail(PA_ERR_SHAPE, "partition_tokens %d must be 0 or a positive multiple of 16",
                    partition_tokens);
    *out = partition_tokens ? partition_tokens
                            : auto_partition(pool, num_seqs, num_q_heads, max_blocks_per_seq);
    return PA_OK;
}

int check_heads(const pa_pool_t *pool, int32_t num_seqs, int32_t num_q_heads,
                int32_t max_blocks_per_seq) {
    if (num_seqs < 0) return fail(PA_ERR_SHAPE, "num_seqs %d is negative", num_seqs);
    if (num_q_heads <= 0 || num_q_heads % pool->num_kv_heads != 0)
        return fail(PA_ERR_SHAPE, "num_q_heads %d must be a positive multiple of num_kv_heads %d",
                    num_q_heads, pool->num_kv_heads);
    if (max_blocks_per_seq <= 0 || max_blocks_per_seq > (1 << 26))
        return fail(PA_ERR_SHAPE, "max_blocks_per_seq %d out of range", max_blocks_per_seq);
    return PA_OK;
}

// Partial results per row, the partitions merged into each (group_parts) and
// the grouped kernel's wave mode for these arguments; the workspace holds
// the partials.
struct Split {
    int32_t slots, group_parts, mode;
};

Split split_for(const pa_pool_t *pool, int32_t num_seqs, int32_t num_q_heads,
                int32_t max_blocks_per_seq, int32_t ptok) {
    const int64_t max_tokens = (int64_t)max_blocks_per_seq * PA_BLOCK_SIZE;
    const int32_t raw = (int32_t)((max_tokens + ptok - 1) / ptok);
    Split sp{raw, 1, pa::kFourWaves};
    if (grouped_kernel(pool, num_q_heads)) {
        sp.mode = wave_mode(pool, num_seqs, num_q_heads, raw, ptok);
        if (sp.mode == pa::kPartGroups) {
            sp.group_parts = pa::kGroupParts;
            sp.slots = (raw + pa::kGroupParts - 1) / pa::kGroupParts;
        }
    }
    return sp;
}

size_t workspace_for(const pa_pool_t *pool, int32_t num_seqs, int32_t num_q_heads,
                     int32_t max_blocks_per_seq, int32_t ptok, int32_t *nparts_out) {
    const int64_t np = split_for(pool, num_seqs, num_q_heads, max_blocks_per_seq, ptok).slots;
    if (nparts_out) *nparts_out = (int32_t)np;
    if (np <= 1) return 0;
    const int64_t rows = (int64_t)num_seqs * num_q_heads * np;
    // acc [rows][D] then m [rows] then l [rows], each region 256-byte aligned
    const int64_t acc = ((rows * pool->head_dim * 4 + 255) / 256) * 256;
    const int64_t ml = ((rows * 4 + 255) / 256) * 256;
    return (size_t)(acc + 2 * ml);
}

// ---- decode of prefix-sharing groups ---------------------------------------

// A group's block list is at most max_group members x max_blocks_per_seq
// blocks (no shared prefix).  The library's partition length keeps each
// group in one partition -- no partial results, no merge -- when the list
// fits one workgroup's LDS list and the groups alone give enough workgroups;
// otherwise it halves the length (down to 1024 tokens) until they do.
int32_t shared_auto_partition(const pa_pool_t *pool, int32_t num_groups, int32_t max_group,
                              int32_t max_blocks_per_seq) {
    const int64_t list_tokens = (int64_t)max_group * max_blocks_per_seq * PA_BLOCK_SIZE;
    const int64_t rows = (int64_t)num_groups * pool->num_kv_heads;
    int64_t ptok = list_tokens < pa::kSharedListMax * PA_BLOCK_SIZE ? list_tokens
                                                                    : pa::kSharedListMax * PA_BLOCK_SIZE;
    while (ptok > 1024 && rows * ((list_tokens + ptok - 1) / ptok) < 512)
        ptok = ((ptok / 2 + 15) / 16) * 16;
    return (int32_t)(ptok < 16 ? 16 : ptok);
}

int check_shared_args(const pa_pool_t *pool, int32_t num_seqs, int32_t num_q_heads,
                      int32_t max_blocks_per_seq, int32_t num_groups, int32_t max_group,
                      int32_t partition_tokens, int32_t *ptok_out) {
    int rc = check_pool(pool);
    if (rc != PA_OK) return rc;
    rc = check_heads(pool, num_seqs, num_q_heads, max_blocks_per_seq);
    if (rc != PA_OK) return rc;
    if (pool->kv_dtype == PA_F32)
        return fail(PA_ERR_UNSUPPORTED, "prefix-shared decode needs a bf16 or fp8 pool");
    const int32_t G = num_q_heads / pool->num_kv_heads;
    if (num_groups < 0 || (num_seqs > 0 && num_groups == 0) || num_groups > num_seqs)
        return fail(PA_ERR_SHAPE, "num_groups %d must be in [1, num_seqs %d]", num_groups, num_seqs);
    if (max_group < 1 || (int64_t)max_group * G > 16)
        return fail(PA_ERR_SHAPE, "max_group_size %d x query group %d must be in [1, 16]", max_group, G);
    if (partition_tokens < 0 || partition_tokens % PA_BLOCK_SIZE != 0 ||
        partition_tokens > pa::kSharedListMax * PA_BLOCK_SIZE)
        return fail(PA_ERR_SHAPE, "partition_tokens %d must be 0 or a multiple of 16 up to %d",
                    partition_tokens, pa::kSharedListMax * PA_BLOCK_SIZE);
    *ptok_out = partition_tokens ? partition_tokens
                                 : shared_auto_partition(pool, num_groups, max_group, max_blocks_per_seq);
    return PA_OK;
}

// Partitions per group at most, and the workspace: fp32 partials per
// (sequence, query head) row and partition, then each group's partition count.
size_t shared_workspace_for(const pa_pool_t *pool, int32_t num_seqs, int32_t num_q_heads,
                            int32_t max_blocks_per_seq, int32_t num_groups, int32_t max_group, int32_t ptok,
                            int32_t *nparts_out) {
    const int64_t list_tokens = (int64_t)max_group * max_blocks_per_seq * PA_BLOCK_SIZE;
    const int64_t np = (list_tokens + ptok - 1) / ptok;
    if (nparts_out) *nparts_out = (int32_t)np;
    if (np <= 1) return 0;
    const int64_t rows = (int64_t)num_seqs * num_q_heads * np;
    const int64_t acc = ((rows * pool->head_dim * 4 + 255) / 256) * 256;
    const int64_t ml = ((rows * 4 + 255) / 256) * 256;
    const int64_t cnt = (((int64_t)num_groups * 4 + 255) / 256) * 256;
    return (size_t)(acc + 2 * ml + cnt);
}

// ---- debug mode: index checks before every operation -------------------

std::atomic<int> g_debug{-1};  // -1 until PA_DEBUG has been read

bool debug_on() {
    int d = g_debug.load();
    if (d < 0) {
        const char *env = getenv("PA_DEBUG");
        int want = env && strcmp(env, "1") == 0 ? 1 : 0;
        g_debug.compare_exchange_strong(d, want);
        d = g_debug.load();
    }
    return d == 1;
}

// One buffer per device (report words, then the check workspace), grown on
// demand; held under the lock for the whole check, which ends with a
// stream synchronisation, so no call can still be using it when another
// takes it.
std::mutex g_debug_mu;
std::vector<std::pair<void *, size_t>> g_debug_buf;

const char *fault_names(int kinds, char *buf, size_t n) {
    static const char *names[] = {"context length out of range", "block id out of range",
                                  "slot out of range",           "slot repeated",
                                  "pair id out of range",        "destination repeated",
                                  "destination is a source",     "host slot repeated",
                                  "query_start not non-decreasing from 0"};
    buf[0] = '\0';
    for (int k = 0; k < 9; ++k) {
        if (!(kinds & (1 << k))) continue;
        if (buf[0]) strncat(buf, ", ", n - strlen(buf) - 1);
        strncat(buf, names[k], n - strlen(buf) - 1);
    }
    return buf;
}

// Runs `launch(report, workspace)` on `st`, waits, and turns faults into
// PA_ERR_INDEX.  Called with the operation's arguments already validated.
template <class Launch>
int debug_check(const char *what, int64_t ws_bytes, hipStream_t st, Launch launch) {
    std::lock_guard<std::mutex> lock(g_debug_mu);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if ((int)g_debug_buf.size() <= dev) g_debug_buf.resize(dev + 1, {nullptr, 0});
    auto &buf = g_debug_buf[dev];
    const size_t need = 256 + (size_t)ws_bytes;
    if (buf.second < need) {
        if (buf.first) {
            e = hipFree(buf.first);
            if (e != hipSuccess) return fail(PA_ERR_HIP, "hipFree: %s", hipGetErrorString(e));
        }
        buf = {nullptr, 0};
        e = hipMalloc(&buf.first, need);
        if (e != hipSuccess) return fail(PA_ERR_HIP, "debug buffer: %s", hipGetErrorString(e));
        buf.second = need;
    }
    int32_t *report = static_cast<int32_t *>(buf.first);
    e = launch(report, static_cast<char *>(buf.first) + 256);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    int32_t h[3] = {0, 0, -1};
    if (e == hipSuccess) e = hipMemcpy(h, report, sizeof(h), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "%s index check: %s", what, hipGetErrorString(e));
    if (h[0] > 0) {
        char names[256];
        return fail(PA_ERR_INDEX, "%s: %d index faults (%s), first at element %d", what, h[0],
                    fault_names(h[1], names, sizeof(names)), h[2]);
    }
    return PA_OK;
}

int check_report_args(const int32_t *report) {
    if (!report) return fail(PA_ERR_NULL, "report is NULL");
    if ((reinterpret_cast<uintptr_t>(report) & 3u) != 0)
        return fail(PA_ERR_ALIGN, "report must be 4-byte aligned");
    return PA_OK;
}

int check_workspace_args(const pa_pool_t *pool, int32_t num_host_slots, const void *workspace,
                         size_t workspace_bytes) {
    const size_t need = (size_t)pa::check_workspace_bytes(pool->num_blocks, num_host_slots);
    if (!workspace || workspace_bytes < need)
        return fail(PA_ERR_WORKSPACE, "check workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if ((reinterpret_cast<uintptr_t>(workspace) & 3u) != 0)
        return fail(PA_ERR_ALIGN, "workspace must be 4-byte aligned");
    return PA_OK;
}

}  // namespace

extern "C" {

size_t pa_pool_bytes(const pa_pool_t *pool) {
    if (check_pool(pool) != PA_OK) return 0;
    return (size_t)pool->num_blocks * pool->num_kv_heads * (size_t)tile_bytes(pool);
}

int32_t pa_decode_partition_tokens(const pa_pool_t *pool, int32_t num_seqs, int32_t num_q_heads,
                                   int32_t max_blocks_per_seq, int32_t partition_tokens) {
    int rc = check_pool(pool);
    if (rc == PA_OK) rc = check_heads(pool, num_seqs, num_q_heads, max_blocks_per_seq);
    if (rc != PA_OK) return rc;
    int32_t ptok = 0;
    rc = resolve_partition(pool, num_seqs, num_q_heads, max_blocks_per_seq, partition_tokens, &ptok);
    return rc == PA_OK ? ptok : rc;
}

size_t pa_decode_workspace_size(const pa_pool_t *pool, int32_t num_seqs, int32_t num_q_heads,
                                int32_t max_blocks_per_seq, int32_t partition_tokens) {
    const int32_t ptok = pa_decode_partition_tokens(pool, num_seqs, num_q_heads,
                                                    max_blocks_per_seq, partition_tokens);
    if (ptok <= 0) return 0;
    return workspace_for(pool, num_seqs, num_q_heads, max_blocks_per_seq, ptok, nullptr);
}

int pa_decode(const pa_pool_t *pool, const void *q, int32_t q_dtype, int32_t num_seqs,
              int32_t num_q_heads, const int32_t *block_tables, int32_t max_blocks_per_seq,
              const int32_t *context_lens, float scale, float *out, int32_t partition_tokens,
              void *workspace, size_t workspace_bytes, void *stream) {
    return pa_decode_ex(pool, q, q_dtype, num_seqs, num_q_heads, block_tables, max_blocks_per_seq,
                        context_lens, scale, out, partition_tokens, workspace, workspace_bytes,
                        PA_DECODE_STREAM_KV, stream);
}

}  // extern "C"

namespace {

// Split-K scratch of pa_decode_noalloc: one copy per device, at its own
// device address.  Host code never uses the array's name as an address (on
// the host it names a stand-in): the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
__device__ __align__(256) unsigned char scratch[PA_DECODE_NOALLOC_MAX_SCRATCH];

std::mutex g_scratch_mu;
void *g_scratch_ptr[64] = {};

// The current device's copy of `scratch` (NULL and a failed status on error).
int scratch_for_current_device(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return fail(PA_ERR_HIP, "device %d: at most 64 devices are supported", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(PA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return PA_OK;
}

// pa_decode_ex, and pa_decode_append when k_new is not NULL.  `checks`:
// debug mode may run its index checks (they allocate a buffer).
int decode_impl(const pa_pool_t *pool, const void *q, int32_t q_dtype, int32_t num_seqs,
                int32_t num_q_heads, const int32_t *block_tables, int32_t max_blocks_per_seq,
                const int32_t *context_lens, float scale, float *out, int32_t partition_tokens,
                void *workspace, size_t workspace_bytes, uint32_t flags, const void *k_new,
                const void *v_new, int32_t kv_dtype, void *stream, bool checks = true) {
    if (flags & ~(uint32_t)PA_DECODE_SHARED_KV)
        return fail(PA_ERR_SHAPE, "unknown decode flags 0x%x", flags);
    int rc = check_pool(pool);
    if (rc != PA_OK) return rc;
    rc = check_heads(pool, num_seqs, num_q_heads, max_blocks_per_seq);
    if (rc != PA_OK) return rc;
    const int want_q = pool->kv_dtype == PA_F32 ? PA_F32 : PA_BF16;
    if (q_dtype != want_q)
        return fail(PA_ERR_DTYPE, "q_dtype %d does not match a kv_dtype %d pool (needs %d)", q_dtype,
                    pool->kv_dtype, want_q);
    if (!isfinite(scale)) return fail(PA_ERR_RANGE, "scale is not finite");
    int32_t ptok = 0;
    rc = resolve_partition(pool, num_seqs, num_q_heads, max_blocks_per_seq, partition_tokens, &ptok);
    if (rc != PA_OK) return rc;
    if (num_seqs == 0) return ok();
    if (!q || !block_tables || !context_lens || !out)
        return fail(PA_ERR_NULL, "q, block_tables, context_lens and out must be non-NULL");
    // the kernels write out (and read q) with 16-byte accesses
    if (!aligned16(q) || !aligned16(out)) return fail(PA_ERR_ALIGN, "q and out must be 16-byte aligned");
    int32_t np = 1;
    const size_t need = workspace_for(pool, num_seqs, num_q_heads, max_blocks_per_seq, ptok, &np);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (need > 0 && !aligned16(workspace)) return fail(PA_ERR_ALIGN, "workspace must be 16-byte aligned");
    if (k_new || v_new) {
        if (!k_new || !v_new) return fail(PA_ERR_NULL, "k_new and v_new must both be given");
        const bool dtype_ok = pool->kv_dtype == PA_FP8_E4M3 ? (kv_dtype == PA_BF16 || kv_dtype == PA_F32)
                                                            : kv_dtype == pool->kv_dtype;
        if (!dtype_ok)
            return fail(PA_ERR_DTYPE, "new-token dtype %d cannot be written to a kv_dtype %d pool", kv_dtype,
                        pool->kv_dtype);
    }

    pa::DecodeParams p{};
    p.k_pool = pool->k_pool;
    p.v_pool = pool->v_pool;
    p.q = q;
    p.out = out;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.num_blocks = pool->num_blocks;
    p.num_kv_heads = pool->num_kv_heads;
    p.num_q_heads = num_q_heads;
    p.group = num_q_heads / pool->num_kv_heads;
    p.num_seqs = num_seqs;
    p.max_blocks_per_seq = max_blocks_per_seq;
    const Split sp = split_for(pool, num_seqs, num_q_heads, max_blocks_per_seq, ptok);
    p.partition_tokens = ptok;
    p.group_parts = sp.group_parts;
    p.max_partitions = sp.slots;
    p.wave_mode = sp.mode;
    const double kscale = pool->kv_dtype == PA_FP8_E4M3 ? (double)pool->k_scale : 1.0;
    p.qk_scale_log2 = (float)((double)scale * kscale * 1.4426950408889634);
    p.out_scale = pool->kv_dtype == PA_FP8_E4M3 ? pool->v_scale : 1.0f;
    p.shared_kv = (flags & PA_DECODE_SHARED_KV) ? 1 : 0;
    p.k_new = k_new;
    p.v_new = v_new;
    p.new_dtype = kv_dtype;
    p.inv_k_scale = pool->kv_dtype == PA_FP8_E4M3 ? 1.0f / pool->k_scale : 1.0f;
    p.inv_v_scale = pool->kv_dtype == PA_FP8_E4M3 ? 1.0f / pool->v_scale : 1.0f;
    if (need > 0) {
        const int64_t rows = (int64_t)num_seqs * num_q_heads * np;
        char *ws = static_cast<char *>(workspace);
        const int64_t acc = ((rows * pool->head_dim * 4 + 255) / 256) * 256;
        const int64_t ml = ((rows * 4 + 255) / 256) * 256;
        p.ws_acc = reinterpret_cast<float *>(ws);
        p.ws_m = reinterpret_cast<float *>(ws + acc);
        p.ws_l = reinterpret_cast<float *>(ws + acc + ml);
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (checks && debug_on()) {
        rc = debug_check("pa_decode", 0, st, [&](int32_t *report, void *) {
            return pa::launch_check_tables(block_tables, context_lens, num_seqs, max_blocks_per_seq,
                                           pool->num_blocks, report, st);
        });
        if (rc != PA_OK) return rc;
        if (k_new) {
            // the newest tokens' slots, then the cache write's slot check on them
            const int64_t slot_bytes = (((int64_t)num_seqs * 4 + 255) / 256) * 256;
            rc = debug_check("pa_decode_append", slot_bytes + pa::check_workspace_bytes(pool->num_blocks, 0),
                             st, [&](int32_t *report, void *ws) {
                                 int32_t *slots = static_cast<int32_t *>(ws);
                                 hipError_t e = pa::launch_append_slots(block_tables, context_lens, num_seqs,
                                                                        max_blocks_per_seq, pool->num_blocks,
                                                                        slots, st);
                                 if (e != hipSuccess) return e;
                                 return pa::launch_check_slots(slots, num_seqs, pool->num_blocks,
                                                               static_cast<char *>(ws) + slot_bytes, report, st);
                             });
            if (rc != PA_OK) return rc;
        }
    }
    const bool mfma = pa::mfma_path_supported(pool->kv_dtype, pool->head_dim, p.group);
    if (k_new && !mfma && p.group > 1) {
        // several workgroups read each KV head's last block: the new tokens
        // are written by a kernel of their own first
        hipError_t e = pa::launch_append_tokens(pool->kv_dtype, pool->head_dim, p, st);
        if (e != hipSuccess) return fail(PA_ERR_HIP, "append kernel: %s", hipGetErrorString(e));
        p.k_new = p.v_new = nullptr;
    }
    const pa::LaunchEvents ev{g_ev_before, g_ev_after};
    g_ev_before = g_ev_after = nullptr;
    hipError_t e = mfma ? pa::launch_decode_mfma(pool->kv_dtype, pool->head_dim, p, st, &ev)
                        : pa::launch_decode_valu(pool->kv_dtype, pool->head_dim, p, st, &ev);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "decode partition kernel: %s", hipGetErrorString(e));
    if (np > 1) {
        e = pa::launch_decode_reduce(pool->head_dim, p, st);
        if (e != hipSuccess) return fail(PA_ERR_HIP, "decode reduce kernel: %s", hipGetErrorString(e));
    }
    return ok();
}

}  // namespace

extern "C" {

int pa_decode_ex(const pa_pool_t *pool, const void *q, int32_t q_dtype, int32_t num_seqs,
                 int32_t num_q_heads, const int32_t *block_tables, int32_t max_blocks_per_seq,
                 const int32_t *context_lens, float scale, float *out, int32_t partition_tokens,
                 void *workspace, size_t workspace_bytes, uint32_t flags, void *stream) {
    return decode_impl(pool, q, q_dtype, num_seqs, num_q_heads, block_tables, max_blocks_per_seq,
                       context_lens, scale, out, partition_tokens, workspace, workspace_bytes, flags,
                       nullptr, nullptr, 0, stream);
}

int pa_decode_noalloc(const pa_pool_t *pool, const void *q, int32_t q_dtype, int32_t num_seqs,
                      int32_t num_q_heads, const int32_t *block_tables, int32_t max_blocks_per_seq,
                      const int32_t *context_lens, float scale, float *out, int32_t partition_tokens,
                      uint32_t flags, void *stream) {
    // the arguments' own checks first (as pa_decode_ex makes them), then the
    // size of the partials against the static scratch
    int rc = check_pool(pool);
    if (rc == PA_OK) rc = check_heads(pool, num_seqs, num_q_heads, max_blocks_per_seq);
    int32_t ptok = 0;
    if (rc == PA_OK)
        rc = resolve_partition(pool, num_seqs, num_q_heads, max_blocks_per_seq, partition_tokens, &ptok);
    if (rc != PA_OK) return rc;
    const size_t need = workspace_for(pool, num_seqs, num_q_heads, max_blocks_per_seq, ptok, nullptr);
    if (need > PA_DECODE_NOALLOC_MAX_SCRATCH)
        return fail(PA_ERR_WORKSPACE,
                    "split-K partials of %zu bytes exceed the %zu-byte static scratch of "
                    "pa_decode_noalloc (use pa_decode_ex with a workspace, or longer partitions)",
                    need, (size_t)PA_DECODE_NOALLOC_MAX_SCRATCH);
    void *ws = nullptr;
    if (need > 0 && num_seqs > 0) {
        rc = scratch_for_current_device(&ws);
        if (rc != PA_OK) return rc;
    }
    return decode_impl(pool, q, q_dtype, num_seqs, num_q_heads, block_tables, max_blocks_per_seq,
                       context_lens, scale, out, partition_tokens, ws,
                       ws ? (size_t)PA_DECODE_NOALLOC_MAX_SCRATCH : 0, flags, nullptr, nullptr, 0,
                       stream, /*checks=*/false);
}

size_t pa_decode_prefix_shared_workspace_size(const pa_pool_t *pool, int32_t num_seqs, int32_t num_q_heads,
                                              int32_t max_blocks_per_seq, int32_t num_groups,
                                              int32_t max_group_size, int32_t partition_tokens) {
    int32_t ptok = 0;
    if (check_shared_args(pool, num_seqs, num_q_heads, max_blocks_per_seq, num_groups, max_group_size,
                          partition_tokens, &ptok) != PA_OK)
        return 0;
    return shared_workspace_for(pool, num_seqs, num_q_heads, max_blocks_per_seq, num_groups, max_group_size,
                                ptok, nullptr);
}

int pa_decode_prefix_shared_plan(const pa_pool_t *pool, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t max_blocks_per_seq, int32_t num_groups, int32_t max_group_size,
                                 int32_t partition_tokens, int32_t plan[2]) {
    if (!plan) return fail(PA_ERR_NULL, "plan must be non-NULL");
    int32_t ptok = 0, np = 0;
    const int rc = check_shared_args(pool, num_seqs, num_q_heads, max_blocks_per_seq, num_groups,
                                     max_group_size, partition_tokens, &ptok);
    if (rc != PA_OK) return rc;
    shared_workspace_for(pool, num_seqs, num_q_heads, max_blocks_per_seq, num_groups, max_group_size, ptok,
                         &np);
    plan[0] = ptok;
    plan[1] = np;
    return ok();
}

int pa_decode_prefix_shared(const pa_pool_t *pool, const void *q, int32_t q_dtype, int32_t num_seqs,
                            int32_t num_q_heads, const int32_t *block_tables, int32_t max_blocks_per_seq,
                            const int32_t *context_lens, const int32_t *group_start,
                            const int32_t *prefix_blocks, int32_t num_groups, int32_t max_group_size,
                            float scale, float *out, int32_t partition_tokens, void *workspace,
                            size_t workspace_bytes, uint32_t flags, void *stream) {
    if (flags & ~(uint32_t)PA_DECODE_SHARED_KV)
        return fail(PA_ERR_SHAPE, "unknown decode flags 0x%x", flags);
    int32_t ptok = 0;
    int rc = check_shared_args(pool, num_seqs, num_q_heads, max_blocks_per_seq, num_groups, max_group_size,
                               partition_tokens, &ptok);
    if (rc != PA_OK) return rc;
    if (q_dtype != PA_BF16)
        return fail(PA_ERR_DTYPE, "q_dtype %d: prefix-shared decode takes PA_BF16 queries", q_dtype);
    if (!isfinite(scale)) return fail(PA_ERR_RANGE, "scale is not finite");
    if (num_seqs == 0) return ok();
    if (!q || !block_tables || !context_lens || !out || !group_start || !prefix_blocks)
        return fail(PA_ERR_NULL, "q, block_tables, context_lens, group_start, prefix_blocks and out "
                                 "must be non-NULL");
    if (!aligned16(q) || !aligned16(out)) return fail(PA_ERR_ALIGN, "q and out must be 16-byte aligned");
    int32_t np = 1;
    const size_t need = shared_workspace_for(pool, num_seqs, num_q_heads, max_blocks_per_seq, num_groups,
                                             max_group_size, ptok, &np);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (need > 0 && !aligned16(workspace)) return fail(PA_ERR_ALIGN, "workspace must be 16-byte aligned");

    pa::DecodeParams p{};
    p.k_pool = pool->k_pool;
    p.v_pool = pool->v_pool;
    p.q = q;
    p.out = out;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.num_blocks = pool->num_blocks;
    p.num_kv_heads = pool->num_kv_heads;
    p.num_q_heads = num_q_heads;
    p.group = num_q_heads / pool->num_kv_heads;
    p.num_seqs = num_seqs;
    p.max_blocks_per_seq = max_blocks_per_seq;
    p.partition_tokens = ptok;
    p.group_parts = 1;
    p.max_partitions = np;
    const double kscale = pool->kv_dtype == PA_FP8_E4M3 ? (double)pool->k_scale : 1.0;
    p.qk_scale_log2 = (float)((double)scale * kscale * 1.4426950408889634);
    p.out_scale = pool->kv_dtype == PA_FP8_E4M3 ? pool->v_scale : 1.0f;
    p.shared_kv = (flags & PA_DECODE_SHARED_KV) ? 1 : 0;
    p.group_start = group_start;
    p.prefix_blocks = prefix_blocks;
    p.num_groups = num_groups;
    p.max_group = max_group_size;
    if (need > 0) {
        const int64_t rows = (int64_t)num_seqs * num_q_heads * np;
        char *ws = static_cast<char *>(workspace);
        const int64_t acc = ((rows * pool->head_dim * 4 + 255) / 256) * 256;
        const int64_t ml = ((rows * 4 + 255) / 256) * 256;
        p.ws_acc = reinterpret_cast<float *>(ws);
        p.ws_m = reinterpret_cast<float *>(ws + acc);
        p.ws_l = reinterpret_cast<float *>(ws + acc + ml);
        p.ws_nparts = reinterpret_cast<int32_t *>(ws + acc + 2 * ml);
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (debug_on()) {
        rc = debug_check("pa_decode_prefix_shared", 0, st, [&](int32_t *report, void *) {
            return pa::launch_check_tables(block_tables, context_lens, num_seqs, max_blocks_per_seq,
                                           pool->num_blocks, report, st);
        });
        if (rc != PA_OK) return rc;
    }
    const pa::LaunchEvents ev{g_ev_before, g_ev_after};
    g_ev_before = g_ev_after = nullptr;
    hipError_t e = pa::launch_decode_shared(pool->kv_dtype, pool->head_dim, p, st, &ev);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "prefix-shared decode kernel: %s", hipGetErrorString(e));
    if (np > 1) {
        e = pa::launch_decode_shared_reduce(pool->head_dim, p, st);
        if (e != hipSuccess) return fail(PA_ERR_HIP, "prefix-shared reduce kernel: %s", hipGetErrorString(e));
    }
    return ok();
}

int pa_decode_append(const pa_pool_t *pool, const void *q, int32_t q_dtype, int32_t num_seqs,
                     int32_t num_q_heads, const int32_t *block_tables, int32_t max_blocks_per_seq,
                     const int32_t *context_lens, float scale, float *out, int32_t partition_tokens,
                     void *workspace, size_t workspace_bytes, uint32_t flags, const void *k_new,
                     const void *v_new, int32_t kv_dtype, void *stream) {
    if (num_seqs > 0 && (!k_new || !v_new)) return fail(PA_ERR_NULL, "k_new and v_new must be non-NULL");
    return decode_impl(pool, q, q_dtype, num_seqs, num_q_heads, block_tables, max_blocks_per_seq,
                       context_lens, scale, out, partition_tokens, workspace, workspace_bytes, flags,
                       k_new, v_new, kv_dtype, stream);
}

int pa_prefill(const pa_pool_t *pool, const void *q, int32_t q_dtype, int32_t num_seqs,
               int32_t num_q_heads, const int32_t *query_start, int32_t max_query_len,
               const int32_t *block_tables, int32_t max_blocks_per_seq,
               const int32_t *context_lens, float scale, float *out, void *stream) {
    int rc = check_pool(pool);
    if (rc != PA_OK) return rc;
    rc = check_heads(pool, num_seqs, num_q_heads, max_blocks_per_seq);
    if (rc != PA_OK) return rc;
    const int group = num_q_heads / pool->num_kv_heads;
    if (!pa::prefill_supported(pool->kv_dtype, pool->head_dim, group))
        return fail(PA_ERR_UNSUPPORTED,
                    "prefill needs a bf16 or fp8 pool and a query group the kernel tiles (kv_dtype %d, group %d)",
                    pool->kv_dtype, group);
    if (q_dtype != PA_BF16) return fail(PA_ERR_DTYPE, "prefill q_dtype must be PA_BF16, got %d", q_dtype);
    if (!isfinite(scale)) return fail(PA_ERR_RANGE, "scale is not finite");
    if (max_query_len < 0) return fail(PA_ERR_SHAPE, "max_query_len %d is negative", max_query_len);
    if (num_seqs == 0 || max_query_len == 0) return ok();
    if (!q || !query_start || !block_tables || !context_lens || !out)
        return fail(PA_ERR_NULL, "q, query_start, block_tables, context_lens and out must be non-NULL");
    if (!aligned16(q) || !aligned16(out)) return fail(PA_ERR_ALIGN, "q and out must be 16-byte aligned");

    pa::PrefillParams p{};
    p.k_pool = pool->k_pool;
    p.v_pool = pool->v_pool;
    p.q = q;
    p.out = out;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.query_start = query_start;
    p.num_blocks = pool->num_blocks;
    p.num_kv_heads = pool->num_kv_heads;
    p.num_q_heads = num_q_heads;
    p.group = group;
    p.num_seqs = num_seqs;
    p.max_blocks_per_seq = max_blocks_per_seq;
    p.max_query_len = max_query_len;
    const int tile = pa::prefill_tile_tokens(pool->head_dim, group);
    p.num_tiles = (max_query_len + tile - 1) / tile;
    const double kscale = pool->kv_dtype == PA_FP8_E4M3 ? (double)pool->k_scale : 1.0;
    p.qk_scale_log2 = (float)((double)scale * kscale * 1.4426950408889634);
    p.out_scale = pool->kv_dtype == PA_FP8_E4M3 ? pool->v_scale : 1.0f;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (debug_on()) {
        rc = debug_check("pa_prefill", 0, st, [&](int32_t *report, void *) {
            return pa::launch_check_tables(block_tables, context_lens, num_seqs, max_blocks_per_seq,
                                           pool->num_blocks, report, st);
        });
        if (rc == PA_OK)
            rc = debug_check("pa_prefill", 0, st, [&](int32_t *report, void *) {
                return pa::launch_check_query_start(query_start, num_seqs, report, st);
            });
        if (rc != PA_OK) return rc;
    }
    const pa::LaunchEvents ev{g_ev_before, g_ev_after};
    g_ev_before = g_ev_after = nullptr;
    hipError_t e = pa::launch_prefill(pool->kv_dtype, pool->head_dim, p, st, &ev);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "prefill kernel: %s", hipGetErrorString(e));
    return ok();
}

int pa_reshape_and_cache(const pa_pool_t *pool, const void *k, const void *v, int32_t kv_dtype,
                         const int32_t *slot_mapping, int32_t num_tokens, void *stream) {
    int rc = check_pool(pool);
    if (rc != PA_OK) return rc;
    const bool dtype_ok = pool->kv_dtype == PA_FP8_E4M3
                              ? (kv_dtype == PA_BF16 || kv_dtype == PA_F32)
                              : kv_dtype == pool->kv_dtype;
    if (!dtype_ok)
        return fail(PA_ERR_DTYPE, "input dtype %d cannot be written to a kv_dtype %d pool", kv_dtype,
                    pool->kv_dtype);
    if (num_tokens < 0) return fail(PA_ERR_SHAPE, "num_tokens %d is negative", num_tokens);
    if (num_tokens == 0) return ok();
    if (!k || !v || !slot_mapping) return fail(PA_ERR_NULL, "k, v and slot_mapping must be non-NULL");
    if (!aligned16(k) || !aligned16(v)) return fail(PA_ERR_ALIGN, "k and v must be 16-byte aligned");
    pa::CacheParams p{};
    p.k_pool = pool->k_pool;
    p.v_pool = pool->v_pool;
    p.k = k;
    p.v = v;
    p.slot_mapping = slot_mapping;
    p.num_tokens = num_tokens;
    p.num_blocks = pool->num_blocks;
    p.num_kv_heads = pool->num_kv_heads;
    p.inv_k_scale = pool->kv_dtype == PA_FP8_E4M3 ? 1.0f / pool->k_scale : 1.0f;
    p.inv_v_scale = pool->kv_dtype == PA_FP8_E4M3 ? 1.0f / pool->v_scale : 1.0f;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (debug_on()) {
        rc = debug_check("pa_reshape_and_cache", pa::check_workspace_bytes(pool->num_blocks, 0), st,
                         [&](int32_t *report, void *ws) {
                             return pa::launch_check_slots(slot_mapping, num_tokens, pool->num_blocks,
                                                           ws, report, st);
                         });
        if (rc != PA_OK) return rc;
    }
    hipError_t e = pa::launch_reshape_and_cache(pool->kv_dtype, kv_dtype, pool->head_dim, p, st);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "reshape_and_cache kernel: %s", hipGetErrorString(e));
    return ok();
}

int pa_copy_blocks(const pa_pool_t *pool, const int32_t *src_dst_pairs, int32_t num_pairs,
                   void *stream) {
    int rc = check_pool(pool);
    if (rc != PA_OK) return rc;
    if (num_pairs < 0) return fail(PA_ERR_SHAPE, "num_pairs %d is negative", num_pairs);
    if (num_pairs == 0) return ok();
    if (!src_dst_pairs) return fail(PA_ERR_NULL, "src_dst_pairs is NULL");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (debug_on()) {
        rc = debug_check("pa_copy_blocks", pa::check_workspace_bytes(pool->num_blocks, 0), st,
                         [&](int32_t *report, void *ws) {
                             return pa::launch_check_pairs(src_dst_pairs, num_pairs, pool->num_blocks, 0,
                                                           false, ws, report, st);
                         });
        if (rc != PA_OK) return rc;
    }
    hipError_t e = pa::launch_copy_blocks(pool->k_pool, pool->v_pool, src_dst_pairs, num_pairs,
                                          pool->num_blocks, pool->num_kv_heads * tile_bytes(pool), st);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "copy_blocks kernel: %s", hipGetErrorString(e));
    return ok();
}

int pa_swap_blocks(const pa_pool_t *pool, void *host_k, void *host_v, int32_t num_host_slots,
                   const int32_t *block_slot_pairs, int32_t num_pairs, int32_t direction,
                   void *stream) {
    int rc = check_pool(pool);
    if (rc != PA_OK) return rc;
    if (direction != PA_SWAP_OUT && direction != PA_SWAP_IN)
        return fail(PA_ERR_SHAPE, "direction %d must be PA_SWAP_OUT or PA_SWAP_IN", direction);
    if (num_pairs < 0 || num_host_slots < 0)
        return fail(PA_ERR_SHAPE, "num_pairs %d and num_host_slots %d must be >= 0", num_pairs,
                    num_host_slots);
    if (num_pairs == 0) return ok();
    if (!host_k || !host_v || !block_slot_pairs)
        return fail(PA_ERR_NULL, "host_k, host_v and block_slot_pairs must be non-NULL");
    if (!aligned16(host_k) || !aligned16(host_v))
        return fail(PA_ERR_ALIGN, "host_k and host_v must be 16-byte aligned");
    // the device-side addresses of the pinned host pools (fails for pageable memory)
    void *dk = nullptr, *dv = nullptr;
    hipError_t e = hipHostGetDevicePointer(&dk, host_k, 0);
    if (e == hipSuccess) e = hipHostGetDevicePointer(&dv, host_v, 0);
    if (e != hipSuccess)
        return fail(PA_ERR_HIP, "host pools must be pinned, device-mapped host memory: %s",
                    hipGetErrorString(e));
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (debug_on()) {
        rc = debug_check("pa_swap_blocks", pa::check_workspace_bytes(pool->num_blocks, num_host_slots),
                         st, [&](int32_t *report, void *ws) {
                             return pa::launch_check_pairs(block_slot_pairs, num_pairs, pool->num_blocks,
                                                           num_host_slots, true, ws, report, st);
                         });
        if (rc != PA_OK) return rc;
    }
    e = pa::launch_swap_blocks(pool->k_pool, pool->v_pool, dk, dv, block_slot_pairs, num_pairs,
                               pool->num_blocks, num_host_slots,
                               pool->num_kv_heads * tile_bytes(pool), direction == PA_SWAP_OUT, st);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "swap_blocks kernel: %s", hipGetErrorString(e));
    return ok();
}

size_t pa_check_workspace_size(const pa_pool_t *pool, int32_t num_host_slots) {
    if (check_pool(pool) != PA_OK || num_host_slots < 0) return 0;
    return (size_t)pa::check_workspace_bytes(pool->num_blocks, num_host_slots);
}

int pa_check_tables(const pa_pool_t *pool, int32_t num_seqs, const int32_t *block_tables,
                    int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t *report,
                    void *stream) {
    int rc = check_pool(pool);
    if (rc == PA_OK) rc = check_report_args(report);
    if (rc != PA_OK) return rc;
    if (num_seqs < 0) return fail(PA_ERR_SHAPE, "num_seqs %d is negative", num_seqs);
    if (max_blocks_per_seq <= 0 || max_blocks_per_seq > (1 << 26))
        return fail(PA_ERR_SHAPE, "max_blocks_per_seq %d out of range", max_blocks_per_seq);
    if (num_seqs > 0 && (!block_tables || !context_lens))
        return fail(PA_ERR_NULL, "block_tables and context_lens must be non-NULL");
    hipError_t e = pa::launch_check_tables(block_tables, context_lens, num_seqs, max_blocks_per_seq,
                                           pool->num_blocks, report, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PA_ERR_HIP, "table check: %s", hipGetErrorString(e));
    return ok();
}

int pa_check_query_start(int32_t num_seqs, const int32_t *query_start, int32_t *report, void *stream) {
    int rc = check_report_args(report);
    if (rc != PA_OK) return rc;
    if (num_seqs < 0) return fail(PA_ERR_SHAPE, "num_seqs %d is negative", num_seqs);
    if (!query_start) return fail(PA_ERR_NULL, "query_start is NULL");
    hipError_t e = pa::launch_check_query_start(query_start, num_seqs, report,
                                                static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PA_ERR_HIP, "query_start check: %s", hipGetErrorString(e));
    return ok();
}

int pa_check_slots(const pa_pool_t *pool, const int32_t *slot_mapping, int32_t num_tokens,
                   void *workspace, size_t workspace_bytes, int32_t *report, void *stream) {
    int rc = check_pool(pool);
    if (rc == PA_OK) rc = check_report_args(report);
    if (rc == PA_OK) rc = check_workspace_args(pool, 0, workspace, workspace_bytes);
    if (rc != PA_OK) return rc;
    if (num_tokens < 0) return fail(PA_ERR_SHAPE, "num_tokens %d is negative", num_tokens);
    if (num_tokens > 0 && !slot_mapping) return fail(PA_ERR_NULL, "slot_mapping is NULL");
    hipError_t e = pa::launch_check_slots(slot_mapping, num_tokens, pool->num_blocks, workspace, report,
                                          static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PA_ERR_HIP, "slot check: %s", hipGetErrorString(e));
    return ok();
}

int pa_check_copy_pairs(const pa_pool_t *pool, const int32_t *src_dst_pairs, int32_t num_pairs,
                        void *workspace, size_t workspace_bytes, int32_t *report, void *stream) {
    int rc = check_pool(pool);
    if (rc == PA_OK) rc = check_report_args(report);
    if (rc == PA_OK) rc = check_workspace_args(pool, 0, workspace, workspace_bytes);
    if (rc != PA_OK) return rc;
    if (num_pairs < 0) return fail(PA_ERR_SHAPE, "num_pairs %d is negative", num_pairs);
    if (num_pairs > 0 && !src_dst_pairs) return fail(PA_ERR_NULL, "src_dst_pairs is NULL");
    hipError_t e = pa::launch_check_pairs(src_dst_pairs, num_pairs, pool->num_blocks, 0, false,
                                          workspace, report, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PA_ERR_HIP, "copy pair check: %s", hipGetErrorString(e));
    return ok();
}

int pa_check_swap_pairs(const pa_pool_t *pool, int32_t num_host_slots,
                        const int32_t *block_slot_pairs, int32_t num_pairs, void *workspace,
                        size_t workspace_bytes, int32_t *report, void *stream) {
    int rc = check_pool(pool);
    if (rc == PA_OK) rc = check_report_args(report);
    if (rc != PA_OK) return rc;
    if (num_pairs < 0 || num_host_slots < 0)
        return fail(PA_ERR_SHAPE, "num_pairs %d and num_host_slots %d must be >= 0", num_pairs,
                    num_host_slots);
    rc = check_workspace_args(pool, num_host_slots, workspace, workspace_bytes);
    if (rc != PA_OK) return rc;
    if (num_pairs > 0 && !block_slot_pairs) return fail(PA_ERR_NULL, "block_slot_pairs is NULL");
    hipError_t e = pa::launch_check_pairs(block_slot_pairs, num_pairs, pool->num_blocks, num_host_slots,
                                          true, workspace, report, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PA_ERR_HIP, "swap pair check: %s", hipGetErrorString(e));
    return ok();
}

int pa_set_debug(int on) {
    const int was = debug_on() ? 1 : 0;
    g_debug.store(on ? 1 : 0);
    return was;
}

int pa_decode_variant(const pa_pool_t *pool, int32_t num_q_heads) {
    int rc = check_pool(pool);
    if (rc == PA_OK) rc = check_heads(pool, 0, num_q_heads, 1);
    if (rc != PA_OK) return rc;
    return pa::mfma_path_supported(pool->kv_dtype, pool->head_dim,
                                   num_q_heads / pool->num_kv_heads) ? 1 : 0;
}

int pa_decode_plan(const pa_pool_t *pool, int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                   int32_t partition_tokens, int32_t plan[4]) {
    int rc = check_pool(pool);
    if (rc == PA_OK) rc = check_heads(pool, num_seqs, num_q_heads, max_blocks_per_seq);
    if (rc != PA_OK) return rc;
    if (!plan) return fail(PA_ERR_NULL, "plan is NULL");
    int32_t ptok = 0;
    rc = resolve_partition(pool, num_seqs, num_q_heads, max_blocks_per_seq, partition_tokens, &ptok);
    if (rc != PA_OK) return rc;
    const Split sp = split_for(pool, num_seqs, num_q_heads, max_blocks_per_seq, ptok);
    plan[0] = !grouped_kernel(pool, num_q_heads) ? 0 : (sp.mode == pa::kPartGroups ? 2 : 1);
    plan[1] = ptok;
    plan[2] = sp.slots;
    plan[3] = sp.group_parts;
    return ok();
}

int pa_set_profile_events(void *before, void *after) {
    if ((before == nullptr) != (after == nullptr))
        return fail(PA_ERR_NULL, "pass both events or neither");
    g_ev_before = static_cast<hipEvent_t>(before);
    g_ev_after = static_cast<hipEvent_t>(after);
    return ok();
}

const char *pa_strerror(int status) {
    switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "required pointer is NULL";
    case PA_ERR_DTYPE: return "unsupported dtype or dtype pairing";
    case PA_ERR_SHAPE: return "invalid shape";
    case PA_ERR_UNSUPPORTED: return "unsupported block size or head dim";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_RANGE: return "scale out of range";
    case PA_ERR_INDEX: return "index data breaks the operation's preconditions (debug mode)";
    default: return "unknown status";
    }
}

const char *pa_last_error(void) { return g_last_error; }

const char *pa_build_info(void) {
    return "libpa gfx950: decode (vector-ALU partition kernel, matrix-core GQA kernel, split-K "
           "reduce), causal chunked prefill (matrix-core), reshape_and_cache (fp32/bf16/fp8-e4m3), "
           "copy_blocks, swap_blocks, device-side index checks";
}

}  // extern "C"
