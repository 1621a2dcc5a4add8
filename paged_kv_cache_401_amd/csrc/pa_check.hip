// pa_check.hip -- device-side checks of the index data that the other entry
// points read from device memory and trust: context lengths and block tables,
// chunk offsets, slots of a cache write, and block pairs of a copy or swap.
//
// Each check fills a report of three int32 in device memory: the number of
// faults, the OR of their kinds (PA_FAULT_*) and the smallest index of an
// element at fault (sequence, token or pair; -1 when there is none).  Every
// element is judged on its own, so the report does not depend on the order
// in which threads run.  Repeats are found with two bitmaps in a caller's
// workspace: a first atomic OR marks an id as seen, and an OR that finds the
// bit already set marks it as repeated; a second pass then flags every
// element whose id is marked repeated (all of its occurrences).
#include <limits.h>

#include "pa.h"
#include "pa_internal.h"

namespace pa {
namespace {

__device__ __forceinline__ void note_fault(int32_t *report, int kind, int32_t index) {
    atomicAdd(report + 0, 1);
    atomicOr(report + 1, kind);
    atomicMin(report + 2, index);
}

// report = {0 faults, no kinds, no index yet}: lanes 0..2 each write one word
__global__ void report_init_kernel(int32_t *report) {
    const int i = threadIdx.x;
    if (i < 3) report[i] = i == 2 ? INT_MAX : 0;
}

// no fault: the index word becomes -1
__global__ void report_finish_kernel(int32_t *report) {
    const int i = threadIdx.x;
    if (i == 2 && report[i] == INT_MAX) report[i] = -1;
}

__global__ __launch_bounds__(kThreads) void fill_zero_kernel(uint32_t *buf, int64_t words) {
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < words;
         i += (int64_t)gridDim.x * kThreads)
        buf[i] = 0u;
}

// marks id in `seen`; a second visit marks it in `rep`
__device__ __forceinline__ void mark(uint32_t *seen, uint32_t *rep, int64_t id) {
    const uint32_t bit = 1u << (id & 31);
    if (atomicOr(seen + (id >> 5), bit) & bit) atomicOr(rep + (id >> 5), bit);
}

__device__ __forceinline__ bool marked(const uint32_t *bits, int64_t id) {
    return (bits[id >> 5] >> (id & 31)) & 1u;
}

// One workgroup per sequence: its context length must lie in
// [0, max_blocks_per_seq * 16] and the table entries it reads (the first
// ceil(ctx / 16), ctx clamped to that range) in [0, num_blocks).
__global__ __launch_bounds__(kThreads) void check_tables_kernel(const int32_t *tables,
                                                                const int32_t *context_lens,
                                                                int32_t max_blocks_per_seq,
                                                                int32_t num_blocks, int32_t *report) {
    const int s = blockIdx.x;
    const int64_t cap = (int64_t)max_blocks_per_seq * kBlock;
    const int32_t c = context_lens[s];
    if (threadIdx.x == 0 && (c < 0 || c > cap)) note_fault(report, PA_FAULT_CONTEXT_LEN, s);
    const int64_t cc = c < 0 ? 0 : (c > cap ? cap : c);
    const int64_t nb = (cc + kBlock - 1) / kBlock;
    const int32_t *row = tables + (int64_t)s * max_blocks_per_seq;
    int bad = 0;
    for (int64_t j = threadIdx.x; j < nb; j += kThreads) {
        const int32_t b = row[j];
        bad |= b < 0 || b >= num_blocks;
    }
    if (__syncthreads_or(bad) && threadIdx.x == 0) note_fault(report, PA_FAULT_BLOCK_ID, s);
}

// query_start[0] must be 0 and the offsets must not decrease
__global__ __launch_bounds__(kThreads) void check_query_start_kernel(const int32_t *qs,
                                                                     int32_t num_seqs,
                                                                     int32_t *report) {
    for (int64_t s = (int64_t)blockIdx.x * kThreads + threadIdx.x; s <= num_seqs;
         s += (int64_t)gridDim.x * kThreads) {
        const bool bad = s == 0 ? qs[0] != 0 : qs[s] < qs[s - 1];
        if (bad) note_fault(report, PA_FAULT_QUERY_START, (int32_t)s);
    }
}

__global__ __launch_bounds__(kThreads) void mark_slots_kernel(const int32_t *slots, int32_t n,
                                                              int64_t num_slots, uint32_t *seen,
                                                              uint32_t *rep, int32_t *report) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= n) return;
    const int32_t slot = slots[i];
    if (slot < 0) return;  // skipped token
    if (slot >= num_slots)
        note_fault(report, PA_FAULT_SLOT_RANGE, (int32_t)i);
    else
        mark(seen, rep, slot);
}

__global__ __launch_bounds__(kThreads) void repeated_slots_kernel(const int32_t *slots, int32_t n,
                                                                  int64_t num_slots,
                                                                  const uint32_t *rep,
                                                                  int32_t *report) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= n) return;
    const int32_t slot = slots[i];
    if (slot >= 0 && slot < num_slots && marked(rep, slot))
        note_fault(report, PA_FAULT_SLOT_REPEATED, (int32_t)i);
}

// Copy pairs (src, dst): both in [0, num_blocks); destinations distinct and
// never a source.  Swap pairs (block, host slot): block in [0, num_blocks),
// slot in [0, num_host_slots); blocks distinct and slots distinct.
__global__ __launch_bounds__(kThreads) void mark_pairs_kernel(const int32_t *pairs, int32_t n,
                                                              int32_t num_blocks, int32_t second_limit,
                                                              int swap, uint32_t *a_seen,
                                                              uint32_t *a_rep, uint32_t *b_seen,
                                                              uint32_t *b_rep, int32_t *report) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= n) return;
    const int32_t x = pairs[2 * i], y = pairs[2 * i + 1];
    const bool ok = swap ? (x >= 0 && x < num_blocks && y >= 0 && y < second_limit)
                         : (x >= 0 && x < num_blocks && y >= 0 && y < num_blocks);
    if (!ok) {
        note_fault(report, PA_FAULT_PAIR_RANGE, (int32_t)i);
        return;
    }
    if (swap) {
        mark(a_seen, a_rep, x);  // device blocks
        mark(b_seen, b_rep, y);  // host slots
    } else {
        mark(a_seen, a_rep, y);  // destinations
        const uint32_t bit = 1u << (x & 31);
        atomicOr(b_seen + (x >> 5), bit);  // sources
    }
}

__global__ __launch_bounds__(kThreads) void repeated_pairs_kernel(const int32_t *pairs, int32_t n,
                                                                  int32_t num_blocks,
                                                                  int32_t second_limit, int swap,
                                                                  const uint32_t *a_rep,
                                                                  const uint32_t *b_seen,
                                                                  const uint32_t *b_rep,
                                                                  int32_t *report) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= n) return;
    const int32_t x = pairs[2 * i], y = pairs[2 * i + 1];
    const bool ok = swap ? (x >= 0 && x < num_blocks && y >= 0 && y < second_limit)
                         : (x >= 0 && x < num_blocks && y >= 0 && y < num_blocks);
    if (!ok) return;
    if (swap) {
        if (marked(a_rep, x)) note_fault(report, PA_FAULT_DST_REPEATED, (int32_t)i);
        if (marked(b_rep, y)) note_fault(report, PA_FAULT_HOST_SLOT_REPEATED, (int32_t)i);
    } else {
        if (marked(a_rep, y)) note_fault(report, PA_FAULT_DST_REPEATED, (int32_t)i);
        if (marked(b_seen, y)) note_fault(report, PA_FAULT_DST_IS_SRC, (int32_t)i);
    }
}

unsigned grid_for(int64_t n) {
    const int64_t g = (n + kThreads - 1) / kThreads;
    return (unsigned)(g < 1 ? 1 : (g > 65536 ? 65536 : g));
}

int64_t bitmap_words(int64_t ids) { return (ids + 31) / 32; }

hipError_t zero_words(uint32_t *buf, int64_t words, hipStream_t stream) {
    fill_zero_kernel<<<dim3(grid_for(words)), dim3(kThreads), 0, stream>>>(buf, words);
    return hipGetLastError();
}

}  // namespace

// The slot each sequence's newest token goes to in a decode step that writes
// it (position ctx - 1 through the table): -1 for an empty context or a
// table entry outside the pool (the step writes nothing there; the tables
// check reports the entry).
__global__ __launch_bounds__(kThreads) void append_slots_kernel(const int32_t *tables,
                                                                const int32_t *context_lens,
                                                                int32_t num_seqs, int32_t mbs,
                                                                int32_t num_blocks, int32_t *slots) {
    const int64_t s = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (s >= num_seqs) return;
    int64_t c = context_lens[s];
    c = c < 0 ? 0 : (c > (int64_t)mbs * kBlock ? (int64_t)mbs * kBlock : c);
    int32_t slot = -1;
    if (c > 0) {
        const int32_t b = tables[s * mbs + (c - 1) / kBlock];
        if (b >= 0 && b < num_blocks) slot = b * kBlock + (int32_t)((c - 1) % kBlock);
    }
    slots[s] = slot;
}

int64_t check_workspace_bytes(int32_t num_blocks, int32_t num_host_slots) {
    const int64_t slots = 2 * bitmap_words((int64_t)num_blocks * kBlock);
    const int64_t copy = 3 * bitmap_words(num_blocks);
    const int64_t swap = 2 * bitmap_words(num_blocks) + 2 * bitmap_words(num_host_slots);
    int64_t w = slots > copy ? slots : copy;
    w = w > swap ? w : swap;
    return ((w * 4 + 255) / 256) * 256;
}

hipError_t launch_check_tables(const int32_t *tables, const int32_t *context_lens, int32_t num_seqs,
                               int32_t max_blocks_per_seq, int32_t num_blocks, int32_t *report,
                               hipStream_t stream) {
    report_init_kernel<<<1, 64, 0, stream>>>(report);
    if (num_seqs > 0)
        check_tables_kernel<<<dim3((unsigned)num_seqs), dim3(kThreads), 0, stream>>>(
            tables, context_lens, max_blocks_per_seq, num_blocks, report);
    report_finish_kernel<<<1, 64, 0, stream>>>(report);
    return hipGetLastError();
}

hipError_t launch_check_query_start(const int32_t *qs, int32_t num_seqs, int32_t *report,
                                    hipStream_t stream) {
    report_init_kernel<<<1, 64, 0, stream>>>(report);
    check_query_start_kernel<<<dim3(grid_for((int64_t)num_seqs + 1)), dim3(kThreads), 0, stream>>>(
        qs, num_seqs, report);
    report_finish_kernel<<<1, 64, 0, stream>>>(report);
    return hipGetLastError();
}

hipError_t launch_check_slots(const int32_t *slots, int32_t n, int32_t num_blocks, void *workspace,
                              int32_t *report, hipStream_t stream) {
    const int64_t num_slots = (int64_t)num_blocks * kBlock;
    const int64_t w = bitmap_words(num_slots);
    uint32_t *seen = static_cast<uint32_t *>(workspace), *rep = seen + w;
    report_init_kernel<<<1, 64, 0, stream>>>(report);
    hipError_t e = zero_words(seen, 2 * w, stream);
    if (e != hipSuccess) return e;
    if (n > 0) {
        const unsigned g = (unsigned)(((int64_t)n + kThreads - 1) / kThreads);
        mark_slots_kernel<<<dim3(g), dim3(kThreads), 0, stream>>>(slots, n, num_slots, seen, rep, report);
        repeated_slots_kernel<<<dim3(g), dim3(kThreads), 0, stream>>>(slots, n, num_slots, rep, report);
    }
    report_finish_kernel<<<1, 64, 0, stream>>>(report);
    return hipGetLastError();
}

hipError_t launch_append_slots(const int32_t *tables, const int32_t *context_lens, int32_t num_seqs,
                               int32_t mbs, int32_t num_blocks, int32_t *slots, hipStream_t stream) {
    if (num_seqs <= 0) return hipSuccess;
    const unsigned g = (unsigned)(((int64_t)num_seqs + kThreads - 1) / kThreads);
    append_slots_kernel<<<dim3(g), dim3(kThreads), 0, stream>>>(tables, context_lens, num_seqs, mbs,
                                                                 num_blocks, slots);
    return hipGetLastError();
}

hipError_t launch_check_pairs(const int32_t *pairs, int32_t n, int32_t num_blocks,
                              int32_t num_host_slots, bool swap, void *workspace, int32_t *report,
                              hipStream_t stream) {
    const int64_t wb = bitmap_words(num_blocks);
    const int64_t ws = swap ? bitmap_words(num_host_slots) : wb;
    uint32_t *a_seen = static_cast<uint32_t *>(workspace), *a_rep = a_seen + wb;
    uint32_t *b_seen = a_rep + wb, *b_rep = b_seen + ws;
    report_init_kernel<<<1, 64, 0, stream>>>(report);
    hipError_t e = zero_words(a_seen, 2 * wb + (swap ? 2 * ws : ws), stream);
    if (e != hipSuccess) return e;
    if (n > 0) {
        const unsigned g = (unsigned)(((int64_t)n + kThreads - 1) / kThreads);
        mark_pairs_kernel<<<dim3(g), dim3(kThreads), 0, stream>>>(pairs, n, num_blocks, num_host_slots,
                                                                   swap ? 1 : 0, a_seen, a_rep, b_seen,
                                                                   b_rep, report);
        repeated_pairs_kernel<<<dim3(g), dim3(kThreads), 0, stream>>>(
            pairs, n, num_blocks, num_host_slots, swap ? 1 : 0, a_rep, b_seen, b_rep, report);
    }
    report_finish_kernel<<<1, 64, 0, stream>>>(report);
    return hipGetLastError();
}

}  // namespace pa
