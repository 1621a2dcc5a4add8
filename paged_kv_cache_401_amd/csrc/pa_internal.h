// pa_internal.h -- launch interfaces shared by the library's translation units.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

enum KvType : int { kF32 = 0, kBF16 = 1, kFP8 = 2 };

constexpr int kBlock = 16;       // tokens per block
constexpr int kThreads = 256;    // threads per workgroup of every kernel (4 wavefronts)
constexpr int kGroupParts = 4;   // partitions per workgroup of the grouped kernel's partition groups

// How the grouped (matrix-core) decode kernel maps work to wavefronts.
enum WaveMode : int {
    kFourWaves = 0,   // one partition per workgroup, four wavefronts taking every 4th block
    kOneWave = 1,     // one partition per one-wavefront workgroup
    kPartGroups = 2,  // kGroupParts consecutive partitions per workgroup, one per wavefront,
                      // merged on chip into one partial result
    kOneWaveDeep = 3, // as kOneWave with three blocks in flight per wavefront (bf16 pools;
                      // 2 waves/SIMD)
};

inline int elem_bytes(int kv) { return kv == kF32 ? 4 : (kv == kBF16 ? 2 : 1); }

struct DecodeParams {
    const void *k_pool;
    const void *v_pool;
    const void *q;             // [S][Hq][D], fp32 for an fp32 pool, bf16 otherwise
    float *out;                // [S][Hq][D]
    const int32_t *block_tables;
    const int32_t *context_lens;
    float *ws_acc;             // [S][Hq][NP][D] partial numerators
    float *ws_m;               // [S][Hq][NP]   partial maxima (log2 domain)
    float *ws_l;               // [S][Hq][NP]   partial denominators
    int32_t num_blocks;
    int32_t num_kv_heads;
    int32_t num_q_heads;
    int32_t group;             // Hq / Hkv
    int32_t num_seqs;
    int32_t max_blocks_per_seq;
    int32_t partition_tokens;  // tokens per partition (multiple of 16)
    int32_t group_parts;       // partitions merged into one partial result (kGroupParts with
                               // kPartGroups, else 1)
    int32_t max_partitions;    // partial results per row: ceil(max_blocks_per_seq * 16 /
                               // (partition_tokens * group_parts))
    int32_t wave_mode;         // grouped kernel: WaveMode
    float qk_scale_log2;       // scale * k_scale * log2(e)
    float out_scale;           // v_scale (1 for 16/32-bit pools)
    int32_t shared_kv;         // blocks shared across sequences: cached, not streaming, loads
    // newest token of every sequence, written by the decode kernel itself to
    // the slot of position context_len - 1 (k_new == nullptr: none)
    const void *k_new;         // [S][Hkv][D] of new_dtype
    const void *v_new;
    int32_t new_dtype;         // kBF16 or kF32 (the pool's dtype unless fp8)
    float inv_k_scale;         // fp32(1 / k_scale), fp8 pools only
    float inv_v_scale;
    // groups of sequences sharing the first blocks of their tables (the
    // shared-prefix kernel only): members of group i are sequences
    // group_start[i] .. group_start[i+1]-1, sharing prefix_blocks[i] blocks
    const int32_t *group_start;   // [num_groups + 1]
    const int32_t *prefix_blocks; // [num_groups]
    int32_t num_groups;
    int32_t max_group;            // members per group at most (max_group * group <= 16)
    int32_t *ws_nparts;           // [num_groups] partitions of each group (split runs only)
};

// Blocks per partition of the shared-prefix kernel at most: a workgroup
// lists its partition's blocks in LDS.
constexpr int kSharedListMax = 512;

struct PrefillParams {
    const void *k_pool;
    const void *v_pool;
    const void *q;             // bf16 [total chunk tokens][Hq][D]
    float *out;                // [total chunk tokens][Hq][D]
    const int32_t *block_tables;
    const int32_t *context_lens;
    const int32_t *query_start;  // [S + 1]
    int32_t num_blocks;
    int32_t num_kv_heads;
    int32_t num_q_heads;
    int32_t group;
    int32_t num_seqs;
    int32_t max_blocks_per_seq;
    int32_t max_query_len;
    int32_t num_tiles;         // ceil(max_query_len / tile tokens)
    float qk_scale_log2;
    float out_scale;
};

struct CacheParams {
    void *k_pool;
    void *v_pool;
    const void *k;
    const void *v;
    const int32_t *slot_mapping;
    int64_t num_tokens;
    int32_t num_blocks;
    int32_t num_kv_heads;
    float inv_k_scale;         // fp32(1 / k_scale), fp8 pools only
    float inv_v_scale;
};

// Timing events of one kernel launch (a measurement aid): when `start` is
// set, the kernel goes out through hipExtLaunchKernel, whose dispatch stores
// the kernel's start and end times in `start` and `stop`.
struct LaunchEvents {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

// Launch `kernel` (one by-value argument) on `stream`, timed by `ev` if given.
template <class P>
inline hipError_t launch_kernel(void (*kernel)(P), dim3 grid, dim3 block, hipStream_t stream,
                                const LaunchEvents *ev, P arg) {
    void *argv[] = {static_cast<void *>(&arg)};
    if (ev && ev->start)
        return hipExtLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, argv, 0, stream,
                                  ev->start, ev->stop, 0);
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, argv, 0, stream);
}

// Each launcher enqueues on `stream` and returns the launch status; the
// partition (and prefill) kernels' launches are timed by `ev` when given.
hipError_t launch_decode_valu(int kv, int head_dim, const DecodeParams &p, hipStream_t stream,
                              const LaunchEvents *ev = nullptr);
hipError_t launch_decode_mfma(int kv, int head_dim, const DecodeParams &p, hipStream_t stream,
                              const LaunchEvents *ev = nullptr);
bool mfma_path_supported(int kv, int head_dim, int group);
hipError_t launch_decode_reduce(int head_dim, const DecodeParams &p, hipStream_t stream);
// decode of prefix-sharing groups (matrix-core), and its split-K merge
hipError_t launch_decode_shared(int kv, int head_dim, const DecodeParams &p, hipStream_t stream,
                                const LaunchEvents *ev = nullptr);
hipError_t launch_decode_shared_reduce(int head_dim, const DecodeParams &p, hipStream_t stream);
// each sequence's newest token (p.k_new / p.v_new) to the slot of position
// context_len - 1, as a kernel of its own
hipError_t launch_append_tokens(int kv, int head_dim, const DecodeParams &p, hipStream_t stream);
bool prefill_supported(int kv, int head_dim, int group);
int prefill_tile_tokens(int head_dim, int group);  // chunk tokens per prefill workgroup
hipError_t launch_prefill(int kv, int head_dim, const PrefillParams &p, hipStream_t stream,
                          const LaunchEvents *ev = nullptr);
hipError_t launch_reshape_and_cache(int pool_kv, int in_kv, int head_dim, const CacheParams &p,
                                    hipStream_t stream);
hipError_t launch_copy_blocks(void *k_pool, void *v_pool, const int32_t *pairs, int32_t num_pairs,
                              int32_t num_blocks, int64_t block_bytes, hipStream_t stream);

hipError_t launch_swap_blocks(void *k_pool, void *v_pool, void *host_k, void *host_v,
                              const int32_t *pairs, int32_t num_pairs, int32_t num_blocks,
                              int32_t num_host_slots, int64_t block_bytes, bool to_host,
                              hipStream_t stream);

// Index checks (pa_check.hip); each fills a report int32[3] on `stream`.
int64_t check_workspace_bytes(int32_t num_blocks, int32_t num_host_slots);
hipError_t launch_check_tables(const int32_t *tables, const int32_t *context_lens, int32_t num_seqs,
                               int32_t max_blocks_per_seq, int32_t num_blocks, int32_t *report,
                               hipStream_t stream);
hipError_t launch_check_query_start(const int32_t *qs, int32_t num_seqs, int32_t *report,
                                    hipStream_t stream);
hipError_t launch_append_slots(const int32_t *tables, const int32_t *context_lens, int32_t num_seqs,
                               int32_t mbs, int32_t num_blocks, int32_t *slots, hipStream_t stream);
hipError_t launch_check_slots(const int32_t *slots, int32_t n, int32_t num_blocks, void *workspace,
                              int32_t *report, hipStream_t stream);
hipError_t launch_check_pairs(const int32_t *pairs, int32_t n, int32_t num_blocks,
                              int32_t num_host_slots, bool swap, void *workspace, int32_t *report,
                              hipStream_t stream);

}  // namespace pa
