// pa_mfma_util.h -- operand helpers shared by the matrix-core kernels
// (grouped-query decode and prefill) for gfx950's v_mfma_f32_16x16x32_bf16.
//
// Operand layouts of that instruction (lane = 16 c + n):
//   A (16 x 32): lane holds A[row n][8 c .. 8 c + 7]
//   B (32 x 16): lane holds B[8 c .. 8 c + 7][column n]
//   C (16 x 16): lane holds C[4 c .. 4 c + 3][column n]
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr float kNegInfF = -__builtin_inff();

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }
// two words of bf16 pairs as the 4-element operand of a 16-deep matrix-core product
typedef short bf16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4 as_bf16x4(uint32_t w0, uint32_t w1) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(bf16x4, u32x2{w0, w1});
}

// 16-byte load marked non-temporal: decode reads every K/V byte once, and on
// MI355X streaming reads sustain ~7.1 TB/s this way against ~6.4 TB/s with
// ordinary loads (a 4 KiB random-tile gather: 6.86 against 6.12 TB/s)
__device__ __forceinline__ u32x4 load_stream(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// K/V load with the decode kernels' cache policy: non-temporal when every
// byte is read once (STREAM), an ordinary cached load when blocks are shared
// by several sequences whose workgroups run together (shared prompts), so
// that later readers find them in cache
template <bool STREAM>
__device__ __forceinline__ u32x4 load_kv(const void *p) {
    if constexpr (STREAM)
        return load_stream(p);
    else
        return *reinterpret_cast<const u32x4 *>(p);
}

// Buffer resource covering one pool tile: loads through it are bounds-checked
// by the hardware, and a resource of size 0 turns every load into a zero
// that touches no memory.  The decode loop issues the same loads every
// iteration through such resources -- past the end of a wavefront's blocks,
// or for a block id outside the pool, the size is 0 -- so the compiler can
// count the loads still in flight exactly, where loads behind branches make
// it wait for all of them.  Word 3 selects a 32-bit data format (required for
// untyped buffer loads on this architecture).
constexpr int kBufWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void *tile, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(tile), 0, bytes, kBufWord3);
}

// 16-byte load at byte offset `off` of a tile resource, non-temporal when
// STREAM (the cache policy of load_kv)
template <bool STREAM>
__device__ __forceinline__ u32x4 load_tile(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, STREAM ? 2 : 0));
}

// 8- and 4-byte loads at byte offset `off` of a tile resource (cached)
__device__ __forceinline__ uint2 load_tile_b64(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t load_tile_b32(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// Reductions over lanes i and i ^ 16, and i and i ^ 32, with gfx950's
// cross-row lane swaps: no LDS traffic, unlike a shuffle through
// ds_bpermute.  Applied to two copies of x, a swap leaves x_i in one and
// x_(i^16) (or x_(i^32)) in the other, in an order that differs between
// rows; max and + do not depend on it.
__device__ __forceinline__ float max_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Longest-first work order for small batches.  Workgroups are dispatched in
// index order, so the sequence a workgroup takes is the one whose rank, by
// context length descending (ties by index), is its sequence slot `r`: long
// contexts start first and short ones fill the end (on MI355X a 32-sequence
// batch with lengths uniform in [1, 2048] decodes 9 % faster this way).  One
// wavefront ranks up to 64 sequences with a 64-step comparison loop; larger
// batches keep index order.  Every lane returns the same sequence.
constexpr int kOrderMaxSeqs = 64;
__device__ __forceinline__ int sequence_of_rank(const int32_t *context_lens, int num_seqs, int cap,
                                                int r) {
    if (num_seqs <= 1 || num_seqs > kOrderMaxSeqs) return r;
    const int lane = threadIdx.x & 63;
    int mine = -1;
    if (lane < num_seqs) {
        mine = context_lens[lane];
        mine = mine < 0 ? 0 : (mine > cap ? cap : mine);
    }
    int rank = 0;
    for (int j = 0; j < num_seqs; ++j) {
        const int cj = __builtin_amdgcn_readlane(mine, j);
        rank += (cj > mine || (cj == mine && j < lane)) ? 1 : 0;
    }
    const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < num_seqs && rank == r);
    return hit ? (int)__builtin_ctzll(hit) : r;
}

// The work item of this workgroup in a grid of rows x max_partitions: the
// first `rows` workgroups take partition 0 of rows 0..rows-1; workgroup
// rows + j takes row j / (max_partitions - 1), partition
// 1 + (j % (max_partitions - 1) + row) % (max_partitions - 1).
__device__ __forceinline__ void pair_and_partition(int rows, int max_partitions, int &row, int &part) {
    const int i = (int)blockIdx.x;
    if (i < rows) {
        row = i;
        part = 0;
    } else {
        const int j = i - rows;
        const int m = max_partitions - 1;
        row = j / m;
        part = 1 + (j % m + row) % m;
    }
}

// four fp8 E4M3FN codes (one word) -> four bf16 in two words (exact):
// lo = codes 0, 1 and hi = codes 2, 3
__device__ __forceinline__ void e4m3x4_to_bf16(uint32_t w, uint32_t &lo, uint32_t &hi) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
    lo = __builtin_bit_cast(uint32_t, a);
    hi = __builtin_bit_cast(uint32_t, b);
}

// p = hi + lo with hi = p truncated to bf16 and lo = the remainder truncated
// to bf16: together they carry p to 16 significant bits
__device__ __forceinline__ void split_bf16(float p, uint32_t &hi, uint32_t &lo) {
    const uint32_t u = __float_as_uint(p);
    hi = u >> 16;
    lo = __float_as_uint(p - __uint_as_float(u & 0xffff0000u)) >> 16;
}

// P^T as [hi(p0..p3) | lo(p0..p3)]: the words of the two 16-deep operands
// (hi, lo) of the P.V product, or of a 32-deep one against [V | V]
__device__ __forceinline__ bf16x8 p_operand_hi_lo(const float (&pr)[4]) {
    uint32_t h0, l0, h1, l1, h2, l2, h3, l3;
    split_bf16(pr[0], h0, l0);
    split_bf16(pr[1], h1, l1);
    split_bf16(pr[2], h2, l2);
    split_bf16(pr[3], h3, l3);
    u32x4 pw;
    pw[0] = h0 | (h1 << 16);
    pw[1] = h2 | (h3 << 16);
    pw[2] = l0 | (l1 << 16);
    pw[3] = l2 | (l3 << 16);
    return as_bf16x8(pw);
}

// Keep masks for the bf16 pairs (tokens 4c, 4c+1) and (4c+2, 4c+3) of a V
// cell: all ones for tokens below `nvalid`, zero above
__device__ __forceinline__ void v_keep_masks(int c, int nvalid, uint32_t &keep01, uint32_t &keep23) {
    keep01 = (4 * c + 0 < nvalid ? 0x0000ffffu : 0u) | (4 * c + 1 < nvalid ? 0xffff0000u : 0u);
    keep23 = (4 * c + 2 < nvalid ? 0x0000ffffu : 0u) | (4 * c + 3 < nvalid ? 0xffff0000u : 0u);
}

}  // namespace pa
