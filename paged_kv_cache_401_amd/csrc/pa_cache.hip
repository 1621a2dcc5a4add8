// pa_cache.hip -- the kernels that keep the paged pool consistent, and the
// block swap between the device pool and host memory.
//
// reshape_and_cache: each new token's K/V goes to slot `slot % 16` of block
// `slot / 16` (the slot rule of the worked example on the "PagedAttention"
// glossary page, how paging works; only the new token's K/V is appended, as
// the French page's second article, "what is the KV cache", describes).
// copy_blocks: the copy-on-write step of the same glossary page's section on
// sharing blocks between sequences.
// swap_blocks: fine-grained eviction -- when memory runs short, small blocks
// move to CPU memory instead of whole sequences (French page, "how
// PagedAttention solves this problem").
#include "pa_internal.h"

namespace pa {
namespace {

// fp32 -> OCP E4M3FN with round-to-nearest-even and saturation to +-448,
// done on the bit pattern: NaN keeps its sign as S.1111.111; magnitudes at or
// above 448 (infinity included) become 448; normal results keep the top three
// mantissa bits and round on the remaining twenty; results below 2^-6 are
// multiples of 2^-9 rounded from the full 24-bit significand.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return sign | 0x7fu;        // NaN
    if (a >= 0x43e00000u) return sign | 0x7eu;       // |x| >= 448
    const uint32_t e = a >> 23;                      // biased fp32 exponent
    if (e >= 121u) {                                 // |x| >= 2^-6: normal E4M3
        const uint32_t mant = a & 0x7fffffu;
        uint32_t code = ((e - 120u) << 3) | (mant >> 20);
        const uint32_t rest = mant & 0xfffffu;
        if (rest > 0x80000u || (rest == 0x80000u && (code & 1u))) code += 1u;
        return sign | code;
    }
    if (e == 0u) return sign;                        // fp32 subnormal: rounds to 0
    const uint32_t sig = (a & 0x7fffffu) | 0x800000u; // value = sig * 2^(e - 150)
    const uint32_t shift = 141u - e;                 // code = value * 2^9 = sig >> shift
    if (shift >= 32u) return sign;
    uint32_t code = sig >> shift;
    const uint32_t rest = sig & ((1u << shift) - 1u);
    const uint32_t half = 1u << (shift - 1u);
    if (rest > half || (rest == half && (code & 1u))) code += 1u;
    return sign | code;
}

template <int IN>
__device__ __forceinline__ float load_in(const void *base, int64_t idx) {
    if constexpr (IN == kF32) {
        return reinterpret_cast<const float *>(base)[idx];
    } else {
        const uint32_t h = reinterpret_cast<const uint16_t *>(base)[idx];
        return __uint_as_float(h << 16);
    }
}

// One thread per (token, KV head, head-dim element).
template <int POOL, int IN, int D>
__global__ __launch_bounds__(kThreads) void reshape_and_cache_kernel(CacheParams p) {
    constexpr int EB = POOL == kF32 ? 4 : (POOL == kBF16 ? 2 : 1);
    constexpr int X = 16 / EB;   // K: elements per 16-byte run
    constexpr int W = 4 / EB;    // V: head-dim elements per 16-byte cell
    const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t total = p.num_tokens * p.num_kv_heads * D;
    if (idx >= total) return;
    const int d = (int)(idx % D);
    const int64_t row = idx / D;
    const int g = (int)(row % p.num_kv_heads);
    const int64_t tok = row / p.num_kv_heads;
    const int32_t slot = p.slot_mapping[tok];
    if (slot < 0) return;
    const int64_t b = slot >> 4;
    const int t = slot & 15;
    if (b >= p.num_blocks) return;
    const int64_t tile = (b * p.num_kv_heads + g) * (int64_t)(kBlock * D);
    const int64_t ko = tile + ((d / X) * kBlock + t) * X + (d % X);
    const int64_t vo = tile + ((t >> 2) * (D / W) + d / W) * (4 * W) + (d % W) * 4 + (t & 3);
    if constexpr (POOL == kFP8) {
        const float xk = load_in<IN>(p.k, idx) * p.inv_k_scale;
        const float xv = load_in<IN>(p.v, idx) * p.inv_v_scale;
        reinterpret_cast<uint8_t *>(p.k_pool)[ko] = (uint8_t)f32_to_e4m3(xk);
        reinterpret_cast<uint8_t *>(p.v_pool)[vo] = (uint8_t)f32_to_e4m3(xv);
    } else if constexpr (POOL == kBF16) {
        reinterpret_cast<uint16_t *>(p.k_pool)[ko] = reinterpret_cast<const uint16_t *>(p.k)[idx];
        reinterpret_cast<uint16_t *>(p.v_pool)[vo] = reinterpret_cast<const uint16_t *>(p.v)[idx];
    } else {
        reinterpret_cast<uint32_t *>(p.k_pool)[ko] = reinterpret_cast<const uint32_t *>(p.k)[idx];
        reinterpret_cast<uint32_t *>(p.v_pool)[vo] = reinterpret_cast<const uint32_t *>(p.v)[idx];
    }
}

// Workgroup (pair, pool, part): 16-byte copies of one part of the whole block
// (all KV heads), U x 4 KiB per part; each thread issues its U loads before
// its stores.  Source and destination never overlap (destinations are
// distinct and none is a source).  Measured on MI355X: whole 32 KiB blocks
// per workgroup (U = 8) are fastest for a few hundred pairs, 16 KiB parts
// (U = 4) once thousands of pairs fill the chip.
template <int U>
__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(char *k_pool, char *v_pool,
                                                               const int32_t *pairs,
                                                               int32_t num_blocks,
                                                               int64_t block_bytes) {
    const int32_t src = pairs[2 * blockIdx.x];
    const int32_t dst = pairs[2 * blockIdx.x + 1];
    if (src < 0 || dst < 0 || src >= num_blocks || dst >= num_blocks) return;
    char *base = blockIdx.y ? v_pool : k_pool;
    const uint4 *__restrict__ s = reinterpret_cast<const uint4 *>(base + (int64_t)src * block_bytes);
    uint4 *__restrict__ d = reinterpret_cast<uint4 *>(base + (int64_t)dst * block_bytes);
    const int64_t n = block_bytes / 16;
    const int64_t i0 = (int64_t)blockIdx.z * kThreads * U;
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t i = i0 + (int64_t)u * kThreads + threadIdx.x;
        if (i < n) v[u] = s[i];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t i = i0 + (int64_t)u * kThreads + threadIdx.x;
        if (i < n) d[i] = v[u];
    }
}

template <int U>
hipError_t launch_copy(void *k_pool, void *v_pool, const int32_t *pairs, int32_t num_pairs,
                       int32_t num_blocks, int64_t block_bytes, hipStream_t stream) {
    const int64_t part = (int64_t)kThreads * U * 16;
    const int64_t parts = (block_bytes + part - 1) / part;
    if (parts > 65535) return hipErrorInvalidValue;
    copy_blocks_kernel<U><<<dim3((unsigned)num_pairs, 2, (unsigned)parts), dim3(kThreads), 0, stream>>>(
        static_cast<char *>(k_pool), static_cast<char *>(v_pool), pairs, num_blocks, block_bytes);
    return hipGetLastError();
}

// Workgroup (pair, pool, part) of a block swap: one 8 KiB part of a whole
// block (all KV heads) between the device pool and the host pool.  Swap-out
// reads the device block and writes host slot bytes over the host link;
// swap-in reads host slot bytes and writes the device block.  Each thread
// issues all its loads before its stores: host reads are long round trips.
constexpr int kSwapUnroll = 4;
constexpr int64_t kSwapPartBytes = (int64_t)kThreads * kSwapUnroll * 16;  // 16 KiB

__global__ __launch_bounds__(kThreads) void swap_blocks_kernel(char *k_pool, char *v_pool,
                                                               char *host_k, char *host_v,
                                                               const int32_t *pairs,
                                                               int32_t num_blocks,
                                                               int32_t num_host_slots,
                                                               int64_t block_bytes, int to_host) {
    const int32_t b = pairs[2 * blockIdx.x];
    const int32_t h = pairs[2 * blockIdx.x + 1];
    if (b < 0 || h < 0 || b >= num_blocks || h >= num_host_slots) return;
    char *dev = (blockIdx.y ? v_pool : k_pool) + (int64_t)b * block_bytes;
    char *hst = (blockIdx.y ? host_v : host_k) + (int64_t)h * block_bytes;
    const uint4 *__restrict__ s = reinterpret_cast<const uint4 *>(to_host ? dev : hst);
    uint4 *__restrict__ d = reinterpret_cast<uint4 *>(to_host ? hst : dev);
    const int64_t n = block_bytes / 16;
    const int64_t i0 = (int64_t)blockIdx.z * (kSwapPartBytes / 16);
    uint4 v[kSwapUnroll];
#pragma unroll
    for (int u = 0; u < kSwapUnroll; ++u) {
        const int64_t i = i0 + (int64_t)u * kThreads + threadIdx.x;
        if (i < n) v[u] = s[i];
    }
#pragma unroll
    for (int u = 0; u < kSwapUnroll; ++u) {
        const int64_t i = i0 + (int64_t)u * kThreads + threadIdx.x;
        if (i < n) d[i] = v[u];
    }
}

template <int POOL, int IN, int D>
hipError_t launch_rc(const CacheParams &p, hipStream_t stream) {
    const int64_t total = p.num_tokens * p.num_kv_heads * D;
    const int64_t blocks = (total + kThreads - 1) / kThreads;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    reshape_and_cache_kernel<POOL, IN, D><<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(p);
    return hipGetLastError();
}

template <int POOL, int IN>
hipError_t launch_rc_d(int head_dim, const CacheParams &p, hipStream_t stream) {
    return head_dim == 64 ? launch_rc<POOL, IN, 64>(p, stream) : launch_rc<POOL, IN, 128>(p, stream);
}

}  // namespace

hipError_t launch_reshape_and_cache(int pool_kv, int in_kv, int head_dim, const CacheParams &p,
                                    hipStream_t stream) {
    if (pool_kv == kF32) return launch_rc_d<kF32, kF32>(head_dim, p, stream);
    if (pool_kv == kBF16) return launch_rc_d<kBF16, kBF16>(head_dim, p, stream);
    if (in_kv == kBF16) return launch_rc_d<kFP8, kBF16>(head_dim, p, stream);
    return launch_rc_d<kFP8, kF32>(head_dim, p, stream);
}

hipError_t launch_copy_blocks(void *k_pool, void *v_pool, const int32_t *pairs, int32_t num_pairs,
                              int32_t num_blocks, int64_t block_bytes, hipStream_t stream) {
    if (num_pairs < 1024)
        return launch_copy<8>(k_pool, v_pool, pairs, num_pairs, num_blocks, block_bytes, stream);
    return launch_copy<4>(k_pool, v_pool, pairs, num_pairs, num_blocks, block_bytes, stream);
}

hipError_t launch_swap_blocks(void *k_pool, void *v_pool, void *host_k, void *host_v,
                              const int32_t *pairs, int32_t num_pairs, int32_t num_blocks,
                              int32_t num_host_slots, int64_t block_bytes, bool to_host,
                              hipStream_t stream) {
    const int64_t parts = (block_bytes + kSwapPartBytes - 1) / kSwapPartBytes;
    if (parts > 65535) return hipErrorInvalidValue;
    swap_blocks_kernel<<<dim3((unsigned)num_pairs, 2, (unsigned)parts), dim3(kThreads), 0, stream>>>(
        static_cast<char *>(k_pool), static_cast<char *>(v_pool), static_cast<char *>(host_k),
        static_cast<char *>(host_v), pairs, num_blocks, num_host_slots, block_bytes, to_host ? 1 : 0);
    return hipGetLastError();
}

}  // namespace pa
