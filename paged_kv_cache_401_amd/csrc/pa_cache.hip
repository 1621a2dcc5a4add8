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
#include "pa_store.h"

#include <type_traits>

namespace pa {
namespace {

// One 16-byte K run of one token -- head dims r X .. r X + X - 1, X = 16 /
// pool element bytes -- and the same dims of V, to the token's slot.  Both
// inputs are read with vector loads before anything is stored, so a thread
// makes one round trip to memory; the K run goes out as one 16-byte store,
// the V elements (spread over the cells of the token's 4-token group) one by
// one.  Stores are non-temporal, as for single elements.
template <int POOL, int IN, int D>
__device__ __forceinline__ void write_run(const CacheParams &p, int64_t tok, int g, int r, int32_t slot) {
    typedef uint32_t w4 __attribute__((ext_vector_type(4)));
    constexpr int EB = POOL == kF32 ? 4 : (POOL == kBF16 ? 2 : 1);
    constexpr int IB = IN == kF32 ? 4 : 2;
    constexpr int X = 16 / EB;                      // elements per K run
    constexpr int W = 4 / EB;                       // V: dims per 16-byte cell
    constexpr int NU = X * IB / 16;                 // 16-byte input units per run
    if (slot < 0) return;
    const int64_t b = slot >> 4;
    if (b >= p.num_blocks) return;
    const int t = slot & 15;
    const int64_t e = (tok * p.num_kv_heads + g) * D + r * X;   // first input element
    w4 kin[NU], vin[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        kin[u] = reinterpret_cast<const w4 *>(static_cast<const char *>(p.k) + e * IB)[u];
        vin[u] = reinterpret_cast<const w4 *>(static_cast<const char *>(p.v) + e * IB)[u];
    }
    // input element j of the run as pool bits
    auto elem = [&](const w4 (&in)[NU], int j, float inv) -> uint32_t {
        uint32_t word;
        if constexpr (IN == kF32) word = in[j / 4][j % 4];
        else word = (in[j / 8][(j % 8) / 2] >> (16 * (j % 2))) & 0xffffu;
        if constexpr (POOL == kFP8)
            return f32_to_e4m3((IN == kF32 ? __uint_as_float(word) : __uint_as_float(word << 16)) * inv);
        else
            return word;
    };
    const int64_t tile = (b * p.num_kv_heads + g) * (int64_t)(kBlock * D);   // elements
    w4 kw;
    if constexpr (POOL == kFP8) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            kw[q] = elem(kin, 4 * q, p.inv_k_scale) | (elem(kin, 4 * q + 1, p.inv_k_scale) << 8) |
                    (elem(kin, 4 * q + 2, p.inv_k_scale) << 16) | (elem(kin, 4 * q + 3, p.inv_k_scale) << 24);
    } else {
        kw = kin[0];
    }
    __builtin_nontemporal_store(kw, reinterpret_cast<w4 *>(static_cast<char *>(p.k_pool) +
                                                           (tile + (int64_t)(r * kBlock + t) * X) * EB));
#pragma unroll
    for (int j = 0; j < X; ++j) {
        const int d = r * X + j;
        const int64_t vo = tile + ((t >> 2) * (D / W) + d / W) * (4 * W) + (d % W) * 4 + (t & 3);
        const uint32_t vraw = elem(vin, j, p.inv_v_scale);
        if constexpr (POOL == kFP8)
            __builtin_nontemporal_store((uint8_t)vraw, static_cast<uint8_t *>(p.v_pool) + vo);
        else if constexpr (POOL == kBF16)
            __builtin_nontemporal_store((uint16_t)vraw, static_cast<uint16_t *>(p.v_pool) + vo);
        else
            __builtin_nontemporal_store(vraw, static_cast<uint32_t *>(p.v_pool) + vo);
    }
}

// Four consecutive input elements starting at element `idx` as fp8 codes
// (byte i = element i), each scaled by `inv` and rounded as f32_to_e4m3 does.
template <int IN>
__device__ __forceinline__ uint32_t encode4(const void *base, int64_t idx, float inv) {
    float x[4];
    if constexpr (IN == kF32) {
        const float4 v = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(base) + idx);
        x[0] = v.x, x[1] = v.y, x[2] = v.z, x[3] = v.w;
    } else {
        const uint2 v = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(base) + idx);
        x[0] = __uint_as_float(v.x << 16), x[1] = __uint_as_float(v.x & 0xffff0000u);
        x[2] = __uint_as_float(v.y << 16), x[3] = __uint_as_float(v.y & 0xffff0000u);
    }
    return f32x4_to_e4m3(x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv);
}

// Workgroup (window of 16 input tokens, up to HPW KV heads).  A run is 16
// consecutive input tokens whose slots are one whole block in order
// (16 b .. 16 b + 15: a prompt written block by block).  The workgroup of the
// window holding a run's first token writes that block's K and V tiles of
// its heads with 16-byte stores: K unit (run r, token t) is the 16-byte run r
// of token t's input row (converted for an fp8 pool), V cell (token group tg,
// dims W dw ..) is gathered from four tokens' inputs -- for a bf16 pool two
// neighbouring cells at once, from 8-byte loads of four dims.  Each thread
// issues all its loads before its first store.  (The loads are ordinary
// ones: several work items read parts of one input line.)  Tokens of the window that no
// run covers go to their slots one K run per thread (write_run: a decode
// step's tokens, each in a different sequence, or the partial last block of
// a prompt).  Runs are found by every wavefront alike: lane l looks at token
// w0 - 16 + l, and ballots mark the tokens whose slot follows the previous
// one's.
template <int POOL, int IN, int D, int HPW>
__global__ __launch_bounds__(kThreads) void reshape_and_cache_kernel(CacheParams p) {
    constexpr int EB = POOL == kF32 ? 4 : (POOL == kBF16 ? 2 : 1);
    constexpr int IB = IN == kF32 ? 4 : 2;          // input bytes per element
    constexpr int X = 16 / EB;                      // K: elements per 16-byte run
    constexpr int W = 4 / EB;                       // V: dims per 16-byte cell
    constexpr int K_UNITS = kBlock * D * EB / 16;   // 16-byte units of one tile
    const int64_t w0 = (int64_t)blockIdx.x * kBlock;
    const int g0 = blockIdx.y * HPW;
    const int nh = p.num_kv_heads - g0 < HPW ? p.num_kv_heads - g0 : HPW;  // heads of this workgroup
    const int lane = threadIdx.x & 63;

    const int64_t tok = w0 - kBlock + lane;
    const int32_t v = tok >= 0 && tok < p.num_tokens ? p.slot_mapping[tok] : -2;
    const int32_t nxt = __shfl_down(v, 1);
    const uint64_t follows = __builtin_amdgcn_ballot_w64(lane < 63 && v >= 0 && (uint32_t)nxt == (uint32_t)v + 1u);
    const bool start = v >= 0 && (v & 15) == 0 && (v >> 4) < p.num_blocks && lane <= 48 &&
                       ((follows >> lane) & 0x7fffull) == 0x7fffull;
    const uint64_t starts = __builtin_amdgcn_ballot_w64(start);
    // window tokens (lanes 16..31) covered by a run starting at lane 1..31
    uint64_t covered = 0;
    for (uint64_t m = starts & 0xfffffffeull; m != 0; m &= m - 1) covered |= 0xffffull << __builtin_ctzll(m);
    const uint32_t cov = (uint32_t)(covered >> 16) & 0xffffu;
    const uint32_t mine = (uint32_t)(starts >> 16) & 0xffffu;

    const int64_t nt = p.num_tokens - w0 < kBlock ? p.num_tokens - w0 : kBlock;
    constexpr int NR = D / X;                        // K runs per token and head
    // A grid of depth 2 splits each window's tiles: z = 0 writes the K tiles
    // (and the lone tokens), z = 1 the V tiles.
    const bool do_k = blockIdx.z == 0, do_v = blockIdx.z == 1 || gridDim.z == 1;
    for (int e = threadIdx.x; do_k && e < nt * NR * nh; e += kThreads) {
        const int t = e / (NR * nh), hh = (e / NR) % nh, r = e % NR;
        if (!((cov >> t) & 1u)) write_run<POOL, IN, D>(p, w0 + t, g0 + hh, r, p.slot_mapping[w0 + t]);
    }
    if (!mine) return;
    const int64_t i0 = w0 + __builtin_ctz(mine);    // the run's first token
    const int32_t s0 = p.slot_mapping[i0];
    const int64_t step = (int64_t)p.num_kv_heads * D;  // next token, same head and dim
    // first input element of token t, head hh
    auto row = [&](int t, int hh) { return (i0 + t) * step + (int64_t)(g0 + hh) * D; };
    // pool unit u of head hh's tile
    auto unit = [&](void *pool, int hh, int u) {
        return reinterpret_cast<uint4 *>(pool) + ((int64_t)(s0 >> 4) * p.num_kv_heads + g0 + hh) * K_UNITS + u;
    };

    // The tiles in three phases -- every thread's input loads, then the
    // conversions (whose fp8 NaN test may branch), then the 16-byte stores --
    // so all loads are in flight before the first one is waited for.  FULL:
    // all HPW heads present (the usual case).
    constexpr int CPI = POOL == kBF16 ? 2 : 1;       // V cells per work item
    constexpr int VU = K_UNITS / CPI;                // V work items per tile
    constexpr int KI = (HPW * K_UNITS + kThreads - 1) / kThreads;
    constexpr int VI = (HPW * VU + kThreads - 1) / kThreads;
    constexpr int NKU = X * IB / 16;                 // 16-byte input units per K unit
    constexpr int VB = W * CPI * IB;                 // input bytes per token of a V item
    using VWord = typename std::conditional<VB == 4, uint32_t,
                  typename std::conditional<VB == 8, uint2, uint4>::type>::type;
    auto tiles = [&](auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        // every item of the K (V) loops exists: all heads present, and the
        // items a multiple of the workgroup's threads
        constexpr bool KFULL = FULL && (HPW * K_UNITS) % kThreads == 0;
        constexpr bool VFULL = FULL && (HPW * VU) % kThreads == 0;
        // K item i = hh * K_UNITS + (r * 16 + t); V item i = hh * VU +
        // (tg * (D / W / CPI) + q), cells CPI q .. CPI q + CPI - 1 of token group tg
        auto k_in = [&](int i) {
            const int hh = i / K_UNITS, u = i % K_UNITS;
            return row(u % kBlock, hh) + (u / kBlock) * X;
        };
        auto v_in = [&](int i) {
            const int hh = i / VU, u = i % VU;
            return row(4 * (u / (D / W / CPI)), hh) + W * CPI * (u % (D / W / CPI));
        };
        uint4 kr[KI][NKU];
        VWord vr[VI][4];
#pragma unroll
        for (int j = 0; j < KI; ++j) {
            const int i = threadIdx.x + j * kThreads;
            if (!do_k || (!KFULL && i >= nh * K_UNITS)) break;
            const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const char *>(p.k) + k_in(i) * IB);
#pragma unroll
            for (int c = 0; c < NKU; ++c) kr[j][c] = src[c];
        }
#pragma unroll
        for (int j = 0; j < VI; ++j) {
            const int i = threadIdx.x + j * kThreads;
            if (!do_v || (!VFULL && i >= nh * VU)) break;
            const int64_t e = v_in(i);
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
                vr[j][tt] = *reinterpret_cast<const VWord *>(static_cast<const char *>(p.v) + (e + tt * step) * IB);
        }
        uint4 kw[KI], vw[VI][CPI];
#pragma unroll
        for (int j = 0; j < KI; ++j) {
            if constexpr (POOL == kFP8) {
                uint32_t c4[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {  // input elements 4 q .. 4 q + 3
                    float x[4];
#pragma unroll
                    for (int z = 0; z < 4; ++z) {
                        const int el = 4 * q + z;
                        if constexpr (IN == kF32) {
                            x[z] = __uint_as_float(kr[j][el / 4][el % 4]);
                        } else {
                            const uint32_t wd = kr[j][el / 8][(el % 8) / 2];
                            x[z] = __uint_as_float(el % 2 ? wd & 0xffff0000u : wd << 16);
                        }
                        x[z] *= p.inv_k_scale;
                    }
                    c4[q] = f32x4_to_e4m3(x[0], x[1], x[2], x[3]);
                }
                kw[j] = uint4{c4[0], c4[1], c4[2], c4[3]};
            } else {
                kw[j] = kr[j][0];
            }
        }
#pragma unroll
        for (int j = 0; j < VI; ++j) {
            if constexpr (POOL == kFP8) {  // word j: tokens 0..3 of dim 4 q + j
                uint32_t c[4];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    float x[4];
#pragma unroll
                    for (int z = 0; z < 4; ++z) {
                        if constexpr (IN == kF32) {
                            x[z] = __uint_as_float(vr[j][tt][z]);
                        } else {
                            const uint32_t wd = z < 2 ? vr[j][tt].x : vr[j][tt].y;
                            x[z] = __uint_as_float(z % 2 ? wd & 0xffff0000u : wd << 16);
                        }
                        x[z] *= p.inv_v_scale;
                    }
                    c[tt] = f32x4_to_e4m3(x[0], x[1], x[2], x[3]);
                }
                // c[tt] byte j = (token tt, dim j): transpose the 4 x 4 bytes
                const uint32_t a0 = __builtin_amdgcn_perm(c[1], c[0], 0x05010400u);  // t0d0 t1d0 t0d1 t1d1
                const uint32_t a1 = __builtin_amdgcn_perm(c[3], c[2], 0x05010400u);  // t2d0 t3d0 t2d1 t3d1
                const uint32_t b0 = __builtin_amdgcn_perm(c[1], c[0], 0x07030602u);  // t0d2 t1d2 t0d3 t1d3
                const uint32_t b1 = __builtin_amdgcn_perm(c[3], c[2], 0x07030602u);  // t2d2 t3d2 t2d3 t3d3
                vw[j][0].x = __builtin_amdgcn_perm(a1, a0, 0x05040100u);  // d0: t0 t1 t2 t3
                vw[j][0].y = __builtin_amdgcn_perm(a1, a0, 0x07060302u);  // d1
                vw[j][0].z = __builtin_amdgcn_perm(b1, b0, 0x05040100u);  // d2
                vw[j][0].w = __builtin_amdgcn_perm(b1, b0, 0x07060302u);  // d3
            } else if constexpr (POOL == kBF16) {
                // dims 4 q .. 4 q + 3 of tokens 0..3; cell 0 holds dims 4 q, 4 q + 1
                // as words (t0 t1)(t2 t3) of each dim, cell 1 dims 4 q + 2, 4 q + 3
                const uint2 *x = vr[j];
                vw[j][0].x = __builtin_amdgcn_perm(x[1].x, x[0].x, 0x05040100u);
                vw[j][0].y = __builtin_amdgcn_perm(x[3].x, x[2].x, 0x05040100u);
                vw[j][0].z = __builtin_amdgcn_perm(x[1].x, x[0].x, 0x07060302u);
                vw[j][0].w = __builtin_amdgcn_perm(x[3].x, x[2].x, 0x07060302u);
                vw[j][1].x = __builtin_amdgcn_perm(x[1].y, x[0].y, 0x05040100u);
                vw[j][1].y = __builtin_amdgcn_perm(x[3].y, x[2].y, 0x05040100u);
                vw[j][1].z = __builtin_amdgcn_perm(x[1].y, x[0].y, 0x07060302u);
                vw[j][1].w = __builtin_amdgcn_perm(x[3].y, x[2].y, 0x07060302u);
            } else {  // fp32: tokens 0..3 of dim q
                vw[j][0] = uint4{vr[j][0], vr[j][1], vr[j][2], vr[j][3]};
            }
        }
#pragma unroll
        for (int j = 0; j < KI; ++j) {
            const int i = threadIdx.x + j * kThreads;
            if (!do_k || (!KFULL && i >= nh * K_UNITS)) break;
            store16_nt(unit(p.k_pool, i / K_UNITS, i % K_UNITS), kw[j]);
        }
#pragma unroll
        for (int j = 0; j < VI; ++j) {
            const int i = threadIdx.x + j * kThreads;
            if (!do_v || (!VFULL && i >= nh * VU)) break;
#pragma unroll
            for (int cc = 0; cc < CPI; ++cc) store16_nt(unit(p.v_pool, i / VU, (i % VU) * CPI + cc), vw[j][cc]);
        }
    };
    if (nh == HPW)
        tiles(std::true_type{});
    else
        tiles(std::false_type{});
}

// Workgroup (pair, pool, part): 16-byte copies of one part of the whole block
// (all KV heads), U x 4 KiB per part; each thread issues its U loads before
// its stores, which are non-temporal.  Source and destination never overlap
// (destinations are distinct and none is a source).  Measured on MI355X:
// whole 32 KiB blocks per workgroup (U = 8) are fastest for a few hundred
// pairs, 16 KiB parts (U = 4) once thousands of pairs fill the chip.
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
        if (i < n) store16_nt(d + i, v[u]);
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

// Workgroup (sequence, KV head): each sequence's newest token to the slot of
// position context_len - 1, through its block table (a decode step whose
// attention kernel cannot write it itself).
// A context longer than its table row can hold (the attention clamps it)
// has no slot for its newest token: nothing is written.
template <int POOL, int D>
__global__ __launch_bounds__(kThreads) void append_tokens_kernel(DecodeParams p) {
    const int s = blockIdx.x, g = blockIdx.y;
    const int ctx = p.context_lens[s];
    if (ctx <= 0 || ctx > p.max_blocks_per_seq * kBlock) return;
    const int32_t *table = p.block_tables + (int64_t)s * p.max_blocks_per_seq;
    for (int d = threadIdx.x; d < D; d += kThreads) append_element<POOL, D>(p, table, s, g, ctx - 1, d);
}

// Heads per cache-write workgroup: for bulk writes (prompts: thousands of
// windows) 8 with a 16/32-bit pool and 2 with an fp8 pool, whose encoding
// makes every work item heavier (the 70B-like fill: 8 heads 1.695 ms, 2
// heads 1.718; the fp8 fill: 8 heads 0.596 ms, 4 heads 0.560, 2 heads
// 0.548); 1 for small writes (a decode step's lone tokens, whose writes are
// latency-bound round trips and need the workgroups: 256 tokens x 8 heads
// took 17.8 us from 16 eight-head workgroups against ~4 us from 128).
template <int POOL>
constexpr int kCacheHeads = POOL == kFP8 ? 2 : 8;
// ... and with 8 heads, K and V tiles from separate workgroups (twice as
// many, each reading and writing 32 KiB: the 70B-like fill 1.689 ->
// 1.665 ms; the fp8 fill with 2 heads is 0.5 % slower split)
template <int POOL>
constexpr unsigned kCacheSplit = kCacheHeads<POOL> == 8 ? 2u : 1u;
constexpr int64_t kCacheBulkGroups = 2048;  // workgroups of the bulk grid from which it is used

template <int POOL, int IN, int D>
hipError_t launch_rc(const CacheParams &p, hipStream_t stream) {
    constexpr int HPW = kCacheHeads<POOL>;
    const int64_t groups = (p.num_tokens + kBlock - 1) / kBlock;
    if (groups > 0x7fffffffLL || p.num_kv_heads > 65535) return hipErrorInvalidValue;
    const int64_t hgroups = (p.num_kv_heads + HPW - 1) / HPW;
    if (groups * hgroups >= kCacheBulkGroups)
        reshape_and_cache_kernel<POOL, IN, D, HPW>
            <<<dim3((unsigned)groups, (unsigned)hgroups, kCacheSplit<POOL>), dim3(kThreads), 0, stream>>>(p);
    else
        reshape_and_cache_kernel<POOL, IN, D, 1>
            <<<dim3((unsigned)groups, (unsigned)p.num_kv_heads), dim3(kThreads), 0, stream>>>(p);
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

hipError_t launch_append_tokens(int kv, int head_dim, const DecodeParams &p, hipStream_t stream) {
    if (p.num_seqs <= 0) return hipSuccess;
    if (p.num_kv_heads > 65535) return hipErrorInvalidValue;
    const dim3 grid((unsigned)p.num_seqs, (unsigned)p.num_kv_heads);
    if (kv == kF32)
        head_dim == 64 ? append_tokens_kernel<kF32, 64><<<grid, dim3(kThreads), 0, stream>>>(p)
                       : append_tokens_kernel<kF32, 128><<<grid, dim3(kThreads), 0, stream>>>(p);
    else if (kv == kBF16)
        head_dim == 64 ? append_tokens_kernel<kBF16, 64><<<grid, dim3(kThreads), 0, stream>>>(p)
                       : append_tokens_kernel<kBF16, 128><<<grid, dim3(kThreads), 0, stream>>>(p);
    else
        head_dim == 64 ? append_tokens_kernel<kFP8, 64><<<grid, dim3(kThreads), 0, stream>>>(p)
                       : append_tokens_kernel<kFP8, 128><<<grid, dim3(kThreads), 0, stream>>>(p);
    return hipGetLastError();
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
