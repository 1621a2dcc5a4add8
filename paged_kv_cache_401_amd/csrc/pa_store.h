// pa_store.h -- storing single K/V elements into the pool's tiles: the fp8
// encoder and the tile offsets of one (block, KV head, token, dim) element,
// shared by the cache write and the decode kernels that append each
// sequence's newest token themselves.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {

// s_waitcnt immediate waiting for every outstanding vector memory access
// (vmcnt 0; the export and LDS/scalar counts left at their maximum)
constexpr int kWaitVmem = 0x0F70;

// fp32 -> OCP E4M3FN with round-to-nearest-even and saturation to +-448;
// NaN keeps its sign as S.1111.111.  The hardware conversion rounds to
// nearest even; a clamp to +-448 (v_med3_f32) first gives the saturation.
// NaN, which the clamp would turn into +-448, is set apart.  The cache write
// built on it is checked against a table-search encoder of the same rule on
// every one of the 2^32 fp32 bit patterns.
__device__ __forceinline__ float sat448(float x) { return __builtin_amdgcn_fmed3f(x, -448.f, 448.f); }

__device__ __forceinline__ uint32_t e4m3_nan(float x) {
    return ((__float_as_uint(x) >> 24) & 0x80u) | 0x7fu;
}

__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
    const uint32_t code = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(x), 0.f, 0, false) & 0xffu;
    return x != x ? e4m3_nan(x) : code;
}

// four values -> four codes, byte i = value i
__device__ __forceinline__ uint32_t f32x4_to_e4m3(float x0, float x1, float x2, float x3) {
    uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(x0), sat448(x1), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(x2), sat448(x3), w, true);
    if ((x0 != x0) | (x1 != x1) | (x2 != x2) | (x3 != x3)) {
        const float xs[4] = {x0, x1, x2, x3};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (xs[i] != xs[i]) w = (w & ~(0xffu << (8 * i))) | (e4m3_nan(xs[i]) << (8 * i));
    }
    return w;
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

// 16-byte store marked non-temporal.  For the pool's bulk writes (block
// copies, whole-tile cache writes) it let copies of thousands of blocks run
// at 7.7 TB/s read + write against 5.4 with plain stores.
__device__ __forceinline__ void store16_nt(void *dst, uint4 v) {
    typedef uint32_t w4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(w4{v.x, v.y, v.z, v.w}, static_cast<w4 *>(dst));
}

// Element d of one token's K and V, given as the pool's element bits (fp8
// code, bf16 or fp32 bits), to position t of the tiles of block b, KV head g.
// A lone token touches one 16-byte run per K run and spreads over the V
// cells of its 4-token group, so its stores are marked non-temporal: held as
// streaming lines they cost a decode step measurably less than plain stores.
template <int POOL, int D>
__device__ __forceinline__ void store_kv_raw(void *k_pool, void *v_pool, int64_t b, int num_kv_heads, int g,
                                             int t, int d, uint32_t kraw, uint32_t vraw) {
    constexpr int EB = POOL == kF32 ? 4 : (POOL == kBF16 ? 2 : 1);
    constexpr int X = 16 / EB;   // K: elements per 16-byte run
    constexpr int W = 4 / EB;    // V: head-dim elements per 16-byte cell
    const int64_t tile = (b * num_kv_heads + g) * (int64_t)(kBlock * D);
    const int64_t ko = tile + ((d / X) * kBlock + t) * X + (d % X);
    const int64_t vo = tile + ((t >> 2) * (D / W) + d / W) * (4 * W) + (d % W) * 4 + (t & 3);
    if constexpr (POOL == kFP8) {
        __builtin_nontemporal_store((uint8_t)kraw, reinterpret_cast<uint8_t *>(k_pool) + ko);
        __builtin_nontemporal_store((uint8_t)vraw, reinterpret_cast<uint8_t *>(v_pool) + vo);
    } else if constexpr (POOL == kBF16) {
        __builtin_nontemporal_store((uint16_t)kraw, reinterpret_cast<uint16_t *>(k_pool) + ko);
        __builtin_nontemporal_store((uint16_t)vraw, reinterpret_cast<uint16_t *>(v_pool) + vo);
    } else {
        __builtin_nontemporal_store(kraw, reinterpret_cast<uint32_t *>(k_pool) + ko);
        __builtin_nontemporal_store(vraw, reinterpret_cast<uint32_t *>(v_pool) + vo);
    }
}

// Element d of one token's K and V (input element index `idx` in k and v,
// of dtype IN) to position t of the tiles of block b, KV head g (pool dtype
// POOL; fp8 codes scaled by inv_k / inv_v).
template <int POOL, int IN, int D>
__device__ __forceinline__ void store_kv_element(void *k_pool, void *v_pool, const void *k, const void *v,
                                                 int64_t idx, int64_t b, int num_kv_heads, int g, int t, int d,
                                                 float inv_k, float inv_v) {
    uint32_t kraw, vraw;
    if constexpr (POOL == kFP8) {
        kraw = f32_to_e4m3(load_in<IN>(k, idx) * inv_k);
        vraw = f32_to_e4m3(load_in<IN>(v, idx) * inv_v);
    } else if constexpr (POOL == kBF16) {
        kraw = reinterpret_cast<const uint16_t *>(k)[idx];
        vraw = reinterpret_cast<const uint16_t *>(v)[idx];
    } else {
        kraw = reinterpret_cast<const uint32_t *>(k)[idx];
        vraw = reinterpret_cast<const uint32_t *>(v)[idx];
    }
    store_kv_raw<POOL, D>(k_pool, v_pool, b, num_kv_heads, g, t, d, kraw, vraw);
}

// Element d (of head g) of sequence s's newest token -- input row s of
// k_new / v_new ([num_seqs][num_kv_heads][D]) -- to the slot of position
// pos through the sequence's block table; an id outside the pool is
// skipped.  The input dtype is a runtime value (bf16 or fp32; the pool's own
// dtype unless the pool is fp8).
template <int POOL, int D>
__device__ __forceinline__ void append_element(const DecodeParams &p, const int32_t *table, int s, int g,
                                               int pos, int d) {
    const int32_t b = table[pos / kBlock];
    if (b < 0 || b >= p.num_blocks) return;
    const int64_t idx = ((int64_t)s * p.num_kv_heads + g) * D + d;
    void *kp = const_cast<void *>(p.k_pool);
    void *vp = const_cast<void *>(p.v_pool);
    if constexpr (POOL == kFP8) {
        if (p.new_dtype == kF32)
            store_kv_element<POOL, kF32, D>(kp, vp, p.k_new, p.v_new, idx, b, p.num_kv_heads, g, pos % kBlock, d,
                                            p.inv_k_scale, p.inv_v_scale);
        else
            store_kv_element<POOL, kBF16, D>(kp, vp, p.k_new, p.v_new, idx, b, p.num_kv_heads, g, pos % kBlock,
                                             d, p.inv_k_scale, p.inv_v_scale);
    } else {
        store_kv_element<POOL, POOL, D>(kp, vp, p.k_new, p.v_new, idx, b, p.num_kv_heads, g, pos % kBlock, d,
                                        1.f, 1.f);
    }
}

// The newest token of sequence s, head g, split in two phases so that a
// decode wavefront can issue the input loads, then its own block loads, and
// store the token when the inputs arrive: lane `lane` holds elements
// d = lane + 64 i (i < D / 64) of K and of V as raw input words.
template <int D>
struct NewToken {
    uint32_t k[D / 64], v[D / 64];
    int64_t b;  // block of the newest position (< 0: nothing to write)
};

template <int POOL, int D>
__device__ __forceinline__ NewToken<D> append_load(const DecodeParams &p, const int32_t *table, int s, int g,
                                                   int pos, int lane) {
    NewToken<D> nt;
    const int32_t b = table[pos / kBlock];
    nt.b = b >= 0 && b < p.num_blocks ? b : -1;
    const int64_t row = ((int64_t)s * p.num_kv_heads + g) * D;
    const bool f32 = POOL == kF32 || (POOL == kFP8 && p.new_dtype == kF32);
#pragma unroll
    for (int i = 0; i < D / 64; ++i) {
        const int64_t idx = row + lane + 64 * i;
        if (f32) {
            nt.k[i] = reinterpret_cast<const uint32_t *>(p.k_new)[idx];
            nt.v[i] = reinterpret_cast<const uint32_t *>(p.v_new)[idx];
        } else {
            nt.k[i] = reinterpret_cast<const uint16_t *>(p.k_new)[idx];
            nt.v[i] = reinterpret_cast<const uint16_t *>(p.v_new)[idx];
        }
    }
    return nt;
}

template <int POOL, int D>
__device__ __forceinline__ void append_store(const DecodeParams &p, const NewToken<D> &nt, int g, int pos,
                                             int lane) {
    if (nt.b < 0) return;
    void *kp = const_cast<void *>(p.k_pool);
    void *vp = const_cast<void *>(p.v_pool);
#pragma unroll
    for (int i = 0; i < D / 64; ++i) {
        uint32_t kraw = nt.k[i], vraw = nt.v[i];
        if constexpr (POOL == kFP8) {
            const bool f32 = p.new_dtype == kF32;
            const float kx = f32 ? __uint_as_float(kraw) : __uint_as_float(kraw << 16);
            const float vx = f32 ? __uint_as_float(vraw) : __uint_as_float(vraw << 16);
            kraw = f32_to_e4m3(kx * p.inv_k_scale);
            vraw = f32_to_e4m3(vx * p.inv_v_scale);
        }
        store_kv_raw<POOL, D>(kp, vp, nt.b, p.num_kv_heads, g, pos % kBlock, lane + 64 * i, kraw, vraw);
    }
}

}  // namespace pa
