// pa_decode_mfma.hip -- matrix-core decode kernel for grouped-query attention.
//
// When G = Hq / Hkv query heads share one KV head (grouped-query attention,
// "PagedAttention" glossary page, related techniques), each 16-token block
// read through the block table ("how paging works") serves G queries, and the
// two products of decode attention become small dense contractions:
//     S^T[16 tokens][16 heads]  = K[16][D] . Q^T[D][16]           (heads >= G are zero)
//     O^T[D][16 heads]         += V^T[D][16 tokens] . P^T[16][16]
// Both run on gfx950's matrix cores (v_mfma_f32_16x16x32_bf16 for the
// scores, v_mfma_f32_16x16x16_bf16 -- or _f16 with an fp8 pool -- for P.V)
// with fp32 accumulation.  An fp8 (E4M3FN) pool is widened in registers
// (K to bf16, V to fp16), which is exact.
//
// Work split: one workgroup per (sequence, KV head, partition of
// partition_tokens tokens); its four wavefronts take every fourth block and
// keep their own online-softmax state (running max m and sum l per head,
// base-2 exponent domain), merged through LDS at the end.  Short split-K
// partitions go to one-wavefront workgroups that walk all of their blocks.  Longer contexts
// leave per-partition (m, l, O) in the workspace for the reduce kernel.
//
// Operand layouts (lane = 16 c + n, n = lane % 16):
//   K (A operand, rows = tokens): the pool's K tile stores each token's head
//     vector in 16-byte runs, token-major per run, so lane (n, c) loads run
//     c + 4u of token n with one 16-byte load; all 64 lanes read 1 KiB of
//     contiguous memory.  Contraction index (c, r) of step u is head dim
//     8 (4u + c) + r for bf16, 16 (c + 4j) + 8 h + r for fp8 (run c + 4j,
//     half h); Q^T uses the same mapping.
//   S^T (result): lane (n, c) holds tokens 4c..4c+3 of head n, which is
//     exactly the P^T operand layout of the second product, so probabilities
//     never leave their lane.
//   V (A operand, rows = head dims): the pool's V tile stores 16-byte cells of
//     4 consecutive tokens x W head dims, so lane (n, c) loads the cell of
//     tokens 4c..4c+3 and head dims W (16 jj + n) .. +W-1 with one load.
//   P^T is split into bf16 high and low parts (p = hi + lo to 16 significant
//     bits); each 16 x 16 output tile takes two 16-deep products of the same
//     V operand (tokens 4c..4c+3), one against hi and one against lo, so P
//     enters at ~16-bit precision.  With an fp8 pool, V is widened to fp16
//     instead (exact for every E4M3 code) and P rounded to fp16 (relative
//     error <= 2^-11, far inside an fp8 cache's tolerance): one 16-deep fp16
//     product per tile.
//   Tokens past the context are excluded by selection: their scores are set
//     to -inf and their V operand elements to zero before the product.
#include "pa_internal.h"
#include "pa_mfma_util.h"
#include "pa_store.h"

#include <type_traits>

namespace pa {
namespace {

constexpr float kNegInf = kNegInfF;
constexpr float kLazyMax = 8.0f;  // raise the running maximum only past 2^8 (base-2 scores)

// LDS of one workgroup: the wavefronts' softmax states and numerators of
// the first NC matrix-core columns, merged at the end of a work item
template <int D, int NW, int NC = 16>
struct DecodeLds {
    float m[NW][NC];
    float l[NW][NC];
    float acc[NW][D * (NC + 1)];   // [wave][d][head], padded
    // the newest token's K and V as the pool stores them (head-dim order;
    // used by the wavefront that writes it)
    alignas(16) uint8_t tok_k[D * 2];
    alignas(16) uint8_t tok_v[D * 2];
    uint32_t done;           // wavefronts of a partition group that have finished
};

// Where a wavefront's blocks come from: blocks j = jb + stride * k (k < nk)
// of one sequence's block table, tokens below tok1 (its partition's end)
// attended by every column (query head).
struct TableBlocks {
    static constexpr bool kColumnMask = false;
    const int32_t *table;   // the sequence's table row
    int jb, stride, nk, tok1;
    // the physical block of step k (-1 past the end)
    __device__ __forceinline__ int32_t id(int k) const {
        const int32_t b = table[jb + stride * min(k, nk - 1)];
        return k < nk ? b : -1;
    }
    // its position in the sequence's table
    __device__ __forceinline__ int block(int k) const { return jb + stride * k; }
    // tokens of step k's block attended (>= 1; 16 or more: all of them) and
    // the columns [lo, hi) that attend it
    __device__ __forceinline__ void mask(int k, int &nvalid, int &lo, int &hi) const {
        nvalid = tok1 - block(k) * kBlock;
        lo = 0;
        hi = 16;
    }
};

// One wavefront's walk over the blocks of `src` for KV head g: scores,
// online softmax and P.V accumulate into m (running maximum, base-2 domain),
// l (running sum, per-column total on return) and acc (numerators, the MFMA
// C layout: lane (n, c) holds column n).  Column n is the query row qcol of
// this lane (nullptr: an unused column, zero query); the first ncols
// columns are real.  `writer`: this wavefront reads the block holding
// position ctx - 1 of sequence s and writes the decode step's newest token
// (DecodeParams::k_new / v_new) into it (APPEND only); it stages the token
// in tok_k / tok_v (LDS, 2 D bytes each).
//
// The newest token: the writer loads the token's inputs before its block
// loads and stages them in LDS, encoded as the pool stores them; when the
// block arrives, the lanes that hold the token's K runs and V cell elements
// take them from there into its registers, and after the loop they store
// them to the pool.  Stores issued before later loads would make every wait
// on those loads wait for the stores as well (one counter covers both, in
// issue order), and under full read traffic stores are slow.
template <int KV, int D, bool STREAM, bool APPEND, class Src, int NB = 2>
__device__ __forceinline__ void walk_blocks(const DecodeParams &p, int s, int g, const Src &src,
                                            const uint16_t *qcol, int ncols, int ctx, bool writer,
                                            uint8_t *tok_k, uint8_t *tok_v, float &m, float &l,
                                            floatx4 (&acc)[D / 16]) {
    constexpr int EB = KV == kBF16 ? 2 : 1;
    constexpr int TILE_BYTES = kBlock * D * EB;
    constexpr int NQK = D / 32;                   // QK steps (32-deep) per block
    constexpr int NKL = KV == kBF16 ? NQK : NQK / 2;  // 16-byte K loads per lane per block
    constexpr int W = 4 / EB;                     // V: head dims per 16-byte cell
    constexpr int NVL = D / W / 16;               // 16-byte V loads per lane per block
    constexpr int NT = D / 16;                    // 16 x 16 output tiles (= NVL * W)

    const int lane = threadIdx.x & 63;
    const int n = lane & 15;
    const int c = lane >> 4;
    const int32_t *table = p.block_tables + (int64_t)s * p.max_blocks_per_seq;
    const int tn = (ctx - 1) & (kBlock - 1);   // the newest token's slot in its block
    const int jlast = (ctx - 1) / kBlock;      // ... and its block
    const int nk = src.nk;

    // Q^T operands: column n's query row (zero for unused columns), head dims
    // per the K mapping
    bf16x8 qop[NQK];
    {
#pragma unroll
        for (int u = 0; u < NQK; ++u) {
            int d0;
            if constexpr (KV == kBF16)
                d0 = 8 * (4 * u + c);
            else
                d0 = 16 * (c + 4 * (u >> 1)) + 8 * (u & 1);
            u32x4 v = {0u, 0u, 0u, 0u};
            if (qcol) v = *reinterpret_cast<const u32x4 *>(qcol + d0);
            qop[u] = as_bf16x8(v);
        }
    }

    m = kNegInf;
    l = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};

    const char *kbase = static_cast<const char *>(p.k_pool);
    const char *vbase = static_cast<const char *>(p.v_pool);
    const int koff = (c * kBlock + n) * 16;        // run c, token n
    const int voff = (c * (D / W) + n) * 16;       // cell (tokens 4c.., dims W*n..)
    auto valid = [&](int32_t b) { return b >= 0 && b < p.num_blocks; };

    // one tile of a pool as a buffer resource: empty (loads give zeros and
    // touch no memory) for an id outside the pool or past the end (-1)
    auto tile = [&](const char *base, int32_t b) {
        const bool ok = valid(b);
        return tile_rsrc(base + ((int64_t)(ok ? b : 0) * p.num_kv_heads + g) * TILE_BYTES, ok ? TILE_BYTES : 0);
    };
    // FENCED: keep the loads in program order (the prologue issues them in
    // the loop's order, so the loop's waits hold from its first iteration)
    auto load_k = [&](int32_t b, u32x4 (&kr)[NKL], auto fenced) {
        const auto r = tile(kbase, b);
#pragma unroll
        for (int i = 0; i < NKL; ++i) {
            kr[i] = load_tile<STREAM>(r, koff + i * 4 * kBlock * 16);
            if constexpr (decltype(fenced)::value) __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto load_v = [&](int32_t b, u32x4 (&vr)[NVL], auto fenced) {
        const auto r = tile(vbase, b);
#pragma unroll
        for (int i = 0; i < NVL; ++i) {
            vr[i] = load_tile<STREAM>(r, voff + i * 16 * 16);
            if constexpr (decltype(fenced)::value) __builtin_amdgcn_sched_barrier(0);
        }
    };
    constexpr std::true_type kFenced{};
    constexpr std::false_type kFree{};

    // S^T = K . Q^T for one block
    auto qk = [&](const u32x4 (&kr)[NKL]) {
        floatx4 sacc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (KV == kBF16) {
#pragma unroll
            for (int u = 0; u < NQK; ++u)
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[u]), qop[u], sacc, 0, 0, 0);
        } else {
#pragma unroll
            for (int i = 0; i < NKL; ++i) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    uint32_t a0, a1, a2, a3;
                    e4m3x4_to_bf16(kr[i][2 * h], a0, a1);
                    e4m3x4_to_bf16(kr[i][2 * h + 1], a2, a3);
                    const u32x4 a = {a0, a1, a2, a3};
                    sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), qop[2 * i + h], sacc,
                                                                   0, 0, 0);
                }
            }
        }
        return sacc;
    };

    // online softmax and O^T += V^T . P^T for a block whose first nvalid
    // tokens are attended by columns [lo, hi)
    auto softmax_pv = [&](floatx4 sacc, const u32x4 (&vr)[NVL], int nvalid, int lo, int hi) {
        // online softmax over this block (tokens 4c..4c+3 of column n in this lane)
        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sc[i] = sacc[i] * p.qk_scale_log2;
            if (4 * c + i >= nvalid) sc[i] = kNegInf;
            if constexpr (Src::kColumnMask) {
                if (n < lo || n >= hi) sc[i] = kNegInf;
            }
        }
        // The running maximum is raised lazily: only when some lane's score
        // exceeds it by more than 8 (base 2) is the column maximum exchanged
        // across lanes and the running state rescaled; otherwise the block's
        // probabilities stay below 2^8 against the old maximum.  (Before a
        // column's first finite score its maximum is -inf, so the first
        // block always raises it.)
        float bm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        float alpha = 1.f;
        if (__builtin_amdgcn_ballot_w64(bm > m + kLazyMax) != 0) {
            bm = max_xor32(max_xor16(bm));
            const float m_new = fmaxf(m, bm);
            // a masked column may still have -inf here: -inf - (-inf) would
            // be NaN, its (zero) state needs no rescale
            alpha = m_new == kNegInf ? 1.f : __builtin_amdgcn_exp2f(m - m_new);
            m = m_new;
        }
        // A masked column may meet a block before any token it attends: its
        // maximum is still -inf; exponents against 0 keep its sum and
        // numerators at 0.
        const float m_ref = m == kNegInf ? 0.f : m;
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(sc[i] - m_ref);
        // fp8 pool: P rounded to fp16 (relative error <= 2^-11) against V
        // widened to fp16 (exact for every E4M3 code), one 16-deep product
        // per tile; the sum adds the same rounded values.  bf16 / fp32-like
        // pools: P carried as bf16 hi + lo (16 significant bits).
        f16x4 pf;
        if constexpr (KV == kFP8) {
            const f16x2 h01 = {(_Float16)pr[0], (_Float16)pr[1]};
            const f16x2 h23 = {(_Float16)pr[2], (_Float16)pr[3]};
            const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
            l = __builtin_amdgcn_fdot2(h23, one, __builtin_amdgcn_fdot2(h01, one, l * alpha, false), false);
            pf = f16x4{h01[0], h01[1], h23[0], h23[1]};
        } else {
            l = l * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
        }
        // rescale the numerators only when some real column's maximum moved
        if (__builtin_amdgcn_ballot_w64(n < ncols && alpha != 1.f) != 0) {
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[t] *= alpha;
        }

        // P^T operands: hi(p0..p3) and lo(p0..p3), tokens 4c..4c+3
        bf16x4 phi = {}, plo = {};
        if constexpr (KV != kFP8) {
            const u32x4 pw = as_u32x4(p_operand_hi_lo(pr));
            phi = as_bf16x4(pw[0], pw[1]);
            plo = as_bf16x4(pw[2], pw[3]);
        }

        // zero the V elements of tokens past the context (last block only;
        // they may hold anything, NaN included)
        uint32_t keep01 = 0xffffffffu, keep23 = 0xffffffffu;
        if (nvalid < kBlock) v_keep_masks(c, nvalid, keep01, keep23);

        // O^T += V^T . P^T per 16 x 16 tile, as two 16-deep products (against
        // hi, then lo) straight from the V registers: no [V | V] operand to
        // assemble.  (Masking only inside a branch for the last block
        // duplicated this loop and cost the kernel 20-35 registers.)
#pragma unroll
        for (int jj = 0; jj < NVL; ++jj) {
#pragma unroll
            for (int w = 0; w < W; ++w) {
                floatx4 &o = acc[jj * W + w];
                if constexpr (KV == kFP8) {
                    const f16x2 lo2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(vr[jj][w], 1.0f, false);
                    const f16x2 hi2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(vr[jj][w], 1.0f, true);
                    const uint32_t v01 = __builtin_bit_cast(uint32_t, lo2) & keep01;
                    const uint32_t v23 = __builtin_bit_cast(uint32_t, hi2) & keep23;
                    const f16x4 a = __builtin_bit_cast(f16x4, (uint64_t)v01 | ((uint64_t)v23 << 32));
                    o = __builtin_amdgcn_mfma_f32_16x16x16f16(a, pf, o, 0, 0, 0);
                } else {
                    const uint32_t v01 = vr[jj][2 * w], v23 = vr[jj][2 * w + 1];
                    const bf16x4 a = as_bf16x4(v01 & keep01, v23 & keep23);
                    o = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, phi, o, 0, 0, 0);
                    o = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, plo, o, 0, 0, 0);
                }
            }
        }
    };

    // This wavefront's blocks are j = jb + stride k, k = 0..nk-1; their ids
    // come from the table by scalar loads, one block ahead of their use.  Two
    // register buffers hold blocks k and k + 1; block k + 2 reuses block k's
    // buffer half by half: its K loads are issued as soon as block k's scores
    // are computed, its V loads once block k's V is consumed, so a wavefront
    // keeps close to two blocks in flight in the registers of one.  Every step
    // issues the same loads (empty resources past the end), which lets each
    // wait cover exactly the loads it needs.
    if (nk > 0) {
        auto id_at = [&](int k) -> int32_t { return src.id(k); };
        // the newest token's inputs go out first (lane elements lane + 64 i)
        NewToken<D> nt;
        if (APPEND && writer) nt = append_load<KV, D>(p, table, s, g, ctx - 1, lane);
        static_assert(NB == 2 || NB == 3, "two or three register buffers");
        u32x4 kb[NB][NKL], vb[NB][NVL];
        int32_t idb[NB];
#pragma unroll
        for (int d = 0; d < NB; ++d) {
            idb[d] = id_at(d);
            load_k(idb[d], kb[d], kFenced);
            load_v(idb[d], vb[d], kFenced);
        }
        // ... and into LDS, encoded as the pool stores them, in head-dim
        // order: waiting for the inputs holds none of the block loads above
        if constexpr (APPEND) {
            if (writer) {
#pragma unroll
                for (int i = 0; i < D / 64; ++i) {
                    const int d = lane + 64 * i;
                    if constexpr (KV == kBF16) {
                        reinterpret_cast<uint16_t *>(tok_k)[d] = (uint16_t)nt.k[i];
                        reinterpret_cast<uint16_t *>(tok_v)[d] = (uint16_t)nt.v[i];
                    } else {
                        const bool f32 = p.new_dtype == kF32;
                        const float kx = f32 ? __uint_as_float(nt.k[i]) : __uint_as_float(nt.k[i] << 16);
                        const float vx = f32 ? __uint_as_float(nt.v[i]) : __uint_as_float(nt.v[i] << 16);
                        tok_k[d] = (uint8_t)f32_to_e4m3(kx * p.inv_k_scale);
                        tok_v[d] = (uint8_t)f32_to_e4m3(vx * p.inv_v_scale);
                    }
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            }
        }
        // The token into the registers of its block, as its own loads would
        // return it once stored: lanes n == tn take K runs c + 4i (bytes
        // 16 (c + 4i) of the staged K), lanes c == tn / 4 the elements of
        // token tn % 4 in their V cells (element (w, r) of a cell sits at
        // byte (4 w + r) EB; the staged V word at byte 4 (16 jj + n) holds
        // the cell's W head dims).
        auto patch = [&](u32x4 (&kr)[NKL], u32x4 (&vr)[NVL]) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if (n == tn) {
#pragma unroll
                for (int i = 0; i < NKL; ++i) kr[i] = *reinterpret_cast<const u32x4 *>(tok_k + 16 * (c + 4 * i));
            }
            if (c == (tn >> 2)) {
                const int r = tn & 3;
#pragma unroll
                for (int jj = 0; jj < NVL; ++jj) {
                    const uint32_t x = *reinterpret_cast<const uint32_t *>(tok_v + 4 * (16 * jj + n));
#pragma unroll
                    for (int w = 0; w < W; ++w) {
                        if constexpr (KV == kBF16) {
                            const uint32_t e = (x >> (16 * w)) & 0xffffu;
                            const uint32_t sh = 16u * (uint32_t)(r & 1);
#pragma unroll
                            for (int h = 0; h < 2; ++h)
                                if ((r >> 1) == h)
                                    vr[jj][2 * w + h] = (vr[jj][2 * w + h] & ~(0xffffu << sh)) | (e << sh);
                        } else {
                            const uint32_t e = (x >> (8 * w)) & 0xffu;
                            const uint32_t sh = 8u * (uint32_t)r;
                            vr[jj][w] = (vr[jj][w] & ~(0xffu << sh)) | (e << sh);
                        }
                    }
                }
            }
        };

        int32_t id_pre = id_at(NB);
        auto step = [&](int d, int kk) {
            const int32_t id_after = id_pre;  // block kk + NB
            id_pre = id_at(kk + NB + 1);
            if (APPEND && writer && src.block(kk) == jlast) patch(kb[d], vb[d]);
            const floatx4 sacc = qk(kb[d]);
            load_k(id_after, kb[d], kFree);
            if (valid(idb[d])) {
                int nvalid, lo, hi;
                src.mask(kk, nvalid, lo, hi);
                softmax_pv(sacc, vb[d], nvalid, lo, hi);
            }
            load_v(id_after, vb[d], kFree);
            idb[d] = id_after;
        };
        int k = 0;
        if constexpr (NB == 3) {
            for (; k + 2 < nk; k += 3) {
                step(0, k);
                step(1, k + 1);
                step(2, k + 2);
            }
            if (k < nk) step(0, k);
            if (k + 1 < nk) step(1, k + 1);
        } else {
            for (; k + 1 < nk; k += 2) {
                step(0, k);
                step(1, k + 1);
            }
            if (k < nk) step(0, k);
        }

        // the token to the pool (an id outside the pool is skipped): K runs
        // as 16-byte stores, V elements one by one
        if constexpr (APPEND) {
            if (writer && nt.b >= 0) {
                const int64_t tile0 = (nt.b * p.num_kv_heads + g) * TILE_BYTES;
                char *kt = const_cast<char *>(kbase) + tile0;
                char *vt = const_cast<char *>(vbase) + tile0;
                if (n == tn) {
#pragma unroll
                    for (int i = 0; i < NKL; ++i)
                        store16_nt(kt + ((c + 4 * i) * kBlock + tn) * 16,
                                   *reinterpret_cast<const uint4 *>(tok_k + 16 * (c + 4 * i)));
                }
                if (c == (tn >> 2)) {
#pragma unroll
                    for (int jj = 0; jj < NVL; ++jj) {
                        const uint32_t x = *reinterpret_cast<const uint32_t *>(tok_v + 4 * (16 * jj + n));
#pragma unroll
                        for (int w = 0; w < W; ++w) {
                            const int off = ((tn >> 2) * (D / W) + 16 * jj + n) * 16 + (w * 4 + (tn & 3)) * EB;
                            if constexpr (KV == kBF16)
                                __builtin_nontemporal_store((uint16_t)(x >> (16 * w)), reinterpret_cast<uint16_t *>(vt + off));
                            else
                                __builtin_nontemporal_store((uint8_t)(x >> (8 * w)), reinterpret_cast<uint8_t *>(vt + off));
                        }
                    }
                }
            }
        }
    }

    // per-head totals of the lane-partial sums
    l = add_xor32(add_xor16(l));
}

// This lane's query row for column n = lane % 16 of sequence s, KV head g:
// query head g G + n, none for n >= G.
template <int D>
__device__ __forceinline__ const uint16_t *query_column(const DecodeParams &p, int s, int g) {
    const int n = threadIdx.x & 15;
    if (n >= p.group) return nullptr;
    return reinterpret_cast<const uint16_t *>(p.q) + ((int64_t)s * p.num_q_heads + (int64_t)g * p.group + n) * D;
}

// One wavefront's (m, l, numerators) to slot `w` of the workgroup's LDS, in
// [w][d][head] order.
template <int D, int NW, int W, int NC = 16>
__device__ __forceinline__ void state_to_lds(DecodeLds<D, NW, NC> &sm, int w, float m, float l,
                                             const floatx4 (&acc)[D / 16]) {
    constexpr int LDS_STRIDE = NC + 1;
    constexpr int NVL = D / W / 16;
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;
    const int c = lane >> 4;
    if (n >= NC) return;   // columns past NC hold no query head
    if (c == 0) {
        sm.m[w][n] = m;
        sm.l[w][n] = l;
    }
#pragma unroll
    for (int jj = 0; jj < NVL; ++jj)
#pragma unroll
        for (int ww = 0; ww < W; ++ww)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d = W * (16 * jj + 4 * c + i) + ww;
                sm.acc[w][d * LDS_STRIDE + n] = acc[jj * W + ww][i];
            }
}

// Merge the first `nw` wavefront states in LDS and write the result of
// columns 0 .. ncols-1, column hh being query head g G + hh % G of sequence
// s + hh / G: threads t0, t0 + tstride, ... each take 4 consecutive head
// dims of one column and store them with one 16-byte store -- the final
// output row (divided by the sum, times the value scale) when `final`, else
// the partial (numerators, maximum, sum) of slot `slot` of the row.  The stores that end
// a work item cost far more than their bytes while the chip streams K/V
// (timed on MI355X: the 512-token fp8 long-tail batch ran 20 % faster with
// them switched off), so there are 4x fewer of them than with one per dim.
// Final outputs go out non-temporal; split-K partials stay cacheable, since
// the reduce kernel reads them right after.
template <int D, int NW, int NC = 16>
__device__ __forceinline__ void merge_and_store(const DecodeParams &p, const DecodeLds<D, NW, NC> &sm, int s,
                                                int g, int slot, bool final, int nw, int t0,
                                                int tstride, int ncols) {
    constexpr int LDS_STRIDE = NC + 1;
    constexpr int D4 = D / 4;
    const int G = p.group;
    for (int idx = t0; idx < ncols * D4; idx += tstride) {
        const int hh = idx / D4;
        const int d0 = 4 * (idx % D4);
        float M = sm.m[0][hh];
        for (int w = 1; w < nw; ++w) M = fmaxf(M, sm.m[w][hh]);
        float L = 0.f;
        float O[4] = {0.f, 0.f, 0.f, 0.f};
        for (int w = 0; w < nw; ++w) {
            const float f = sm.m[w][hh] == kNegInf ? 0.f : exp2f(sm.m[w][hh] - M);
            L += sm.l[w][hh] * f;
#pragma unroll
            for (int e = 0; e < 4; ++e) O[e] += sm.acc[w][(d0 + e) * LDS_STRIDE + hh] * f;
        }
        const int64_t row = (int64_t)(s + hh / G) * p.num_q_heads + (int64_t)g * G + hh % G;
        if (final) {
            float r[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = L > 0.f ? (O[e] / L) * p.out_scale : 0.f;
            store16_nt(p.out + row * D + d0, __builtin_bit_cast(uint4, r));
        } else {
            const int64_t pr = row * p.max_partitions + slot;
            *reinterpret_cast<uint4 *>(p.ws_acc + pr * D + d0) = __builtin_bit_cast(uint4, O);
            if (d0 == 0) {
                p.ws_m[pr] = M;
                p.ws_l[pr] = L;
            }
        }
    }
}

// One work item: partition `part` of sequence s, KV head g, with context
// length ctx (already clamped to the table's capacity), computed by the NW
// wavefronts of the calling workgroup, which take every NW-th block and are
// merged through LDS.  APPEND: the decode step's newest tokens are written
// by this call unless `clamped` (the context was longer than its table row:
// no slot to write).
template <int KV, int D, bool STREAM, int NW, bool APPEND, int NB = 2>
__device__ __forceinline__ void decode_item(const DecodeParams &p, int s, int g, int part, int ctx,
                                            bool clamped, DecodeLds<D, NW> &sm) {
    constexpr int W = KV == kBF16 ? 2 : 4;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nparts = (ctx + p.partition_tokens - 1) / p.partition_tokens;
    if (part >= (nparts > 1 ? nparts : 1)) return;
    const int tok0 = part * p.partition_tokens;
    const int tok1 = min(ctx, tok0 + p.partition_tokens);
    const int blk0 = tok0 / kBlock;
    const int blk1 = (tok1 + kBlock - 1) / kBlock;
    // the newest token is written by the wavefront that reads the last
    // block of the partition holding it (the only reader of that block for
    // this KV head)
    const bool writer = APPEND && !clamped && tok1 == ctx && ctx > 0 && wv == (blk1 - 1 - blk0) % NW;
    const int nk = blk1 - blk0 > wv ? (blk1 - blk0 - wv + NW - 1) / NW : 0;
    const TableBlocks src{p.block_tables + (int64_t)s * p.max_blocks_per_seq, blk0 + wv, NW, nk, tok1};
    float m, l;
    floatx4 acc[D / 16];
    walk_blocks<KV, D, STREAM, APPEND, TableBlocks, NB>(p, s, g, src, query_column<D>(p, s, g), p.group, ctx,
                                                         writer, sm.tok_k, sm.tok_v, m, l, acc);
    state_to_lds<D, NW, W>(sm, wv, m, l, acc);
    __syncthreads();
    merge_and_store<D, NW>(p, sm, s, g, part, nparts <= 1, NW, threadIdx.x, 64 * NW, p.group);
}

__device__ __forceinline__ int clamp_ctx(const DecodeParams &p, int ctx) {
    const int cap = p.max_blocks_per_seq * kBlock;
    return ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
}

// One workgroup of NW wavefronts per (sequence, KV head, partition) slot of
// a rows x max_partitions grid.
// NB: register buffers per wavefront (blocks in flight); three take 200 VGPRs
// (2 waves/SIMD) at head dim 128.
template <int KV, int D, bool STREAM, int NW, bool APPEND, int NB = 2>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NB == 3 ? 2 : 3))) void decode_mfma_kernel(DecodeParams p) {
    __shared__ DecodeLds<D, NW> sm;
    // Work order: the first num_seqs x num_kv_heads workgroups take partition
    // 0 of every (sequence, KV head) pair -- all real work, spread evenly over
    // the eight XCDs (workgroup i runs on XCD i % 8).  The others take
    // partitions 1.. of one pair each, rotated by the pair index, so the
    // empty slots of pairs with fewer partitions than the longest stay mixed
    // with real work rather than piling up at the end.  The plain order
    // (partition fastest) had slowed long-tail batches up to 3x at some
    // partition lengths.
    int bid, part;
    pair_and_partition(p.num_seqs * p.num_kv_heads, p.max_partitions, bid, part);
    const int g = bid % p.num_kv_heads;
    const int s = sequence_of_rank(p.context_lens, p.num_seqs, p.max_blocks_per_seq * kBlock,
                                   bid / p.num_kv_heads);
    const int raw_ctx = p.context_lens[s];
    const int ctx = clamp_ctx(p, raw_ctx);
    decode_item<KV, D, STREAM, NW, APPEND, NB>(p, s, g, part, ctx, raw_ctx > ctx, sm);
}

// Partition groups: one workgroup of NG wavefronts per (sequence, KV head,
// group of NG consecutive partitions) slot of a rows x max_partitions grid
// (work order as above).  Wavefront w walks partition NG * group + w alone,
// its blocks in order, with its own softmax state.  The wavefront that
// finishes last -- counted with an LDS atomic, so that no wavefront waits for
// another -- merges the group's states and writes them once: the output row
// when the group covers the whole context, else the group's partial result
// for the reduce kernel.  HBM so sees one partial per NG partitions instead
// of one per partition, and contexts of up to NG partitions need no reduce.
// Wavefronts with no partition (past the end of a short context) leave at
// once, after the one barrier that publishes the cleared counter.
// NC: LDS columns, 8 when the group has at most 8 query heads (half the LDS,
// so more partly filled workgroups fit a CU: the fp8 long tail 0.1657 ->
// 0.1648 ms), else 16.
template <int KV, int D, bool STREAM, int NG, bool APPEND, int NC>
__global__ __launch_bounds__(64 * NG) __attribute__((amdgpu_waves_per_eu(3))) void decode_group_kernel(DecodeParams p) {
    __shared__ DecodeLds<D, NG, NC> sm;
    constexpr int W = KV == kBF16 ? 2 : 4;
    int bid, grp;
    pair_and_partition(p.num_seqs * p.num_kv_heads, p.max_partitions, bid, grp);
    const int g = bid % p.num_kv_heads;
    const int s = sequence_of_rank(p.context_lens, p.num_seqs, p.max_blocks_per_seq * kBlock,
                                   bid / p.num_kv_heads);
    const int raw_ctx = p.context_lens[s];
    const int ctx = clamp_ctx(p, raw_ctx);
    const int ptok = p.partition_tokens;
    const int nparts = (ctx + ptok - 1) / ptok;
    const int ngroups = (nparts + NG - 1) / NG;
    if (grp >= (ngroups > 1 ? ngroups : 1)) return;     // the whole workgroup
    if (threadIdx.x == 0) sm.done = 0u;
    __syncthreads();
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // partitions of this group; an empty context has one (wavefront 0 writes
    // its zero row)
    const int nreal = nparts <= grp * NG ? 1 : min(NG, nparts - grp * NG);
    if (wv >= nreal) return;
    const int tok0 = (grp * NG + wv) * ptok;
    const int tok1 = min(ctx, tok0 + ptok);
    const int blk0 = tok0 / kBlock;
    const int blk1 = (tok1 + kBlock - 1) / kBlock;
    // the newest token is written by the wavefront whose partition holds it
    const bool writer = APPEND && raw_ctx == ctx && tok1 == ctx && ctx > 0;
    const TableBlocks src{p.block_tables + (int64_t)s * p.max_blocks_per_seq, blk0, 1, blk1 - blk0, tok1};
    float m, l;
    floatx4 acc[D / 16];
    walk_blocks<KV, D, STREAM, APPEND>(p, s, g, src, query_column<D>(p, s, g), p.group, ctx, writer,
                                       sm.tok_k, sm.tok_v, m, l, acc);
    state_to_lds<D, NG, W, NC>(sm, wv, m, l, acc);
    // this wavefront's state is in LDS before it counts itself as done; the
    // last one to count sees every other state
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    uint32_t before = 0u;
    if ((threadIdx.x & 63) == 0)
        before = __hip_atomic_fetch_add(&sm.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    before = __builtin_amdgcn_readfirstlane(before);
    if (before != (uint32_t)(nreal - 1)) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    merge_and_store<D, NG, NC>(p, sm, s, g, grp, ngroups <= 1, nreal, threadIdx.x & 63, 64, p.group);
}

// Blocks of one partition of a prefix-sharing group, from the list its
// workgroup built in LDS: entry v names the physical block and which tokens
// and columns attend it ((first column << 16) | (end column << 8) | tokens).
// The wavefront takes entries jb + stride k (k < nk).
struct ListBlocks {
    static constexpr bool kColumnMask = true;
    const int32_t *ids;
    const int32_t *info;
    int jb, stride, nk;
    __device__ __forceinline__ int32_t id(int k) const {
        const int32_t b = __builtin_amdgcn_readfirstlane(ids[jb + stride * min(k, nk - 1)]);
        return k < nk ? b : -1;
    }
    __device__ __forceinline__ int block(int) const { return -1; }
    __device__ __forceinline__ void mask(int k, int &nvalid, int &lo, int &hi) const {
        const int x = __builtin_amdgcn_readfirstlane(info[jb + stride * k]);
        nvalid = x & 0xff;
        hi = (x >> 8) & 0xff;
        lo = x >> 16;
    }
};

template <int D, int NW>
struct SharedLds {
    DecodeLds<D, NW> st;
    int32_t ids[kSharedListMax];
    int32_t info[kSharedListMax];
    int32_t member_ctx[16];
    int32_t member_cum[17];   // suffix blocks of the members before member m
};

// Decode of prefix-sharing groups: one workgroup of NW wavefronts per
// (group, KV head, partition) slot of a (groups x KV heads) x max_partitions
// grid (work order as above).  The members of a group hold the same first
// pb blocks in their tables -- a prompt shared by parallel samples or beams,
// a cached system prompt (glossary page, sharing blocks between sequences).
// Every query head of every member is a column of one 16-column matrix-core
// tile (members x G <= 16), so each shared block is read once for the whole
// group; each member's own blocks after the shared ones are attended by that
// member's columns only (the others' scores are -inf there).  The group's
// blocks, shared ones first, then member 0's own, member 1's, ..., form a
// list cut into partitions of partition_tokens / 16 blocks; the workgroup
// lists its partition's blocks in LDS and its wavefronts take every NW-th
// entry.  A group with one partition writes its output rows at once, else
// one partial per member row for the shared reduce kernel.
template <int KV, int D, bool STREAM, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(3))) void decode_shared_kernel(DecodeParams p) {
    __shared__ SharedLds<D, NW> sm;
    constexpr int W = KV == kBF16 ? 2 : 4;
    int bid, part;
    pair_and_partition(p.num_groups * p.num_kv_heads, p.max_partitions, bid, part);
    const int gi = bid / p.num_kv_heads;
    const int g = bid % p.num_kv_heads;
    const int G = p.group;
    const int lane = threadIdx.x & 63;
    const int cap = p.max_blocks_per_seq * kBlock;
    // the group's members (device data: clamped to the batch and max_group)
    const int s0 = p.group_start[gi];
    int M = p.group_start[gi + 1] - s0;
    if (s0 < 0 || s0 >= p.num_seqs) M = 0;
    M = M < 0 ? 0 : min(M, min(p.max_group, p.num_seqs - s0));
    M = __builtin_amdgcn_readfirstlane(M);
    if (M == 0) return;
    // members' context lengths, the shared whole blocks (at most what every
    // member holds) and each member's own blocks after them
    int myctx = 0x7fffffff;
    if (lane < M) {
        const int c = p.context_lens[s0 + lane];
        myctx = c < 0 ? 0 : (c > cap ? cap : c);
    }
    int minctx = myctx;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) minctx = min(minctx, __shfl_xor(minctx, o));
    minctx = __builtin_amdgcn_readfirstlane(minctx);
    int pb = p.prefix_blocks[gi];
    pb = __builtin_amdgcn_readfirstlane(max(0, min(pb, minctx / kBlock)));
    const int own = lane < M ? (myctx + kBlock - 1) / kBlock - pb : 0;
    int cum = own;   // inclusive prefix sum over members
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
        const int t = __shfl_up(cum, o);
        if (lane >= o) cum += t;
    }
    const int total = pb + __builtin_amdgcn_readlane(cum, 15);
    const int B = p.partition_tokens / kBlock;
    const int nparts = (total + B - 1) / B;
    if (part >= (nparts > 1 ? nparts : 1)) return;   // the whole workgroup
    if (threadIdx.x < 16) {
        sm.member_ctx[threadIdx.x] = lane < M ? myctx : 0;
        sm.member_cum[threadIdx.x] = cum - own;   // exclusive
    }
    if (threadIdx.x == 16) sm.member_cum[16] = total - pb;
    if (part == 0 && g == 0 && threadIdx.x == 0 && p.ws_nparts) p.ws_nparts[gi] = nparts;
    __syncthreads();
    // this partition's blocks: shared ones (every member's columns) or
    // member m's own (its columns), with the tokens attended
    const int v0 = part * B;
    const int nv = min(total, v0 + B) - v0;
    const int32_t *tables = p.block_tables;
    for (int t = threadIdx.x; t < nv; t += 64 * NW) {
        const int v = v0 + t;
        int mem = 0, j = v, lo = 0, hi = M * G, nvalid = kBlock;
        if (v >= pb) {
            const int u = v - pb;
            for (int mm = 1; mm < M; ++mm)
                if (u >= sm.member_cum[mm]) mem = mm;
            j = pb + u - sm.member_cum[mem];
            lo = mem * G;
            hi = lo + G;
            nvalid = min(kBlock, sm.member_ctx[mem] - j * kBlock);
        }
        sm.ids[t] = tables[(int64_t)(s0 + mem) * p.max_blocks_per_seq + j];
        sm.info[t] = (lo << 16) | (hi << 8) | nvalid;
    }
    __syncthreads();
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nk = nv > wv ? (nv - wv + NW - 1) / NW : 0;
    const ListBlocks src{sm.ids, sm.info, wv, NW, nk};
    // column n: query head g G + n % G of member n / G
    const int n = lane & 15;
    const uint16_t *qcol = n < M * G ? reinterpret_cast<const uint16_t *>(p.q) +
                                           ((int64_t)(s0 + n / G) * p.num_q_heads + (int64_t)g * G + n % G) * D
                                     : nullptr;
    float m, l;
    floatx4 acc[D / 16];
    walk_blocks<KV, D, STREAM, false>(p, s0, g, src, qcol, M * G, 1, false, sm.st.tok_k, sm.st.tok_v, m, l,
                                      acc);
    state_to_lds<D, NW, W>(sm.st, wv, m, l, acc);
    __syncthreads();
    merge_and_store<D, NW>(p, sm.st, s0, g, part, nparts <= 1, NW, threadIdx.x, 64 * NW, M * G);
}

template <int KV, int D, bool STREAM, bool APPEND>
hipError_t launch_variant(const DecodeParams &p, int64_t grid, hipStream_t stream, const LaunchEvents *ev) {
    // one-wavefront workgroups walk all of a partition's blocks and need no
    // merge; the caller picks them for batches with at least two (sequence,
    // KV head) rows per SIMD, and partition groups for short partitions
    const dim3 g((unsigned)grid);
    if (p.wave_mode == kFourWaves)
        return launch_kernel(decode_mfma_kernel<KV, D, STREAM, 4, APPEND>, g, dim3(256), stream, ev, p);
    if constexpr (KV == kBF16) {
        if (p.wave_mode == kOneWaveDeep)
            return launch_kernel(decode_mfma_kernel<KV, D, STREAM, 1, APPEND, 3>, g, dim3(64), stream, ev, p);
    }
    if (p.wave_mode == kOneWave || p.wave_mode == kOneWaveDeep)
        return launch_kernel(decode_mfma_kernel<KV, D, STREAM, 1, APPEND>, g, dim3(64), stream, ev, p);
    if (p.group <= 8)
        return launch_kernel(decode_group_kernel<KV, D, STREAM, kGroupParts, APPEND, 8>, g,
                             dim3(64 * kGroupParts), stream, ev, p);
    return launch_kernel(decode_group_kernel<KV, D, STREAM, kGroupParts, APPEND, 16>, g, dim3(64 * kGroupParts),
                         stream, ev, p);
}

template <int KV, int D>
hipError_t launch(const DecodeParams &p, hipStream_t stream, const LaunchEvents *ev) {
    const int64_t grid = (int64_t)p.num_seqs * p.num_kv_heads * p.max_partitions;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    const bool append = p.k_new != nullptr;
    if (p.shared_kv)
        return append ? launch_variant<KV, D, false, true>(p, grid, stream, ev)
                      : launch_variant<KV, D, false, false>(p, grid, stream, ev);
    return append ? launch_variant<KV, D, true, true>(p, grid, stream, ev)
                  : launch_variant<KV, D, true, false>(p, grid, stream, ev);
}

template <int KV, int D>
hipError_t launch_shared(const DecodeParams &p, hipStream_t stream, const LaunchEvents *ev) {
    const int64_t grid = (int64_t)p.num_groups * p.num_kv_heads * p.max_partitions;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    const dim3 g((unsigned)grid), b(256);
    if (p.shared_kv) return launch_kernel(decode_shared_kernel<KV, D, false, 4>, g, b, stream, ev, p);
    return launch_kernel(decode_shared_kernel<KV, D, true, 4>, g, b, stream, ev, p);
}

}  // namespace

hipError_t launch_decode_shared(int kv, int head_dim, const DecodeParams &p, hipStream_t stream,
                                const LaunchEvents *ev) {
    if (kv == kBF16)
        return head_dim == 64 ? launch_shared<kBF16, 64>(p, stream, ev) : launch_shared<kBF16, 128>(p, stream, ev);
    return head_dim == 64 ? launch_shared<kFP8, 64>(p, stream, ev) : launch_shared<kFP8, 128>(p, stream, ev);
}

bool mfma_path_supported(int kv, int head_dim, int group) {
    return (kv == kBF16 || kv == kFP8) && (head_dim == 64 || head_dim == 128) && group >= 2 &&
           group <= 16;
}

hipError_t launch_decode_mfma(int kv, int head_dim, const DecodeParams &p, hipStream_t stream,
                              const LaunchEvents *ev) {
    if (kv == kBF16)
        return head_dim == 64 ? launch<kBF16, 64>(p, stream, ev) : launch<kBF16, 128>(p, stream, ev);
    return head_dim == 64 ? launch<kFP8, 64>(p, stream, ev) : launch<kFP8, 128>(p, stream, ev);
}

}  // namespace pa
