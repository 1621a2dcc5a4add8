// pa_prefill.hip -- paged (chunked) prefill attention on matrix cores.
//
// What is computed: each sequence's chunk of new tokens -- the last n of its
// ctx cached tokens, whose K/V the cache write has already stored -- attends
// causally over the paged context: the chunk token at position p sees the
// K/V of tokens 0..p, the tokens generation would have seen when producing
// it (French page, second article, what the KV cache is).  The context is
// read block by block through the block table ("PagedAttention" glossary
// page, how paging works), which is what the glossary page's related
// techniques call FlashAttention-style kernels that read paged blocks: the
// scores are never written to memory, an online softmax keeps a running max
// and sum per row.
//
// Rows and work split.  The query heads of one KV head g (G = Hq / Hkv of
// them) and BQ = 128 / G consecutive chunk tokens form 128 rows
// (row r = token r / G, head g G + r % G); one workgroup (4 wavefronts) takes
// one such tile of one sequence, and each wavefront owns 32 of its rows as
// two 16-column matrix-core groups.  Workgroups are issued latest tile
// first, so the longest causal ranges start first.
//
// Staging.  The workgroup walks blocks 0 .. (its last row's position) / 16.
// Every block's K and V tiles are loaded once per workgroup and written to
// one of two LDS stages (the next block is already in flight in registers
// while the current one is computed, and is written to the other stage
// afterwards; one barrier per block).  The stage holds K as bf16 runs and V as
// duplicated bf16 cells that are directly the A operands of both products
// (fp8 widened and tokens past the context zeroed once, at staging).
//
// Per block, for each 16-row group (operand layouts as in the grouped decode
// kernel):
//     S^T[16 tokens][16 rows]  = K[16][D] . Q^T[D][16]
//     O^T[D][16 rows]         += V^T[D][16 tokens] . P^T[16][16]
// with P carried as bf16 hi + lo (16 significant bits).  Causal masking sets
// the score of every token past a row's position to -inf (selection).  The
// running maximum is raised lazily: only when some lane's block maximum
// exceeds it by more than 8 (in log2 units) is the row maximum exchanged
// across lanes and are the numerators rescaled, so probabilities stay below
// 2^8 and most blocks skip both.
#include "pa_internal.h"
#include "pa_mfma_util.h"

#include <type_traits>

namespace pa {
namespace {

constexpr int kGroups = 2;                                    // 16-row groups per wavefront
constexpr int kRowsPerWave = 16 * kGroups;                    // 32
constexpr int kRowsPerTile = kRowsPerWave * (kThreads / 64);  // 128
constexpr float kLazyMax = 8.0f;  // rescale when a block's max exceeds the running max by 2^8

// [hi(p0..p3) | lo(p0..p3)] as bf16 pairs, packed with byte permutes: hi keeps
// each p's top 16 bits, lo the top 16 bits of the remainder
__device__ __forceinline__ bf16x8 p_hi_lo_perm(const float (&pr)[4]) {
    uint32_t u[4], r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        u[i] = __float_as_uint(pr[i]);
        r[i] = __float_as_uint(pr[i] - __uint_as_float(u[i] & 0xffff0000u));
    }
    const u32x4 w = {__builtin_amdgcn_perm(u[1], u[0], 0x07060302u),
                     __builtin_amdgcn_perm(u[3], u[2], 0x07060302u),
                     __builtin_amdgcn_perm(r[1], r[0], 0x07060302u),
                     __builtin_amdgcn_perm(r[3], r[2], 0x07060302u)};
    return as_bf16x8(w);
}

template <int KV, int D>
__global__ __launch_bounds__(kThreads) void prefill_mfma_kernel(PrefillParams p) {
    constexpr int EB = KV == kBF16 ? 2 : 1;
    constexpr int TILE_BYTES = kBlock * D * EB;                  // one pool tile (K or V)
    // LDS stage: K as a bf16 tile in the bf16 pool order (D/8 runs x 16 tokens
    // x 16 bytes), then V as D x 4 duplicated bf16 cells: cell (token group
    // tg, dim d) = [t0 t1 | t2 t3 | t0 t1 | t2 t3] of dim d, tokens 4 tg..4 tg+3,
    // zeroed past the context -- exactly the A operand [V | V] of the
    // hi + lo P.V product
    constexpr int KS_UNITS = kBlock * D * 2 / 16;
    constexpr int VS_UNITS = 4 * D;
    constexpr int STAGE_UNITS = KS_UNITS + VS_UNITS;
    constexpr int NQK = D / 32;  // 32-deep q.K steps per block
    constexpr int NT = D / 16;   // 16 x 16 output tiles per group: tile T = head dims 16 T .. 16 T + 15

    __shared__ __attribute__((aligned(16))) u32x4 stage[2][STAGE_UNITS];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 15;
    const int c = lane >> 4;

    const int G = p.group;
    const int BQ = kRowsPerTile / G;
    const int sg = p.num_seqs * p.num_kv_heads;
    const int tile = p.num_tiles - 1 - (int)(blockIdx.x / sg);
    const int s = (int)(blockIdx.x % sg) / p.num_kv_heads;
    const int g = (int)(blockIdx.x % sg) % p.num_kv_heads;

    int ctx = p.context_lens[s];
    ctx = ctx < 0 ? 0 : (ctx > p.max_blocks_per_seq * kBlock ? p.max_blocks_per_seq * kBlock : ctx);
    const int q0 = p.query_start[s];
    int n_chunk = p.query_start[s + 1] - q0;
    n_chunk = n_chunk < 0 ? 0 : n_chunk;
    const int first = ctx - n_chunk;  // position of chunk token 0 (< 0: chunk longer than context)
    // only the chunk's first max_query_len tokens are computed, each at its own position
    const int n_new = n_chunk > p.max_query_len ? p.max_query_len : n_chunk;
    if (tile * BQ >= n_new) return;
    // the workgroup's blocks: up to its last row's position
    const int pos_last = first + min(tile * BQ + BQ, n_new) - 1;
    const int nblk_wg = pos_last < 0 ? 0 : pos_last / kBlock + 1;

    // this lane's two rows (one per group): chunk token, head, position
    int row_tok[kGroups], row_head[kGroups], pos_mask[kGroups];
    bool valid[kGroups], live[kGroups];
    int minpos = 0x7fffffff;
#pragma unroll
    for (int k = 0; k < kGroups; ++k) {
        const int r = kRowsPerWave * wave + 16 * k + n;
        row_tok[k] = tile * BQ + r / G;
        row_head[k] = g * G + r % G;
        valid[k] = r < BQ * G && row_tok[k] < n_new;
        const int pos = first + row_tok[k];
        live[k] = valid[k] && pos >= 0;
        // rows that produce no output are masked like the context's last token
        pos_mask[k] = live[k] ? pos : ctx - 1;
        minpos = min(minpos, pos_mask[k]);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) minpos = min(minpos, __shfl_xor(minpos, o));
    // the same in every lane: as a uniform value the per-block mask test is a
    // scalar branch, not an exec-masked region issued on every block
    minpos = __builtin_amdgcn_readfirstlane(minpos);

    // Q^T operands (zero for rows outside the chunk): head dims 8 (4 u + c) .. +7
    // for step u, matching the staged bf16 K runs
    bf16x8 qop[kGroups][NQK];
#pragma unroll
    for (int k = 0; k < kGroups; ++k) {
        const uint16_t *qrow = reinterpret_cast<const uint16_t *>(p.q) +
                               ((int64_t)(q0 + row_tok[k]) * p.num_q_heads + row_head[k]) * D;
#pragma unroll
        for (int u = 0; u < NQK; ++u) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (valid[k]) v = *reinterpret_cast<const u32x4 *>(qrow + 8 * (4 * u + c));
            qop[k][u] = as_bf16x8(v);
        }
    }

    float m[kGroups], m_lazy[kGroups], m_use[kGroups], l[kGroups];  // m_lazy = m + kLazyMax
    floatx4 acc[kGroups][NT];
#pragma unroll
    for (int k = 0; k < kGroups; ++k) {
        m[k] = kNegInfF;
        m_lazy[k] = kNegInfF;
        m_use[k] = 0.f;
        l[k] = 0.f;
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[k][t] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

    const int32_t *table = p.block_tables + (int64_t)s * p.max_blocks_per_seq;
    const char *kpool = static_cast<const char *>(p.k_pool);
    const char *vpool = static_cast<const char *>(p.v_pool);
    auto ok = [&](int32_t b) { return b >= 0 && b < p.num_blocks; };

    // Staging.  K: thread t < KU loads pool unit t of the block's K tile and
    // writes it to the stage (fp8: widened to two bf16 runs).  V: thread t
    // writes stage cells t, t + 256, ... (cell (tg, d) = unit tg * D + d) and
    // loads the words of dim d from the pool cell holding it (bf16: 8 bytes,
    // fp8: 4); the lanes of one pool cell together load its 16 bytes.  Every lane writes one whole 16-byte
    // unit after its neighbour's, which keeps the LDS stores free of bank
    // conflicts.  The loads go through tile resources, so a lane past the K
    // tile, or a block id out of range, loads zeros without touching memory.
    constexpr int KU = TILE_BYTES / 16;   // K pool units per block (<= 256)
    constexpr int VLOADS = VS_UNITS / kThreads;
    constexpr int W = 4 / EB;             // head dims per pool V cell
    static_assert(KU <= kThreads && VS_UNITS % kThreads == 0, "staging split");
    using VWords = typename std::conditional<KV == kBF16, uint2, uint32_t>::type;
    auto gload = [&](int32_t b, u32x4 &kr, VWords (&vr)[VLOADS]) {
        const bool good = ok(b);
        const int64_t off = ((int64_t)(good ? b : 0) * p.num_kv_heads + g) * TILE_BYTES;
        const auto kt = tile_rsrc(kpool + off, good ? TILE_BYTES : 0);
        const auto vt = tile_rsrc(vpool + off, good ? TILE_BYTES : 0);
        kr = load_tile<false>(kt, threadIdx.x * 16);
#pragma unroll
        for (int i = 0; i < VLOADS; ++i) {
            const int su = threadIdx.x + i * kThreads;
            const int tg = su / D, d = su % D;
            const int off = (tg * (D / W) + d / W) * 16 + (d % W) * (4 * EB);
            if constexpr (KV == kBF16)
                vr[i] = load_tile_b64(vt, off);
            else
                vr[i] = load_tile_b32(vt, off);
        }
    };
    // ... and writes them to a stage in the LDS order above (fp8 widened to
    // bf16, exact); V of tokens at or past `nvalid` is zeroed
    auto swrite = [&](int st, const u32x4 &kr, const VWords (&vr)[VLOADS], int nvalid) {
        u32x4 *ks = stage[st];
        u32x4 *vs = stage[st] + KS_UNITS;
        const int t = threadIdx.x;
        if (t < KU) {
            if constexpr (KV == kBF16) {
                ks[t] = kr;
            } else {  // fp8 run t / 16 (16 dims) of token t % 16 -> two bf16 runs
                const int rr = t >> 4, tt = t & 15;
                uint32_t a0, a1, a2, a3, b0, b1, b2, b3;
                e4m3x4_to_bf16(kr[0], a0, a1);
                e4m3x4_to_bf16(kr[1], a2, a3);
                e4m3x4_to_bf16(kr[2], b0, b1);
                e4m3x4_to_bf16(kr[3], b2, b3);
                ks[(2 * rr) * kBlock + tt] = u32x4{a0, a1, a2, a3};
                ks[(2 * rr + 1) * kBlock + tt] = u32x4{b0, b1, b2, b3};
            }
        }
#pragma unroll
        for (int i = 0; i < VLOADS; ++i) {
            const int su = t + i * kThreads;
            uint32_t w0, w1;  // tokens (t0 t1) and (t2 t3) of dim d as bf16 pairs
            if constexpr (KV == kBF16) {
                w0 = vr[i].x;
                w1 = vr[i].y;
            } else {
                e4m3x4_to_bf16(vr[i], w0, w1);
            }
            if (nvalid < kBlock) {  // the context's last block: zero the tokens past it
                uint32_t k01, k23;
                v_keep_masks(su / D, nvalid, k01, k23);
                w0 &= k01;
                w1 &= k23;
            }
            // The upper pair as explicit copies: from the duplicated pair
            // {w0, w1, w0, w1} this compiler (hipcc of ROCm 7.2) has emitted
            // a 16-byte store whose upper half was the address register.
            uint32_t c0, c1;
            asm("v_mov_b32 %0, %2\n\tv_mov_b32 %1, %3" : "=v"(c0), "=v"(c1) : "v"(w0), "v"(w1));
            vs[su] = u32x4{w0, w1, c0, c1};
        }
    };

    // Block j from stage st.  `bias` is -inf when the block id is out of
    // range (its zero K gives zero scores, and every token is masked) and 0
    // otherwise, which leaves the product's rounding unchanged; MASK: some
    // row's position falls inside the block (the causal mask is applied).
    auto compute_block = [&](auto mask_tag, int st, int j, float bias) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const u32x4 *ks = stage[st] + c * kBlock + n;  // K run c (+ 4 per step), token n
        const u32x4 *vs = stage[st] + KS_UNITS + c * D + n;  // V cell (token group c, dim n (+ 16 T))
        bf16x8 kop[NQK];
#pragma unroll
        for (int u = 0; u < NQK; ++u) kop[u] = as_bf16x8(ks[u * 4 * kBlock]);

        // scores of both groups first, so their matrix-core products issue back to back
        floatx4 sacc[kGroups];
#pragma unroll
        for (int k = 0; k < kGroups; ++k) {
            sacc[k] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < NQK; ++u)
                sacc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[u], qop[k][u], sacc[k], 0, 0, 0);
        }
        // Scaled scores; tokens 4c + i past a row's position are masked by
        // selection.  The scaled score itself (not a fused multiply-add with
        // the max) enters the exponent, so the token holding the max gets
        // probability exactly 1.
        float sc[kGroups][4], bl[kGroups];
        bool want = false;
#pragma unroll
        for (int k = 0; k < kGroups; ++k) {
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[k][i] = __builtin_fmaf(sacc[k][i], p.qk_scale_log2, bias);
            if constexpr (MASK) {
                const int lim = pos_mask[k] - j * kBlock - 4 * c;
#pragma unroll
                for (int i = 0; i < 4; ++i) sc[k][i] = i > lim ? kNegInfF : sc[k][i];
            }
            bl[k] = fmaxf(fmaxf(sc[k][0], sc[k][1]), fmaxf(sc[k][2], sc[k][3]));
            want = want || bl[k] > m_lazy[k];
        }
        // the row max is exchanged across lanes, and the running max raised
        // (rescaling the numerators), only when some lane's block max exceeds
        // the running max by more than the margin; otherwise every probability
        // stays below 2^8 and the max stays put
        if (__builtin_amdgcn_ballot_w64(want) != 0) {
#pragma unroll
            for (int k = 0; k < kGroups; ++k) {
                const float bm = max_xor32(max_xor16(bl[k]));
                const bool grow = bm > m_lazy[k];
                const float m_new = grow ? bm : m[k];
                const float mu = m_new == kNegInfF ? 0.f : m_new;
                const float alpha = grow ? __builtin_amdgcn_exp2f(m[k] - mu) : 1.f;
                m[k] = m_new;
                m_lazy[k] = m_new + kLazyMax;
                m_use[k] = mu;
                l[k] *= alpha;
#pragma unroll
                for (int t = 0; t < NT; ++t) acc[k][t] *= alpha;
            }
        }
        bf16x8 pop[kGroups];
#pragma unroll
        for (int k = 0; k < kGroups; ++k) {
            float pr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(sc[k][i] - m_use[k]);
            l[k] += (pr[0] + pr[1]) + (pr[2] + pr[3]);
            pop[k] = p_hi_lo_perm(pr);
        }

        // O^T += V^T . P^T: the staged cell is the ready [V | V] operand
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const bf16x8 a = as_bf16x8(vs[16 * t]);
#pragma unroll
            for (int k = 0; k < kGroups; ++k)
                acc[k][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pop[k], acc[k][t], 0, 0, 0);
        }
    };

    // Block ids come by scalar loads from the table, two blocks ahead.  Block
    // j is computed from stage j & 1 while block j + 1 is in flight in
    // registers; block j + 1 then goes to the other stage and block j + 2's
    // loads are issued (every step issues the same loads), and one barrier
    // ends the step.
    auto id_at = [&](int j) -> int32_t {
        const int32_t b = table[min(j, nblk_wg - 1)];
        return j < nblk_wg ? b : -1;
    };
    if (nblk_wg > 0) {
        int32_t id_cur = id_at(0), id_next = id_at(1);
        u32x4 kpre;
        VWords vpre[VLOADS];
        gload(id_cur, kpre, vpre);
        swrite(0, kpre, vpre, ctx);
        gload(id_next, kpre, vpre);
        __syncthreads();
        // blocks before jm lie at or before every row's position of the
        // wavefront (no causal mask); the rest are masked
        const int jm = min((minpos + 1) / kBlock, nblk_wg);
        auto next = [&](int j) {
            const int32_t id_after = id_at(j + 2);
            if (j + 1 < nblk_wg) swrite((j + 1) & 1, kpre, vpre, ctx - (j + 1) * kBlock);
            gload(id_after, kpre, vpre);
            id_cur = id_next;
            id_next = id_after;
            __syncthreads();
        };
        // Every wavefront computes every block of the workgroup: blocks past
        // its own rows are masked out by the causal test (at most one block
        // for G = 8), and a straight-line loop body keeps the accumulators
        // in place.
        for (int j = 0; j < jm; ++j) {
            compute_block(std::false_type{}, j & 1, j, ok(id_cur) ? 0.f : kNegInfF);
            next(j);
        }
        for (int j = jm; j < nblk_wg; ++j) {
            compute_block(std::true_type{}, j & 1, j, ok(id_cur) ? 0.f : kNegInfF);
            next(j);
        }
    }

    // rows: out = O / l (times v_scale); rows before the context start are zero.
    // Tile T element i is head dim 16 T + 4 c + i: one float4 per tile.
#pragma unroll
    for (int k = 0; k < kGroups; ++k) {
        float lt = l[k];
        lt = add_xor32(add_xor16(lt));
        if (!valid[k]) continue;
        const float f = live[k] && lt > 0.f ? p.out_scale / lt : 0.f;
        float *orow = p.out + ((int64_t)(q0 + row_tok[k]) * p.num_q_heads + row_head[k]) * D;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float4 v = live[k] ? make_float4(acc[k][t][0] * f, acc[k][t][1] * f, acc[k][t][2] * f,
                                                   acc[k][t][3] * f)
                                     : make_float4(0.f, 0.f, 0.f, 0.f);
            *reinterpret_cast<float4 *>(orow + 16 * t + 4 * c) = v;
        }
    }
}

template <int KV, int D>
hipError_t launch(const PrefillParams &p, hipStream_t stream, const LaunchEvents *ev) {
    const int64_t grid = (int64_t)p.num_tiles * p.num_seqs * p.num_kv_heads;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    return launch_kernel(prefill_mfma_kernel<KV, D>, dim3((unsigned)grid), dim3(kThreads), stream, ev, p);
}

}  // namespace

int prefill_tile_tokens(int head_dim, int group) { return (void)head_dim, kRowsPerTile / group; }

bool prefill_supported(int kv, int head_dim, int group) {
    return (kv == kBF16 || kv == kFP8) && (head_dim == 64 || head_dim == 128) && group >= 1 &&
           group <= kRowsPerTile;
}

hipError_t launch_prefill(int kv, int head_dim, const PrefillParams &p, hipStream_t stream,
                          const LaunchEvents *ev) {
    if (kv == kBF16)
        return head_dim == 64 ? launch<kBF16, 64>(p, stream, ev) : launch<kBF16, 128>(p, stream, ev);
    return head_dim == 64 ? launch<kFP8, 64>(p, stream, ev) : launch<kFP8, 128>(p, stream, ev);
}

}  // namespace pa
