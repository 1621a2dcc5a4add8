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
// two 16-column matrix-core groups.  The tiles of one (sequence, KV head)
// pair run together on one XCD, latest tile (longest causal range) first.
//
// Staging.  The workgroup walks its blocks 0 .. (its last row's position) / 16
// two at a time: a step covers blocks 2 i and 2 i + 1.  Every step's K and V
// tiles are loaded once per workgroup and written to one of two LDS stages (the
// next step is already in flight in registers while the current one is
// computed, and is written to the other stage afterwards; one barrier per
// step).  The stage holds K as bf16 runs and V as fp16 cells that are directly
// the A operands of both products (fp8 widened, bf16 V narrowed to fp16, and
// tokens past the context zeroed once, at staging).
//
// Per step, for each 16-row group (operand layouts as in the grouped decode
// kernel):
//     S^T[16 tokens][16 rows]  = K[16][D] . Q^T[D][16]           (each block)
//     O^T[D][16 rows]         += V^T[D][32 tokens] . P^T[32][16]  (both blocks)
// with P rounded to fp16 for the second product (relative error <= 2^-11;
// the row sum adds the same rounded values).  fp16 holds every E4M3 value
// exactly, and a bf16 value exactly when its magnitude lies in [2^-14, 2^16)
// and within 2^-25 below it; bf16 V of magnitude 2^16 or more is outside the
// kernel's domain (it becomes infinite).  Causal masking sets the score
// of every token past a row's position to -inf (selection).  The running
// maximum is raised lazily: only when some lane's exponent exceeds it by
// more than 8 (in log2 units) is the row maximum exchanged across lanes and
// are the numerators rescaled, so probabilities stay below 2^8 and most steps
// skip both.
#include "pa_internal.h"
#include "pa_mfma_util.h"

#include <type_traits>

namespace pa {
namespace {

constexpr int kGroups = 2;                                    // 16-row groups per wavefront
constexpr int kRowsPerWave = 16 * kGroups;                    // 32
constexpr int kRowsPerTile = kRowsPerWave * (kThreads / 64);  // 128
constexpr int kXcds = 8;          // accelerator complex dies; workgroup b runs on XCD b % 8
constexpr float kLazyMax = 8.0f;  // rescale when a step's max exceeds the running max by 2^8

// Pairs interleaved per XCD.  When every chunk may span its whole context
// (whole prompts: the tiles of a pair range from one block to the full
// causal length) and a pair has few tiles, the last pair's longest tile
// would start last and run alone; taking 4 pairs together, their tiles
// interleaved longest first, shortens that tail.  Chunks over long cached
// contexts (tiles of nearly equal length, more tiles per pair) keep one pair
// at a time, which keeps the blocks in flight in the XCD's L2.
__host__ __device__ __forceinline__ int pair_window(const PrefillParams &p) {
    return (p.num_tiles <= 16 && 2 * (int64_t)p.max_query_len >= (int64_t)p.max_blocks_per_seq * kBlock) ? 4
                                                                                                         : 1;
}

__device__ __forceinline__ uint32_t f16x2_bits(f16x2 h) { return __builtin_bit_cast(uint32_t, h); }

// two bf16 (one word) -> two fp16 (one word), rounded to nearest: exact for
// magnitudes in [2^-14, 2^16) (fp16 keeps bf16's 8 significant bits), within
// 2^-25 below (the fp16 subnormal grid is 2^-24); 2^16 and above overflow
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
    const f16x2 h = {(_Float16)__uint_as_float(w << 16), (_Float16)__uint_as_float(w & 0xffff0000u)};
    return f16x2_bits(h);
}

// four E4M3 codes -> four fp16 (exact: E4M3 has 4 significant bits and
// exponents -9 .. 8, all inside fp16)
__device__ __forceinline__ void e4m3x4_to_f16(uint32_t w, uint32_t &lo, uint32_t &hi) {
    lo = f16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
    hi = f16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
}

template <int KV, int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 3))) void prefill_mfma_kernel(PrefillParams p) {
    constexpr int EB = KV == kBF16 ? 2 : 1;
    constexpr int TILE_BYTES = kBlock * D * EB;                  // one pool tile (K or V)
    // LDS stage of one step (two blocks A = 2 i, B = 2 i + 1): K of A, then K
    // of B, each as a bf16 tile in the bf16 pool order (D/8 runs x 16 tokens x
    // 16 bytes), then V as D x 4 fp16 cells: cell (token group tg, dim d) =
    // [A t0..t3 | B t0..t3] of dim d, tokens 4 tg..4 tg+3 of each block, zeroed
    // past the context -- exactly the A operand of the 32-deep P.V product
    // over the step's 32 tokens
    constexpr int KS_UNITS = kBlock * D * 2 / 16;
    constexpr int VS_UNITS = 4 * D;
    constexpr int STAGE_UNITS = 2 * KS_UNITS + VS_UNITS;
    constexpr int NQK = D / 32;  // 32-deep q.K steps per block
    constexpr int NT = D / 16;   // 16 x 16 output tiles per group: tile T = head dims 16 T .. 16 T + 15

    __shared__ __attribute__((aligned(16))) u32x4 stage[2][STAGE_UNITS];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 15;
    const int c = lane >> 4;

    const int G = p.group;
    const int BQ = kRowsPerTile / G;
    // Workgroup b runs on XCD b % 8.  Each (sequence, KV head) pair -- whose
    // tiles all read the same blocks -- goes to one XCD (pair q to XCD q % 8),
    // and an XCD takes its pairs a window of PW at a time, the window's tiles
    // together, longest first (pair by pair within a rank): the blocks the
    // tiles in flight share stay in that XCD's L2.  Workgroups past the last
    // pair have nothing to do.
    const int pairs = p.num_seqs * p.num_kv_heads;
    const int PW = pair_window(p);
    const int xcd = (int)(blockIdx.x % kXcds);
    const int local = (int)(blockIdx.x / kXcds);
    const int span = PW * p.num_tiles;
    const int in_win = local % span;
    const int pair = xcd + kXcds * ((local / span) * PW + in_win % PW);
    if (pair >= pairs) return;
    const int tile = p.num_tiles - 1 - in_win / PW;
    const int s = pair / p.num_kv_heads;
    const int g = pair % p.num_kv_heads;

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

    // this lane's two rows (one per group): chunk token, head, position (also
    // recomputed after the loop rather than kept live across it)
    struct Row {
        int tok, head;
        bool valid, live;
    };
    auto row_of = [&](int k) {
        const int r = kRowsPerWave * wave + 16 * k + n;
        Row w;
        w.tok = tile * BQ + r / G;
        w.head = g * G + r % G;
        w.valid = r < BQ * G && w.tok < n_new;
        w.live = w.valid && first + w.tok >= 0;
        return w;
    };
    int pos_mask[kGroups];
    int minpos = 0x7fffffff, maxpos = -1;
#pragma unroll
    for (int k = 0; k < kGroups; ++k) {
        const Row w = row_of(k);
        // rows that produce no output are masked like the context's last token
        pos_mask[k] = w.live ? first + w.tok : ctx - 1;
        minpos = min(minpos, pos_mask[k]);
        maxpos = max(maxpos, pos_mask[k]);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        minpos = min(minpos, __shfl_xor(minpos, o));
        maxpos = max(maxpos, __shfl_xor(maxpos, o));
    }
    // the same in every lane: as uniform values the per-step mask tests are
    // scalar branches, not exec-masked regions issued on every step
    minpos = __builtin_amdgcn_readfirstlane(minpos);
    maxpos = __builtin_amdgcn_readfirstlane(maxpos);

    // Q^T operands (zero for rows outside the chunk): head dims 8 (4 u + c) .. +7
    // for step u, matching the staged bf16 K runs
    bf16x8 qop[kGroups][NQK];
#pragma unroll
    for (int k = 0; k < kGroups; ++k) {
        const Row w = row_of(k);
        const uint16_t *qrow = reinterpret_cast<const uint16_t *>(p.q) +
                               ((int64_t)(q0 + w.tok) * p.num_q_heads + w.head) * D;
#pragma unroll
        for (int u = 0; u < NQK; ++u) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (w.valid) v = *reinterpret_cast<const u32x4 *>(qrow + 8 * (4 * u + c));
            qop[k][u] = as_bf16x8(v);
        }
    }

    // per row: running max (log2 units), sum, and the exponent above which the
    // max is raised (-inf until the first raise, then the margin)
    float m[kGroups], l[kGroups], thr[kGroups];
    floatx4 acc[kGroups][NT];
#pragma unroll
    for (int k = 0; k < kGroups; ++k) {
        m[k] = 0.f;
        l[k] = 0.f;
        thr[k] = kNegInfF;
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[k][t] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

    const int32_t *table = p.block_tables + (int64_t)s * p.max_blocks_per_seq;
    const char *kpool = static_cast<const char *>(p.k_pool);
    const char *vpool = static_cast<const char *>(p.v_pool);
    auto ok = [&](int32_t b) { return b >= 0 && b < p.num_blocks; };

    // Staging of one step.  K: the step's 2 KU pool units (KU per block) are
    // spread over the threads -- one unit of each block per thread when
    // KU = 256, else thread t takes unit t % KU of block t / KU (the same for
    // a whole wavefront) -- and written to the stage (fp8: widened to two
    // bf16 runs).  V: thread t writes stage cells t, t + 256,
    // ... (cell (tg, d) = unit tg * D + d) and loads the words of dim d of both
    // blocks from the pool cells holding them (bf16: 8 bytes each, fp8: 4);
    // the lanes of one pool cell together load its 16 bytes.  Every lane
    // writes one whole 16-byte unit after its neighbour's, which keeps the
    // LDS stores free of bank conflicts.  The loads go through tile
    // resources, so a block id out of range loads zeros without touching
    // memory.
    constexpr int KU = TILE_BYTES / 16;   // K pool units per block (64, 128 or 256)
    constexpr int KI = KU == kThreads ? 2 : 1;  // K units per thread and step
    constexpr int VLOADS = VS_UNITS / kThreads;
    constexpr int W = 4 / EB;             // head dims per pool V cell
    static_assert(KU % 64 == 0 && KU <= kThreads && VS_UNITS % kThreads == 0, "staging split");
    using VWords = typename std::conditional<KV == kBF16, uint2, uint32_t>::type;
    const int wave_t0 = __builtin_amdgcn_readfirstlane((int)threadIdx.x);  // first thread of the wavefront
    auto gload = [&](int32_t ba, int32_t bb, u32x4 (&kr)[KI], VWords (&vr)[VLOADS][2]) {
        const bool good_a = ok(ba), good_b = ok(bb);
        const int64_t off_a = ((int64_t)(good_a ? ba : 0) * p.num_kv_heads + g) * TILE_BYTES;
        const int64_t off_b = ((int64_t)(good_b ? bb : 0) * p.num_kv_heads + g) * TILE_BYTES;
        const auto ka = tile_rsrc(kpool + off_a, good_a ? TILE_BYTES : 0);
        const auto kb = tile_rsrc(kpool + off_b, good_b ? TILE_BYTES : 0);
        const auto va = tile_rsrc(vpool + off_a, good_a ? TILE_BYTES : 0);
        const auto vb = tile_rsrc(vpool + off_b, good_b ? TILE_BYTES : 0);
        if constexpr (KU == kThreads) {  // one unit of each block per thread
            kr[0] = load_tile<false>(ka, threadIdx.x * 16);
            kr[1] = load_tile<false>(kb, threadIdx.x * 16);
        } else if (wave_t0 < 2 * KU) {   // block wave_t0 / KU, unit t % KU
            kr[0] = load_tile<false>(wave_t0 < KU ? ka : kb, (threadIdx.x % KU) * 16);
        }
#pragma unroll
        for (int i = 0; i < VLOADS; ++i) {
            const int su = threadIdx.x + i * kThreads;
            const int tg = su / D, d = su % D;
            const int off = (tg * (D / W) + d / W) * 16 + (d % W) * (4 * EB);
            if constexpr (KV == kBF16) {
                vr[i][0] = load_tile_b64(va, off);
                vr[i][1] = load_tile_b64(vb, off);
            } else {
                vr[i][0] = load_tile_b32(va, off);
                vr[i][1] = load_tile_b32(vb, off);
            }
        }
    };
    // ... and writes them to a stage in the LDS order above (K: fp8 widened to
    // bf16; V: widened to fp16), the V of tokens at or past `nvalid` (counted
    // from block A's first token) zeroed
    auto swrite = [&](int st, const u32x4 (&kr)[KI], const VWords (&vr)[VLOADS][2], int nvalid) {
        u32x4 *ks = stage[st];
        u32x4 *vs = stage[st] + 2 * KS_UNITS;
#pragma unroll
        for (int i = 0; i < KI; ++i) {
            // unit e = t + 256 i: block e / KU (wavefront-uniform), unit e % KU
            const int e0 = KU == kThreads ? kThreads * i : wave_t0;
            if (KU == kThreads || wave_t0 < 2 * KU) {
                u32x4 *kb = ks + (e0 < KU ? 0 : KS_UNITS);
                const int u = (int)threadIdx.x % KU;
                if constexpr (KV == kBF16) {
                    kb[u] = kr[i];
                } else {  // fp8 run u / 16 (16 dims) of token u % 16 -> two bf16 runs
                    const int rr = u >> 4, tt = u & 15;
                    uint32_t a0, a1, a2, a3, b0, b1, b2, b3;
                    e4m3x4_to_bf16(kr[i][0], a0, a1);
                    e4m3x4_to_bf16(kr[i][1], a2, a3);
                    e4m3x4_to_bf16(kr[i][2], b0, b1);
                    e4m3x4_to_bf16(kr[i][3], b2, b3);
                    kb[(2 * rr) * kBlock + tt] = u32x4{a0, a1, a2, a3};
                    kb[(2 * rr + 1) * kBlock + tt] = u32x4{b0, b1, b2, b3};
                }
            }
        }
#pragma unroll
        for (int i = 0; i < VLOADS; ++i) {
            const int su = threadIdx.x + i * kThreads;
            uint32_t w[4];  // A (t0 t1), A (t2 t3), B (t0 t1), B (t2 t3) of dim d as fp16 pairs
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                if constexpr (KV == kBF16) {
                    w[2 * b] = bf16x2_to_f16x2(vr[i][b].x);
                    w[2 * b + 1] = bf16x2_to_f16x2(vr[i][b].y);
                } else {
                    e4m3x4_to_f16(vr[i][b], w[2 * b], w[2 * b + 1]);
                }
                const int nv = nvalid - b * kBlock;
                if (nv < kBlock) {  // the context's last block (or past it): zero the tokens past it
                    uint32_t k01, k23;
                    v_keep_masks(su / D, nv, k01, k23);
                    w[2 * b] &= k01;
                    w[2 * b + 1] &= k23;
                }
            }
            vs[su] = u32x4{w[0], w[1], w[2], w[3]};
        }
    };

    // Step i: blocks j = 2 i and j + 1, from stage st = i & 1.  `bias_a` / `bias_b` is
    // -inf when that block's id is out of range (its zero K gives zero
    // scores, and every token is masked) and 0 otherwise, which leaves the
    // product's rounding unchanged; MASK: some row's position falls inside
    // the step (the causal mask is applied).
    auto compute_step = [&](auto mask_tag, int st, int j, float bias_a, float bias_b) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const u32x4 *ks = stage[st] + c * kBlock + n;  // K run c (+ 4 per step), token n
        const u32x4 *vs = stage[st] + 2 * KS_UNITS + c * D + n;  // V cell (token group c, dim n (+ 16 T))

        // scores of both blocks and groups first, so their matrix-core
        // products issue back to back: sacc[k][b] = S^T of block b, group k
        floatx4 sacc[kGroups][2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
#pragma unroll
            for (int k = 0; k < kGroups; ++k) sacc[k][b] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < NQK; ++u) {
                const bf16x8 kop = as_bf16x8(ks[b * KS_UNITS + u * 4 * kBlock]);
#pragma unroll
                for (int k = 0; k < kGroups; ++k)
                    sacc[k][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[k][u], sacc[k][b], 0, 0, 0);
            }
        }
        // Exponents relative to the running max, e = score * scale * log2(e)
        // - m, one fused multiply-add per score (e[k][4 b + i] = token 4 c + i
        // of block b); tokens past a row's position are masked by selection.
        float e[kGroups][8], bl[kGroups];
        bool want = false;
#pragma unroll
        for (int k = 0; k < kGroups; ++k) {
            const float ca = bias_a - m[k], cb = bias_b - m[k];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                e[k][i] = __builtin_fmaf(sacc[k][0][i], p.qk_scale_log2, ca);
                e[k][4 + i] = __builtin_fmaf(sacc[k][1][i], p.qk_scale_log2, cb);
            }
            if constexpr (MASK) {
                const int lim = pos_mask[k] - j * kBlock - 4 * c;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    e[k][i] = i > lim ? kNegInfF : e[k][i];
                    e[k][4 + i] = kBlock + i > lim ? kNegInfF : e[k][4 + i];
                }
            }
            bl[k] = fmaxf(fmaxf(fmaxf(e[k][0], e[k][1]), fmaxf(e[k][2], e[k][3])),
                          fmaxf(fmaxf(e[k][4], e[k][5]), fmaxf(e[k][6], e[k][7])));
            want = want || bl[k] > thr[k];
        }
        // The running max m is raised only when some lane's exponent exceeds
        // the threshold (the margin 8, or -inf before the row's first
        // unmasked token): then the row's largest exponent d is exchanged
        // across lanes, m grows by d, the numerators and the sum are rescaled
        // by 2^-d (zero at the first raise) and the step's exponents lowered
        // by d, so the row's max token gets probability exactly 1.  Otherwise
        // every probability stays below 2^8 and m stays put.
        if (__builtin_amdgcn_ballot_w64(want) != 0) {
#pragma unroll
            for (int k = 0; k < kGroups; ++k) {
                const float bm = max_xor32(max_xor16(bl[k]));
                const bool grow = bm > thr[k];
                const float d = grow ? bm : 0.f;
                const float alpha = grow ? (thr[k] == kNegInfF ? 0.f : __builtin_amdgcn_exp2f(-d)) : 1.f;
                m[k] += d;
                thr[k] = grow ? kLazyMax : thr[k];
                l[k] *= alpha;
#pragma unroll
                for (int t = 0; t < NT; ++t) acc[k][t] *= alpha;
#pragma unroll
                for (int i = 0; i < 8; ++i) e[k][i] -= d;
            }
        }
        // P^T operands: the step's 8 probabilities of the lane rounded to
        // fp16; the row sum adds the rounded values, so the output is a
        // weighted mean of V with exactly the weights the product used
        f16x8 pop[kGroups];
#pragma unroll
        for (int k = 0; k < kGroups; ++k) {
            f16x2 h[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                h[i] = f16x2{(_Float16)__builtin_amdgcn_exp2f(e[k][2 * i]),
                             (_Float16)__builtin_amdgcn_exp2f(e[k][2 * i + 1])};
            const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
            float ls = l[k];
#pragma unroll
            for (int i = 0; i < 4; ++i) ls = __builtin_amdgcn_fdot2(h[i], one, ls, false);
            l[k] = ls;
            pop[k] = f16x8{h[0][0], h[0][1], h[1][0], h[1][1], h[2][0], h[2][1], h[3][0], h[3][1]};
        }

        // O^T += V^T . P^T over the step's 32 tokens: the staged cell is the ready operand
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const f16x8 a = __builtin_bit_cast(f16x8, vs[16 * t]);
#pragma unroll
            for (int k = 0; k < kGroups; ++k)
                acc[k][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pop[k], acc[k][t], 0, 0, 0);
        }
    };

    // Block ids come by scalar loads from the table, one step ahead.  Step i
    // is computed from stage i & 1 while step i + 1 is in flight in
    // registers; step i + 1 then goes to the other stage and step i + 2's
    // loads are issued (every step issues the same loads), and one barrier
    // ends the step.
    auto id_at = [&](int j) -> int32_t {
        const int32_t b = table[min(j, nblk_wg - 1)];
        return j < nblk_wg ? b : -1;
    };
    if (nblk_wg > 0) {
        const int nstep = (nblk_wg + 1) / 2;
        int32_t ida = id_at(0), idb = id_at(1), nida = id_at(2), nidb = id_at(3);
        u32x4 kpre[KI];
        VWords vpre[VLOADS][2];
        gload(ida, idb, kpre, vpre);
        swrite(0, kpre, vpre, ctx);
        gload(nida, nidb, kpre, vpre);
        __syncthreads();
        // steps whose blocks lie at or before every row's position of the
        // wavefront (no causal mask); the rest are masked
        const int sm = min((minpos + 1) / kBlock, nblk_wg) / 2;
        auto next = [&](int i) {
            const int32_t a2 = id_at(2 * i + 4), b2 = id_at(2 * i + 5);
            if (i + 1 < nstep) swrite((i + 1) & 1, kpre, vpre, ctx - (2 * i + 2) * kBlock);
            gload(a2, b2, kpre, vpre);
            ida = nida;
            idb = nidb;
            nida = a2;
            nidb = b2;
            __syncthreads();
        };
        // Every wavefront computes every step of the workgroup: blocks past
        // its own rows are masked out by the causal test, and a straight-line
        // loop body keeps the accumulators in place.
        for (int i = 0; i < sm; ++i) {
            compute_step(std::false_type{}, i & 1, 2 * i, ok(ida) ? 0.f : kNegInfF, ok(idb) ? 0.f : kNegInfF);
            next(i);
        }
        // A step wholly past every row of this wavefront (its first token
        // beyond the wavefront's largest position: with one query head per
        // KV head a tile spans 128 positions) only stages for the others:
        // its scores would all be -inf, adding exact zeros.
        const int sx = min(maxpos / (2 * kBlock) + 1, nstep);
        for (int i = sm; i < nstep; ++i) {
            if (i < sx)
                compute_step(std::true_type{}, i & 1, 2 * i, ok(ida) ? 0.f : kNegInfF,
                             ok(idb) ? 0.f : kNegInfF);
            next(i);
        }
    }

    // rows: out = O / l (times v_scale); rows before the context start are zero.
    // Tile T element i is head dim 16 T + 4 c + i: one float4 per tile.
#pragma unroll
    for (int k = 0; k < kGroups; ++k) {
        float lt = l[k];
        lt = add_xor32(add_xor16(lt));
        const Row w = row_of(k);
        if (!w.valid) continue;
        const float f = w.live && lt > 0.f ? p.out_scale / lt : 0.f;
        float *orow = p.out + ((int64_t)(q0 + w.tok) * p.num_q_heads + w.head) * D;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float4 v = w.live ? make_float4(acc[k][t][0] * f, acc[k][t][1] * f, acc[k][t][2] * f,
                                                   acc[k][t][3] * f)
                                     : make_float4(0.f, 0.f, 0.f, 0.f);
            *reinterpret_cast<float4 *>(orow + 16 * t + 4 * c) = v;
        }
    }
}

template <int KV, int D>
hipError_t launch(const PrefillParams &p, hipStream_t stream, const LaunchEvents *ev) {
    const int64_t pairs = (int64_t)p.num_seqs * p.num_kv_heads;
    const int64_t per_round = (int64_t)kXcds * pair_window(p);  // pairs per round of windows
    const int64_t grid = (int64_t)p.num_tiles * per_round * ((pairs + per_round - 1) / per_round);
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
