// pa_decode.hip -- paged single-query decode attention on vector ALUs, and
// the split-K merge.
//
// What is computed (source pages by title and section): every sequence's one
// query attends over its ctx cached tokens, read block by block through its
// block table in logical order ("PagedAttention" glossary page, how paging
// works; Russian page on vLLM's KV cache, logical order vs physical
// placement); query heads in a group share one KV head (glossary page,
// related techniques).  The result is softmax(scale * q K^T) V.
//
// Work split: one workgroup per (sequence, query head, partition of
// `partition_tokens` tokens).  Each of its four wavefronts walks every fourth
// block of the partition and keeps its own running maximum m, running sum l
// and numerator acc (online softmax, base-2 exponent domain); the four are
// merged through LDS.  A context longer than one partition leaves (m, l, acc)
// per partition in the workspace and the reduce kernel merges them in
// partition order.
//
// Lane roles inside a wavefront, per 16-token block (lane = 16 * c + t):
//   q.K:  lane (t, c) multiplies token t's 16-byte K runs c, c+4, c+8, ... by
//         the matching q elements; the four partial sums of token t (lanes
//         t, t+16, t+32, t+48) are added with two butterfly shuffles.
//   P.V:  lane (t, c) reads the V cells of tokens 4c..4c+3 for head dims
//         W*(16 jj + t) .. +W-1 and accumulates them weighted by those four
//         tokens' probabilities; the four token quarters are added once, after
//         the last block.
// Masked tokens (position >= ctx) get score -inf, i.e. weight exactly 0, by
// selection: the values they read are never multiplied in.
#include "pa_internal.h"
#include "pa_mfma_util.h"
#include "pa_store.h"

#include <type_traits>

namespace pa {
namespace {

constexpr float kNegInf = -__builtin_inff();

// Element e of a 16-byte chunk of fp32 values.
__device__ __forceinline__ float chunk_f32(const uint4 &v, int e) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    return __uint_as_float(w[e]);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// a.lo * b.lo + a.hi * b.hi + acc for two packed bf16 pairs (v_dot2_f32_bf16;
// the bf16 products are exact in fp32)
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), acc, false);
}

// four fp8 codes (one word) -> bf16 pairs (codes 0,1) and (codes 2,3), exact
__device__ __forceinline__ void e4m3x4_to_bf16(uint32_t w, uint32_t &lo, uint32_t &hi) {
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
    hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}

// p0, p1 -> bf16 pairs hi = (trunc(p0), trunc(p1)) and lo = the remainders,
// truncated: hi + lo carries each p to 16 significant bits
__device__ __forceinline__ void split_pair(float p0, float p1, uint32_t &hi, uint32_t &lo) {
    const uint32_t u0 = __float_as_uint(p0), u1 = __float_as_uint(p1);
    const uint32_t r0 = __float_as_uint(p0 - __uint_as_float(u0 & 0xffff0000u));
    const uint32_t r1 = __float_as_uint(p1 - __uint_as_float(u1 & 0xffff0000u));
    hi = (u0 >> 16) | (u1 & 0xffff0000u);
    lo = (r0 >> 16) | (r1 & 0xffff0000u);
}

// max of x and the value lane-permuted by the DPP control CTRL (within rows)
template <int CTRL>
__device__ __forceinline__ float max_dpp(float x) {
    const int y = __builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, 0xf, 0xf, false);
    return fmaxf(x, __int_as_float(y));
}

__device__ __forceinline__ float wave_max16(float x) {
    // maximum over the 16 lanes of a row with data-parallel lane moves (no LDS):
    // swap neighbours, then pairs (quad permutations [1 0 3 2] and [2 3 0 1]),
    // then mirror each half row and the whole row
    x = max_dpp<0xB1>(x);
    x = max_dpp<0x4E>(x);
    x = max_dpp<0x141>(x);
    x = max_dpp<0x140>(x);
    return x;
}

template <int KV, int D, bool STREAM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(KV == kF32 ? 1 : (KV == kBF16 ? 2 : 4)))) void decode_valu_kernel(DecodeParams p) {
    constexpr int EB = KV == kF32 ? 4 : (KV == kBF16 ? 2 : 1);
    constexpr int X = 16 / EB;          // K: elements per 16-byte run
    constexpr int W = 4 / EB;           // V: head-dim elements per 16-byte cell
    constexpr int NKL = D / X / 4;      // K runs per lane per block
    constexpr int NVL = D / W / 16;     // V cells per lane per block
    constexpr int TILE_BYTES = kBlock * D * EB;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wv = __builtin_amdgcn_readfirstlane(wave);   // the same, as a uniform value
    const int t = lane & 15;
    const int c = lane >> 4;

    // work order as in the matrix-core kernel: partition 0 of every row
    // first, then each row's later partitions, rotated by row
    int bid, part;
    pair_and_partition(p.num_seqs * p.num_q_heads, p.max_partitions, bid, part);
    const int h = bid % p.num_q_heads;
    const int s = sequence_of_rank(p.context_lens, p.num_seqs, p.max_blocks_per_seq * kBlock,
                                   bid / p.num_q_heads);
    const int g = h / p.group;

    const int raw_ctx = p.context_lens[s];
    const int ctx = raw_ctx < 0 ? 0 : (raw_ctx > p.max_blocks_per_seq * kBlock ? p.max_blocks_per_seq * kBlock : raw_ctx);
    const int nparts = (ctx + p.partition_tokens - 1) / p.partition_tokens;
    if (part >= (nparts > 1 ? nparts : 1)) return;
    const int tok0 = part * p.partition_tokens;
    const int tok1 = min(ctx, tok0 + p.partition_tokens);
    const int blk0 = tok0 / kBlock;
    const int blk1 = (tok1 + kBlock - 1) / kBlock;
    const int32_t *table = p.block_tables + (int64_t)s * p.max_blocks_per_seq;

    // A decode step's newest token (one query head per KV head here, so this
    // workgroup alone reads KV head g's last block) is written by the
    // wavefront that reads the last block of the partition holding position
    // ctx - 1 (wavefronts take every fourth block).  It loads the token's
    // inputs first, issues its block loads, and stores the token when the
    // inputs arrive: its own later loads of the block see the stores (a
    // wavefront's memory accesses stay in order), and nothing waits for them.
    // A context longer than its table row (clamped above) has no slot for its
    // newest token and writes nothing.
    const bool writer = p.k_new != nullptr && tok1 == ctx && ctx > 0 && raw_ctx == ctx &&
                        wv == (blk1 - 1 - blk0) % 4;

    // q elements matching this lane's K runs: fp32 values for an fp32 pool,
    // else the raw bf16 pairs (dims 2i, 2i+1 of run c + 4j in word i), which
    // line up with the K run's bf16 pairs (fp8 runs are widened pairwise)
    constexpr int QW = KV == kF32 ? 1 : X / 2;  // bf16 pairs per run
    const int64_t qrow = ((int64_t)s * p.num_q_heads + h) * D;
    float qv[KV == kF32 ? NKL : 1][KV == kF32 ? X : 1];
    uint32_t qw[KV == kF32 ? 1 : NKL][QW];
#pragma unroll
    for (int j = 0; j < NKL; ++j) {
        const int d0 = (c + 4 * j) * X;
        if constexpr (KV == kF32) {
#pragma unroll
            for (int x = 0; x < X; ++x) qv[j][x] = reinterpret_cast<const float *>(p.q)[qrow + d0 + x];
        } else {
            const uint4 *src = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(p.q) +
                                                               qrow + d0);
#pragma unroll
            for (int i = 0; i < QW / 4; ++i) {
                const uint4 v = src[i];
                qw[j][4 * i + 0] = v.x;
                qw[j][4 * i + 1] = v.y;
                qw[j][4 * i + 2] = v.z;
                qw[j][4 * i + 3] = v.w;
            }
        }
    }

    float m = kNegInf;
    float l = 0.f;
    float acc[NVL][W];
#pragma unroll
    for (int jj = 0; jj < NVL; ++jj)
#pragma unroll
        for (int w = 0; w < W; ++w) acc[jj][w] = 0.f;

    const char *kbase = static_cast<const char *>(p.k_pool);
    const char *vbase = static_cast<const char *>(p.v_pool);

    auto valid = [&](int32_t b) { return b >= 0 && b < p.num_blocks; };
    // one tile of a pool as a buffer resource: empty (loads give zeros and
    // touch no memory) for an id outside the pool or past the end (-1)
    auto tile = [&](const char *base, int32_t b) {
        const bool ok = valid(b);
        return tile_rsrc(base + ((int64_t)(ok ? b : 0) * p.num_kv_heads + g) * TILE_BYTES, ok ? TILE_BYTES : 0);
    };
    // FENCED keeps the loads in program order (the prologue issues them in the
    // loop's order, so the loop's waits hold from its first iteration)
    auto load_k = [&](int32_t b, uint4 (&kc)[NKL], auto fenced) {
        const auto r = tile(kbase, b);
#pragma unroll
        for (int jk = 0; jk < NKL; ++jk) {
            kc[jk] = __builtin_bit_cast(uint4, load_tile<STREAM>(r, ((c + 4 * jk) * kBlock + t) * 16));
            if constexpr (decltype(fenced)::value) __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto load_v = [&](int32_t b, uint4 (&vc)[NVL], auto fenced) {
        const auto r = tile(vbase, b);
#pragma unroll
        for (int jj = 0; jj < NVL; ++jj) {
            vc[jj] = __builtin_bit_cast(uint4, load_tile<STREAM>(r, (c * (D / W) + 16 * jj + t) * 16));
            if constexpr (decltype(fenced)::value) __builtin_amdgcn_sched_barrier(0);
        }
    };
    constexpr std::true_type kFenced{};
    constexpr std::false_type kFree{};

    // this lane's partial q . K (its four K runs of token t)
    auto qk = [&](const uint4 (&kc)[NKL]) {
        float part_dot = 0.f;
#pragma unroll
        for (int jk = 0; jk < NKL; ++jk) {
            if constexpr (KV == kF32) {
#pragma unroll
                for (int x = 0; x < X; ++x) part_dot += qv[jk][x] * chunk_f32(kc[jk], x);
            } else if constexpr (KV == kBF16) {
                part_dot = dot2(kc[jk].x, qw[jk][0], part_dot);
                part_dot = dot2(kc[jk].y, qw[jk][1], part_dot);
                part_dot = dot2(kc[jk].z, qw[jk][2], part_dot);
                part_dot = dot2(kc[jk].w, qw[jk][3], part_dot);
            } else {
                const uint32_t kw[4] = {kc[jk].x, kc[jk].y, kc[jk].z, kc[jk].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    uint32_t lo, hi;
                    e4m3x4_to_bf16(kw[i], lo, hi);
                    part_dot = dot2(lo, qw[jk][2 * i], part_dot);
                    part_dot = dot2(hi, qw[jk][2 * i + 1], part_dot);
                }
            }
        }
        return part_dot;
    };

    // online softmax over block j and acc += p . V
    auto softmax_pv = [&](float part_dot, const uint4 (&vc)[NVL], int j) {
        part_dot = add_xor32(add_xor16(part_dot));

        float sc = part_dot * p.qk_scale_log2;
        if (j * kBlock + t >= tok1) sc = kNegInf;
        const float m_new = fmaxf(m, wave_max16(sc));
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);
        const float pt = __builtin_amdgcn_exp2f(sc - m_new);
        m = m_new;

        // probabilities of tokens 4c..4c+3; tokens past the context are left
        // out by selection (their V bytes may hold anything, NaN included)
        const int nvalid = tok1 - j * kBlock;
        float pw[4];
        bool live[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pw[i] = __shfl(pt, 4 * c + i);
            live[i] = 4 * c + i < nvalid;
        }
        l = l * alpha + ((pw[0] + pw[1]) + (pw[2] + pw[3]));
        if (alpha != 1.f) {  // alpha is the same in every lane
#pragma unroll
            for (int jj = 0; jj < NVL; ++jj)
#pragma unroll
                for (int w = 0; w < W; ++w) acc[jj][w] *= alpha;
        }
        if constexpr (KV == kF32) {
#pragma unroll
            for (int jj = 0; jj < NVL; ++jj) {
#pragma unroll
                for (int w = 0; w < W; ++w) {
                    float sum = 0.f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float term = pw[i] * chunk_f32(vc[jj], 4 * w + i);
                        sum += live[i] ? term : 0.f;
                    }
                    acc[jj][w] += sum;
                }
            }
        } else {
            // P as bf16 hi + lo pairs against the V cell's bf16 token pairs;
            // V elements of tokens past the context are zeroed first
            uint32_t p01h, p01l, p23h, p23l;
            split_pair(pw[0], pw[1], p01h, p01l);
            split_pair(pw[2], pw[3], p23h, p23l);
            const uint32_t keep01 = (live[0] ? 0x0000ffffu : 0u) | (live[1] ? 0xffff0000u : 0u);
            const uint32_t keep23 = (live[2] ? 0x0000ffffu : 0u) | (live[3] ? 0xffff0000u : 0u);
#pragma unroll
            for (int jj = 0; jj < NVL; ++jj) {
                const uint32_t vw[4] = {vc[jj].x, vc[jj].y, vc[jj].z, vc[jj].w};
#pragma unroll
                for (int w = 0; w < W; ++w) {
                    uint32_t v01, v23;
                    if constexpr (KV == kBF16) {
                        v01 = vw[2 * w];
                        v23 = vw[2 * w + 1];
                    } else {
                        e4m3x4_to_bf16(vw[w], v01, v23);
                    }
                    v01 &= keep01;
                    v23 &= keep23;
                    float a = acc[jj][w];
                    a = dot2(v01, p01h, a);
                    a = dot2(v23, p23h, a);
                    a = dot2(v01, p01l, a);
                    a = dot2(v23, p23l, a);
                    acc[jj][w] = a;
                }
            }
        }
    };

    // This wavefront's blocks are j = blk0 + wave + 4k, k = 0..nk-1; their ids
    // come from the table by scalar loads, one block ahead of their use.  NB
    // register buffers hold blocks k .. k + NB - 1; block k + NB reuses block
    // k's buffer half by half (K once its dot products are formed, V once it
    // is consumed), and every step issues the same loads (empty resources
    // past the end), so each wait covers exactly the loads it needs.  bf16
    // pools keep three blocks in flight (176 VGPRs at head dim 128, 2
    // waves/SIMD: the 13B-like batch 0.1077 -> 0.1060 ms), the others two.
    const int nk = blk1 - blk0 > wv ? (blk1 - blk0 - wv + 3) / 4 : 0;
    if (nk > 0) {
        const int32_t *wtable = table + blk0 + wv;
        auto id_at = [&](int k) -> int32_t {
            const int32_t b = wtable[4 * min(k, nk - 1)];
            return k < nk ? b : -1;
        };
        // with NB blocks or fewer the last one is loaded in the prologue: the
        // token is stored before it then
        constexpr int NB = KV == kBF16 ? 3 : 2;
        const bool early = writer && nk <= NB;
        NewToken<D> nt;
        if (writer) nt = append_load<KV, D>(p, table, s, g, ctx - 1, lane);
        if (early) append_store<KV, D>(p, nt, g, ctx - 1, lane);
        uint4 kb[NB][NKL], vb[NB][NVL];
        int32_t idb[NB];
#pragma unroll
        for (int d = 0; d < NB; ++d) {
            idb[d] = id_at(d);
            load_k(idb[d], kb[d], kFenced);
            load_v(idb[d], vb[d], kFenced);
        }
        if (writer && !early) append_store<KV, D>(p, nt, g, ctx - 1, lane);
        int32_t id_pre = id_at(NB);
        auto step = [&](int d, int kk) {
            const int32_t id_after = id_pre;  // block kk + NB
            id_pre = id_at(kk + NB + 1);
            const float part = qk(kb[d]);
            load_k(id_after, kb[d], kFree);
            if (valid(idb[d])) softmax_pv(part, vb[d], blk0 + wv + 4 * kk);
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
    }

    // add the four token quarters (rows c = 0..3)
    l = add_xor32(add_xor16(l));
#pragma unroll
    for (int jj = 0; jj < NVL; ++jj)
#pragma unroll
        for (int w = 0; w < W; ++w) acc[jj][w] = add_xor32(add_xor16(acc[jj][w]));

    __shared__ float sm_m[4], sm_l[4];
    __shared__ float sm_acc[4][D];
    if (lane == 0) {
        sm_m[wave] = m;
        sm_l[wave] = l;
    }
    if (c == 0) {
#pragma unroll
        for (int jj = 0; jj < NVL; ++jj)
#pragma unroll
            for (int w = 0; w < W; ++w) sm_acc[wave][(16 * jj + t) * W + w] = acc[jj][w];
    }
    __syncthreads();

    // merge and write, 4 consecutive head dims per lane as one 16-byte
    // store (the stores that end a work item cost far more than their bytes
    // while the chip streams K/V): final outputs non-temporal, split-K
    // partials cacheable for the reduce kernel that reads them next
    constexpr int D4 = D / 4;
    if (threadIdx.x < D4) {
        const int d0 = 4 * threadIdx.x;
        const float M = fmaxf(fmaxf(sm_m[0], sm_m[1]), fmaxf(sm_m[2], sm_m[3]));
        float L = 0.f;
        float O[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float f = sm_m[w] == kNegInf ? 0.f : exp2f(sm_m[w] - M);
            L += sm_l[w] * f;
#pragma unroll
            for (int e = 0; e < 4; ++e) O[e] += sm_acc[w][d0 + e] * f;
        }
        const int64_t row = (int64_t)s * p.num_q_heads + h;
        if (nparts <= 1) {
            float r[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = L > 0.f ? (O[e] / L) * p.out_scale : 0.f;
            store16_nt(p.out + row * D + d0, __builtin_bit_cast(uint4, r));
        } else {
            const int64_t pr = row * p.max_partitions + part;
            *reinterpret_cast<uint4 *>(p.ws_acc + pr * D + d0) = __builtin_bit_cast(uint4, O);
            if (d0 == 0) {
                p.ws_m[pr] = M;
                p.ws_l[pr] = L;
            }
        }
    }
}

// Merge the partitions of one (sequence, query head) row, in partition order:
// M = max_p m_p, out = sum_p acc_p 2^(m_p - M) / sum_p l_p 2^(m_p - M).
// One wavefront per row; lane i holds head dims E*i .. E*i+E-1.  The
// partition weights are computed 64 at a time, one per lane, and broadcast
// with readlane, so the partial numerators of eight partitions are in flight
// at once; the first four are loaded with the partition maxima and sums,
// before the merged maximum is known.
template <int D>
__device__ __forceinline__ void reduce_row(const DecodeParams &p, int64_t row, int nparts) {
    constexpr int E = D / 64;
    const int lane = threadIdx.x & 63;
    const float *ms = p.ws_m + row * p.max_partitions;
    const float *ls = p.ws_l + row * p.max_partitions;
    const float *as = p.ws_acc + row * p.max_partitions * D + E * lane;

    // Every load that does not depend on the merged maximum goes out at once:
    // this lane's partition (m, l) and the first PRE partitions' numerators;
    // only their use waits for M.
    constexpr int PRE = 4;
    const float m0 = lane < nparts ? ms[lane] : kNegInf;
    const float l0 = lane < nparts ? ls[lane] : 0.f;
    float pre[PRE][E];
#pragma unroll
    for (int u = 0; u < PRE; ++u) {
        const float *a = as + (int64_t)u * D;
#pragma unroll
        for (int e = 0; e < E; ++e) pre[u][e] = u < nparts ? a[e] : 0.f;
    }

    float M = m0;
    for (int i = lane + 64; i < nparts; i += 64) M = fmaxf(M, ms[i]);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));

    float L = 0.f;
    float O[E];
#pragma unroll
    for (int e = 0; e < E; ++e) O[e] = 0.f;
    // numerator of partition base + j, weighted by lane j's weight f
    auto add = [&](float f, int base, int j) {
        const float fj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), j));
        const float *a = as + (int64_t)(base + j) * D;
        if constexpr (E == 2) {
            const float2 v = *reinterpret_cast<const float2 *>(a);
            O[0] += v.x * fj;
            O[1] += v.y * fj;
        } else {
            O[0] += a[0] * fj;
        }
    };
    if (M != kNegInf) {
        {   // partitions 0..63, the first PRE of them preloaded
            const float f = lane < nparts && m0 != kNegInf ? exp2f(m0 - M) : 0.f;
            L += lane < nparts ? l0 * f : 0.f;
            const int cnt = min(64, nparts);
#pragma unroll
            for (int u = 0; u < PRE; ++u) {
                const float fj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), u));
#pragma unroll
                for (int e = 0; e < E; ++e) O[e] += u < cnt ? pre[u][e] * fj : 0.f;
            }
            int j = PRE;
            for (; j + 8 <= cnt; j += 8) {
#pragma unroll
                for (int u = 0; u < 8; ++u) add(f, 0, j + u);
            }
            for (; j < cnt; ++j) add(f, 0, j);
        }
        for (int base = 64; base < nparts; base += 64) {
            const int i = base + lane;
            const float mi = i < nparts ? ms[i] : kNegInf;
            const float f = mi != kNegInf ? exp2f(mi - M) : 0.f;
            L += i < nparts ? ls[i] * f : 0.f;
            const int cnt = min(64, nparts - base);
            int j = 0;
            for (; j + 8 <= cnt; j += 8) {
#pragma unroll
                for (int u = 0; u < 8; ++u) add(f, base, j + u);
            }
            for (; j < cnt; ++j) add(f, base, j);
        }
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) L += __shfl_xor(L, o);
    }
    float *dst = p.out + row * D + E * lane;
#pragma unroll
    for (int e = 0; e < E; ++e) dst[e] = L > 0.f ? (O[e] / L) * p.out_scale : 0.f;
}

// One wavefront per (sequence, query head) row with more than one partial
// result (four rows per workgroup).
template <int D>
__global__ __launch_bounds__(kThreads) void decode_reduce_kernel(DecodeParams p) {
    const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);  // s * Hq + h
    if (row >= (int64_t)p.num_seqs * p.num_q_heads) return;
    const int s = (int)(row / p.num_q_heads);
    int ctx = p.context_lens[s];
    ctx = ctx < 0 ? 0 : (ctx > p.max_blocks_per_seq * kBlock ? p.max_blocks_per_seq * kBlock : ctx);
    const int unit = p.partition_tokens * p.group_parts;   // tokens per partial result
    const int nparts = (ctx + unit - 1) / unit;
    if (nparts <= 1) return;  // written by the partition kernel
    reduce_row<D>(p, row, nparts);
}

// The shared-prefix kernel's merge: one wavefront per (group, member, query
// head) row of a group that had more than one partition (the partition
// kernel recorded each group's count).
template <int D>
__global__ __launch_bounds__(kThreads) void decode_shared_reduce_kernel(DecodeParams p) {
    const int per_group = p.max_group * p.num_q_heads;
    const int r = (int)blockIdx.y * (kThreads / 64) + (threadIdx.x >> 6);
    if (r >= per_group) return;
    const int gi = blockIdx.x;
    const int s0 = p.group_start[gi];
    int M = p.group_start[gi + 1] - s0;
    if (s0 < 0 || s0 >= p.num_seqs) M = 0;
    M = M < 0 ? 0 : min(M, min(p.max_group, p.num_seqs - s0));
    const int member = r / p.num_q_heads;
    if (member >= M) return;
    const int nparts = p.ws_nparts[gi];
    if (nparts <= 1) return;  // written by the partition kernel
    reduce_row<D>(p, (int64_t)(s0 + member) * p.num_q_heads + r % p.num_q_heads, min(nparts, p.max_partitions));
}

template <int KV, int D>
hipError_t launch_valu(const DecodeParams &p, hipStream_t stream, const LaunchEvents *ev) {
    const int64_t grid = (int64_t)p.num_seqs * p.num_q_heads * p.max_partitions;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    const dim3 g((unsigned)grid), b(kThreads);
    if (p.shared_kv) return launch_kernel(decode_valu_kernel<KV, D, false>, g, b, stream, ev, p);
    return launch_kernel(decode_valu_kernel<KV, D, true>, g, b, stream, ev, p);
}

template <int KV>
hipError_t launch_valu_d(int head_dim, const DecodeParams &p, hipStream_t stream, const LaunchEvents *ev) {
    return head_dim == 64 ? launch_valu<KV, 64>(p, stream, ev) : launch_valu<KV, 128>(p, stream, ev);
}

}  // namespace

hipError_t launch_decode_valu(int kv, int head_dim, const DecodeParams &p, hipStream_t stream,
                              const LaunchEvents *ev) {
    if (kv == kF32) return launch_valu_d<kF32>(head_dim, p, stream, ev);
    if (kv == kBF16) return launch_valu_d<kBF16>(head_dim, p, stream, ev);
    return launch_valu_d<kFP8>(head_dim, p, stream, ev);
}

hipError_t launch_decode_shared_reduce(int head_dim, const DecodeParams &p, hipStream_t stream) {
    const int per_group = p.max_group * p.num_q_heads;
    const dim3 grid((unsigned)p.num_groups, (unsigned)((per_group + kThreads / 64 - 1) / (kThreads / 64)));
    if (head_dim == 64)
        decode_shared_reduce_kernel<64><<<grid, dim3(kThreads), 0, stream>>>(p);
    else
        decode_shared_reduce_kernel<128><<<grid, dim3(kThreads), 0, stream>>>(p);
    return hipGetLastError();
}

hipError_t launch_decode_reduce(int head_dim, const DecodeParams &p, hipStream_t stream) {
    const int64_t rows = (int64_t)p.num_seqs * p.num_q_heads;
    const int64_t grid = (rows + kThreads / 64 - 1) / (kThreads / 64);
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    if (head_dim == 64)
        decode_reduce_kernel<64><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(p);
    else
        decode_reduce_kernel<128><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace pa
