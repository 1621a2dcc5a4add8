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
// one such tile of one sequence.  Each wavefront owns 32 rows as two
// 16-column matrix-core groups and walks blocks 0 .. (its last row's
// position) / 16 on its own: no LDS and no barrier.  Its four wavefronts read
// the same K/V tiles, which the second and later readers find in cache.
// Workgroups are issued latest tile first, so the longest causal ranges
// start first.
//
// Per block, for each 16-row group (operand layouts as in the grouped decode
// kernel: K and V go from the pool's tiled layout straight into A operands
// with one 16-byte load per lane per run/cell):
//     S^T[16 tokens][16 rows]  = K[16][D] . Q^T[D][16]
//     O^T[D][16 rows]         += V^T[D][16 tokens] . P^T[16][16]
// with P carried as bf16 hi + lo (16 significant bits).  Causal masking sets
// the score of every token past a row's position to -inf (selection); the V
// elements of slots past the context are zeroed before the product.
#include "pa_internal.h"
#include "pa_mfma_util.h"

namespace pa {
namespace {

template <int KV, int D, int kGroups>
__global__ __launch_bounds__(kThreads) void prefill_mfma_kernel(PrefillParams p) {
    constexpr int kRowsPerWave = 16 * kGroups;
    constexpr int kRowsPerTile = kRowsPerWave * (kThreads / 64);
    constexpr int EB = KV == kBF16 ? 2 : 1;
    constexpr int TILE_BYTES = kBlock * D * EB;
    constexpr int NQK = D / 32;                       // 32-deep q.K steps per block
    constexpr int NKL = KV == kBF16 ? NQK : NQK / 2;  // 16-byte K loads per lane per block
    constexpr int W = 4 / EB;                         // V: head dims per 16-byte cell
    constexpr int NVL = D / W / 16;                   // 16-byte V loads per lane per block
    constexpr int NT = D / 16;                        // 16 x 16 output tiles per group

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
    int n_new = p.query_start[s + 1] - q0;
    n_new = n_new < 0 ? 0 : (n_new > p.max_query_len ? p.max_query_len : n_new);
    const int first = ctx - n_new;  // position of chunk token 0 (< 0: chunk longer than context)
    if (tile * BQ >= n_new) return;

    // this lane's two rows (one per group): chunk token, head, position
    int row_tok[kGroups], row_head[kGroups], pos_mask[kGroups];
    bool valid[kGroups], live[kGroups];
    int maxpos = -1, minpos = 0x7fffffff;
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
        if (live[k]) maxpos = max(maxpos, pos);
        minpos = min(minpos, pos_mask[k]);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        maxpos = max(maxpos, __shfl_xor(maxpos, o));
        minpos = min(minpos, __shfl_xor(minpos, o));
    }
    const int nblk = maxpos < 0 ? 0 : maxpos / kBlock + 1;

    // Q^T operands (zero for rows outside the chunk), head dims per the K mapping
    bf16x8 qop[kGroups][NQK];
#pragma unroll
    for (int k = 0; k < kGroups; ++k) {
        const uint16_t *qrow = reinterpret_cast<const uint16_t *>(p.q) +
                               ((int64_t)(q0 + row_tok[k]) * p.num_q_heads + row_head[k]) * D;
#pragma unroll
        for (int u = 0; u < NQK; ++u) {
            int d0;
            if constexpr (KV == kBF16)
                d0 = 8 * (4 * u + c);
            else
                d0 = 16 * (c + 4 * (u >> 1)) + 8 * (u & 1);
            u32x4 v = {0u, 0u, 0u, 0u};
            if (valid[k]) v = *reinterpret_cast<const u32x4 *>(qrow + d0);
            qop[k][u] = as_bf16x8(v);
        }
    }

    float m[kGroups], l[kGroups];
    floatx4 acc[kGroups][NT];
#pragma unroll
    for (int k = 0; k < kGroups; ++k) {
        m[k] = kNegInfF;
        l[k] = 0.f;
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[k][t] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

    const int32_t *table = p.block_tables + (int64_t)s * p.max_blocks_per_seq;
    const char *kbase = static_cast<const char *>(p.k_pool);
    const char *vbase = static_cast<const char *>(p.v_pool);
    const int koff = (c * kBlock + n) * 16;   // K run c, token n
    const int voff = (c * (D / W) + n) * 16;  // V cell (tokens 4c.., dims W n..)

    auto load_block = [&](int32_t b, u32x4 (&kr)[NKL], u32x4 (&vr)[NVL]) {
        const int64_t t0 = ((int64_t)b * p.num_kv_heads + g) * TILE_BYTES;
        const char *kt = kbase + t0 + koff;
        const char *vt = vbase + t0 + voff;
#pragma unroll
        for (int i = 0; i < NKL; ++i) kr[i] = *reinterpret_cast<const u32x4 *>(kt + i * 4 * kBlock * 16);
#pragma unroll
        for (int i = 0; i < NVL; ++i) vr[i] = *reinterpret_cast<const u32x4 *>(vt + i * 16 * 16);
    };

    auto compute_block = [&](const u32x4 (&kr)[NKL], const u32x4 (&vr)[NVL], int j) {
        // K operands (fp8 widened to bf16 once, used by both groups)
        bf16x8 kop[NQK];
        if constexpr (KV == kBF16) {
#pragma unroll
            for (int u = 0; u < NQK; ++u) kop[u] = as_bf16x8(kr[u]);
        } else {
#pragma unroll
            for (int i = 0; i < NKL; ++i)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    uint32_t a0, a1, a2, a3;
                    e4m3x4_to_bf16(kr[i][2 * h], a0, a1);
                    e4m3x4_to_bf16(kr[i][2 * h + 1], a2, a3);
                    kop[2 * i + h] = as_bf16x8(u32x4{a0, a1, a2, a3});
                }
        }
        const bool need_mask = j * kBlock + kBlock - 1 > minpos;
        const int nvalid = ctx - j * kBlock;
        uint32_t keep01 = 0xffffffffu, keep23 = 0xffffffffu;
        if (nvalid < kBlock) v_keep_masks(c, nvalid, keep01, keep23);

        bf16x8 pop[kGroups];
#pragma unroll
        for (int k = 0; k < kGroups; ++k) {
            floatx4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < NQK; ++u)
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[u], qop[k][u], sacc, 0, 0, 0);
            float sc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sc[i] = sacc[i] * p.qk_scale_log2;
                if (need_mask && j * kBlock + 4 * c + i > pos_mask[k]) sc[i] = kNegInfF;
            }
            float bm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
            bm = fmaxf(bm, __shfl_xor(bm, 16));
            bm = fmaxf(bm, __shfl_xor(bm, 32));
            // block 0 holds token 0 <= every row's position, so m_new is finite
            // from the first block on; the guard only keeps a row whose first
            // block id is out of range free of NaN
            const float m_new = fmaxf(m[k], bm);
            const float m_use = m_new == kNegInfF ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m[k] - m_use);
            float pr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(sc[i] - m_use);
            m[k] = m_new;
            l[k] = l[k] * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
            if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
                for (int t = 0; t < NT; ++t) acc[k][t] *= alpha;
            }
            pop[k] = p_operand_hi_lo(pr);
        }

        // O^T += V^T . P^T, one MFMA per 16 x 16 output tile and group
#pragma unroll
        for (int jj = 0; jj < NVL; ++jj) {
#pragma unroll
            for (int w = 0; w < W; ++w) {
                uint32_t v01, v23;
                if constexpr (KV == kBF16) {
                    v01 = vr[jj][2 * w];
                    v23 = vr[jj][2 * w + 1];
                } else {
                    e4m3x4_to_bf16(vr[jj][w], v01, v23);
                }
                v01 &= keep01;
                v23 &= keep23;
                const bf16x8 a = as_bf16x8(u32x4{v01, v23, v01, v23});
#pragma unroll
                for (int k = 0; k < kGroups; ++k)
                    acc[k][jj * W + w] =
                        __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pop[k], acc[k][jj * W + w], 0, 0, 0);
            }
        }
    };

    // blocks 0 .. nblk-1: ids fetched 64 at a time into one VGPR; block k+1's
    // loads are issued before block k is computed (register buffers A and B)
    for (int k0 = 0; k0 < nblk; k0 += 64) {
        const int kend = min(nblk, k0 + 64);
        int32_t ids = -1;
        if (k0 + lane < kend) ids = table[k0 + lane];
        auto block_id = [&](int k) { return __builtin_amdgcn_readlane(ids, k - k0); };
        auto ok = [&](int32_t b) { return b >= 0 && b < p.num_blocks; };
        u32x4 kA[NKL], vA[NVL], kB[NKL], vB[NVL];
        int k = k0;
        int32_t bA = block_id(k);
        bool okA = ok(bA);
        if (okA) load_block(bA, kA, vA);
        while (true) {
            const int k1 = k + 1;
            bool okB = false;
            if (k1 < kend) {
                const int32_t bB = block_id(k1);
                okB = ok(bB);
                if (okB) load_block(bB, kB, vB);
            }
            if (okA) compute_block(kA, vA, k);
            if (k1 >= kend) break;
            const int k2 = k1 + 1;
            okA = false;
            if (k2 < kend) {
                bA = block_id(k2);
                okA = ok(bA);
                if (okA) load_block(bA, kA, vA);
            }
            if (okB) compute_block(kB, vB, k1);
            if (k2 >= kend) break;
            k = k2;
        }
    }

    // rows: out = O / l (times v_scale); rows before the context start are zero
#pragma unroll
    for (int k = 0; k < kGroups; ++k) {
        float lt = l[k];
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
        if (!valid[k]) continue;
        const float f = live[k] && lt > 0.f ? p.out_scale / lt : 0.f;
        float *orow = p.out + ((int64_t)(q0 + row_tok[k]) * p.num_q_heads + row_head[k]) * D;
        // tile (jj, w) element i is head dim W (16 jj + 4 c + i) + w: 4W contiguous floats per jj
#pragma unroll
        for (int jj = 0; jj < NVL; ++jj) {
            float v[4 * W];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int w = 0; w < W; ++w) v[i * W + w] = live[k] ? acc[k][jj * W + w][i] * f : 0.f;
            float4 *dst = reinterpret_cast<float4 *>(orow + W * (16 * jj + 4 * c));
#pragma unroll
            for (int e = 0; e < W; ++e) dst[e] = make_float4(v[4 * e], v[4 * e + 1], v[4 * e + 2], v[4 * e + 3]);
        }
    }
}

// 16-row groups per wavefront: more rows reuse each K/V load more often but
// hold more accumulators (two groups at head dim 128 exceed 256 registers)
#ifndef PA_PREFILL_GROUPS_D128
#define PA_PREFILL_GROUPS_D128 1
#endif
constexpr int groups_for(int head_dim) { return head_dim == 64 ? 2 : PA_PREFILL_GROUPS_D128; }

template <int KV, int D>
hipError_t launch(const PrefillParams &p, hipStream_t stream) {
    const int64_t grid = (int64_t)p.num_tiles * p.num_seqs * p.num_kv_heads;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    prefill_mfma_kernel<KV, D, groups_for(D)><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace

int prefill_tile_tokens(int head_dim, int group) { return 16 * groups_for(head_dim) * (kThreads / 64) / group; }

bool prefill_supported(int kv, int head_dim, int group) {
    return (kv == kBF16 || kv == kFP8) && (head_dim == 64 || head_dim == 128) && group >= 1 &&
           group <= 16 * groups_for(head_dim) * (kThreads / 64);
}

hipError_t launch_prefill(int kv, int head_dim, const PrefillParams &p, hipStream_t stream) {
    if (kv == kBF16) return head_dim == 64 ? launch<kBF16, 64>(p, stream) : launch<kBF16, 128>(p, stream);
    return head_dim == 64 ? launch<kFP8, 64>(p, stream) : launch<kFP8, 128>(p, stream);
}

}  // namespace pa
