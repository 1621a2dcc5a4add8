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

namespace pa {
namespace {

constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// OCP E4M3FN code -> fp32, exact: the code's exponent and mantissa fields are
// placed in an fp32 pattern (a value 2^-120 times too small; subnormal codes
// land on fp32 subnormals) and multiplied by 2^120.  S.1111.111 is NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
    const uint32_t mag = code & 0x7fu;
    const float f = __uint_as_float(((code & 0x80u) << 24) | (mag << 20)) * 0x1p120f;
    return mag == 0x7fu ? __uint_as_float(0x7fc00000u) : f;
}

// Element e of a 16-byte chunk holding elements of type KV.
template <int KV>
__device__ __forceinline__ float chunk_elem(const uint4 &v, int e) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    if constexpr (KV == kF32) {
        return __uint_as_float(w[e]);
    } else if constexpr (KV == kBF16) {
        return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
    } else {
        return e4m3_to_f32((w[e >> 2] >> (8 * (e & 3))) & 0xffu);
    }
}

__device__ __forceinline__ float wave_max16(float x) {
    // maximum over the 16 lanes of a row (xor butterfly inside the row)
    x = fmaxf(x, __shfl_xor(x, 1));
    x = fmaxf(x, __shfl_xor(x, 2));
    x = fmaxf(x, __shfl_xor(x, 4));
    x = fmaxf(x, __shfl_xor(x, 8));
    return x;
}

template <int KV, int D>
__global__ __launch_bounds__(kThreads) void decode_valu_kernel(DecodeParams p) {
    constexpr int EB = KV == kF32 ? 4 : (KV == kBF16 ? 2 : 1);
    constexpr int X = 16 / EB;          // K: elements per 16-byte run
    constexpr int W = 4 / EB;           // V: head-dim elements per 16-byte cell
    constexpr int NKL = D / X / 4;      // K runs per lane per block
    constexpr int NVL = D / W / 16;     // V cells per lane per block
    constexpr int TILE_BYTES = kBlock * D * EB;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int t = lane & 15;
    const int c = lane >> 4;

    int bid = blockIdx.x;
    const int part = bid % p.max_partitions;
    bid /= p.max_partitions;
    const int h = bid % p.num_q_heads;
    const int s = bid / p.num_q_heads;
    const int g = h / p.group;

    int ctx = p.context_lens[s];
    ctx = ctx < 0 ? 0 : (ctx > p.max_blocks_per_seq * kBlock ? p.max_blocks_per_seq * kBlock : ctx);
    const int nparts = (ctx + p.partition_tokens - 1) / p.partition_tokens;
    if (part >= (nparts > 1 ? nparts : 1)) return;
    const int tok0 = part * p.partition_tokens;
    const int tok1 = min(ctx, tok0 + p.partition_tokens);
    const int blk0 = tok0 / kBlock;
    const int blk1 = (tok1 + kBlock - 1) / kBlock;

    // q elements matching this lane's K runs
    float qv[NKL][X];
    const int64_t qrow = ((int64_t)s * p.num_q_heads + h) * D;
#pragma unroll
    for (int j = 0; j < NKL; ++j) {
#pragma unroll
        for (int x = 0; x < X; ++x) {
            const int d = (c + 4 * j) * X + x;
            if constexpr (KV == kF32) {
                qv[j][x] = reinterpret_cast<const float *>(p.q)[qrow + d];
            } else {
                qv[j][x] = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(p.q)[qrow + d] << 16);
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

    const int32_t *table = p.block_tables + (int64_t)s * p.max_blocks_per_seq;
    const char *kbase = static_cast<const char *>(p.k_pool);
    const char *vbase = static_cast<const char *>(p.v_pool);

    auto load_block = [&](int32_t b, uint4 (&kc)[NKL], uint4 (&vc)[NVL]) {
        const int64_t tile = ((int64_t)b * p.num_kv_heads + g) * TILE_BYTES;
        const char *kt = kbase + tile;
        const char *vt = vbase + tile;
#pragma unroll
        for (int jk = 0; jk < NKL; ++jk)
            kc[jk] = *reinterpret_cast<const uint4 *>(kt + ((c + 4 * jk) * kBlock + t) * 16);
#pragma unroll
        for (int jj = 0; jj < NVL; ++jj)
            vc[jj] = *reinterpret_cast<const uint4 *>(vt + (c * (D / W) + 16 * jj + t) * 16);
    };

    auto compute_block = [&](const uint4 (&kc)[NKL], const uint4 (&vc)[NVL], int j) {
        float part_dot = 0.f;
#pragma unroll
        for (int jk = 0; jk < NKL; ++jk)
#pragma unroll
            for (int x = 0; x < X; ++x) part_dot += qv[jk][x] * chunk_elem<KV>(kc[jk], x);
        part_dot += __shfl_xor(part_dot, 16);
        part_dot += __shfl_xor(part_dot, 32);

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
#pragma unroll
        for (int jj = 0; jj < NVL; ++jj) {
#pragma unroll
            for (int w = 0; w < W; ++w) {
                float sum = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float term = pw[i] * chunk_elem<KV>(vc[jj], 4 * w + i);
                    sum += live[i] ? term : 0.f;
                }
                acc[jj][w] += sum;
            }
        }
    };

    // This wavefront's blocks are j = blk0 + wave + 4k, k = 0..nk-1; ids are
    // fetched 64 at a time into one VGPR, and block k+1's loads are issued
    // before block k is computed (register buffers A and B in turn).
    const int nk = blk1 - blk0 > wave ? (blk1 - blk0 - wave + 3) / 4 : 0;
    for (int k0 = 0; k0 < nk; k0 += 64) {
        const int kend = min(nk, k0 + 64);
        int32_t ids = -1;
        if (k0 + lane < kend) ids = table[blk0 + wave + 4 * (k0 + lane)];
        auto block_id = [&](int k) { return __builtin_amdgcn_readlane(ids, k - k0); };
        auto valid = [&](int32_t b) { return b >= 0 && b < p.num_blocks; };
        uint4 kA[NKL], vA[NVL], kB[NKL], vB[NVL];
        int k = k0;
        int32_t bA = block_id(k);
        bool okA = valid(bA);
        if (okA) load_block(bA, kA, vA);
        while (true) {
            const int k1 = k + 1;
            bool okB = false;
            if (k1 < kend) {
                const int32_t bB = block_id(k1);
                okB = valid(bB);
                if (okB) load_block(bB, kB, vB);
            }
            if (okA) compute_block(kA, vA, blk0 + wave + 4 * k);
            if (k1 >= kend) break;
            const int k2 = k1 + 1;
            okA = false;
            if (k2 < kend) {
                bA = block_id(k2);
                okA = valid(bA);
                if (okA) load_block(bA, kA, vA);
            }
            if (okB) compute_block(kB, vB, blk0 + wave + 4 * k1);
            if (k2 >= kend) break;
            k = k2;
        }
    }

    // add the four token quarters (rows c = 0..3)
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
#pragma unroll
    for (int jj = 0; jj < NVL; ++jj)
#pragma unroll
        for (int w = 0; w < W; ++w) {
            acc[jj][w] += __shfl_xor(acc[jj][w], 16);
            acc[jj][w] += __shfl_xor(acc[jj][w], 32);
        }

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

    if (threadIdx.x < D) {
        const int d = threadIdx.x;
        const float M = fmaxf(fmaxf(sm_m[0], sm_m[1]), fmaxf(sm_m[2], sm_m[3]));
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float f = sm_m[w] == kNegInf ? 0.f : exp2f(sm_m[w] - M);
            L += sm_l[w] * f;
            O += sm_acc[w][d] * f;
        }
        const int64_t row = (int64_t)s * p.num_q_heads + h;
        if (nparts <= 1) {
            p.out[row * D + d] = L > 0.f ? (O / L) * p.out_scale : 0.f;
        } else {
            const int64_t pr = row * p.max_partitions + part;
            p.ws_acc[pr * D + d] = O;
            if (d == 0) {
                p.ws_m[pr] = M;
                p.ws_l[pr] = L;
            }
        }
    }
}

// Merge the partitions of one (sequence, query head) row, in partition order:
// M = max_p m_p, out = sum_p acc_p 2^(m_p - M) / sum_p l_p 2^(m_p - M).
template <int D>
__global__ __launch_bounds__(kThreads) void decode_reduce_kernel(DecodeParams p) {
    const int64_t row = blockIdx.x;  // s * Hq + h
    const int s = (int)(row / p.num_q_heads);
    int ctx = p.context_lens[s];
    ctx = ctx < 0 ? 0 : (ctx > p.max_blocks_per_seq * kBlock ? p.max_blocks_per_seq * kBlock : ctx);
    const int nparts = (ctx + p.partition_tokens - 1) / p.partition_tokens;
    if (nparts <= 1) return;  // written by the partition kernel
    const int d = threadIdx.x;
    if (d >= D) return;
    const float *ms = p.ws_m + row * p.max_partitions;
    const float *ls = p.ws_l + row * p.max_partitions;
    const float *as = p.ws_acc + row * p.max_partitions * D;
    float M = kNegInf;
    for (int i = 0; i < nparts; ++i) M = fmaxf(M, ms[i]);
    float L = 0.f, O = 0.f;
    if (M != kNegInf) {
        for (int i = 0; i < nparts; ++i) {
            const float f = exp2f(ms[i] - M);
            L += ls[i] * f;
            O += as[(int64_t)i * D + d] * f;
        }
    }
    p.out[row * D + d] = L > 0.f ? (O / L) * p.out_scale : 0.f;
}

template <int KV, int D>
hipError_t launch_valu(const DecodeParams &p, hipStream_t stream) {
    const int64_t grid = (int64_t)p.num_seqs * p.num_q_heads * p.max_partitions;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    decode_valu_kernel<KV, D><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(p);
    return hipGetLastError();
}

template <int KV>
hipError_t launch_valu_d(int head_dim, const DecodeParams &p, hipStream_t stream) {
    return head_dim == 64 ? launch_valu<KV, 64>(p, stream) : launch_valu<KV, 128>(p, stream);
}

}  // namespace

hipError_t launch_decode_valu(int kv, int head_dim, const DecodeParams &p, hipStream_t stream) {
    if (kv == kF32) return launch_valu_d<kF32>(head_dim, p, stream);
    if (kv == kBF16) return launch_valu_d<kBF16>(head_dim, p, stream);
    return launch_valu_d<kFP8>(head_dim, p, stream);
}

hipError_t launch_decode_reduce(int head_dim, const DecodeParams &p, hipStream_t stream) {
    const int64_t grid = (int64_t)p.num_seqs * p.num_q_heads;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    if (head_dim == 64)
        decode_reduce_kernel<64><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(p);
    else
        decode_reduce_kernel<128><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace pa
