/*
 * pa_oracle.c -- plain, slow, fp64 CPU oracle for paged decode attention and
 * the two operations that keep the paged KV pool consistent.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header or constant generator with
 * the GPU library; the pool layout and dtype codes below are an interface that
 * both sides implement independently.
 *
 * What it follows (citations are to the source pages by title and section):
 *  - "PagedAttention" glossary page (Ultralytics, Spanish), section on how
 *    paging works and its PyTorch schematic: the KV cache of a request lives
 *    in fixed-size 16-token blocks taken from a shared pool; token `pos`
 *    lives in block `table[pos / 16]` at slot `pos % 16`; reading through the
 *    table in table order returns the request's keys unchanged.
 *  - Same page, section on sharing blocks between sequences: several tables
 *    may name one physical block; before a sequence writes into a block that
 *    others still use, the block is copied (copy-on-write).
 *  - Same page, section on related techniques: grouped-query attention shares
 *    one KV head among several query heads; an 8-bit (FP8) cache stores K/V
 *    in half the bytes of a 16-bit one.
 *  - Russian page on PagedAttention and the vLLM KV cache, section on logical
 *    order vs physical placement: attention reads the data through the table
 *    keeping the logical order.
 *  - French page, second article, section on what the KV cache is: to
 *    produce token n+1 the model needs K and V of tokens 1..n; only the new
 *    token's K/V is computed and appended to the cache.
 *
 * The pages print no attention formula.  The reading taken is the standard
 * scaled dot-product attention of one query over the gathered context:
 *     s_t = scale * <q, K_t>,  out = sum_t exp(s_t - max s) V_t / sum_t exp(s_t - max s)
 * written out directly in fp64 (no blocking, no online rescaling, no split).
 *
 * Pool layout (an interface, implemented separately by the GPU library):
 *   k_pool and v_pool each hold NB*Hkv tiles; tile (b, g) starts at element
 *   (b*Hkv + g) * 16 * D and holds the 16 token slots of block b for KV head g.
 *   Within a K tile, element (t, d) sits at ((d / X) * 16 + t) * X + d % X
 *   with X = 16 / elem_bytes (16-byte runs of the head dimension, one per
 *   token, token-major inside a run).
 *   Within a V tile, element (t, d) sits at
 *   ((t / 4) * (D / W) + d / W) * 4 * W + (d % W) * 4 + t % 4
 *   with W = 4 / elem_bytes (16-byte cells of 4 consecutive tokens by W
 *   consecutive head-dim elements, tokens fastest).
 * The pages fix which (block, slot) a token occupies, not the byte order
 * inside a block; this order is the GPU library's choice and is reproduced
 * here so that pools can be compared byte for byte.
 *
 * dtype codes: 0 = fp32, 1 = bf16, 2 = fp8 OCP E4M3FN (bias 7, max 448,
 * no infinities, NaN = S.1111.111).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8 = 2 };

static int orc_elem_bytes(int dt)
{
    return dt == ORC_F32 ? 4 : (dt == ORC_BF16 ? 2 : 1);
}

/* ---------------------------------------------------------------- fp8 codec */

/* Value of an OCP E4M3FN code, from the format's definition: sign bit,
 * 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 is subnormal
 * (m/8 * 2^-6); S.1111.111 is NaN; there is no infinity. */
double orc_fp8_decode(uint8_t code)
{
    int sign = code >> 7;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double mag;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* The 127 finite non-negative magnitudes, indexed by code 0x00..0x7E; they
 * increase with the code. */
static double orc_fp8_mag[127];
static int orc_fp8_ready = 0;

static void orc_fp8_init(void)
{
    if (orc_fp8_ready)
        return;
    for (int c = 0; c < 127; c++)
        orc_fp8_mag[c] = orc_fp8_decode((uint8_t)c);
    orc_fp8_ready = 1;
}

/* Round an fp32 value to the nearest E4M3FN value, ties to the even code
 * (even mantissa), saturating magnitudes beyond 448 to +-448.  NaN maps to
 * the NaN code with the input's sign.  All comparisons are exact in fp64. */
uint8_t orc_fp8_encode(float x)
{
    orc_fp8_init();
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    if (isnan(x))
        return (uint8_t)(sign | 0x7F);
    double a = fabs((double)x);
    if (a >= orc_fp8_mag[126])
        return (uint8_t)(sign | 0x7E);
    /* largest code lo with mag[lo] <= a (binary search on the sorted table) */
    int lo = 0, hi = 126;
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (orc_fp8_mag[mid] <= a)
            lo = mid;
        else
            hi = mid;
    }
    double dlo = a - orc_fp8_mag[lo];
    double dhi = orc_fp8_mag[hi] - a;
    int c;
    if (dlo < dhi)
        c = lo;
    else if (dhi < dlo)
        c = hi;
    else
        c = (lo % 2 == 0) ? lo : hi;
    return (uint8_t)(sign | c);
}

void orc_fp8_encode_array(const float *x, uint8_t *out, int64_t n)
{
    orc_fp8_init();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_fp8_encode(x[i]);
}

/* ------------------------------------------------------------ pool layout */

static int64_t orc_k_offset(int64_t b, int g, int t, int d, int Hkv, int D, int eb)
{
    int X = 16 / eb;
    int64_t tile = (b * Hkv + g) * 16 * (int64_t)D;
    return tile + ((int64_t)(d / X) * 16 + t) * X + d % X;
}

static int64_t orc_v_offset(int64_t b, int g, int t, int d, int Hkv, int D, int eb)
{
    int W = 4 / eb;
    int64_t tile = (b * Hkv + g) * 16 * (int64_t)D;
    return tile + ((int64_t)(t / 4) * (D / W) + d / W) * 4 * W + (d % W) * 4 + t % 4;
}

/* Read element `idx` of a pool or input array of dtype `dt` as a real number
 * (fp8 codes are decoded and multiplied by their scale). */
static double orc_load(const uint8_t *base, int64_t idx, int dt, double fp8_scale)
{
    if (dt == ORC_F32) {
        float f;
        memcpy(&f, base + idx * 4, 4);
        return (double)f;
    }
    if (dt == ORC_BF16) {
        uint16_t h;
        uint32_t u;
        float f;
        memcpy(&h, base + idx * 2, 2);
        u = (uint32_t)h << 16;
        memcpy(&f, &u, 4);
        return (double)f;
    }
    return orc_fp8_decode(base[idx]) * fp8_scale;
}

/* Same, as the fp32 value of a 16/32-bit input element. */
static float orc_load_f32(const uint8_t *base, int64_t idx, int dt)
{
    if (dt == ORC_F32) {
        float f;
        memcpy(&f, base + idx * 4, 4);
        return f;
    } else {
        uint16_t h;
        uint32_t u;
        float f;
        memcpy(&h, base + idx * 2, 2);
        u = (uint32_t)h << 16;
        memcpy(&f, &u, 4);
        return f;
    }
}

/* ------------------------------------------------- cache write (scatter) */

/* For each new token i and KV head g, store k[i][g][:] and v[i][g][:] in the
 * slot named by slot_mapping[i]: block slot/16, position slot%16 (the slot
 * rule of the worked example).  A negative slot skips the token.  A 16/32-bit
 * pool of the input's dtype receives the input bits unchanged; an fp8 pool
 * receives encode(x * inv_scale) with x the input as fp32 and
 * inv_scale = 1/scale rounded to fp32, the product rounded to fp32.
 * Tokens are processed in index order. */
void orc_reshape_and_cache(uint8_t *k_pool, uint8_t *v_pool, int pool_dt,
                           int64_t num_blocks, int Hkv, int D,
                           const uint8_t *k, const uint8_t *v, int in_dt,
                           const int32_t *slot_mapping, int64_t num_tokens,
                           float k_scale, float v_scale)
{
    int peb = orc_elem_bytes(pool_dt);
    int ieb = orc_elem_bytes(in_dt);
    float inv_k = 1.0f / k_scale;
    float inv_v = 1.0f / v_scale;
    for (int64_t i = 0; i < num_tokens; i++) {
        int32_t slot = slot_mapping[i];
        if (slot < 0)
            continue;
        int64_t b = slot / 16;
        int t = slot % 16;
        if (b >= num_blocks)
            continue;
        for (int g = 0; g < Hkv; g++) {
            for (int d = 0; d < D; d++) {
                int64_t src = ((int64_t)i * Hkv + g) * D + d;
                int64_t kd = orc_k_offset(b, g, t, d, Hkv, D, peb);
                int64_t vd = orc_v_offset(b, g, t, d, Hkv, D, peb);
                if (pool_dt == ORC_FP8) {
                    float xk = orc_load_f32(k, src, in_dt);
                    float xv = orc_load_f32(v, src, in_dt);
                    float yk = xk * inv_k;
                    float yv = xv * inv_v;
                    k_pool[kd] = orc_fp8_encode(yk);
                    v_pool[vd] = orc_fp8_encode(yv);
                } else {
                    memcpy(k_pool + kd * peb, k + src * ieb, (size_t)peb);
                    memcpy(v_pool + vd * peb, v + src * ieb, (size_t)peb);
                }
            }
        }
    }
}

/* ------------------------------------------------- copy-on-write block copy */

/* For each pair (src, dst), in order, copy every KV head's K and V tile of
 * block src over those of block dst. */
void orc_copy_blocks(uint8_t *k_pool, uint8_t *v_pool, int pool_dt, int Hkv, int D,
                     const int32_t *pairs, int64_t num_pairs)
{
    size_t bytes = (size_t)Hkv * 16 * (size_t)D * (size_t)orc_elem_bytes(pool_dt);
    for (int64_t p = 0; p < num_pairs; p++) {
        int64_t src = pairs[2 * p], dst = pairs[2 * p + 1];
        memmove(k_pool + dst * bytes, k_pool + src * bytes, bytes);
        memmove(v_pool + dst * bytes, v_pool + src * bytes, bytes);
    }
}

/* --------------------------------------------------- swap to / from host */

/* For each pair (device block, host slot), in order: direction 0 copies
 * every KV head's K and V tile of the block into the slot of the host pools
 * (a slot holds one whole block), direction 1 copies the slot back into the
 * block (the French page: when memory is full, small pages move to the CPU).
 * Pairs with an id outside [0, num_blocks) or [0, num_slots) are skipped. */
void orc_swap_blocks(uint8_t *k_pool, uint8_t *v_pool, uint8_t *host_k, uint8_t *host_v,
                     int pool_dt, int Hkv, int D, int64_t num_blocks, int64_t num_slots,
                     const int32_t *pairs, int64_t num_pairs, int direction)
{
    size_t bytes = (size_t)Hkv * 16 * (size_t)D * (size_t)orc_elem_bytes(pool_dt);
    for (int64_t p = 0; p < num_pairs; p++) {
        int64_t b = pairs[2 * p], h = pairs[2 * p + 1];
        if (b < 0 || b >= num_blocks || h < 0 || h >= num_slots)
            continue;
        if (direction == 0) {
            memcpy(host_k + h * bytes, k_pool + b * bytes, bytes);
            memcpy(host_v + h * bytes, v_pool + b * bytes, bytes);
        } else {
            memcpy(k_pool + b * bytes, host_k + h * bytes, bytes);
            memcpy(v_pool + b * bytes, host_v + h * bytes, bytes);
        }
    }
}

/* ------------------------------------------------------ gather (read back) */

/* Copy the raw elements of tokens 0..n-1 of KV head g, read through `table`
 * in logical order, into out[n][D] (elements of the pool's dtype). */
void orc_gather(const uint8_t *pool, int is_v, int pool_dt, int Hkv, int D,
                const int32_t *table, int64_t n, int g, uint8_t *out)
{
    int eb = orc_elem_bytes(pool_dt);
    for (int64_t pos = 0; pos < n; pos++) {
        int64_t b = table[pos / 16];
        int t = (int)(pos % 16);
        for (int d = 0; d < D; d++) {
            int64_t off = is_v ? orc_v_offset(b, g, t, d, Hkv, D, eb)
                               : orc_k_offset(b, g, t, d, Hkv, D, eb);
            memcpy(out + (pos * D + d) * eb, pool + off * eb, (size_t)eb);
        }
    }
}

/* ------------------------------------------------------ decode attention */

/* One output row: the query row stored at q[qrow][0..D) (query head h)
 * against tokens 0..n-1 of KV head g = h / (Hq / Hkv), gathered through the
 * sequence's block table `table` in logical order.  n <= 0 gives a zero row. */
static void orc_attend_row(const uint8_t *k_pool, const uint8_t *v_pool, int pool_dt,
                           double k_scale, double v_scale, int Hkv, int D,
                           const uint8_t *q, int q_dt, int64_t qrow, int Hq, int h,
                           const int32_t *table, int64_t n, double scale,
                           double *out_row, double *score, double *kbuf)
{
    int eb = orc_elem_bytes(pool_dt);
    int group = Hq / Hkv;
    int g = h / group;
    for (int d = 0; d < D; d++)
        out_row[d] = 0.0;
    if (n <= 0)
        return;
    for (int d = 0; d < D; d++)
        kbuf[d] = orc_load(q, qrow * D + d, q_dt, 1.0);
    double m = -INFINITY;
    for (int64_t t = 0; t < n; t++) {
        int64_t b = table[t / 16];
        int o = (int)(t % 16);
        double dot = 0.0;
        for (int d = 0; d < D; d++)
            dot += kbuf[d] * orc_load(k_pool, orc_k_offset(b, g, o, d, Hkv, D, eb), pool_dt, k_scale);
        score[t] = scale * dot;
        if (score[t] > m)
            m = score[t];
    }
    double denom = 0.0;
    for (int64_t t = 0; t < n; t++) {
        double w = exp(score[t] - m);
        int64_t b = table[t / 16];
        int o = (int)(t % 16);
        denom += w;
        for (int d = 0; d < D; d++)
            out_row[d] += w * orc_load(v_pool, orc_v_offset(b, g, o, d, Hkv, D, eb), pool_dt, v_scale);
    }
    for (int d = 0; d < D; d++)
        out_row[d] /= denom;
}

/* Decode row: the one query of sequence s (q laid out [S][Hq][D]), head h,
 * against all ctx[s] tokens of its context. */
static void orc_attend_one(const uint8_t *k_pool, const uint8_t *v_pool, int pool_dt,
                           double k_scale, double v_scale, int Hkv, int D,
                           const uint8_t *q, int q_dt, int Hq, const int32_t *tables,
                           int MBS, const int32_t *ctx, double scale, int s, int h,
                           double *out_row, double *score, double *kbuf)
{
    int64_t qrow = (int64_t)s * Hq + h;
    orc_attend_row(k_pool, v_pool, pool_dt, k_scale, v_scale, Hkv, D, q, q_dt, qrow, Hq, h,
                   tables + (int64_t)s * MBS, ctx[s], scale, out_row, score, kbuf);
}

/* Decode attention for all (s, h) rows, or for the `num_rows` rows listed in
 * rows[2*i] = s, rows[2*i+1] = h (out then holds num_rows x D values).
 * Each row is computed serially, so results do not depend on `threads`. */
int orc_paged_attention(const uint8_t *k_pool, const uint8_t *v_pool, int pool_dt,
                        float k_scale, float v_scale, int Hkv, int D,
                        const uint8_t *q, int q_dt, int S, int Hq,
                        const int32_t *tables, int MBS, const int32_t *ctx,
                        float scale, double *out, const int32_t *rows,
                        int64_t num_rows, int threads)
{
    if (Hkv <= 0 || Hq % Hkv != 0)
        return -1;
    int64_t total = rows ? num_rows : (int64_t)S * Hq;
    int64_t max_n = 1;
    for (int s = 0; s < S; s++)
        if (ctx[s] > max_n)
            max_n = ctx[s];
#ifdef _OPENMP
    if (threads > 0)
        omp_set_num_threads(threads);
#endif
    int failed = 0;
#pragma omp parallel
    {
        double *score = (double *)malloc(sizeof(double) * (size_t)max_n);
        double *kbuf = (double *)malloc(sizeof(double) * (size_t)D);
        if (!score || !kbuf) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t r = 0; r < total; r++) {
            int s, h;
            if (rows) {
                s = rows[2 * r];
                h = rows[2 * r + 1];
            } else {
                s = (int)(r / Hq);
                h = (int)(r % Hq);
            }
            if (score && kbuf)
                orc_attend_one(k_pool, v_pool, pool_dt, (double)k_scale, (double)v_scale,
                               Hkv, D, q, q_dt, Hq, tables, MBS, ctx, (double)scale, s, h,
                               out + r * D, score, kbuf);
        }
        free(score);
        free(kbuf);
    }
    return failed ? -2 : 0;
}

/* ------------------------------------------------ prefill (chunked) attention */

/* Prefill of a chunk of new tokens per sequence.  The chunk of sequence s is
 * the last n_s = query_start[s+1] - query_start[s] tokens of its ctx[s]-token
 * context, already written to the pool (the page on the KV cache: the
 * prompt's K/V is stored first; the Russian page: memory for the input is
 * allocated first).  Chunk token i sits at position p = ctx[s] - n_s + i and,
 * as in generation, sees the K/V of itself and every earlier token
 * (positions 0..p) -- the same attention a decode step with ctx = p + 1
 * would compute for it.  q and out are [query_start[S]][Hq][D]; a row with
 * p < 0 (a chunk longer than its context) is zero.
 * With `rows`, only the listed (chunk row, head) pairs are computed, rows[2i]
 * being the global chunk-token index and rows[2i+1] the head, and out holds
 * num_rows x D values.  Each row is computed serially. */
int orc_prefill_attention(const uint8_t *k_pool, const uint8_t *v_pool, int pool_dt,
                          float k_scale, float v_scale, int Hkv, int D,
                          const uint8_t *q, int q_dt, int S, int Hq,
                          const int32_t *query_start, const int32_t *tables, int MBS,
                          const int32_t *ctx, float scale, double *out,
                          const int32_t *rows, int64_t num_rows, int threads)
{
    if (Hkv <= 0 || Hq % Hkv != 0 || S < 0)
        return -1;
    int64_t total_q = query_start[S];
    int64_t total = rows ? num_rows : total_q * Hq;
    int64_t max_n = 1;
    for (int s = 0; s < S; s++)
        if (ctx[s] > max_n)
            max_n = ctx[s];
#ifdef _OPENMP
    if (threads > 0)
        omp_set_num_threads(threads);
#endif
    int failed = 0;
#pragma omp parallel
    {
        double *score = (double *)malloc(sizeof(double) * (size_t)max_n);
        double *kbuf = (double *)malloc(sizeof(double) * (size_t)D);
        if (!score || !kbuf) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < total; r++) {
            int64_t qi;
            int h;
            if (rows) {
                qi = rows[2 * r];
                h = rows[2 * r + 1];
            } else {
                qi = r / Hq;
                h = (int)(r % Hq);
            }
            /* the sequence whose chunk holds global chunk token qi */
            int s = 0;
            while (s < S - 1 && query_start[s + 1] <= qi)
                s++;
            int64_t n_new = query_start[s + 1] - query_start[s];
            int64_t i = qi - query_start[s];
            int64_t pos = (int64_t)ctx[s] - n_new + i;
            if (score && kbuf)
                orc_attend_row(k_pool, v_pool, pool_dt, (double)k_scale, (double)v_scale, Hkv, D,
                               q, q_dt, qi * Hq + h, Hq, h, tables + (int64_t)s * MBS, pos + 1,
                               (double)scale, out + r * D, score, kbuf);
        }
        free(score);
        free(kbuf);
    }
    return failed ? -2 : 0;
}

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
