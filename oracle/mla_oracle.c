/*
 * CPU oracle for absorbed MLA decode over a paged latent cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant with
 * the HIP library; both sides only see the same seeded host inputs.
 *
 * Everything here is the plain definition, evaluated in double precision on
 * the exact stored input values (fp32 / bf16 / fp8-e4m3 codes are decoded to
 * double without rounding).  No blocking, fusion or reordering beyond the
 * definitions cited below.  The only parallelism is an OpenMP loop over
 * independent output rows.
 *
 * Sources (the four pages on DeepSeek MLA):
 *  [huny]    blog.huny.dev, "DeepSeek Multi-Head Latent Attention(MLA) 해부 ..."
 *  [donmain] donmain.dev, "KV Cache를 10분의 1로 줄인 MLA의 트릭"
 *  [vllm]    blog.secrett2633.cloud, "[vLLM] Multi-head Latent Attention:
 *            KV 캐시를 압축하는 DeepSeek의 어텐션"
 *  [thaki]   thakicloud.com, "transformer-attention-kv-cache-math"
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Storage formats of a cached token row [c (d_c) | k^R (d_r)]. */
enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_FP8_E4M3 = 2, ORACLE_F16 = 3, ORACLE_FP8_E5M2 = 4,
       ORACLE_FP8_E4M3_ROW = 5 };

/* Tokens per paged block: the FlashMLA backend accepts only 64
 * ([vllm], "FlashMLABackend: 하드웨어 요구사항"). */
#define ORACLE_BLOCK 64

/* Threads the OpenMP loops use (reported next to oracle timings). */
int oracle_threads(void) { return omp_get_max_threads(); }

/* ---------------------------------------------------------------------- */
/* Number formats, decoded from their definitions.                          */
/* ---------------------------------------------------------------------- */

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double oracle_bf16_to_f64(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP FP8 E4M3 ("fn" variant): 1 sign, 4 exponent bits (bias 7), 3 mantissa
 * bits, no infinities, S.1111.111 is NaN, exponent field 0 is subnormal.
 * The fp8 latent cache is named in [huny] §6 (FP8 E4M3 or E5M2) and
 * [vllm] "FP8 MLA 지원". */
double oracle_e4m3_to_f64(uint8_t code)
{
    int s = code >> 7, e = (code >> 3) & 0xF, m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);                 /* m/8 * 2^(1-7) */
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* IEEE binary16: 1 sign, 5 exponent bits (bias 15), 10 mantissa bits;
 * exponent field 0 is subnormal (m * 2^-24), 31 is inf / NaN.  The fp16 cache
 * is one of the kv-cache dtypes of [vllm] "FlashMLABackend". */
double oracle_f16_to_f64(uint16_t bits)
{
    int s = bits >> 15, e = (bits >> 10) & 0x1F, m = bits & 0x3FF;
    double v;
    if (e == 31) return m ? NAN : (s ? -INFINITY : INFINITY);
    if (e == 0)
        v = ldexp((double)m, -24);
    else
        v = ldexp(1.0 + (double)m / 1024.0, e - 15);
    return s ? -v : v;
}

/* OCP FP8 E5M2: 1 sign, 5 exponent bits (bias 15), 2 mantissa bits, IEEE-like
 * (exponent 31: mantissa 0 = inf, else NaN), exponent 0 subnormal (m/4 2^-14).
 * [huny] §6 names E4M3 or E5M2 for the latent cache. */
double oracle_e5m2_to_f64(uint8_t code)
{
    int s = code >> 7, e = (code >> 2) & 0x1F, m = code & 3;
    double v;
    if (e == 31) return m ? NAN : (s ? -INFINITY : INFINITY);
    if (e == 0)
        v = ldexp((double)m, -16);                /* m/4 * 2^(1-15) */
    else
        v = ldexp(1.0 + (double)m / 4.0, e - 15);
    return s ? -v : v;
}

/* Round-to-nearest-even into E5M2, saturating to +-57344 (the largest finite
 * value) as the E4M3 encoder saturates; NaN -> 0x7F.  Scan of every
 * non-negative finite code, ties to the even mantissa. */
uint8_t oracle_f64_to_e5m2(double x)
{
    if (isnan(x)) return 0x7F;
    uint8_t sign = (x < 0) ? 0x80 : 0x00;
    double a = fabs(x);
    if (a >= 57344.0) return sign | 0x7B;
    int best = 0;
    double best_err = INFINITY;
    for (int c = 0; c <= 0x7B; ++c) {
        double err = fabs(oracle_e5m2_to_f64((uint8_t)c) - a);
        if (err < best_err || (err == best_err && (c & 1) == 0)) {
            best = c;
            best_err = err;
        }
    }
    return sign | (uint8_t)best;
}

/* Round-to-nearest-even into E4M3, saturating to +-448 (the largest finite
 * value).  Done the slow, obvious way: scan every non-negative finite code for
 * the nearest value; on a tie take the code whose mantissa LSB is 0. */
uint8_t oracle_f64_to_e4m3(double x)
{
    if (isnan(x)) return 0x7F;
    uint8_t sign = (x < 0) ? 0x80 : 0x00;
    double a = fabs(x);
    if (a >= 448.0) return sign | 0x7E;
    int best = 0;
    double best_err = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        double err = fabs(oracle_e4m3_to_f64((uint8_t)c) - a);
        if (err < best_err || (err == best_err && (c & 1) == 0)) {
            best = c;
            best_err = err;
        }
    }
    return sign | (uint8_t)best;
}

/* ---------------------------------------------------------------------- */
/* Paged latent cache                                                       */
/* ---------------------------------------------------------------------- */

/* Bytes of one 64-token block in each storage format.
 *  F32 / BF16: 64 rows of [c | k^R], the combined kv_c_and_k_pe row of
 *              [vllm] "FlashMLAImpl: 어텐션 연산" (576 wide in DeepSeek-V2,
 *              [donmain] "위치 정보와 압축의 충돌").
 *  FP8:        c as e4m3 codes [64][d_c], then k^R kept in bf16 [64][d_r]
 *              ([huny] §6: the RoPE key keeps 16-bit precision), with one
 *              fp32 scale per block held in a separate array.
 *  F16:        64 rows of [c | k^R] in IEEE fp16 ([vllm] kv-cache dtypes).
 *  FP8 E5M2:   as FP8 with e5m2 codes ([huny] §6 "E4M3 or E5M2").
 *  FP8 E4M3 row: the whole row [c | k^R] as e4m3 codes [64][d_c + d_r], one
 *              scale per block for both parts (an fp8 cache read literally
 *              as "the cache stored as e4m3"). */
int64_t oracle_block_bytes(int fmt, int d_c, int d_r)
{
    switch (fmt) {
    case ORACLE_F32:  return (int64_t)ORACLE_BLOCK * (d_c + d_r) * 4;
    case ORACLE_BF16: return (int64_t)ORACLE_BLOCK * (d_c + d_r) * 2;
    case ORACLE_FP8_E4M3:
    case ORACLE_FP8_E5M2: return (int64_t)ORACLE_BLOCK * d_c + (int64_t)ORACLE_BLOCK * d_r * 2;
    case ORACLE_F16: return (int64_t)ORACLE_BLOCK * (d_c + d_r) * 2;
    case ORACLE_FP8_E4M3_ROW: return (int64_t)ORACLE_BLOCK * (d_c + d_r);
    default: return -1;
    }
}

/* Decode logical token p of sequence b into c[d_c], kr[d_r] (doubles).
 * The row lives in block bt[b][p / 64], slot p % 64 (PagedAttention block
 * table, [huny] §6 and [vllm] "MLA의 MQA 디코딩 경로"). */
static void load_row(const uint8_t *pool, int fmt, const float *blk_scale,
                     const int32_t *bt, int bt_stride, int b, int p,
                     int d_c, int d_r, double *c, double *kr)
{
    int64_t blk = bt[(int64_t)b * bt_stride + p / ORACLE_BLOCK];
    int slot = p % ORACLE_BLOCK;
    const uint8_t *base = pool + blk * oracle_block_bytes(fmt, d_c, d_r);
    if (fmt == ORACLE_F32) {
        const float *row = (const float *)base + (int64_t)slot * (d_c + d_r);
        for (int f = 0; f < d_c; ++f) c[f] = (double)row[f];
        for (int f = 0; f < d_r; ++f) kr[f] = (double)row[d_c + f];
    } else if (fmt == ORACLE_BF16) {
        const uint16_t *row = (const uint16_t *)base + (int64_t)slot * (d_c + d_r);
        for (int f = 0; f < d_c; ++f) c[f] = oracle_bf16_to_f64(row[f]);
        for (int f = 0; f < d_r; ++f) kr[f] = oracle_bf16_to_f64(row[d_c + f]);
    } else if (fmt == ORACLE_F16) {
        const uint16_t *row = (const uint16_t *)base + (int64_t)slot * (d_c + d_r);
        for (int f = 0; f < d_c; ++f) c[f] = oracle_f16_to_f64(row[f]);
        for (int f = 0; f < d_r; ++f) kr[f] = oracle_f16_to_f64(row[d_c + f]);
    } else if (fmt == ORACLE_FP8_E4M3_ROW) {
        const uint8_t *row = base + (int64_t)slot * (d_c + d_r);
        double sc = (double)blk_scale[blk];
        for (int f = 0; f < d_c; ++f) c[f] = oracle_e4m3_to_f64(row[f]) * sc;
        for (int f = 0; f < d_r; ++f) kr[f] = oracle_e4m3_to_f64(row[d_c + f]) * sc;
    } else {
        const uint8_t *crow = base + (int64_t)slot * d_c;
        const uint16_t *krow = (const uint16_t *)(base + (int64_t)ORACLE_BLOCK * d_c) + (int64_t)slot * d_r;
        double sc = (double)blk_scale[blk];
        for (int f = 0; f < d_c; ++f)
            c[f] = (fmt == ORACLE_FP8_E5M2 ? oracle_e5m2_to_f64(crow[f]) : oracle_e4m3_to_f64(crow[f])) * sc;
        for (int f = 0; f < d_r; ++f) kr[f] = oracle_bf16_to_f64(krow[f]);
    }
}

/* Paged gather: out[b][p][:] = bytes of the row of logical token p of
 * sequence b, for p < seq_lens[b]; the rest of out is left untouched.
 * For FP8 the logical row is the d_c code bytes followed by the 2*d_r bytes
 * of the bf16 RoPE key. */
int oracle_gather(const void *pool_v, int fmt, int d_c, int d_r,
                  const int32_t *bt, int bt_stride, const int32_t *seq_lens,
                  int B, int max_tokens, void *out_v)
{
    const uint8_t *pool = (const uint8_t *)pool_v;
    uint8_t *out = (uint8_t *)out_v;
    int64_t blk_bytes = oracle_block_bytes(fmt, d_c, d_r);
    if (blk_bytes < 0) return -1;
    int64_t row_bytes = blk_bytes / ORACLE_BLOCK;
    for (int b = 0; b < B; ++b) {
        if (seq_lens[b] > max_tokens) return -2;
        for (int p = 0; p < seq_lens[b]; ++p) {
            int64_t blk = bt[(int64_t)b * bt_stride + p / ORACLE_BLOCK];
            int slot = p % ORACLE_BLOCK;
            uint8_t *dst = out + ((int64_t)b * max_tokens + p) * row_bytes;
            const uint8_t *base = pool + blk * blk_bytes;
            if (fmt == ORACLE_FP8_E4M3 || fmt == ORACLE_FP8_E5M2) {
                memcpy(dst, base + (int64_t)slot * d_c, (size_t)d_c);
                memcpy(dst + d_c, base + (int64_t)ORACLE_BLOCK * d_c + (int64_t)slot * d_r * 2,
                       (size_t)d_r * 2);
            } else {
                memcpy(dst, base + slot * row_bytes, (size_t)row_bytes);
            }
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Absorbed decode                                                          */
/* ---------------------------------------------------------------------- */

/*
 * For every query row (b, t, h), with T-major rows r = (b*q_len + t)*n_h + h:
 *
 *   visible cached positions   p in [lo, hi),  hi <= seq_lens[b] - q_len + t + 1
 *     (the query tokens of a sequence are its last q_len positions and each
 *      sees itself and everything before it: speculative multi-token decode,
 *      [vllm] "FlashMLAImpl" reshape for spec decode);
 *   score   s_p = scale * ( q~ . c_p  +  q^R . k^R_p )
 *     (content + RoPE decomposition, [huny] §2-3 score equation; the content
 *      term uses the W^UK-absorbed query q~ against the cached latent,
 *      [huny] §3-1 absorption equation, [donmain] "위치 정보와 압축의 충돌");
 *   weights A_p = exp(s_p) / sum_q exp(s_q)   (softmax, [huny] §3-2);
 *   output  o = sum_p A_p c_p   (latent-space value sum, [huny] §3-2 equation)
 *   lse     = ln sum_p exp(s_p)  (returned with the output, [vllm]
 *             can_return_lse_for_decode).
 *
 * The exponentials are taken relative to the row maximum, which changes no
 * value.  A row with no visible position returns o = 0 and lse = -inf.
 *
 * win_lo / win_hi (optional, per sequence) restrict the cached positions to
 * [win_lo[b], win_hi[b]); they give the per-split partial results.
 * rows (optional) lists the flat row indices to compute (n_rows of them);
 * outputs are then packed in that order.  NULL computes every row.
 * q_lat is [rows_total][d_c], q_rope [rows_total][d_r] (doubles).
 */
int oracle_decode(const void *pool_v, int fmt, const float *blk_scale,
                  const int32_t *bt, int bt_stride, const int32_t *seq_lens,
                  int B, int q_len, int n_h, int d_c, int d_r,
                  const double *q_lat, const double *q_rope, double scale,
                  const int32_t *win_lo, const int32_t *win_hi,
                  const int64_t *rows, int64_t n_rows,
                  double *o_lat, double *lse)
{
    const uint8_t *pool = (const uint8_t *)pool_v;
    if (oracle_block_bytes(fmt, d_c, d_r) < 0) return -1;
    int64_t total = (int64_t)B * q_len * n_h;
    int64_t n_out = rows ? n_rows : total;
    int bad = 0;

#pragma omp parallel
    {
        double *c = (double *)malloc(sizeof(double) * (size_t)(d_c + d_r));
        double *kr = c + d_c;
        double *s = NULL;
        int64_t s_cap = 0;
#pragma omp for schedule(dynamic, 4)
        for (int64_t i = 0; i < n_out; ++i) {
            int64_t r = rows ? rows[i] : i;
            if (r < 0 || r >= total) { bad = 1; continue; }
            int b = (int)(r / ((int64_t)q_len * n_h));
            int t = (int)((r / n_h) % q_len);
            const double *qc = q_lat + r * d_c;
            const double *qr = q_rope + r * d_r;
            double *o = o_lat + i * d_c;
            int lo = win_lo ? win_lo[b] : 0;
            int hi = seq_lens[b] - q_len + t + 1;
            if (win_hi && win_hi[b] < hi) hi = win_hi[b];
            if (lo < 0) lo = 0;
            for (int f = 0; f < d_c; ++f) o[f] = 0.0;
            if (hi <= lo) { lse[i] = -INFINITY; continue; }
            if (hi - lo > s_cap) {
                free(s);
                s_cap = hi - lo;
                s = (double *)malloc(sizeof(double) * (size_t)s_cap);
            }
            /* scores */
            double m = -INFINITY;
            for (int p = lo; p < hi; ++p) {
                load_row(pool, fmt, blk_scale, bt, bt_stride, b, p, d_c, d_r, c, kr);
                double dot = 0.0;
                for (int f = 0; f < d_c; ++f) dot += qc[f] * c[f];
                for (int f = 0; f < d_r; ++f) dot += qr[f] * kr[f];
                s[p - lo] = scale * dot;
                if (s[p - lo] > m) m = s[p - lo];
            }
            /* softmax-weighted sum of the latent rows */
            double l = 0.0;
            for (int p = lo; p < hi; ++p) l += exp(s[p - lo] - m);
            for (int p = lo; p < hi; ++p) {
                load_row(pool, fmt, blk_scale, bt, bt_stride, b, p, d_c, d_r, c, kr);
                double a = exp(s[p - lo] - m) / l;
                for (int f = 0; f < d_c; ++f) o[f] += a * c[f];
            }
            lse[i] = m + log(l);
        }
        free(s);
        free(c);
    }
    return bad ? -3 : 0;
}

/*
 * Merge of per-split results.  If split k covered positions P_k and returned
 * o_k = sum_{P_k} e^{s_p} c_p / sum_{P_k} e^{s_p} and lse_k = ln sum_{P_k} e^{s_p},
 * then over the union: o = sum_k e^{lse_k} o_k / sum_k e^{lse_k} and
 * lse = ln sum_k e^{lse_k}.  (The pages only name the per-sequence split
 * count, [vllm] "FP8 MLA 지원" num_splits; this is the identity it relies on.)
 * o_part is [n_split][rows][d_c], lse_part [n_split][rows].  Splits with
 * lse = -inf carry no weight; if all do, o = 0 and lse = -inf.
 */
int oracle_combine(const double *o_part, const double *lse_part, int n_split,
                   int64_t rows, int d_c, double *o, double *lse)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double m = -INFINITY;
        for (int k = 0; k < n_split; ++k)
            if (lse_part[(int64_t)k * rows + r] > m) m = lse_part[(int64_t)k * rows + r];
        double *dst = o + r * d_c;
        for (int f = 0; f < d_c; ++f) dst[f] = 0.0;
        if (m == -INFINITY) { lse[r] = -INFINITY; continue; }
        double wsum = 0.0;
        for (int k = 0; k < n_split; ++k) {
            double lk = lse_part[(int64_t)k * rows + r];
            if (lk == -INFINITY) continue;
            double w = exp(lk - m);
            wsum += w;
            const double *src = o_part + ((int64_t)k * rows + r) * d_c;
            for (int f = 0; f < d_c; ++f) dst[f] += w * src[f];
        }
        for (int f = 0; f < d_c; ++f) dst[f] /= wsum;
        lse[r] = m + log(wsum);
    }
    return 0;
}
