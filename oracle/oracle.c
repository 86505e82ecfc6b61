/*
 * oracle.c -- plain, slow, CPU-only oracle for the DSA layer.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load this library.  It shares no code,
 * header, table or helper with the GPU library and must never be used on
 * the product path.
 *
 * What it computes (Kwai Keye-VL-2.0 technical report, as summarised on the
 * xllm-io review page, section "核心公式"; and the report's section 2.3,
 * "DSA for long-context multimodal modelling"):
 *
 *   (1) lightning indexer   I[t,s] = sum_j w[t,j] * ReLU(q^I[t,j] . k^I[s])
 *                           for every causal pair s <= t (section 2.3.1:
 *                           the indexer scores the current query against
 *                           every previous token; one key head shared by
 *                           all indexer heads, MQA style)
 *   (2) top-k index set     Omega_t = { s : I[t,s] in Top-k(I[t,:]) }
 *                           (k = 2048 in the report; a parameter here)
 *   (3) GQA sparse          u[t,g] = Attn(h[t,g], { c[s,g] : s in Omega_t })
 *       aggregation         with the same Omega_t for every KV group
 *                           (section 2.3.2), outputs concatenated over g.
 *
 * Arithmetic: every floating-point step is done in double.  FP8 (OCP E4M3)
 * codes are decoded to exact integers n with value n * 2^-9, so an indexer
 * dot product of two FP8 vectors is an exact int64 sum; the per-token fp32
 * scales are applied afterwards in double.
 *
 * Readings of points the pages leave open (each listed in the design notes):
 *  - s = t is a candidate (positions 0..t), so |Omega_t| = min(k, t+1).
 *  - no extra constant inside I (the formula has none).
 *  - dequantised indexer vectors are q_scale[t]*fp8(q) and k_scale[s]*fp8(k).
 *  - Top-k ties go to the lower position; -0 and +0 compare equal.
 *  - Omega_t is reported in ascending position order, padded with -1.
 *  - Attn is plain softmax attention, logits scaled by sm_scale, no bias.
 *  - query head h belongs to KV group h / (Hq / G).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- decoding */

/* OCP 8-bit floating point, E4M3 variant: 1 sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits, subnormals when the exponent field is 0, no
 * infinities, and S.1111.111 is NaN (so the largest finite value is
 * 1.75 * 2^8 = 448).  Returns the value as an integer multiple of 2^-9:
 *   exponent field 0:  value = m * 2^-3 * 2^(1-7)        = m * 2^-9
 *   exponent field e:  value = (8+m) * 2^-3 * 2^(e-7)    = ((8+m) << (e-1)) * 2^-9
 * *is_nan is set for the two NaN codes. */
int64_t oracle_e4m3_to_units(uint8_t code, int* is_nan)
{
    int sign = code >> 7;
    int e = (code >> 3) & 15;
    int m = code & 7;
    int64_t n;
    *is_nan = (e == 15 && m == 7);
    if (*is_nan) return 0;
    if (e == 0) n = m;
    else n = (int64_t)(8 + m) << (e - 1);
    return sign ? -n : n;
}

double oracle_e4m3_to_double(uint8_t code)
{
    int nan;
    int64_t n = oracle_e4m3_to_units(code, &nan);
    if (nan) return NAN;
    if (n == 0 && (code >> 7)) return -0.0;
    return ldexp((double)n, -9);
}

/* bfloat16 is the upper half of an IEEE binary32 pattern. */
static double bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double oracle_bf16_to_double(uint16_t b) { return bf16_to_double(b); }

/* element i of a q / k / v array stored in `dtype` (0 = fp32, 1 = bf16) */
static double load_elem(const void* base, int dtype, int64_t i)
{
    if (dtype == ORACLE_F32) return (double)((const float*)base)[i];
    return bf16_to_double(((const uint16_t*)base)[i]);
}

/* ------------------------------------------------------- lightning indexer */

/* Decode n codes into integer units of 2^-9; returns nonzero if any is NaN. */
static int decode_codes(const uint8_t* codes, int64_t n, int64_t* units)
{
    int any_nan = 0;
    for (int64_t i = 0; i < n; ++i) {
        int nan;
        units[i] = oracle_e4m3_to_units(codes[i], &nan);
        any_nan |= nan;
    }
    return any_nan;
}

/* One score I[t,s] for FP8 inputs, given the decoded codes of token t's
 * H^I query vectors (qn, H^I*d_I units) and of token s's key (kn, d_I units). */
static double score_fp8(const int64_t* qn, double qscale, const float* wrow,
                        const int64_t* kn, double kscale, int HI, int dI)
{
    double acc = 0.0;
    for (int j = 0; j < HI; ++j) {
        int64_t dot = 0;
        for (int i = 0; i < dI; ++i)
            dot += qn[(int64_t)j * dI + i] * kn[i];          /* exact: |a*b| < 2^36 */
        /* q^I[t,j] . k^I[s] with both vectors dequantised:
         * (qscale * a * 2^-9) . (kscale * b * 2^-9) */
        double x = qscale * kscale * ldexp((double)dot, -18);
        double relu = x > 0.0 ? x : 0.0;
        acc += (double)wrow[j] * relu;
    }
    return acc;
}

/* One score I[t,s] for fp32 inputs (no scales). */
static double score_f32(const float* qrow, const float* wrow, const float* krow,
                        int HI, int dI)
{
    double acc = 0.0;
    for (int j = 0; j < HI; ++j) {
        double dot = 0.0;
        for (int i = 0; i < dI; ++i)
            dot += (double)qrow[(int64_t)j * dI + i] * (double)krow[i];
        double relu = dot > 0.0 ? dot : 0.0;
        acc += (double)wrow[j] * relu;
    }
    return acc;
}

void oracle_index_scores(const void* q_idx, const float* q_scale, const float* w,
                         const void* k_idx, const float* k_scale, int idx_dtype,
                         int Tq, int Tk, int HI, int dI, int64_t q_pos0,
                         const int32_t* rows, int nrows, double* scores)
{
    (void)Tq;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nrows; ++r) {
        int t = rows[r];                       /* query row, position q_pos0 + t */
        int64_t pos = q_pos0 + t;
        double* out = scores + (int64_t)r * Tk;
        int64_t* qn = (int64_t*)malloc((size_t)HI * dI * sizeof(int64_t));
        int64_t* kn = (int64_t*)malloc((size_t)dI * sizeof(int64_t));
        int q_nan = 0;
        if (idx_dtype == ORACLE_FP8_E4M3)
            q_nan = decode_codes((const uint8_t*)q_idx + (int64_t)t * HI * dI, (int64_t)HI * dI, qn);
        for (int64_t s = 0; s < Tk; ++s) {
            if (s > pos) { out[s] = -INFINITY; continue; }
            if (idx_dtype == ORACLE_FP8_E4M3) {
                int k_nan = decode_codes((const uint8_t*)k_idx + s * dI, dI, kn);
                out[s] = (q_nan || k_nan) ? NAN
                       : score_fp8(qn, q_scale[t], w + (int64_t)t * HI, kn, k_scale[s], HI, dI);
            } else {
                const float* q = (const float*)q_idx + (int64_t)t * HI * dI;
                const float* k = (const float*)k_idx + s * dI;
                out[s] = score_f32(q, w + (int64_t)t * HI, k, HI, dI);
            }
        }
        free(qn);
        free(kn);
    }
}

/* ------------------------------------------------------------------- top-k */

typedef struct { double score; int64_t pos; } cand_t;

/* larger score first; among equal scores the lower position first.
 * -0.0 == +0.0 under C comparison, so the two zeros tie. */
static int cmp_cand(const void* a, const void* b)
{
    const cand_t* x = (const cand_t*)a;
    const cand_t* y = (const cand_t*)b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    return (x->pos < y->pos) ? -1 : (x->pos > y->pos);
}

static int cmp_i32(const void* a, const void* b)
{
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

void oracle_topk(const double* scores, int64_t ld, int nrows, const int64_t* pos,
                 int k, int32_t* idx, double* kth)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nrows; ++r) {
        int64_t n_cand = pos[r] + 1;             /* candidates 0..pos */
        int64_t n = n_cand < k ? n_cand : k;
        int32_t* out = idx + (int64_t)r * k;
        if (n_cand <= 0) {                       /* no candidate at all */
            for (int i = 0; i < k; ++i) out[i] = -1;
            if (kth) kth[r] = NAN;
            continue;
        }
        cand_t* c = (cand_t*)malloc((size_t)n_cand * sizeof(cand_t));
        for (int64_t s = 0; s < n_cand; ++s) {
            c[s].score = scores[(int64_t)r * ld + s];
            c[s].pos = s;
        }
        qsort(c, (size_t)n_cand, sizeof(cand_t), cmp_cand);
        for (int64_t i = 0; i < n; ++i) out[i] = (int32_t)c[i].pos;
        qsort(out, (size_t)n, sizeof(int32_t), cmp_i32);
        for (int64_t i = n; i < k; ++i) out[i] = -1;
        if (kth) kth[r] = c[n - 1].score;
        free(c);
    }
}

/* --------------------------------------------------------------- attention */

/* Softmax attention of query row t over the positions listed in sel[0..k),
 * entries < 0 skipped.  The K/V row of logical position s for the sequence
 * `seq` is found through `kv_row` (contiguous, or through a block table). */
typedef struct {
    const int32_t* block_table;   /* NULL: contiguous */
    int max_blocks;
    int block_size;
} kv_map_t;

static int64_t kv_row(const kv_map_t* m, int seq, int64_t s)
{
    if (!m->block_table) return s;
    int64_t blk = m->block_table[(int64_t)seq * m->max_blocks + s / m->block_size];
    return blk * m->block_size + s % m->block_size;
}

static void attend_row(const void* q, const void* k, const void* v, int dtype,
                       const kv_map_t* map, int seq, const int32_t* sel, int kk,
                       int64_t t, int Hq, int G, int d, double sm_scale, double* out)
{
    int heads_per_group = Hq / G;
    double* logit = (double*)malloc((size_t)(kk > 0 ? kk : 1) * sizeof(double));
    for (int h = 0; h < Hq; ++h) {
        int g = h / heads_per_group;
        int64_t qoff = (t * Hq + h) * (int64_t)d;
        double m = -INFINITY;
        int used = 0;
        for (int i = 0; i < kk; ++i) {
            if (sel[i] < 0) continue;
            int64_t row = kv_row(map, seq, sel[i]);
            int64_t koff = (row * G + g) * (int64_t)d;
            double dot = 0.0;
            for (int e = 0; e < d; ++e)
                dot += load_elem(q, dtype, qoff + e) * load_elem(k, dtype, koff + e);
            logit[i] = sm_scale * dot;
            if (logit[i] > m) m = logit[i];
            ++used;
        }
        double* o = out + (int64_t)h * d;
        for (int e = 0; e < d; ++e) o[e] = 0.0;
        if (!used) continue;                      /* empty set: output 0 */
        double denom = 0.0;
        for (int i = 0; i < kk; ++i) {
            if (sel[i] < 0) continue;
            double p = exp(logit[i] - m);
            denom += p;
            int64_t row = kv_row(map, seq, sel[i]);
            int64_t voff = (row * G + g) * (int64_t)d;
            for (int e = 0; e < d; ++e) o[e] += p * load_elem(v, dtype, voff + e);
        }
        for (int e = 0; e < d; ++e) o[e] /= denom;
    }
    free(logit);
}

void oracle_sparse_gqa_attn(const void* q, const void* k, const void* v, int dtype,
                            const int32_t* block_table, int max_blocks, int block_size,
                            const int32_t* row_seq, const int32_t* idx, int kk,
                            const int32_t* rows, int nrows, int Hq, int G, int d,
                            double sm_scale, double* out)
{
    kv_map_t map = { block_table, max_blocks, block_size };
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nrows; ++r) {
        int t = rows[r];
        int seq = row_seq ? row_seq[t] : 0;
        attend_row(q, k, v, dtype, &map, seq, idx + (int64_t)t * kk, kk, t, Hq, G, d,
                   sm_scale, out + (int64_t)r * Hq * d);
    }
}

/* ------------------------------------------------------------ paged decode */

void oracle_decode(const void* q, const uint8_t* q_idx, const float* q_scale, const float* w,
                   const uint8_t* kidx_cache, const float* kidx_scale,
                   const void* k_cache, const void* v_cache, int dtype,
                   const int32_t* block_table, const int32_t* seq_lens,
                   int max_blocks, int block_size, int HI, int dI, int Hq, int G, int d,
                   int k, double sm_scale, const int32_t* seqs, int nseqs,
                   int32_t* idx_out, double* kth_out, double* out)
{
    kv_map_t map = { block_table, max_blocks, block_size };
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nseqs; ++r) {
        int b = seqs[r];
        int64_t len = seq_lens[b];
        int64_t pos = len - 1;                    /* the new token's own entries are cached */
        double* sc = (double*)malloc((size_t)len * sizeof(double));
        int64_t* qn = (int64_t*)malloc((size_t)HI * dI * sizeof(int64_t));
        int64_t* kn = (int64_t*)malloc((size_t)dI * sizeof(int64_t));
        int q_nan = decode_codes(q_idx + (int64_t)b * HI * dI, (int64_t)HI * dI, qn);
        for (int64_t s = 0; s < len; ++s) {
            int64_t row = kv_row(&map, b, s);
            int k_nan = decode_codes(kidx_cache + row * dI, dI, kn);
            sc[s] = (q_nan || k_nan) ? NAN
                  : score_fp8(qn, q_scale[b], w + (int64_t)b * HI, kn, kidx_scale[row], HI, dI);
        }
        free(qn);
        free(kn);
        int32_t* sel = idx_out + (int64_t)r * k;
        double kth;
        /* one row at a time: the outer loop already runs in parallel */
        {
            int64_t n_cand = pos + 1;
            int64_t n = n_cand < k ? n_cand : k;
            cand_t* c = (cand_t*)malloc((size_t)n_cand * sizeof(cand_t));
            for (int64_t s = 0; s < n_cand; ++s) { c[s].score = sc[s]; c[s].pos = s; }
            qsort(c, (size_t)n_cand, sizeof(cand_t), cmp_cand);
            for (int64_t i = 0; i < n; ++i) sel[i] = (int32_t)c[i].pos;
            qsort(sel, (size_t)n, sizeof(int32_t), cmp_i32);
            for (int64_t i = n; i < k; ++i) sel[i] = -1;
            kth = c[n - 1].score;
            free(c);
        }
        if (kth_out) kth_out[r] = kth;
        attend_row(q, k_cache, v_cache, dtype, &map, b, sel, k, b, Hq, G, d, sm_scale,
                   out + (int64_t)r * Hq * d);
        free(sc);
    }
}

/* ------------------------------------------------------- FP8 quantisation */

/* The indexer runs on FP8 inputs (Keye-VL-2.0 report, section 2.3.1; the
 * xllm-io review credits FP8 for the indexer's efficiency).  The pages give no
 * recipe; the reading used throughout is per-token absmax scaling into OCP
 * E4M3: scale = amax / 448 over the token's values (1 when amax = 0), each
 * value divided by the scale in fp32, clamped to [-448, 448], and rounded to
 * the nearest E4M3 value with ties to the even code.  The rounding here is the
 * plain definition: the nearest of the 127 non-negative finite E4M3 values by
 * exhaustive search. */
static uint8_t e4m3_nearest(float v)
{
    const int neg = signbit(v) != 0;
    const double a = fabs((double)v);
    int best = 0;
    double best_d = INFINITY;
    for (int c = 0; c < 127; ++c) {                    /* 0x00 .. 0x7E, ascending values */
        const double d = fabs(oracle_e4m3_to_double((uint8_t)c) - a);
        if (d < best_d || (d == best_d && (c & 1) == 0)) { best = c; best_d = d; }
    }
    return (uint8_t)(best | (neg ? 0x80 : 0));
}

void oracle_quantize_e4m3(const void* x, int x_dtype, int T, int n, uint8_t* codes, float* scale)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        float amax = 0.f;
        for (int i = 0; i < n; ++i) {
            const int64_t o = (int64_t)t * n + i;
            const float v = x_dtype == ORACLE_BF16 ? (float)bf16_to_double(((const uint16_t*)x)[o])
                                                   : ((const float*)x)[o];
            if (fabsf(v) > amax) amax = fabsf(v);
        }
        const float s = amax > 0.f ? amax / 448.0f : 1.0f;
        scale[t] = s;
        for (int i = 0; i < n; ++i) {
            const int64_t o = (int64_t)t * n + i;
            const float v = x_dtype == ORACLE_BF16 ? (float)bf16_to_double(((const uint16_t*)x)[o])
                                                   : ((const float*)x)[o];
            float y = v / s;
            if (y > 448.0f) y = 448.0f;
            if (y < -448.0f) y = -448.0f;
            codes[o] = e4m3_nearest(y);
        }
    }
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
#else
    return 1;
#endif
}
