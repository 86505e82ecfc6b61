/*
 * oracle_train.c -- plain CPU oracle for the training side of the DSA layer:
 * the backward of the sparse GQA attention and the sparse indexer loss.
 *
 * TEST INFRASTRUCTURE, like oracle.c: only the test suite, the smoke check and
 * the CPU baseline leg of the benchmark load this library; it shares nothing
 * with the GPU library.
 *
 * What it computes:
 *  - the attention of oracle.c (Keye-VL-2.0 report section 2.3.2; xllm-io
 *    review page, section "核心公式", third formula) with its log-sum-exp, and
 *    the gradients of that attention with respect to q, K and V, written out
 *    from the definition of softmax attention: for one query head,
 *      P_i = exp(l_i - lse),  l_i = sm_scale * q . K[s_i],
 *      dP_i = dout . V[s_i],  dl_i = P_i * (dP_i - sum_j P_j dP_j),
 *      dq = sm_scale sum_i dl_i K[s_i],  dK[s_i] += sm_scale dl_i q,
 *      dV[s_i] += P_i dout;
 *  - the sparse indexer loss of the report's section 2.3.3 (review page,
 *    "核心公式", sparse adaptation loss): for query t and KV group g the target
 *    p[t,:,g] aggregates the attention of the group's query heads (their mean,
 *    which already sums to 1 over Omega_t, so truncating to the selected set
 *    and renormalising changes nothing), and
 *      L[t] = sum_g KL( p[t,Omega_t,g] || softmax(I[t,Omega_t]) ),
 *    whose gradient with respect to I[t,s], s in Omega_t, is
 *      sum_g ( softmax(I[t,Omega_t])_s - p[t,s,g] );
 *    the target is a constant (the report detaches the indexer's inputs from
 *    the main model, so the loss trains the indexer only);
 *  - the dense warm-up loss of the same section (review page, "核心公式", dense
 *    warm-up loss): the same divergence with the set of row t the whole causal
 *    prefix, so it follows the sparse one with that set;
 *  - the indexer scores at the selected positions and the gradient of
 *    sum_{t,i} g[t,i] I[t, Omega_t[i]] (or, for the warm-up loss, of
 *    sum_{t, s <= pos} g[t,s] I[t,s]) with respect to the dequantised
 *    indexer inputs q^I, w and k^I (FP8 rounding taken as the identity;
 *    ReLU'(0) = 0).
 * Every step is in double; -1 entries of an index list are skipped.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static double elem(const void* base, int dtype, int64_t i)
{
    if (dtype == ORACLE_F32) return (double)((const float*)base)[i];
    return oracle_bf16_to_double(((const uint16_t*)base)[i]);
}

/* Softmax probabilities of one query head over its index list (P[i] = 0 for padding);
 * returns the log-sum-exp of the logits, -inf if the list has no valid entry. */
static double head_probs(const void* q, const void* k, int dtype, const int32_t* sel, int kk,
                         int64_t t, int h, int g, int Hq, int G, int d, double sm_scale,
                         double* P)
{
    double m = -INFINITY;
    for (int i = 0; i < kk; ++i) {
        P[i] = -INFINITY;
        if (sel[i] < 0) continue;
        double dot = 0.0;
        for (int e = 0; e < d; ++e)
            dot += elem(q, dtype, (t * Hq + h) * (int64_t)d + e) *
                   elem(k, dtype, ((int64_t)sel[i] * G + g) * d + e);
        P[i] = sm_scale * dot;
        if (P[i] > m) m = P[i];
    }
    if (m == -INFINITY) {
        for (int i = 0; i < kk; ++i) P[i] = 0.0;
        return -INFINITY;
    }
    double sum = 0.0;
    for (int i = 0; i < kk; ++i) sum += sel[i] < 0 ? 0.0 : exp(P[i] - m);
    double lse = m + log(sum);
    for (int i = 0; i < kk; ++i) P[i] = sel[i] < 0 ? 0.0 : exp(P[i] - lse);
    return lse;
}

void oracle_attn_lse(const void* q, const void* k, const void* v, int dtype, const int32_t* idx,
                     int kk, int T, int Hq, int G, int d, double sm_scale, double* out,
                     double* lse)
{
    int hpg = Hq / G;
#pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < T; ++t) {
        double* P = (double*)malloc((size_t)(kk > 0 ? kk : 1) * sizeof(double));
        const int32_t* sel = idx + (int64_t)t * kk;
        for (int h = 0; h < Hq; ++h) {
            int g = h / hpg;
            lse[(int64_t)t * Hq + h] = head_probs(q, k, dtype, sel, kk, t, h, g, Hq, G, d,
                                                  sm_scale, P);
            double* o = out + ((int64_t)t * Hq + h) * d;
            for (int e = 0; e < d; ++e) {
                double acc = 0.0;
                for (int i = 0; i < kk; ++i)
                    if (sel[i] >= 0) acc += P[i] * elem(v, dtype, ((int64_t)sel[i] * G + g) * d + e);
                o[e] = acc;
            }
        }
        free(P);
    }
}

/* dl[i] for one head: P_i (dP_i - sum_j P_j dP_j), dP_i = dout . V[s_i]. */
static void head_dlogits(const void* v, const void* dout, int dtype, const int32_t* sel, int kk,
                         int64_t t, int h, int g, int Hq, int G, int d, const double* P,
                         double* dl)
{
    double D = 0.0;
    for (int i = 0; i < kk; ++i) {
        dl[i] = 0.0;
        if (sel[i] < 0) continue;
        double dp = 0.0;
        for (int e = 0; e < d; ++e)
            dp += elem(dout, dtype, (t * Hq + h) * (int64_t)d + e) *
                  elem(v, dtype, ((int64_t)sel[i] * G + g) * d + e);
        dl[i] = dp;
        D += P[i] * dp;
    }
    for (int i = 0; i < kk; ++i) dl[i] = sel[i] < 0 ? 0.0 : P[i] * (dl[i] - D);
}

void oracle_attn_bwd(const void* q, const void* k, const void* v, int dtype, const int32_t* idx,
                     int kk, int T, int Tk, int Hq, int G, int d, double sm_scale,
                     const void* dout, double* dq, double* dk, double* dv)
{
    int hpg = Hq / G;
    memset(dk, 0, (size_t)Tk * G * d * sizeof(double));
    memset(dv, 0, (size_t)Tk * G * d * sizeof(double));
    /* the groups touch disjoint parts of dK and dV, so they run in parallel */
#pragma omp parallel for schedule(static, 1)
    for (int g = 0; g < G; ++g) {
        double* P = (double*)malloc((size_t)(kk > 0 ? kk : 1) * sizeof(double));
        double* dl = (double*)malloc((size_t)(kk > 0 ? kk : 1) * sizeof(double));
        for (int t = 0; t < T; ++t) {
            const int32_t* sel = idx + (int64_t)t * kk;
            for (int h = g * hpg; h < (g + 1) * hpg; ++h) {
                head_probs(q, k, dtype, sel, kk, t, h, g, Hq, G, d, sm_scale, P);
                head_dlogits(v, dout, dtype, sel, kk, t, h, g, Hq, G, d, P, dl);
                double* dqh = dq + ((int64_t)t * Hq + h) * d;
                for (int e = 0; e < d; ++e) dqh[e] = 0.0;
                for (int i = 0; i < kk; ++i) {
                    if (sel[i] < 0) continue;
                    int64_t kv = ((int64_t)sel[i] * G + g) * d;
                    for (int e = 0; e < d; ++e) {
                        dqh[e] += sm_scale * dl[i] * elem(k, dtype, kv + e);
                        dk[kv + e] += sm_scale * dl[i] * elem(q, dtype, (t * Hq + h) * (int64_t)d + e);
                        dv[kv + e] += P[i] * elem(dout, dtype, (t * Hq + h) * (int64_t)d + e);
                    }
                }
            }
        }
        free(P);
        free(dl);
    }
}

/* The loss of one row over the index list sel[0 .. kk) (entries -1 skipped) and its gradient
 * with respect to the scores I[0 .. kk) of those entries; P, p, qI are scratch of kk doubles. */
static double row_kl(const void* q, const void* k, int dtype, const int32_t* sel, int kk, int t,
                     int Hq, int G, int d, double sm_scale, const double* I, double* dI, double* P,
                     double* p, double* qI)
{
    int hpg = Hq / G;
    /* the indexer's distribution over the set; qI holds its logarithm I - logsumexp(I), which
     * stays finite where exp underflows */
    double m = -INFINITY, z = 0.0;
    for (int i = 0; i < kk; ++i) if (sel[i] >= 0 && I[i] > m) m = I[i];
    for (int i = 0; i < kk; ++i) z += sel[i] >= 0 ? exp(I[i] - m) : 0.0;
    double lz = m + log(z);
    for (int i = 0; i < kk; ++i) qI[i] = sel[i] >= 0 ? I[i] - lz : 0.0;
    double loss = 0.0;
    for (int i = 0; i < kk; ++i) dI[i] = 0.0;
    for (int g = 0; g < G; ++g) {
        for (int i = 0; i < kk; ++i) p[i] = 0.0;
        for (int h = g * hpg; h < (g + 1) * hpg; ++h) {
            head_probs(q, k, dtype, sel, kk, t, h, g, Hq, G, d, sm_scale, P);
            for (int i = 0; i < kk; ++i) p[i] += P[i] / hpg;
        }
        for (int i = 0; i < kk; ++i) {
            if (sel[i] < 0) continue;
            if (p[i] > 0.0) loss += p[i] * (log(p[i]) - qI[i]);
            dI[i] += exp(qI[i]) - p[i];
        }
    }
    return loss;
}

void oracle_indexer_kl(const void* q, const void* k, int dtype, const int32_t* idx, int kk, int T,
                       int Hq, int G, int d, double sm_scale, const double* vals, double* kl,
                       double* dI)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < T; ++t) {
        size_t n = (size_t)(kk > 0 ? kk : 1) * sizeof(double);
        double* P = (double*)malloc(n);
        double* p = (double*)malloc(n);
        double* qI = (double*)malloc(n);
        kl[t] = row_kl(q, k, dtype, idx + (int64_t)t * kk, kk, t, Hq, G, d, sm_scale,
                       vals + (int64_t)t * kk, dI + (int64_t)t * kk, P, p, qI);
        free(P);
        free(p);
        free(qI);
    }
}

/* The dense warm-up loss is the same divergence taken over every key of the causal prefix:
 * row t sits at position q_pos0 + t and its set is {0, 1, .., q_pos0 + t} (cut at Tk). */
void oracle_indexer_warmup_kl(const void* q, const void* k, int dtype, int T, int Tk,
                              int64_t q_pos0, int Hq, int G, int d, double sm_scale,
                              const double* scores, double* kl, double* dI)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < T; ++t) {
        int64_t pos = q_pos0 + t;
        int n = (int)(pos + 1 < Tk ? pos + 1 : Tk);
        size_t bytes = (size_t)(n > 0 ? n : 1) * sizeof(double);
        int32_t* sel = (int32_t*)malloc((size_t)(n > 0 ? n : 1) * sizeof(int32_t));
        double* P = (double*)malloc(bytes);
        double* p = (double*)malloc(bytes);
        double* qI = (double*)malloc(bytes);
        for (int s = 0; s < n; ++s) sel[s] = s;
        double* drow = dI + (int64_t)t * Tk;
        kl[t] = row_kl(q, k, dtype, sel, n, t, Hq, G, d, sm_scale, scores + (int64_t)t * Tk, drow,
                       P, p, qI);
        for (int s = n; s < Tk; ++s) drow[s] = 0.0;
        free(sel);
        free(P);
        free(p);
        free(qI);
    }
}

/* dequantised indexer query (HI x dI) of row t and key of position s */
static void deq_query(const void* q_idx, const float* q_scale, int idx_dtype, int64_t t, int HI,
                      int dI, double* out)
{
    int64_t n = (int64_t)HI * dI;
    for (int64_t i = 0; i < n; ++i)
        out[i] = idx_dtype == ORACLE_FP8_E4M3
                     ? q_scale[t] * oracle_e4m3_to_double(((const uint8_t*)q_idx)[t * n + i])
                     : (double)((const float*)q_idx)[t * n + i];
}

static void deq_key(const void* k_idx, const float* k_scale, int idx_dtype, int64_t s, int dI,
                    double* out)
{
    for (int i = 0; i < dI; ++i)
        out[i] = idx_dtype == ORACLE_FP8_E4M3
                     ? k_scale[s] * oracle_e4m3_to_double(((const uint8_t*)k_idx)[s * dI + i])
                     : (double)((const float*)k_idx)[s * dI + i];
}

/* x = q^I[t,j] . k^I[s] of the dequantised vectors.  For FP8 the dot product of the codes
 * is taken exactly in integer units of 2^-9 (as in the forward oracle), so a product that is
 * exactly zero stays zero and the ReLU decision is exact. */
static double indexer_dot(const void* q_idx, const float* q_scale, const void* k_idx,
                          const float* k_scale, int idx_dtype, int64_t t, int j, int64_t s, int HI,
                          int dI)
{
    if (idx_dtype == ORACLE_FP8_E4M3) {
        const uint8_t* qc = (const uint8_t*)q_idx + (t * HI + j) * (int64_t)dI;
        const uint8_t* kc = (const uint8_t*)k_idx + s * dI;
        int64_t dot = 0;
        int nan;
        for (int e = 0; e < dI; ++e)
            dot += oracle_e4m3_to_units(qc[e], &nan) * oracle_e4m3_to_units(kc[e], &nan);
        return (double)q_scale[t] * (double)k_scale[s] * ldexp((double)dot, -18);
    }
    const float* q = (const float*)q_idx + (t * HI + j) * (int64_t)dI;
    const float* k = (const float*)k_idx + s * dI;
    double dot = 0.0;
    for (int e = 0; e < dI; ++e) dot += (double)q[e] * (double)k[e];
    return dot;
}

void oracle_index_scores_at(const void* q_idx, const float* q_scale, const float* w,
                            const void* k_idx, const float* k_scale, int idx_dtype, int T,
                            int HI, int dI, const int32_t* idx, int kk, double* vals)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < T; ++t) {
        for (int i = 0; i < kk; ++i) {
            int s = idx[(int64_t)t * kk + i];
            if (s < 0) { vals[(int64_t)t * kk + i] = -INFINITY; continue; }
            double acc = 0.0;
            for (int j = 0; j < HI; ++j) {
                double x = indexer_dot(q_idx, q_scale, k_idx, k_scale, idx_dtype, t, j, s, HI, dI);
                acc += (double)w[(int64_t)t * HI + j] * (x > 0.0 ? x : 0.0);
            }
            vals[(int64_t)t * kk + i] = acc;
        }
    }
}

/* Adds the gradients of gi * I[t,s] to dq (row t's HI x dI block), dw (row t's HI entries)
 * and dk_idx; qv is row t's dequantised query, kv scratch of dI doubles. */
static void add_score_grads(const void* q_idx, const float* q_scale, const float* w,
                            const void* k_idx, const float* k_scale, int idx_dtype, int64_t t,
                            int64_t s, double gi, int HI, int dI, const double* qv, double* kv,
                            double* dq, double* dw, double* dk_idx)
{
    deq_key(k_idx, k_scale, idx_dtype, s, dI, kv);
    for (int j = 0; j < HI; ++j) {
        double x = indexer_dot(q_idx, q_scale, k_idx, k_scale, idx_dtype, t, j, s, HI, dI);
        if (x <= 0.0) continue;               /* ReLU'(x) = 0 for x <= 0 */
        double wj = (double)w[t * HI + j];
        dw[j] += gi * x;
        for (int e = 0; e < dI; ++e) {
            dq[(int64_t)j * dI + e] += gi * wj * kv[e];
            dk_idx[s * dI + e] += gi * wj * qv[(int64_t)j * dI + e];
        }
    }
}

void oracle_index_scores_bwd(const void* q_idx, const float* q_scale, const float* w,
                             const void* k_idx, const float* k_scale, int idx_dtype, int T,
                             int Tk, int HI, int dI, const int32_t* idx, int kk, const double* g,
                             double* dq_idx, double* dw, double* dk_idx)
{
    memset(dk_idx, 0, (size_t)Tk * dI * sizeof(double));
    double* qv = (double*)malloc((size_t)HI * dI * sizeof(double));
    double* kv = (double*)malloc((size_t)dI * sizeof(double));
    for (int t = 0; t < T; ++t) {
        deq_query(q_idx, q_scale, idx_dtype, t, HI, dI, qv);
        double* dq = dq_idx + (int64_t)t * HI * dI;
        memset(dq, 0, (size_t)HI * dI * sizeof(double));
        for (int j = 0; j < HI; ++j) dw[(int64_t)t * HI + j] = 0.0;
        for (int i = 0; i < kk; ++i) {
            int s = idx[(int64_t)t * kk + i];
            if (s < 0) continue;
            add_score_grads(q_idx, q_scale, w, k_idx, k_scale, idx_dtype, t, s,
                            g[(int64_t)t * kk + i], HI, dI, qv, kv, dq, dw + (int64_t)t * HI,
                            dk_idx);
        }
    }
    free(qv);
    free(kv);
}

/* The same gradients for a dense g [T, Tk] over the causal prefix: row t (position
 * q_pos0 + t) takes g[t, s] for every s <= q_pos0 + t; the entries beyond are ignored. */
void oracle_index_scores_bwd_dense(const void* q_idx, const float* q_scale, const float* w,
                                   const void* k_idx, const float* k_scale, int idx_dtype, int T,
                                   int Tk, int HI, int dI, int64_t q_pos0, const double* g,
                                   double* dq_idx, double* dw, double* dk_idx)
{
    memset(dk_idx, 0, (size_t)Tk * dI * sizeof(double));
    double* qv = (double*)malloc((size_t)HI * dI * sizeof(double));
    double* kv = (double*)malloc((size_t)dI * sizeof(double));
    for (int t = 0; t < T; ++t) {
        deq_query(q_idx, q_scale, idx_dtype, t, HI, dI, qv);
        double* dq = dq_idx + (int64_t)t * HI * dI;
        memset(dq, 0, (size_t)HI * dI * sizeof(double));
        for (int j = 0; j < HI; ++j) dw[(int64_t)t * HI + j] = 0.0;
        int64_t last = q_pos0 + t < Tk - 1 ? q_pos0 + t : Tk - 1;
        for (int64_t s = 0; s <= last; ++s)
            add_score_grads(q_idx, q_scale, w, k_idx, k_scale, idx_dtype, t, s,
                            g[(int64_t)t * Tk + s], HI, dI, qv, kv, dq, dw + (int64_t)t * HI,
                            dk_idx);
    }
    free(qv);
    free(kv);
}
