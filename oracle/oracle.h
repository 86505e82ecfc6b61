/*
 * oracle.h -- C interface of the CPU oracle (test infrastructure only).
 *
 * Layouts (row-major, all host memory):
 *   q_idx [Tq, HI, dI] (FP8 E4M3 codes or fp32), q_scale [Tq], w [Tq, HI]
 *   k_idx [Tk, dI],                               k_scale [Tk]
 *   q [T, Hq, d], k / v [Tk, G, d]  or paged [NB, block_size, G, d]
 *   idx [T, k]  ascending positions, -1 padding
 * Results are double precision.
 */
#ifndef DSA_ORACLE_H
#define DSA_ORACLE_H
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_FP8_E4M3 = 2 };

int64_t oracle_e4m3_to_units(uint8_t code, int* is_nan);
double oracle_e4m3_to_double(uint8_t code);
double oracle_bf16_to_double(uint16_t b);

/* scores[r, s] = I[rows[r], s] for s < Tk; -inf where s > q_pos0 + rows[r]. */
void oracle_index_scores(const void* q_idx, const float* q_scale, const float* w,
                         const void* k_idx, const float* k_scale, int idx_dtype,
                         int Tq, int Tk, int HI, int dI, int64_t q_pos0,
                         const int32_t* rows, int nrows, double* scores);

/* Row r holds candidates 0..pos[r] of scores[r, :].  idx[r, :] gets the
 * min(k, pos[r]+1) selected positions ascending, then -1; kth[r] (nullable)
 * gets the score of the last position in selection order. */
void oracle_topk(const double* scores, int64_t ld, int nrows, const int64_t* pos,
                 int k, int32_t* idx, double* kth);

/* out[r, h, :] = attention of query row rows[r] over idx[rows[r], :]. */
void oracle_sparse_gqa_attn(const void* q, const void* k, const void* v, int dtype,
                            const int32_t* block_table, int max_blocks, int block_size,
                            const int32_t* row_seq, const int32_t* idx, int kk,
                            const int32_t* rows, int nrows, int Hq, int G, int d,
                            double sm_scale, double* out);

/* Full decode step for sequences seqs[0..nseqs): query at position
 * seq_lens[b]-1, FP8 indexer over the paged key cache, top-k, attention. */
void oracle_decode(const void* q, const uint8_t* q_idx, const float* q_scale, const float* w,
                   const uint8_t* kidx_cache, const float* kidx_scale,
                   const void* k_cache, const void* v_cache, int dtype,
                   const int32_t* block_table, const int32_t* seq_lens,
                   int max_blocks, int block_size, int HI, int dI, int Hq, int G, int d,
                   int k, double sm_scale, const int32_t* seqs, int nseqs,
                   int32_t* idx_out, double* kth_out, double* out);

/* Per-token E4M3 quantisation of x [T, n] (ORACLE_F32 or ORACLE_BF16): codes [T, n],
 * scale [T] = amax / 448 (1 for an all-zero row); codes = nearest E4M3 of clamp(x / scale),
 * ties to the even code. */
void oracle_quantize_e4m3(const void* x, int x_dtype, int T, int n, uint8_t* codes, float* scale);

/* ---- training side (oracle_train.c): all arrays of T rows, contiguous K/V [Tk, G, d] ---- */

/* Attention over idx as oracle_sparse_gqa_attn, plus lse[t, h] = ln sum_i exp(logit_i)
 * (-inf for a row without valid entries, whose output is 0). */
void oracle_attn_lse(const void* q, const void* k, const void* v, int dtype, const int32_t* idx,
                     int kk, int T, int Hq, int G, int d, double sm_scale, double* out,
                     double* lse);

/* Gradients of sum dout * out with respect to q [T,Hq,d], k and v [Tk,G,d] (overwritten);
 * dout [T, Hq, d] in `dtype`. */
void oracle_attn_bwd(const void* q, const void* k, const void* v, int dtype, const int32_t* idx,
                     int kk, int T, int Tk, int Hq, int G, int d, double sm_scale,
                     const void* dout, double* dq, double* dk, double* dv);

/* Sparse indexer loss per row, kl[t] = sum_g KL(p[t,:,g] || softmax(vals[t,:])) over the
 * valid entries of idx[t,:] (p = mean attention probability of the group's heads), and
 * dI[t,i] = d kl[t] / d vals[t,i] (0 for padding).  vals [T, kk] = I[t, idx[t,i]]. */
void oracle_indexer_kl(const void* q, const void* k, int dtype, const int32_t* idx, int kk, int T,
                       int Hq, int G, int d, double sm_scale, const double* vals, double* kl,
                       double* dI);

/* Dense warm-up indexer loss (report section 2.3.3; review page, "核心公式", dense warm-up
 * loss): as oracle_indexer_kl with the set of row t the whole causal prefix
 * {0 .. q_pos0 + t} (cut at Tk); scores [T, Tk] = I[t, s]; dI [T, Tk] (0 beyond the prefix). */
void oracle_indexer_warmup_kl(const void* q, const void* k, int dtype, int T, int Tk,
                              int64_t q_pos0, int Hq, int G, int d, double sm_scale,
                              const double* scores, double* kl, double* dI);

/* vals[t, i] = I[t, idx[t, i]] (-inf for padding). */
void oracle_index_scores_at(const void* q_idx, const float* q_scale, const float* w,
                            const void* k_idx, const float* k_scale, int idx_dtype, int T,
                            int HI, int dI, const int32_t* idx, int kk, double* vals);

/* Gradients of sum_{t,i} g[t,i] * I[t, idx[t,i]] with respect to the dequantised q^I
 * [T,HI,dI], w [T,HI] and k^I [Tk,dI] (overwritten). */
void oracle_index_scores_bwd(const void* q_idx, const float* q_scale, const float* w,
                             const void* k_idx, const float* k_scale, int idx_dtype, int T,
                             int Tk, int HI, int dI, const int32_t* idx, int kk, const double* g,
                             double* dq_idx, double* dw, double* dk_idx);

/* The same for a dense g [T, Tk]: row t takes g[t, s] for s <= q_pos0 + t only. */
void oracle_index_scores_bwd_dense(const void* q_idx, const float* q_scale, const float* w,
                                   const void* k_idx, const float* k_scale, int idx_dtype, int T,
                                   int Tk, int HI, int dI, int64_t q_pos0, const double* g,
                                   double* dq_idx, double* dw, double* dk_idx);

int oracle_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
