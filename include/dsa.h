/*
 * dsa.h -- C interface of libdsa, the DeepSeek Sparse Attention (DSA) layer in
 * the GQA form of the Kwai Keye-VL-2.0 report, for AMD MI355X (gfx950).
 *
 * The layer (report section 2.3; xllm-io review page, section "核心公式"):
 *   1. lightning indexer   I[t,s] = sum_j w[t,j] * ReLU(q^I[t,j] . k^I[s])  for s <= t,
 *      one FP8 key vector per token shared by all H^I indexer heads (MQA style);
 *   2. top-k               Omega_t = the min(k, t+1) positions with the largest I[t,:];
 *   3. GQA sparse attention u[t,g] = softmax attention of token t's query heads in
 *      group g over { (K[s,g], V[s,g]) : s in Omega_t }, the same Omega_t for
 *      every group; outputs concatenated over groups.
 *
 * Conventions common to every call
 *  - Every pointer argument is DEVICE memory owned by the caller, unless noted.
 *    The library keeps no pointer after a call returns, allocates nothing and
 *    never synchronises: work is queued on `stream` and its results are ready
 *    when the stream reaches that point.
 *  - Arrays are dense row-major with the shapes given in brackets.  Arrays of
 *    vectors (q, k, v, out, indexer codes, w, scores, workspace) must be
 *    16-byte aligned; per-token scales, index lists, block tables and
 *    sequence lengths need only 4-byte alignment.
 *  - Positions are absolute and 0-based; the causal rule is s <= position, so
 *    the token itself is a candidate.
 *  - Query head h belongs to KV group h / (Hq / G).
 *  - FP8 means OCP E4M3 (bias 7, max 448, S.1111.111 = NaN) with a per-token
 *    fp32 scale: value = scale * e4m3(code).
 *  - bf16 inputs give bf16 outputs and fp32 inputs give fp32 outputs; all
 *    internal accumulation is fp32.
 *  - Errors: all arguments are checked on the host before anything is queued,
 *    so a call that fails with DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED or
 *    DSA_ERR_WORKSPACE has queued nothing.  A failed kernel launch returns
 *    DSA_ERR_HIP.  dsa_last_error() then describes the failure (per thread).
 *    Faults inside a kernel surface at the caller's next synchronisation.
 *  - Index values read from device memory (Omega entries, block-table
 *    entries, sequence lengths) are bounds-checked by the kernels: an entry
 *    outside its valid range is skipped, never dereferenced.
 *  - Calls are reentrant; concurrent calls on different streams are safe.
 */
#ifndef LIBDSA_DSA_H
#define LIBDSA_DSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DSA_OK = 0,
    DSA_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, bad size or shape */
    DSA_ERR_UNSUPPORTED = 2,   /* valid but not implemented (head size, dtype mix) */
    DSA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than the size query says */
    DSA_ERR_HIP = 4            /* a HIP runtime call or kernel launch failed */
} dsa_status_t;

typedef enum { DSA_F32 = 0, DSA_BF16 = 1, DSA_FP8_E4M3 = 2 } dsa_dtype_t;

/* Static text for a status code. */
const char* dsa_status_string(dsa_status_t s);
/* Detail of the last failed call on this host thread ("" if none). */
const char* dsa_last_error(void);
/* Library version, major * 10000 + minor * 100 + patch. */
int dsa_version(void);

/*
 * Lightning indexer (report section 2.3.1; review page "核心公式", first formula).
 *
 *   scores[i, s] = sum_j w[i, j] * ReLU(q^I[i, j] . k^I[s])   for s <= q_pos0 + i
 *   scores[i, s] = -INFINITY                                  for s >  q_pos0 + i
 * for 0 <= i < Tq, 0 <= s < Tk.  Row i is the query at position q_pos0 + i.
 *
 * idx_dtype = DSA_FP8_E4M3: q_idx uint8 [Tq, HI, dI], q_scale [Tq], k_idx uint8
 *   [Tk, dI], k_scale [Tk]; dI must be 128, 1 <= HI <= 128, HI % 4 == 0.  Products
 *   run on FP8 matrix cores with fp32 accumulation, then ReLU, the w-weighted
 *   head sum and the scales in fp32.
 * idx_dtype = DSA_F32: q_idx float [Tq, HI, dI], k_idx float [Tk, dI], scales
 *   ignored (may be NULL); dI % 4 == 0, dI <= 128, HI * dI <= 1024.
 * w: float [Tq, HI], any sign.  scores: float, row stride ld_scores >= Tk,
 *   ld_scores % 4 == 0.  Requires Tk >= q_pos0 + Tq (every query sees its prefix).
 * Workspace: dsa_index_scores_workspace_size() bytes of device memory (the FP8
 *   path keeps a per-token mix of the w-weighted indexer queries there: 512 bytes
 *   per query row; the fp32 path needs none and ws may be NULL).  The scores
 *   are computed as sum_j w ReLU(x_j) = 1/2 (sum_j w_j x_j + sum_j w_j |x_j|),
 *   except where the two terms cancel (|A| + |L| > 15 |A + L|): those blocks are
 *   recomputed in the direct form on exact bf16 products (an all-negative score is
 *   exactly 0).
 */
size_t dsa_index_scores_workspace_size(int Tq, int HI, int dI, dsa_dtype_t idx_dtype);
dsa_status_t dsa_index_scores(const void* q_idx, const float* q_scale, const float* w,
                              const void* k_idx, const float* k_scale, dsa_dtype_t idx_dtype,
                              int Tq, int Tk, int HI, int dI, int64_t q_pos0,
                              float* scores, int64_t ld_scores, void* ws, size_t ws_bytes,
                              hipStream_t stream);

/*
 * Top-k index set (review page "核心公式", second formula; k = 2048 in the
 * report; deterministic selection, report section 5.2.1).
 *
 * Row i (position p = q_pos0 + i) selects n = min(k, p + 1) of the candidates
 * s = 0..p of scores[i, :]: the n largest, equal scores going to the lower s,
 * -0.0 equal to +0.0.  idx [Tq, k] int32 receives them in ascending order,
 * followed by -1.  Rows with p + 1 <= k need no selection and read nothing.
 * Scores are expected finite; NaN orders above +inf (positive NaN) or below
 * -inf (negative NaN).  1 <= k <= 8192; ld_scores >= Tk >= q_pos0 + Tq.
 * Workspace: dsa_topk_workspace_size() bytes (0 for many rows; ws may then be
 * NULL).  For few long rows a workspace of that size lets the library split each
 * row across workgroups and merge the parts; without it the result is the same,
 * computed by one workgroup per row.
 */
size_t dsa_topk_workspace_size(int Tq, int Tk, int k);
dsa_status_t dsa_topk(const float* scores, int64_t ld_scores, int Tq, int Tk, int64_t q_pos0,
                      int k, int32_t* idx, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * GQA sparse aggregation (report section 2.3.2; review page "核心公式", third
 * formula): for every query row t and head h in group g = h / (Hq / G),
 *   out[t, h, :] = softmax_s(sm_scale * q[t, h, :] . K[s, g, :]) V[s, g, :]
 * over the positions s listed in idx[t, 0..k) (entries < 0 are skipped), the
 * same list for every group.  A row with no valid entry gives zeros.
 *
 * dtype DSA_BF16 (bf16 matrix cores, fp32 softmax) or DSA_F32 (fp32 vector
 * ALU); d must be 128; Hq % G == 0 and Hq / G <= 16.
 * q [Tq, Hq, d]; out [Tq, Hq, d] (same dtype).
 * Contiguous K/V (block_table == NULL): k, v [n_kv, G, d]; entries outside
 *   [0, n_kv) are skipped.
 * Paged K/V (block_table != NULL): k, v [n_kv, block_size, G, d] with n_kv
 *   physical blocks; position s of sequence b lives in block
 *   block_table[b, s / block_size] at slot s % block_size; block_table is
 *   [n_seq, max_blocks].  row_seq [Tq] gives the sequence of each row (NULL:
 *   row t is sequence t).  seq_lens [n_seq] (NULL: no length limit beyond
 *   max_blocks * block_size) bounds the valid positions of each sequence.
 * ws (nullable): with at least dsa_sparse_gqa_attn_workspace_size() bytes the
 *   library may split long rows across workgroups and combine the partial
 *   softmax results; with NULL every row is done by one workgroup.
 */
size_t dsa_sparse_gqa_attn_workspace_size(int Tq, int k, int Hq, int d);
dsa_status_t dsa_sparse_gqa_attn(const void* q, const void* k, const void* v, dsa_dtype_t dtype,
                                 int n_kv, const int32_t* block_table, int max_blocks,
                                 int block_size, const int32_t* row_seq, const int32_t* seq_lens,
                                 const int32_t* idx, int Tq, int topk, int Hq, int G, int d,
                                 float sm_scale, void* out, void* ws, size_t ws_bytes,
                                 hipStream_t stream);

/*
 * GQA sparse attention with adjacent-query Top-KV deduplication (report section
 * 5.3, sparse attention optimisation: adjacent queries select largely the same
 * keys).  The rows are grouped in blocks of 16 by absolute position (row i is
 * at position q_pos0 + i; a block holds positions 16 B .. 16 B + 15).  For each
 * block the union of its rows' Omega is formed with a 16-bit mask per union
 * position (which rows selected it); a marked block gathers each union
 * position's K/V rows once and computes all its rows over the union, masking
 * in the matrix products' accumulator layout the positions a row did not
 * select.  The result is out as dsa_sparse_gqa_attn computes it for contiguous
 * bf16 K/V (the same terms in the same order), up to the rounding of the
 * online softmax's steps.  mode 0 marks a block when 2 x (union size) is below
 * its number of selected entries (the measured cost of a union position, which
 * every row of the block computes, against a selected entry of the per-query
 * kernel); the other blocks run the per-query kernel.  mode 1 marks every
 * block.  dsa_prefill makes the same mode-0 choice for every chunk.
 * q, k, v, out, idx, n_kv: as dsa_sparse_gqa_attn with DSA_BF16, contiguous
 * K/V, Hq == 8 G, d == 128, topk <= 2048, n_kv <= 262144; a row's entries
 * must be distinct (as top-k produces them).  Workspace:
 * dsa_sparse_gqa_attn_dedup_workspace_size() bytes.
 */
size_t dsa_sparse_gqa_attn_dedup_workspace_size(int Tq, int64_t q_pos0, int topk);
dsa_status_t dsa_sparse_gqa_attn_dedup(const void* q, const void* k, const void* v, int n_kv,
                                       const int32_t* idx, int Tq, int64_t q_pos0, int topk,
                                       int Hq, int G, int d, float sm_scale, int mode, void* out,
                                       void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Fused prefill of one sequence: indexer -> top-k -> sparse attention for the
 * Tq queries at positions q_pos0 .. q_pos0 + Tq - 1 over the Tk = q_pos0 + Tq
 * keys (report sections 2.3.1-2.3.2).  Queries are processed in chunks of
 * chunk_rows rows (the chunked indexer of report section 5.2.1, split along
 * the query axis); every row still sees its whole prefix, so chunking changes
 * no result.  chunk_rows <= 0 means one chunk.
 *
 * q [Tq, Hq, d], k / v [Tk, G, d] (dtype), q_idx / q_scale / w [Tq, ...] and
 * k_idx / k_scale [Tk, ...] as in dsa_index_scores, out [Tq, Hq, d].
 * idx_out (nullable) [Tq, topk] receives every row's Omega as dsa_topk writes it.
 *
 * Results equal those of dsa_index_scores -> dsa_topk -> dsa_sparse_gqa_attn
 * bit for bit.  For an FP8 indexer with HI <= 64 and topk <= 8192, chunks
 * whose rows see 48K to 512K keys take a candidate path instead of writing
 * full score rows: the indexer first scores about Tk/64 sampled keys per row,
 * a lower bound for each row's topk-th score is taken from the samples
 * (padded by 5 sigma in rank), the indexer then keeps only the scores at or
 * above the bound (at most 8192 per row), and Omega is selected exactly from
 * those.  A row whose kept scores cannot give the exact answer (fewer than
 * topk, or more than 8192 of them; about 1e-7 per row on generic data, but
 * certain with massive ties) makes the library redo its whole chunk over full
 * score rows, on the device and without a host synchronisation.
 *
 * Workspace: dsa_prefill_workspace_size() bytes; it holds one chunk's fp32
 * score matrix (chunk_rows x Tk), its index sets when idx_out is NULL, the
 * samples (chunk_rows x up to 8192 fp32), the candidate lists (chunk_rows x
 * 8192 x 8 bytes) and per-row bounds and counters.
 */
size_t dsa_prefill_workspace_size(int Tq, int64_t q_pos0, int chunk_rows, int topk);
/*
 * Diagnostics of the candidate path: the byte offset, within a prefill
 * workspace of these arguments, of two int32 counters that a dsa_prefill call
 * taking the candidate path rewrites: [0] the chunks that took it, [1] the rows
 * whose candidates could not give the exact answer (their chunks were redone
 * over full score rows).  A call that takes the path for no chunk leaves them
 * untouched.  Returns SIZE_MAX for invalid sizes.
 */
size_t dsa_prefill_stats_offset(int Tq, int64_t q_pos0, int chunk_rows, int topk);
dsa_status_t dsa_prefill(const void* q, const void* k, const void* v, dsa_dtype_t dtype,
                         const void* q_idx, const float* q_scale, const float* w,
                         const void* k_idx, const float* k_scale, dsa_dtype_t idx_dtype,
                         int Tq, int64_t q_pos0, int Hq, int G, int d, int HI, int dI, int topk,
                         float sm_scale, int chunk_rows, void* out, int32_t* idx_out,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Packed variable-length prefill (report section 5.1.2: DSA for batches of
 * sequences of different lengths): nseq sequences packed along the token
 * dimension, sequence i holding tokens cu_seqlens[i] .. cu_seqlens[i+1] - 1 of
 * every per-token array.  Each sequence is an independent causal prefill: its
 * rows see only its own keys, scores exist only over its own prefix, and the
 * top-k runs only over that region, so every sequence's results are those of
 * dsa_prefill on it alone (q_pos0 = 0), bit for bit.
 *
 * cu_seqlens: int32 [nseq + 1] in HOST memory, cu_seqlens[0] = 0, non-decreasing;
 *   empty sequences are allowed.  T = cu_seqlens[nseq] tokens in total.
 * q, k, v, q_idx, q_scale, w, k_idx, k_scale, out: as for dsa_prefill with T rows.
 * idx_out (nullable) int32 [T, topk]: Omega of each row as positions LOCAL to its
 *   sequence (0-based; add cu_seqlens[i] for rows of the packed arrays), -1 padded.
 * chunk_rows: query rows per chunk within each sequence (0 = whole sequence).
 * Workspace: dsa_prefill_workspace_size(max_len, 0, chunk_rows, topk) bytes, max_len
 *   being the longest sequence; the candidate-path counters of the whole call are at
 *   dsa_prefill_stats_offset(max_len, 0, chunk_rows, topk).  The sequences run one
 *   after another on `stream`, sharing the workspace.
 */
dsa_status_t dsa_prefill_varlen(const void* q, const void* k, const void* v, dsa_dtype_t dtype,
                                const void* q_idx, const float* q_scale, const float* w,
                                const void* k_idx, const float* k_scale, dsa_dtype_t idx_dtype,
                                const int32_t* cu_seqlens, int nseq, int Hq, int G, int d, int HI,
                                int dI, int topk, float sm_scale, int chunk_rows, void* out,
                                int32_t* idx_out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Paged decode step (report section 5.3): one new query per sequence b, at
 * position seq_lens[b] - 1, whose own K/V/k^I entries are already in the
 * caches.  Runs the FP8 indexer over the sequence's paged indexer keys, the
 * top-k, and sparse attention over the paged K/V.
 *
 * q [B, Hq, d] (dtype), q_idx uint8 [B, HI, dI], q_scale [B], w [B, HI];
 * kidx_cache uint8 [num_blocks, block_size, dI], kidx_scale [num_blocks, block_size];
 * k_cache / v_cache [num_blocks, block_size, G, d] (dtype);
 * block_table int32 [B, max_blocks]; seq_lens int32 [B] (device).
 * A sequence length outside [1, max_blocks * block_size] yields a zero output
 * row and an index row of -1.  dI must be 128 and block_size 64 (one cache block
 * is one 64-key indexer step); dtype DSA_BF16 or DSA_F32.
 * out [B, Hq, d]; idx_out (nullable) [B, topk].
 * When max_blocks * block_size is 48K..512K, HI <= 64 and topk <= 8192 the
 * step takes the same sampled-bound candidate path as dsa_prefill (scores of
 * about max_len/64 sampled positions per sequence, a padded lower bound of the
 * topk-th score, only the scores above it kept, exact selection, and a
 * device-side redo of the step over full score rows if any sequence's kept
 * scores cannot give the exact answer); the results are those of the full
 * score rows bit for bit.
 * Workspace: dsa_decode_workspace_size() bytes.
 */
size_t dsa_decode_workspace_size(int B, int max_blocks, int block_size, int topk, int Hq, int d);
/* As dsa_prefill_stats_offset, for a decode workspace ([0] = 1 when the step took the
 * candidate path); SIZE_MAX when these shapes never take it. */
size_t dsa_decode_stats_offset(int B, int max_blocks, int block_size, int topk, int Hq, int d);
dsa_status_t dsa_decode(const void* q, const void* q_idx, const float* q_scale, const float* w,
                        const void* kidx_cache, const float* kidx_scale, const void* k_cache,
                        const void* v_cache, dsa_dtype_t dtype, const int32_t* block_table,
                        const int32_t* seq_lens, int B, int num_blocks, int max_blocks,
                        int block_size, int Hq, int G, int d, int HI, int dI, int topk,
                        float sm_scale, void* out, int32_t* idx_out, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/*
 * dsa_decode without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Arguments, checks and results are those of dsa_decode (the same kernels,
 * bit for bit); the workspace is a scratch area the library keeps in device memory on
 * every GPU it runs on, held until the process ends, of dsa_decode_noalloc_max_workspace()
 * bytes (96 MiB; the 64-sequence step over 256K-token caches needs about 82 MiB).  A step
 * whose dsa_decode_workspace_size() exceeds that fails with DSA_ERR_WORKSPACE and queues
 * nothing.  The step runs on the current device (`stream` must belong to it) and allocates
 * and frees nothing.  All calls on one GPU share its scratch: calls that overlap on one GPU
 * (on other streams or from other host threads) race, and the caller must order them.  No
 * result depends on what an earlier call left in the scratch.  The candidate-path counters
 * of dsa_decode_stats_offset() are not available.
 */
size_t dsa_decode_noalloc_max_workspace(void);
dsa_status_t dsa_decode_noalloc(const void* q, const void* q_idx, const float* q_scale,
                                const float* w, const void* kidx_cache, const float* kidx_scale,
                                const void* k_cache, const void* v_cache, dsa_dtype_t dtype,
                                const int32_t* block_table, const int32_t* seq_lens, int B,
                                int num_blocks, int max_blocks, int block_size, int Hq, int G,
                                int d, int HI, int dI, int topk, float sm_scale, void* out,
                                int32_t* idx_out, hipStream_t stream);

/*
 * Per-token FP8 quantisation of indexer vectors (the FP8 inputs of report
 * section 2.3.1's indexer; the pages give no recipe, and this is the reading
 * every call above assumes): for each row t of x [T, n],
 *   scale[t] = max_i |x[t, i]| / 448   (1 when the row is all zeros),
 *   codes[t, i] = the E4M3 code nearest to clamp(x[t, i] / scale[t], -448, 448),
 *                 ties to the code with an even last bit,
 * with both divisions in fp32, correctly rounded.  x: fp32 or bf16 [T, n]
 * (x_dtype DSA_F32 or DSA_BF16, 4-byte aligned); codes uint8 [T, n] (any
 * alignment); scale float [T].  Rows of q^I [T, HI * dI] are quantised with
 * n = HI * dI (one scale per query token, the layout dsa_index_scores reads);
 * rows of k^I with n = dI.  Non-finite inputs are not supported.  No workspace.
 */
dsa_status_t dsa_quantize_e4m3(const void* x, dsa_dtype_t x_dtype, int T, int n, uint8_t* codes,
                               float* scale, hipStream_t stream);

/*
 * Cache append (report section 5.3 serves decode from paged caches): writes
 * one new token per sequence b into the caches that dsa_decode reads, at
 * absolute position positions[b] (device int32 [B]) of sequence b:
 *   slot = block_table[b, positions[b] / block_size] * block_size
 *          + positions[b] % block_size
 *   k_cache[slot] = k_new[b], v_cache[slot] = v_new[b]     (rows of G * d, dtype)
 *   kidx_cache[slot], kidx_scale[slot] = dsa_quantize_e4m3 of kidx_new[b] (dI values)
 * k_new / v_new [B, G, d] (dtype DSA_BF16 or DSA_F32; a row of G * d elements
 * must be a multiple of 16 bytes); kidx_new [B, dI] fp32 or bf16 (kidx_dtype),
 * 4-byte aligned; caches laid out as for dsa_decode.  A position outside
 * [0, max_blocks * block_size) or a block-table entry outside [0, num_blocks)
 * skips that sequence (nothing written).  The caller gives every sequence its
 * own slot: two sequences writing one slot race.  A decode step after the
 * append passes seq_lens[b] = positions[b] + 1.  No workspace.
 */
dsa_status_t dsa_cache_append(const void* k_new, const void* v_new, dsa_dtype_t dtype,
                              const void* kidx_new, dsa_dtype_t kidx_dtype,
                              const int32_t* positions, const int32_t* block_table, int B,
                              int num_blocks, int max_blocks, int block_size, int G, int d, int dI,
                              void* k_cache, void* v_cache, uint8_t* kidx_cache,
                              float* kidx_scale, hipStream_t stream);

/*
 * ---- Training side: the sparse adaptation stage of report section 2.3.3 ----
 * The indexer is trained with L = sum_t sum_g KL(p[t,S_t,g] || softmax(I[t,S_t])),
 * S_t = Omega_t (review page, "核心公式", sparse adaptation loss), keeping only the
 * post-top-k indexer scores in the forward (report section 5.1.2).
 */

/*
 * Indexer scores at the selected positions: vals[t, i] = I[t, idx[t, i]] for t < Tq,
 * i < topk (the score of dsa_index_scores), -INFINITY where idx[t, i] is -1 or outside
 * [0, Tk).  FP8 only (dI = 128, 1 <= HI <= 128).  q_idx [Tq, HI, dI], q_scale [Tq],
 * w [Tq, HI], k_idx [Tk, dI], k_scale [Tk], idx int32 [Tq, topk] -> vals float [Tq, topk].
 * Computed in fp32 from the decoded codes.  No workspace.
 */
dsa_status_t dsa_index_scores_at(const void* q_idx, const float* q_scale, const float* w,
                                 const void* k_idx, const float* k_scale, dsa_dtype_t idx_dtype,
                                 int Tq, int Tk, int HI, int dI, const int32_t* idx, int topk,
                                 float* vals, hipStream_t stream);

/*
 * Backward of dsa_index_scores_at: given g float [Tq, topk] = dL/dvals, the gradients of L
 * with respect to the dequantised indexer inputs (FP8 rounding taken as the identity,
 * ReLU'(0) = 0):  dq_idx float [Tq, HI, dI] and dw float [Tq, HI] are written; dk_idx
 * float [Tk, dI] is ACCUMULATED (zero it first).  Entries of idx that are -1 or out of range
 * contribute nothing.  FP8 only, dI = 128, 1 <= HI <= 64.
 * With a workspace of dsa_index_scores_at_bwd_workspace_size() bytes (nonzero when HI is a
 * multiple of 16) the dk_idx contributions are stored per (row, entry) for chunks of rows and
 * summed per position in row order: dk_idx is then bit-reproducible.  With ws = NULL
 * (ws_bytes 0) they are added with fp32 atomic adds, whose order, and so the last bits, vary.
 * A key listed more than once in a row (top-k never does so) counts every time in both forms;
 * with a workspace its extra copies are added atomically after the ordered sums, so such rows
 * lose only the bit-reproducibility.
 */
size_t dsa_index_scores_at_bwd_workspace_size(int Tq, int Tk, int HI, int topk);
dsa_status_t dsa_index_scores_at_bwd(const void* q_idx, const float* q_scale, const float* w,
                                     const void* k_idx, const float* k_scale,
                                     dsa_dtype_t idx_dtype, int Tq, int Tk, int HI, int dI,
                                     const int32_t* idx, int topk, const float* g,
                                     float* dq_idx, float* dw, float* dk_idx, void* ws,
                                     size_t ws_bytes, hipStream_t stream);

/*
 * Sparse attention forward that also keeps what the backward needs: as dsa_sparse_gqa_attn
 * over contiguous K/V [n_kv, G, d], plus lse float [Tq, Hq] = ln sum_{s in Omega_t}
 * exp(sm_scale q . K[s]) per query head (-INFINITY for a row with no valid entry).
 * Workspace: dsa_sparse_gqa_attn_workspace_size() bytes (may be NULL for Tq >= 2048).
 */
dsa_status_t dsa_sparse_gqa_attn_lse(const void* q, const void* k, const void* v,
                                     dsa_dtype_t dtype, int n_kv, const int32_t* idx, int Tq,
                                     int topk, int Hq, int G, int d, float sm_scale, void* out,
                                     float* lse, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Backward of the sparse GQA attention, with the sparse indexer loss fused in (report
 * section 5.1.2: the attention backward recomputes the softmax, so the loss's target is
 * reduced there).  BF16, contiguous K/V, d = 128.  From the forward's out and lse and the
 * incoming gradient dout [Tq, Hq, d] (bf16), with P = exp(sm_scale q.K[s] - lse) over the
 * valid entries s of idx[t, :]:
 *   dq [Tq, Hq, d] (bf16, written) = sm_scale sum_s dS_s K[s],  dS_s = P_s (dout.V[s] - dout.out);
 *   dk, dv float [n_kv, G, d] ACCUMULATED (zero them first): dk[s] += sm_scale sum_h dS_s q_h,
 *   dv[s] += sum_h P_s dout_h over each group's heads.
 * With a workspace of dsa_sparse_gqa_attn_bwd_workspace_size() bytes the contributions are
 * stored per (row, entry, group) for chunks of rows and summed per position in row order:
 * dk and dv are then bit-reproducible.  With ws = NULL (ws_bytes 0) they are added with fp32
 * atomic adds, whose order, and so the last bits, vary between runs.  A key listed more than
 * once in a row (top-k never does so) counts every time, as in the forward; with a workspace
 * its extra copies are added atomically after the ordered sums (those rows lose only the
 * bit-reproducibility).
 * When vals float [Tq, topk] (= dsa_index_scores_at at idx) is given (topk <= 2048), also
 *   kl float [Tq]: sum_g KL(p[t,:,g] || softmax(vals[t,:])) over the valid entries, p[t,s,g]
 *     the mean of the group's heads' P (report section 2.3.3, sparse adaptation loss),
 *   dI float [Tq, topk]: d kl[t] / d vals[t, i] = G softmax(vals[t,:])_i - sum_g p[t,i,g]
 *     (0 for padding), ready for dsa_index_scores_at_bwd.
 * vals, kl and dI may all be NULL.
 */
size_t dsa_sparse_gqa_attn_bwd_workspace_size(int Tq, int topk, int G, int n_kv);
dsa_status_t dsa_sparse_gqa_attn_bwd(const void* q, const void* k, const void* v,
                                     dsa_dtype_t dtype, int n_kv, const int32_t* idx, int Tq,
                                     int topk, int Hq, int G, int d, float sm_scale,
                                     const void* out, const void* dout, const float* lse,
                                     void* dq, float* dk, float* dv, const float* vals, float* kl,
                                     float* dI, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * ---- Training side: the dense warm-up stage of report section 2.3.3 ----
 * Before the sparse stage the indexer is trained against the dense attention with
 * L = sum_t sum_g KL(p[t,:,g] || softmax(I[t,:])) over every key s <= t (review page,
 * "核心公式", dense warm-up loss).  One step: dsa_index_scores (the full causal rows of I),
 * dsa_indexer_warmup_kl (turns them into dL/dI in place), dsa_index_scores_bwd_dense.
 * Rows may be processed in chunks (q_pos0 > 0), as in prefill.
 */

/*
 * Dense warm-up loss and its gradient.  q [Tq, Hq, d] and K [Tk, G, d] bf16 (d = 128) are the
 * main attention's query heads (row t at position q_pos0 + t) and keys; head h belongs to
 * group h / (Hq / G).  p[t,s,g] is the mean over the group's heads of
 * softmax_s(sm_scale q_h . K[s, g]) over s <= q_pos0 + t; lse float [Tq, Hq] (natural log of
 * that softmax's normaliser, as a dense attention forward returns it) may be passed to skip
 * its computation, or NULL.  scores float [Tq, ld_scores] holds I[t, s] for s <= q_pos0 + t
 * (as dsa_index_scores writes it) and is overwritten there with
 *   dL/dI[t, s] = G softmax(I[t, 0..pos])_s - sum_g p[t,s,g];
 * entries beyond the prefix are left as they are.  kl float [Tq] receives
 * sum_g KL(p[t,:,g] || softmax(I[t,:])).  The target p is a constant (the indexer's inputs are
 * detached from the main model).  Supported: Hq / G in {1, 2, 4, 8, 16} with
 * G * max(1, Hq / G / 4) <= 8; Tk >= q_pos0 + Tq.  fp32 softmax from bf16 matrix-core scores.
 * No workspace; deterministic.
 */
dsa_status_t dsa_indexer_warmup_kl(const void* q, const void* k, dsa_dtype_t dtype, int Tq, int Tk,
                                   int64_t q_pos0, int Hq, int G, int d, float sm_scale,
                                   const float* lse, float* scores, int64_t ld_scores, float* kl,
                                   hipStream_t stream);

/*
 * Backward of the dense indexer scores: given g float [Tq, ld_g] = dL/dI[t, s] for
 * s <= q_pos0 + t (entries beyond are ignored), the gradients with respect to the
 * dequantised indexer inputs (FP8 rounding taken as the identity, ReLU'(0) = 0):
 * dq_idx float [Tq, HI, dI] and dw float [Tq, HI] are written; dk_idx float [Tk, dI] is
 * ACCUMULATED (zero it first; chunks of rows add into it in call order).  FP8 only,
 * dI = 128, HI in {16, 32, 48, 64}; scales non-negative (as the quantiser makes them).
 * The gradient G = dI w [x > 0] is rounded to bf16 for the two matrix-core products.
 * Workspace: dsa_index_scores_bwd_dense_workspace_size() bytes (bf16 copies of the codes and
 * partial sums of dk_idx over ranges of rows, added in a fixed order): every output is
 * bit-reproducible.
 */
size_t dsa_index_scores_bwd_dense_workspace_size(int Tq, int Tk, int HI);
dsa_status_t dsa_index_scores_bwd_dense(const void* q_idx, const float* q_scale, const float* w,
                                        const void* k_idx, const float* k_scale,
                                        dsa_dtype_t idx_dtype, int Tq, int Tk, int HI, int dI,
                                        int64_t q_pos0, const float* g, int64_t ld_g,
                                        float* dq_idx, float* dw, float* dk_idx, void* ws,
                                        size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* LIBDSA_DSA_H */
