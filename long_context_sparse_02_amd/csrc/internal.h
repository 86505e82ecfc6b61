// internal.h -- launchers shared between the libdsa translation units.
// Each launcher queues one kernel on `stream` and returns the launch status;
// arguments have already been validated by the C entry points.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dsa.h"

namespace dsa {

// Records the detail of a failure for dsa_last_error() (per thread) and returns st.
dsa_status_t api_fail(dsa_status_t st, const char* fmt, ...);
// Every argument check of dsa_decode except the workspace's; DSA_OK when they pass.
dsa_status_t decode_check_args(const void* q, const void* q_idx, const float* q_scale,
                               const float* w, const void* kidx_cache, const float* kidx_scale,
                               const void* k_cache, const void* v_cache, dsa_dtype_t dtype,
                               const int32_t* block_table, const int32_t* seq_lens, int B,
                               int num_blocks, int max_blocks, int block_size, int Hq, int G,
                               int d, int HI, int dI, int topk, void* out, int32_t* idx_out);
// Bytes of the per-GPU device scratch behind dsa_decode_noalloc (the 64-sequence decode
// step over 256K-token caches needs about 82 MiB).
constexpr size_t kNoAllocScratchBytes = (size_t)96 << 20;

// Lightning indexer, contiguous keys (prefill).  Row i is position q_pos0 + i.
// The FP8 kernel needs index_fp8_workspace_bytes(Tq) bytes of device scratch.
// run_if (nullable): the launch does nothing unless *run_if != 0 when it runs (resident
// path only).  qmix_ready: the workspace already holds this chunk's qmix pre-pass.
size_t index_fp8_workspace_bytes(int Tq);
hipError_t launch_index_fp8(const uint8_t* q_idx, const float* q_scale, const float* w,
                            const uint8_t* k_idx, const float* k_scale, int Tq, int Tk, int HI,
                            int64_t q_pos0, float* scores, int64_t ld, void* ws,
                            hipStream_t stream, const int* run_if = nullptr,
                            bool qmix_ready = false);
// Candidate pipeline of the fused prefill (FP8, HI <= 64).  Sample: the qmix pre-pass, then
// the scores of S sampled keys per row (S a multiple of 1024, or 0 for the pre-pass alone)
// into samples [Tq, S].
// Candidates (qmix ready): every causal score >= tau[row] appended to
// row's list cand [Tq, cap] as (order key, position); cnt[row] counts all of them (it must
// start at 0) and may exceed cap, in which case only cap pairs were stored.
hipError_t launch_index_fp8_sample(const uint8_t* q_idx, const float* q_scale, const float* w,
                                   const uint8_t* k_idx, const float* k_scale, int Tq, int Tk,
                                   int HI, int64_t q_pos0, float* samples, int S, void* ws,
                                   hipStream_t stream);
hipError_t launch_index_fp8_candidates(const uint8_t* q_idx, const float* q_scale,
                                       const float* w, const uint8_t* k_idx,
                                       const float* k_scale, int Tq, int Tk, int HI,
                                       int64_t q_pos0, const float* tau, int32_t* cnt,
                                       uint2* cand, int cap, void* ws, hipStream_t stream);
hipError_t launch_index_f32(const float* q_idx, const float* w, const float* k_idx, int Tq,
                            int Tk, int HI, int dI, int64_t q_pos0, float* scores, int64_t ld,
                            hipStream_t stream);
// Lightning indexer over a paged key cache, one query per sequence (decode).
// scores [B, ld]; entries s >= seq_len are left unwritten.
hipError_t launch_index_fp8_paged(const uint8_t* q_idx, const float* q_scale, const float* w,
                                  const uint8_t* kidx_cache, const float* kidx_scale,
                                  const int32_t* block_table, const int32_t* seq_lens, int B,
                                  int num_blocks, int max_blocks, int block_size, int HI,
                                  float* scores, int64_t ld, hipStream_t stream,
                                  const int* run_if = nullptr);
// Candidate pipeline of the decode step, as for the prefill: the scores of S sampled
// positions of each sequence (S a multiple of 64) into samples [B, S], then every score
// >= tau[b] appended to the sequence's list cand [B, cap] (cnt[b] must start at 0).
hipError_t launch_index_fp8_paged_sample(const uint8_t* q_idx, const float* q_scale,
                                         const float* w, const uint8_t* kidx_cache,
                                         const float* kidx_scale, const int32_t* block_table,
                                         const int32_t* seq_lens, int B, int num_blocks,
                                         int max_blocks, int block_size, int HI, float* samples,
                                         int S, hipStream_t stream);
hipError_t launch_index_fp8_paged_candidates(const uint8_t* q_idx, const float* q_scale,
                                             const float* w, const uint8_t* kidx_cache,
                                             const float* kidx_scale, const int32_t* block_table,
                                             const int32_t* seq_lens, int B, int num_blocks,
                                             int max_blocks, int block_size, int HI,
                                             const float* tau, int32_t* cnt, uint2* cand, int cap,
                                             hipStream_t stream);

// Top-k per row.  Candidates of row i: 0 .. n_i-1 with n_i = q_pos0 + i + 1, or
// n_i = row_len[i] when row_len is given (0 if outside [0, Tk]).  With a workspace of
// topk_workspace_bytes() bytes, few long rows are split into segments and merged.
size_t topk_workspace_bytes(int Tq, int Tk, int k);
hipError_t launch_topk(const float* scores, int64_t ld, int Tq, int Tk, int64_t q_pos0,
                       const int32_t* row_len, int k, int32_t* idx, void* ws, hipStream_t stream,
                       const int* run_if = nullptr);
// Fused-prefill selection.  Bound: for each row of n = q_pos0 + row + 1 > cap candidates, a
// lower bound for the k-th largest score from the row's S samples, padded so that it fails
// (fewer than k scores at or above it, or more than cap) with probability ~1e-7; rows with
// n <= cap get -FLT_MAX (every causal score is a candidate).  It also zeroes cnt.  Select:
// Omega of each row from its candidate list (ascending, ties to the lower position, -1
// padded).  fallback points to int[3]: [0] the chunk's flag, zeroed by the bound launch and
// set by a row whose list cannot give the exact answer; [1] candidate chunks and [2] such
// rows in this call (reset by the bound launch of the call's first candidate chunk, `first`).
constexpr int kCandCap = 8192;
int fused_sample_count(int Tk);
// row_len (nullable): row lengths n = row_len[row] instead of q_pos0 + row + 1 (rows with a
// length outside [1, max_len] select nothing: an index row of -1).
hipError_t launch_topk_bound(const float* samples, int S, int Tq, int64_t q_pos0,
                             const int32_t* row_len, int max_len, int k, float* tau, int32_t* cnt,
                             int* fallback, int first, hipStream_t stream);
hipError_t launch_topk_select(const uint2* cand, const int32_t* cnt, int Tq, int64_t q_pos0,
                              const int32_t* row_len, int max_len, int k, int32_t* idx,
                              int* fallback, hipStream_t stream);

struct AttnArgs {
    const void* q; const void* k; const void* v; void* out;
    const int32_t* idx; int Tq; int topk; int Hq; int G; int d; float sm_scale;
    int n_kv;                                  // contiguous rows, or physical blocks
    const int32_t* block_table; int max_blocks; int block_size;
    const int32_t* row_seq; const int32_t* seq_lens;
    int bf16;                                  // 1: bf16 I/O, 0: fp32 I/O
    float* lse = nullptr;                      // optional [Tq, Hq]: natural-log log-sum-exp
    // contiguous bf16 only: row i is at position pos0 + i.  Rows the deduplicated attention
    // computes are skipped: positions below prefix_skip, and rows of 16-row blocks marked in
    // dedup_info (the union kernel's per-block info of this launch's rows)
    int64_t pos0 = 0;
    int64_t prefix_skip = 0;
    const int32_t* dedup_info = nullptr;
};
// Backward of the bf16 attention over contiguous K/V (d = 128, heads per group <= 16), with
// the sparse indexer loss fused in when vals is set (topk <= 2048 then).  dq is written (bf16);
// dk, dv (fp32 [n_kv, G, d]) are accumulated with atomic adds; kl [Tq] and dI [Tq, topk] are
// written when vals [Tq, topk] (the indexer scores at idx) is given.
struct AttnBwdArgs {
    const void* q; const void* k; const void* v; const void* out; const void* dout;
    const float* lse; const int32_t* idx; int Tq; int topk; int Hq; int G; int n_kv;
    float sm_scale;
    void* dq; float* dk; float* dv;
    const float* vals; float* kl; float* dI;
    // Rows r0 .. r0 + Tq - 1 of the index lists are processed.  With stg set, the dK / dV
    // contributions of entry e = (row - r0) * topk + i and group g are stored at
    // stg[(e * G + g) * 256 + {0: dV, 128: dK} + 0..127] instead of being added atomically.
    int r0 = 0;
    float* stg = nullptr;
};
hipError_t launch_sparse_attn_bwd(const AttnBwdArgs& a, hipStream_t stream);
// The deterministic reduction of staged contributions (chunk of C rows starting at row r0):
// mark each key's selecting rows in a bitmask [n_kv][C / 32], count and scan them into
// offsets [n_kv + 1] (offs needs n_kv + 1 + ceil(n_kv / 256) entries: the block totals follow),
// list each key's entries in row order, and add their sums into dk / dv.
// width 256: rows of [dV 128 | dK 128] per group into dv / dk [n_kv, G, 128];
// width 128: rows of 128 into dk [n_kv, 128] (G = 1, dv unused).
// dup (C * topk bytes) marks the entries that repeat a key already listed earlier in their
// row's list (whichever of the copies marks the bit first is listed); their contributions are
// added atomically after the ordered sums, so repeated keys count every time, in an order that
// is not reproducible (lists of distinct keys, as top-k gives, keep the reproducible sums).
hipError_t launch_stage_reduce(const int32_t* idx, int r0, int C, int topk, int n_kv, int G,
                               const float* stg, uint32_t* mask, int32_t* offs, int32_t* list,
                               uint8_t* dup, float* dk, float* dv, hipStream_t stream,
                               int width = 256);
// Splits used for a given shape when a workspace is available (1 = no split).
int attn_num_splits(int Tq, int topk);
size_t attn_partials_bytes(int Tq, int nsplit, int Hq, int d);
hipError_t launch_sparse_attn(const AttnArgs& a, int nsplit, float* partials, hipStream_t stream);

// Adjacent-query Top-KV deduplication (dedup.hip).  Blocks of kDedupRows adjacent query rows,
// aligned to absolute positions (block b of a chunk starting at position q_pos0 holds its rows
// at positions 16 (q_pos0 / 16 + b) .. + 15, so chunk sizes that are multiples of 16 give the
// same blocks); the union kernel writes info[3 b .. 3 b + 2] = {union size, selections,
// marked} per block,
// and for a marked block (kappa * union < selections) the ascending union list[b, 0 .. U) and
// the 16-bit masks of the rows that selected each position (list and mask rows of
// kDedupRows * topk entries).  It adds the marked blocks to *counter.  The dedup attention
// then computes the marked blocks' rows (bf16, Hq == 8 G, contiguous K/V); a per-query launch
// given dedup_info computes the rest.
constexpr int kDedupRows = 16;
constexpr int kDedupMaxTopk = 2048;
constexpr int kDedupMaxWords = 8192;         // positions < 262144
bool dedup_supported(int Hq, int G, int d, int topk, int64_t n_pos, int bf16);
// Positions below which every row of a sequence of len positions is in a whole-prefix block.
int64_t prefix_block_limit(int64_t len, int topk);
int dedup_blocks(int Tq, int64_t q_pos0);    // blocks of a chunk of Tq rows at q_pos0
hipError_t launch_dedup_union(const int32_t* idx, int Tq, int64_t q_pos0, int topk, int n_pos,
                              float kappa, int32_t* info, int32_t* ulist, uint16_t* umask,
                              int* counter, hipStream_t stream);
hipError_t launch_dedup_attn(const AttnArgs& a, int64_t q_pos0, const int32_t* info,
                             const int32_t* ulist, const uint16_t* umask, hipStream_t stream);
// n 32-bit zeros (a kernel, so that it may be captured into graphs).
hipError_t launch_fill_zero(uint32_t* p, int64_t n, hipStream_t stream);

// Blocks of whole-prefix rows: rows at positions t whose 16-row block (positions 16 B .. 16 B
// + 15 of their sequence) holds only rows with t + 1 <= topk select {0 .. t}, so a block's union
// is {0 .. min(16 B + 16, len) - 1} and a row's mask is u <= t: the deduplicated attention
// needs no union kernel for them.  A launch covers up to kMaxPrefixSegs segments (a sequence,
// or one chunk's part of it): segment i has its position 0 at launch row row0[i] and K/V row
// kv0[i], len[i] positions in all, and the launch takes its blocks blk0[i] .. blk0[i] +
// (blk_start[i + 1] - blk_start[i]) - 1; rows outside [0, Tq) of the launch are skipped.
// Passed by value as a kernel argument.
constexpr int kMaxPrefixSegs = 128;
struct PrefixBlocks {
    int n;
    int blk_start[kMaxPrefixSegs + 1];
    int row0[kMaxPrefixSegs];
    int kv0[kMaxPrefixSegs];
    int len[kMaxPrefixSegs];
    int blk0[kMaxPrefixSegs];
};
// The deduplicated attention of such blocks (bf16, Hq == 8 G, contiguous K/V from a.k / a.v;
// a.q, a.out: the launch's rows, a.Tq of them).
hipError_t launch_dedup_prefix_attn(const AttnArgs& a, const PrefixBlocks& pb, hipStream_t stream);
// Index lists of short sequences packed back to back (every row keeps its whole prefix):
// start[i] is the first row of sequence i relative to the launch, start[n] the row count;
// idx[r, e] = e for e <= t, -1 after.
struct SeqStarts {
    int n;
    int start[kMaxPrefixSegs + 1];
};
hipError_t launch_prefix_idx(const SeqStarts& rows, int topk, int32_t* idx, hipStream_t stream);

// Per-token E4M3 quantisation of x [T, n] (fp32, or bf16 when x_bf16): codes [T, n], scale [T].
hipError_t launch_quantize_e4m3(const void* x, int x_bf16, int T, int n, uint8_t* codes,
                                float* scale, hipStream_t stream);
// Append one token per sequence into the paged caches (rows of kv_row_bytes, a multiple of
// 16; kidx_new fp32 or bf16 [B, dI], quantised on the way in).
hipError_t launch_cache_append(const void* k_new, const void* v_new, int kv_row_bytes,
                               const void* kidx_new, int kidx_bf16, int dI,
                               const int32_t* positions, const int32_t* block_table, int B,
                               int num_blocks, int max_blocks, int block_size, void* k_cache,
                               void* v_cache, uint8_t* kidx_cache, float* kidx_scale,
                               hipStream_t stream);

// Training side: indexer scores at the selected positions and their backward (FP8, dI = 128).
hipError_t launch_index_at(const uint8_t* q_idx, const float* q_scale, const float* w,
                           const uint8_t* k_idx, const float* k_scale, int T, int Tk, int HI,
                           const int32_t* idx, int topk, float* vals, hipStream_t stream);
// Rows r0 .. r0 + T - 1.  With stg set (and H^I a multiple of 16), the dk contribution of
// entry e = (row - r0) * topk + i is stored at stg[e * 128 .. +128) instead of added atomically.
hipError_t launch_index_at_bwd(const uint8_t* q_idx, const float* q_scale, const float* w,
                               const uint8_t* k_idx, const float* k_scale, int T, int Tk, int HI,
                               const int32_t* idx, int topk, const float* g, float* dq, float* dw,
                               float* dk, hipStream_t stream, int r0 = 0, float* stg = nullptr);
bool index_at_bwd_stages(int HI);            // whether the staged form exists for this H^I

// Dense warm-up stage of the indexer's training (warmup.hip).
bool warmup_kl_supported(int Hq, int G);
hipError_t launch_warmup_kl(const uint16_t* q, const uint16_t* k, int Tq, int Tk, int64_t q_pos0,
                            int Hq, int G, float sm_scale, const float* lse, float* scores,
                            int64_t ld, float* kl, hipStream_t stream);
struct WarmupBwdPlan {
    int ldk, kblocks, nsplit, rows_per_split;
    size_t kt_bytes, qt_bytes, part_bytes, total;
};
WarmupBwdPlan plan_warmup_bwd(int Tq, int Tk, int HI);
hipError_t launch_warmup_ix_bwd(const uint8_t* q_idx, const float* q_scale, const float* w,
                                const uint8_t* k_idx, const float* k_scale, int Tq, int Tk, int HI,
                                int64_t q_pos0, const float* g, int64_t ld, float* dq, float* dw,
                                float* dk, void* ws, hipStream_t stream);

}  // namespace dsa
