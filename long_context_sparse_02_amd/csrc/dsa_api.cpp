// dsa_api.cpp -- C entry points of libdsa: argument checks, workspace
// planning and the chunked prefill / paged decode drivers.  Every check runs
// on the host before anything is queued; all work goes onto the caller's
// stream with no synchronisation.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/dsa.h"
#include "internal.h"

#define DSA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_err[512];

dsa_status_t fail(dsa_status_t st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

}  // namespace

dsa_status_t dsa::api_fail(dsa_status_t st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

namespace {

dsa_status_t hip_fail(hipError_t e, const char* what) {
    return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

#define REQUIRE(cond, st, ...) \
    do { if (!(cond)) return fail(st, __VA_ARGS__); } while (0)
#define REQUIRE_PTR(p) \
    do { \
        if (!(p)) return fail(DSA_ERR_INVALID_ARG, "%s is NULL", #p); \
        if (!aligned16(p)) return fail(DSA_ERR_INVALID_ARG, "%s is not 16-byte aligned", #p); \
    } while (0)
// scalar-accessed arrays (scales, index lists, block tables) need only 4-byte alignment
#define REQUIRE_PTR4(p) \
    do { \
        if (!(p)) return fail(DSA_ERR_INVALID_ARG, "%s is NULL", #p); \
        if (!aligned4(p)) return fail(DSA_ERR_INVALID_ARG, "%s is not 4-byte aligned", #p); \
    } while (0)
#define REQUIRE_OPT_PTR4(p) \
    do { if ((p) && !aligned4(p)) return fail(DSA_ERR_INVALID_ARG, "%s is not 4-byte aligned", #p); } while (0)
#define REQUIRE_OPT_PTR(p) \
    do { if ((p) && !aligned16(p)) return fail(DSA_ERR_INVALID_ARG, "%s is not 16-byte aligned", #p); } while (0)

constexpr size_t kAlign = 256;
constexpr int kCandMinKeys = 49152;          // fused prefill: candidate path from this many keys
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t ld_for(int64_t Tk) { return (Tk + 3) / 4 * 4; }

dsa_status_t check_indexer(const void* q_idx, const float* q_scale, const float* w,
                           const void* k_idx, const float* k_scale, dsa_dtype_t idx_dtype,
                           int Tq, int Tk, int HI, int dI, int64_t q_pos0) {
    REQUIRE(Tq >= 0 && Tk >= 0, DSA_ERR_INVALID_ARG, "negative size (Tq=%d, Tk=%d)", Tq, Tk);
    REQUIRE(q_pos0 >= 0, DSA_ERR_INVALID_ARG, "q_pos0 must be >= 0 (got %lld)", (long long)q_pos0);
    REQUIRE((int64_t)Tk >= q_pos0 + Tq, DSA_ERR_INVALID_ARG,
            "Tk (%d) must cover every query's prefix (q_pos0 + Tq = %lld)", Tk,
            (long long)(q_pos0 + Tq));
    REQUIRE(HI >= 1, DSA_ERR_INVALID_ARG, "HI must be >= 1 (got %d)", HI);
    REQUIRE_PTR(q_idx);
    REQUIRE_PTR(w);
    REQUIRE_PTR(k_idx);
    if (idx_dtype == DSA_FP8_E4M3) {
        REQUIRE(dI == 128, DSA_ERR_UNSUPPORTED, "FP8 indexer needs dI == 128 (got %d)", dI);
        REQUIRE(HI <= 128 && HI % 4 == 0, DSA_ERR_UNSUPPORTED,
                "FP8 indexer needs HI %% 4 == 0 and HI <= 128 (got %d)", HI);
        REQUIRE_PTR4(q_scale);
        REQUIRE_PTR4(k_scale);
    } else if (idx_dtype == DSA_F32) {
        REQUIRE(dI >= 4 && dI <= 128 && dI % 4 == 0, DSA_ERR_UNSUPPORTED,
                "fp32 indexer needs dI %% 4 == 0 and 4 <= dI <= 128 (got %d)", dI);
        REQUIRE((int64_t)HI * dI <= 1024, DSA_ERR_UNSUPPORTED,
                "fp32 indexer needs HI * dI <= 1024 (got %d * %d)", HI, dI);
    } else {
        return fail(DSA_ERR_UNSUPPORTED, "indexer dtype %d is not FP8_E4M3 or F32", (int)idx_dtype);
    }
    return DSA_OK;
}

size_t indexer_ws_bytes(int Tq, dsa_dtype_t idx_dtype) {
    return idx_dtype == DSA_FP8_E4M3 ? round_up(dsa::index_fp8_workspace_bytes(Tq)) : 0;
}

dsa_status_t run_indexer(const void* q_idx, const float* q_scale, const float* w,
                         const void* k_idx, const float* k_scale, dsa_dtype_t idx_dtype, int Tq,
                         int Tk, int HI, int dI, int64_t q_pos0, float* scores, int64_t ld,
                         void* ws, hipStream_t stream) {
    hipError_t e;
    if (idx_dtype == DSA_FP8_E4M3)
        e = dsa::launch_index_fp8(static_cast<const uint8_t*>(q_idx), q_scale, w,
                                  static_cast<const uint8_t*>(k_idx), k_scale, Tq, Tk, HI, q_pos0,
                                  scores, ld, ws, stream);
    else
        e = dsa::launch_index_f32(static_cast<const float*>(q_idx), w,
                                  static_cast<const float*>(k_idx), Tq, Tk, HI, dI, q_pos0, scores,
                                  ld, stream);
    return e == hipSuccess ? DSA_OK : hip_fail(e, "indexer launch");
}

dsa_status_t check_attn_shape(dsa_dtype_t dtype, int Hq, int G, int d, int topk) {
    REQUIRE(dtype == DSA_BF16 || dtype == DSA_F32, DSA_ERR_UNSUPPORTED,
            "attention dtype %d is not BF16 or F32", (int)dtype);
    REQUIRE(d == 128, DSA_ERR_UNSUPPORTED, "head size d must be 128 (got %d)", d);
    REQUIRE(G >= 1 && Hq >= 1 && Hq % G == 0, DSA_ERR_INVALID_ARG,
            "Hq (%d) must be a positive multiple of G (%d)", Hq, G);
    REQUIRE(Hq / G <= 16, DSA_ERR_UNSUPPORTED, "at most 16 query heads per group (got %d)", Hq / G);
    REQUIRE(topk >= 1 && topk <= 8192, DSA_ERR_INVALID_ARG, "topk must be in [1, 8192] (got %d)", topk);
    return DSA_OK;
}

}  // namespace

DSA_EXPORT const char* dsa_status_string(dsa_status_t s) {
    switch (s) {
        case DSA_OK: return "DSA_OK";
        case DSA_ERR_INVALID_ARG: return "DSA_ERR_INVALID_ARG";
        case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED";
        case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE";
        case DSA_ERR_HIP: return "DSA_ERR_HIP";
    }
    return "DSA_ERR_UNKNOWN";
}

DSA_EXPORT const char* dsa_last_error(void) { return g_err; }

DSA_EXPORT int dsa_version(void) { return 10000; }

DSA_EXPORT size_t dsa_index_scores_workspace_size(int Tq, int HI, int dI, dsa_dtype_t idx_dtype) {
    (void)HI; (void)dI;
    if (Tq <= 0) return 0;
    return indexer_ws_bytes(Tq, idx_dtype);
}

DSA_EXPORT dsa_status_t dsa_index_scores(const void* q_idx, const float* q_scale, const float* w,
                                         const void* k_idx, const float* k_scale,
                                         dsa_dtype_t idx_dtype, int Tq, int Tk, int HI, int dI,
                                         int64_t q_pos0, float* scores, int64_t ld_scores,
                                         void* ws, size_t ws_bytes, hipStream_t stream) {
    g_err[0] = 0;
    dsa_status_t st = check_indexer(q_idx, q_scale, w, k_idx, k_scale, idx_dtype, Tq, Tk, HI, dI, q_pos0);
    if (st != DSA_OK) return st;
    REQUIRE_PTR(scores);
    REQUIRE(ld_scores >= Tk && ld_scores % 4 == 0, DSA_ERR_INVALID_ARG,
            "ld_scores (%lld) must be >= Tk (%d) and a multiple of 4", (long long)ld_scores, Tk);
    const size_t need = indexer_ws_bytes(Tq, idx_dtype);
    if (need) {
        REQUIRE(ws && aligned16(ws) && ws_bytes >= need, DSA_ERR_WORKSPACE,
                "indexer needs %zu workspace bytes (got %zu%s)", need, ws_bytes, ws ? "" : ", ws is NULL");
    }
    return run_indexer(q_idx, q_scale, w, k_idx, k_scale, idx_dtype, Tq, Tk, HI, dI, q_pos0, scores,
                       ld_scores, ws, stream);
}

DSA_EXPORT size_t dsa_topk_workspace_size(int Tq, int Tk, int k) {
    if (Tq <= 0 || Tk <= 0 || k <= 0) return 0;
    const size_t n = dsa::topk_workspace_bytes(Tq, Tk, k);
    return n ? round_up(n) : 0;
}

DSA_EXPORT dsa_status_t dsa_topk(const float* scores, int64_t ld_scores, int Tq, int Tk,
                                 int64_t q_pos0, int k, int32_t* idx, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
    g_err[0] = 0;
    REQUIRE(Tq >= 0 && Tk >= 0 && q_pos0 >= 0, DSA_ERR_INVALID_ARG, "negative size or position");
    REQUIRE((int64_t)Tk >= q_pos0 + Tq, DSA_ERR_INVALID_ARG,
            "Tk (%d) must cover every query's prefix (q_pos0 + Tq = %lld)", Tk, (long long)(q_pos0 + Tq));
    REQUIRE(k >= 1 && k <= 8192, DSA_ERR_INVALID_ARG, "k must be in [1, 8192] (got %d)", k);
    REQUIRE_PTR(scores);
    REQUIRE_PTR4(idx);
    REQUIRE(ld_scores >= Tk && ld_scores % 4 == 0, DSA_ERR_INVALID_ARG,
            "ld_scores (%lld) must be >= Tk (%d) and a multiple of 4", (long long)ld_scores, Tk);
    REQUIRE_OPT_PTR(ws);
    // a workspace smaller than the size query is simply not used (single-pass rows)
    const size_t need = dsa::topk_workspace_bytes(Tq, Tk, k);
    void* use_ws = (ws && ws_bytes >= need && need) ? ws : nullptr;
    hipError_t e = dsa::launch_topk(scores, ld_scores, Tq, Tk, q_pos0, nullptr, k, idx, use_ws, stream);
    return e == hipSuccess ? DSA_OK : hip_fail(e, "top-k launch");
}

DSA_EXPORT size_t dsa_sparse_gqa_attn_workspace_size(int Tq, int k, int Hq, int d) {
    if (Tq <= 0 || k <= 0 || Hq <= 0 || d <= 0) return 0;
    return round_up(dsa::attn_partials_bytes(Tq, dsa::attn_num_splits(Tq, k), Hq, d));
}

namespace {

dsa_status_t run_attn(const void* q, const void* k, const void* v, dsa_dtype_t dtype, int n_kv,
                      const int32_t* block_table, int max_blocks, int block_size,
                      const int32_t* row_seq, const int32_t* seq_lens, const int32_t* idx, int Tq,
                      int topk, int Hq, int G, int d, float sm_scale, void* out, void* ws,
                      size_t ws_bytes, hipStream_t stream) {
    dsa::AttnArgs a;
    a.q = q; a.k = k; a.v = v; a.out = out; a.idx = idx; a.Tq = Tq; a.topk = topk; a.Hq = Hq;
    a.G = G; a.d = d; a.sm_scale = sm_scale; a.n_kv = n_kv; a.block_table = block_table;
    a.max_blocks = max_blocks; a.block_size = block_size; a.row_seq = row_seq;
    a.seq_lens = seq_lens; a.bf16 = dtype == DSA_BF16;
    int nsplit = dsa::attn_num_splits(Tq, topk);
    if (!ws || ws_bytes < dsa::attn_partials_bytes(Tq, nsplit, Hq, d)) nsplit = 1;
    hipError_t e = dsa::launch_sparse_attn(a, nsplit, static_cast<float*>(ws), stream);
    return e == hipSuccess ? DSA_OK : hip_fail(e, "attention launch");
}

}  // namespace

DSA_EXPORT dsa_status_t dsa_sparse_gqa_attn(const void* q, const void* k, const void* v,
                                            dsa_dtype_t dtype, int n_kv, const int32_t* block_table,
                                            int max_blocks, int block_size, const int32_t* row_seq,
                                            const int32_t* seq_lens, const int32_t* idx, int Tq,
                                            int topk, int Hq, int G, int d, float sm_scale,
                                            void* out, void* ws, size_t ws_bytes,
                                            hipStream_t stream) {
    g_err[0] = 0;
    dsa_status_t st = check_attn_shape(dtype, Hq, G, d, topk);
    if (st != DSA_OK) return st;
    REQUIRE(Tq >= 0 && n_kv >= 0, DSA_ERR_INVALID_ARG, "negative size (Tq=%d, n_kv=%d)", Tq, n_kv);
    REQUIRE_PTR(q); REQUIRE_PTR(k); REQUIRE_PTR(v); REQUIRE_PTR4(idx); REQUIRE_PTR(out);
    REQUIRE_OPT_PTR(ws);
    if (block_table) {
        REQUIRE_PTR4(block_table);
        REQUIRE_OPT_PTR4(row_seq);
        REQUIRE_OPT_PTR4(seq_lens);
        REQUIRE(max_blocks >= 1 && block_size >= 1, DSA_ERR_INVALID_ARG,
                "paged K/V needs max_blocks >= 1 and block_size >= 1 (got %d, %d)", max_blocks, block_size);
        REQUIRE((int64_t)n_kv * block_size < INT32_MAX, DSA_ERR_UNSUPPORTED,
                "paged cache holds too many tokens (%lld)", (long long)n_kv * block_size);
    }
    return run_attn(q, k, v, dtype, n_kv, block_table, max_blocks, block_size, row_seq, seq_lens,
                    idx, Tq, topk, Hq, G, d, sm_scale, out, ws, ws_bytes, stream);
}

namespace {

struct PrefillPlan {
    int chunk;
    int64_t Tk;
    int64_t ld;
    int S;                                     // samples per row: the most any chunk takes
    size_t scores_bytes, idx_bytes, index_bytes;
    size_t samples_bytes, tau_bytes, cnt_bytes, cand_bytes, flag_bytes, total;
};

// Relative cost of one union position of a 16-row block (gathered once, computed for all 16
// queries) against one selected (row, position) entry of the per-query attention, measured on
// gfx950 (8K-row chunks of the 128K layer): the union kernels break even with the per-query
// kernel at a union of about 28% of the selections.  A block takes the deduplicated attention
// when kDedupKappa * union < selections.
constexpr float kDedupKappa = 3.5f;

// The workspace holds one chunk's scores, its index sets and the indexer's scratch (sized for
// FP8, the larger of the two indexer paths), plus the candidate pipeline's buffers: samples,
// per-row bounds and counters, candidate lists and the fallback flag.  A chunk's sample count
// grows with the keys it sees until the candidate path ends (fused_sample_count < 0), so the
// sample buffer is sized for the longest prefix that still takes the path.
PrefillPlan plan_prefill(int Tq, int64_t q_pos0, int chunk_rows, int topk) {
    PrefillPlan p;
    p.chunk = (chunk_rows <= 0 || chunk_rows > Tq) ? Tq : chunk_rows;
    p.Tk = q_pos0 + Tq;
    p.ld = ld_for(p.Tk);
    const int64_t last_cand_tk = 64LL * dsa::kCandCap - 1;
    p.S = dsa::fused_sample_count((int)std::min<int64_t>(p.Tk, last_cand_tk));
    const int S = p.S > 0 ? p.S : 0;
    p.scores_bytes = round_up((size_t)p.chunk * p.ld * sizeof(float));
    p.idx_bytes = round_up((size_t)p.chunk * topk * sizeof(int32_t));
    p.index_bytes = indexer_ws_bytes(p.chunk, DSA_FP8_E4M3);
    p.samples_bytes = round_up((size_t)p.chunk * S * sizeof(float));
    p.tau_bytes = round_up((size_t)p.chunk * sizeof(uint32_t));
    p.cnt_bytes = round_up((size_t)p.chunk * sizeof(int32_t));
    p.cand_bytes = round_up((size_t)p.chunk * dsa::kCandCap * sizeof(uint2));
    p.flag_bytes = kAlign;
    p.total = p.scores_bytes + p.idx_bytes + p.index_bytes + p.samples_bytes + p.tau_bytes +
              p.cnt_bytes + p.cand_bytes + p.flag_bytes;
    return p;
}

struct PrefillBuffers {
    float* scores; int32_t* idx_ws; void* index_ws; float* samples; float* tau; int32_t* cnt;
    uint2* cand; int* fallback;
    int chunk; int S;                          // capacities: rows per chunk, samples per row
};

PrefillBuffers carve_prefill(void* ws, const PrefillPlan& plan) {
    PrefillBuffers b;
    char* wp = static_cast<char*>(ws);
    b.scores = reinterpret_cast<float*>(wp);                         wp += plan.scores_bytes;
    b.idx_ws = reinterpret_cast<int32_t*>(wp);                       wp += plan.idx_bytes;
    b.index_ws = wp;                                                 wp += plan.index_bytes;
    b.samples = reinterpret_cast<float*>(wp);                        wp += plan.samples_bytes;
    b.tau = reinterpret_cast<float*>(wp);                            wp += plan.tau_bytes;
    b.cnt = reinterpret_cast<int32_t*>(wp);                          wp += plan.cnt_bytes;
    b.cand = reinterpret_cast<uint2*>(wp);                           wp += plan.cand_bytes;
    b.fallback = reinterpret_cast<int*>(wp);
    b.chunk = plan.chunk;
    b.S = plan.S > 0 ? plan.S : 0;
    return b;
}

struct PrefillArgs {
    const void* q; const void* k; const void* v; dsa_dtype_t dtype;
    const void* q_idx; const float* q_scale; const float* w; const void* k_idx;
    const float* k_scale; dsa_dtype_t idx_dtype;
    int Hq, G, d, HI, dI, topk; float sm_scale;
    void* out; int32_t* idx_out;
};

// One sequence's prefill (arguments already checked): query rows q_pos0 .. q_pos0 + Tq - 1,
// keys 0 .. q_pos0 + Tq - 1, in chunks of at most b.chunk rows.  `first_cand` is true until a
// chunk of the call has taken the candidate path (the first one clears the counters).
dsa_status_t run_prefill(const PrefillArgs& a, int Tq, int64_t q_pos0, const PrefillBuffers& b,
                         bool& first_cand, hipStream_t stream) {
    const size_t qrow = (size_t)a.Hq * a.d * (a.dtype == DSA_BF16 ? 2 : 4);
    const size_t qirow = (size_t)a.HI * a.dI * (a.idx_dtype == DSA_FP8_E4M3 ? 1 : 4);
    const int topk = a.topk, HI = a.HI;
    // The candidate pipeline needs the resident FP8 indexer and a bounded candidate list;
    // other shapes run the indexer and top-k over full score rows.
    const bool cand_path = a.idx_dtype == DSA_FP8_E4M3 && HI <= 64 && topk <= dsa::kCandCap;
    const int64_t ld = ld_for(q_pos0 + Tq);
    for (int r0 = 0; r0 < Tq; r0 += b.chunk) {
        const int rows = (Tq - r0 < b.chunk) ? Tq - r0 : b.chunk;
        const int64_t pos0 = q_pos0 + r0;
        const int tk = (int)(pos0 + rows);                     // keys this chunk can see
        const void* qi_c = static_cast<const char*>(a.q_idx) + r0 * qirow;
        const float* qs_c = a.q_scale ? a.q_scale + r0 : nullptr;
        const float* w_c = a.w + (int64_t)r0 * HI;
        int32_t* idx_c = a.idx_out ? a.idx_out + (int64_t)r0 * topk : b.idx_ws;
        // short prefixes: streaming the full score rows costs less than the sample pass and
        // the per-row select (measured break-even near 40K keys)
        int S = cand_path && tk >= kCandMinKeys ? dsa::fused_sample_count(tk) : -1;
        if (S > b.S) S = -1;                                   // (cannot happen: S grows with tk)
        dsa_status_t st;
        hipError_t e = hipSuccess;
        if (tk <= topk) {
            // every row of the chunk keeps its whole prefix: the top-k writes 0..t without
            // reading scores, so none are computed
            e = dsa::launch_topk(b.scores, ld, rows, tk, pos0, nullptr, topk, idx_c, nullptr, stream);
            if (e != hipSuccess) return hip_fail(e, "top-k launch");
        } else if (S >= 0) {
            // sampled bound -> candidates at or above it -> exact select from the candidates;
            // a row whose candidates cannot give the exact answer raises the fallback flag,
            // and the two gated launches then redo the chunk over full score rows
            const auto* qi8 = static_cast<const uint8_t*>(qi_c);
            const auto* ki8 = static_cast<const uint8_t*>(a.k_idx);
            e = dsa::launch_index_fp8_sample(qi8, qs_c, w_c, ki8, a.k_scale, rows, tk, HI, pos0,
                                             b.samples, S, b.index_ws, stream);
            if (e == hipSuccess)
                e = dsa::launch_topk_bound(b.samples, S, rows, pos0, nullptr, 0, topk, b.tau, b.cnt,
                                           b.fallback, first_cand ? 1 : 0, stream);
            first_cand = false;
            if (e == hipSuccess)
                e = dsa::launch_index_fp8_candidates(qi8, qs_c, w_c, ki8, a.k_scale, rows, tk, HI,
                                                     pos0, b.tau, b.cnt, b.cand, dsa::kCandCap,
                                                     b.index_ws, stream);
            if (e == hipSuccess)
                e = dsa::launch_topk_select(b.cand, b.cnt, rows, pos0, nullptr, 0, topk, idx_c,
                                            b.fallback, stream);
            if (e == hipSuccess)
                e = dsa::launch_index_fp8(qi8, qs_c, w_c, ki8, a.k_scale, rows, tk, HI, pos0,
                                          b.scores, ld, b.index_ws, stream, b.fallback, true);
            if (e == hipSuccess)
                e = dsa::launch_topk(b.scores, ld, rows, tk, pos0, nullptr, topk, idx_c, nullptr,
                                     stream, b.fallback);
            if (e != hipSuccess) return hip_fail(e, "prefill selection launch");
        } else {
            st = run_indexer(qi_c, qs_c, w_c, a.k_idx, a.k_scale, a.idx_dtype, rows, tk, HI, a.dI,
                             pos0, b.scores, ld, b.index_ws, stream);
            if (st != DSA_OK) return st;
            e = dsa::launch_topk(b.scores, ld, rows, tk, pos0, nullptr, topk, idx_c, nullptr, stream);
            if (e != hipSuccess) return hip_fail(e, "top-k launch");
        }
        // Rows in 16-row blocks of whole prefixes (every row of the block keeps all of its
        // t + 1 positions) take the deduplicated attention: the block's union is its prefix
        // and needs no union kernel.  The union attention wins clearly only there: on the
        // workloads measured, other blocks' shared rows already hit in L2 for the per-query
        // kernel (dsa_sparse_gqa_attn_dedup offers the union for any selection).
        const void* q_c = static_cast<const char*>(a.q) + r0 * qrow;
        void* out_c = static_cast<char*>(a.out) + r0 * qrow;
        const int64_t lim = dsa::prefix_block_limit(q_pos0 + Tq, topk);
        const bool dedup = a.dtype == DSA_BF16 && a.Hq == 8 * a.G && a.d == 128 && pos0 < lim;
        if (dedup) {
            dsa::PrefixBlocks pb;
            pb.n = 1;
            pb.row0[0] = (int)-pos0;
            pb.kv0[0] = 0;
            pb.len[0] = (int)(q_pos0 + Tq);
            pb.blk0[0] = (int)(pos0 / dsa::kDedupRows);
            const int64_t hi = std::min<int64_t>(pos0 + rows, lim);
            pb.blk_start[0] = 0;
            pb.blk_start[1] = (int)((hi + dsa::kDedupRows - 1) / dsa::kDedupRows) - pb.blk0[0];
            dsa::AttnArgs at;
            at.q = q_c; at.k = a.k; at.v = a.v; at.out = out_c; at.idx = idx_c; at.Tq = rows;
            at.topk = topk; at.Hq = a.Hq; at.G = a.G; at.d = a.d; at.sm_scale = a.sm_scale;
            at.n_kv = tk; at.block_table = nullptr; at.max_blocks = 0; at.block_size = 0;
            at.row_seq = nullptr; at.seq_lens = nullptr; at.bf16 = 1;
            e = dsa::launch_dedup_prefix_attn(at, pb, stream);
            if (e != hipSuccess) return hip_fail(e, "prefix attention launch");
            if (pos0 + rows > lim) {
                at.pos0 = pos0;
                at.prefix_skip = lim;
                e = dsa::launch_sparse_attn(at, 1, nullptr, stream);
                if (e != hipSuccess) return hip_fail(e, "attention launch");
            }
            continue;
        }
        st = run_attn(q_c, a.k, a.v, a.dtype, tk, nullptr, 0, 0, nullptr, nullptr, idx_c, rows,
                      topk, a.Hq, a.G, a.d, a.sm_scale, out_c, nullptr, 0, stream);
        if (st != DSA_OK) return st;
    }
    return DSA_OK;
}

}  // namespace

DSA_EXPORT size_t dsa_sparse_gqa_attn_dedup_workspace_size(int Tq, int64_t q_pos0, int topk) {
    if (Tq <= 0 || q_pos0 < 0 || topk <= 0 || topk > dsa::kDedupMaxTopk) return 0;
    const size_t nb = (size_t)dsa::dedup_blocks(Tq, q_pos0);
    return round_up(nb * 3 * sizeof(int32_t)) + round_up(nb * dsa::kDedupRows * topk * 4) +
           round_up(nb * dsa::kDedupRows * topk * 2) + kAlign;
}

DSA_EXPORT dsa_status_t dsa_sparse_gqa_attn_dedup(const void* q, const void* k, const void* v,
                                                  int n_kv, const int32_t* idx, int Tq,
                                                  int64_t q_pos0, int topk, int Hq, int G, int d,
                                                  float sm_scale, int mode, void* out, void* ws,
                                                  size_t ws_bytes, hipStream_t stream) {
    g_err[0] = 0;
    dsa_status_t st = check_attn_shape(DSA_BF16, Hq, G, d, topk);
    if (st != DSA_OK) return st;
    REQUIRE(Tq >= 0 && n_kv >= 0 && q_pos0 >= 0, DSA_ERR_INVALID_ARG,
            "negative size or position (Tq=%d, n_kv=%d)", Tq, n_kv);
    REQUIRE(mode == 0 || mode == 1, DSA_ERR_INVALID_ARG, "mode must be 0 or 1 (got %d)", mode);
    REQUIRE(dsa::dedup_supported(Hq, G, d, topk, std::max(n_kv, 1), 1), DSA_ERR_UNSUPPORTED,
            "deduplicated attention needs Hq == 8 G, d == 128, topk <= %d and n_kv <= %d",
            dsa::kDedupMaxTopk, 32 * dsa::kDedupMaxWords);
    REQUIRE_PTR(q); REQUIRE_PTR(k); REQUIRE_PTR(v); REQUIRE_PTR4(idx); REQUIRE_PTR(out);
    if (Tq == 0) return DSA_OK;
    const size_t need = dsa_sparse_gqa_attn_dedup_workspace_size(Tq, q_pos0, topk);
    REQUIRE(ws && aligned16(ws) && ws_bytes >= need, DSA_ERR_WORKSPACE,
            "deduplicated attention needs %zu workspace bytes (got %zu%s)", need, ws_bytes,
            ws ? "" : ", ws is NULL");
    const size_t nb = (size_t)dsa::dedup_blocks(Tq, q_pos0);
    char* wp = static_cast<char*>(ws);
    int32_t* info = reinterpret_cast<int32_t*>(wp);   wp += round_up(nb * 3 * sizeof(int32_t));
    int32_t* list = reinterpret_cast<int32_t*>(wp);   wp += round_up(nb * dsa::kDedupRows * topk * 4);
    uint16_t* mask = reinterpret_cast<uint16_t*>(wp); wp += round_up(nb * dsa::kDedupRows * topk * 2);
    int* counter = reinterpret_cast<int*>(wp);
    hipError_t e = dsa::launch_fill_zero(reinterpret_cast<uint32_t*>(counter), 1, stream);
    if (e == hipSuccess)
        e = dsa::launch_dedup_union(idx, Tq, q_pos0, topk, n_kv, mode == 1 ? 0.f : kDedupKappa,
                                    info, list, mask, counter, stream);
    if (e != hipSuccess) return hip_fail(e, "dedup union launch");
    dsa::AttnArgs at;
    at.q = q; at.k = k; at.v = v; at.out = out; at.idx = idx; at.Tq = Tq; at.topk = topk;
    at.Hq = Hq; at.G = G; at.d = d; at.sm_scale = sm_scale; at.n_kv = n_kv;
    at.block_table = nullptr; at.max_blocks = 0; at.block_size = 0; at.row_seq = nullptr;
    at.seq_lens = nullptr; at.bf16 = 1;
    e = dsa::launch_dedup_attn(at, q_pos0, info, list, mask, stream);
    if (e != hipSuccess) return hip_fail(e, "dedup attention launch");
    at.dedup_info = info;
    at.pos0 = q_pos0;
    e = dsa::launch_sparse_attn(at, 1, nullptr, stream);
    return e == hipSuccess ? DSA_OK : hip_fail(e, "attention launch");
}

DSA_EXPORT size_t dsa_prefill_workspace_size(int Tq, int64_t q_pos0, int chunk_rows, int topk) {
    if (Tq <= 0 || q_pos0 < 0 || topk <= 0) return 0;
    return plan_prefill(Tq, q_pos0, chunk_rows, topk).total;
}

DSA_EXPORT size_t dsa_prefill_stats_offset(int Tq, int64_t q_pos0, int chunk_rows, int topk) {
    if (Tq <= 0 || q_pos0 < 0 || topk <= 0) return (size_t)-1;
    const PrefillPlan p = plan_prefill(Tq, q_pos0, chunk_rows, topk);
    return p.total - p.flag_bytes + sizeof(int);
}

DSA_EXPORT dsa_status_t dsa_prefill(const void* q, const void* k, const void* v, dsa_dtype_t dtype,
                                    const void* q_idx, const float* q_scale, const float* w,
                                    const void* k_idx, const float* k_scale,
                                    dsa_dtype_t idx_dtype, int Tq, int64_t q_pos0, int Hq, int G,
                                    int d, int HI, int dI, int topk, float sm_scale,
                                    int chunk_rows, void* out, int32_t* idx_out, void* ws,
                                    size_t ws_bytes, hipStream_t stream) {
    g_err[0] = 0;
    REQUIRE(Tq >= 0 && q_pos0 >= 0, DSA_ERR_INVALID_ARG, "negative size or position");
    REQUIRE(q_pos0 + Tq <= INT32_MAX - 4, DSA_ERR_UNSUPPORTED, "sequence too long");
    const int Tk = (int)(q_pos0 + Tq);
    dsa_status_t st = check_indexer(q_idx, q_scale, w, k_idx, k_scale, idx_dtype, Tq, Tk, HI, dI, q_pos0);
    if (st != DSA_OK) return st;
    st = check_attn_shape(dtype, Hq, G, d, topk);
    if (st != DSA_OK) return st;
    REQUIRE_PTR(q); REQUIRE_PTR(k); REQUIRE_PTR(v); REQUIRE_PTR(out);
    REQUIRE_OPT_PTR4(idx_out);
    if (Tq == 0) return DSA_OK;
    const PrefillPlan plan = plan_prefill(Tq, q_pos0, chunk_rows, topk);
    REQUIRE(ws && aligned16(ws) && ws_bytes >= plan.total, DSA_ERR_WORKSPACE,
            "prefill needs %zu workspace bytes (got %zu%s)", plan.total, ws_bytes,
            ws ? "" : ", ws is NULL");
    const PrefillArgs a{q, k, v, dtype, q_idx, q_scale, w, k_idx, k_scale, idx_dtype,
                        Hq, G, d, HI, dI, topk, sm_scale, out, idx_out};
    bool first_cand = true;
    return run_prefill(a, Tq, q_pos0, carve_prefill(ws, plan), first_cand, stream);
}

DSA_EXPORT dsa_status_t dsa_prefill_varlen(const void* q, const void* k, const void* v,
                                           dsa_dtype_t dtype, const void* q_idx,
                                           const float* q_scale, const float* w,
                                           const void* k_idx, const float* k_scale,
                                           dsa_dtype_t idx_dtype, const int32_t* cu_seqlens,
                                           int nseq, int Hq, int G, int d, int HI, int dI,
                                           int topk, float sm_scale, int chunk_rows, void* out,
                                           int32_t* idx_out, void* ws, size_t ws_bytes,
                                           hipStream_t stream) {
    g_err[0] = 0;
    REQUIRE(nseq >= 0, DSA_ERR_INVALID_ARG, "negative number of sequences (%d)", nseq);
    REQUIRE(cu_seqlens != nullptr, DSA_ERR_INVALID_ARG, "cu_seqlens is NULL");
    REQUIRE(cu_seqlens[0] == 0, DSA_ERR_INVALID_ARG, "cu_seqlens[0] must be 0 (got %d)",
            cu_seqlens[0]);
    int max_len = 0;
    for (int i = 0; i < nseq; ++i) {
        const int len = cu_seqlens[i + 1] - cu_seqlens[i];
        REQUIRE(cu_seqlens[i + 1] >= cu_seqlens[i], DSA_ERR_INVALID_ARG,
                "cu_seqlens must not decrease (entry %d: %d after %d)", i + 1, cu_seqlens[i + 1],
                cu_seqlens[i]);
        if (len > max_len) max_len = len;
    }
    const int T = cu_seqlens[nseq];
    REQUIRE(T <= INT32_MAX - 4, DSA_ERR_UNSUPPORTED, "batch too long");
    // the longest sequence fixes the shapes every check below needs
    dsa_status_t st = check_indexer(q_idx, q_scale, w, k_idx, k_scale, idx_dtype, max_len,
                                    max_len, HI, dI, 0);
    if (st != DSA_OK) return st;
    st = check_attn_shape(dtype, Hq, G, d, topk);
    if (st != DSA_OK) return st;
    REQUIRE_PTR(q); REQUIRE_PTR(k); REQUIRE_PTR(v); REQUIRE_PTR(out);
    REQUIRE_OPT_PTR4(idx_out);
    if (max_len == 0) return DSA_OK;
    const PrefillPlan plan = plan_prefill(max_len, 0, chunk_rows, topk);
    REQUIRE(ws && aligned16(ws) && ws_bytes >= plan.total, DSA_ERR_WORKSPACE,
            "varlen prefill needs %zu workspace bytes (got %zu%s)", plan.total, ws_bytes,
            ws ? "" : ", ws is NULL");
    const PrefillBuffers b = carve_prefill(ws, plan);
    const size_t qrow = (size_t)Hq * d * (dtype == DSA_BF16 ? 2 : 4);
    const size_t kvrow = (size_t)G * d * (dtype == DSA_BF16 ? 2 : 4);
    const size_t qirow = (size_t)HI * dI * (idx_dtype == DSA_FP8_E4M3 ? 1 : 4);
    const size_t kirow = (size_t)dI * (idx_dtype == DSA_FP8_E4M3 ? 1 : 4);
    // Runs of consecutive sequences of at most topk tokens (bf16, Hq == 8 G): every row keeps
    // its whole prefix, so no score is needed, and up to kMaxPrefixSegs of them share one
    // launch of the deduplicated prefix attention (and one launch writing their index lists):
    // the same blocks and arithmetic as dsa_prefill on each alone.  Longer sequences take the
    // chunk driver one by one.
    const bool batch_short = dtype == DSA_BF16 && Hq == 8 * G && d == 128;
    int run0 = -1;                                  // first sequence of the open run
    auto flush = [&](int i1) -> dsa_status_t {
        const int i0 = run0;
        run0 = -1;
        const int64_t R0 = cu_seqlens[i0];
        const int rows = cu_seqlens[i1] - cu_seqlens[i0];
        if (rows == 0) return DSA_OK;
        dsa::SeqStarts ss;
        dsa::PrefixBlocks pb;
        ss.n = pb.n = i1 - i0;
        pb.blk_start[0] = 0;
        for (int j = 0; j < ss.n; ++j) {
            const int st0 = cu_seqlens[i0 + j] - (int)R0;
            const int len = cu_seqlens[i0 + j + 1] - cu_seqlens[i0 + j];
            ss.start[j] = st0;
            pb.row0[j] = pb.kv0[j] = st0;
            pb.len[j] = len;
            pb.blk0[j] = 0;
            pb.blk_start[j + 1] = pb.blk_start[j] + (len + dsa::kDedupRows - 1) / dsa::kDedupRows;
        }
        ss.start[ss.n] = rows;
        hipError_t e = hipSuccess;
        if (idx_out) e = dsa::launch_prefix_idx(ss, topk, idx_out + R0 * topk, stream);
        if (e != hipSuccess) return hip_fail(e, "short-sequence index launch");
        dsa::AttnArgs a;
        a.q = static_cast<const char*>(q) + R0 * qrow;
        a.k = static_cast<const char*>(k) + R0 * kvrow;
        a.v = static_cast<const char*>(v) + R0 * kvrow;
        a.out = static_cast<char*>(out) + R0 * qrow;
        a.idx = nullptr; a.Tq = rows; a.topk = topk; a.Hq = Hq; a.G = G; a.d = d;
        a.sm_scale = sm_scale; a.n_kv = rows; a.block_table = nullptr; a.max_blocks = 0;
        a.block_size = 0; a.row_seq = nullptr; a.seq_lens = nullptr; a.bf16 = 1;
        e = dsa::launch_dedup_prefix_attn(a, pb, stream);
        return e == hipSuccess ? DSA_OK : hip_fail(e, "short-sequence attention launch");
    };
    bool first_cand = true;
    for (int i = 0; i < nseq; ++i) {
        const int64_t s0 = cu_seqlens[i];
        const int len = cu_seqlens[i + 1] - cu_seqlens[i];
        if (batch_short && len <= topk) {
            if (run0 < 0) run0 = i;
            if (i + 1 - run0 == dsa::kMaxPrefixSegs) {
                st = flush(i + 1);
                if (st != DSA_OK) return st;
            }
            continue;
        }
        if (run0 >= 0) {
            st = flush(i);
            if (st != DSA_OK) return st;
        }
        if (len == 0) continue;
        const PrefillArgs a{static_cast<const char*>(q) + s0 * qrow,
                            static_cast<const char*>(k) + s0 * kvrow,
                            static_cast<const char*>(v) + s0 * kvrow, dtype,
                            static_cast<const char*>(q_idx) + s0 * qirow,
                            q_scale ? q_scale + s0 : nullptr, w + s0 * HI,
                            static_cast<const char*>(k_idx) + s0 * kirow,
                            k_scale ? k_scale + s0 : nullptr, idx_dtype, Hq, G, d, HI, dI, topk,
                            sm_scale, static_cast<char*>(out) + s0 * qrow,
                            idx_out ? idx_out + s0 * topk : nullptr};
        st = run_prefill(a, len, 0, b, first_cand, stream);
        if (st != DSA_OK) return st;
    }
    if (run0 >= 0) return flush(nseq);
    return DSA_OK;
}

namespace {

struct DecodePlan {
    int64_t ld;
    int nsplit;
    int S;                                     // samples per sequence (candidate path), or -1
    size_t scores_bytes, idx_bytes, part_bytes, topk_bytes;
    size_t samples_bytes, tau_bytes, cnt_bytes, cand_bytes, flag_bytes, total;
};

// Scores of every sequence, index sets, attention partials, the segmented top-k's scratch,
// and the candidate pipeline's buffers (as for the prefill, one row per sequence).
DecodePlan plan_decode(int B, int max_blocks, int block_size, int topk, int Hq, int d) {
    DecodePlan p;
    const int max_len = (int)((int64_t)max_blocks * block_size);
    p.ld = ld_for(max_len);
    p.scores_bytes = round_up((size_t)B * p.ld * sizeof(float));
    p.idx_bytes = round_up((size_t)B * topk * sizeof(int32_t));
    p.nsplit = dsa::attn_num_splits(B, topk);
    p.part_bytes = round_up(dsa::attn_partials_bytes(B, p.nsplit, Hq, d));
    p.topk_bytes = round_up(dsa::topk_workspace_bytes(B, max_len, topk));
    p.S = max_len >= kCandMinKeys ? dsa::fused_sample_count(max_len) : -1;
    const int S = p.S > 0 ? p.S : 0;
    const bool cand = p.S > 0;
    p.samples_bytes = round_up((size_t)B * S * sizeof(float));
    p.tau_bytes = cand ? round_up((size_t)B * sizeof(float)) : 0;
    p.cnt_bytes = cand ? round_up((size_t)B * sizeof(int32_t)) : 0;
    p.cand_bytes = cand ? round_up((size_t)B * dsa::kCandCap * sizeof(uint2)) : 0;
    p.flag_bytes = cand ? kAlign : 0;
    p.total = p.scores_bytes + p.idx_bytes + p.part_bytes + p.topk_bytes + p.samples_bytes +
              p.tau_bytes + p.cnt_bytes + p.cand_bytes + p.flag_bytes;
    return p;
}

}  // namespace

DSA_EXPORT size_t dsa_decode_workspace_size(int B, int max_blocks, int block_size, int topk,
                                            int Hq, int d) {
    if (B <= 0 || max_blocks <= 0 || block_size <= 0 || topk <= 0 || Hq <= 0 || d <= 0) return 0;
    return plan_decode(B, max_blocks, block_size, topk, Hq, d).total;
}

DSA_EXPORT size_t dsa_decode_stats_offset(int B, int max_blocks, int block_size, int topk, int Hq,
                                          int d) {
    if (B <= 0 || max_blocks <= 0 || block_size <= 0 || topk <= 0 || Hq <= 0 || d <= 0) return (size_t)-1;
    const DecodePlan p = plan_decode(B, max_blocks, block_size, topk, Hq, d);
    return p.flag_bytes ? p.total - p.flag_bytes + sizeof(int) : (size_t)-1;
}

// Every argument check of the decode step except the workspace's (shared with the
// no-allocation entry point).
dsa_status_t dsa::decode_check_args(const void* q, const void* q_idx, const float* q_scale,
                                    const float* w, const void* kidx_cache,
                                    const float* kidx_scale, const void* k_cache,
                                    const void* v_cache, dsa_dtype_t dtype,
                                    const int32_t* block_table, const int32_t* seq_lens, int B,
                                    int num_blocks, int max_blocks, int block_size, int Hq, int G,
                                    int d, int HI, int dI, int topk, void* out,
                                    int32_t* idx_out) {
    g_err[0] = 0;
    REQUIRE(B >= 0 && num_blocks >= 0, DSA_ERR_INVALID_ARG, "negative size (B=%d, num_blocks=%d)", B, num_blocks);
    REQUIRE(max_blocks >= 1 && block_size >= 1, DSA_ERR_INVALID_ARG,
            "max_blocks and block_size must be >= 1 (got %d, %d)", max_blocks, block_size);
    REQUIRE((int64_t)max_blocks * block_size <= INT32_MAX - 4, DSA_ERR_UNSUPPORTED,
            "max_blocks * block_size too large");
    REQUIRE((int64_t)num_blocks * block_size < INT32_MAX, DSA_ERR_UNSUPPORTED,
            "paged cache holds too many tokens");
    REQUIRE(dI == 128, DSA_ERR_UNSUPPORTED, "decode indexer needs dI == 128 (got %d)", dI);
    REQUIRE(block_size == 64, DSA_ERR_UNSUPPORTED, "decode needs 64-token cache blocks (got %d)",
            block_size);
    REQUIRE(HI >= 1 && HI <= 128 && HI % 4 == 0, DSA_ERR_UNSUPPORTED,
            "decode indexer needs HI %% 4 == 0 and HI <= 128 (got %d)", HI);
    dsa_status_t st = check_attn_shape(dtype, Hq, G, d, topk);
    if (st != DSA_OK) return st;
    REQUIRE_PTR(q); REQUIRE_PTR(q_idx); REQUIRE_PTR4(q_scale); REQUIRE_PTR(w);
    REQUIRE_PTR(kidx_cache); REQUIRE_PTR4(kidx_scale); REQUIRE_PTR(k_cache); REQUIRE_PTR(v_cache);
    REQUIRE_PTR4(block_table); REQUIRE_PTR4(seq_lens); REQUIRE_PTR(out);
    REQUIRE_OPT_PTR4(idx_out);
    return DSA_OK;
}

DSA_EXPORT dsa_status_t dsa_decode(const void* q, const void* q_idx, const float* q_scale,
                                   const float* w, const void* kidx_cache, const float* kidx_scale,
                                   const void* k_cache, const void* v_cache, dsa_dtype_t dtype,
                                   const int32_t* block_table, const int32_t* seq_lens, int B,
                                   int num_blocks, int max_blocks, int block_size, int Hq, int G,
                                   int d, int HI, int dI, int topk, float sm_scale, void* out,
                                   int32_t* idx_out, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
    const dsa_status_t st = dsa::decode_check_args(q, q_idx, q_scale, w, kidx_cache, kidx_scale,
                                                   k_cache, v_cache, dtype, block_table, seq_lens,
                                                   B, num_blocks, max_blocks, block_size, Hq, G,
                                                   d, HI, dI, topk, out, idx_out);
    if (st != DSA_OK || B == 0) return st;
    const DecodePlan plan = plan_decode(B, max_blocks, block_size, topk, Hq, d);
    REQUIRE(ws && aligned16(ws) && ws_bytes >= plan.total, DSA_ERR_WORKSPACE,
            "decode needs %zu workspace bytes (got %zu%s)", plan.total, ws_bytes, ws ? "" : ", ws is NULL");
    char* wp = static_cast<char*>(ws);
    float* scores = reinterpret_cast<float*>(wp);                    wp += plan.scores_bytes;
    int32_t* idx_ws = reinterpret_cast<int32_t*>(wp);                wp += plan.idx_bytes;
    float* partials = reinterpret_cast<float*>(wp);                  wp += plan.part_bytes;
    void* topk_ws = plan.topk_bytes ? wp : nullptr;                  wp += plan.topk_bytes;
    float* samples = reinterpret_cast<float*>(wp);                   wp += plan.samples_bytes;
    float* tau = reinterpret_cast<float*>(wp);                       wp += plan.tau_bytes;
    int32_t* cnt = reinterpret_cast<int32_t*>(wp);                   wp += plan.cnt_bytes;
    uint2* cand = reinterpret_cast<uint2*>(wp);                      wp += plan.cand_bytes;
    int* fallback = reinterpret_cast<int*>(wp);
    int32_t* idx_c = idx_out ? idx_out : idx_ws;
    const int max_len = max_blocks * block_size;
    const auto* qi8 = static_cast<const uint8_t*>(q_idx);
    const auto* kc8 = static_cast<const uint8_t*>(kidx_cache);

    hipError_t e = hipSuccess;
    if (plan.S > 0 && HI <= 64 && topk <= dsa::kCandCap) {
        // sampled bound -> candidates at or above it -> exact select; if any sequence's
        // candidates cannot give the exact answer, the two gated launches redo the step over
        // full score rows (as in the prefill)
        e = dsa::launch_index_fp8_paged_sample(qi8, q_scale, w, kc8, kidx_scale, block_table,
                                               seq_lens, B, num_blocks, max_blocks, block_size,
                                               HI, samples, plan.S, stream);
        if (e == hipSuccess)
            e = dsa::launch_topk_bound(samples, plan.S, B, 0, seq_lens, max_len, topk, tau, cnt,
                                       fallback, 1, stream);
        if (e == hipSuccess)
            e = dsa::launch_index_fp8_paged_candidates(qi8, q_scale, w, kc8, kidx_scale,
                                                       block_table, seq_lens, B, num_blocks,
                                                       max_blocks, block_size, HI, tau, cnt,
                                                       cand, dsa::kCandCap, stream);
        if (e == hipSuccess)
            e = dsa::launch_topk_select(cand, cnt, B, 0, seq_lens, max_len, topk, idx_c, fallback,
                                        stream);
        if (e == hipSuccess)
            e = dsa::launch_index_fp8_paged(qi8, q_scale, w, kc8, kidx_scale, block_table,
                                            seq_lens, B, num_blocks, max_blocks, block_size, HI,
                                            scores, plan.ld, stream, fallback);
        if (e == hipSuccess)
            e = dsa::launch_topk(scores, plan.ld, B, max_len, 0, seq_lens, topk, idx_c, nullptr,
                                 stream, fallback);
        if (e != hipSuccess) return hip_fail(e, "decode selection launch");
    } else {
        e = dsa::launch_index_fp8_paged(qi8, q_scale, w, kc8, kidx_scale, block_table, seq_lens,
                                        B, num_blocks, max_blocks, block_size, HI, scores,
                                        plan.ld, stream);
        if (e != hipSuccess) return hip_fail(e, "decode indexer launch");
        e = dsa::launch_topk(scores, plan.ld, B, max_len, 0, seq_lens, topk, idx_c, topk_ws, stream);
        if (e != hipSuccess) return hip_fail(e, "decode top-k launch");
    }
    return run_attn(q, k_cache, v_cache, dtype, num_blocks, block_table, max_blocks, block_size,
                    nullptr, seq_lens, idx_c, B, topk, Hq, G, d, sm_scale, out, partials,
                    plan.part_bytes, stream);
}

DSA_EXPORT dsa_status_t dsa_quantize_e4m3(const void* x, dsa_dtype_t x_dtype, int T, int n,
                                          uint8_t* codes, float* scale, hipStream_t stream) {
    g_err[0] = 0;
    REQUIRE(T >= 0 && n >= 1, DSA_ERR_INVALID_ARG, "bad size (T=%d, n=%d)", T, n);
    REQUIRE(x_dtype == DSA_F32 || x_dtype == DSA_BF16, DSA_ERR_UNSUPPORTED,
            "quantisation input must be F32 or BF16 (got %d)", (int)x_dtype);
    if (T == 0) return DSA_OK;
    REQUIRE_PTR4(x); REQUIRE_PTR4(scale);
    REQUIRE(codes != nullptr, DSA_ERR_INVALID_ARG, "codes is NULL");
    const hipError_t e = dsa::launch_quantize_e4m3(x, x_dtype == DSA_BF16, T, n, codes, scale, stream);
    return e == hipSuccess ? DSA_OK : hip_fail(e, "quantisation launch");
}

DSA_EXPORT dsa_status_t dsa_cache_append(const void* k_new, const void* v_new, dsa_dtype_t dtype,
                                         const void* kidx_new, dsa_dtype_t kidx_dtype,
                                         const int32_t* positions, const int32_t* block_table,
                                         int B, int num_blocks, int max_blocks, int block_size,
                                         int G, int d, int dI, void* k_cache, void* v_cache,
                                         uint8_t* kidx_cache, float* kidx_scale,
                                         hipStream_t stream) {
    g_err[0] = 0;
    REQUIRE(B >= 0 && num_blocks >= 0 && max_blocks >= 1 && block_size >= 1, DSA_ERR_INVALID_ARG,
            "bad size (B=%d, num_blocks=%d, max_blocks=%d, block_size=%d)", B, num_blocks,
            max_blocks, block_size);
    REQUIRE(dtype == DSA_BF16 || dtype == DSA_F32, DSA_ERR_UNSUPPORTED,
            "K/V dtype must be BF16 or F32 (got %d)", (int)dtype);
    REQUIRE(kidx_dtype == DSA_F32 || kidx_dtype == DSA_BF16, DSA_ERR_UNSUPPORTED,
            "indexer key input must be F32 or BF16 (got %d)", (int)kidx_dtype);
    REQUIRE(G >= 1 && d >= 1 && dI >= 1, DSA_ERR_INVALID_ARG, "bad head sizes (G=%d, d=%d, dI=%d)",
            G, d, dI);
    const int64_t row_bytes = (int64_t)G * d * (dtype == DSA_BF16 ? 2 : 4);
    REQUIRE(row_bytes % 16 == 0 && row_bytes <= INT32_MAX, DSA_ERR_UNSUPPORTED,
            "a K/V row (G * d elements) must be a multiple of 16 bytes");
    REQUIRE((int64_t)max_blocks * block_size <= INT32_MAX, DSA_ERR_UNSUPPORTED,
            "max_blocks * block_size too large");
    if (B == 0) return DSA_OK;
    REQUIRE_PTR(k_new); REQUIRE_PTR(v_new); REQUIRE_PTR4(kidx_new); REQUIRE_PTR4(positions);
    REQUIRE_PTR4(block_table); REQUIRE_PTR(k_cache); REQUIRE_PTR(v_cache);
    REQUIRE_PTR4(kidx_scale);
    REQUIRE(kidx_cache != nullptr, DSA_ERR_INVALID_ARG, "kidx_cache is NULL");
    const hipError_t e = dsa::launch_cache_append(
        k_new, v_new, (int)row_bytes, kidx_new, kidx_dtype == DSA_BF16, dI, positions, block_table,
        B, num_blocks, max_blocks, block_size, k_cache, v_cache, kidx_cache, kidx_scale, stream);
    return e == hipSuccess ? DSA_OK : hip_fail(e, "cache append launch");
}

namespace {

dsa_status_t check_index_at(const void* q_idx, const float* q_scale, const float* w,
                            const void* k_idx, const float* k_scale, dsa_dtype_t idx_dtype,
                            int Tq, int Tk, int HI, int dI, const int32_t* idx, int topk,
                            int max_heads) {
    REQUIRE(Tq >= 0 && Tk >= 0 && topk >= 1, DSA_ERR_INVALID_ARG,
            "bad size (Tq=%d, Tk=%d, topk=%d)", Tq, Tk, topk);
    REQUIRE(idx_dtype == DSA_FP8_E4M3, DSA_ERR_UNSUPPORTED,
            "the training-side indexer takes FP8 inputs (got dtype %d)", (int)idx_dtype);
    REQUIRE(dI == 128, DSA_ERR_UNSUPPORTED, "FP8 indexer needs dI == 128 (got %d)", dI);
    REQUIRE(HI >= 1 && HI <= max_heads, DSA_ERR_UNSUPPORTED, "HI must be 1..%d (got %d)",
            max_heads, HI);
    REQUIRE_PTR(q_idx); REQUIRE_PTR4(q_scale); REQUIRE_PTR4(w); REQUIRE_PTR(k_idx);
    REQUIRE_PTR4(k_scale); REQUIRE_PTR4(idx);
    return DSA_OK;
}

}  // namespace

DSA_EXPORT dsa_status_t dsa_index_scores_at(const void* q_idx, const float* q_scale,
                                            const float* w, const void* k_idx,
                                            const float* k_scale, dsa_dtype_t idx_dtype, int Tq,
                                            int Tk, int HI, int dI, const int32_t* idx, int topk,
                                            float* vals, hipStream_t stream) {
    g_err[0] = 0;
    dsa_status_t st = check_index_at(q_idx, q_scale, w, k_idx, k_scale, idx_dtype, Tq, Tk, HI, dI,
                                     idx, topk, 128);
    if (st != DSA_OK) return st;
    REQUIRE_PTR4(vals);
    const hipError_t e = dsa::launch_index_at(static_cast<const uint8_t*>(q_idx), q_scale, w,
                                              static_cast<const uint8_t*>(k_idx), k_scale, Tq, Tk,
                                              HI, idx, topk, vals, stream);
    return e == hipSuccess ? DSA_OK : hip_fail(e, "indexer-at launch");
}

namespace {

// Chunks of the staged indexer backward: at most 1024 rows (a 32-word row bitmask per key)
// and 1 GiB of staged dk^I contributions (512 bytes per selected entry).
struct IxBwdPlan {
    int chunk;
    size_t stg_bytes, mask_bytes, offs_bytes, list_bytes, dup_bytes, total;
};

IxBwdPlan plan_ix_bwd(int Tq, int Tk, int topk) {
    IxBwdPlan p;
    const size_t per_row = (size_t)topk * 128 * sizeof(float);
    int64_t c = (int64_t)((size_t(1) << 30) / per_row) / 32 * 32;
    c = std::max<int64_t>(32, std::min<int64_t>(c, 1024));
    const int64_t tq32 = ((int64_t)Tq + 31) / 32 * 32;
    p.chunk = (int)std::min<int64_t>(c, tq32);
    p.stg_bytes = round_up((size_t)p.chunk * per_row);
    p.mask_bytes = round_up((size_t)Tk * (p.chunk / 32) * sizeof(uint32_t));
    p.offs_bytes = round_up(((size_t)Tk + 1 + ((size_t)Tk + 255) / 256) * sizeof(int32_t));
    p.list_bytes = round_up((size_t)p.chunk * topk * sizeof(int32_t));
    p.dup_bytes = round_up((size_t)p.chunk * topk);
    p.total = p.stg_bytes + p.mask_bytes + p.offs_bytes + p.list_bytes + p.dup_bytes;
    return p;
}

}  // namespace

DSA_EXPORT size_t dsa_index_scores_at_bwd_workspace_size(int Tq, int Tk, int HI, int topk) {
    if (Tq <= 0 || Tk <= 0 || topk <= 0 || !dsa::index_at_bwd_stages(HI)) return 0;
    return plan_ix_bwd(Tq, Tk, topk).total;
}

DSA_EXPORT dsa_status_t dsa_index_scores_at_bwd(const void* q_idx, const float* q_scale,
                                                const float* w, const void* k_idx,
                                                const float* k_scale, dsa_dtype_t idx_dtype,
                                                int Tq, int Tk, int HI, int dI,
                                                const int32_t* idx, int topk, const float* g,
                                                float* dq_idx, float* dw, float* dk_idx,
                                                void* ws, size_t ws_bytes, hipStream_t stream) {
    g_err[0] = 0;
    dsa_status_t st = check_index_at(q_idx, q_scale, w, k_idx, k_scale, idx_dtype, Tq, Tk, HI, dI,
                                     idx, topk, 64);
    if (st != DSA_OK) return st;
    REQUIRE_PTR4(g); REQUIRE_PTR(dq_idx); REQUIRE_PTR4(dw); REQUIRE_PTR(dk_idx);
    const auto* qi8 = static_cast<const uint8_t*>(q_idx);
    const auto* ki8 = static_cast<const uint8_t*>(k_idx);
    if (!ws) {                                     // atomic adds straight into dk_idx
        REQUIRE(ws_bytes == 0, DSA_ERR_WORKSPACE, "ws is NULL but ws_bytes is %zu", ws_bytes);
        const hipError_t e = dsa::launch_index_at_bwd(qi8, q_scale, w, ki8, k_scale, Tq, Tk, HI,
                                                      idx, topk, g, dq_idx, dw, dk_idx, stream);
        return e == hipSuccess ? DSA_OK : hip_fail(e, "indexer backward launch");
    }
    REQUIRE(dsa::index_at_bwd_stages(HI), DSA_ERR_UNSUPPORTED,
            "the staged indexer backward needs HI a multiple of 16 (got %d); pass ws = NULL", HI);
    if (Tq == 0) return DSA_OK;
    const IxBwdPlan plan = plan_ix_bwd(Tq, Tk, topk);
    REQUIRE(aligned16(ws) && ws_bytes >= plan.total, DSA_ERR_WORKSPACE,
            "the staged indexer backward needs %zu workspace bytes (got %zu)", plan.total, ws_bytes);
    char* wp = static_cast<char*>(ws);
    float* stg = reinterpret_cast<float*>(wp);              wp += plan.stg_bytes;
    uint32_t* mask = reinterpret_cast<uint32_t*>(wp);       wp += plan.mask_bytes;
    int32_t* offs = reinterpret_cast<int32_t*>(wp);         wp += plan.offs_bytes;
    int32_t* list = reinterpret_cast<int32_t*>(wp);         wp += plan.list_bytes;
    uint8_t* dup = reinterpret_cast<uint8_t*>(wp);
    for (int r0 = 0; r0 < Tq; r0 += plan.chunk) {
        const int rows = std::min(plan.chunk, Tq - r0);
        hipError_t e = dsa::launch_index_at_bwd(qi8, q_scale, w, ki8, k_scale, rows, Tk, HI, idx,
                                                topk, g, dq_idx, dw, dk_idx, stream, r0, stg);
        if (e == hipSuccess && Tk > 0)
            e = dsa::launch_stage_reduce(idx, r0, rows, topk, Tk, 1, stg, mask, offs, list, dup,
                                         dk_idx, nullptr, stream, 128);
        if (e != hipSuccess) return hip_fail(e, "indexer backward launch");
    }
    return DSA_OK;
}

DSA_EXPORT dsa_status_t dsa_sparse_gqa_attn_lse(const void* q, const void* k, const void* v,
                                                dsa_dtype_t dtype, int n_kv, const int32_t* idx,
                                                int Tq, int topk, int Hq, int G, int d,
                                                float sm_scale, void* out, float* lse, void* ws,
                                                size_t ws_bytes, hipStream_t stream) {
    g_err[0] = 0;
    dsa_status_t st = check_attn_shape(dtype, Hq, G, d, topk);
    if (st != DSA_OK) return st;
    REQUIRE(Tq >= 0 && n_kv >= 0, DSA_ERR_INVALID_ARG, "negative size (Tq=%d, n_kv=%d)", Tq, n_kv);
    REQUIRE_PTR(q); REQUIRE_PTR(k); REQUIRE_PTR(v); REQUIRE_PTR4(idx); REQUIRE_PTR(out);
    REQUIRE_PTR4(lse); REQUIRE_OPT_PTR(ws);
    dsa::AttnArgs a;
    a.q = q; a.k = k; a.v = v; a.out = out; a.idx = idx; a.Tq = Tq; a.topk = topk; a.Hq = Hq;
    a.G = G; a.d = d; a.sm_scale = sm_scale; a.n_kv = n_kv; a.block_table = nullptr;
    a.max_blocks = 0; a.block_size = 0; a.row_seq = nullptr; a.seq_lens = nullptr;
    a.bf16 = dtype == DSA_BF16; a.lse = lse;
    int nsplit = dsa::attn_num_splits(Tq, topk);
    if (!ws || ws_bytes < dsa::attn_partials_bytes(Tq, nsplit, Hq, d)) nsplit = 1;
    const hipError_t e = dsa::launch_sparse_attn(a, nsplit, static_cast<float*>(ws), stream);
    return e == hipSuccess ? DSA_OK : hip_fail(e, "attention launch");
}

namespace {

// The staged (deterministic) backward works on chunks of query rows whose dK / dV
// contributions (1 KiB per selected entry and KV group) fit this many bytes.
constexpr size_t kStageBudget = size_t(4) << 30;

struct BwdPlan {
    int chunk;
    size_t stg_bytes, mask_bytes, offs_bytes, list_bytes, dup_bytes, total;
};

BwdPlan plan_bwd(int Tq, int topk, int G, int n_kv) {
    BwdPlan p;
    const size_t per_row = (size_t)topk * G * 256 * sizeof(float);
    int64_t c = (int64_t)(kStageBudget / per_row) / 32 * 32;
    if (c < 32) c = 32;
    const int64_t tq32 = ((int64_t)Tq + 31) / 32 * 32;
    p.chunk = (int)std::min<int64_t>(c, tq32);
    p.stg_bytes = round_up((size_t)p.chunk * per_row);
    p.mask_bytes = round_up((size_t)n_kv * (p.chunk / 32) * sizeof(uint32_t));
    p.offs_bytes = round_up(((size_t)n_kv + 1 + ((size_t)n_kv + 255) / 256) * sizeof(int32_t));
    p.list_bytes = round_up((size_t)p.chunk * topk * sizeof(int32_t));
    p.dup_bytes = round_up((size_t)p.chunk * topk);
    p.total = p.stg_bytes + p.mask_bytes + p.offs_bytes + p.list_bytes + p.dup_bytes;
    return p;
}

}  // namespace

DSA_EXPORT size_t dsa_sparse_gqa_attn_bwd_workspace_size(int Tq, int topk, int G, int n_kv) {
    if (Tq <= 0 || topk <= 0 || G <= 0 || n_kv <= 0) return 0;
    return plan_bwd(Tq, topk, G, n_kv).total;
}

DSA_EXPORT dsa_status_t dsa_sparse_gqa_attn_bwd(const void* q, const void* k, const void* v,
                                                dsa_dtype_t dtype, int n_kv, const int32_t* idx,
                                                int Tq, int topk, int Hq, int G, int d,
                                                float sm_scale, const void* out,
                                                const void* dout, const float* lse, void* dq,
                                                float* dk, float* dv, const float* vals,
                                                float* kl, float* dI, void* ws, size_t ws_bytes,
                                                hipStream_t stream) {
    g_err[0] = 0;
    dsa_status_t st = check_attn_shape(dtype, Hq, G, d, topk);
    if (st != DSA_OK) return st;
    REQUIRE(dtype == DSA_BF16, DSA_ERR_UNSUPPORTED, "the attention backward takes BF16 (got %d)",
            (int)dtype);
    REQUIRE(Tq >= 0 && n_kv >= 0, DSA_ERR_INVALID_ARG, "negative size (Tq=%d, n_kv=%d)", Tq, n_kv);
    REQUIRE_PTR(q); REQUIRE_PTR(k); REQUIRE_PTR(v); REQUIRE_PTR4(idx); REQUIRE_PTR(out);
    REQUIRE_PTR(dout); REQUIRE_PTR4(lse); REQUIRE_PTR(dq); REQUIRE_PTR4(dk); REQUIRE_PTR4(dv);
    if (vals) {
        REQUIRE(topk <= 2048, DSA_ERR_UNSUPPORTED,
                "the fused indexer loss takes topk <= 2048 (got %d)", topk);
        REQUIRE_PTR4(vals); REQUIRE_PTR4(kl); REQUIRE_PTR4(dI);
    }
    dsa::AttnBwdArgs a{q, k, v, out, dout, lse, idx, Tq, topk, Hq, G, n_kv, sm_scale,
                       dq, dk, dv, vals, vals ? kl : nullptr, vals ? dI : nullptr};
    if (!ws) {                                     // atomic adds straight into dk / dv
        REQUIRE(ws_bytes == 0, DSA_ERR_WORKSPACE, "ws is NULL but ws_bytes is %zu", ws_bytes);
        const hipError_t e = dsa::launch_sparse_attn_bwd(a, stream);
        return e == hipSuccess ? DSA_OK : hip_fail(e, "attention backward launch");
    }
    if (Tq == 0 || n_kv == 0) {
        const hipError_t e = dsa::launch_sparse_attn_bwd(a, stream);   // dq (zeros), kl, dI
        return e == hipSuccess ? DSA_OK : hip_fail(e, "attention backward launch");
    }
    const BwdPlan plan = plan_bwd(Tq, topk, G, n_kv);
    REQUIRE(aligned16(ws) && ws_bytes >= plan.total, DSA_ERR_WORKSPACE,
            "the staged attention backward needs %zu workspace bytes (got %zu)", plan.total,
            ws_bytes);
    char* wp = static_cast<char*>(ws);
    float* stg = reinterpret_cast<float*>(wp);              wp += plan.stg_bytes;
    uint32_t* mask = reinterpret_cast<uint32_t*>(wp);       wp += plan.mask_bytes;
    int32_t* offs = reinterpret_cast<int32_t*>(wp);         wp += plan.offs_bytes;
    int32_t* list = reinterpret_cast<int32_t*>(wp);         wp += plan.list_bytes;
    uint8_t* dup = reinterpret_cast<uint8_t*>(wp);
    for (int r0 = 0; r0 < Tq; r0 += plan.chunk) {
        const int rows = std::min(plan.chunk, Tq - r0);
        a.r0 = r0;
        a.Tq = rows;
        a.stg = stg;
        hipError_t e = dsa::launch_sparse_attn_bwd(a, stream);
        if (e == hipSuccess)
            e = dsa::launch_stage_reduce(idx, r0, rows, topk, n_kv, G, stg, mask, offs, list, dup, dk,
                                         dv, stream);
        if (e != hipSuccess) return hip_fail(e, "attention backward launch");
    }
    return DSA_OK;
}

// ---- Dense warm-up stage (report section 2.3.3; review page, dense warm-up loss) ----

DSA_EXPORT dsa_status_t dsa_indexer_warmup_kl(const void* q, const void* k, dsa_dtype_t dtype,
                                              int Tq, int Tk, int64_t q_pos0, int Hq, int G,
                                              int d, float sm_scale, const float* lse,
                                              float* scores, int64_t ld_scores, float* kl,
                                              hipStream_t stream) {
    g_err[0] = 0;
    REQUIRE(dtype == DSA_BF16, DSA_ERR_UNSUPPORTED, "the warm-up loss takes BF16 q and K (got %d)",
            (int)dtype);
    REQUIRE(d == 128, DSA_ERR_UNSUPPORTED, "head size d must be 128 (got %d)", d);
    REQUIRE(G >= 1 && Hq >= 1 && Hq % G == 0, DSA_ERR_INVALID_ARG,
            "Hq (%d) must be a positive multiple of G (%d)", Hq, G);
    REQUIRE(dsa::warmup_kl_supported(Hq, G), DSA_ERR_UNSUPPORTED,
            "the warm-up loss takes Hq/G in {1, 2, 4, 8, 16} with G * max(1, Hq/G/4) <= 8 "
            "(got Hq=%d, G=%d)", Hq, G);
    REQUIRE(Tq >= 0 && Tk >= 0 && q_pos0 >= 0, DSA_ERR_INVALID_ARG, "negative size or position");
    REQUIRE((int64_t)Tk >= q_pos0 + Tq, DSA_ERR_INVALID_ARG,
            "Tk (%d) must cover every query's prefix (q_pos0 + Tq = %lld)", Tk,
            (long long)(q_pos0 + Tq));
    REQUIRE(ld_scores >= Tk, DSA_ERR_INVALID_ARG, "ld_scores (%lld) must be >= Tk (%d)",
            (long long)ld_scores, Tk);
    REQUIRE_PTR(q); REQUIRE_PTR(k); REQUIRE_PTR4(scores); REQUIRE_OPT_PTR4(lse); REQUIRE_PTR4(kl);
    const hipError_t e = dsa::launch_warmup_kl(static_cast<const uint16_t*>(q),
                                               static_cast<const uint16_t*>(k), Tq, Tk, q_pos0, Hq,
                                               G, sm_scale, lse, scores, ld_scores, kl, stream);
    return e == hipSuccess ? DSA_OK : hip_fail(e, "warm-up loss launch");
}

DSA_EXPORT size_t dsa_index_scores_bwd_dense_workspace_size(int Tq, int Tk, int HI) {
    if (Tq <= 0 || Tk <= 0 || HI <= 0 || HI % 16 || HI > 64) return 0;
    return round_up(dsa::plan_warmup_bwd(Tq, Tk, HI).total);
}

DSA_EXPORT dsa_status_t dsa_index_scores_bwd_dense(const void* q_idx, const float* q_scale,
                                                   const float* w, const void* k_idx,
                                                   const float* k_scale, dsa_dtype_t idx_dtype,
                                                   int Tq, int Tk, int HI, int dI, int64_t q_pos0,
                                                   const float* g, int64_t ld_g, float* dq_idx,
                                                   float* dw, float* dk_idx, void* ws,
                                                   size_t ws_bytes, hipStream_t stream) {
    g_err[0] = 0;
    REQUIRE(idx_dtype == DSA_FP8_E4M3, DSA_ERR_UNSUPPORTED,
            "the training-side indexer takes FP8 inputs (got dtype %d)", (int)idx_dtype);
    REQUIRE(dI == 128, DSA_ERR_UNSUPPORTED, "FP8 indexer needs dI == 128 (got %d)", dI);
    REQUIRE(HI >= 16 && HI <= 64 && HI % 16 == 0, DSA_ERR_UNSUPPORTED,
            "the dense indexer backward takes HI in {16, 32, 48, 64} (got %d)", HI);
    REQUIRE(Tq >= 0 && Tk >= 0 && q_pos0 >= 0, DSA_ERR_INVALID_ARG, "negative size or position");
    REQUIRE((int64_t)Tk >= q_pos0 + Tq, DSA_ERR_INVALID_ARG,
            "Tk (%d) must cover every query's prefix (q_pos0 + Tq = %lld)", Tk,
            (long long)(q_pos0 + Tq));
    REQUIRE(ld_g >= Tk, DSA_ERR_INVALID_ARG, "ld_g (%lld) must be >= Tk (%d)", (long long)ld_g, Tk);
    REQUIRE_PTR(q_idx); REQUIRE_PTR4(q_scale); REQUIRE_PTR4(w); REQUIRE_PTR(k_idx);
    REQUIRE_PTR4(k_scale); REQUIRE_PTR4(g); REQUIRE_PTR(dq_idx); REQUIRE_PTR4(dw);
    REQUIRE_PTR(dk_idx);
    if (Tq == 0) return DSA_OK;
    const size_t need = round_up(dsa::plan_warmup_bwd(Tq, Tk, HI).total);
    REQUIRE(ws && aligned16(ws) && ws_bytes >= need, DSA_ERR_WORKSPACE,
            "the dense indexer backward needs %zu workspace bytes (got %zu%s)", need, ws_bytes,
            ws ? "" : ", ws is NULL");
    const hipError_t e = dsa::launch_warmup_ix_bwd(
        static_cast<const uint8_t*>(q_idx), q_scale, w, static_cast<const uint8_t*>(k_idx), k_scale,
        Tq, Tk, HI, q_pos0, g, ld_g, dq_idx, dw, dk_idx, ws, stream);
    return e == hipSuccess ? DSA_OK : hip_fail(e, "dense indexer backward launch");
}
