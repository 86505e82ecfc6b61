// topk.hip -- deterministic per-row Top-k for gfx950.
//
// Omega_t = the min(k, t+1) positions s <= t with the largest I[t,s] (xllm-io
// review page "核心公式", second formula), equal scores going to the lower
// position so that the selection is deterministic (Keye-VL-2.0 report section
// 5.2.1), listed in ascending position order.
//
// One workgroup of 1024 threads owns a row; scores are compared through an
// order-preserving 32-bit key (-0 and +0 map to the same key).
//   1. A sample of the row (n / 512 runs, 16 to 256, of 16 contiguous scores: about 1/32
//      of the row) gives, by two
//      radix digits of a select in LDS, a key that is a lower bound for the k-th
//      largest with high probability (the sample rank is padded by about 3
//      sigma, the bound is the low edge of that sample key's bin).
//   2. One pass over the row copies every score at or above that bound, with
//      its position, into LDS in position order (block-wide prefix sums), with
//      two steps of loads in flight; the first two are issued before step 1.
//   3. If that candidate set holds at least k and fits in LDS, an exact radix
//      select among the candidates finds the k-th largest key and how many of
//      the keys equal to it to take; an ordered compaction of the candidates
//      then writes the selection directly in ascending position order, ties
//      resolved to the lower positions.
//   4. Otherwise (the sample misjudged, or too many ties) the same exact select
//      and compaction run over the row in global memory: correct for every
//      input, only slower.
// Radix selects place their first digit at the top set bit of (max - min) of
// the keys involved, so the bins spread over the values actually present.
// Rows with t + 1 <= k need no selection and read nothing (they take 0..t).
#include <cfloat>

#include "device_common.h"
#include "internal.h"

namespace dsa {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(v, o, 64);
        if (lane >= o) v += y;
    }
    return v;
}

// Exclusive prefix sum over the workgroup in thread order; *total gets the sum.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t incl = wave_incl_scan(v, lane);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        uint32_t x = lane < kTopkWaves ? wsum[lane] : 0u;
        x = wave_incl_scan(x, lane);
        if (lane < kTopkWaves) wsum[kTopkWaves + lane] = x;
    }
    __syncthreads();
    const uint32_t base = wave > 0 ? wsum[kTopkWaves + wave - 1] : 0u;
    *total = wsum[2 * kTopkWaves - 1];
    __syncthreads();
    return base + incl - v;
}

__device__ __forceinline__ uint32_t block_reduce_minmax(uint32_t mn, uint32_t mx, uint32_t* red,
                                                        uint32_t* out_max) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        mn = min(mn, (uint32_t)__shfl_xor(mn, o, 64));
        mx = max(mx, (uint32_t)__shfl_xor(mx, o, 64));
    }
    if (lane == 0) { red[wave] = mn; red[kTopkWaves + wave] = mx; }
    __syncthreads();
    uint32_t a = red[0], b = red[kTopkWaves];
    for (int i = 1; i < kTopkWaves; ++i) { a = min(a, red[i]); b = max(b, red[kTopkWaves + i]); }
    __syncthreads();
    *out_max = b;
    return a;
}

// Four consecutive elements starting at i (multiple of 4); missing ones read as 0.
__device__ __forceinline__ void load4(const float* __restrict__ src, int64_t i, int64_t n,
                                      float v[4]) {
    if (i + 3 < n) {
        const float4 x = *reinterpret_cast<const float4*>(src + i);
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    } else {
        for (int e = 0; e < 4; ++e) v[e] = (i + e < n) ? src[i + e] : 0.f;
    }
}

// Range of the keys get(0..m).
template <class Get>
__device__ __forceinline__ void key_range(Get get, int64_t m, uint32_t* red, uint32_t& kmin,
                                          uint32_t& kmax) {
    uint32_t mn = 0xffffffffu, mx = 0u;
    for (int64_t i = threadIdx.x; i < m; i += kTopkThreads) {
        const uint32_t k = get(i);
        mn = min(mn, k);
        mx = max(mx, k);
    }
    kmin = block_reduce_minmax(mn, mx, red, &kmax);
}

// Exact select of the R-th largest (1 <= R <= m) of the keys get(0..m), all in
// [kmin, kmax].  On return an element is above the threshold iff
// ((key - kmin) & mask) > prefix and tied with it iff == prefix; `need` of the
// tied elements complete the R.  Stopped after max_passes digits, kmin + prefix
// is still a lower bound for the R-th largest key (the low edge of its bin).
// A pass is one histogram of the digit over the elements still in the running, then wave 0
// alone scans the bins from the top (32 per lane) and finds the bin holding the need-th
// element: two barriers a pass.  With hist2 (a second kBins buffer) the next pass's bins are
// cleared while this pass builds its own; without it, a third barrier separates the clearing.
template <class Get>
__device__ void radix_select(Get get, int64_t m, uint32_t R, uint32_t kmin, uint32_t kmax,
                             uint32_t* hist, uint32_t* hist2, uint32_t* sh, uint32_t& prefix,
                             uint32_t& mask, uint32_t& need, int max_passes = 32) {
    const int tid = threadIdx.x, lane = tid & 63;
    const uint32_t range = kmax - kmin;
    int hi = range ? 32 - __clz(range) : 0;
    prefix = 0;
    mask = 0;
    need = R;
    uint32_t* cur = hist;
    uint32_t* nxt = hist2 ? hist2 : hist;
    if (hi > 0) {
        for (int i = tid; i < kBins; i += kTopkThreads) cur[i] = 0;
        __syncthreads();
    }
    while (hi > 0) {
        const int lo = hi > kDigitBits ? hi - kDigitBits : 0;
        const uint32_t dmask = (1u << (hi - lo)) - 1u;
        if (hist2)                                    // the buffer of the pass after this one
            for (int i = tid; i < kBins; i += kTopkThreads) nxt[i] = 0;
        for (int64_t i = tid; i < m; i += kTopkThreads) {
            const uint32_t rel = get(i) - kmin;
            if ((rel & mask) == prefix) atomicAdd(&cur[(rel >> lo) & dmask], 1u);
        }
        __syncthreads();
        if (tid < 64) {
            // lane l holds bins kBins-1-32l .. kBins-32-32l, from the top down
            constexpr int kPerLane = kBins / 64;
            const int base = kBins - kPerLane * (lane + 1);   // the lane's bins: base .. base+31
            const uint4* b4 = reinterpret_cast<const uint4*>(cur + base);
            uint32_t sum = 0;
#pragma unroll
            for (int j = 0; j < kPerLane / 4; ++j) {
                const uint4 v = b4[j];
                sum += (v.x + v.y) + (v.z + v.w);
            }
            uint32_t incl = sum;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t y = __shfl_up(incl, o, 64);
                if (lane >= o) incl += y;
            }
            // the lane whose bins hold the need-th element (exactly one), then its 32 bins
            // from the top, one per lane of the wave's first half
            const uint32_t above_l = incl - sum;
            const int tl = __ffsll(__ballot(above_l < need && need <= incl)) - 1;
            const uint32_t above_t = __shfl(above_l, tl, 64);
            const int tbase = kBins - kPerLane * (tl + 1);
            const uint32_t c = lane < kPerLane ? cur[tbase + kPerLane - 1 - lane] : 0u;
            uint32_t ci = c;
#pragma unroll
            for (int o = 1; o < kPerLane; o <<= 1) {
                const uint32_t y = __shfl_up(ci, o, 64);
                if (lane >= o) ci += y;
            }
            const int f = __ffsll(__ballot(lane < kPerLane && need <= above_t + ci)) - 1;
            if (lane == f) {
                sh[0] = tbase + kPerLane - 1 - f;
                sh[1] = above_t + ci - c;
                sh[2] = c;
            }
        }
        __syncthreads();
        const uint32_t bin = sh[0], in_bin = sh[2];
        need -= sh[1];
        prefix |= bin << lo;
        mask |= dmask << lo;
        hi = lo;
        const bool done = in_bin == need || --max_passes == 0;   // the whole bin is taken, or bound only
        if (!hist2) {
            if (!done && hi > 0) {                    // wave 0 read the bins before the barrier
                for (int i = tid; i < kBins; i += kTopkThreads) cur[i] = 0;
                __syncthreads();
            }
        } else {
            uint32_t* t = cur; cur = nxt; nxt = t;
        }
        if (done) break;
    }
    __syncthreads();                                  // sh and the bins are free again
}

// Ordered compaction: element i (in position order) is selected when above the
// threshold, or tied and among the first `need` tied ones; its output slot is
// (# above before it) + min(# tied before it, need).
template <class Get, class Pos>
__device__ void compact(Get get, Pos pos_of, int64_t m, uint32_t kmin, uint32_t prefix,
                        uint32_t mask, uint32_t need, uint32_t* wsum, int32_t* __restrict__ out,
                        uint32_t* __restrict__ out_key = nullptr) {
    const int tid = threadIdx.x;
    uint32_t gt_base = 0, eq_base = 0;
    for (int64_t c0 = 0; c0 < m; c0 += 4 * kTopkThreads) {
        const int64_t i0 = c0 + (int64_t)tid * 4;
        uint32_t gt = 0, eq = 0, cnt = 0;
        for (int e = 0; e < 4; ++e) {
            if (i0 + e < m) {
                const uint32_t r = (get(i0 + e) - kmin) & mask;
                if (r > prefix) { gt |= 1u << e; ++cnt; }
                else if (r == prefix) { eq |= 1u << e; cnt += 1u << 16; }
            }
        }
        uint32_t total;
        const uint32_t excl = block_excl_scan(cnt, wsum, &total);
        uint32_t gt_before = gt_base + (excl & 0xffffu);
        uint32_t eq_before = eq_base + (excl >> 16);
        for (int e = 0; e < 4; ++e) {
            if (gt & (1u << e)) {
                const uint32_t slot = gt_before + min(eq_before, need);
                out[slot] = pos_of(i0 + e);
                if (out_key) out_key[slot] = get(i0 + e);
                ++gt_before;
            } else if (eq & (1u << e)) {
                if (eq_before < need) {
                    out[gt_before + eq_before] = pos_of(i0 + e);
                    if (out_key) out_key[gt_before + eq_before] = get(i0 + e);
                }
                ++eq_before;
            }
        }
        gt_base += total & 0xffffu;
        eq_base += total >> 16;
    }
}

constexpr int kCap = 7936;                // LDS candidate capacity (two workgroups per CU fit)
constexpr int kSampleRuns = 256;          // sample: up to 256 runs of 16 contiguous scores
constexpr int kSample = kSampleRuns * 16;

// Row length of workgroup row `row`: q_pos0 + row + 1, or row_len[row] when given
// (an out-of-range length means no candidates).
__device__ __forceinline__ int64_t row_length(int row, int Tk, int64_t q_pos0,
                                              const int32_t* __restrict__ row_len) {
    if (!row_len) return q_pos0 + row + 1;
    const int64_t n = row_len[row];
    return (n < 0 || n > Tk) ? 0 : n;
}

// With nseg == 1 a workgroup selects the top-k of a whole row into idx.  With
// nseg > 1 (rows too few to fill the GPU) workgroup (row, sg) selects the top-k
// of the row's positions [sg * seg_len, (sg + 1) * seg_len) into its slot of
// idx ([rows, nseg, k], ascending absolute positions, -1 padded); the union of
// the segments' selections contains the row's selection, ties included (each
// segment keeps its lowest-position ties), and topk_merge_kernel finishes it.
__global__ __launch_bounds__(kTopkThreads, 8) void topk_kernel(   // 8 waves per SIMD: two workgroups per CU
    const float* __restrict__ scores, int64_t ld, int Tk, int64_t q_pos0,
    const int32_t* __restrict__ row_len, int k, int nseg, int64_t seg_len,
    int32_t* __restrict__ idx, const int* __restrict__ run_if)
{
    if (run_if && *run_if == 0) return;              // gated launch with nothing to do
    __shared__ uint32_t ck[kCap];             // candidate keys, in position order
    __shared__ int32_t ci[kCap];              // their positions (the sample reuses this array)
    __shared__ __attribute__((aligned(16))) uint32_t hist[kBins], hist2[kBins];
    __shared__ uint32_t wsum[2 * kTopkWaves];
    __shared__ uint32_t sh[4];

    const int row = blockIdx.x / nseg, sg = blockIdx.x - row * nseg;
    const int tid = threadIdx.x;
    const int64_t n_row = row_length(row, Tk, q_pos0, row_len);
    const int64_t begin = nseg > 1 ? (int64_t)sg * seg_len : 0;
    int64_t n = nseg > 1 ? min(seg_len, n_row - begin) : n_row;
    if (n < 0) n = 0;
    int32_t* __restrict__ out = idx + (int64_t)blockIdx.x * k;
    // segments also hand their keys to the merge stage (second half of the buffer)
    uint32_t* __restrict__ out_key =
        nseg > 1 ? reinterpret_cast<uint32_t*>(idx + (int64_t)gridDim.x * k) + (int64_t)blockIdx.x * k
                 : nullptr;
    const float* __restrict__ src = scores + (int64_t)row * ld + begin;
    if (n <= k) {                                     // short row: everything is selected
        for (int i = tid; i < k; i += kTopkThreads) {
            out[i] = i < n ? (int32_t)(begin + i) : -1;
            if (out_key && i < n) out_key[i] = order_key(src[i]);
        }
        return;
    }
    int64_t m;                                        // number of candidates in LDS
    bool in_lds = true;

    if (n <= kCap) {
        // every load first (clamped into the row), then the keys: one round trip for the row
        // instead of one per 1024 scores
        constexpr int kIt = (kCap + kTopkThreads - 1) / kTopkThreads;
        float v[kIt];
#pragma unroll
        for (int j = 0; j < kIt; ++j) v[j] = src[min<int64_t>(tid + (int64_t)j * kTopkThreads, n - 1)];
#pragma unroll
        for (int j = 0; j < kIt; ++j) {
            const int64_t i = tid + (int64_t)j * kTopkThreads;
            if (i < n) {
                ck[i] = order_key(v[j]);
                ci[i] = (int32_t)(begin + i);
            }
        }
        m = n;
        __syncthreads();
    } else {
        // The streamed loads below are unconditional, from quad addresses clamped to
        // the last whole quad of the row (a branch around a load makes the compiler
        // wait for every load in flight where the paths join); the pass covers the
        // n_main = n & ~3 positions of whole quads, and the <= 3 tail positions follow it.
        const int64_t n_main = n & ~(int64_t)3;       // > kCap
        const int64_t last4 = n_main - 4;
        auto quad = [&](int64_t i) { return *reinterpret_cast<const float4*>(src + min(i, last4)); };

        // 1. sample -> lower bound for the k-th largest key (runs start on quads and
        //    end well inside the row)
        // n / 512 runs (at least 16): the sample reads about 1/32 of the row at any length
        uint32_t* smp = reinterpret_cast<uint32_t*>(ci);
        const int runs = (int)min<int64_t>(kSampleRuns, max<int64_t>(16, n >> 9));
        const int S = runs * 16;
        const int run = min(tid >> 2, runs - 1), part = tid & 3;
        const float4 sv = quad((((int64_t)run * n / runs) & ~(int64_t)3) + 4 * part);

        // the first two steps of the pass below stream in while the sample is ranked
        constexpr int kPer = 8;                       // consecutive scores per thread per step
        constexpr int64_t kStepLen = (int64_t)kPer * kTopkThreads;
        auto fetch = [&](int64_t c0, float4* dst) {
            const int64_t i0 = c0 + (int64_t)tid * kPer;
#pragma unroll
            for (int q = 0; q < kPer / 4; ++q) dst[q] = quad(i0 + 4 * q);
        };
        float4 b0[kPer / 4], b1[kPer / 4], b2[kPer / 4];
        fetch(0, b0);
        fetch(kStepLen, b1);

        if (4 * tid < S) {
            smp[4 * tid + 0] = order_key(sv.x);
            smp[4 * tid + 1] = order_key(sv.y);
            smp[4 * tid + 2] = order_key(sv.z);
            smp[4 * tid + 3] = order_key(sv.w);
        }
        __syncthreads();
        // sample rank of the bound: the expected rank of the k-th largest score, r = k S / n,
        // padded by 6 sigma (+8) of independent draws: about k + 1800 candidates at any row
        // length.  The 16 scores of a run are not independent when high scores come in
        // clusters of positions; then a row can end with fewer than k candidates (the slow
        // path below), about one in 4000 on clustered keys, against one in 40 at 3 sigma.
        const double r = (double)k * S / (double)n;
        uint32_t r_lo = (uint32_t)ceil(r + 6.0 * sqrt(r) + 8.0);
        if (r_lo > (uint32_t)S) r_lo = S;
        auto get_s = [&](int64_t i) { return smp[i]; };
        uint32_t smin, smax, sp, sm, sn;
        key_range(get_s, S, wsum, smin, smax);
        // two digits are enough: the bin's low edge sits at most one bin width (2^-22
        // of the sample's key range) below the r_lo-th largest sample key.  (Keys are
        // not linear in the value, so one 2^-11 bin can span a large value range.)
        radix_select(get_s, S, r_lo, smin, smax, hist, hist2, sh, sp, sm, sn, 2);
        const uint32_t bound = smin + sp;             // <= the r_lo-th largest sample key
        __syncthreads();                              // the sample is dead from here on

        // 2. one pass: every score with key >= bound, in position order, into LDS,
        //    kPer consecutive scores per thread per step and two steps in flight
        //    (a three-slot ring, unrolled so that every slot is a fixed register set)
        uint32_t base_cnt = 0;
        auto step = [&](int64_t c0, const float4* cur) {
            const int64_t i0 = c0 + (int64_t)tid * kPer;
            uint32_t flag = 0, cnt = 0;
#pragma unroll
            for (int q = 0; q < kPer / 4; ++q) {
                const float v[4] = {cur[q].x, cur[q].y, cur[q].z, cur[q].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = 4 * q + e;
                    if (i0 + j < n_main && order_key(v[e]) >= bound) { flag |= 1u << j; ++cnt; }
                }
            }
            uint32_t total;
            uint32_t p = base_cnt + block_excl_scan(cnt, wsum, &total);
            if (flag) {
#pragma unroll
                for (int q = 0; q < kPer / 4; ++q) {
                    const float v[4] = {cur[q].x, cur[q].y, cur[q].z, cur[q].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int j = 4 * q + e;
                        if (flag & (1u << j)) {
                            if (p < (uint32_t)kCap) { ck[p] = order_key(v[e]); ci[p] = (int32_t)(begin + i0 + j); }
                            ++p;
                        }
                    }
                }
            }
            base_cnt += total;
        };
        for (int64_t c0 = 0; c0 < n_main; c0 += 3 * kStepLen) {
            fetch(c0 + 2 * kStepLen, b2);
            step(c0, b0);
            if (c0 + kStepLen >= n_main) break;
            fetch(c0 + 3 * kStepLen, b0);
            step(c0 + kStepLen, b1);
            if (c0 + 2 * kStepLen >= n_main) break;
            fetch(c0 + 4 * kStepLen, b1);
            step(c0 + 2 * kStepLen, b2);
        }
        if (n_main < n) {                             // tail: one position per thread
            const int64_t i = n_main + tid;
            uint32_t key = 0, take = 0;
            if (i < n) { key = order_key(src[i]); take = key >= bound; }
            uint32_t total;
            const uint32_t p = base_cnt + block_excl_scan(take, wsum, &total);
            if (take && p < (uint32_t)kCap) { ck[p] = key; ci[p] = (int32_t)(begin + i); }
            base_cnt += total;
        }
        __syncthreads();
        m = base_cnt;
        in_lds = m >= (int64_t)k && m <= kCap;
    }

    uint32_t kmin, kmax, prefix, mask, need;
    if (in_lds) {
        // 3. exact select among the candidates
        auto get_c = [&](int64_t i) { return ck[i]; };
        auto pos_c = [&](int64_t i) { return ci[i]; };
        key_range(get_c, m, wsum, kmin, kmax);
        radix_select(get_c, m, (uint32_t)k, kmin, kmax, hist, hist2, sh, prefix, mask, need);
        compact(get_c, pos_c, m, kmin, prefix, mask, need, wsum, out, out_key);
    } else {
        // 4. fallback: the same exact select and compaction over the row in memory
        auto get_g = [&](int64_t i) { return order_key(src[i]); };
        auto pos_g = [&](int64_t i) { return (int32_t)(begin + i); };
        key_range(get_g, n, wsum, kmin, kmax);
        radix_select(get_g, n, (uint32_t)k, kmin, kmax, hist, hist2, sh, prefix, mask, need);
        compact(get_g, pos_g, n, kmin, prefix, mask, need, wsum, out, out_key);
    }
}

// Second stage of a segmented top-k: the nseg * k candidates of a row (positions
// ascending within and across segments, with their keys) are copied into LDS in
// position order and the exact select + ordered compaction produce the row's
// final ascending set.
constexpr int kMergeCap = 8192;           // merge stage: up to 4 segments of k = 2048

__global__ __launch_bounds__(kTopkThreads) void topk_merge_kernel(
    const float* __restrict__ scores, int64_t ld, int Tk, int64_t q_pos0,
    const int32_t* __restrict__ row_len, int k, int nseg, const int32_t* __restrict__ cand,
    int32_t* __restrict__ idx)
{
    __shared__ uint32_t ck[kMergeCap];
    __shared__ int32_t ci[kMergeCap];
    __shared__ __attribute__((aligned(16))) uint32_t hist[kBins];
    __shared__ uint32_t wsum[2 * kTopkWaves];
    __shared__ uint32_t sh[4];
    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t n = row_length(row, Tk, q_pos0, row_len);
    int32_t* __restrict__ out = idx + (int64_t)row * k;
    if (n <= k) {
        for (int i = tid; i < k; i += kTopkThreads) out[i] = i < n ? i : -1;
        return;
    }
    const int32_t* __restrict__ c = cand + (int64_t)row * nseg * k;
    const uint32_t* __restrict__ ckey =
        reinterpret_cast<const uint32_t*>(cand + (int64_t)gridDim.x * nseg * k) + (int64_t)row * nseg * k;
    const int total_in = nseg * k;                    // <= kMergeCap (checked by the launcher)
    uint32_t base_cnt = 0;
    for (int c0 = 0; c0 < total_in; c0 += 4 * kTopkThreads) {
        const int i0 = c0 + tid * 4;
        int32_t pos[4];
        uint32_t flag = 0, cnt = 0;
        for (int e = 0; e < 4; ++e) {
            pos[e] = (i0 + e < total_in) ? c[i0 + e] : -1;
            if (pos[e] >= 0) { flag |= 1u << e; ++cnt; }
        }
        uint32_t total;
        uint32_t p = base_cnt + block_excl_scan(cnt, wsum, &total);
        for (int e = 0; e < 4; ++e) {
            if (flag & (1u << e)) {
                ck[p] = ckey[i0 + e];
                ci[p] = pos[e];
                ++p;
            }
        }
        base_cnt += total;
    }
    __syncthreads();
    const int64_t m = base_cnt;
    auto get_c = [&](int64_t i) { return ck[i]; };
    auto pos_c = [&](int64_t i) { return ci[i]; };
    uint32_t kmin, kmax, prefix, mask, need;
    key_range(get_c, m, wsum, kmin, kmax);
    radix_select(get_c, m, (uint32_t)k, kmin, kmax, hist, nullptr, sh, prefix, mask, need);
    compact(get_c, pos_c, m, kmin, prefix, mask, need, wsum, out);
}

// ---- fused prefill: bound from a sample, exact select from a candidate list ----

// In-place ascending bitonic sort of a[0..len) (len <= cap of the array, padded to the next
// power of two with 0xffffffff, which must fit in the array).
__device__ void bitonic_sort_asc(uint32_t* a, int len) {
    const int tid = threadIdx.x;
    int P = 1;
    while (P < len) P <<= 1;
    for (int i = len + tid; i < P; i += kTopkThreads) a[i] = 0xffffffffu;
    __syncthreads();
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < (P >> 1); i += kTopkThreads) {
                const int lo = 2 * stride * (i / stride) + (i & (stride - 1));
                const int hi = lo + stride;
                const bool asc = (lo & size) == 0;
                const uint32_t x = a[lo], y = a[hi];
                if ((x > y) == asc) { a[lo] = y; a[hi] = x; }
            }
            __syncthreads();
        }
    }
}

static_assert(kCandCap % kTopkThreads == 0, "candidate lists and sample rows load in whole rounds");

// Lower bound of row `row`'s k-th largest score from its S samples (see launch_topk_bound).
__global__ __launch_bounds__(kTopkThreads) void topk_bound_kernel(
    const float* __restrict__ samples, int S, int64_t q_pos0, const int32_t* __restrict__ row_len,
    int max_len, int k, float* __restrict__ tau, int32_t* __restrict__ cnt, int* __restrict__ fallback,
    int first)
{
    __shared__ uint32_t smp[kCandCap];
    __shared__ __attribute__((aligned(16))) uint32_t hist[kBins];
    __shared__ uint32_t wsum[2 * kTopkWaves];
    __shared__ uint32_t sh[4];
    const int row = blockIdx.x, tid = threadIdx.x;
    if (tid == 0) {
        cnt[row] = 0;
        if (row == 0) {                               // flag of this chunk; call statistics
            fallback[0] = 0;
            if (first) { fallback[1] = 1; fallback[2] = 0; } else { fallback[1] += 1; }
        }
    }
    const int64_t n = row_len ? row_length(row, max_len, 0, row_len) : q_pos0 + row + 1;
    if (n <= kCandCap || S <= 0) {                   // every causal score is a candidate
        if (tid == 0) tau[row] = -FLT_MAX;
        return;
    }
    // every load first (clamped to the row's samples), then the keys: one round trip
    const float* __restrict__ src = samples + (int64_t)row * S;
    constexpr int kIt = kCandCap / kTopkThreads;
    float v[kIt];
#pragma unroll
    for (int j = 0; j < kIt; ++j) v[j] = src[min(tid + j * kTopkThreads, S - 1)];
#pragma unroll
    for (int j = 0; j < kIt; ++j)
        if (tid + j * kTopkThreads < S) smp[tid + j * kTopkThreads] = order_key(v[j]);
    __syncthreads();
    // rank of the bound among the samples: the expected rank of the k-th largest score,
    // r = k S / n, padded by 5 sigma (+8): fewer than k scores at or above the bound needs
    // >= r_lo samples above the k-th largest score, a ~1e-7 tail event
    const double r = (double)k * S / (double)n;
    uint32_t r_lo = (uint32_t)ceil(r + 5.0 * sqrt(r) + 8.0);
    if (r_lo > (uint32_t)S) r_lo = S;
    auto get_s = [&](int64_t i) { return smp[i]; };
    uint32_t smin, smax, sp, sm, sn;
    key_range(get_s, S, wsum, smin, smax);
    radix_select(get_s, S, r_lo, smin, smax, hist, nullptr, sh, sp, sm, sn, 2);
    // back to a float: a score is >= it exactly when its key is >= the bound key (the key
    // lies between two sample keys, so it is a finite value's key)
    if (tid == 0) {
        const uint32_t key = smin + sp;
        const uint32_t u = (key & 0x80000000u) ? (key & 0x7fffffffu) : ~key;
        tau[row] = __uint_as_float(u);
    }
}

// Omega of one row from its candidate list: exact select of the k-th largest key, the
// candidates above it plus the lowest-position ties, sorted ascending.
__global__ __launch_bounds__(kTopkThreads, 8) void topk_select_kernel(
    const uint2* __restrict__ cand, const int32_t* __restrict__ cnt, int64_t q_pos0,
    const int32_t* __restrict__ row_len, int max_len, int k, int32_t* __restrict__ idx,
    int* __restrict__ fallback)
{
    __shared__ uint32_t ck[kCandCap];                 // keys, later the selected positions
    __shared__ uint32_t ci[kCandCap];                 // positions, later the tied positions
    __shared__ __attribute__((aligned(16))) uint32_t hist[kBins];
    __shared__ uint32_t wsum[2 * kTopkWaves];
    __shared__ uint32_t sh[4];
    const int row = blockIdx.x, tid = threadIdx.x;
    const int64_t n = row_len ? row_length(row, max_len, 0, row_len) : q_pos0 + row + 1;
    int32_t* __restrict__ out = idx + (int64_t)row * k;
    if (n <= k) {                                     // (n = 0: an invalid length, all -1)
        for (int i = tid; i < k; i += kTopkThreads) out[i] = i < n ? i : -1;
        return;
    }
    const int m = cnt[row];
    if (m < k || m > kCandCap) {                      // the bound missed: exact path for the chunk
        if (tid == 0) { fallback[0] = 1; atomicAdd(fallback + 2, 1); }
        return;
    }
    // every load first (clamped to the list), then the LDS stores: one round trip for the list
    const uint2* __restrict__ src = cand + (int64_t)row * kCandCap;
    constexpr int kIt = kCandCap / kTopkThreads;
    uint2 cv[kIt];
#pragma unroll
    for (int j = 0; j < kIt; ++j) cv[j] = src[min(tid + j * kTopkThreads, m - 1)];
#pragma unroll
    for (int j = 0; j < kIt; ++j) {
        const int i = tid + j * kTopkThreads;
        if (i < m) {
            ck[i] = cv[j].x;
            ci[i] = cv[j].y;
        }
    }
    __syncthreads();
    auto get_c = [&](int64_t i) { return ck[i]; };
    uint32_t kmin, kmax, prefix, mask, need;
    key_range(get_c, m, wsum, kmin, kmax);
    radix_select(get_c, m, (uint32_t)k, kmin, kmax, hist, nullptr, sh, prefix, mask, need);
    // split in place: positions above the threshold to ck[0..), tied positions to ci[0..)
    // (an element's new slot never exceeds its old index, and a step's elements are all
    // read before any is written)
    uint32_t n_gt = 0, n_eq = 0;
    for (int c0 = 0; c0 < m; c0 += 4 * kTopkThreads) {
        const int i0 = c0 + tid * 4;
        uint32_t key[4], pos[4], gt = 0, eq = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            key[e] = 0; pos[e] = 0;
            if (i0 + e < m) {
                key[e] = ck[i0 + e];
                pos[e] = ci[i0 + e];
                const uint32_t rel = (key[e] - kmin) & mask;
                if (rel > prefix) gt |= 1u << e;
                else if (rel == prefix) eq |= 1u << e;
            }
        }
        uint32_t total;
        const uint32_t excl = block_excl_scan(__popc(gt) | (__popc(eq) << 16), wsum, &total);
        uint32_t pg = n_gt + (excl & 0xffffu), pe = n_eq + (excl >> 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (gt & (1u << e)) ck[pg++] = pos[e];
            else if (eq & (1u << e)) ci[pe++] = pos[e];
        }
        n_gt += total & 0xffffu;
        n_eq += total >> 16;
        __syncthreads();
    }
    // the need lowest tied positions complete the set
    if (n_eq > need) bitonic_sort_asc(ci, (int)n_eq);
    for (int j = tid; j < (int)need; j += kTopkThreads) ck[n_gt + j] = ci[j];
    __syncthreads();
    if (n > 32 * (int64_t)kCandCap) {                // no room for a bitmap of the row
        bitonic_sort_asc(ck, k);
        for (int i = tid; i < k; i += kTopkThreads) out[i] = (int32_t)ck[i];
        return;
    }
    // ascending order through a bitmap of the row's positions (in ci, now free): each
    // thread owns a run of words, and a prefix sum of their bit counts places its positions
    const int nw = (int)((n + 31) >> 5);
    for (int i = tid; i < nw; i += kTopkThreads) ci[i] = 0u;
    __syncthreads();
    for (int j = tid; j < k; j += kTopkThreads) atomicOr(&ci[ck[j] >> 5], 1u << (ck[j] & 31u));
    __syncthreads();
    const int wpt = (nw + kTopkThreads - 1) / kTopkThreads;
    const int w0 = tid * wpt, w1 = min(w0 + wpt, nw);
    uint32_t c = 0;
    for (int i = w0; i < w1; ++i) c += __popc(ci[i]);
    uint32_t total;
    uint32_t p = block_excl_scan(c, wsum, &total);
    for (int i = w0; i < w1; ++i) {
        uint32_t word = ci[i];
        while (word) {
            const int b = __ffs(word) - 1;
            out[p++] = i * 32 + b;
            word &= word - 1u;
        }
    }
}

}  // namespace

int topk_num_segments(int Tq, int Tk, int k)
{
    // few rows: split each row so that >= 256 workgroups stream the scores
    if (Tq <= 0 || Tq >= 128 || (int64_t)Tk < 4 * (int64_t)k) return 1;
    int nseg = kMergeCap / k;
    if (nseg > 8) nseg = 8;
    while (nseg > 1 && (int64_t)Tq * nseg > 512) nseg >>= 1;
    return nseg < 2 ? 1 : nseg;
}

size_t topk_workspace_bytes(int Tq, int Tk, int k)
{
    const int nseg = topk_num_segments(Tq, Tk, k);
    return nseg > 1 ? (size_t)Tq * nseg * k * 2 * sizeof(int32_t) : 0;   // positions + keys
}

hipError_t launch_topk(const float* scores, int64_t ld, int Tq, int Tk, int64_t q_pos0,
                       const int32_t* row_len, int k, int32_t* idx, void* ws, hipStream_t stream,
                       const int* run_if)
{
    if (Tq == 0) return hipSuccess;
    const int nseg = ws ? topk_num_segments(Tq, Tk, k) : 1;
    if (nseg > 1 && run_if) return hipErrorInvalidValue;   // gating exists for one pass only
    if (nseg == 1) {
        hipLaunchKernelGGL(topk_kernel, dim3(Tq), dim3(kTopkThreads), 0, stream, scores, ld, Tk,
                           q_pos0, row_len, k, 1, (int64_t)Tk, idx, run_if);
        return hipGetLastError();
    }
    const int64_t seg_len = (((int64_t)Tk + nseg - 1) / nseg + 3) & ~(int64_t)3;   // segments start on quads
    int32_t* cand = static_cast<int32_t*>(ws);
    hipLaunchKernelGGL(topk_kernel, dim3(Tq * nseg), dim3(kTopkThreads), 0, stream, scores, ld, Tk,
                       q_pos0, row_len, k, nseg, seg_len, cand, run_if);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_merge_kernel, dim3(Tq), dim3(kTopkThreads), 0, stream, scores, ld, Tk,
                       q_pos0, row_len, k, nseg, cand, idx);
    return hipGetLastError();
}

int fused_sample_count(int Tk)
{
    // about one sample per 64 candidates (at least 2048), so that the padded bound keeps
    // the expected candidate count near k (1 + 5/sqrt(32) + 8/32) and far below kCandCap
    if (Tk <= kCandCap) return 0;
    int S = (Tk / 64 + 1023) / 1024 * 1024;
    if (S < 2048) S = 2048;
    return S > kCandCap ? -1 : S;                    // -1: too long for the candidate path
}

namespace {

// Index lists of packed short sequences whose rows keep their whole prefix: row r at position
// t of its sequence gets 0 .. t, then -1.  One workgroup per row, 16-byte stores.
__global__ __launch_bounds__(256) void prefix_idx_kernel(SeqStarts rows, int topk,
                                                         int32_t* __restrict__ idx)
{
    const int r = blockIdx.x;
    int lo = 0, hi = rows.n - 1;                     // the row's sequence: largest start <= r
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (rows.start[mid] <= r) lo = mid; else hi = mid - 1;
    }
    const int t = r - rows.start[lo];
    int32_t* __restrict__ out = idx + (int64_t)r * topk;
    for (int e = threadIdx.x; e < topk; e += 256) out[e] = e <= t ? e : -1;
}

}  // namespace

hipError_t launch_prefix_idx(const SeqStarts& rows, int topk, int32_t* idx, hipStream_t stream)
{
    if (rows.n < 1 || rows.n > kMaxPrefixSegs) return hipErrorInvalidValue;
    const int T = rows.start[rows.n];
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL(prefix_idx_kernel, dim3((unsigned)T), dim3(256), 0, stream, rows, topk, idx);
    return hipGetLastError();
}

hipError_t launch_topk_bound(const float* samples, int S, int Tq, int64_t q_pos0,
                             const int32_t* row_len, int max_len, int k, float* tau, int32_t* cnt,
                             int* fallback, int first, hipStream_t stream)
{
    if (Tq == 0) return hipSuccess;
    if (S > kCandCap) return hipErrorInvalidValue;
    hipLaunchKernelGGL(topk_bound_kernel, dim3(Tq), dim3(kTopkThreads), 0, stream, samples, S,
                       q_pos0, row_len, max_len, k, tau, cnt, fallback, first);
    return hipGetLastError();
}

hipError_t launch_topk_select(const uint2* cand, const int32_t* cnt, int Tq, int64_t q_pos0,
                              const int32_t* row_len, int max_len, int k, int32_t* idx,
                              int* fallback, hipStream_t stream)
{
    if (Tq == 0) return hipSuccess;
    if (k > kCandCap) return hipErrorInvalidValue;
    hipLaunchKernelGGL(topk_select_kernel, dim3(Tq), dim3(kTopkThreads), 0, stream, cand, cnt,
                       q_pos0, row_len, max_len, k, idx, fallback);
    return hipGetLastError();
}

}  // namespace dsa
