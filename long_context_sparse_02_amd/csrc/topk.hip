// topk.hip -- deterministic per-row Top-k for gfx950.
//
// Omega_t = the min(k, t+1) positions s <= t with the largest I[t,s] (xllm-io
// review page "核心公式", second formula), equal scores going to the lower
// position so that the selection is deterministic (Keye-VL-2.0 report section
// 5.2.1), listed in ascending position order.
//
// Exact radix select on an order-preserving 32-bit key.  One workgroup of 1024
// threads owns a row:
//   1. min / max of the row's keys;
//   2. radix passes over key - min, most significant digit first, with the
//      first digit placed at the top set bit of (max - min) so that the bins
//      spread over the scores actually present (scores of one row usually
//      span only a few binades, which a fixed exponent-first digit would
//      crowd into a handful of bins); each pass builds an LDS histogram of the
//      elements still tied with the prefix and picks the bin holding the k-th
//      largest; it stops early when that bin is taken whole;
//   3. one ordered compaction pass: elements above the threshold, plus the
//      first `need` elements equal to it in position order; a block-wide
//      prefix sum gives every selected element its output slot directly, so
//      the output comes out ascending with no sort.
// Rows with t + 1 <= k need no selection and read nothing (they take 0..t).
#include "device_common.h"
#include "internal.h"

namespace dsa {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;

// Larger float -> larger unsigned key; -0 and +0 map to the same key.
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

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

// Four consecutive elements starting at i (multiple of 4); missing ones get `fill`.
__device__ __forceinline__ void load4(const float* __restrict__ src, int64_t i, int64_t n,
                                      float v[4]) {
    if (i + 3 < n) {
        const float4 x = *reinterpret_cast<const float4*>(src + i);
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    } else {
        for (int e = 0; e < 4; ++e) v[e] = (i + e < n) ? src[i + e] : 0.f;
    }
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(
    const float* __restrict__ scores, int64_t ld, int Tk, int64_t q_pos0,
    const int32_t* __restrict__ row_len, int k, int32_t* __restrict__ idx)
{
    __shared__ uint32_t hist[kBins];
    __shared__ uint32_t wsum[2 * kTopkWaves];
    __shared__ uint32_t s_bin, s_above;

    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    int64_t n;
    if (row_len) {
        n = row_len[row];
        if (n < 0 || n > Tk) n = 0;                   // invalid length: no candidates
    } else {
        n = q_pos0 + row + 1;
    }
    int32_t* __restrict__ out = idx + (int64_t)row * k;
    if (n <= k) {                                     // short row: everything is selected
        for (int i = tid; i < k; i += kTopkThreads) out[i] = i < n ? i : -1;
        return;
    }
    const float* __restrict__ src = scores + (int64_t)row * ld;

    // 1. key range of the row
    uint32_t mn = 0xffffffffu, mx = 0u;
    for (int64_t i = (int64_t)tid * 4; i < n; i += 4 * kTopkThreads) {
        float v[4];
        load4(src, i, n, v);
        for (int e = 0; e < 4; ++e) {
            if (i + e < n) {
                const uint32_t key = order_key(v[e]);
                mn = min(mn, key);
                mx = max(mx, key);
            }
        }
    }
    uint32_t kmax;
    const uint32_t kmin = block_reduce_minmax(mn, mx, wsum, &kmax);
    const uint32_t range = kmax - kmin;
    int hi = range ? 32 - __clz(range) : 0;           // bits of (key - kmin) that vary

    // 2. radix passes on rel = key - kmin, digits of <= 11 bits from the top
    uint32_t prefix = 0, mask = 0;                    // rel & mask == prefix: still tied
    uint32_t need = (uint32_t)k;                      // still to take among the tied
    while (hi > 0) {
        const int lo = hi > kDigitBits ? hi - kDigitBits : 0;
        const uint32_t dmask = (1u << (hi - lo)) - 1u;
        for (int i = tid; i < kBins; i += kTopkThreads) hist[i] = 0;
        __syncthreads();
        for (int64_t i = (int64_t)tid * 4; i < n; i += 4 * kTopkThreads) {
            float v[4];
            load4(src, i, n, v);
            for (int e = 0; e < 4; ++e) {
                if (i + e < n) {
                    const uint32_t rel = order_key(v[e]) - kmin;
                    if ((rel & mask) == prefix) atomicAdd(&hist[(rel >> lo) & dmask], 1u);
                }
            }
        }
        __syncthreads();
        // bins in descending order: thread t takes bins 2047-2t and 2046-2t
        const uint32_t h0 = hist[kBins - 1 - 2 * tid], h1 = hist[kBins - 2 - 2 * tid];
        uint32_t total;
        const uint32_t above = block_excl_scan(h0 + h1, wsum, &total);
        if (above < need && need <= above + h0) {
            s_bin = kBins - 1 - 2 * tid;
            s_above = above;
        } else if (above + h0 < need && need <= above + h0 + h1) {
            s_bin = kBins - 2 - 2 * tid;
            s_above = above + h0;
        }
        __syncthreads();
        const uint32_t bin = s_bin;
        need -= s_above;
        const uint32_t in_bin = hist[bin];
        prefix |= bin << lo;
        mask |= dmask << lo;
        __syncthreads();                              // hist is rebuilt by the next pass
        hi = lo;
        if (in_bin == need) break;                    // the whole bin is taken
    }

    // 3. ordered compaction: position of an element = (# above before it) +
    //    min(# tied before it, need)
    uint32_t gt_base = 0, eq_base = 0;
    for (int64_t c0 = 0; c0 < n; c0 += 4 * kTopkThreads) {
        const int64_t i0 = c0 + (int64_t)tid * 4;
        float v[4];
        load4(src, i0, n, v);
        uint32_t gt = 0, eq = 0, cnt = 0;
        for (int e = 0; e < 4; ++e) {
            if (i0 + e < n) {
                const uint32_t r = (order_key(v[e]) - kmin) & mask;
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
                out[gt_before + min(eq_before, need)] = (int32_t)(i0 + e);
                ++gt_before;
            } else if (eq & (1u << e)) {
                if (eq_before < need) out[gt_before + eq_before] = (int32_t)(i0 + e);
                ++eq_before;
            }
        }
        gt_base += total & 0xffffu;
        eq_base += total >> 16;
    }
}

}  // namespace

hipError_t launch_topk(const float* scores, int64_t ld, int Tq, int Tk, int64_t q_pos0,
                       const int32_t* row_len, int k, int32_t* idx, hipStream_t stream)
{
    if (Tq == 0) return hipSuccess;
    hipLaunchKernelGGL(topk_kernel, dim3(Tq), dim3(kTopkThreads), 0, stream, scores, ld, Tk,
                       q_pos0, row_len, k, idx);
    return hipGetLastError();
}

}  // namespace dsa
