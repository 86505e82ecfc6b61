// indexer.hip -- lightning indexer kernels for gfx950.
//
// I[t,s] = sum_j w[t,j] * ReLU(q^I[t,j] . k^I[s]) for s <= t (Keye-VL-2.0
// report section 2.3.1; xllm-io review page "核心公式", first formula), with one
// FP8 key vector per token shared by all indexer heads.
//
// FP8 prefill kernel: the dot products run on the 16x16x128 FP8 matrix core
// with d_I = 128 as the whole contraction.  A (rows) = 16 keys, B (columns) =
// 16 query tokens for one indexer head j, so each lane's four results are four
// keys of ONE token and the head loop (ReLU, w-weighted sum) stays inside the
// lane: no cross-lane reduction.  The per-token scales factor out of the ReLU
// (they are positive) and are applied once in the epilogue.
//
// A wave keeps its NK key tiles (16*NK keys, 8 VGPRs each) in registers for the
// whole head loop and streams one 32-byte slice of q^I per lane per head, which
// the four waves of a workgroup (same 16 tokens, different keys) share through
// L1/L2.  Work items are ordered token-tile-major and mapped so that
// consecutive items run on one XCD: the key blocks of a token tile are
// processed together and the tile's 128 KB of q^I stays in that XCD's L2.
#include "device_common.h"
#include "internal.h"

namespace dsa {
namespace {

constexpr int kIdxWaves = 4;

__device__ __forceinline__ v8i load32B(const uint8_t* p) {
    const v4i* v = reinterpret_cast<const v4i*>(p);
    v4i lo = v[0], hi = v[1];
    return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

template <int NK>
__global__ __launch_bounds__(256) void index_fp8_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ k_idx,
    const float* __restrict__ k_scale, int Tq, int Tk, int HI, int64_t q_pos0,
    float* __restrict__ scores, int64_t ld, int n_kb)
{
    constexpr int kKeysPerWave = 16 * NK;
    constexpr int kKeysPerWG = kIdxWaves * kKeysPerWave;
    const int work = xcd_remap(blockIdx.x, gridDim.x);
    const int tt = work / n_kb;
    const int kb = work - tt * n_kb;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;

    const int t = tt * 16 + col;                      // this lane's query row
    const bool t_ok = t < Tq;
    const int tc = t_ok ? t : Tq - 1;
    const int64_t pos = q_pos0 + t;
    const int64_t pos_hi = q_pos0 + min(tt * 16 + 15, Tq - 1);
    const int s_base = kb * kKeysPerWG + wave * kKeysPerWave;
    float* __restrict__ out_row = scores + (int64_t)tc * ld;
    if (s_base >= Tk) return;

    if ((int64_t)s_base > pos_hi) {                   // tile entirely above the diagonal
        if (t_ok) {
#pragma unroll
            for (int i = 0; i < NK; ++i) {
                const int s0 = s_base + 16 * i + 4 * grp;
                if (s0 + 3 < Tk) {
                    *reinterpret_cast<float4*>(out_row + s0) =
                        make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
                } else {
                    for (int e = 0; e < 4; ++e)
                        if (s0 + e < Tk) out_row[s0 + e] = -INFINITY;
                }
            }
        }
        return;
    }

    // A operands: key rows s_base + 16 i + col, 32 bytes per lane (slice grp)
    v8i a[NK];
#pragma unroll
    for (int i = 0; i < NK; ++i) {
        const int s = s_base + 16 * i + col;
        a[i] = (s < Tk) ? load32B(k_idx + (int64_t)s * 128 + grp * 32) : v8i{0, 0, 0, 0, 0, 0, 0, 0};
    }

    float acc[NK][4];
#pragma unroll
    for (int i = 0; i < NK; ++i)
        for (int e = 0; e < 4; ++e) acc[i][e] = 0.f;

    const uint8_t* __restrict__ qp = q_idx + (int64_t)tc * HI * 128 + grp * 32;
    const float* __restrict__ wp = w + (int64_t)tc * HI;
    const v4f zero = {0.f, 0.f, 0.f, 0.f};

    v8i b_next = load32B(qp);
    for (int j0 = 0; j0 < HI; j0 += 4) {
        const float4 w4 = *reinterpret_cast<const float4*>(wp + j0);
        const float wj[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const v8i b = b_next;
            const int jn = j0 + jj + 1;
            if (jn < HI) b_next = load32B(qp + (int64_t)jn * 128);
#pragma unroll
            for (int i = 0; i < NK; ++i) {
                const v4f d = mfma_fp8_16x16x128(a[i], b, zero);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][e] += wj[jj] * fmaxf(d[e], 0.f);
            }
        }
    }

    if (!t_ok) return;
    const float qs = q_scale[tc];
#pragma unroll
    for (int i = 0; i < NK; ++i) {
        const int s0 = s_base + 16 * i + 4 * grp;
        float r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int s = s0 + e;
            const float ks = (s < Tk) ? k_scale[s] : 0.f;
            r[e] = ((int64_t)s <= pos) ? acc[i][e] * (qs * ks) : -INFINITY;
        }
        if (s0 + 3 < Tk) {
            *reinterpret_cast<float4*>(out_row + s0) = make_float4(r[0], r[1], r[2], r[3]);
        } else {
            for (int e = 0; e < 4; ++e)
                if (s0 + e < Tk) out_row[s0 + e] = r[e];
        }
    }
}

// fp32 indexer (small head counts; correctness path).  16 tokens x 16 keys per
// workgroup, one (token, key) pair per thread, operands staged in LDS.
__global__ __launch_bounds__(256) void index_f32_kernel(
    const float* __restrict__ q_idx, const float* __restrict__ w, const float* __restrict__ k_idx,
    int Tq, int Tk, int HI, int dI, int64_t q_pos0, float* __restrict__ scores, int64_t ld)
{
    __shared__ float qs_[16 * 1024];
    __shared__ float ks_[16 * 129];
    __shared__ float ws_[16 * 256];
    const int t0 = blockIdx.y * 16, s0 = blockIdx.x * 16;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const int t = t0 + ty, s = s0 + tx;
    const int64_t pos_hi = q_pos0 + min(t0 + 15, Tq - 1);
    if ((int64_t)s0 > pos_hi) {
        if (t < Tq && s < Tk) scores[(int64_t)t * ld + s] = -INFINITY;
        return;
    }
    const int qlen = HI * dI;
    for (int i = threadIdx.x; i < 16 * qlen; i += 256) {
        const int r = i / qlen, c = i - r * qlen;
        qs_[r * qlen + c] = (t0 + r < Tq) ? q_idx[(int64_t)(t0 + r) * qlen + c] : 0.f;
    }
    for (int i = threadIdx.x; i < 16 * dI; i += 256) {
        const int r = i / dI, c = i - r * dI;
        ks_[r * 129 + c] = (s0 + r < Tk) ? k_idx[(int64_t)(s0 + r) * dI + c] : 0.f;
    }
    for (int i = threadIdx.x; i < 16 * HI; i += 256) {
        const int r = i / HI, c = i - r * HI;
        ws_[r * HI + c] = (t0 + r < Tq) ? w[(int64_t)(t0 + r) * HI + c] : 0.f;
    }
    __syncthreads();
    if (t >= Tq || s >= Tk) return;
    float acc = 0.f;
    for (int j = 0; j < HI; ++j) {
        const float* qv = qs_ + ty * qlen + j * dI;
        const float* kv = ks_ + tx * 129;
        float dot = 0.f;
        for (int i = 0; i < dI; ++i) dot = fmaf(qv[i], kv[i], dot);
        acc += ws_[ty * HI + j] * fmaxf(dot, 0.f);
    }
    scores[(int64_t)t * ld + s] = ((int64_t)s <= q_pos0 + t) ? acc : -INFINITY;
}

// Paged decode indexer: one query token per sequence, keys in a paged cache.
// A (rows) = 16 indexer heads, B (columns) = 16 keys: a lane's four results are
// four heads of one key, reduced in-lane (ReLU, w) and then across the four
// lane groups; all HI/16 head tiles stay in registers for the whole key loop.
constexpr int kDecKeysPerWave = 512;   // 8 iterations of 64 keys
constexpr int kDecKeysPerWG = kIdxWaves * kDecKeysPerWave;

__global__ __launch_bounds__(256) void index_fp8_paged_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ kcache,
    const float* __restrict__ kscale, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, int num_blocks, int max_blocks, int block_size, int HI,
    float* __restrict__ scores, int64_t ld, int n_split)
{
    const int work = xcd_remap(blockIdx.x, gridDim.x);
    const int b = work / n_split, sp = work - b * n_split;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int64_t cap = (int64_t)max_blocks * block_size;
    const int64_t len = seq_lens[b];
    if (len < 1 || len > cap) return;
    const int64_t s_begin = (int64_t)sp * kDecKeysPerWG + (int64_t)wave * kDecKeysPerWave;
    if (s_begin >= len) return;
    const int64_t s_end = min(len, s_begin + kDecKeysPerWave);

    // query head tiles (A) and their weights: tile m covers heads 16 m .. 16 m + 15
    const int n_ht = (HI + 15) >> 4;
    v8i qa[8];
    float wv[8][4];
    const uint8_t* qrow = q_idx + (int64_t)b * HI * 128;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int h = 16 * m + col;
        qa[m] = (m < n_ht && h < HI) ? load32B(qrow + (int64_t)h * 128 + grp * 32)
                                     : v8i{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int hh = 16 * m + 4 * grp + i;
            wv[m][i] = (m < n_ht && hh < HI) ? w[(int64_t)b * HI + hh] : 0.f;
        }
    }
    const float qs = q_scale[b];
    const int32_t* bt = block_table + (int64_t)b * max_blocks;
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    float* __restrict__ out = scores + (int64_t)b * ld;

    for (int64_t s0 = s_begin; s0 < s_end; s0 += 64) {
        // four 16-key tiles; this lane's key in tile u is s0 + 16 u + col
        v8i kb[4];
        int64_t row[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t s = s0 + 16 * u + col;
            row[u] = -1;
            if (s < s_end) {
                const int blk = bt[s / block_size];
                if (blk >= 0 && blk < num_blocks) row[u] = (int64_t)blk * block_size + s % block_size;
            }
            kb[u] = row[u] >= 0 ? load32B(kcache + row[u] * 128 + grp * 32)
                                : v8i{0, 0, 0, 0, 0, 0, 0, 0};
        }
        float part[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float acc = 0.f;
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                if (m < n_ht) {
                    const v4f d = mfma_fp8_16x16x128(qa[m], kb[u], zero);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc += wv[m][i] * fmaxf(d[i], 0.f);
                }
            }
            acc += __shfl_xor(acc, 16, 64);
            acc += __shfl_xor(acc, 32, 64);
            part[u] = acc;
        }
        // lane group u writes tile u: 64 consecutive keys per store instruction
        float mine = part[0];
#pragma unroll
        for (int u = 1; u < 4; ++u) mine = (grp == u) ? part[u] : mine;
        int64_t my_row = row[0];
#pragma unroll
        for (int u = 1; u < 4; ++u) my_row = (grp == u) ? row[u] : my_row;
        const int64_t s = s0 + lane;
        if (s < s_end) out[s] = (my_row >= 0) ? mine * (qs * kscale[my_row]) : -INFINITY;
    }
}

}  // namespace

hipError_t launch_index_fp8(const uint8_t* q_idx, const float* q_scale, const float* w,
                            const uint8_t* k_idx, const float* k_scale, int Tq, int Tk, int HI,
                            int64_t q_pos0, float* scores, int64_t ld, hipStream_t stream)
{
    constexpr int NK = 8;
    const int n_tt = (Tq + 15) / 16;
    const int n_kb = (Tk + kIdxWaves * 16 * NK - 1) / (kIdxWaves * 16 * NK);
    const int64_t n = (int64_t)n_tt * n_kb;
    if (n == 0) return hipSuccess;
    if (n > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(index_fp8_kernel<NK>, dim3((unsigned)n), dim3(256), 0, stream, q_idx,
                       q_scale, w, k_idx, k_scale, Tq, Tk, HI, q_pos0, scores, ld, n_kb);
    return hipGetLastError();
}

hipError_t launch_index_f32(const float* q_idx, const float* w, const float* k_idx, int Tq,
                            int Tk, int HI, int dI, int64_t q_pos0, float* scores, int64_t ld,
                            hipStream_t stream)
{
    if (Tq == 0 || Tk == 0) return hipSuccess;
    dim3 grid((Tk + 15) / 16, (Tq + 15) / 16);
    hipLaunchKernelGGL(index_f32_kernel, grid, dim3(256), 0, stream, q_idx, w, k_idx, Tq, Tk, HI,
                       dI, q_pos0, scores, ld);
    return hipGetLastError();
}

hipError_t launch_index_fp8_paged(const uint8_t* q_idx, const float* q_scale, const float* w,
                                  const uint8_t* kidx_cache, const float* kidx_scale,
                                  const int32_t* block_table, const int32_t* seq_lens, int B,
                                  int num_blocks, int max_blocks, int block_size, int HI,
                                  float* scores, int64_t ld, hipStream_t stream)
{
    const int64_t cap = (int64_t)max_blocks * block_size;
    const int n_split = (int)((cap + kDecKeysPerWG - 1) / kDecKeysPerWG);
    const int64_t n = (int64_t)B * n_split;
    if (n == 0) return hipSuccess;
    if (n > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(index_fp8_paged_kernel, dim3((unsigned)n), dim3(256), 0, stream, q_idx,
                       q_scale, w, kidx_cache, kidx_scale, block_table, seq_lens, num_blocks,
                       max_blocks, block_size, HI, scores, ld, n_split);
    return hipGetLastError();
}

}  // namespace dsa
