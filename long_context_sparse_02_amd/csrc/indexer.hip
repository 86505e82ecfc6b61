// indexer.hip -- lightning indexer kernels for gfx950.
//
// I[t,s] = sum_j w[t,j] * ReLU(q^I[t,j] . k^I[s]) for s <= t (Keye-VL-2.0
// report section 2.3.1; xllm-io review page "核心公式", first formula), with one
// FP8 key vector per token shared by all indexer heads.
//
// FP8 prefill kernel: the dot products run on the 16x16x128 FP8 matrix core
// with d_I = 128 as the whole contraction.  A (rows) = 16 keys, B (columns) =
// 16 query tokens for one indexer head j, so each lane's four results are four
// keys of ONE token and the head loop stays inside the lane: no cross-lane
// reduction.  The per-token scales factor out of the ReLU (they are positive)
// and are applied once in the epilogue.
//
// The head sum is evaluated through ReLU(x) = (x + |x|) / 2:
//   sum_j w_j ReLU(x_j) = 1/2 (qmix . k) + 1/2 sum_j w_j |x_j|,
//   qmix = sum_j w_j q_j  (the w-weighted mix of the token's indexer queries).
// The first term is one dot product per (token, key) pair for all heads; a
// pre-pass builds qmix per token as a bf16 hi + lo pair (about 16 significant
// bits) and the main kernel seeds its accumulators with it on the bf16 matrix
// core (keys are exact in bf16).  The second term then costs ONE vector
// instruction per product, an fma with an |x| source modifier, instead of a
// max and an fma.  On gfx950 a wave's vector ALU work does not overlap its own
// matrix-core work, so halving it is worth about 1.3x on this kernel.
//
// The rewrite is exact algebra but not exact arithmetic: when most heads' dot
// products are negative, the two terms nearly cancel and their rounding errors
// (the FP8 matrix core aligns its products to the largest one with about 2^-15
// of Sigma|products| of error; the bf16 hi + lo qmix carries 2^-17) are left
// over a small or zero score.  So each score is checked: with A = sum_j w_j |x_j|
// and L = qmix . k, a wave whose block holds any entry with
// |A| + |L| > kCancel * |A + L| (at w >= 0: the negative heads outweigh the
// positive ones 7 to 1) recomputes that block exactly in the direct form,
// sum_j w_j max(x_j, 0), with x_j from the bf16 matrix core on the exact bf16
// values of the codes (fp32 accumulation; exact zeros stay zero).  Measured on
// gfx950 against the exact scores: below that ratio the rewrite's error stays
// under a quarter of the score tolerance; Gaussian queries and keys almost
// never reach it, so the check costs about two vector instructions per score.
//
// A wave keeps its NK key tiles (16*NK keys, 8 VGPRs each) in registers for the
// whole head loop.  The four waves of a workgroup share the same 16 tokens, so
// q^I is staged cooperatively in LDS, 8 heads (16 KB) at a time and
// double-buffered: the next batch's global loads are in flight while the
// current batch runs on the matrix cores.  Within a batch the loop is software
// pipelined by one head: the MFMAs of head j are issued before the epilogue of
// head j-1, whose results are then long complete.  Work items are ordered token-tile-major and
// mapped so that consecutive items run on one XCD: the key blocks of a token
// tile are processed together and the tile's 128 KB of q^I stays in that
// XCD's L2.
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

// Exact OCP E4M3 decode (bias 7, 3 mantissa bits; finite codes).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20))
                        : (float)m * 0.001953125f;           // m * 2^-9
    return (c & 0x80u) ? -mag : mag;
}

// qmix[t] = sum_j w[t,j] * fp8(q^I[t,j,:]) as bf16 hi [t][0][:] and lo [t][1][:]
// (hi = RNE(qmix), lo = RNE(qmix - hi)).  One wave per token, two dims per lane.
__global__ __launch_bounds__(256) void qmix_kernel(const uint8_t* __restrict__ q_idx,
                                                   const float* __restrict__ w, int Tq, int HI,
                                                   uint16_t* __restrict__ qmix)
{
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (t >= Tq) return;
    const uint8_t* q = q_idx + (int64_t)t * HI * 128 + 2 * lane;
    const float* wr = w + (int64_t)t * HI;
    float s0 = 0.f, s1 = 0.f;
    for (int j = 0; j < HI; ++j) {
        const uint32_t two = *reinterpret_cast<const uint16_t*>(q + (int64_t)j * 128);
        const float wj = wr[j];
        s0 = fmaf(wj, e4m3_to_f32(two & 0xffu), s0);
        s1 = fmaf(wj, e4m3_to_f32(two >> 8), s1);
    }
    const uint16_t h0 = f32_to_bf16_bits(s0), h1 = f32_to_bf16_bits(s1);
    const uint16_t l0 = f32_to_bf16_bits(s0 - bf16_bits_to_f32(h0));
    const uint16_t l1 = f32_to_bf16_bits(s1 - bf16_bits_to_f32(h1));
    uint32_t* out = reinterpret_cast<uint32_t*>(qmix + (int64_t)t * 256);
    out[lane] = h0 | ((uint32_t)h1 << 16);
    out[64 + lane] = l0 | ((uint32_t)l1 << 16);
}

// Eight FP8 codes (bytes 8m .. 8m+7 of a key slice) as eight bf16 values (exact).
__device__ __forceinline__ v8bf fp8x8_to_bf16(const v8i& a, int m) {
    typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
    const uint32_t d0 = (uint32_t)a[2 * m], d1 = (uint32_t)a[2 * m + 1];
    const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false);
    const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true);
    const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false);
    const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true);
    return v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Cancellation guard of the |x| rewrite (see the file header).
constexpr float kCancel = 15.f;

// Guard metric of one entry: > 0 when the rewrite cannot be trusted for it.
__device__ __forceinline__ float cancel_metric(float a, float l) {
    return fabsf(a) + fabsf(l) - kCancel * fabsf(a + l);
}

// Exact direct form for NK key tiles of one wave: ex[i][e] = 2 sum_j w_j max(x_j, 0) for the
// heads j0 .. j1-1 staged at q_row (head j at q_row + j * head_stride bytes; this lane's
// 32-byte slice) with weights w_row[j * w_stride], added to ex.  x_j comes from the bf16 matrix
// core on the exact bf16 values of the FP8 codes (fp32 accumulation).  ka: the key tiles'
// bf16 operands.  Factor 2: the epilogue scales by q_scale / 2 for the rewrite's halves.
template <int NK>
__device__ __forceinline__ void exact_heads(const v8bf (&ka)[NK][4], const uint8_t* q_row,
                                            int head_stride, const float* w_row, int w_stride,
                                            int j0, int j1, float (&ex)[NK][4]) {
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    for (int j = j0; j < j1; ++j) {
        const uint8_t* qp = q_row + j * head_stride;
        const v4i lo = *reinterpret_cast<const v4i*>(qp);
        const v4i hi = *reinterpret_cast<const v4i*>(qp + 16);
        const v8i qc = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        const float w2 = 2.f * w_row[j * w_stride];
        v4f x[NK];
#pragma unroll
        for (int i = 0; i < NK; ++i) x[i] = zero;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const v8bf qb = fp8x8_to_bf16(qc, m);
#pragma unroll
            for (int i = 0; i < NK; ++i) x[i] = mfma_bf16_16x16x32(ka[i][m], qb, x[i]);
        }
#pragma unroll
        for (int i = 0; i < NK; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) ex[i][e] = fmaf(w2, fmaxf(x[i][e], 0.f), ex[i][e]);
    }
}

constexpr int kHeadBatch = 8;            // indexer heads staged in LDS at a time
constexpr int kQPitch = 144;             // LDS row pitch (bytes) of one token's 128 codes

template <int NK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void index_fp8_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ k_idx,
    const float* __restrict__ k_scale, const uint16_t* __restrict__ qmix, int Tq, int Tk,
    int HI, int64_t q_pos0, float* __restrict__ scores, int64_t ld, int n_kb)
{
    constexpr int kKeysPerWave = 16 * NK;
    constexpr int kKeysPerWG = kIdxWaves * kKeysPerWave;
    // q^I of the workgroup's 16 tokens for one batch of heads, double-buffered
    __shared__ __attribute__((aligned(16))) uint8_t q_lds[2][kHeadBatch][16][kQPitch];
    __shared__ float w_lds[2][kHeadBatch][16];

    const int work = xcd_remap(blockIdx.x, gridDim.x);
    const int tt = work / n_kb;
    const int kb = work - tt * n_kb;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, grp = lane >> 4;

    const int t0 = tt * 16;
    const int t = t0 + col;                           // this lane's query row
    const bool t_ok = t < Tq;
    const int tc = t_ok ? t : Tq - 1;
    const int64_t pos = q_pos0 + t;
    const int64_t pos_hi = q_pos0 + min(t0 + 15, Tq - 1);
    const int wg_base = kb * kKeysPerWG;
    const int s_base = wg_base + wave * kKeysPerWave;
    float* __restrict__ out_row = scores + (int64_t)tc * ld;
    // a wave tile entirely above the diagonal (or past Tk) only writes -inf
    const bool active = s_base < Tk && (int64_t)s_base <= pos_hi;

    auto fill_masked = [&]() {
        if (!t_ok || s_base >= Tk) return;
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
    };
    if ((int64_t)wg_base > pos_hi) {                  // uniform over the workgroup
        fill_masked();
        return;
    }

    // A operands: key rows s_base + 16 i + col, 32 bytes per lane (slice grp)
    v8i a[NK];
#pragma unroll
    for (int i = 0; i < NK; ++i) {
        const int s = s_base + 16 * i + col;
        a[i] = (active && s < Tk) ? load32B(k_idx + (int64_t)s * 128 + grp * 32)
                                  : v8i{0, 0, 0, 0, 0, 0, 0, 0};
    }

    // cooperative staging of one head batch: 1024 16-byte chunks, 4 per thread
    const int n_batch = (HI + kHeadBatch - 1) / kHeadBatch;
    v4i stage[4];
    float wstage = 0.f;
    auto load_batch = [&](int b) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int id = tid + 256 * i;
            const int c = id & 7, tok = (id >> 3) & 15, hh = id >> 7;
            const int h = b * kHeadBatch + hh;
            const int tr = min(t0 + tok, Tq - 1);
            stage[i] = (h < HI) ? *reinterpret_cast<const v4i*>(q_idx + ((int64_t)tr * HI + h) * 128 + c * 16)
                                : v4i{0, 0, 0, 0};
        }
        if (tid < 16 * kHeadBatch) {
            const int tok = tid & 15, hh = tid >> 4;
            const int h = b * kHeadBatch + hh;
            wstage = (h < HI) ? w[(int64_t)min(t0 + tok, Tq - 1) * HI + h] : 0.f;
        }
    };
    auto store_batch = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int id = tid + 256 * i;
            const int c = id & 7, tok = (id >> 3) & 15, hh = id >> 7;
            *reinterpret_cast<v4i*>(&q_lds[buf][hh][tok][c * 16]) = stage[i];
        }
        if (tid < 16 * kHeadBatch) w_lds[buf][tid >> 4][tid & 15] = wstage;
    };

    // acc = sum_j w_j |x_j| over the head loop; the linear term qmix . k follows it
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    float acc[NK][4];
#pragma unroll
    for (int i = 0; i < NK; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][e] = 0.f;
    // the epilogue of "head -1" adds 0 * max(0, 0): no special first iteration
    v4f dprev[NK];
#pragma unroll
    for (int i = 0; i < NK; ++i) dprev[i] = zero;
    float wprev = 0.f;

    load_batch(0);
    store_batch(0);
    __syncthreads();
    for (int b = 0; b < n_batch; ++b) {
        const int buf = b & 1;
        if (b + 1 < n_batch) load_batch(b + 1);       // in flight during this batch's math
        if (active) {
#pragma unroll
            for (int hh = 0; hh < kHeadBatch; ++hh) {
                const uint8_t* qrow = &q_lds[buf][hh][col][grp * 32];
                const v4i lo = *reinterpret_cast<const v4i*>(qrow);
                const v4i hi = *reinterpret_cast<const v4i*>(qrow + 16);
                const v8i bq = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                const float wj = w_lds[buf][hh][col];
                v4f dcur[NK];
#pragma unroll
                for (int i = 0; i < NK; ++i) dcur[i] = mfma_fp8_16x16x128(a[i], bq, zero);
                // w-weighted |x| of the previous head while these run (one fma each)
#pragma unroll
                for (int i = 0; i < NK; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[i][e] = fmaf(wprev, fabsf(dprev[i][e]), acc[i][e]);
#pragma unroll
                for (int i = 0; i < NK; ++i) dprev[i] = dcur[i];
                wprev = wj;
            }
        }
        if (b + 1 < n_batch) store_batch(buf ^ 1);
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < NK; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][e] = fmaf(wprev, fabsf(dprev[i][e]), acc[i][e]);
    // the linear term (bf16 matrix core) and the cancellation guard
    bool redo = false;
    if (active) {
        const uint16_t* qm = qmix + (int64_t)tc * 256 + grp * 32;
        float worst = -INFINITY;
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            v4f lin = zero;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const v8bf bh = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4i*>(qm + 8 * m));
                const v8bf bl = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4i*>(qm + 128 + 8 * m));
                const v8bf ka = fp8x8_to_bf16(a[i], m);
                lin = mfma_bf16_16x16x32(ka, bh, lin);
                lin = mfma_bf16_16x16x32(ka, bl, lin);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                worst = fmaxf(worst, cancel_metric(acc[i][e], lin[e]));
                acc[i][e] += lin[e];
            }
        }
        redo = __ballot(worst > 0.f) != 0;            // uniform over the wave
    }
    // a wave with an entry the rewrite cannot be trusted for recomputes its block exactly;
    // the whole workgroup stages q^I again, one head batch at a time
    if (__syncthreads_or(redo)) {
        v8bf ka[NK][4];
        if (redo) {
#pragma unroll
            for (int i = 0; i < NK; ++i)
#pragma unroll
                for (int m = 0; m < 4; ++m) ka[i][m] = fp8x8_to_bf16(a[i], m);
#pragma unroll
            for (int i = 0; i < NK; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][e] = 0.f;
        }
        for (int b = 0; b < n_batch; ++b) {
            load_batch(b);
            store_batch(0);
            __syncthreads();
            if (redo)
                exact_heads<NK>(ka, &q_lds[0][0][col][grp * 32], 16 * kQPitch, &w_lds[0][0][col],
                                16, 0, kHeadBatch, acc);
            __syncthreads();
        }
    }
    if (!active) {
        fill_masked();
        return;
    }

    if (!t_ok) return;
    const float qs = 0.5f * q_scale[tc];                // (linear + |x| terms) / 2
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

// Resident-q variant for HI <= 64: a workgroup of 16 waves loads the whole q^I
// tile of its 16 tokens (all heads, 144 KB with padding) into LDS once, then
// walks a group of key blocks (1024 keys each, 64 per wave) with no further
// barrier.  Each wave's keys live in registers for its head loop; with four
// waves per SIMD drifting out of phase, one wave's matrix-core work overlaps
// another's vector ALU work and memory waits (a wave's own VALU and MFMA
// instructions do not overlap on gfx950).
//
// Three output modes share the arithmetic, so a score is the same bits in each:
//   kModeScores      every causal score of the chunk into scores[row, s] (-inf above the
//                    diagonal), optionally gated by a device flag (*run_if != 0);
//   kModeSample      the scores of S sampled key positions per token tile (stratified over
//                    [0, t0] with a hashed offset in each stratum) into samples[row, j];
//   kModeCandidates  only the causal scores >= tau[row] (a finite bound), appended as
//                    (key, position) pairs to the row's list (atomic counter per row; at most
//                    cap pairs are stored, the counter keeps counting).
#ifndef DSA_IDX_RES_NK
#define DSA_IDX_RES_NK 4
#endif
#ifndef DSA_IDX_RES_WAVES
#define DSA_IDX_RES_WAVES 16
#endif
constexpr int kResHeads = 64;
constexpr int kResWaves = DSA_IDX_RES_WAVES;
constexpr int kResNK = DSA_IDX_RES_NK;
constexpr int kModeScores = 0, kModeSample = 1, kModeCandidates = 2;

// Sampled key position j of a token tile whose first token sees keys 0 .. n0-1: one key in
// each of S equal strata of [0, n0), at a hashed offset inside its stratum.
__device__ __forceinline__ int sample_pos(int j, int S, int n0, int tile) {
    const int lo = (int)((int64_t)j * n0 / S);
    const int hi = (int)((int64_t)(j + 1) * n0 / S);
    uint32_t h = (uint32_t)j * 0x9E3779B1u ^ (uint32_t)tile * 0x85EBCA77u;
    h ^= h >> 15; h *= 0x2C1B3C6Du; h ^= h >> 12;
    const int width = hi - lo;
    return width > 1 ? lo + (int)(h % (uint32_t)width) : min(lo, n0 - 1);
}

// Token tiles of 16 rows, counted from the chunk's first, whose last token (position
// q_pos0 + min(16 tt + 15, Tq - 1)) sees no key at or after k0: the tiles that have no causal
// score in a key group starting at k0.
__host__ __device__ inline int tiles_above(int64_t k0, int64_t q_pos0, int Tq, int n_tt) {
    const int64_t d = k0 - q_pos0;
    if (d >= Tq) return n_tt;
    if (d <= 0) return 0;
    const int64_t full = d / 16;            // tiles before the last one: 16 tt + 16 <= d
    return full < n_tt - 1 ? (int)full : n_tt - 1;
}

struct ResOut {
    float* scores; int64_t ld;                  // kModeScores
    const int* run_if;                          // kModeScores: skip unless *run_if != 0 (nullable)
    float* samples; int S;                      // kModeSample: [rows, S]
    const float* tau; int32_t* cnt;             // kModeCandidates: per-row bound and counter
    uint2* cand; int cap;                       //   [rows, cap] of (order key, position)
};

template <int NK, int MODE>
__global__ __launch_bounds__(kResWaves * 64) __attribute__((amdgpu_waves_per_eu(kResWaves / 4, kResWaves / 4)))
void index_fp8_resident_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ k_idx,
    const float* __restrict__ k_scale, const uint16_t* __restrict__ qmix, int Tq, int Tk,
    int HI, int64_t q_pos0, ResOut o, int n_kb, int n_kg, int kg, int n_work)
{
    constexpr int kKeysPerWave = 16 * NK;
    constexpr int kKeysPerBlock = kResWaves * kKeysPerWave;
    __shared__ __attribute__((aligned(16))) uint8_t q_lds[kResHeads][16][kQPitch];
    __shared__ float w_lds[kResHeads][16];
    __shared__ __attribute__((aligned(16))) uint16_t qm_lds[16][264];   // padded rows: no bank conflicts

    if (MODE == kModeScores && o.run_if && *o.run_if == 0) return;
    // The first n_work workgroups are the (key group, token tile) pairs with causal scores,
    // key-group-major and without the tiles wholly above the diagonal, so that equal
    // contiguous shares of them (one per XCD) carry about equal work and the workgroups
    // resident on one XCD share a key group (hot in that XCD's L2).  In kModeScores the
    // workgroups after them fill the pairs above the diagonal with -inf.
    const int n_tt = (Tq + 15) / 16;
    const bool fill = (int)blockIdx.x >= n_work;
    int g = 0, tt = 0;
    {
        int rem = fill ? (int)blockIdx.x - n_work : xcd_remap(blockIdx.x, n_work);
        for (;; ++g) {
            const int above = MODE == kModeSample
                ? 0 : tiles_above((int64_t)g * kg * kKeysPerBlock, q_pos0, Tq, n_tt);
            const int here = fill ? above : n_tt - above;
            if (rem < here || g == n_kg - 1) { tt = (fill ? 0 : above) + rem; break; }
            rem -= here;
        }
    }
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int t0 = tt * 16;
    const int t = t0 + col;
    const bool t_ok = t < Tq;
    const int tc = t_ok ? t : Tq - 1;
    const int64_t pos = q_pos0 + t;
    const int64_t pos_hi = q_pos0 + min(t0 + 15, Tq - 1);
    const int kb_begin = g * kg, kb_end = min(n_kb, kb_begin + kg);
    // keys the tile's first token sees (the sample strata cover them)
    const int n0 = (int)min<int64_t>(q_pos0 + t0 + 1, Tk);
    float* __restrict__ out_row = MODE == kModeScores ? o.scores + (int64_t)tc * o.ld : nullptr;

    // whole group above the diagonal: only -inf to write.  Each wave fills whole token rows
    // of the group's columns, 1 KiB per instruction.
    if (MODE == kModeScores && fill) {
        const int c_end = min(kb_end * kKeysPerBlock, Tk);
        const float4 ninf = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        static_assert(kResWaves == 16 || kResWaves == 8 || kResWaves == 4, "rows per wave");
#pragma unroll
        for (int rr = 0; rr < 16 / kResWaves; ++rr) {
            const int r = wave + rr * kResWaves;
            if (t0 + r >= Tq) break;
            float* __restrict__ row_w = o.scores + (int64_t)(t0 + r) * o.ld;
            for (int c = kb_begin * kKeysPerBlock + 4 * lane; c < c_end; c += 256) {
                if (c + 3 < c_end) {
                    *reinterpret_cast<float4*>(row_w + c) = ninf;
                } else {
                    for (int e = 0; e < 4; ++e)
                        if (c + e < c_end) row_w[c + e] = -INFINITY;
                }
            }
        }
        return;
    }

    // stage q^I (all heads, padded to a multiple of 8 with zeros), w and qmix
    const int HP = (HI + 7) & ~7;
    for (int id = tid; id < 16 * HP * 8; id += kResWaves * 64) {
        const int c = id & 7, rest = id >> 3;
        const int h = rest % HP, tok = rest / HP;
        const int tr = min(t0 + tok, Tq - 1);
        const v4i v = (h < HI) ? *reinterpret_cast<const v4i*>(q_idx + ((int64_t)tr * HI + h) * 128 + c * 16)
                               : v4i{0, 0, 0, 0};
        *reinterpret_cast<v4i*>(&q_lds[h][tok][c * 16]) = v;
    }
    for (int id = tid; id < 16 * HP; id += kResWaves * 64) {
        const int h = id % HP, tok = id / HP;
        w_lds[h][tok] = (h < HI) ? w[(int64_t)min(t0 + tok, Tq - 1) * HI + h] : 0.f;
    }
    for (int id = tid; id < 16 * 32; id += kResWaves * 64) {
        const int c = id & 31, tok = id >> 5;
        *reinterpret_cast<v4i*>(&qm_lds[tok][c * 8]) =
            *reinterpret_cast<const v4i*>(qmix + (int64_t)min(t0 + tok, Tq - 1) * 256 + c * 8);
    }
    __syncthreads();

    const float qs = 0.5f * q_scale[tc];              // (linear + |x| terms) / 2
    const float tau_t = MODE == kModeCandidates ? o.tau[tc] : 0.f;
    const int pos32 = (int)pos;                       // pos < Tk <= INT32_MAX
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    const int n_keys = MODE == kModeSample ? o.S : Tk;   // logical keys of this launch

    // key row of tile i of a wave block (sampled positions in kModeSample; rows >= Tk are
    // clamped into the array: they lie above the diagonal and are masked)
    auto key_row = [&](int s_base, int i) {
        return MODE == kModeSample ? sample_pos(min(s_base + 16 * i + col, n_keys - 1), o.S, n0, tt)
                                   : min(s_base + 16 * i + col, Tk - 1);
    };
    // scale, causal mask and output of one wave block (keys s_base ..) from its head sums
    auto finish = [&](const int s_base, float (&acc)[NK][4], const float (&ksl)[NK]) {
        // every lane takes part in the scale shuffles (no early exit for tokens past Tq),
        // and every path consumes the scale loads before the next block reuses them
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            // causal limit in 32 bits: key s0 + e is visible iff e <= pos - s0
            const int lim = pos32 - (s_base + 16 * i + 4 * grp);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float ks = __shfl(ksl[i], 4 * grp + e, 64);   // lane 4 grp + e loaded key s0 + e
                const float r = acc[i][e] * (qs * ks);
                acc[i][e] = (MODE == kModeSample || e <= lim) ? r : -INFINITY;
            }
        }
        if (MODE == kModeCandidates) {
            // lane (col, grp) holds keys s_base + 16 i + 4 grp + e of token col; keep the ones
            // at or above the row's bound (entries above the diagonal hold -inf, below any
            // bound; the bound is finite) and reserve room with one atomic per token
            uint32_t keep = 0;
#pragma unroll
            for (int i = 0; i < NK; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) keep |= (acc[i][e] >= tau_t ? 1u : 0u) << (4 * i + e);
            if (!t_ok) keep = 0;
            // counts over the token's four lanes (grp 0..3) with lane-xor exchanges only
            const uint32_t c = __popc(keep);
            const uint32_t x1 = __shfl_xor(c, 16, 64);        // grp ^ 1
            const uint32_t pair = c + x1;
            const uint32_t x2 = __shfl_xor(pair, 32, 64);     // the other pair
            const uint32_t total = pair + x2;
            uint32_t b0 = 0;
            if (grp == 0 && total) b0 = (uint32_t)atomicAdd(o.cnt + t, (int)total);
            const uint32_t b1 = b0 + __shfl_xor(b0, 16, 64);
            uint32_t off = b1 + __shfl_xor(b1, 32, 64);       // the token's base (from grp 0)
            off += ((grp & 2) ? x2 : 0u) + ((grp & 1) ? x1 : 0u);
            // rows of this token tile start at the uniform t0 * cap; 32-bit offsets within
            uint2* __restrict__ dst = o.cand + (int64_t)t0 * o.cap;
            const uint32_t row_off = (uint32_t)col * (uint32_t)o.cap;
#pragma unroll
            for (int i = 0; i < NK; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (keep & (1u << (4 * i + e))) {
                        if (off < (uint32_t)o.cap)
                            dst[row_off + off] = make_uint2(order_key(acc[i][e]),
                                                            (uint32_t)(s_base + 16 * i + 4 * grp + e));
                        ++off;
                    }
            return;
        }
        if (!t_ok) return;
        float* __restrict__ dst = MODE == kModeSample ? o.samples + (int64_t)tc * o.S : out_row;
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int s0 = s_base + 16 * i + 4 * grp;
            if (MODE == kModeSample || s0 + 3 < Tk) {
                *reinterpret_cast<float4*>(dst + s0) = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
            } else {
                for (int e = 0; e < 4; ++e)
                    if (s0 + e < Tk) dst[s0 + e] = acc[i][e];
            }
        }
    };

    uint32_t redo = 0;            // wave blocks (bit kb - kb_begin) to recompute exactly
    for (int kb = kb_begin; kb < kb_end; ++kb) {
        const int s_base = kb * kKeysPerBlock + wave * kKeysPerWave;   // logical key index
        if (s_base >= n_keys) break;
        if (MODE != kModeSample && (int64_t)s_base > pos_hi) {   // wave tile above the diagonal
            if (MODE == kModeScores && t_ok) {
#pragma unroll
                for (int i = 0; i < NK; ++i) {
                    const int s0 = s_base + 16 * i + 4 * grp;
                    if (s0 + 3 < Tk)
                        *reinterpret_cast<float4*>(out_row + s0) =
                            make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
                    else
                        for (int e = 0; e < 4; ++e)
                            if (s0 + e < Tk) out_row[s0 + e] = -INFINITY;
                }
            }
            continue;
        }
        // keys (A operands) of this wave, 16 NK keys, 32 bytes per lane per tile, and the
        // scale of key 16 i + col: unconditional loads from rows clamped into the array
        // (keys s >= Tk lie above the diagonal and are masked below), so no branch makes
        // the compiler wait for them before it has to
        v8i a[NK];
        float ksl[NK];
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int s = key_row(s_base, i);
            a[i] = load32B(k_idx + (int64_t)s * 128 + grp * 32);
            ksl[i] = k_scale[s];
        }
        // all of the block's loads are in flight before any math: keep the compiler
        // from sinking some of them below the first uses of the others
        asm volatile("" ::: "memory");
        // head loop, acc = sum_j w_j |x_j|: the B operand (q^I of head j for the 16 tokens)
        // is read from LDS one head ahead, and the |x| epilogue of head j-1 follows the
        // MFMAs of head j
        float acc[NK][4];
#pragma unroll
        for (int i = 0; i < NK; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][e] = 0.f;
        v4f dprev[NK];
#pragma unroll
        for (int i = 0; i < NK; ++i) dprev[i] = zero;
        float wprev = 0.f;
        const uint8_t* qbase = &q_lds[0][col][grp * 32];
        v4i nlo = *reinterpret_cast<const v4i*>(qbase);
        v4i nhi = *reinterpret_cast<const v4i*>(qbase + 16);
        float nw = w_lds[0][col];
        for (int j0 = 0; j0 < HP; j0 += 8) {
#pragma unroll
            for (int hh = 0; hh < 8; ++hh) {
                const int j = j0 + hh;
                const v8i bq = {nlo.x, nlo.y, nlo.z, nlo.w, nhi.x, nhi.y, nhi.z, nhi.w};
                const float wj = nw;
                const int jn = (j + 1 < HP) ? j + 1 : j;
                nlo = *reinterpret_cast<const v4i*>(qbase + jn * 16 * kQPitch);
                nhi = *reinterpret_cast<const v4i*>(qbase + jn * 16 * kQPitch + 16);
                nw = w_lds[jn][col];
                v4f dcur[NK];
#pragma unroll
                for (int i = 0; i < NK; ++i) dcur[i] = mfma_fp8_16x16x128(a[i], bq, zero);
#pragma unroll
                for (int i = 0; i < NK; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[i][e] = fmaf(wprev, fabsf(dprev[i][e]), acc[i][e]);
#pragma unroll
                for (int i = 0; i < NK; ++i) dprev[i] = dcur[i];
                wprev = wj;
            }
        }
#pragma unroll
        for (int i = 0; i < NK; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][e] = fmaf(wprev, fabsf(dprev[i][e]), acc[i][e]);
        // the linear term qmix . k (bf16 matrix core), one 32-wide slice m of the contraction
        // at a time for every tile, then the cancellation guard
        {
            const uint16_t* qm = &qm_lds[col][grp * 32];
            v4f lin[NK];
#pragma unroll
            for (int i = 0; i < NK; ++i) lin[i] = zero;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const v8bf bh = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4i*>(qm + 8 * m));
                const v8bf bl = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4i*>(qm + 128 + 8 * m));
#pragma unroll
                for (int i = 0; i < NK; ++i) {
                    const v8bf ka = fp8x8_to_bf16(a[i], m);
                    lin[i] = mfma_bf16_16x16x32(ka, bh, lin[i]);
                    lin[i] = mfma_bf16_16x16x32(ka, bl, lin[i]);
                }
            }
            float worst = -INFINITY;
#pragma unroll
            for (int i = 0; i < NK; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    worst = fmaxf(worst, cancel_metric(acc[i][e], lin[i][e]));
                    acc[i][e] += lin[i][e];
                }
            if (__ballot(worst > 0.f) != 0) {          // uniform over the wave
                redo |= 1u << (kb - kb_begin);
                continue;
            }
        }
        finish(s_base, acc, ksl);
    }
    // blocks the rewrite cannot be trusted for: the direct form on the bf16 matrix core, one
    // key tile at a time, codes and scales loaded again (after the main loop, so that its
    // registers are free)
    while (redo != 0) {
        const int kb = kb_begin + __builtin_ctz(redo);
        redo &= redo - 1;
        const int s_base = kb * kKeysPerBlock + wave * kKeysPerWave;
        float acc[NK][4];
        float ksl[NK];
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int s = key_row(s_base, i);
            const v8i ki = load32B(k_idx + (int64_t)s * 128 + grp * 32);
            ksl[i] = k_scale[s];
            v8bf ka[1][4];
            float ex[1][4] = {{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int m = 0; m < 4; ++m) ka[0][m] = fp8x8_to_bf16(ki, m);
            exact_heads<1>(ka, &q_lds[0][col][grp * 32], 16 * kQPitch, &w_lds[0][col], 16, 0, HP,
                           ex);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][e] = ex[0][e];
        }
        finish(s_base, acc, ksl);
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
// lane groups.  The kernel is bound by the k^I stream (132 bytes per key), so
// registers go to pages in flight: the workgroup's four waves share the query's
// head tiles and weights through LDS, each wave owns kDecPagesPerWave
// consecutive pages (twice that when keeping candidates), reads their block ids
// once, and keeps the next kDecDepth pages' codes and scales in flight while it
// computes the current one.  Candidate mode holds both groups' scores and masks
// until its stores: it gets the registers of 3 waves per SIMD, not 4.
#ifndef DSA_DEC_PAGES_PER_WAVE
#define DSA_DEC_PAGES_PER_WAVE 8
#endif
#ifndef DSA_DEC_DEPTH
#define DSA_DEC_DEPTH 1
#endif
constexpr int kDecPagesPerWave = DSA_DEC_PAGES_PER_WAVE;
static_assert(kDecPagesPerWave >= 1 && kDecPagesPerWave <= 64, "block ids live one per lane");
constexpr int kDecDepth = DSA_DEC_DEPTH;
constexpr int kDecQPitch = 144;                    // bytes per head row in LDS (conflict-free b128 reads)

struct PageRegs {
    v8i k[4];          // four 16-key tiles of the page (this lane: key 16 u + col, slice grp)
    float scale;       // k_scale of key `lane` of the page
};

#ifndef DSA_DEC_WAVES
#define DSA_DEC_WAVES 4
#endif
// Output modes, as in the prefill kernel: every score of the sequence into scores[b, s];
// the scores of S sampled positions (per-key stratified, hashed offsets) into
// samples[b, j] (a "page" is then 64 consecutive samples); or only the scores >= tau[b]
// appended as (order key, position) to the sequence's list, one atomic per group of pages.
struct PagedOut {
    float* scores; int64_t ld; const int* run_if;
    float* samples; int S;
    const float* tau; int32_t* cnt; uint2* cand; int cap;
};

// Sampled keys cost two dependent round trips per page (block id, then key) and a sample
// launch is small, so its waves take fewer pages each.  A candidate-mode wave takes two
// groups of pages: the slot reservation (an atomic round trip) of the first group is issued
// between the groups and its reply arrives while the second group streams, so only one
// reservation per 2 kDecPagesPerWave pages is waited for.
template <int MODE> constexpr int paged_groups() { return MODE == kModeCandidates ? 2 : 1; }
template <int MODE> constexpr int paged_ppw() {
    return MODE == kModeSample ? 2 : kDecPagesPerWave * paged_groups<MODE>();
}

template <int NHT, int MODE>                       // 16-head tiles of the query
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MODE == kModeCandidates ? 3 : DSA_DEC_WAVES)))
void index_fp8_paged_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ kcache,
    const float* __restrict__ kscale, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, int num_blocks, int max_blocks, int block_size, int HI,
    PagedOut o, int n_split)
{
    constexpr int PPW = paged_ppw<MODE>();
    __shared__ __attribute__((aligned(16))) uint8_t q_lds[16 * NHT * kDecQPitch];
    __shared__ __attribute__((aligned(16))) float w_lds[16 * NHT];
    if (MODE == kModeScores && o.run_if && *o.run_if == 0) return;
    // block_size is 64 here (checked by the launcher): one page = one 64-key iteration
    const int work = xcd_remap(blockIdx.x, gridDim.x);
    const int b = work / n_split, sp = work - b * n_split;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int page0 = (sp * kIdxWaves + wave) * PPW;

    // 1. one round trip for everything the pages depend on: the sequence length,
    //    the block ids of this wave's pages (clamped into the table row), the
    //    query's head rows (heads >= HI read head HI-1 and are zeroed) and weights
    const int64_t len = seq_lens[b];
    const int bt = MODE == kModeSample ? 0 : block_table[(int64_t)b * max_blocks +
                               min(page0 + min(lane, PPW - 1), max_blocks - 1)];
    constexpr int kQChunks = 16 * NHT * 8;         // 16-byte chunks of the head tiles
    constexpr int kQPer = (kQChunks + 255) / 256;
    v4i qv[kQPer];
    const uint8_t* qrow = q_idx + (int64_t)b * HI * 128;
#pragma unroll
    for (int r = 0; r < kQPer; ++r) {
        const int c = min(tid + 256 * r, kQChunks - 1), h = c >> 3;
        qv[r] = *reinterpret_cast<const v4i*>(qrow + (int64_t)min(h, HI - 1) * 128 + (c & 7) * 16);
    }
    const float wq = w[(int64_t)b * HI + min(tid, HI - 1)];
    const float qs = q_scale[b];
    const float tau_b = MODE == kModeCandidates ? o.tau[b] : 0.f;

    const int64_t cap = (int64_t)max_blocks * 64;
    if (len < 1 || len > cap || num_blocks <= 0) return;       // uniform over the workgroup
    // pages of this launch: the sequence's key pages, or S / 64 pages of samples
    const int n_pages = MODE == kModeSample ? o.S / 64 : (int)((len + 63) >> 6);
    if (sp * kIdxWaves * PPW >= n_pages) return;   // uniform over the workgroup
    const int np = max(0, min(PPW, n_pages - page0));
    // 2. block ids of this wave's pages (-1 when outside the cache)
    const int blk_l = (lane < np && bt >= 0 && bt < num_blocks) ? bt : -1;
    const int last = max(np - 1, 0);
    // unconditional loads (an invalid block reads block 0 and is masked to -inf
    // afterwards): no branch around them, so the next pages stay in flight
    auto fetch = [&](int i, PageRegs& r) {
        if (MODE == kModeSample) {
            // lane (col, grp) loads sample 64 pg + 16 u + col of tile u, and the scale of
            // sample 64 pg + lane (tile grp); an invalid block id reads row 0 and is masked
            const int pg = page0 + i;
            int srow = 0;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int pos = sample_pos(min(pg * 64 + 16 * u + col, o.S - 1), o.S, (int)len, b);
                const int blk = block_table[(int64_t)b * max_blocks + (pos >> 6)];
                const int row = (blk >= 0 && blk < num_blocks) ? blk * 64 + (pos & 63) : -1;
                r.k[u] = load32B(kcache + (int64_t)max(row, 0) * 128 + grp * 32);
                if (u == grp) srow = row;
            }
            r.scale = srow >= 0 ? kscale[srow] : -INFINITY;   // -inf scale marks the sample invalid
            return;
        }
        const int blk = __shfl(blk_l, i, 64);
        const int64_t base = (int64_t)(blk < 0 ? 0 : blk) * 64;
#pragma unroll
        for (int u = 0; u < 4; ++u) r.k[u] = load32B(kcache + (base + 16 * u + col) * 128 + grp * 32);
        r.scale = kscale[base + lane];
    };
    PageRegs ring[kDecDepth + 1];
    float res[PPW];                   // scores, stored after the page loop
    constexpr int NG = paged_groups<MODE>(), GP = PPW / NG;
    uint64_t kept[PPW];               // candidate mode: lanes of each page at or above the bound
    uint32_t gbase[NG];               // candidate mode: first slot of each group (lane 0)
    // candidate mode: group g's kept scores as (order key, position) from its reserved slot
    auto write_group = [&](int g) {
        uint2* __restrict__ dst = o.cand + (int64_t)b * o.cap;
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        // the reply is read here, not where the atomic was issued
        uint32_t gb = gbase[g];
        asm volatile("" : "+v"(gb));
        uint32_t base = __shfl(gb, 0, 64);
#pragma unroll
        for (int j = g * GP; j < (g + 1) * GP; ++j) {
            const uint32_t slot = base + __popcll(kept[j] & below);
            if (((kept[j] >> lane) & 1ull) && slot < (uint32_t)o.cap)
                dst[slot] = make_uint2(order_key(res[j]), (uint32_t)((page0 + j) * 64 + lane));
            base += __popcll(kept[j]);
        }
    };
#pragma unroll
    for (int i = 0; i < kDecDepth; ++i) fetch(min(i, last), ring[i]);
    // 3. stage the head tiles and weights while the first pages are in flight
#pragma unroll
    for (int r = 0; r < kQPer; ++r) {
        const int c = tid + 256 * r;
        if (c < kQChunks) {
            const int h = c >> 3;
            *reinterpret_cast<v4i*>(q_lds + h * kDecQPitch + (c & 7) * 16) =
                (h < HI) ? qv[r] : v4i{0, 0, 0, 0};
        }
    }
    if (tid < 16 * NHT) w_lds[tid] = (tid < HI) ? wq : 0.f;
    __syncthreads();

    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    // fully unrolled (a rolled loop makes the compiler wait on in-flight pages at
    // the back edge): ring slots are compile-time constants
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
      if (i < np) {                   // uniform over the wave
        fetch(min(i + kDecDepth, last), ring[(i + kDecDepth) % (kDecDepth + 1)]);
        const PageRegs& cur = ring[i % (kDecDepth + 1)];
        // keep the compiler from hoisting the loop-invariant LDS tiles into registers
        asm volatile("" ::: "memory");
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < NHT; ++m) {
            const uint8_t* qa_p = q_lds + (16 * m + col) * kDecQPitch + grp * 32;
            v8i qa;
            const v4i lo = *reinterpret_cast<const v4i*>(qa_p);
            const v4i hi = *reinterpret_cast<const v4i*>(qa_p + 16);
            qa[0] = lo[0]; qa[1] = lo[1]; qa[2] = lo[2]; qa[3] = lo[3];
            qa[4] = hi[0]; qa[5] = hi[1]; qa[6] = hi[2]; qa[7] = hi[3];
            const v4f wv = *reinterpret_cast<const v4f*>(w_lds + 16 * m + 4 * grp);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const v4f d = mfma_fp8_16x16x128(qa, cur.k[u], zero);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[u] += wv[e] * fmaxf(d[e], 0.f);
            }
        }
        // acc[u] at lane (col, grp) is key 16 u + col over heads 4 grp .. 4 grp + 3 of
        // each tile; a two-step exchange leaves lane l with key l summed over all heads
        const bool b1 = grp & 2, b0 = grp & 1;
        float k0 = b1 ? acc[2] : acc[0], k1 = b1 ? acc[3] : acc[1];
        const float t0 = b1 ? acc[0] : acc[2], t1 = b1 ? acc[1] : acc[3];
        k0 += __shfl_xor(t0, 32, 64);
        k1 += __shfl_xor(t1, 32, 64);
        float mine = b0 ? k1 : k0;
        mine += __shfl_xor(b0 ? k0 : k1, 16, 64);
        if (MODE == kModeSample) {
            res[i] = cur.scale == -INFINITY ? -INFINITY : mine * (qs * cur.scale);
        } else {
            const bool valid = __shfl(blk_l, i, 64) >= 0;
            res[i] = valid ? mine * (qs * cur.scale) : -INFINITY;
        }
      }
        if (MODE == kModeCandidates && (i + 1) % GP == 0) {
            // keep the group's keys at or above the sequence's bound (invalid and
            // out-of-range keys hold -inf or are excluded); one atomic reserves the room,
            // its reply is read after the page loop
            const int g = i / GP;
            uint32_t total = 0;
#pragma unroll
            for (int j = g * GP; j < (g + 1) * GP; ++j) {
                const int64_t s = (int64_t)(page0 + j) * 64 + lane;
                kept[j] = __ballot(j < np && s < len && res[j] >= tau_b);
                total += __popcll(kept[j]);
            }
            gbase[g] = 0;
            if (lane == 0 && total) gbase[g] = (uint32_t)atomicAdd(o.cnt + b, (int)total);
        }
    }
    if (MODE == kModeCandidates) {
        // after the page loop: a wait for one reply here would also wait for the pages
        // in flight (the compiler does not count an atomic's reply in order with loads)
#pragma unroll
        for (int g = 0; g < NG; ++g) write_group(g);
        return;
    }
    // score stores interleaved with the page stream slow it down: issue them last
    float* __restrict__ out = MODE == kModeSample ? o.samples + (int64_t)b * o.S : o.scores + (int64_t)b * o.ld;
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
        if (i >= np) break;
        const int64_t s = (int64_t)(page0 + i) * 64 + lane;
        if (MODE == kModeSample || s < len) out[s] = res[i];
    }
}

}  // namespace

size_t index_fp8_workspace_bytes(int Tq) { return (size_t)Tq * 256 * sizeof(uint16_t); }

namespace {

hipError_t launch_qmix(const uint8_t* q_idx, const float* w, int Tq, int HI, void* ws,
                       hipStream_t stream)
{
    hipLaunchKernelGGL(qmix_kernel, dim3((Tq + 3) / 4), dim3(256), 0, stream, q_idx, w, Tq, HI,
                       static_cast<uint16_t*>(ws));
    return hipGetLastError();
}

// The resident kernel over n_keys logical keys in blocks of 1024; each workgroup takes a
// group of up to kg_max of them so the one-time q^I staging is amortised, while keeping
// >= 8 workgroups per CU in total.
template <int MODE>
hipError_t launch_resident(const uint8_t* q_idx, const float* q_scale, const float* w,
                           const uint8_t* k_idx, const float* k_scale, int Tq, int Tk, int HI,
                           int64_t q_pos0, const ResOut& o, int n_keys, int kg_max, void* ws,
                           hipStream_t stream)
{
    const int n_tt = (Tq + 15) / 16;
    const int n_kb1 = (n_keys + kResWaves * 16 * kResNK - 1) / (kResWaves * 16 * kResNK);
    if (n_tt == 0 || n_kb1 == 0) return hipSuccess;
    int kg = n_kb1 / 8;
    kg = kg < 1 ? 1 : (kg > kg_max ? kg_max : kg);
    const int n_kg = (n_kb1 + kg - 1) / kg;
    if ((int64_t)n_tt * n_kg > INT32_MAX) return hipErrorInvalidValue;
    // pairs (key group, token tile) with causal scores, and in kModeScores the -inf ones
    int n_work = 0, n_fill = 0;
    for (int g = 0; g < n_kg; ++g) {
        const int above = MODE == kModeSample
            ? 0 : tiles_above((int64_t)g * kg * kResWaves * 16 * kResNK, q_pos0, Tq, n_tt);
        n_work += n_tt - above;
        if (MODE == kModeScores) n_fill += above;
    }
    hipLaunchKernelGGL((index_fp8_resident_kernel<kResNK, MODE>), dim3((unsigned)(n_work + n_fill)),
                       dim3(kResWaves * 64), 0, stream, q_idx, q_scale, w, k_idx, k_scale,
                       static_cast<const uint16_t*>(ws), Tq, Tk, HI, q_pos0, o, n_kb1, n_kg, kg,
                       n_work);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_index_fp8(const uint8_t* q_idx, const float* q_scale, const float* w,
                            const uint8_t* k_idx, const float* k_scale, int Tq, int Tk, int HI,
                            int64_t q_pos0, float* scores, int64_t ld, void* ws, hipStream_t stream,
                            const int* run_if, bool qmix_ready)
{
    constexpr int NK = 8;
    const int n_tt = (Tq + 15) / 16;
    const int n_kb = (Tk + kIdxWaves * 16 * NK - 1) / (kIdxWaves * 16 * NK);
    const int64_t n = (int64_t)n_tt * n_kb;
    if (n == 0) return hipSuccess;
    if (n > INT32_MAX) return hipErrorInvalidValue;
    if (!qmix_ready) {
        const hipError_t e = launch_qmix(q_idx, w, Tq, HI, ws, stream);
        if (e != hipSuccess) return e;
    }
    if (HI <= kResHeads) {
        ResOut o = {};
        o.scores = scores; o.ld = ld; o.run_if = run_if;
        return launch_resident<kModeScores>(q_idx, q_scale, w, k_idx, k_scale, Tq, Tk, HI, q_pos0,
                                            o, Tk, 16, ws, stream);
    }
    if (run_if) return hipErrorInvalidValue;            // gating exists on the resident path only
    hipLaunchKernelGGL(index_fp8_kernel<NK>, dim3((unsigned)n), dim3(256), 0, stream, q_idx,
                       q_scale, w, k_idx, k_scale, static_cast<const uint16_t*>(ws), Tq, Tk, HI,
                       q_pos0, scores, ld, n_kb);
    return hipGetLastError();
}

hipError_t launch_index_fp8_sample(const uint8_t* q_idx, const float* q_scale, const float* w,
                                   const uint8_t* k_idx, const float* k_scale, int Tq, int Tk,
                                   int HI, int64_t q_pos0, float* samples, int S, void* ws,
                                   hipStream_t stream)
{
    if (HI > kResHeads || S < 0 || S % (kResWaves * 16 * kResNK) != 0) return hipErrorInvalidValue;
    const hipError_t e = launch_qmix(q_idx, w, Tq, HI, ws, stream);
    if (e != hipSuccess || S == 0) return e;            // S == 0: the pre-pass only
    ResOut o = {};
    o.samples = samples; o.S = S;
    return launch_resident<kModeSample>(q_idx, q_scale, w, k_idx, k_scale, Tq, Tk, HI, q_pos0, o,
                                        S, 2, ws, stream);
}

hipError_t launch_index_fp8_candidates(const uint8_t* q_idx, const float* q_scale,
                                       const float* w, const uint8_t* k_idx,
                                       const float* k_scale, int Tq, int Tk, int HI,
                                       int64_t q_pos0, const float* tau, int32_t* cnt,
                                       uint2* cand, int cap, void* ws, hipStream_t stream)
{
    if (HI > kResHeads) return hipErrorInvalidValue;
    ResOut o = {};
    o.tau = tau; o.cnt = cnt; o.cand = cand; o.cap = cap;
    return launch_resident<kModeCandidates>(q_idx, q_scale, w, k_idx, k_scale, Tq, Tk, HI, q_pos0,
                                            o, Tk, 16, ws, stream);
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

namespace {

// pages: pages per sequence the launch walks (max_blocks for keys, S / 64 for samples)
template <int MODE>
hipError_t launch_paged(const uint8_t* q_idx, const float* q_scale, const float* w,
                        const uint8_t* kidx_cache, const float* kidx_scale,
                        const int32_t* block_table, const int32_t* seq_lens, int B, int num_blocks,
                        int max_blocks, int block_size, int HI, const PagedOut& o, int pages,
                        hipStream_t stream)
{
    if (block_size != 64) return hipErrorInvalidValue;
    const int pages_per_wg = kIdxWaves * paged_ppw<MODE>();
    const int n_split = (pages + pages_per_wg - 1) / pages_per_wg;
    const int64_t n = (int64_t)B * n_split;
    if (n == 0) return hipSuccess;
    if (n > INT32_MAX) return hipErrorInvalidValue;
    if (HI <= 64)
        hipLaunchKernelGGL((index_fp8_paged_kernel<4, MODE>), dim3((unsigned)n), dim3(256), 0, stream,
                           q_idx, q_scale, w, kidx_cache, kidx_scale, block_table, seq_lens,
                           num_blocks, max_blocks, block_size, HI, o, n_split);
    else
        hipLaunchKernelGGL((index_fp8_paged_kernel<8, MODE>), dim3((unsigned)n), dim3(256), 0, stream,
                           q_idx, q_scale, w, kidx_cache, kidx_scale, block_table, seq_lens,
                           num_blocks, max_blocks, block_size, HI, o, n_split);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_index_fp8_paged(const uint8_t* q_idx, const float* q_scale, const float* w,
                                  const uint8_t* kidx_cache, const float* kidx_scale,
                                  const int32_t* block_table, const int32_t* seq_lens, int B,
                                  int num_blocks, int max_blocks, int block_size, int HI,
                                  float* scores, int64_t ld, hipStream_t stream, const int* run_if)
{
    PagedOut o = {};
    o.scores = scores; o.ld = ld; o.run_if = run_if;
    return launch_paged<kModeScores>(q_idx, q_scale, w, kidx_cache, kidx_scale, block_table,
                                     seq_lens, B, num_blocks, max_blocks, block_size, HI, o,
                                     max_blocks, stream);
}

hipError_t launch_index_fp8_paged_sample(const uint8_t* q_idx, const float* q_scale,
                                         const float* w, const uint8_t* kidx_cache,
                                         const float* kidx_scale, const int32_t* block_table,
                                         const int32_t* seq_lens, int B, int num_blocks,
                                         int max_blocks, int block_size, int HI, float* samples,
                                         int S, hipStream_t stream)
{
    if (S <= 0 || S % 64 != 0) return hipErrorInvalidValue;
    PagedOut o = {};
    o.samples = samples; o.S = S;
    return launch_paged<kModeSample>(q_idx, q_scale, w, kidx_cache, kidx_scale, block_table,
                                     seq_lens, B, num_blocks, max_blocks, block_size, HI, o,
                                     S / 64, stream);
}

hipError_t launch_index_fp8_paged_candidates(const uint8_t* q_idx, const float* q_scale,
                                             const float* w, const uint8_t* kidx_cache,
                                             const float* kidx_scale, const int32_t* block_table,
                                             const int32_t* seq_lens, int B, int num_blocks,
                                             int max_blocks, int block_size, int HI,
                                             const float* tau, int32_t* cnt, uint2* cand, int cap,
                                             hipStream_t stream)
{
    PagedOut o = {};
    o.tau = tau; o.cnt = cnt; o.cand = cand; o.cap = cap;
    return launch_paged<kModeCandidates>(q_idx, q_scale, w, kidx_cache, kidx_scale, block_table,
                                         seq_lens, B, num_blocks, max_blocks, block_size, HI, o,
                                         max_blocks, stream);
}

}  // namespace dsa
