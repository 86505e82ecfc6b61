// train.hip -- the training side of the DSA layer for gfx950: the lightning
// indexer at the selected positions and its backward.
//
// The sparse adaptation stage of the Keye-VL-2.0 report (section 2.3.3; xllm-io
// review page, "核心公式", sparse adaptation loss) trains the indexer with
//   L = sum_t sum_g KL( p[t, S_t, g] || softmax(I[t, S_t]) ),  S_t = Omega_t,
// and the report's section 5.1.2 keeps only the post-top-k indexer scores
// I[t, Omega_t] in the forward.  These kernels compute those scores and, given
// dL/dI[t, Omega_t[i]], the gradients with respect to the dequantised indexer
// inputs q^I, w and k^I (FP8 rounding taken as the identity, ReLU'(0) = 0):
//   x[t,j,s] = q^I[t,j] . k^I[s],    I[t,s] = sum_j w[t,j] ReLU(x[t,j,s]),
//   G[t,j,s] = dI[t,s] w[t,j] [x > 0],
//   dw[t,j]  = sum_s dI[t,s] ReLU(x[t,j,s]),
//   dq[t,j]  = sum_s G[t,j,s] k^I[s],     dk[s] += sum_j G[t,j,s] q^I[t,j].
// FP8 inputs (OCP E4M3 codes, per-token fp32 scales), d_I = 128, one workgroup
// per query row.  For H^I a multiple of 16 the scores and the backward run on the
// matrix cores (x on the FP8 one, the products with G in bf16); other head counts
// run on the vector ALU in fp32 from the decoded codes (exact values), the
// backward then adding dk^I atomically.
#include "device_common.h"
#include "internal.h"

namespace dsa {
namespace {

constexpr int kIxThreads = 256;
constexpr int kIxBlock = 256;              // selected positions per block (one per thread)
constexpr int kIxHIMax = 64;               // indexer heads handled by the backward
constexpr int kIxGPitch = kIxHIMax + 4;    // LDS row pitch of the per-position head gradients

// OCP E4M3 code -> value (finite codes; the two NaN codes are not expected here)
__device__ __forceinline__ float e4m3_value(uint32_t c)
{
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
    return (c & 0x80u) ? -mag : mag;
}

__device__ __forceinline__ uint32_t code_at(const v4i* kc, int e)
{
    return ((uint32_t)kc[e >> 4][(e >> 2) & 3] >> ((e & 3) * 8)) & 255u;
}

// Raw dot products (code values, scales not applied) of the key codes kc (128 codes in
// registers) with heads j0 .. j0 + 15 of the row's decoded query qv [HI][128] in LDS.
__device__ __forceinline__ void head_dots16(const float* qv, int j0, int HI, const v4i* kc,
                                            float* acc)
{
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) acc[jj] = 0.f;
    for (int e4 = 0; e4 < 32; ++e4) {
        float kv[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) kv[b] = e4m3_value(code_at(kc, 4 * e4 + b));
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
            if (j0 + jj < HI) {
                const float4 q4 = *reinterpret_cast<const float4*>(qv + (j0 + jj) * 128 + 4 * e4);
                acc[jj] += q4.x * kv[0] + q4.y * kv[1] + q4.z * kv[2] + q4.w * kv[3];
            }
        }
    }
}

__device__ __forceinline__ void load_query(const uint8_t* __restrict__ q_idx, int64_t t, int HI,
                                           float* qv)
{
    const uint8_t* src = q_idx + t * HI * 128;
    for (int i = threadIdx.x; i < HI * 128; i += kIxThreads) qv[i] = e4m3_value(src[i]);
}

__device__ __forceinline__ void load_key(const uint8_t* __restrict__ k_idx, int s, v4i* kc)
{
    const v4i* src = reinterpret_cast<const v4i*>(k_idx + (int64_t)s * 128);
#pragma unroll
    for (int c = 0; c < 8; ++c) kc[c] = src[c];
}

// vals[t, i] = I[t, idx[t, i]]; -inf where the entry is padding or out of range.
__global__ __launch_bounds__(kIxThreads) void index_at_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ q_scale, const float* __restrict__ w,
    const uint8_t* __restrict__ k_idx, const float* __restrict__ k_scale, int Tk, int HI,
    const int32_t* __restrict__ idx, int topk, float* __restrict__ vals)
{
    __shared__ __attribute__((aligned(16))) float qv[128 * 128];
    __shared__ float wl[128];
    const int64_t t = blockIdx.x;
    load_query(q_idx, t, HI, qv);
    for (int j = threadIdx.x; j < HI; j += kIxThreads) wl[j] = w[t * HI + j];
    __syncthreads();
    const float qs = q_scale[t];
    for (int i = threadIdx.x; i < topk; i += kIxThreads) {
        const int s = idx[t * topk + i];
        float out = -INFINITY;
        if (s >= 0 && s < Tk) {
            v4i kc[8];
            load_key(k_idx, s, kc);
            const float sc = qs * k_scale[s];
            float I = 0.f;
            for (int j0 = 0; j0 < HI; j0 += 16) {
                float acc[16];
                head_dots16(qv, j0, HI, kc, acc);
#pragma unroll
                for (int jj = 0; jj < 16; ++jj)
                    if (j0 + jj < HI) I += wl[j0 + jj] * fmaxf(acc[jj] * sc, 0.f);
            }
            out = I;
        }
        vals[t * topk + i] = out;
    }
}

// The same on the FP8 matrix core when H^I is a multiple of 16: a 16-head tile of the row's
// query on A, 16 selected keys (gathered rows of codes) on B, so a lane's four results are
// four heads of one key and the ReLU-weighted head sum stays in the lane until a final
// exchange across the four lane groups.  Waves take key tiles in turn.
template <int NHT>
__global__ __launch_bounds__(kIxThreads) void index_at_mfma_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ q_scale, const float* __restrict__ w,
    const uint8_t* __restrict__ k_idx, const float* __restrict__ k_scale, int Tk,
    const int32_t* __restrict__ idx, int topk, float* __restrict__ vals)
{
    constexpr int HI = NHT * 16;
    const int64_t t = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    v8i qa[NHT];
    float wv[NHT][4];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
        qa[ht] = *reinterpret_cast<const v8i*>(q_idx + (t * HI + ht * 16 + col) * 128 + grp * 32);
#pragma unroll
        for (int i = 0; i < 4; ++i) wv[ht][i] = w[t * HI + ht * 16 + 4 * grp + i];
    }
    const float qs = q_scale[t];
    for (int tile = wave; tile * 16 < topk; tile += kIxThreads / 64) {
        const int i = tile * 16 + col;
        const int s = i < topk ? idx[t * topk + i] : -1;
        const bool ok = s >= 0 && s < Tk;
        const int sr = ok ? s : 0;                      // in-bounds row for padding entries
        const v8i kb = *reinterpret_cast<const v8i*>(k_idx + (int64_t)sr * 128 + grp * 32);
        const float sc = qs * k_scale[sr];
        float I = 0.f;
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
            const v4f x = mfma_fp8_16x16x128(qa[ht], kb, v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int r = 0; r < 4; ++r) I += wv[ht][r] * fmaxf(x[r] * sc, 0.f);
        }
        I += __shfl_xor(I, 16, 64);
        I += __shfl_xor(I, 32, 64);
        if (grp == 0 && i < topk) vals[t * topk + i] = ok ? I : -INFINITY;
    }
}

// Backward, one workgroup per query row, blocks of 256 selected positions:
//  A  thread = position p: the H^I dot products, stored as r[p, j] = dI_p ReLU(x[j, p])
//     in LDS (r != 0 exactly where x > 0, when dI_p != 0, so G[j, p] = dI_p w_j [r != 0]);
//  B  thread = (d_I column e, half of the block), for each position p of its half:
//     dk[s_p, e] += q_scale sum_j G[j,p] q[j,e]  (one coalesced atomic add per position
//     and wave), dq[j, e] += G[j,p] k_scale[p] k[p,e] in registers, and dw[e] += r[p, e]
//     for the threads whose column is a head index.
__global__ __launch_bounds__(kIxThreads) void index_at_bwd_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ q_scale, const float* __restrict__ w,
    const uint8_t* __restrict__ k_idx, const float* __restrict__ k_scale, int Tk, int HI,
    const int32_t* __restrict__ idx, int topk, const float* __restrict__ g,
    float* __restrict__ dq, float* __restrict__ dw, float* __restrict__ dk)
{
    __shared__ __attribute__((aligned(16))) float qv[kIxHIMax * 128];          // 32 KB
    __shared__ __attribute__((aligned(16))) float rl[kIxBlock * kIxGPitch];    // 68 KB
    __shared__ __attribute__((aligned(16))) uint8_t kcl[kIxBlock * 128];       // 32 KB
    __shared__ float ksl[kIxBlock];
    __shared__ float gl[kIxBlock];
    __shared__ int sl[kIxBlock];
    __shared__ __attribute__((aligned(16))) float wl[kIxHIMax];
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    load_query(q_idx, t, HI, qv);
    for (int j = tid; j < kIxHIMax; j += kIxThreads) wl[j] = j < HI ? w[t * HI + j] : 0.f;
    __syncthreads();
    const float qs = q_scale[t];
    const int e = tid & 127, half = tid >> 7;
    float qcol[kIxHIMax];                       // q[j, e] of this thread's column
#pragma unroll
    for (int j = 0; j < kIxHIMax; ++j) qcol[j] = j < HI ? qv[j * 128 + e] : 0.f;
    float dqa[kIxHIMax];                        // dq[j, e] over this thread's positions
#pragma unroll
    for (int j = 0; j < kIxHIMax; ++j) dqa[j] = 0.f;
    float dwa = 0.f;                            // dw[e] (e < HI) over this thread's positions
    // the walk stops after the row's last valid entry (its padding adds nothing)
    int k_end = 0;
    {
        __shared__ int ext;
        if (tid < 64) {
            const int x = row_extent(idx + t * topk, topk, tid);
            if (tid == 0) ext = x;
        }
        __syncthreads();
        k_end = ext;
    }

    for (int i0 = 0; i0 < k_end; i0 += kIxBlock) {
        {   // A: thread = position i0 + tid
            const int i = i0 + tid;
            const int s = i < topk ? idx[t * topk + i] : -1;
            const bool ok = s >= 0 && s < Tk;
            const float gi = ok ? g[t * topk + i] : 0.f;
            float* rrow = rl + tid * kIxGPitch;
            sl[tid] = ok ? s : -1;
            gl[tid] = gi;
            if (ok) {
                v4i kc[8];
                load_key(k_idx, s, kc);
#pragma unroll
                for (int c = 0; c < 8; ++c) reinterpret_cast<v4i*>(kcl + tid * 128)[c] = kc[c];
                const float ks = k_scale[s];
                ksl[tid] = ks;
                const float sc = qs * ks;
                for (int j0 = 0; j0 < HI; j0 += 16) {
                    float acc[16];
                    head_dots16(qv, j0, HI, kc, acc);
#pragma unroll
                    for (int jj = 0; jj < 16; ++jj)
                        if (j0 + jj < HI) rrow[j0 + jj] = gi * fmaxf(acc[jj] * sc, 0.f);
                }
                for (int j = HI; j < kIxHIMax; ++j) rrow[j] = 0.f;
            } else {
                ksl[tid] = 0.f;
                for (int j = 0; j < kIxHIMax; ++j) rrow[j] = 0.f;
            }
        }
        __syncthreads();
        // B: thread = column e, positions half*128 .. +128 of the block
        for (int pp = 0; pp < kIxBlock / 2; ++pp) {
            const int p = half * (kIxBlock / 2) + pp;
            const int s = sl[p];
            if (s < 0) continue;                          // uniform across the wave
            const float* rrow = rl + p * kIxGPitch;
            const float gi = gl[p];
            const float kv = e4m3_value(kcl[p * 128 + e]) * ksl[p];
            if (e < HI) dwa += rrow[e];
            float a = 0.f;
#pragma unroll
            for (int j = 0; j < kIxHIMax; j += 4) {
                const float4 r4 = *reinterpret_cast<const float4*>(rrow + j);
                const float4 w4 = *reinterpret_cast<const float4*>(wl + j);
                const float g0 = r4.x != 0.f ? gi * w4.x : 0.f, g1 = r4.y != 0.f ? gi * w4.y : 0.f;
                const float g2 = r4.z != 0.f ? gi * w4.z : 0.f, g3 = r4.w != 0.f ? gi * w4.w : 0.f;
                a += g0 * qcol[j] + g1 * qcol[j + 1] + g2 * qcol[j + 2] + g3 * qcol[j + 3];
                dqa[j] += g0 * kv;
                dqa[j + 1] += g1 * kv;
                dqa[j + 2] += g2 * kv;
                dqa[j + 3] += g3 * kv;
            }
            atomicAdd(dk + (int64_t)s * 128 + e, a * qs);
        }
        __syncthreads();
    }
    // the two halves of each column meet in LDS (reusing rl)
    float* red = rl;                                      // [2][64][128] floats fit in rl
#pragma unroll
    for (int j = 0; j < kIxHIMax; ++j) red[(half * kIxHIMax + j) * 128 + e] = dqa[j];
    if (e < kIxHIMax) red[2 * kIxHIMax * 128 + half * kIxHIMax + e] = dwa;
    __syncthreads();
    for (int i = tid; i < HI * 128; i += kIxThreads) {
        const int j = i >> 7, c = i & 127;
        dq[(t * HI + j) * 128 + c] = red[j * 128 + c] + red[(kIxHIMax + j) * 128 + c];
    }
    for (int j = tid; j < HI; j += kIxThreads)
        dw[t * HI + j] = red[2 * kIxHIMax * 128 + j] + red[2 * kIxHIMax * 128 + kIxHIMax + j];
}

// Backward on the matrix cores (H^I a multiple of 16, at most 64).  One workgroup (4 waves)
// per query row walks the row's selected positions, 32 per step:
//   - the workgroup stages the step's key codes, key scales and dI in LDS, loaded during the
//     step before;
//   - wave w (w < H^I / 16) computes X = q^I k^T for head tile w (heads on A, keys on B) on
//     the FP8 matrix core, forms G = dI w [x > 0], accumulates dw for its heads, and writes G
//     as bf16 twice into tiles shared by the workgroup: heads x keys with the key scales
//     folded in (A of dq = G K) and keys x heads (A of dk = G^T q);
//   - after a barrier every wave takes 32 of the 128 d_I columns of both products: dq [all
//     heads x its columns] accumulates in registers (bf16 products of G and the key codes,
//     which bf16 holds exactly); dk [32 keys x its columns] passes through LDS to the staging
//     buffer per (row, entry) in 16-byte stores (summed per position afterwards), or to
//     memory with atomic adds.
// G is rounded to bf16 for the two products (2^-8 relative per term, bf16's unit roundoff).
constexpr int kBwdKeys = 32;

__device__ __forceinline__ uint16_t e4m3_bf16_bits(uint32_t c)
{
    return (uint16_t)(__float_as_uint(e4m3_value(c)) >> 16);   // exact: 4 significant bits
}

// Two floats rounded to bf16 (to nearest even, by the hardware's packed conversion).
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    bf2v r;
    r.x = (__bf16)a;
    r.y = (__bf16)b;
    return __builtin_bit_cast(uint32_t, r);
}

template <int NHT>
__global__ __launch_bounds__(kIxThreads) void index_at_bwd_mfma_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ q_scale, const float* __restrict__ w,
    const uint8_t* __restrict__ k_idx, const float* __restrict__ k_scale, int Tk,
    const int32_t* __restrict__ idx, int topk, const float* __restrict__ g,
    float* __restrict__ dq, float* __restrict__ dw, float* __restrict__ dk, int r0,
    float* __restrict__ stg)
{
    constexpr int HI = NHT * 16;
    constexpr int NHC = (HI + 31) / 32;                  // 32-head chunks of the dk product
    __shared__ __attribute__((aligned(16))) uint16_t ga[2][64][kBwdKeys + 8];   // heads x keys
    __shared__ __attribute__((aligned(16))) uint16_t gb[2][kBwdKeys][64 + 8];   // keys x heads
    __shared__ __attribute__((aligned(16))) uint8_t kcs[2][kBwdKeys][128 + 16]; // key codes
    __shared__ __attribute__((aligned(16))) float st[4][kBwdKeys][32 + 4];      // dk staging
    __shared__ float gil[2][kBwdKeys], ksl[2][kBwdKeys];                        // dI, k scale
    __shared__ int posl[2][kBwdKeys];                                           // s, or -1
    const int64_t t = r0 + blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int c0 = 32 * wave;                            // this wave's d_I columns
    // heads beyond HI stay zero in the keys x heads tiles
    for (int i = tid; i < 2 * kBwdKeys * 72; i += kIxThreads) (&gb[0][0][0])[i] = 0;
    const bool xw = wave < NHT;                          // this wave owns head tile `wave`
    v8i qa = {0, 0, 0, 0, 0, 0, 0, 0};
    float wv[4] = {0.f, 0.f, 0.f, 0.f};
    if (xw) {
        qa = *reinterpret_cast<const v8i*>(q_idx + (t * HI + 16 * wave + col) * 128 + grp * 32);
#pragma unroll
        for (int r = 0; r < 4; ++r) wv[r] = w[t * HI + 16 * wave + 4 * grp + r];
    }
    // B operands of dk = G^T q: q codes (bf16, exact) for heads 32 hc + 8 grp + j, column d
    v8bf qb[NHC][2];
#pragma unroll
    for (int hc = 0; hc < NHC; ++hc)
#pragma unroll
        for (int dtl = 0; dtl < 2; ++dtl) {
            v8s x;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int h = 32 * hc + 8 * grp + j;
                x[j] = h < HI ? (short)e4m3_bf16_bits(q_idx[(t * HI + h) * 128 + c0 + 16 * dtl + col]) : (short)0;
            }
            qb[hc][dtl] = __builtin_bit_cast(v8bf, x);
        }
    const float qs = q_scale[t];
    v4f dqa[NHT][2];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) dqa[ht][0] = dqa[ht][1] = v4f{0.f, 0.f, 0.f, 0.f};
    float dwa[4] = {0.f, 0.f, 0.f, 0.f};

    // staging of a step: thread tid copies 16 code bytes of entry i0 + tid / 8 (from a valid
    // row: invalid entries read row 0 and are marked -1); every eighth thread also its dI
    // and key scale.  Positions are read two steps ahead, so the step's code loads do not
    // wait on them.
    const int kk = (tid & 255) / 8, part = tid % 8;
    auto pos_at = [&](int i0) -> int {
        const int i = i0 + kk;
        const int s = idx[t * topk + min(i, topk - 1)];
        return (i < topk && s >= 0 && s < Tk) ? s : -1;
    };
    auto fetch = [&](int i0, int sv, v4i& cb, float& gv, float& kv) {
        const int sc = sv >= 0 ? sv : 0;
        cb = *reinterpret_cast<const v4i*>(k_idx + (int64_t)sc * 128 + 16 * part);
        gv = g[t * topk + min(i0 + kk, topk - 1)];
        kv = k_scale[sc];
    };
    auto stash = [&](int buf, const v4i& cb, int sv, float gv, float kv) {
        if (tid < 256) {
            *reinterpret_cast<v4i*>(&kcs[buf][kk][16 * part]) = cb;
            if (part == 0) {
                posl[buf][kk] = sv;
                gil[buf][kk] = sv >= 0 ? gv : 0.f;
                ksl[buf][kk] = sv >= 0 ? kv : 0.f;
            }
        }
    };
    int s_next;                                          // positions of the next step
    {
        const int sv = pos_at(0);
        s_next = pos_at(kBwdKeys);
        v4i cb;
        float gv, kv;
        fetch(0, sv, cb, gv, kv);
        stash(0, cb, sv, gv, kv);
    }
    __syncthreads();
    // the walk stops after the row's last valid entry (its padding adds nothing; staged
    // entries past it are never read by the reduction, which skips padding)
    const int k_end = row_extent(idx + t * topk, topk, lane);
    int buf = 0;
    for (int i0 = 0; i0 < k_end; i0 += kBwdKeys, buf ^= 1) {
        const bool more = i0 + kBwdKeys < k_end;
        const int s_after = pos_at(i0 + 2 * kBwdKeys);   // past the end: clamped, unused
        v4i cb = {0, 0, 0, 0};
        float gv = 0.f, kv = 0.f;
        fetch(i0 + kBwdKeys, s_next, cb, gv, kv);        // past the end: clamped, unused
        // G for this wave's head tile
        if (xw) {
#pragma unroll
            for (int kt2 = 0; kt2 < 2; ++kt2) {
                const int key = 16 * kt2 + col;
                const v8i kb = *reinterpret_cast<const v8i*>(&kcs[buf][key][grp * 32]);
                const v4f x = mfma_fp8_16x16x128(qa, kb, v4f{0.f, 0.f, 0.f, 0.f});
                const float gi = gil[buf][key], ks = ksl[buf][key];
                const float sc = qs * ks;
                float gvv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float xv = x[r] * sc;
                    gvv[r] = xv > 0.f ? gi * wv[r] : 0.f;
                    dwa[r] = fmaf(gi, fmaxf(xv, 0.f), dwa[r]);
                    ga[buf][16 * wave + 4 * grp + r][key] = (uint16_t)(pack_bf16x2(gvv[r] * ks, 0.f) & 0xffffu);
                }
                *reinterpret_cast<uint2*>(&gb[buf][key][16 * wave + 4 * grp]) =
                    make_uint2(pack_bf16x2(gvv[0], gvv[1]), pack_bf16x2(gvv[2], gvv[3]));
            }
        }
        __syncthreads();
        // dq[heads, c0 .. c0 + 32) += G' K: A = G' (head row, keys 8 grp ..), B = key codes
        v8bf kbop[2];
#pragma unroll
        for (int dtl = 0; dtl < 2; ++dtl) {
            v8s x;
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] = (short)e4m3_bf16_bits(kcs[buf][8 * grp + j][c0 + 16 * dtl + col]);
            kbop[dtl] = __builtin_bit_cast(v8bf, x);
        }
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
            const v8bf a = *reinterpret_cast<const v8bf*>(&ga[buf][16 * ht + col][8 * grp]);
            dqa[ht][0] = mfma_bf16_16x16x32(a, kbop[0], dqa[ht][0]);
            dqa[ht][1] = mfma_bf16_16x16x32(a, kbop[1], dqa[ht][1]);
        }
        // dk[keys, c0 .. c0 + 32) = q_scale G^T q
#pragma unroll
        for (int kt2 = 0; kt2 < 2; ++kt2)
#pragma unroll
            for (int dtl = 0; dtl < 2; ++dtl) {
                v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int hc = 0; hc < NHC; ++hc) {
                    const v8bf a = *reinterpret_cast<const v8bf*>(&gb[buf][16 * kt2 + col][32 * hc + 8 * grp]);
                    acc = mfma_bf16_16x16x32(a, qb[hc][dtl], acc);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) st[wave][16 * kt2 + 4 * grp + r][16 * dtl + col] = acc[r] * qs;
            }
        __builtin_amdgcn_wave_barrier();
        if (stg) {
            // 32 keys x 32 columns in 16-byte pieces: a piece per lane and step, 8 keys per
            // instruction (streaming stores, reduced later); entries past topk are skipped
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int f = (j * 64 + lane) * 4, key = f / 32, cc = f % 32;
                const int i = i0 + key;
                if (i < topk) {
                    const float4 v = *reinterpret_cast<const float4*>(&st[wave][key][cc]);
                    float4* dst = reinterpret_cast<float4*>(stg + ((t - r0) * topk + i) * 128 + c0 + cc);
                    __builtin_nontemporal_store(v.x, &dst->x);
                    __builtin_nontemporal_store(v.y, &dst->y);
                    __builtin_nontemporal_store(v.z, &dst->z);
                    __builtin_nontemporal_store(v.w, &dst->w);
                }
            }
        } else {
            // two keys per instruction, 32 consecutive floats each
            for (int m = 0; m < kBwdKeys / 2; ++m) {
                const int key = 2 * m + (lane >> 5);
                const int s = posl[buf][key];
                if (s >= 0) atomicAdd(dk + (int64_t)s * 128 + c0 + (lane & 31), st[wave][key][lane & 31]);
            }
        }
        if (more) stash(buf ^ 1, cb, s_next, gv, kv);
        s_next = s_after;
        __syncthreads();
    }
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
        for (int dtl = 0; dtl < 2; ++dtl)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dq[(t * HI + 16 * ht + 4 * grp + r) * 128 + c0 + 16 * dtl + col] = dqa[ht][dtl][r];
    if (xw) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float v = dwa[r];
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, 64);
            if (col == 0) dw[t * HI + 16 * wave + 4 * grp + r] = v;
        }
    }
}

}  // namespace

hipError_t launch_index_at(const uint8_t* q_idx, const float* q_scale, const float* w,
                           const uint8_t* k_idx, const float* k_scale, int T, int Tk, int HI,
                           const int32_t* idx, int topk, float* vals, hipStream_t stream)
{
    if (T == 0) return hipSuccess;
    const dim3 grid(T), block(kIxThreads);
    switch (HI % 16 == 0 ? HI / 16 : 0) {
    case 1: hipLaunchKernelGGL(index_at_mfma_kernel<1>, grid, block, 0, stream, q_idx, q_scale, w, k_idx, k_scale, Tk, idx, topk, vals); break;
    case 2: hipLaunchKernelGGL(index_at_mfma_kernel<2>, grid, block, 0, stream, q_idx, q_scale, w, k_idx, k_scale, Tk, idx, topk, vals); break;
    case 4: hipLaunchKernelGGL(index_at_mfma_kernel<4>, grid, block, 0, stream, q_idx, q_scale, w, k_idx, k_scale, Tk, idx, topk, vals); break;
    case 8: hipLaunchKernelGGL(index_at_mfma_kernel<8>, grid, block, 0, stream, q_idx, q_scale, w, k_idx, k_scale, Tk, idx, topk, vals); break;
    default:
        hipLaunchKernelGGL(index_at_kernel, grid, block, 0, stream, q_idx, q_scale, w, k_idx,
                           k_scale, Tk, HI, idx, topk, vals);
    }
    return hipGetLastError();
}

bool index_at_bwd_stages(int HI) { return HI % 16 == 0 && HI <= kIxHIMax; }

hipError_t launch_index_at_bwd(const uint8_t* q_idx, const float* q_scale, const float* w,
                               const uint8_t* k_idx, const float* k_scale, int T, int Tk, int HI,
                               const int32_t* idx, int topk, const float* g, float* dq, float* dw,
                               float* dk, hipStream_t stream, int r0, float* stg)
{
    if (T == 0) return hipSuccess;
    if (HI > kIxHIMax) return hipErrorInvalidValue;
    const dim3 grid(T), block(kIxThreads);
    switch (HI % 16 == 0 ? HI / 16 : 0) {
    case 1: hipLaunchKernelGGL(index_at_bwd_mfma_kernel<1>, grid, block, 0, stream, q_idx, q_scale, w, k_idx, k_scale, Tk, idx, topk, g, dq, dw, dk, r0, stg); break;
    case 2: hipLaunchKernelGGL(index_at_bwd_mfma_kernel<2>, grid, block, 0, stream, q_idx, q_scale, w, k_idx, k_scale, Tk, idx, topk, g, dq, dw, dk, r0, stg); break;
    case 3: hipLaunchKernelGGL(index_at_bwd_mfma_kernel<3>, grid, block, 0, stream, q_idx, q_scale, w, k_idx, k_scale, Tk, idx, topk, g, dq, dw, dk, r0, stg); break;
    case 4: hipLaunchKernelGGL(index_at_bwd_mfma_kernel<4>, grid, block, 0, stream, q_idx, q_scale, w, k_idx, k_scale, Tk, idx, topk, g, dq, dw, dk, r0, stg); break;
    default:
        if (stg || r0) return hipErrorInvalidValue;    // the vector-ALU form adds atomically
        hipLaunchKernelGGL(index_at_bwd_kernel, grid, block, 0, stream, q_idx, q_scale, w, k_idx,
                           k_scale, Tk, HI, idx, topk, g, dq, dw, dk);
    }
    return hipGetLastError();
}

}  // namespace dsa
