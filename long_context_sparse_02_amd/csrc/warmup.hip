// warmup.hip -- the dense warm-up stage of the indexer's training, for gfx950.
//
// Section 2.3.3 of the Keye-VL-2.0 report trains the lightning indexer first
// against the dense attention (xllm-io review page, "核心公式", dense warm-up
// loss):  L = sum_t sum_g KL( p[t,:,g] || softmax(I[t,:]) ),  the sums over
// every key s <= t, with p[t,:,g] the attention of KV group g's query heads
// (their mean; the indexer's inputs are detached from the main model, so p is
// a constant).  This file holds
//  - warmup_kl_kernel: per query row the log-sum-exp of each head (unless the
//    caller passes it), then p, the row's KL and dL/dI[t,s] = G softmax(I)_s -
//    sum_g p[t,s,g], written over the scores in place.  Scores are bf16
//    matrix-core products with fp32 accumulation, softmax in fp32;
//  - the backward of the dense indexer scores, given dL/dI over the causal
//    prefix: dq^I and dw (one query row per wave, keys streamed through LDS) and
//    dk^I (keys owned by workgroups, query rows streamed, partial sums over row
//    ranges added in a fixed order), both on the FP8 and bf16 matrix cores:
//      x = q^I[t,j] . k^I[s] (FP8 codes, exact products), G = dI w [x > 0],
//      dq[t,j] = sum_s G k^I[s],  dk[s] = sum_{t,j} G q^I[t,j],
//      dw[t,j] = sum_s dI ReLU(x),
//    with G rounded to bf16 for the two products (2^-8 relative per term) and the
//    FP8 codes' values exact in bf16.  Nothing is added atomically, so every
//    output is bit-reproducible.
#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace dsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWuRows = 16;          // query rows per workgroup of the loss kernel
constexpr int kWuKeys = 16;          // keys per step of the loss kernel
constexpr int kWuChunk = 4;          // steps per barrier in the loss kernel's second pass

__device__ __forceinline__ v8bf load8bf(const uint16_t* p) {
    return __builtin_bit_cast(v8bf, *reinterpret_cast<const v4i*>(p));
}

// The hardware's exp2 and log2 (no rescaling around subnormal results: exp2 of an argument
// below -126 gives 0, which only drops probabilities under 2^-126).
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }

// Two floats rounded to bf16 (to nearest even, by the hardware's packed conversion).
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ int pack_bf16x2(float a, float b) {
    bf2v r;
    r.x = (__bf16)a;
    r.y = (__bf16)b;
    return __builtin_bit_cast(int, r);
}

// One step of an online log2-sum-exp2 with a single exp2: (mx, sm) describes
// sum 2^(y - mx) = sm over the values seen so far.
__device__ __forceinline__ void lse_step(float y, bool valid, float& mx, float& sm) {
    const float d = y - mx;                       // +inf while nothing was seen
    const float e = ex2(-fabsf(d));
    const float up = fmaf(sm, e, 1.f), keep = sm + e;
    sm = valid ? (d > 0.f ? up : keep) : sm;
    mx = valid ? fmaxf(mx, y) : mx;
}

// Merge of two (mx, sm) pairs.
__device__ __forceinline__ void lse_merge(float& mx, float& sm, float mo, float so) {
    const float mn = fmaxf(mx, mo);
    const float a = mx == mn ? 1.f : ex2(mx - mn);
    const float b = mo == mn ? 1.f : ex2(mo - mn);
    sm = sm * a + so * b;
    mx = mn;
}

__device__ __forceinline__ void lse_reduce16(float& mx, float& sm) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
        const float mo = __shfl_xor(mx, o, 64), so = __shfl_xor(sm, o, 64);
        lse_merge(mx, sm, mo, so);
    }
}

// Workgroup: G * WPG waves for 16 query rows t0 .. t0+15; wave w serves KV group
// g = w / WPG, query heads g HPG + (w % WPG) HPW + hh, hh < HPW (HPW = min(HPG, 8) heads per
// wave, WPG = HPG / HPW waves per group), so that every key a wave loads meets 16 x HPW query
// heads.  A wave keeps the A operands of its 16 rows x HPW heads in registers (M tiles of 16:
// for HPW <= 4, M row m of the wave is row m / HPW, head m % HPW; for HPW = 8 tile mt holds
// rows 4 (mt % 4) .. +3 with heads 4 (mt / 4) .. +3, so that the 8 heads of a row meet in one
// lane) and streams its group's keys 16 at a time as the B operand.  Keys are walked in chunks
// of 64; only the chunks that reach past some row's position (the last one or two) apply the
// causal mask.
// Both passes are software-pipelined: the work of one step (for HPW = 8: of half its tiles) is
// a slot, and each stage interleaves the matrix-core products of the next slot with the
// vector work on the current one; a key buffer is refilled as soon as its last slot's products
// are issued, two steps ahead of its next use.
// Pass 1 (without lse): per (row, head) the sum of 2^(S c2 - ref_row), c2 = sm_scale log2 e,
// ref_row = c2 max_h S(row, h, key 0) over the row's first heads (key 0 is causal for every
// row).  One exp2 per score and no rescaling; should a head's total leave [2^-80, FLT_MAX] (a
// score more than 2^7 above ref, or a head far below the row's others) the wave walks its keys
// again with a running maximum per (row, head).  Alongside, per row the log-sum-exp of I (rows
// wave + NW j, one key per lane).
// Pass 2, per chunk of 64 keys: each wave's share of p[t,s,g] = sum_h 2^(S c2 - lse2[t,h] -
// log2 HPG) into LDS (and, when the wave holds its whole group, sum_s p log2 p per row in
// registers); after the barrier the (row, key) pairs of the chunk, one per lane, combine the
// groups within the next chunk's first stage: dI = G softmax(I)_s - sum_g p and the KL's
// - sum_g p log2 softmax(I)_s.
template <int HPW, int WPG, int NJ>
__global__ __launch_bounds__(HPW == 8 ? 256 : NJ >= 16 ? 64 : NJ >= 8 ? 192 : NJ >= 4 ? 448 : 512)
void warmup_kl_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, int Tq, int Tk,
    int64_t q_pos0, int Hq, int G, int HPG, float sm_scale, const float* __restrict__ lse_in,
    float* __restrict__ scores, int64_t ld, float* __restrict__ kl)
{
    constexpr int MT = HPW;                              // M tiles per wave (16 rows x HPW)
    constexpr int H = MT == 8 ? 2 : 1;                   // pipeline slots per step
    constexpr int MP = MT / H;                           // tiles per slot
    constexpr int GMAX = (HPW == 8 ? 4 : 8) / WPG;       // most groups a workgroup can hold
    constexpr int KC = kWuChunk * kWuKeys;               // keys per chunk
    constexpr int PP = KC + 16;                          // LDS pitch: the stores hit 64 banks
    __shared__ float pbuf[2][8][kWuRows][PP];
    __shared__ float lse_i2[kWuRows];
    __shared__ float klp[8][kWuRows];                    // per wave and row: sum p log2 p
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int NW = G * WPG;                              // waves (blockDim.x / 64)

    const int g = wave / WPG;
    const int hbase = g * HPG + (wave % WPG) * HPW;     // first query head of this wave
    const int blk = gridDim.x - 1 - blockIdx.x;          // longest rows first
    const int t0 = blk * kWuRows;
    const int rows = min(kWuRows, Tq - t0);
    const int p0 = (int)(q_pos0 + t0);                  // positions fit in int (Tk is an int)
    const int nkeys = p0 + rows;                         // keys 0 .. p0 + rows - 1 (<= Tk)
    const float c2 = sm_scale * kLog2e;

    // (row, head) of M row mm of tile mt
    auto m_row = [](int mt, int mm) { return HPW == 8 ? 4 * (mt & 3) + mm / 4 : (16 * mt + mm) / HPW; };
    auto m_head = [](int mt, int mm) { return HPW == 8 ? 4 * (mt >> 2) + mm % 4 : (16 * mt + mm) % HPW; };
    v8bf qa[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int r = m_row(mt, col), hh = m_head(mt, col);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (r < rows)
                qa[mt][ks] = load8bf(q + ((int64_t)(t0 + r) * Hq + hbase + hh) * 128 + 32 * ks + 8 * grp);
            else
                qa[mt][ks] = __builtin_bit_cast(v8bf, v4i{0, 0, 0, 0});
            // with 8 heads the operands go to the accumulation registers, which the matrix core
            // reads directly, leaving the vector registers to the loop's other values
            if constexpr (HPW == 8) asm volatile("" : "+a"(qa[mt][ks]));
        }
    }
    // query row of this lane's accumulator element (mt, i); the lane's 4 rows are slots
    // q = 0..3 (slot_of), row_q(q) their rows
    auto row_of = [&](int mt, int i) { return m_row(mt, 4 * grp + i); };
    auto slot_of = [](int mt, int i) { return HPW == 8 ? (mt & 3) : HPW == 4 ? mt : HPW == 2 ? 2 * mt + (i >> 1) : i; };
    auto row_q = [&](int qs) {
        return HPW >= 4 ? 4 * qs + grp : HPW == 2 ? 8 * (qs >> 1) + 2 * grp + (qs & 1) : 4 * grp + qs;
    };

    // the wave's group's keys s0 .. s0+15 as B operands (key s0 + col, 8 bf16 per k step);
    // keys past the last are clamped (loaded, never used)
    auto load_keys = [&](int s0, v8bf* kb) {
        const uint16_t* kp = k + ((int64_t)min(s0 + col, nkeys - 1) * G + g) * 128 + 8 * grp;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kb[ks] = load8bf(kp + 32 * ks);
    };
    // scores of the tiles of slot part (part * MP .. +MP-1) against keys kb
    // (k steps outermost: consecutive products go to different tiles and never wait on each
    // other)
    auto qk_part = [&](const v8bf* kb, int part, v4f* acc) {
#pragma unroll
        for (int t = 0; t < MP; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int t = 0; t < MP; ++t) acc[t] = mfma_bf16_16x16x32(qa[part * MP + t][ks], kb[ks], acc[t]);
    };
    // instruction order within a stage: each matrix-core product of the next slot followed by
    // a few vector instructions of the current one, then the stage ends
    auto interleave = [&]() {
#pragma unroll
        for (int n = 0; n < MP * 4; ++n) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);      // three VALU
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // the I part: rows wave + NW j (j < NJ; rows past the block's are skipped), key c0 + lane.
    // Every load is issued, from a clamped address, and its value is used only a stage or more
    // later (a use next to the load would wait for every load in flight, the key prefetches
    // included); I_valid tells which values are inside the causal prefix.
    auto load_I = [&](int c0, float* y) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int r = wave + NW * j, rc = min(r, rows - 1), s = c0 + lane;
            y[j] = scores[(int64_t)(t0 + rc) * ld + min(s, p0 + rc)];
        }
    };
    auto I_valid = [&](int c0, int j) {
        const int r = wave + NW * j;
        return r < rows && c0 + lane <= p0 + r;
    };

    float lse2[MT][4];
    {
        float mxi[NJ], smi[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) { mxi[j] = -INFINITY; smi[j] = 0.f; }
        auto lse_I = [&](int c0, const float* y) {
#pragma unroll
            for (int j = 0; j < NJ; ++j) lse_step(y[j] * kLog2e, I_valid(c0, j), mxi[j], smi[j]);
        };
        if (lse_in) {
            // 4 chunks of loads in flight while the previous 4 are summed
            float ya[4][NJ], yb[4][NJ];
#pragma unroll
            for (int u = 0; u < 4; ++u) load_I(u * KC, ya[u]);
            for (int c0 = 0; c0 < nkeys; c0 += 8 * KC) {
#pragma unroll
                for (int u = 0; u < 4; ++u) load_I(c0 + (4 + u) * KC, yb[u]);
#pragma unroll
                for (int u = 0; u < 4; ++u) lse_I(c0 + u * KC, ya[u]);
                if (c0 + 4 * KC >= nkeys) break;
#pragma unroll
                for (int u = 0; u < 4; ++u) load_I(c0 + (8 + u) * KC, ya[u]);
#pragma unroll
                for (int u = 0; u < 4; ++u) lse_I(c0 + (4 + u) * KC, yb[u]);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = m_row(mt, 4 * grp + i), hh = m_head(mt, 4 * grp + i);
                    lse2[mt][i] = r < rows ? lse_in[(int64_t)(t0 + r) * Hq + hbase + hh] * kLog2e : 0.f;
                }
        } else {
            float ref[4], sm[MT][4];
            v8bf k0[4], k1[4], k2[4], k3[4];                // keys of the chunk's steps 0..3
            v4f a0[MP], a1[MP];
            load_keys(0, k0);
            load_keys(kWuKeys, k1);
            load_keys(2 * kWuKeys, k2);
            load_keys(3 * kWuKeys, k3);
            qk_part(k0, 0, a0);                              // slot 0: step 0, first tiles
            if constexpr (H == 1) load_keys(4 * kWuKeys, k0);
#pragma unroll
            for (int qs = 0; qs < 4; ++qs) ref[qs] = -INFINITY;
#pragma unroll
            for (int t = 0; t < MP; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) ref[slot_of(t, i)] = fmaxf(ref[slot_of(t, i)], a0[t][i] * c2);
#pragma unroll
            for (int qs = 0; qs < 4; ++qs) ref[qs] = __shfl(ref[qs], lane & 48, 64);   // key 0: column 0
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) sm[mt][i] = 0.f;
            // a stage: the sums of slot (s0, part) from cur while the matrix core forms slot
            // (nxt_part) of the keys in src into nxt; refill (if any) then receives the keys
            // at refill_s0
            auto stage1 = [&](int s0, int part, const v4f* cur, v4f* nxt, const v8bf* src, int nxt_part,
                              v8bf* refill, int refill_s0, bool edge, bool last, int c0, const float* y) {
                qk_part(src, nxt_part, nxt);
                if (refill) load_keys(refill_s0, refill);
                const int lim = edge ? s0 + col - p0 : -kWuRows;   // key valid for rows >= lim
#pragma unroll
                for (int t = 0; t < MP; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int mt = part * MP + t;
                        const float e = ex2(fmaf(cur[t][i], c2, -ref[slot_of(mt, i)]));
                        sm[mt][i] += row_of(mt, i) >= lim ? e : 0.f;
                    }
                if (last) lse_I(c0, y);
                interleave();
            };
            // the stages of one chunk (edge: only the steps below nkeys)
            auto chunk1 = [&](int c0, bool edge) {
                float y[NJ];
                load_I(c0, y);
                // step u's keys are in k<u>, refilled with step u + 4's once its last slot's
                // products are issued
                if constexpr (H == 1) {
                    stage1(c0, 0, a0, a1, k1, 0, k1, c0 + 5 * kWuKeys, edge, false, c0, y);
                    if (!edge || c0 + kWuKeys < nkeys)
                        stage1(c0 + kWuKeys, 0, a1, a0, k2, 0, k2, c0 + 6 * kWuKeys, edge, false, c0, y);
                    if (!edge || c0 + 2 * kWuKeys < nkeys)
                        stage1(c0 + 2 * kWuKeys, 0, a0, a1, k3, 0, k3, c0 + 7 * kWuKeys, edge, false, c0, y);
                    if (!edge || c0 + 3 * kWuKeys < nkeys)
                        stage1(c0 + 3 * kWuKeys, 0, a1, a0, k0, 0, k0, c0 + 8 * kWuKeys, edge, !edge, c0, y);
                } else {
                    v8bf* none = nullptr;
                    stage1(c0, 0, a0, a1, k0, 1, k0, c0 + 4 * kWuKeys, edge, false, c0, y);
                    stage1(c0, 1, a1, a0, k1, 0, none, 0, edge, false, c0, y);
                    if (!edge || c0 + kWuKeys < nkeys) {
                        stage1(c0 + kWuKeys, 0, a0, a1, k1, 1, k1, c0 + 5 * kWuKeys, edge, false, c0, y);
                        stage1(c0 + kWuKeys, 1, a1, a0, k2, 0, none, 0, edge, false, c0, y);
                    }
                    if (!edge || c0 + 2 * kWuKeys < nkeys) {
                        stage1(c0 + 2 * kWuKeys, 0, a0, a1, k2, 1, k2, c0 + 6 * kWuKeys, edge, false, c0, y);
                        stage1(c0 + 2 * kWuKeys, 1, a1, a0, k3, 0, none, 0, edge, false, c0, y);
                    }
                    if (!edge || c0 + 3 * kWuKeys < nkeys) {
                        stage1(c0 + 3 * kWuKeys, 0, a0, a1, k3, 1, k3, c0 + 7 * kWuKeys, edge, false, c0, y);
                        stage1(c0 + 3 * kWuKeys, 1, a1, a0, k0, 0, none, 0, edge, !edge, c0, y);
                    }
                }
                if (edge) lse_I(c0, y);                      // (inside the last stage otherwise)
            };
            int c0 = 0;
            for (; c0 + KC - 1 <= p0; c0 += KC) chunk1(c0, false);   // every key of the chunk is causal
            for (; c0 < nkeys; c0 += KC) chunk1(c0, true);           // the last chunks: masked, ragged
            // each head's total over the 16 key lanes
            bool bad = false;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float s = sm[mt][i];
#pragma unroll
                    for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o, 64);
                    sm[mt][i] = s;
                    bad |= !(s >= 0x1p-80f && s <= 3.4028235e38f);
                }
            if (__any(bad)) {
                // the same sums with a running maximum per (row, head) (two exp2 per score),
                // merged over the key lanes
                float mx[MT][4];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) { mx[mt][i] = -INFINITY; sm[mt][i] = 0.f; }
                for (int s0 = 0; s0 < nkeys; s0 += kWuKeys) {
                    load_keys(s0, k0);
                    const int lim = s0 + col - p0;
#pragma unroll
                    for (int part = 0; part < H; ++part) {
                        v4f acc[MP];
                        qk_part(k0, part, acc);
#pragma unroll
                        for (int t = 0; t < MP; ++t)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                // branch-free: a masked key enters as -inf and leaves
                                // (mx, sm) as they were (mu = 0 while nothing is in yet)
                                const int mt = part * MP + t;
                                const float y = row_of(mt, i) >= lim ? acc[t][i] * c2 : -INFINITY;
                                const float nm = fmaxf(mx[mt][i], y);
                                const float mu = nm == -INFINITY ? 0.f : nm;
                                sm[mt][i] = fmaf(sm[mt][i], ex2(mx[mt][i] - mu), ex2(y - mu));
                                mx[mt][i] = nm;
                            }
                    }
                }
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        lse_reduce16(mx[mt][i], sm[mt][i]);
                        lse2[mt][i] = mx[mt][i] + lg2(sm[mt][i]);
                    }
            } else {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) lse2[mt][i] = ref[slot_of(mt, i)] + lg2(sm[mt][i]);
            }
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const float mo = __shfl_xor(mxi[j], o, 64), so = __shfl_xor(smi[j], o, 64);
                lse_merge(mxi[j], smi[j], mo, so);
            }
            const int r = wave + NW * j;
            if (lane == 0 && r < rows) lse_i2[r] = mxi[j] + lg2(smi[j]);
        }
    }
    // 2^(S c2 - lse2h) is a head's probability divided by HPG (a power of two: exact)
    const float lg_hpg = (float)(31 - __builtin_clz(HPG));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) lse2[mt][i] += lg_hpg;
    __syncthreads();

    float kacc[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) kacc[j] = 0.f;
    // per row slot: sum_s p log2 p over the lane's keys (when the wave holds its whole group)
    float kplp[4] = {0.f, 0.f, 0.f, 0.f};
    float ep[4];                                         // HPW = 8: a row's first 4 heads
    auto put = [&](int qs, int b, int cc, float p) {
        pbuf[b][wave][row_q(qs)][cc] = p;
        if constexpr (WPG == 1) kplp[qs] = fmaf(p, lg2(fmaxf(p, 1.17549435e-38f)), kplp[qs]);  // p = 0 adds 0
    };
    // the pairs of a chunk whose p is complete (pend): row wave + NW j, key c0 + lane.  Every
    // pair is computed (reads stay inside the LDS arrays) and only the stores depend on validity.
    auto comb_math = [&](int b, int c0, const float* y, float* dI, bool pend) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int r = min(wave + NW * j, kWuRows - 1);
            float psum = 0.f, plp = 0.f;                         // plp in log2 units
            // the groups' parts, read from clamped slots without branches and dropped past G
#pragma unroll
            for (int gg = 0; gg < GMAX; ++gg) {
                float p = 0.f;
#pragma unroll
                for (int w2 = 0; w2 < WPG; ++w2) p += pbuf[b][min(gg * WPG + w2, NW - 1)][r][lane];
                p = gg < G ? p : 0.f;
                psum += p;
                if constexpr (WPG > 1) plp = fmaf(p, lg2(fmaxf(p, 1.17549435e-38f)), plp);
            }
            const float l2 = fmaf(y[j], kLog2e, -lse_i2[r]);             // log2 softmax(I)_s
            dI[j] = fmaf((float)G, ex2(l2), -psum);
            kacc[j] += pend && I_valid(c0, j) ? fmaf(-l2, psum, plp) : 0.f;
        }
    };
    auto comb_store = [&](int c0, const float* dI, bool pend) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            if (pend && I_valid(c0, j)) scores[(int64_t)(t0 + wave + NW * j) * ld + c0 + lane] = dI[j];
    };
    {
        v8bf k0[4], k1[4], k2[4], k3[4];
        v4f a0[MP], a1[MP];
        load_keys(0, k0);
        load_keys(kWuKeys, k1);
        load_keys(2 * kWuKeys, k2);
        load_keys(3 * kWuKeys, k3);
        qk_part(k0, 0, a0);
        if constexpr (H == 1) load_keys(4 * kWuKeys, k0);
        // y: the I values of the chunk whose pairs are pending; dI: their gradients
        float y[NJ], dI[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) y[j] = 0.f;
        // a stage of pass 2: p of slot (s0, part) from cur into column 16 u + col of buffer b,
        // with the next slot's products as in pass 1, and (comb) the pending chunk's pairs
        auto stage2 = [&](int s0, int part, int u, int b, const v4f* cur, v4f* nxt, const v8bf* src,
                          int nxt_part, v8bf* refill, int refill_s0, bool edge, bool comb, bool pend) {
            qk_part(src, nxt_part, nxt);
            if (refill) load_keys(refill_s0, refill);
            const int lim = edge ? s0 + col - p0 : -kWuRows;
            const int cc = u * kWuKeys + col;
#pragma unroll
            for (int t = 0; t < MP; ++t) {
                const int mt = part * MP + t;
                float e[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float v = ex2(fmaf(cur[t][i], c2, -lse2[mt][i]));
                    e[i] = row_of(mt, i) >= lim ? v : 0.f;
                }
                // this wave's heads of one row sum to its share of p
                if constexpr (HPW == 8) {
                    if (part == 0) ep[t] = (e[0] + e[1]) + (e[2] + e[3]);
                    else put(t, b, cc, ep[t] + ((e[0] + e[1]) + (e[2] + e[3])));
                } else if constexpr (HPW == 4) {
                    put(mt, b, cc, (e[0] + e[1]) + (e[2] + e[3]));
                } else if constexpr (HPW == 2) {
                    put(2 * mt, b, cc, e[0] + e[1]);
                    put(2 * mt + 1, b, cc, e[2] + e[3]);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) put(i, b, cc, e[i]);
                }
            }
            if (comb) comb_math(b ^ 1, s0 - KC, y, dI, pend);
            interleave();
        };
        // chunk c0 into buffer b; its first stage combines the previous chunk (buffer b ^ 1)
        // if pend, after which y receives this chunk's I values
        auto chunk2 = [&](int c0, int b, bool edge, bool pend) {
            v8bf* none = nullptr;
            if constexpr (H == 1) {
                stage2(c0, 0, 0, b, a0, a1, k1, 0, k1, c0 + 5 * kWuKeys, edge, true, pend);
                comb_store(c0 - KC, dI, pend);
                load_I(c0, y);
                if (!edge || c0 + kWuKeys < nkeys)
                    stage2(c0 + kWuKeys, 0, 1, b, a1, a0, k2, 0, k2, c0 + 6 * kWuKeys, edge, false, false);
                if (!edge || c0 + 2 * kWuKeys < nkeys)
                    stage2(c0 + 2 * kWuKeys, 0, 2, b, a0, a1, k3, 0, k3, c0 + 7 * kWuKeys, edge, false, false);
                if (!edge || c0 + 3 * kWuKeys < nkeys)
                    stage2(c0 + 3 * kWuKeys, 0, 3, b, a1, a0, k0, 0, k0, c0 + 8 * kWuKeys, edge, false, false);
            } else {
                stage2(c0, 0, 0, b, a0, a1, k0, 1, k0, c0 + 4 * kWuKeys, edge, true, pend);
                comb_store(c0 - KC, dI, pend);
                load_I(c0, y);
                stage2(c0, 1, 0, b, a1, a0, k1, 0, none, 0, edge, false, false);
                if (!edge || c0 + kWuKeys < nkeys) {
                    stage2(c0 + kWuKeys, 0, 1, b, a0, a1, k1, 1, k1, c0 + 5 * kWuKeys, edge, false, false);
                    stage2(c0 + kWuKeys, 1, 1, b, a1, a0, k2, 0, none, 0, edge, false, false);
                }
                if (!edge || c0 + 2 * kWuKeys < nkeys) {
                    stage2(c0 + 2 * kWuKeys, 0, 2, b, a0, a1, k2, 1, k2, c0 + 6 * kWuKeys, edge, false, false);
                    stage2(c0 + 2 * kWuKeys, 1, 2, b, a1, a0, k3, 0, none, 0, edge, false, false);
                }
                if (!edge || c0 + 3 * kWuKeys < nkeys) {
                    stage2(c0 + 3 * kWuKeys, 0, 3, b, a0, a1, k3, 1, k3, c0 + 7 * kWuKeys, edge, false, false);
                    stage2(c0 + 3 * kWuKeys, 1, 3, b, a1, a0, k0, 0, none, 0, edge, false, false);
                }
            }
            __syncthreads();
        };
        int c0 = 0, b = 0;
        bool pend = false;
        for (; c0 + KC - 1 <= p0; c0 += KC, b ^= 1) {        // every key of the chunk is causal
            chunk2(c0, b, false, pend);
            pend = true;
        }
        for (; c0 < nkeys; c0 += KC, b ^= 1) {               // the last chunks: masked, ragged
            chunk2(c0, b, true, pend);
            pend = true;
        }
        comb_math(b ^ 1, c0 - KC, y, dI, true);
        comb_store(c0 - KC, dI, true);
    }
    // the rows' sum_s p log2 p of each group (WPG = 1): over the 16 key lanes, then per wave
    if constexpr (WPG == 1) {
#pragma unroll
        for (int qs = 0; qs < 4; ++qs) {
            float v = kplp[qs];
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, 64);
            if (col == 0) klp[wave][row_q(qs)] = v;
        }
        __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        float v = wave_sum(kacc[j]);
        const int r = wave + NW * j;
        if constexpr (WPG == 1) {
            if (r < kWuRows) {
#pragma unroll
                for (int gg = 0; gg < GMAX; ++gg) v += gg < NW ? klp[min(gg, NW - 1)][r] : 0.f;  // group order
            }
        }
        if (lane == 0 && r < rows) kl[t0 + r] = v * kLn2;
    }
}

// OCP E4M3 code -> bf16 bits of its value (exact: at most 4 significant bits)
__device__ __forceinline__ uint16_t e4m3_to_bf16(uint32_t c) {
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
    return (uint16_t)((__float_as_uint(mag) >> 16) | ((c & 0x80u) << 8));
}

// dst[n][c][r] = bf16 value of the code src[n][r][c] for r < R (0 for R <= r < ldR),
// c < 128: 64 x 64 tiles through LDS.  Grid (N * ceil(ldR / 64), 2), 256 threads.
__global__ __launch_bounds__(256) void codes_to_bf16_t_kernel(
    const uint8_t* __restrict__ src, uint16_t* __restrict__ dst, int R, int ldR,
    int64_t src_n, int64_t dst_n)
{
    __shared__ __attribute__((aligned(16))) uint16_t tile[64][64 + 8];
    const int rtiles = (ldR + 63) / 64;
    const int64_t n = blockIdx.x / rtiles;
    const int r0 = (blockIdx.x % rtiles) * 64, c0 = blockIdx.y * 64;
    const int tid = threadIdx.x;
    {
        const int r = r0 + tid / 4, cc = 16 * (tid % 4);
        v4i x = {0, 0, 0, 0};
        if (r < R) x = *reinterpret_cast<const v4i*>(src + n * src_n + (int64_t)r * 128 + c0 + cc);
#pragma unroll
        for (int e = 0; e < 16; ++e)
            tile[cc + e][tid / 4] = e4m3_to_bf16(((uint32_t)x[e >> 2] >> ((e & 3) * 8)) & 255u);
    }
    __syncthreads();
    const int c = tid / 4, rr = 16 * (tid % 4);
    if (r0 + rr < ldR) {
        uint16_t* d = dst + n * dst_n + (int64_t)(c0 + c) * ldR + r0 + rr;
        const v4i* sp = reinterpret_cast<const v4i*>(&tile[c][rr]);
        reinterpret_cast<v4i*>(d)[0] = sp[0];
        reinterpret_cast<v4i*>(d)[1] = sp[1];
    }
}

constexpr int kQbWaves = 8;          // query rows (one per wave) per workgroup, dq kernel
constexpr int kQbKeys = 32;          // keys per step

// dq^I and dw: wave w of the workgroup owns query row t = t0 + w (all HI heads, all
// 128 columns: NHT x 8 accumulator tiles).  Per step of 32 keys the workgroup
// stages the key codes and their bf16 values (transposed, [column][key]) in LDS;
// each wave computes x^T (keys on A, its heads on B), G, dw, and then
// dq += G' K with A = G' = bf16(G k_scale) (its head rows, keys as K) and B = the
// keys' bf16 code values.  K slot j of lane group grp stands for key
// 16 (j / 4) + 4 grp + j % 4 on both operands.
template <int NHT>
__global__ __launch_bounds__(512) void warmup_ix_bwd_q_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ q_scale, const float* __restrict__ w,
    const uint8_t* __restrict__ k_idx, const float* __restrict__ k_scale,
    const uint16_t* __restrict__ kt_bf, int ldk, int Tq, int Tk, int64_t q_pos0,
    const float* __restrict__ gI, int64_t ld, float* __restrict__ dq, float* __restrict__ dw)
{
    constexpr int HI = 16 * NHT;
    __shared__ __attribute__((aligned(16))) uint8_t kc[2][kQbKeys][128 + 16];
    __shared__ __attribute__((aligned(16))) uint16_t kt[2][128][kQbKeys + 8];
    __shared__ __attribute__((aligned(16))) uint8_t qcs[kQbWaves][HI][128 + 16];
    __shared__ __attribute__((aligned(16))) float gks[2][kQbWaves][kQbKeys];   // g x k_scale
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int blk = gridDim.x - 1 - blockIdx.x;          // longest rows first
    const int t0 = blk * kQbWaves;
    const int t = t0 + wave;
    const bool row_ok = t < Tq;
    const int64_t pos = q_pos0 + t;
    const int tl = min(t0 + kQbWaves, Tq) - 1;
    const int nkeys = (int)min<int64_t>(q_pos0 + tl + 1, (int64_t)Tk);

    // the wave's query row codes (B operands of x^T), read from LDS at every step
    for (int e = lane; e < HI * 8; e += 64) {
        const v4i v = row_ok ? *reinterpret_cast<const v4i*>(q_idx + ((int64_t)t * HI + e / 8) * 128 + 16 * (e % 8))
                             : v4i{0, 0, 0, 0};
        *reinterpret_cast<v4i*>(&qcs[wave][e / 8][16 * (e % 8)]) = v;
    }
    float wv[NHT];
    const float qs = row_ok ? q_scale[t] : 0.f;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) wv[ht] = row_ok && qs > 0.f ? w[(int64_t)t * HI + 16 * ht + col] : 0.f;
    v4f acc[NHT][8];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) acc[ht][ct] = v4f{0.f, 0.f, 0.f, 0.f};
    float dwa[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) dwa[ht] = 0.f;

    // All global reads of a step are the next step's staging, issued at the top of the step
    // from clamped (valid) addresses and stored to LDS at its end: the key codes, their bf16
    // values [column][key], and g[t, s] k_scale[s] of the workgroup's 8 rows (0 where s is
    // past the row's position or Tk), one float per thread.
    auto fetch = [&](int s0, v4i& cbytes, v4i& bvals, float* gsv) {
        const int s0c = min(s0, ldk - kQbKeys);
        const int key = min(s0c + (tid & 255) / 8, Tk - 1);
        cbytes = *reinterpret_cast<const v4i*>(k_idx + (int64_t)key * 128 + 16 * (tid % 8));
        bvals = *reinterpret_cast<const v4i*>(kt_bf + (int64_t)(tid / 4) * ldk + s0c + 8 * (tid % 4));
        const int rr = min(t0 + (tid & 255) / kQbKeys, Tq - 1);
        const int64_t sg = s0 + (tid & 255) % kQbKeys, pr = q_pos0 + rr;
        gsv[0] = gI[(int64_t)rr * ld + min<int64_t>(sg, pr)];
        gsv[1] = k_scale[(int)min<int64_t>(sg, (int64_t)Tk - 1)];
    };
    // the product is formed when stored, so that the loads stay in flight during the step
    auto stash = [&](int s0, int buf, const v4i& cbytes, const v4i& bvals, const float* gsv) {
        if (tid < 256) {
            *reinterpret_cast<v4i*>(&kc[buf][tid / 8][16 * (tid % 8)]) = cbytes;
            const int64_t sg = s0 + tid % kQbKeys, pr = q_pos0 + t0 + tid / kQbKeys;
            gks[buf][tid / kQbKeys][tid % kQbKeys] = sg <= pr && sg < Tk ? gsv[0] * gsv[1] : 0.f;
        }
        *reinterpret_cast<v4i*>(&kt[buf][tid / 4][8 * (tid % 4)]) = bvals;
    };
    v4i cb = {0, 0, 0, 0}, bv = {0, 0, 0, 0};
    float gsv[2] = {0.f, 0.f};
    if (nkeys > 0) {
        fetch(0, cb, bv, gsv);
        stash(0, 0, cb, bv, gsv);
    }
    __syncthreads();
    int buf = 0;
    for (int s0 = 0; s0 < nkeys; s0 += kQbKeys, buf ^= 1) {
        const bool more = s0 + kQbKeys < nkeys;
        fetch(s0 + kQbKeys, cb, bv, gsv);                 // past the end: clamped, unused
        if (row_ok && s0 <= pos) {
            // with non-negative scales x q_scale k_scale > 0 exactly when x > 0 and both
            // scales are positive; a zero q_scale zeroes wv, a zero k_scale zeroes gk
            float gk[2][4];
#pragma unroll
            for (int kt2 = 0; kt2 < 2; ++kt2) {
                const float4 v = *reinterpret_cast<const float4*>(&gks[buf][wave][16 * kt2 + 4 * grp]);
                gk[kt2][0] = v.x; gk[kt2][1] = v.y; gk[kt2][2] = v.z; gk[kt2][3] = v.w;
            }
            v8bf ga[NHT];
#pragma unroll
            for (int ht = 0; ht < NHT; ++ht) {
                int pk[4];
                const v8i qb = *reinterpret_cast<const v8i*>(&qcs[wave][16 * ht + col][32 * grp]);
#pragma unroll
                for (int kt2 = 0; kt2 < 2; ++kt2) {
                    const v8i a = *reinterpret_cast<const v8i*>(&kc[buf][16 * kt2 + col][32 * grp]);
                    const v4f x = mfma_fp8_16x16x128(a, qb, v4f{0.f, 0.f, 0.f, 0.f});
                    float gv[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        dwa[ht] = fmaf(gk[kt2][i], fmaxf(x[i], 0.f), dwa[ht]);
                        gv[i] = x[i] > 0.f ? gk[kt2][i] * wv[ht] : 0.f;
                    }
                    pk[2 * kt2] = pack_bf16x2(gv[0], gv[1]);
                    pk[2 * kt2 + 1] = pack_bf16x2(gv[2], gv[3]);
                }
                ga[ht] = __builtin_bit_cast(v8bf, v4i{pk[0], pk[1], pk[2], pk[3]});
            }
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) {
                const uint2 lo = *reinterpret_cast<const uint2*>(&kt[buf][16 * ct + col][4 * grp]);
                const uint2 hi = *reinterpret_cast<const uint2*>(&kt[buf][16 * ct + col][16 + 4 * grp]);
                const v8bf kb = __builtin_bit_cast(v8bf, v4i{(int)lo.x, (int)lo.y, (int)hi.x, (int)hi.y});
#pragma unroll
                for (int ht = 0; ht < NHT; ++ht) acc[ht][ct] = mfma_bf16_16x16x32(ga[ht], kb, acc[ht][ct]);
            }
        }
        if (more) stash(s0 + kQbKeys, buf ^ 1, cb, bv, gsv);
        __syncthreads();
    }
    if (!row_ok) return;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dq[((int64_t)t * HI + 16 * ht + 4 * grp + i) * 128 + 16 * ct + col] = acc[ht][ct][i];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
        float v = dwa[ht];
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        if (grp == 0) dw[(int64_t)t * HI + 16 * ht + col] = v * qs;
    }
}

constexpr int kKbWaves = 8;          // waves per workgroup, dk kernel
constexpr int kKbKeysW = 48;         // keys per wave
constexpr int kKbKT = kKbKeysW / 16;  // 16-key tiles per wave
constexpr int kKbKeys = kKbWaves * kKbKeysW;

// Rows [r_begin, r_end) of row range sp that see key block kb: from the range's first row, or
// from the first row whose position reaches the block's first key, to the range's end.
__device__ __forceinline__ void split_rows(int kb, int sp, int rows_per_split, int Tq, int64_t q_pos0,
                                           int& r_begin, int& r_end) {
    const int64_t first = max<int64_t>((int64_t)sp * rows_per_split, (int64_t)kb * kKbKeys - q_pos0);
    r_begin = (int)min<int64_t>(max<int64_t>(first, 0), (int64_t)Tq);
    r_end = (int)min<int64_t>((int64_t)Tq, (int64_t)(sp + 1) * rows_per_split);
}

// dk^I partial sums: workgroup (key block kb, row range sp) owns 384 keys (48 per wave)
// and streams the query rows of its range that see them, one row per step (codes,
// w and the bf16 values [column][head] staged in LDS).  Per row a wave computes x
// (the row's heads on A, its keys on B), G' = bf16(G q_scale), and
// dk += G'^T Q with A = G'^T (its keys, heads as K) and B = the row's bf16 code values.
// K slot j of lane group grp stands for head 32 hc + 16 (j / 4) + 4 grp + j % 4.
// part[sp][s][c] receives the sum over the range's rows (zeros where none applies).
template <int NHT>
__global__ __launch_bounds__(512) void warmup_ix_bwd_k_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ q_scale, const float* __restrict__ w,
    const uint8_t* __restrict__ k_idx, const float* __restrict__ k_scale,
    const uint16_t* __restrict__ qt_bf, int Tq, int Tk, int64_t q_pos0, const float* __restrict__ gI,
    int64_t ld, int rows_per_split, int ldk, float* __restrict__ part)
{
    constexpr int HI = 16 * NHT;
    constexpr int NHC = (NHT + 1) / 2;
    __shared__ __attribute__((aligned(16))) uint8_t qc[2][HI][128 + 16];
    __shared__ __attribute__((aligned(16))) uint16_t qt[2][128][HI + 8];
    __shared__ __attribute__((aligned(16))) float wl[2][HI];
    __shared__ float gsl[2][kKbKeys];                    // g[t, s] q_scale[t], 0 where inapplicable
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int kb = blockIdx.x, sp = blockIdx.y;
    const int sw = kb * kKbKeys + wave * kKbKeysW;      // this wave's first key
    const int sb = kb * kKbKeys;                        // the workgroup's first key
    int r_begin, r_end;
    split_rows(kb, sp, rows_per_split, Tq, q_pos0, r_begin, r_end);
    if (r_begin >= r_end) return;                       // no row sees these keys: no partial

    v8i kbop[kKbKT];
    float ksc[kKbKT];
#pragma unroll
    for (int kt2 = 0; kt2 < kKbKT; ++kt2) {
        const int s = sw + 16 * kt2 + col;
        kbop[kt2] = s < Tk ? *reinterpret_cast<const v8i*>(k_idx + (int64_t)s * 128 + 32 * grp)
                           : v8i{0, 0, 0, 0, 0, 0, 0, 0};
        ksc[kt2] = s < Tk ? k_scale[s] : 0.f;
    }
    v4f acc[kKbKT][8];
#pragma unroll
    for (int kt2 = 0; kt2 < kKbKT; ++kt2)
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) acc[kt2][ct] = v4f{0.f, 0.f, 0.f, 0.f};

    // All global reads of a step are the next row's staging, issued at the top of the step
    // from clamped (valid) addresses and stored to LDS at its end: the row's codes, its bf16
    // values [column][head], w, and g[t, s] q_scale[t] for the workgroup's 384 keys (0 where
    // s is past the row's position or Tk, or a scale is zero).  Threads past a piece count
    // repeat pieces.
    constexpr int kCodeThreads = HI * 8;
    constexpr int NV = (HI * 16 + 511) / 512;
    auto fetch = [&](int t, v4i& cbytes, v4i* bvals, float& wvl, float* gsv) {
        const int tr = min(t, Tq - 1);
        const int ci = tid % kCodeThreads;
        cbytes = *reinterpret_cast<const v4i*>(q_idx + ((int64_t)tr * HI + ci / 8) * 128 + 16 * (ci % 8));
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int piece = (tid + 512 * u) % (HI * 16);
            bvals[u] = *reinterpret_cast<const v4i*>(qt_bf + (int64_t)tr * 128 * HI + (int64_t)piece * 8);
        }
        wvl = w[(int64_t)tr * HI + tid % HI];
        const int64_t sg = sb + tid % kKbKeys, pr = q_pos0 + tr;
        gsv[0] = gI[(int64_t)tr * ld + min<int64_t>(sg, pr)];
        gsv[1] = k_scale[(int)min<int64_t>(sg, (int64_t)Tk - 1)];
        gsv[2] = q_scale[tr];
    };
    // the product is formed when stored, so that the loads stay in flight during the step
    auto stash = [&](int t, int buf, const v4i& cbytes, const v4i* bvals, float wvl, const float* gsv) {
        if (tid < kCodeThreads) *reinterpret_cast<v4i*>(&qc[buf][tid / 8][16 * (tid % 8)]) = cbytes;
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int piece = tid + 512 * u;
            if (piece < HI * 16) {
                const int e = piece * 8;                     // element e of the [128][HI] row
                *reinterpret_cast<v4i*>(&qt[buf][e / HI][e % HI]) = bvals[u];
            }
        }
        if (tid < HI) wl[buf][tid] = wvl;
        if (tid < kKbKeys) {
            const int64_t sg = sb + tid, pr = q_pos0 + t;
            gsl[buf][tid] = sg <= pr && sg < Tk && gsv[1] > 0.f && gsv[2] > 0.f ? gsv[0] * gsv[2] : 0.f;
        }
    };
    v4i cb = {0, 0, 0, 0}, bv[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) bv[u] = v4i{0, 0, 0, 0};
    float wvl = 0.f, gsv[3] = {0.f, 0.f, 0.f};
    fetch(r_begin, cb, bv, wvl, gsv);
    stash(r_begin, 0, cb, bv, wvl, gsv);
    __syncthreads();
    int buf = 0;
    for (int t = r_begin; t < r_end; ++t, buf ^= 1) {
        const bool more = t + 1 < r_end;
        const int64_t pos = q_pos0 + t;
        fetch(t + 1, cb, bv, wvl, gsv);                     // past the end: clamped, unused
        if (sw <= pos) {
            // with non-negative scales x q_scale k_scale > 0 exactly when x > 0 and both
            // scales are positive (zero scales zeroed gsl)
            float gq[kKbKT];
#pragma unroll
            for (int kt2 = 0; kt2 < kKbKT; ++kt2) gq[kt2] = gsl[buf][wave * kKbKeysW + 16 * kt2 + col];
            v8bf ga[kKbKT][NHC];
#pragma unroll
            for (int kt2 = 0; kt2 < kKbKT; ++kt2) {
                int pk[NHC][4];
#pragma unroll
                for (int hc = 0; hc < NHC; ++hc) pk[hc][0] = pk[hc][1] = pk[hc][2] = pk[hc][3] = 0;
#pragma unroll
                for (int ht = 0; ht < NHT; ++ht) {
                    const v8i a = *reinterpret_cast<const v8i*>(&qc[buf][16 * ht + col][32 * grp]);
                    const v4f x = mfma_fp8_16x16x128(a, kbop[kt2], v4f{0.f, 0.f, 0.f, 0.f});
                    const float4 w4 = *reinterpret_cast<const float4*>(&wl[buf][16 * ht + 4 * grp]);
                    const float g0 = x[0] > 0.f ? gq[kt2] * w4.x : 0.f;
                    const float g1 = x[1] > 0.f ? gq[kt2] * w4.y : 0.f;
                    const float g2 = x[2] > 0.f ? gq[kt2] * w4.z : 0.f;
                    const float g3 = x[3] > 0.f ? gq[kt2] * w4.w : 0.f;
                    pk[ht / 2][2 * (ht % 2)] = pack_bf16x2(g0, g1);
                    pk[ht / 2][2 * (ht % 2) + 1] = pack_bf16x2(g2, g3);
                }
#pragma unroll
                for (int hc = 0; hc < NHC; ++hc)
                    ga[kt2][hc] = __builtin_bit_cast(v8bf, v4i{pk[hc][0], pk[hc][1], pk[hc][2], pk[hc][3]});
            }
#pragma unroll
            for (int ct = 0; ct < 8; ++ct)
#pragma unroll
                for (int hc = 0; hc < NHC; ++hc) {
                    const uint2 lo = *reinterpret_cast<const uint2*>(&qt[buf][16 * ct + col][32 * hc + 4 * grp]);
                    uint2 hi = {0u, 0u};
                    if (32 * hc + 16 < HI)
                        hi = *reinterpret_cast<const uint2*>(&qt[buf][16 * ct + col][32 * hc + 16 + 4 * grp]);
                    const v8bf qbv = __builtin_bit_cast(v8bf, v4i{(int)lo.x, (int)lo.y, (int)hi.x, (int)hi.y});
#pragma unroll
                    for (int kt2 = 0; kt2 < kKbKT; ++kt2) acc[kt2][ct] = mfma_bf16_16x16x32(ga[kt2][hc], qbv, acc[kt2][ct]);
                }
        }
        if (more) stash(t + 1, buf ^ 1, cb, bv, wvl, gsv);
        __syncthreads();
    }
    float* pp = part + (int64_t)sp * ldk * 128;
#pragma unroll
    for (int kt2 = 0; kt2 < kKbKT; ++kt2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int s = sw + 16 * kt2 + 4 * grp + i;
            if (s < ldk) {
#pragma unroll
                for (int ct = 0; ct < 8; ++ct) pp[(int64_t)s * 128 + 16 * ct + col] = acc[kt2][ct][i];
            }
        }
}

// dk[s][c] += sum of part[sp][s][c] over the row ranges sp = 0 .. nsplit-1 that hold a row
// seeing key s's block, in that order.
__global__ __launch_bounds__(256) void warmup_dk_sum_kernel(const float* __restrict__ part, int nsplit,
                                                            int64_t stride, int64_t n4, int rows_per_split,
                                                            int Tq, int64_t q_pos0,
                                                            float* __restrict__ dk)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n4) return;
    const int kb = (int)(i / (32 * kKbKeys));           // 32 float4 per key
    float4 a = reinterpret_cast<float4*>(dk)[i];
    for (int sp = 0; sp < nsplit; ++sp) {
        int r_begin, r_end;
        split_rows(kb, sp, rows_per_split, Tq, q_pos0, r_begin, r_end);
        if (r_begin >= r_end) continue;
        const float4 b = reinterpret_cast<const float4*>(part + sp * stride)[i];
        a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
    }
    reinterpret_cast<float4*>(dk)[i] = a;
}

}  // namespace

bool warmup_kl_supported(int Hq, int G)
{
    if (G < 1 || Hq % G) return false;
    const int hpg = Hq / G;
    if (hpg != 1 && hpg != 2 && hpg != 4 && hpg != 8 && hpg != 16) return false;
    // up to 8 waves of at most 4 heads, or up to 4 waves of 8 heads (their registers fill a SIMD)
    const int hpw = hpg < 8 ? hpg : 8, nw = G * (hpg / hpw);
    return hpw == 8 ? nw <= 4 : nw <= 8;
}

hipError_t launch_warmup_kl(const uint16_t* q, const uint16_t* k, int Tq, int Tk, int64_t q_pos0,
                            int Hq, int G, float sm_scale, const float* lse, float* scores,
                            int64_t ld, float* kl, hipStream_t stream)
{
    if (Tq == 0) return hipSuccess;
    if (!warmup_kl_supported(Hq, G)) return hipErrorInvalidValue;
    const int hpg = Hq / G, hpw = hpg < 8 ? hpg : 8, wpg = hpg / hpw, nw = G * wpg;
    // rows per wave in the I part and the combine: wave + nw j for j < nj covers the 16 rows
    int nj2 = 2;
    while (nj2 * nw < kWuRows) nj2 *= 2;
    const dim3 grid((Tq + kWuRows - 1) / kWuRows), block(64 * nw);
#define WU_KL(H, W, J) hipLaunchKernelGGL((warmup_kl_kernel<H, W, J>), grid, block, 0, stream, q, k, Tq, Tk, q_pos0, Hq, G, hpg, sm_scale, lse, scores, ld, kl)
    switch ((hpw * 8 + wpg) * 32 + nj2) {
    case (1 * 8 + 1) * 32 + 16: WU_KL(1, 1, 16); break;
    case (1 * 8 + 1) * 32 + 8: WU_KL(1, 1, 8); break;
    case (1 * 8 + 1) * 32 + 4: WU_KL(1, 1, 4); break;
    case (1 * 8 + 1) * 32 + 2: WU_KL(1, 1, 2); break;
    case (2 * 8 + 1) * 32 + 16: WU_KL(2, 1, 16); break;
    case (2 * 8 + 1) * 32 + 8: WU_KL(2, 1, 8); break;
    case (2 * 8 + 1) * 32 + 4: WU_KL(2, 1, 4); break;
    case (2 * 8 + 1) * 32 + 2: WU_KL(2, 1, 2); break;
    case (4 * 8 + 1) * 32 + 16: WU_KL(4, 1, 16); break;
    case (4 * 8 + 1) * 32 + 8: WU_KL(4, 1, 8); break;
    case (4 * 8 + 1) * 32 + 4: WU_KL(4, 1, 4); break;
    case (4 * 8 + 1) * 32 + 2: WU_KL(4, 1, 2); break;
    case (8 * 8 + 1) * 32 + 16: WU_KL(8, 1, 16); break;
    case (8 * 8 + 1) * 32 + 8: WU_KL(8, 1, 8); break;
    case (8 * 8 + 1) * 32 + 4: WU_KL(8, 1, 4); break;
    case (8 * 8 + 2) * 32 + 8: WU_KL(8, 2, 8); break;
    case (8 * 8 + 2) * 32 + 4: WU_KL(8, 2, 4); break;
    default: return hipErrorInvalidValue;
    }
#undef WU_KL
    return hipGetLastError();
}

WarmupBwdPlan plan_warmup_bwd(int Tq, int Tk, int HI)
{
    WarmupBwdPlan p;
    p.ldk = (Tk + 63) / 64 * 64;
    p.kblocks = (Tk + kKbKeys - 1) / kKbKeys;
    // split the query rows into ranges: about 4096 (key block, row range) pairs, of which
    // the half below the diagonal does work, so that the last workgroups to start (one per
    // CU at a time) leave little of the chip idle at the end
    const int want = 4096;
    p.nsplit = Tq > 0 ? std::max(1, std::min((want + p.kblocks - 1) / p.kblocks, (Tq + 63) / 64)) : 1;
    p.rows_per_split = Tq > 0 ? (Tq + p.nsplit - 1) / p.nsplit : 1;
    p.kt_bytes = (size_t)128 * p.ldk * 2;
    p.qt_bytes = (size_t)Tq * 128 * HI * 2;
    p.part_bytes = (size_t)p.nsplit * p.ldk * 128 * 4;
    auto up = [](size_t n) { return (n + 255) / 256 * 256; };
    p.total = up(p.kt_bytes) + up(p.qt_bytes) + up(p.part_bytes);
    return p;
}

hipError_t launch_warmup_ix_bwd(const uint8_t* q_idx, const float* q_scale, const float* w,
                                const uint8_t* k_idx, const float* k_scale, int Tq, int Tk, int HI,
                                int64_t q_pos0, const float* g, int64_t ld, float* dq, float* dw,
                                float* dk, void* ws, hipStream_t stream)
{
    if (Tq == 0 || Tk == 0) return hipSuccess;
    if (HI % 16 != 0 || HI > 64) return hipErrorInvalidValue;
    const WarmupBwdPlan p = plan_warmup_bwd(Tq, Tk, HI);
    auto up = [](size_t n) { return (n + 255) / 256 * 256; };
    char* wp = static_cast<char*>(ws);
    uint16_t* kt = reinterpret_cast<uint16_t*>(wp);   wp += up(p.kt_bytes);
    uint16_t* qt = reinterpret_cast<uint16_t*>(wp);   wp += up(p.qt_bytes);
    float* part = reinterpret_cast<float*>(wp);
    hipLaunchKernelGGL(codes_to_bf16_t_kernel, dim3(p.ldk / 64, 2), dim3(256), 0, stream, k_idx,
                       kt, Tk, p.ldk, (int64_t)0, (int64_t)0);
    hipLaunchKernelGGL(codes_to_bf16_t_kernel, dim3(Tq, 2), dim3(256), 0, stream, q_idx, qt, HI, HI,
                       (int64_t)HI * 128, (int64_t)HI * 128);
    const dim3 gq((Tq + kQbWaves - 1) / kQbWaves), gk(p.kblocks, p.nsplit), block(512);
    switch (HI / 16) {
    case 1:
        hipLaunchKernelGGL(warmup_ix_bwd_q_kernel<1>, gq, block, 0, stream, q_idx, q_scale, w, k_idx, k_scale, kt, p.ldk, Tq, Tk, q_pos0, g, ld, dq, dw);
        hipLaunchKernelGGL(warmup_ix_bwd_k_kernel<1>, gk, block, 0, stream, q_idx, q_scale, w, k_idx, k_scale, qt, Tq, Tk, q_pos0, g, ld, p.rows_per_split, p.ldk, part);
        break;
    case 2:
        hipLaunchKernelGGL(warmup_ix_bwd_q_kernel<2>, gq, block, 0, stream, q_idx, q_scale, w, k_idx, k_scale, kt, p.ldk, Tq, Tk, q_pos0, g, ld, dq, dw);
        hipLaunchKernelGGL(warmup_ix_bwd_k_kernel<2>, gk, block, 0, stream, q_idx, q_scale, w, k_idx, k_scale, qt, Tq, Tk, q_pos0, g, ld, p.rows_per_split, p.ldk, part);
        break;
    case 3:
        hipLaunchKernelGGL(warmup_ix_bwd_q_kernel<3>, gq, block, 0, stream, q_idx, q_scale, w, k_idx, k_scale, kt, p.ldk, Tq, Tk, q_pos0, g, ld, dq, dw);
        hipLaunchKernelGGL(warmup_ix_bwd_k_kernel<3>, gk, block, 0, stream, q_idx, q_scale, w, k_idx, k_scale, qt, Tq, Tk, q_pos0, g, ld, p.rows_per_split, p.ldk, part);
        break;
    case 4:
        hipLaunchKernelGGL(warmup_ix_bwd_q_kernel<4>, gq, block, 0, stream, q_idx, q_scale, w, k_idx, k_scale, kt, p.ldk, Tq, Tk, q_pos0, g, ld, dq, dw);
        hipLaunchKernelGGL(warmup_ix_bwd_k_kernel<4>, gk, block, 0, stream, q_idx, q_scale, w, k_idx, k_scale, qt, Tq, Tk, q_pos0, g, ld, p.rows_per_split, p.ldk, part);
        break;
    }
    const int64_t n4 = (int64_t)Tk * 128 / 4;
    hipLaunchKernelGGL(warmup_dk_sum_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream,
                       part, p.nsplit, (int64_t)p.ldk * 128, n4, p.rows_per_split, Tq, q_pos0, dk);
    return hipGetLastError();
}

}  // namespace dsa
