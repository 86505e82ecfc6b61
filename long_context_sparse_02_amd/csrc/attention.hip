// attention.hip -- GQA sparse aggregation for gfx950.
//
// u[t,g] = Attn(h[t,g], {c[s,g] : s in Omega_t}) with the SAME Omega_t for
// every KV group g (Keye-VL-2.0 report section 2.3.2; xllm-io review page
// "核心公式", third formula): for each query head h of group g,
//   out[t,h,:] = softmax_s(sm_scale * q[t,h,:] . K[s,g,:]) V[s,g,:],  s in Omega_t.
//
// bf16 kernel: one workgroup (4 waves) per query row, wave w handles groups
// w, w+4, ...; all the row's heads share the one gathered index list.  Per
// step of 32 selected positions a wave
//   - gathers the 32 K rows and 32 V rows of its group with full-line requests
//     (16 lanes cover one 256-byte row, one instruction four rows) and stores
//     them into per-wave LDS tiles: the gather is bound by the number of
//     outstanding L1 misses per CU, so whole-line requests matter more than the
//     extra LDS round trip for K;
//   - computes S^T = K q^T on the bf16 16x16x32 matrix core (rows = positions,
//     columns = the group's heads, padded to 16);
//   - runs an online softmax in the exp2 domain; a lane's softmax values are
//     exactly the B operand of the next product, so no shuffle is needed;
//   - accumulates O^T = V^T P^T (rows = head dims, columns = heads), reading V^T
//     from the LDS tile.
// The next step's K/V loads are issued before the current step's math so the
// gather latency overlaps compute.  Long rows can be split across workgroups;
// partial (max, sum, unnormalised output) triples are merged by a combine
// kernel with the usual log-sum-exp rescaling.
#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace dsa {
namespace {

constexpr int kAttnWaves = 4;
constexpr int kStep = 32;                 // selected positions per step
constexpr int kVPitch = 136;              // LDS row pitch of the V tile (bf16 elements)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct KVStep {
    v4i kk[8];                            // K rows (lane >> 4) + 4 it, 16 bytes each
    v4i vv[8];                            // V rows (lane >> 4) + 4 it, 16 bytes each
    uint32_t valid;                       // bit r: entry r of the step is a usable position
};

// Row of the K/V arrays holding entry e of a query's index list, or -1 when the
// entry is padding, out of range, or maps to a block outside the cache.  Every
// load here is unconditional (clamped to valid memory) so that the compiler keeps
// the gather of the next step in flight instead of waiting at branch joins.
template <bool PAGED>
__device__ __forceinline__ int resolve_row(const AttnArgs& p, const int32_t* __restrict__ idx_row,
                                           int e, int k_end, int seq, int64_t len) {
    const int s = idx_row[min(e, k_end - 1)];
    bool ok = e < k_end && s >= 0 && s < len;
    if (!PAGED) return ok ? s : -1;
    const int sc = ok ? s : 0;
    const int blk = p.block_table[(int64_t)seq * p.max_blocks + sc / p.block_size];
    ok = ok && blk >= 0 && blk < p.n_kv;
    return ok ? blk * p.block_size + sc % p.block_size : -1;
}

template <bool PAGED>
__device__ __forceinline__ void load_step(const AttnArgs& p, const int32_t* __restrict__ idx_row,
                                          int kb0, int k_end, int seq, int64_t len, int g,
                                          int lane, KVStep& st) {
    const int col = lane & 15, grp = lane >> 4;
    const int prow = resolve_row<PAGED>(p, idx_row, kb0 + (lane & 31), k_end, seq, len);
    st.valid = (uint32_t)__ballot(prow >= 0);
    const int G = p.G;
    const uint16_t* __restrict__ K = static_cast<const uint16_t*>(p.k);
    const uint16_t* __restrict__ V = static_cast<const uint16_t*>(p.v);
    // Both K and V rows are gathered with full-line requests: lane l reads 16 bytes of row
    // (l >> 4) + 4 it, so one instruction covers four whole 256-byte rows.  Invalid entries
    // read row 0 (in bounds); their logits are masked to -inf and their V values zeroed, so
    // whatever row 0 holds cannot reach the result.
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int r = __shfl(prow, (lane >> 4) + 4 * it, 64);
        const int64_t off = ((int64_t)max(r, 0) * G + g) * 128 + (lane & 15) * 8;
        st.kk[it] = *reinterpret_cast<const v4i*>(K + off);
        const v4i x = *reinterpret_cast<const v4i*>(V + off);
        const int keep = r >= 0 ? -1 : 0;
        st.vv[it] = v4i{x.x & keep, x.y & keep, x.z & keep, x.w & keep};
    }
    (void)col; (void)grp;
}

template <bool PAGED>
__global__ __launch_bounds__(256, 2) void sparse_attn_bf16_kernel(AttnArgs p, int nsplit,
                                                                  int per_split,
                                                                  float* __restrict__ partials)
{
    __shared__ __attribute__((aligned(16))) uint16_t vt[kAttnWaves][kStep][kVPitch];
    __shared__ __attribute__((aligned(16))) uint16_t kt[kAttnWaves][kStep][kVPitch];
    // rows in groups of 16 dealt round-robin to the XCDs: adjacent rows share an L2, and rows
    // of uneven cost (short rows first) spread evenly (a contiguous share per XCD left the XCDs
    // holding short rows idle: 64 packed sequences of 1K..4K tokens 61.7 -> 31.9 ms)
    const int work = xcd_interleave16(blockIdx.x, gridDim.x);
    const int row = work / nsplit, split = work - row * nsplit;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int hpg = p.Hq / p.G;
    // rows the deduplicated attention computes: positions below prefix_skip (blocks of whole
    // prefixes), or blocks the union kernel marked (uniform over the workgroup)
    if (!PAGED && p.pos0 + row < p.prefix_skip) return;
    if (!PAGED && p.dedup_info && p.dedup_info[3 * ((p.pos0 % kDedupRows + row) / kDedupRows) + 2])
        return;

    int seq = 0;
    int64_t len = p.n_kv;
    if (PAGED) {
        seq = p.row_seq ? p.row_seq[row] : row;
        const int64_t cap = (int64_t)p.max_blocks * p.block_size;
        len = p.seq_lens ? (int64_t)p.seq_lens[seq] : cap;
        if (len > cap) len = 0;
    }
    if (p.n_kv <= 0) len = 0;                         // nothing can be gathered
    const int32_t* __restrict__ idx_row = p.idx + (int64_t)row * p.topk;
    const int k_begin = split * per_split;
    // the row's entries stop at its last valid one (short rows keep t + 1 of them)
    const int k_end = len > 0 ? min(row_extent(idx_row, p.topk, lane), k_begin + per_split) : k_begin;
    const float scale = p.sm_scale * kLog2e;
    const uint16_t* __restrict__ Q = static_cast<const uint16_t*>(p.q);
    uint16_t* vtile = &vt[wave][0][0];
    uint16_t* ktile = &kt[wave][0][0];

    for (int g = wave; g < p.G; g += kAttnWaves) {
        const int head = g * hpg + col;
        v8bf qb[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            v4i x = {0, 0, 0, 0};
            if (col < hpg) x = *reinterpret_cast<const v4i*>(Q + ((int64_t)row * p.Hq + head) * 128 + (4 * m + grp) * 8);
            qb[m] = __builtin_bit_cast(v8bf, x);
        }
        float m_run = -INFINITY, l_part = 0.f;
        v4f o[8];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[dt] = v4f{0.f, 0.f, 0.f, 0.f};

        KVStep cur, nxt;
        if (k_begin < k_end) load_step<PAGED>(p, idx_row, k_begin, k_end, seq, len, g, lane, cur);
        for (int kb0 = k_begin; kb0 < k_end; kb0 += kStep) {
            // K and V rows of this step into the wave's LDS tiles
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                const int off = ((lane >> 4) + 4 * it) * kVPitch + (lane & 15) * 8;
                *reinterpret_cast<v4i*>(ktile + off) = cur.kk[it];
                *reinterpret_cast<v4i*>(vtile + off) = cur.vv[it];
            }
            const uint32_t valid = cur.valid;
            if (kb0 + kStep < k_end)
                load_step<PAGED>(p, idx_row, kb0 + kStep, k_end, seq, len, g, lane, nxt);

            // S^T (positions x heads) for the two 16-position tiles; MFMA m takes head dims
            // 8 (4 m + grp) .. +8 from lane group grp, the same slots as the q operand
            v4f sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const v4i ka = *reinterpret_cast<const v4i*>(ktile + col * kVPitch + (4 * m + grp) * 8);
                const v4i kb = *reinterpret_cast<const v4i*>(ktile + (16 + col) * kVPitch + (4 * m + grp) * 8);
                sa = mfma_bf16_16x16x32(__builtin_bit_cast(v8bf, ka), qb[m], sa);
                sb = mfma_bf16_16x16x32(__builtin_bit_cast(v8bf, kb), qb[m], sb);
            }
            float sl[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * grp + i;
                sl[i] = ((valid >> r) & 1u) ? sa[i] * scale : -INFINITY;
                sl[4 + i] = ((valid >> (16 + r)) & 1u) ? sb[i] * scale : -INFINITY;
            }
            float mx = sl[0];
#pragma unroll
            for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sl[i]);
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float m_new = fmaxf(m_run, mx);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = exp2f(m_run - m_use);
            float pv[8], psum = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) { pv[i] = exp2f(sl[i] - m_use); psum += pv[i]; }
            l_part = l_part * alpha + psum;
            m_run = m_new;
            v8s pb;
#pragma unroll
            for (int i = 0; i < 8; ++i) pb[i] = (short)f32_to_bf16_bits(pv[i]);
            const v8bf pbf = __builtin_bit_cast(v8bf, pb);
            // O^T += V^T P^T over the 8 tiles of 16 head dims
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                v8s va;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    va[j] = (short)vtile[(4 * grp + j) * kVPitch + dt * 16 + col];
                    va[4 + j] = (short)vtile[(16 + 4 * grp + j) * kVPitch + dt * 16 + col];
                }
                o[dt] = o[dt] * alpha;
                o[dt] = mfma_bf16_16x16x32(__builtin_bit_cast(v8bf, va), pbf, o[dt]);
            }
            if (kb0 + kStep < k_end) cur = nxt;
        }
        float l = l_part;
        l += __shfl_xor(l, 16, 64);
        l += __shfl_xor(l, 32, 64);

        if (col < hpg) {
            if (nsplit == 1) {
                const float inv = l > 0.f ? 1.f / l : 0.f;
                uint16_t* outp = static_cast<uint16_t*>(p.out) + ((int64_t)row * p.Hq + head) * 128;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) {
                    const uint32_t lo = f32_to_bf16_bits(o[dt][0] * inv) | ((uint32_t)f32_to_bf16_bits(o[dt][1] * inv) << 16);
                    const uint32_t hi = f32_to_bf16_bits(o[dt][2] * inv) | ((uint32_t)f32_to_bf16_bits(o[dt][3] * inv) << 16);
                    *reinterpret_cast<uint2*>(outp + dt * 16 + 4 * grp) = make_uint2(lo, hi);
                }
                // natural-log log-sum-exp of the logits (m_run is in the scaled log2 domain)
                if (p.lse && grp == 0) p.lse[(int64_t)row * p.Hq + head] = (m_run + __log2f(l)) * kLn2;
            } else {
                float* part = partials + (((int64_t)row * nsplit + split) * p.Hq + head) * (128 + 2);
#pragma unroll
                for (int dt = 0; dt < 8; ++dt)
                    for (int i = 0; i < 4; ++i) part[dt * 16 + 4 * grp + i] = o[dt][i];
                if (grp == 0) { part[128] = m_run; part[129] = l; }
            }
        }
    }
}

// Backward of the bf16 attention (contiguous K/V), with the sparse indexer loss fused in
// (Keye-VL-2.0 report section 5.1.2: the sparse-attention backward already recomputes the
// softmax, so the indexer's KL target is reduced there instead of being stored).  One
// workgroup per query row, wave = KV group as in the forward.  Per step of 32 selected
// positions a wave gathers the K and V rows of its group into LDS and, from the forward's
// log-sum-exp,
//   S^T = K q^T, dP^T = V dO^T              (bf16 matrix core, rows = positions)
//   P = exp(S - lse), dS = P (dP - D),      D = dO . O per head
//   dq^T += K^T dS                          (kept in registers for the whole row)
//   dV^T = dO^T P^T, dK^T = q^T dS^T        (per 16 positions; P and dS pass through LDS
//                                            to become B operands, the results through LDS
//                                            into whole 512-byte rows: streamed to a staging
//                                            buffer per (row, entry, group) and summed per
//                                            position afterwards, or added atomically)
// and, when the indexer scores at Omega_t are given, the group-mean attention
// p[t,s,g] = mean_h P goes into a per-wave LDS row sum (summed in a fixed order, so the
// loss and its gradient are deterministic); at the end of the row the kernel writes
// dI = G softmax(I[t,Omega_t]) - sum_g p and the row's KL sum_g sum_s p ln(p / softmax(I)).
constexpr int kBwdMaxTopk = 2048;
constexpr int kStagePitch = 132;           // floats per staged position row

__global__ __launch_bounds__(256) void sparse_attn_bwd_kernel(AttnBwdArgs p)
{
    __shared__ __attribute__((aligned(16))) uint16_t vt[kAttnWaves][kStep][kVPitch];
    __shared__ __attribute__((aligned(16))) uint16_t kt[kAttnWaves][kStep][kVPitch];
    __shared__ __attribute__((aligned(16))) uint16_t pst[kAttnWaves][2][kStep][16];
    __shared__ float psum[kAttnWaves][kBwdMaxTopk];   // per wave: sum over its groups of p
    __shared__ float red[kAttnWaves];
    const int row = p.r0 + xcd_interleave16(blockIdx.x, gridDim.x);   // as the forward
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int hpg = p.Hq / p.G;
    const int topk = p.topk;
    const bool kl_on = p.vals != nullptr;
    const int32_t* __restrict__ idx_row = p.idx + (int64_t)row * topk;
    const float scale2 = p.sm_scale * kLog2e;
    const uint16_t* __restrict__ Q = static_cast<const uint16_t*>(p.q);
    const uint16_t* __restrict__ O = static_cast<const uint16_t*>(p.out);
    const uint16_t* __restrict__ dO = static_cast<const uint16_t*>(p.dout);
    AttnArgs a;
    a.q = p.q; a.k = p.k; a.v = p.v; a.out = nullptr; a.idx = p.idx; a.Tq = p.Tq; a.topk = topk;
    a.Hq = p.Hq; a.G = p.G; a.d = 128; a.sm_scale = p.sm_scale; a.n_kv = p.n_kv;
    a.block_table = nullptr; a.max_blocks = 0; a.block_size = 0; a.row_seq = nullptr;
    a.seq_lens = nullptr; a.bf16 = 1;
    const int64_t len = p.n_kv > 0 ? p.n_kv : 0;
    // entries after the row's last valid one are padding: they add nothing to any gradient,
    // so the walk stops there (their dI is written as 0 below all the same)
    const int k_end = len > 0 ? row_extent(idx_row, topk, lane) : 0;

    // the indexer's softmax over the row's valid entries: its max and log normaliser
    float mI = 0.f, lnZ = 0.f;
    if (kl_on) {
        float m = -INFINITY;
        for (int i = tid; i < topk; i += 256) {
#pragma unroll
            for (int w = 0; w < kAttnWaves; ++w) psum[w][i] = 0.f;
            const int s = idx_row[i];
            if (s >= 0 && s < len) m = fmaxf(m, p.vals[(int64_t)row * topk + i]);
        }
        m = wave_max(m);
        if (lane == 0) red[wave] = m;
        __syncthreads();
        m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        __syncthreads();
        float z = 0.f;
        for (int i = tid; i < topk; i += 256) {
            const int s = idx_row[i];
            if (s >= 0 && s < len) z += expf(p.vals[(int64_t)row * topk + i] - m);
        }
        z = wave_sum(z);
        if (lane == 0) red[wave] = z;
        __syncthreads();
        z = red[0] + red[1] + red[2] + red[3];
        __syncthreads();
        mI = m;
        lnZ = logf(z);
    }

    float plogp = 0.f;                                  // sum of p ln p over this wave's groups
    for (int g = wave; g < p.G; g += kAttnWaves) {
        const int head = g * hpg + col;
        const bool hv = col < hpg;
        v8bf qb[4], dob[4];
        float D = 0.f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            v4i x = {0, 0, 0, 0}, y = {0, 0, 0, 0}, o = {0, 0, 0, 0};
            if (hv) {
                const int64_t off = ((int64_t)row * p.Hq + head) * 128 + (4 * m + grp) * 8;
                x = *reinterpret_cast<const v4i*>(Q + off);
                y = *reinterpret_cast<const v4i*>(dO + off);
                o = *reinterpret_cast<const v4i*>(O + off);
            }
            qb[m] = __builtin_bit_cast(v8bf, x);
            dob[m] = __builtin_bit_cast(v8bf, y);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                D += bf16_bits_to_f32((uint16_t)y[j]) * bf16_bits_to_f32((uint16_t)o[j]) +
                     bf16_bits_to_f32((uint16_t)((uint32_t)y[j] >> 16)) *
                         bf16_bits_to_f32((uint16_t)((uint32_t)o[j] >> 16));
        }
        D += __shfl_xor(D, 16, 64);
        D += __shfl_xor(D, 32, 64);
        const float lse2 = hv ? p.lse[(int64_t)row * p.Hq + head] * kLog2e : 0.f;
        // A operands of dK^T = q^T dS^T and dV^T = dO^T P^T: row = head dim, k = head 8 grp + j
        v8bf qT[8], doT[8];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            v8s xq, xo;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int h = 8 * grp + j;
                const bool ok = grp < 2 && h < hpg;
                const int64_t off = ((int64_t)row * p.Hq + g * hpg + (ok ? h : 0)) * 128 + dt * 16 + col;
                xq[j] = ok ? (short)Q[off] : (short)0;
                xo[j] = ok ? (short)dO[off] : (short)0;
            }
            qT[dt] = __builtin_bit_cast(v8bf, xq);
            doT[dt] = __builtin_bit_cast(v8bf, xo);
        }
        v4f dqa[8];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) dqa[dt] = v4f{0.f, 0.f, 0.f, 0.f};
        uint16_t* ktile = &kt[wave][0][0];
        uint16_t* vtile = &vt[wave][0][0];
        float* stage = reinterpret_cast<float*>(ktile);  // 16 x kStagePitch floats fit the K tile

        KVStep cur;
        if (k_end > 0) load_step<false>(a, idx_row, 0, k_end, 0, len, g, lane, cur);
        for (int kb0 = 0; kb0 < k_end; kb0 += kStep) {
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                const int off = ((lane >> 4) + 4 * it) * kVPitch + (lane & 15) * 8;
                *reinterpret_cast<v4i*>(ktile + off) = cur.kk[it];
                *reinterpret_cast<v4i*>(vtile + off) = cur.vv[it];
            }
            const uint32_t valid = cur.valid;
            __builtin_amdgcn_wave_barrier();
            v4f sa = {0.f, 0.f, 0.f, 0.f}, sb = sa, pa = sa, pb = sa;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int c = (4 * m + grp) * 8;
                const v4i ka = *reinterpret_cast<const v4i*>(ktile + col * kVPitch + c);
                const v4i kb = *reinterpret_cast<const v4i*>(ktile + (16 + col) * kVPitch + c);
                const v4i va = *reinterpret_cast<const v4i*>(vtile + col * kVPitch + c);
                const v4i vb = *reinterpret_cast<const v4i*>(vtile + (16 + col) * kVPitch + c);
                sa = mfma_bf16_16x16x32(__builtin_bit_cast(v8bf, ka), qb[m], sa);
                sb = mfma_bf16_16x16x32(__builtin_bit_cast(v8bf, kb), qb[m], sb);
                pa = mfma_bf16_16x16x32(__builtin_bit_cast(v8bf, va), dob[m], pa);
                pb = mfma_bf16_16x16x32(__builtin_bit_cast(v8bf, vb), dob[m], pb);
            }
            float P[8], dS[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * grp + i;
                const bool va_ = hv && ((valid >> r) & 1u), vb_ = hv && ((valid >> (16 + r)) & 1u);
                P[i] = va_ ? exp2f(sa[i] * scale2 - lse2) : 0.f;
                P[4 + i] = vb_ ? exp2f(sb[i] * scale2 - lse2) : 0.f;
                dS[i] = P[i] * (pa[i] - D);
                dS[4 + i] = P[4 + i] * (pb[i] - D);
            }
            if (kl_on) {
                float ps[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) ps[i] = P[i];
#pragma unroll
                for (int o = 1; o < 16; o <<= 1)
#pragma unroll
                    for (int i = 0; i < 8; ++i) ps[i] += __shfl_xor(ps[i], o, 64);
                if (col == 0) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int r = i < 4 ? 4 * grp + i : 16 + 4 * grp + (i - 4);
                        if ((valid >> r) & 1u) {
                            const float pg = ps[i] / (float)hpg;
                            psum[wave][kb0 + r] += pg;      // one lane per position
                            if (pg > 0.f) plogp += pg * logf(pg);
                        }
                    }
                }
            }
            // dq^T += K^T dS
            v8s dsb;
#pragma unroll
            for (int i = 0; i < 8; ++i) dsb[i] = (short)f32_to_bf16_bits(dS[i]);
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                v8s kta;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    kta[j] = (short)ktile[(4 * grp + j) * kVPitch + dt * 16 + col];
                    kta[4 + j] = (short)ktile[(16 + 4 * grp + j) * kVPitch + dt * 16 + col];
                }
                dqa[dt] = mfma_bf16_16x16x32(__builtin_bit_cast(v8bf, kta),
                                             __builtin_bit_cast(v8bf, dsb), dqa[dt]);
            }
            // the next step's gather goes out before this step's atomic adds, so that its
            // wait does not queue behind them
            if (kb0 + kStep < k_end) load_step<false>(a, idx_row, kb0 + kStep, k_end, 0, len, g, lane, cur);
            asm volatile("" ::: "memory");
            // P and dS as [position][head] tiles
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pst[wave][0][4 * grp + i][col] = f32_to_bf16_bits(P[i]);
                pst[wave][0][16 + 4 * grp + i][col] = f32_to_bf16_bits(P[4 + i]);
                pst[wave][1][4 * grp + i][col] = (uint16_t)dsb[i];
                pst[wave][1][16 + 4 * grp + i][col] = (uint16_t)dsb[4 + i];
            }
            __builtin_amdgcn_wave_barrier();
            // dV (mat 0) and dK (mat 1), 16 positions at a time
#pragma unroll
            for (int mat = 0; mat < 2; ++mat) {
                float* __restrict__ dst_base = mat ? p.dk : p.dv;
                const float mul = mat ? p.sm_scale : 1.f;
#pragma unroll
                for (int pt = 0; pt < 2; ++pt) {
                    v4i bx = {0, 0, 0, 0};
                    if (grp < 2) bx = *reinterpret_cast<const v4i*>(&pst[wave][mat][pt * 16 + col][8 * grp]);
                    const v8bf bop = __builtin_bit_cast(v8bf, bx);
                    __builtin_amdgcn_wave_barrier();
#pragma unroll
                    for (int dt = 0; dt < 8; ++dt) {
                        const v4f acc = mfma_bf16_16x16x32(mat ? qT[dt] : doT[dt], bop,
                                                           v4f{0.f, 0.f, 0.f, 0.f});
                        *reinterpret_cast<v4f*>(stage + col * kStagePitch + dt * 16 + 4 * grp) = acc * mul;
                    }
                    __builtin_amdgcn_wave_barrier();
                    if (p.stg) {
                        // streaming stores, reduced later: 16 bytes per lane, two positions
                        // (512 bytes each) per instruction
#pragma unroll
                        for (int m = 0; m < 8; ++m) {
                            const int r = 2 * m + (lane >> 5), c4 = 4 * (lane & 31);
                            const int pos = pt * 16 + r;
                            if ((valid >> pos) & 1u) {
                                const float4 a = *reinterpret_cast<const float4*>(stage + r * kStagePitch + c4);
                                const int64_t e = (int64_t)(row - p.r0) * topk + kb0 + pos;
                                float4* dst = reinterpret_cast<float4*>(p.stg + (e * p.G + g) * 256 + mat * 128 + c4);
                                __builtin_nontemporal_store(a.x, &dst->x);
                                __builtin_nontemporal_store(a.y, &dst->y);
                                __builtin_nontemporal_store(a.z, &dst->z);
                                __builtin_nontemporal_store(a.w, &dst->w);
                            }
                        }
                    } else {
                        for (int r = 0; r < 16; ++r) {
                            const int pos = pt * 16 + r;
                            if (!((valid >> pos) & 1u)) continue;       // uniform
                            const float a0 = stage[r * kStagePitch + lane];
                            const float a1 = stage[r * kStagePitch + 64 + lane];
                            const int s = idx_row[kb0 + pos];
                            float* dst = dst_base + ((int64_t)s * p.G + g) * 128;
                            atomicAdd(dst + lane, a0);
                            atomicAdd(dst + 64 + lane, a1);
                        }
                    }
                    __builtin_amdgcn_wave_barrier();
                }
            }
        }
        if (hv) {
            uint16_t* dqp = static_cast<uint16_t*>(p.dq) + ((int64_t)row * p.Hq + head) * 128;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const v4f r = dqa[dt] * p.sm_scale;
                const uint32_t lo = f32_to_bf16_bits(r[0]) | ((uint32_t)f32_to_bf16_bits(r[1]) << 16);
                const uint32_t hi = f32_to_bf16_bits(r[2]) | ((uint32_t)f32_to_bf16_bits(r[3]) << 16);
                *reinterpret_cast<uint2*>(dqp + dt * 16 + 4 * grp) = make_uint2(lo, hi);
            }
        }
    }
    if (!kl_on) return;
    plogp = wave_sum(plogp);
    __syncthreads();                                    // psum complete
    if (lane == 0) red[wave] = plogp;
    float cross = 0.f;
    for (int i = tid; i < topk; i += 256) {
        const int s = idx_row[i];
        const bool ok = s >= 0 && s < len;
        const float lq = ok ? p.vals[(int64_t)row * topk + i] - mI - lnZ : 0.f;   // ln softmax(I)
        const float ps = (psum[0][i] + psum[1][i]) + (psum[2][i] + psum[3][i]);    // fixed order
        if (ok) cross += ps * lq;
        p.dI[(int64_t)row * topk + i] = ok ? (float)p.G * expf(lq) - ps : 0.f;
    }
    cross = wave_sum(cross);
    __syncthreads();
    const float total_plogp = red[0] + red[1] + red[2] + red[3];
    __syncthreads();
    if (lane == 0) red[wave] = cross;
    __syncthreads();
    if (tid == 0) p.kl[row] = total_plogp - (red[0] + red[1] + red[2] + red[3]);
}

// ---- deterministic reduction of the staged dK / dV contributions of a chunk of rows ----
// Each row holds a key at most once (its index list has distinct positions), so a key's
// entries are identified by the rows that select it: a bitmask per key over the chunk's rows
// gives each entry its rank among the key's entries without any sort, and the per-key sums
// run in row order, independent of scheduling.

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* __restrict__ p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        p[i] = 0u;
}

__global__ __launch_bounds__(256) void stage_mark_kernel(const int32_t* __restrict__ idx, int r0,
                                                         int C, int topk, int n_kv, int W,
                                                         uint32_t* __restrict__ mask,
                                                         uint8_t* __restrict__ dup)
{
    const int64_t n = (int64_t)C * topk;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
        const int t = (int)(e / topk);
        const int s = idx[(int64_t)r0 * topk + e];
        uint8_t repeat = 0;
        if (s >= 0 && s < n_kv) {
            const uint32_t bit = 1u << (t & 31);
            repeat = (atomicOr(&mask[(int64_t)s * W + (t >> 5)], bit) & bit) ? 1 : 0;
        }
        dup[e] = repeat;                   // every entry written: no clearing needed
    }
}

// The contributions of repeated keys (entries marked in dup), added atomically after the
// ordered per-key sums.  Lists of distinct keys mark nothing and this kernel only reads dup.
__global__ __launch_bounds__(256) void stage_dup_add_kernel(const int32_t* __restrict__ idx, int r0,
                                                            int C, int topk, int G, int width,
                                                            const uint8_t* __restrict__ dup,
                                                            const float* __restrict__ stg,
                                                            float* __restrict__ dk,
                                                            float* __restrict__ dv)
{
    const int64_t n = (int64_t)C * topk;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
        if (!dup[e]) continue;
        const int s = idx[(int64_t)r0 * topk + e];
        if (width == 128) {
            for (int c = 0; c < 128; ++c) atomicAdd(dk + (int64_t)s * 128 + c, stg[e * 128 + c]);
            continue;
        }
        for (int g = 0; g < G; ++g) {
            const float* src = stg + (e * G + g) * 256;
            for (int c = 0; c < 128; ++c) {
                atomicAdd(dv + ((int64_t)s * G + g) * 128 + c, src[c]);
                atomicAdd(dk + ((int64_t)s * G + g) * 128 + c, src[128 + c]);
            }
        }
    }
}

// Exclusive prefix of the per-key entry counts in three passes: each block of 256 keys scans
// its own counts and leaves its total in bsum; one workgroup scans the block totals; each key
// then adds its block's offset.  offs[n_kv] gets the total.
__global__ __launch_bounds__(256) void stage_count_kernel(const uint32_t* __restrict__ mask,
                                                          int n_kv, int W, int32_t* __restrict__ offs,
                                                          int32_t* __restrict__ bsum)
{
    __shared__ int red[4];
    const int s = blockIdx.x * 256 + threadIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int c = 0;
    if (s < n_kv)
        for (int w = 0; w < W; ++w) c += __popc(mask[(int64_t)s * W + w]);
    int x = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) { const int y = __shfl_up(x, o, 64); if (lane >= o) x += y; }
    if (lane == 63) red[wave] = x;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += red[w];
    if (s < n_kv) offs[s] = base + x - c;
    if (threadIdx.x == 255) bsum[blockIdx.x] = base + x;
}

__global__ __launch_bounds__(1024) void stage_scan_kernel(int32_t* __restrict__ bsum, int nb,
                                                          int32_t* __restrict__ total)
{
    __shared__ int red[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int per = (nb + 1023) / 1024;
    const int b = min(nb, tid * per), e = min(nb, b + per);
    int local = 0;
    for (int i = b; i < e; ++i) local += bsum[i];
    int x = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) { const int y = __shfl_up(x, o, 64); if (lane >= o) x += y; }
    if (lane == 63) red[wave] = x;
    __syncthreads();
    int base = 0, all = 0;
    for (int w = 0; w < 16; ++w) { if (w < wave) base += red[w]; all += red[w]; }
    int run = base + x - local;
    for (int i = b; i < e; ++i) { const int c = bsum[i]; bsum[i] = run; run += c; }
    if (tid == 0) *total = all;
}

__global__ __launch_bounds__(256) void stage_add_kernel(int32_t* __restrict__ offs, int n_kv,
                                                        const int32_t* __restrict__ bsum)
{
    const int s = blockIdx.x * 256 + threadIdx.x;
    if (s < n_kv) offs[s] += bsum[blockIdx.x];
}

__global__ __launch_bounds__(256) void stage_list_kernel(const int32_t* __restrict__ idx, int r0,
                                                         int C, int topk, int n_kv, int W,
                                                         const uint32_t* __restrict__ mask,
                                                         const int32_t* __restrict__ offs,
                                                         const uint8_t* __restrict__ dup,
                                                         int32_t* __restrict__ list)
{
    const int64_t n = (int64_t)C * topk;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
        const int t = (int)(e / topk);
        const int s = idx[(int64_t)r0 * topk + e];
        if (s < 0 || s >= n_kv || dup[e]) continue;    // one listed entry per (key, row)
        const uint32_t* m = mask + (int64_t)s * W;
        int rank = __popc(m[t >> 5] & ((1u << (t & 31)) - 1u));
        for (int w = 0; w < (t >> 5); ++w) rank += __popc(m[w]);
        list[offs[s] + rank] = (int32_t)e;
    }
}

// One workgroup per key, one wave per group: sum the key's staged rows (256 floats: dV then
// dK) in row order and add them into dv / dk.
__global__ __launch_bounds__(256) void stage_reduce_kernel(const float* __restrict__ stg,
                                                           const int32_t* __restrict__ offs,
                                                           const int32_t* __restrict__ list,
                                                           int G, float* __restrict__ dk,
                                                           float* __restrict__ dv)
{
    const int s = blockIdx.x;
    const int b = offs[s], e = offs[s + 1];
    if (b == e) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int g = wave; g < G; g += 4) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        int j = b;
        for (; j + 8 <= e; j += 8) {                     // eight rows in flight, added in order
            v4f x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                x[u] = __builtin_nontemporal_load(
                    reinterpret_cast<const v4f*>(stg + ((int64_t)list[j + u] * G + g) * 256) + lane);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                acc.x += x[u][0]; acc.y += x[u][1]; acc.z += x[u][2]; acc.w += x[u][3];
            }
        }
        for (; j < e; ++j) {
            const v4f x = __builtin_nontemporal_load(
                reinterpret_cast<const v4f*>(stg + ((int64_t)list[j] * G + g) * 256) + lane);
            acc.x += x[0]; acc.y += x[1]; acc.z += x[2]; acc.w += x[3];
        }
        // lanes 0..31 hold dV[4 lane .. +4), lanes 32..63 dK[4 (lane - 32) .. +4)
        float* dst = (lane < 32 ? dv : dk) + ((int64_t)s * G + g) * 128 + 4 * (lane & 31);
        float4 o = *reinterpret_cast<float4*>(dst);
        o.x += acc.x; o.y += acc.y; o.z += acc.z; o.w += acc.w;
        *reinterpret_cast<float4*>(dst) = o;
    }
}

// The same for rows of 128 floats with one destination (the indexer's dk^I): one wave per key.
__global__ __launch_bounds__(64) void stage_reduce128_kernel(const float* __restrict__ stg,
                                                             const int32_t* __restrict__ offs,
                                                             const int32_t* __restrict__ list,
                                                             float* __restrict__ dst)
{
    const int s = blockIdx.x;
    const int b = offs[s], e = offs[s + 1];
    if (b == e) return;
    const int lane = threadIdx.x;
    typedef float v2f __attribute__((ext_vector_type(2)));
    float ax = 0.f, ay = 0.f;
    int j = b;
    for (; j + 8 <= e; j += 8) {                         // eight rows in flight, added in order
        v2f x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            x[u] = __builtin_nontemporal_load(reinterpret_cast<const v2f*>(stg + (int64_t)list[j + u] * 128) + lane);
#pragma unroll
        for (int u = 0; u < 8; ++u) { ax += x[u][0]; ay += x[u][1]; }
    }
    for (; j < e; ++j) {
        const v2f x = __builtin_nontemporal_load(reinterpret_cast<const v2f*>(stg + (int64_t)list[j] * 128) + lane);
        ax += x[0]; ay += x[1];
    }
    float2* o = reinterpret_cast<float2*>(dst + (int64_t)s * 128) + lane;
    float2 v = *o;
    v.x += ax; v.y += ay;
    *o = v;
}

// fp32 kernel (vector ALU; exact-ish reference-grade path).  One workgroup per
// query row, wave per group; 64 selected positions per step, one per lane.
template <bool PAGED>
__global__ __launch_bounds__(256) void sparse_attn_f32_kernel(AttnArgs p, int nsplit, int per_split,
                                                              float* __restrict__ partials)
{
    __shared__ float qs_[kAttnWaves][16][128];
    __shared__ float ps_[kAttnWaves][64][17];
    __shared__ int rows_[kAttnWaves][64];
    const int work = xcd_remap(blockIdx.x, gridDim.x);
    const int row = work / nsplit, split = work - row * nsplit;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int hpg = p.Hq / p.G;
    int seq = 0;
    int64_t len = p.n_kv;
    if (PAGED) {
        seq = p.row_seq ? p.row_seq[row] : row;
        const int64_t cap = (int64_t)p.max_blocks * p.block_size;
        len = p.seq_lens ? (int64_t)p.seq_lens[seq] : cap;
        if (len > cap) len = 0;
    }
    if (p.n_kv <= 0) len = 0;
    const int32_t* __restrict__ idx_row = p.idx + (int64_t)row * p.topk;
    const int k_begin = split * per_split;
    const int k_end = len > 0 ? min(row_extent(idx_row, p.topk, lane), k_begin + per_split) : k_begin;
    const float* __restrict__ Q = static_cast<const float*>(p.q);
    const float* __restrict__ K = static_cast<const float*>(p.k);
    const float* __restrict__ V = static_cast<const float*>(p.v);

    for (int g = wave; g < p.G; g += kAttnWaves) {
        for (int i = lane; i < hpg * 128; i += 64)
            qs_[wave][i / 128][i % 128] = Q[((int64_t)row * p.Hq + g * hpg) * 128 + i];
        __builtin_amdgcn_wave_barrier();
        float m_run[16], l_part[16], o0[16], o1[16];
#pragma unroll
        for (int h = 0; h < 16; ++h) { m_run[h] = -INFINITY; l_part[h] = 0.f; o0[h] = 0.f; o1[h] = 0.f; }
        for (int kb0 = k_begin; kb0 < k_end; kb0 += 64) {
            const int prow = resolve_row<PAGED>(p, idx_row, kb0 + lane, k_end, seq, len);
            rows_[wave][lane] = prow;
            float s[16];
#pragma unroll
            for (int h = 0; h < 16; ++h) s[h] = 0.f;
            if (prow >= 0) {
                const float* kr = K + ((int64_t)prow * p.G + g) * 128;
                for (int e = 0; e < 128; e += 4) {
                    const float4 kv = *reinterpret_cast<const float4*>(kr + e);
#pragma unroll
                    for (int h = 0; h < 16; ++h)
                        if (h < hpg)
                            s[h] += qs_[wave][h][e] * kv.x + qs_[wave][h][e + 1] * kv.y +
                                    qs_[wave][h][e + 2] * kv.z + qs_[wave][h][e + 3] * kv.w;
                }
            }
#pragma unroll
            for (int h = 0; h < 16; ++h) {
                if (h >= hpg) continue;
                const float sv = prow >= 0 ? s[h] * p.sm_scale : -INFINITY;
                const float mx = wave_max(sv);
                const float m_new = fmaxf(m_run[h], mx);
                const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
                const float alpha = expf(m_run[h] - m_use);
                const float pr = expf(sv - m_use);
                l_part[h] = l_part[h] * alpha + pr;
                o0[h] *= alpha;
                o1[h] *= alpha;
                m_run[h] = m_new;
                ps_[wave][lane][h] = pr;
            }
            __builtin_amdgcn_wave_barrier();
            // lanes now own head dims 2 lane, 2 lane + 1
            for (int j = 0; j < 64; ++j) {
                const int r = rows_[wave][j];
                if (r < 0) continue;
                const float2 vv = *reinterpret_cast<const float2*>(V + ((int64_t)r * p.G + g) * 128 + 2 * lane);
#pragma unroll
                for (int h = 0; h < 16; ++h) {
                    if (h < hpg) {
                        const float pr = ps_[wave][j][h];
                        o0[h] += pr * vv.x;
                        o1[h] += pr * vv.y;
                    }
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
#pragma unroll
        for (int h = 0; h < 16; ++h) {
            if (h >= hpg) continue;
            const float l = wave_sum(l_part[h]);
            if (nsplit == 1) {
                const float inv = l > 0.f ? 1.f / l : 0.f;
                float* outp = static_cast<float*>(p.out) + ((int64_t)row * p.Hq + g * hpg + h) * 128;
                *reinterpret_cast<float2*>(outp + 2 * lane) = make_float2(o0[h] * inv, o1[h] * inv);
                if (p.lse && lane == 0) p.lse[(int64_t)row * p.Hq + g * hpg + h] = m_run[h] + logf(l);
            } else {
                float* part = partials + (((int64_t)row * nsplit + split) * p.Hq + g * hpg + h) * (128 + 2);
                part[2 * lane] = o0[h];
                part[2 * lane + 1] = o1[h];
                // m is in the natural-log domain here; the combine kernel expects log2
                if (lane == 0) { part[128] = m_run[h] * kLog2e; part[129] = l; }
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// Merge the nsplit partial softmax results of each (row, head).
__global__ __launch_bounds__(128) void attn_combine_kernel(const float* __restrict__ partials,
                                                           int nsplit, int Hq, int bf16,
                                                           void* __restrict__ out,
                                                           float* __restrict__ lse)
{
    const int row = blockIdx.x / Hq, head = blockIdx.x % Hq;
    const int dim = threadIdx.x;
    const float* base = partials + (((int64_t)row * nsplit) * Hq + head) * 130;
    const int64_t stride = (int64_t)Hq * 130;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, base[s * stride + 128]);
    float L = 0.f, acc = 0.f;
    if (M != -INFINITY) {
        for (int s = 0; s < nsplit; ++s) {
            const float f = exp2f(base[s * stride + 128] - M);
            L += f * base[s * stride + 129];
            acc += f * base[s * stride + dim];
        }
    }
    const float r = L > 0.f ? acc / L : 0.f;
    if (lse && dim == 0) lse[(int64_t)row * Hq + head] = M == -INFINITY ? -INFINITY : (M + __log2f(L)) * kLn2;
    const int64_t o = ((int64_t)row * Hq + head) * 128 + dim;
    if (bf16) static_cast<uint16_t*>(out)[o] = f32_to_bf16_bits(r);
    else static_cast<float*>(out)[o] = r;
}

}  // namespace

#ifndef DSA_ATTN_MIN_SPLIT
#define DSA_ATTN_MIN_SPLIT 256
#endif

int attn_num_splits(int Tq, int topk)
{
    // Enough workgroups to fill 256 CUs several times over; splits of >= DSA_ATTN_MIN_SPLIT positions.
    if (Tq >= 2048) return 1;
    int ns = 1;
    while ((int64_t)Tq * ns < 2048 && topk / (ns * 2) >= DSA_ATTN_MIN_SPLIT) ns *= 2;
    return ns;
}

size_t attn_partials_bytes(int Tq, int nsplit, int Hq, int d)
{
    if (nsplit <= 1) return 0;
    return (size_t)Tq * nsplit * Hq * (d + 2) * sizeof(float);
}

hipError_t launch_sparse_attn(const AttnArgs& a, int nsplit, float* partials, hipStream_t stream)
{
    if (a.Tq == 0) return hipSuccess;
    const int step = a.bf16 ? kStep : 64;
    int per_split = (a.topk + nsplit - 1) / nsplit;
    per_split = (per_split + step - 1) / step * step;
    nsplit = (a.topk + per_split - 1) / per_split;
    if (nsplit < 1) nsplit = 1;
    const int64_t n = (int64_t)a.Tq * nsplit;
    if (n > INT32_MAX) return hipErrorInvalidValue;
    const bool paged = a.block_table != nullptr;
    if (a.bf16) {
        if (paged)
            hipLaunchKernelGGL(sparse_attn_bf16_kernel<true>, dim3((unsigned)n), dim3(256), 0, stream, a, nsplit, per_split, partials);
        else
            hipLaunchKernelGGL(sparse_attn_bf16_kernel<false>, dim3((unsigned)n), dim3(256), 0, stream, a, nsplit, per_split, partials);
    } else {
        if (paged)
            hipLaunchKernelGGL(sparse_attn_f32_kernel<true>, dim3((unsigned)n), dim3(256), 0, stream, a, nsplit, per_split, partials);
        else
            hipLaunchKernelGGL(sparse_attn_f32_kernel<false>, dim3((unsigned)n), dim3(256), 0, stream, a, nsplit, per_split, partials);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || nsplit == 1) return err;
    hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)(a.Tq * a.Hq)), dim3(128), 0, stream, partials,
                       nsplit, a.Hq, a.bf16, a.out, a.lse);
    return hipGetLastError();
}

hipError_t launch_fill_zero(uint32_t* p, int64_t n, hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

hipError_t launch_sparse_attn_bwd(const AttnBwdArgs& a, hipStream_t stream)
{
    if (a.Tq == 0) return hipSuccess;
    if (a.vals && a.topk > kBwdMaxTopk) return hipErrorInvalidValue;
    hipLaunchKernelGGL(sparse_attn_bwd_kernel, dim3((unsigned)a.Tq), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_stage_reduce(const int32_t* idx, int r0, int C, int topk, int n_kv, int G,
                               const float* stg, uint32_t* mask, int32_t* offs, int32_t* list,
                               uint8_t* dup, float* dk, float* dv, hipStream_t stream, int width)
{
    if (width != 256 && width != 128) return hipErrorInvalidValue;
    if (C == 0 || n_kv == 0) return hipSuccess;
    const int W = (C + 31) / 32;
    const int64_t nm = (int64_t)n_kv * W, ne = (int64_t)C * topk;
    const unsigned gm = (unsigned)std::min<int64_t>((nm + 255) / 256, 65536);
    const unsigned ge = (unsigned)std::min<int64_t>((ne + 255) / 256, 65536);
    hipLaunchKernelGGL(fill_u32_kernel, dim3(gm), dim3(256), 0, stream, mask, nm);
    hipLaunchKernelGGL(stage_mark_kernel, dim3(ge), dim3(256), 0, stream, idx, r0, C, topk, n_kv, W, mask, dup);
    const int nb = (n_kv + 255) / 256;
    int32_t* bsum = offs + n_kv + 1;                  // nb more entries after the offsets
    hipLaunchKernelGGL(stage_count_kernel, dim3(nb), dim3(256), 0, stream, mask, n_kv, W, offs, bsum);
    hipLaunchKernelGGL(stage_scan_kernel, dim3(1), dim3(1024), 0, stream, bsum, nb, offs + n_kv);
    hipLaunchKernelGGL(stage_add_kernel, dim3(nb), dim3(256), 0, stream, offs, n_kv, bsum);
    hipLaunchKernelGGL(stage_list_kernel, dim3(ge), dim3(256), 0, stream, idx, r0, C, topk, n_kv, W, mask, offs, dup, list);
    if (width == 256)
        hipLaunchKernelGGL(stage_reduce_kernel, dim3(n_kv), dim3(256), 0, stream, stg, offs, list, G, dk, dv);
    else
        hipLaunchKernelGGL(stage_reduce128_kernel, dim3(n_kv), dim3(64), 0, stream, stg, offs, list, dk);
    hipLaunchKernelGGL(stage_dup_add_kernel, dim3(ge), dim3(256), 0, stream, idx, r0, C, topk, G,
                       width, dup, stg, dk, dv);
    return hipGetLastError();
}

}  // namespace dsa
