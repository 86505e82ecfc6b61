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
#include "device_common.h"
#include "internal.h"

namespace dsa {
namespace {

constexpr int kAttnWaves = 4;
constexpr int kStep = 32;                 // selected positions per step
constexpr int kVPitch = 136;              // LDS row pitch of the V tile (bf16 elements)
constexpr float kLog2e = 1.4426950408889634f;

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
    const int work = xcd_remap(blockIdx.x, gridDim.x);
    const int row = work / nsplit, split = work - row * nsplit;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int hpg = p.Hq / p.G;

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
    const int k_end = len > 0 ? min(p.topk, k_begin + per_split) : k_begin;
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
    const int k_end = len > 0 ? min(p.topk, k_begin + per_split) : k_begin;
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
                                                           void* __restrict__ out)
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
                       nsplit, a.Hq, a.bf16, a.out);
    return hipGetLastError();
}

}  // namespace dsa
