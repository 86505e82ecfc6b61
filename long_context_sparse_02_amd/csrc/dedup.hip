// dedup.hip -- adjacent-query Top-KV deduplication for the prefill's sparse attention
// (Keye-VL-2.0 report section 5.3, sparse attention optimisation: adjacent queries select
// largely the same keys, so a block of them gathers the union of its selections once and
// masks each query's own entries inside the matrix products).
//
// A block is 16 adjacent query rows of a chunk.  Its Omega_t (t in the block) are merged into
// one ascending union list with a 16-bit mask per union position (bit q: row q of the block
// selected it).  For each union position, the attention of query q over Omega_q is the
// attention over the union with the positions whose bit q is clear removed, so
//   out[q, h] = sum_{u : bit q of mask[u]} softmax(sm_scale q_h . K_u) V_u
// is the same sum as the per-query kernel's, over the same positions in the same ascending
// order; only the online softmax's step boundaries (64 union positions here, 32 selected
// positions there) and hence the rounding differ.
//
// Cost model.  Per union position and KV group the block gathers one K and one V row
// (512 bytes) and does the work of all 16 queries (the masked ones included); the per-query
// kernel gathers 512 bytes and does one query's work per selected (row, position).  So the
// union pays when its size U is well below the block's selection count sum_t n_t: the union
// kernel measures both and marks the block for the dedup kernel when kappa * U < sum_t n_t
// (kappa: the measured cost of a union position relative to a selected entry); the
// per-query kernel then skips the block's rows, and every other block runs as before.
#include "device_common.h"
#include "internal.h"

namespace dsa {
namespace {

constexpr int kBlk = kDedupRows;           // query rows per block (16)
constexpr int kUStep = 64;                 // union positions per step of the attention
constexpr int kKPitch = 136;               // LDS row pitch of the K tile (bf16 elements)
constexpr int kVTPitch = 68;               // LDS row pitch of the V^T tile (bf16 elements)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.f;               // log2 headroom of the lazily rescaled softmax

// ---------------------------------------------------------------- union of a block's lists
// Block b holds the chunk's rows at positions 16 B .. 16 B + 15 (B = b + the chunk's first
// block): rows r0 + q for q = q_lo .. q_hi - 1, bit q of a mask.

// Count: an LDS bitmap of the block's selected positions (positions < n_pos <= 32 *
// kDedupMaxWords) gives the union size U; info[b] = {U, selections, marked}, marked when
// kappa * U < selections.  Kept small (the bitmap only) so that several workgroups share a CU:
// every block of every chunk runs it.
__global__ __launch_bounds__(256) void union_count_kernel(const int32_t* __restrict__ idx, int Tq,
                                                          int off, int topk, int n_pos,
                                                          float kappa, int32_t* __restrict__ info,
                                                          int* __restrict__ counter)
{
    __shared__ uint32_t bits[kDedupMaxWords];
    __shared__ int red[8];
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r0 = b * kBlk - off;
    const int q_lo = max(0, -r0), q_hi = min(kBlk, Tq - r0);
    const int nw = (n_pos + 31) >> 5;
    const int nsel_max = (q_hi - q_lo) * topk;
    const int32_t* __restrict__ rows = idx + (int64_t)(r0 + q_lo) * topk;
    for (int w = tid; w < nw; w += 256) bits[w] = 0u;
    __syncthreads();
    int nsel = 0;
    for (int e = tid; e < nsel_max; e += 256) {
        const int s = rows[e];
        if (s >= 0 && s < n_pos) {
            atomicOr(&bits[s >> 5], 1u << (s & 31));
            ++nsel;
        }
    }
    __syncthreads();
    int c = 0;
    for (int w = tid; w < nw; w += 256) c += __popc(bits[w]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        c += __shfl_xor(c, o, 64);
        nsel += __shfl_xor(nsel, o, 64);
    }
    if (lane == 0) { red[wave] = c; red[4 + wave] = nsel; }
    __syncthreads();
    if (tid == 0) {
        const int U = red[0] + red[1] + red[2] + red[3];
        const int sel = red[4] + red[5] + red[6] + red[7];
        const bool use = sel > 0 && kappa * (float)U < (float)sel;
        info[3 * b] = U;
        info[3 * b + 1] = sel;
        info[3 * b + 2] = use ? 1 : 0;
        if (use && counter) atomicAdd(counter, 1);
    }
}

// List (marked blocks only; the others exit at once): the bitmap again, prefix counts of its
// words, then each selection's union slot is its position's rank in the bitmap; list[b, 0 ..
// U) gets the ascending union and mask[b, 0 .. U) the rows that selected each position.
__global__ __launch_bounds__(256) void union_list_kernel(const int32_t* __restrict__ idx, int Tq,
                                                         int off, int topk, int n_pos,
                                                         const int32_t* __restrict__ info,
                                                         int32_t* __restrict__ ulist,
                                                         uint16_t* __restrict__ umask)
{
    __shared__ uint32_t bits[kDedupMaxWords];
    __shared__ int32_t wpre[kDedupMaxWords];
    __shared__ uint32_t m32[kBlk * kDedupMaxTopk / 2];     // two 16-bit masks per word
    __shared__ int red[4];
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (info[3 * b + 2] == 0) return;                       // uniform: a per-query block
    const int U = info[3 * b];
    const int r0 = b * kBlk - off;
    const int q_lo = max(0, -r0), q_hi = min(kBlk, Tq - r0);
    const int nw = (n_pos + 31) >> 5;
    const int nsel_max = (q_hi - q_lo) * topk;
    const int32_t* __restrict__ rows = idx + (int64_t)(r0 + q_lo) * topk;
    const int64_t cap = (int64_t)kBlk * topk;

    for (int w = tid; w < nw; w += 256) bits[w] = 0u;
    for (int i = tid; i < (U + 1) / 2; i += 256) m32[i] = 0u;
    __syncthreads();
    for (int e = tid; e < nsel_max; e += 256) {
        const int s = rows[e];
        if (s >= 0 && s < n_pos) atomicOr(&bits[s >> 5], 1u << (s & 31));
    }
    __syncthreads();
    // exclusive prefix of the words' popcounts: each thread a contiguous run of words
    const int per = (nw + 255) / 256;
    const int w0 = min(tid * per, nw), w1 = min(w0 + per, nw);
    int c = 0;
    for (int w = w0; w < w1; ++w) c += __popc(bits[w]);
    int x = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) red[wave] = x;
    __syncthreads();
    int run = x - c;
    for (int w = 0; w < wave; ++w) run += red[w];
    for (int w = w0; w < w1; ++w) {
        wpre[w] = run;
        run += __popc(bits[w]);
    }
    __syncthreads();
    for (int e = tid; e < nsel_max; e += 256) {
        const int s = rows[e];
        if (s >= 0 && s < n_pos) {
            const uint32_t word = bits[s >> 5];
            const int slot = wpre[s >> 5] + __popc(word & ((1u << (s & 31)) - 1u));
            atomicOr(&m32[slot >> 1], (1u << (q_lo + e / topk)) << (16 * (slot & 1)));
        }
    }
    __syncthreads();
    int32_t* __restrict__ lst = ulist + (int64_t)b * cap;
    uint16_t* __restrict__ msk = umask + (int64_t)b * cap;
    for (int w = w0; w < w1; ++w) {
        uint32_t word = bits[w];
        int slot = wpre[w];
        while (word) {
            const int bit = __ffs(word) - 1;
            word &= word - 1u;
            lst[slot++] = 32 * w + bit;
        }
    }
    for (int i = tid; i < U; i += 256) msk[i] = (uint16_t)(m32[i >> 1] >> (16 * (i & 1)));
}

// ----------------------------------------------------------- attention over a block's union
// One workgroup of 4 waves per (block, KV group) with heads_per_group == 8.  Wave w takes the
// block's queries 4w .. 4w+3: its 32 columns are (query 4w + 2c + col / 8, head col % 8) for
// column tiles c = 0, 1.  Per step of 64 union positions the workgroup gathers their K and V
// rows of the group once (whole-line requests, four rows per instruction) into a shared K tile
// and a transposed V tile; each wave computes S^T = K Q^T (positions x its 32 columns) on the
// bf16 matrix core, masks the positions its queries did not select, runs the online softmax
// per column in the exp2 domain and accumulates O^T = V^T P^T.  A lane's softmax values are
// exactly its B operand for the second product (its positions 4 grp + j of two 16-position
// tiles), so no shuffle is needed.
// Where a block's union comes from: the union kernel's lists (any selections), or, for blocks of
// whole-prefix rows, the positions 0 .. U - 1 themselves with causal masks.
struct UnionLists {
    const int32_t* info; const int32_t* list; const uint16_t* mask;
    int off;                                             // q_pos0 % 16 of the launch
};

__device__ __forceinline__ int find_segment(const PrefixBlocks& pb, int j) {
    int lo = 0, hi = pb.n - 1;                           // largest i with blk_start[i] <= j
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pb.blk_start[mid] <= j) lo = mid; else hi = mid - 1;
    }
    return lo;
}

template <typename Src>
__global__ __launch_bounds__(256, 2) void dedup_attn_kernel(AttnArgs p, Src src)
{
    constexpr bool PREFIX = __is_same(Src, PrefixBlocks);
    __shared__ __attribute__((aligned(16))) uint16_t kt[kUStep][kKPitch];
    __shared__ __attribute__((aligned(16))) uint16_t vtt[128][kVTPitch];
    __shared__ uint16_t mk[kUStep];
    const int G = p.G;
    // prefix blocks grow with their position: the longest go first and neighbours go to
    // different XCDs (dispatch order), so the launch ends evenly; union blocks keep adjacent
    // blocks on one XCD, whose L2 then holds their shared rows
    const int work = PREFIX ? (int)(gridDim.x - 1 - blockIdx.x) : xcd_remap(blockIdx.x, gridDim.x);
    const int b = work / G, g = work - b * G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, grp = lane >> 4;
    int U, r0, kv0 = 0, p0 = 0;                          // r0: launch row of the block's query 0
    const int32_t* __restrict__ lst = nullptr;
    const uint16_t* __restrict__ msk = nullptr;
    uint32_t qvalid = 0xffffu;                           // rows of the block that exist
    if constexpr (PREFIX) {
        const int i = find_segment(src, b);
        p0 = (src.blk0[i] + b - src.blk_start[i]) * kBlk;    // position of query 0
        U = min(p0 + kBlk, src.len[i]);
        r0 = src.row0[i] + p0;
        kv0 = src.kv0[i];
        qvalid = 0u;
        for (int q = 0; q < kBlk; ++q)
            if (p0 + q < src.len[i] && r0 + q >= 0 && r0 + q < p.Tq) qvalid |= 1u << q;
    } else {
        if (src.info[3 * b + 2] == 0) return;            // uniform: a per-query block
        U = src.info[3 * b];
        const int64_t cap = (int64_t)kBlk * p.topk;
        lst = src.list + (int64_t)b * cap;
        msk = src.mask + (int64_t)b * cap;
        r0 = b * kBlk - src.off;
    }
    const uint16_t* __restrict__ Q = static_cast<const uint16_t*>(p.q);
    const uint16_t* __restrict__ K = static_cast<const uint16_t*>(p.k);
    const uint16_t* __restrict__ V = static_cast<const uint16_t*>(p.v);
    const float scale = p.sm_scale * kLog2e;

    // B operands of S^T: column col of tile c is (query 4 wave + 2 c + col / 8, head col % 8);
    // MFMA m takes head dims 8 (4 m + grp) .. +8 from lane group grp
    v8bf qb[2][4];
    int qbit[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int qi = 4 * wave + 2 * c + (col >> 3);
        qbit[c] = 1 << qi;
        const int row = r0 + qi;
        const int head = g * 8 + (col & 7);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            v4i x = {0, 0, 0, 0};
            if (row >= 0 && row < p.Tq && ((qvalid >> qi) & 1u)) x = *reinterpret_cast<const v4i*>(Q + ((int64_t)row * p.Hq + head) * 128 + (4 * m + grp) * 8);
            qb[c][m] = __builtin_bit_cast(v8bf, x);
        }
    }
    float m_run[2] = {-INFINITY, -INFINITY}, l_part[2] = {0.f, 0.f};
    v4f o[8][2];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt][0] = o[dt][1] = v4f{0.f, 0.f, 0.f, 0.f};

    // gather of one step: wave w loads union positions 16 w .. 16 w + 15 of the step, lane l
    // 16 bytes of row 4 it + l / 16 (four whole 256-byte rows per instruction)
    v4i kk[4], vv[4];
    int prow = -1;
    uint16_t mbits = 0;
    auto fetch = [&](int u0) {
        const int u = u0 + 16 * wave + col;
        const bool ok = u < U;
        if constexpr (PREFIX) {
            // position u is selected by the block's rows at positions >= u
            prow = ok ? kv0 + u : -1;
            mbits = ok ? (uint16_t)(qvalid & (0xffffu << min(max(u - p0, 0), 16))) : (uint16_t)0;
        } else {
            const int s = lst[min(u, U - 1)];
            prow = ok ? s : -1;
            mbits = ok ? msk[min(u, U - 1)] : (uint16_t)0;
        }
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int r = __shfl(prow, 4 * it + grp, 64);
            const int64_t off = ((int64_t)max(r, 0) * G + g) * 128 + col * 8;
            kk[it] = *reinterpret_cast<const v4i*>(K + off);
            vv[it] = *reinterpret_cast<const v4i*>(V + off);
        }
    };
    if (U > 0) fetch(0);
    for (int u0 = 0; u0 < U; u0 += kUStep) {
        __syncthreads();                                  // the previous step's reads are done
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int pr = 16 * wave + 4 * it + grp;      // position within the step
            *reinterpret_cast<v4i*>(&kt[pr][col * 8]) = kk[it];
            const v8s x = __builtin_bit_cast(v8s, vv[it]);
#pragma unroll
            for (int j = 0; j < 8; ++j) vtt[col * 8 + j][pr] = (uint16_t)x[j];
        }
        if (grp == 0) mk[16 * wave + col] = mbits;
        __syncthreads();
        if (u0 + kUStep < U) fetch(u0 + kUStep);          // in flight during this step's math

        // S^T: position tiles pt = 0..3 (16 positions each) x column tiles c
        v4f s[4][2];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
            s[pt][0] = s[pt][1] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const v8bf ka = *reinterpret_cast<const v8bf*>(&kt[16 * pt + col][(4 * m + grp) * 8]);
                s[pt][0] = mfma_bf16_16x16x32(ka, qb[0][m], s[pt][0]);
                s[pt][1] = mfma_bf16_16x16x32(ka, qb[1][m], s[pt][1]);
            }
        }
        // masks of this lane's 16 positions: 16 pt + 4 grp + i
        uint32_t mrow[4][4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int i = 0; i < 4; ++i) mrow[pt][i] = mk[16 * pt + 4 * grp + i];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            // raw logits of the positions this column's query selected (the scale is positive,
            // so the maximum commutes with it; it is folded into the exponent below)
            float sl[16];
            float mx = -INFINITY;
#pragma unroll
            for (int pt = 0; pt < 4; ++pt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float v = (mrow[pt][i] & qbit[c]) ? s[pt][c][i] : -INFINITY;
                    sl[4 * pt + i] = v;
                    mx = fmaxf(mx, v);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            // lazy rescaling: the running reference m_run (scaled, log2 units) only moves when a
            // logit exceeds it by more than kLazy, so P stays below 2^kLazy and the accumulators
            // are rescaled rarely (the final division cancels the common factor)
            // (a per-lane decision: a column's arithmetic does not depend on the other columns
            // of the wave, so a row's output is the same whichever rows share its block)
            const float mxs = mx * scale;
            if (mxs > m_run[c] + kLazy) {
                const float alpha = exp2f(m_run[c] - mxs);        // 0 when m_run is -inf
                m_run[c] = mxs;
                l_part[c] *= alpha;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) o[dt][c] = o[dt][c] * alpha;
            }
            const float m_use = (m_run[c] == -INFINITY) ? 0.f : m_run[c];
            float psum = 0.f;
            v8bf pb[2];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float pa = exp2f(fmaf(sl[4 * (2 * h) + i], scale, -m_use));
                    const float pc = exp2f(fmaf(sl[4 * (2 * h + 1) + i], scale, -m_use));
                    psum += pa + pc;
                    pb[h][i] = (__bf16)pa;
                    pb[h][4 + i] = (__bf16)pc;
                }
            l_part[c] += psum;
            // O^T += V^T P^T over 8 tiles of 16 head dims, positions 32 h .. 32 h + 31
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint2 lo = *reinterpret_cast<const uint2*>(&vtt[dt * 16 + col][32 * h + 4 * grp]);
                    const uint2 hi = *reinterpret_cast<const uint2*>(&vtt[dt * 16 + col][32 * h + 16 + 4 * grp]);
                    const v4i va = {(int)lo.x, (int)lo.y, (int)hi.x, (int)hi.y};
                    o[dt][c] = mfma_bf16_16x16x32(__builtin_bit_cast(v8bf, va), pb[h], o[dt][c]);
                }
            }
        }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        float l = l_part[c];
        l += __shfl_xor(l, 16, 64);
        l += __shfl_xor(l, 32, 64);
        const int qi = 4 * wave + 2 * c + (col >> 3);
        const int row = r0 + qi;
        if (row < 0 || row >= p.Tq || !((qvalid >> qi) & 1u)) continue;
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const int head = g * 8 + (col & 7);
        uint16_t* outp = static_cast<uint16_t*>(p.out) + ((int64_t)row * p.Hq + head) * 128;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const uint32_t lo = f32_to_bf16_bits(o[dt][c][0] * inv) | ((uint32_t)f32_to_bf16_bits(o[dt][c][1] * inv) << 16);
            const uint32_t hi = f32_to_bf16_bits(o[dt][c][2] * inv) | ((uint32_t)f32_to_bf16_bits(o[dt][c][3] * inv) << 16);
            *reinterpret_cast<uint2*>(outp + dt * 16 + 4 * grp) = make_uint2(lo, hi);
        }
    }
}

}  // namespace

bool dedup_supported(int Hq, int G, int d, int topk, int64_t n_pos, int bf16) {
    return bf16 && d == 128 && G >= 1 && Hq == 8 * G && topk >= 1 && topk <= kDedupMaxTopk &&
           n_pos >= 1 && n_pos <= 32LL * kDedupMaxWords;
}

int dedup_blocks(int Tq, int64_t q_pos0) {
    const int off = (int)(q_pos0 % kBlk);
    return (Tq + off + kBlk - 1) / kBlk;
}

hipError_t launch_dedup_union(const int32_t* idx, int Tq, int64_t q_pos0, int topk, int n_pos,
                              float kappa, int32_t* info, int32_t* ulist, uint16_t* umask,
                              int* counter, hipStream_t stream)
{
    if (Tq == 0) return hipSuccess;
    if (topk > kDedupMaxTopk || n_pos > 32 * kDedupMaxWords) return hipErrorInvalidValue;
    const int off = (int)(q_pos0 % kBlk);
    const dim3 grid((unsigned)dedup_blocks(Tq, q_pos0));
    hipLaunchKernelGGL(union_count_kernel, grid, dim3(256), 0, stream, idx, Tq, off, topk, n_pos,
                       kappa, info, counter);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(union_list_kernel, grid, dim3(256), 0, stream, idx, Tq, off, topk, n_pos,
                       info, ulist, umask);
    return hipGetLastError();
}

hipError_t launch_dedup_attn(const AttnArgs& a, int64_t q_pos0, const int32_t* info,
                             const int32_t* ulist, const uint16_t* umask, hipStream_t stream)
{
    if (a.Tq == 0) return hipSuccess;
    if (!a.bf16 || a.block_table || a.Hq != 8 * a.G || a.topk > kDedupMaxTopk)
        return hipErrorInvalidValue;
    const int64_t n = (int64_t)dedup_blocks(a.Tq, q_pos0) * a.G;
    if (n > INT32_MAX) return hipErrorInvalidValue;
    const UnionLists src{info, ulist, umask, (int)(q_pos0 % kBlk)};
    hipLaunchKernelGGL(dedup_attn_kernel<UnionLists>, dim3((unsigned)n), dim3(256), 0, stream, a,
                       src);
    return hipGetLastError();
}

hipError_t launch_dedup_prefix_attn(const AttnArgs& a, const PrefixBlocks& pb, hipStream_t stream)
{
    if (a.Tq == 0 || pb.n == 0) return hipSuccess;
    if (!a.bf16 || a.block_table || a.Hq != 8 * a.G || pb.n > kMaxPrefixSegs)
        return hipErrorInvalidValue;
    const int64_t n = (int64_t)pb.blk_start[pb.n] * a.G;
    if (n == 0) return hipSuccess;
    if (n > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(dedup_attn_kernel<PrefixBlocks>, dim3((unsigned)n), dim3(256), 0, stream, a,
                       pb);
    return hipGetLastError();
}

int64_t prefix_block_limit(int64_t len, int topk) {
    return len <= topk ? len : (int64_t)(topk / kBlk) * kBlk;
}

}  // namespace dsa
