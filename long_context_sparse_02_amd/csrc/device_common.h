// device_common.h -- small device helpers shared by the libdsa kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v8s __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// Matrix-core products used by the kernels.  Lane layout (checked on gfx950):
// lane l feeds row (l % 16) of A and column (l % 16) of B, with the same
// assignment of K elements to (l / 16, register slot) on both sides; the
// 16x16 fp32 result gives lane l rows 4*(l/16) .. 4*(l/16)+3 of column l % 16.
__device__ __forceinline__ v4f mfma_fp8_16x16x128(const v8i& a, const v8i& b, const v4f& c) {
    // format 0 = OCP E4M3 for both operands; E8M0 scale 127 = 2^0 (no scaling)
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ v4f mfma_bf16_16x16x32(const v8bf& a, const v8bf& b, const v4f& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// bf16 <-> fp32 (round to nearest even; NaN kept quiet)
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Workgroup id remapped so that consecutive work items run on the same XCD.
// Workgroups are dispatched round-robin over the 8 XCDs (id % 8); XCD x gets
// the contiguous work range [x*q + min(x, r), ...) of the n = 8q + r items.
__device__ __forceinline__ int xcd_remap(int b, int n) {
    const int x = b & 7, slot = b >> 3, q = n >> 3, r = n & 7;
    return x * q + (x < r ? x : r) + slot;
}

// Workgroup id remapped so that groups of 16 consecutive work items run on one XCD and the
// groups are dealt round-robin to the 8 XCDs: neighbouring items still share an XCD's L2, and
// work whose cost varies along the items (short rows first) is spread evenly over the XCDs.
// A bijection on [0, n): items past the last whole 128 keep their own id.
__device__ __forceinline__ int xcd_interleave16(int b, int n) {
    const int n_full = n & ~127;
    if (b >= n_full) return b;
    const int x = b & 7, k = b >> 3;
    return ((((k >> 4) << 3) + x) << 4) + (k & 15);
}

// Larger float -> larger unsigned key; -0 and +0 map to the same key.
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One past the last entry >= 0 of an index row of n entries (0 when there is none).  The
// entries after it are padding, so a kernel that stops there computes what one walking the
// whole row would: short rows (a position t < k keeps only t + 1 entries) cost what they hold.
// A row whose last entry is valid costs one load; others are scanned from the end, 2048
// entries per round trip in coalesced, unconditional loads.  Every lane of the wave must call
// it (the result is wave-uniform).
__device__ __forceinline__ int row_extent(const int32_t* __restrict__ idx_row, int n, int lane) {
    if (n <= 0) return 0;
    if (idx_row[n - 1] >= 0) return n;
    for (int hi = n - 1; hi > 0; hi -= 2048) {
        const int lo = hi > 2048 ? hi - 2048 : 0;
        int best = -1;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const int e = lo + 64 * j + lane;
            const int v = idx_row[min(e, hi - 1)];
            if (e < hi && v >= 0) best = e;
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) best = max(best, __shfl_xor(best, o, 64));
        if (best >= 0) return best + 1;
    }
    return 0;
}

__device__ __forceinline__ float wave_max(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

}  // namespace dsa
