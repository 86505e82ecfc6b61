// cache.hip -- the step before the decode path: per-token FP8 quantisation of
// indexer vectors and the append of a new token into the paged caches.
//
// The lightning indexer runs on FP8 inputs (Keye-VL-2.0 report section 2.3.1;
// the xllm-io review page credits the single FP8 key head for the indexer's
// low cost).  The pages give no quantisation recipe; the one read here (and
// used by every workload) is per-token absmax scaling into OCP E4M3:
// scale = amax / 448 over the token's values (1 for an all-zero token), each
// value divided by the scale in fp32 with correct rounding, clamped to
// [-448, 448] and rounded to the nearest E4M3 value, ties to the even code.
// The rounding is done on the fp32 bit pattern: keep 3 mantissa bits with
// round-to-nearest-even, carrying into the exponent; below 2^-6 (the E4M3
// subnormals, steps of 2^-9) the value is rounded to a multiple of 2^-9.
//
// Decode appends one token per sequence (report section 5.3 serves decode from
// paged caches): its K and V rows are copied into the cache block that the
// sequence's block table maps the position to, and its indexer key is
// quantised on the way into the k^I cache.
#include "device_common.h"
#include "internal.h"

namespace dsa {
namespace {

constexpr int kQuantThreads = 256;

__device__ __forceinline__ uint8_t e4m3_rne(float y)        // |y| <= 448
{
    const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
    const float a = fabsf(y);
    uint32_t code;
    if (a < 0.015625f) {                               // below 2^-6: multiples of 2^-9
        code = (uint32_t)rintf(a * 512.f);             // 0 .. 8 (8 is the smallest normal)
    } else {
        const uint32_t b = __float_as_uint(a);
        int e = (int)(b >> 23) - 127;                  // -6 .. 8
        const uint32_t mant = b & 0x7fffffu;
        uint32_t q = mant >> 20;
        const uint32_t rem = mant & 0xfffffu;
        if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ++q;
        if (q == 8u) { q = 0u; ++e; }
        code = ((uint32_t)(e + 7) << 3) | q;
    }
    return (uint8_t)(code | sign);
}

template <class T> __device__ __forceinline__ float load_val(const T* p, int64_t i);
template <> __device__ __forceinline__ float load_val<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float load_val<uint16_t>(const uint16_t* p, int64_t i) {
    return bf16_bits_to_f32(p[i]);
}

__device__ __forceinline__ float block_max(float v, float* red)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_max(v);
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float m = red[0];
    for (int i = 1; i < kQuantThreads / 64; ++i) m = fmaxf(m, red[i]);
    __syncthreads();
    return m;
}

// Row `row` of x [.., n] into codes [.., n] and scale[row] (one workgroup per row).
template <class T>
__device__ void quantize_row(const T* __restrict__ x, int64_t row, int n, uint8_t* __restrict__ codes,
                             float* __restrict__ scale_out, float* red)
{
    const int tid = threadIdx.x;
    const T* src = x + row * n;
    float amax = 0.f;
    for (int i = tid; i < n; i += kQuantThreads) amax = fmaxf(amax, fabsf(load_val(src, i)));
    amax = block_max(amax, red);
    const float s = amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f;
    if (tid == 0) *scale_out = s;
    uint8_t* dst = codes;
    for (int i = tid; i < n; i += kQuantThreads) {
        float y = __fdiv_rn(load_val(src, i), s);
        y = fminf(fmaxf(y, -448.f), 448.f);
        dst[i] = e4m3_rne(y);
    }
}

// The same for rows of at most kQuantThreads * kVecLoads 16-byte pieces (n a multiple of the
// values per piece, x and codes 16-byte aligned): every thread issues all of its loads at
// once and keeps the values in registers between the maximum and the rounding.
constexpr int kVecLoads = 8;

template <class T> struct Piece;
template <> struct Piece<float> {
    static constexpr int N = 4;
    __device__ static void get(const v4i& r, float* v) {
        for (int i = 0; i < 4; ++i) v[i] = __int_as_float(r[i]);
    }
    __device__ static void put(uint8_t* dst, const uint8_t* c) {
        *reinterpret_cast<uint32_t*>(dst) = c[0] | (c[1] << 8) | (c[2] << 16) | ((uint32_t)c[3] << 24);
    }
};
template <> struct Piece<uint16_t> {
    static constexpr int N = 8;
    __device__ static void get(const v4i& r, float* v) {
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float((uint32_t)r[i] << 16);
            v[2 * i + 1] = __uint_as_float((uint32_t)r[i] & 0xffff0000u);
        }
    }
    __device__ static void put(uint8_t* dst, const uint8_t* c) {
        const uint32_t lo = c[0] | (c[1] << 8) | (c[2] << 16) | ((uint32_t)c[3] << 24);
        const uint32_t hi = c[4] | (c[5] << 8) | (c[6] << 16) | ((uint32_t)c[7] << 24);
        *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
    }
};

template <class T>
__device__ void quantize_row_vec(const T* __restrict__ src, int n, uint8_t* __restrict__ dst,
                                 float* __restrict__ scale_out, float* red)
{
    constexpr int N = Piece<T>::N;
    const int tid = threadIdx.x;
    const int np = n / N;
    float v[kVecLoads][N];
    v4i raw[kVecLoads];
#pragma unroll
    for (int l = 0; l < kVecLoads; ++l)              // clamped, unconditional loads
        raw[l] = reinterpret_cast<const v4i*>(src)[min(tid + l * kQuantThreads, np - 1)];
    float amax = 0.f;
#pragma unroll
    for (int l = 0; l < kVecLoads; ++l) {
        Piece<T>::get(raw[l], v[l]);
        if (tid + l * kQuantThreads < np)
#pragma unroll
            for (int i = 0; i < N; ++i) amax = fmaxf(amax, fabsf(v[l][i]));
    }
    amax = block_max(amax, red);
    const float s = amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f;
    if (tid == 0) *scale_out = s;
#pragma unroll
    for (int l = 0; l < kVecLoads; ++l) {
        const int piece = tid + l * kQuantThreads;
        if (piece < np) {
            uint8_t c[N];
#pragma unroll
            for (int i = 0; i < N; ++i)
                c[i] = e4m3_rne(fminf(fmaxf(__fdiv_rn(v[l][i], s), -448.f), 448.f));
            Piece<T>::put(dst + (int64_t)piece * N, c);
        }
    }
}

template <class T, bool VEC>
__global__ __launch_bounds__(kQuantThreads) void quantize_e4m3_kernel(const T* __restrict__ x, int n,
                                                                      uint8_t* __restrict__ codes,
                                                                      float* __restrict__ scale)
{
    __shared__ float red[kQuantThreads / 64];
    const int64_t row = blockIdx.x;
    if (VEC) quantize_row_vec(x + row * n, n, codes + row * n, scale + row, red);
    else quantize_row(x, row, n, codes + row * n, scale + row, red);
}

// One workgroup per sequence: K and V rows copied (16-byte pieces), the k^I row quantised.
template <class TI>
__global__ __launch_bounds__(kQuantThreads) void cache_append_kernel(
    const uint8_t* __restrict__ k_new, const uint8_t* __restrict__ v_new, int kv_row_bytes,
    const TI* __restrict__ kidx_new, int dI, const int32_t* __restrict__ positions,
    const int32_t* __restrict__ block_table, int num_blocks, int max_blocks, int block_size,
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache, uint8_t* __restrict__ kidx_cache,
    float* __restrict__ kidx_scale)
{
    __shared__ float red[kQuantThreads / 64];
    const int b = blockIdx.x, tid = threadIdx.x;
    const int64_t pos = positions[b];
    if (pos < 0 || pos >= (int64_t)max_blocks * block_size) return;      // uniform
    const int blk = block_table[(int64_t)b * max_blocks + pos / block_size];
    if (blk < 0 || blk >= num_blocks) return;                            // uniform
    const int64_t slot = (int64_t)blk * block_size + pos % block_size;
    const int n16 = kv_row_bytes / 16;
    for (int i = tid; i < n16; i += kQuantThreads) {
        reinterpret_cast<v4i*>(k_cache + slot * kv_row_bytes)[i] =
            reinterpret_cast<const v4i*>(k_new + (int64_t)b * kv_row_bytes)[i];
        reinterpret_cast<v4i*>(v_cache + slot * kv_row_bytes)[i] =
            reinterpret_cast<const v4i*>(v_new + (int64_t)b * kv_row_bytes)[i];
    }
    quantize_row(kidx_new, (int64_t)b, dI, kidx_cache + slot * dI, kidx_scale + slot, red);
}

}  // namespace

hipError_t launch_quantize_e4m3(const void* x, int x_bf16, int T, int n, uint8_t* codes,
                                float* scale, hipStream_t stream)
{
    if (T == 0) return hipSuccess;
    const int per = x_bf16 ? 8 : 4;                   // values per 16-byte piece
    const bool vec = n % per == 0 && n / per <= kQuantThreads * kVecLoads &&
                     (reinterpret_cast<uintptr_t>(x) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(codes) & 15) == 0;
    if (x_bf16) {
        const auto* xb = static_cast<const uint16_t*>(x);
        if (vec) hipLaunchKernelGGL((quantize_e4m3_kernel<uint16_t, true>), dim3(T), dim3(kQuantThreads), 0, stream, xb, n, codes, scale);
        else hipLaunchKernelGGL((quantize_e4m3_kernel<uint16_t, false>), dim3(T), dim3(kQuantThreads), 0, stream, xb, n, codes, scale);
    } else {
        const auto* xf = static_cast<const float*>(x);
        if (vec) hipLaunchKernelGGL((quantize_e4m3_kernel<float, true>), dim3(T), dim3(kQuantThreads), 0, stream, xf, n, codes, scale);
        else hipLaunchKernelGGL((quantize_e4m3_kernel<float, false>), dim3(T), dim3(kQuantThreads), 0, stream, xf, n, codes, scale);
    }
    return hipGetLastError();
}

hipError_t launch_cache_append(const void* k_new, const void* v_new, int kv_row_bytes,
                               const void* kidx_new, int kidx_bf16, int dI,
                               const int32_t* positions, const int32_t* block_table, int B,
                               int num_blocks, int max_blocks, int block_size, void* k_cache,
                               void* v_cache, uint8_t* kidx_cache, float* kidx_scale,
                               hipStream_t stream)
{
    if (B == 0) return hipSuccess;
    const auto* kn = static_cast<const uint8_t*>(k_new);
    const auto* vn = static_cast<const uint8_t*>(v_new);
    auto* kc = static_cast<uint8_t*>(k_cache);
    auto* vc = static_cast<uint8_t*>(v_cache);
    if (kidx_bf16)
        hipLaunchKernelGGL(cache_append_kernel<uint16_t>, dim3(B), dim3(kQuantThreads), 0, stream, kn,
                           vn, kv_row_bytes, static_cast<const uint16_t*>(kidx_new), dI, positions,
                           block_table, num_blocks, max_blocks, block_size, kc, vc, kidx_cache,
                           kidx_scale);
    else
        hipLaunchKernelGGL(cache_append_kernel<float>, dim3(B), dim3(kQuantThreads), 0, stream, kn,
                           vn, kv_row_bytes, static_cast<const float*>(kidx_new), dI, positions,
                           block_table, num_blocks, max_blocks, block_size, kc, vc, kidx_cache,
                           kidx_scale);
    return hipGetLastError();
}

}  // namespace dsa
