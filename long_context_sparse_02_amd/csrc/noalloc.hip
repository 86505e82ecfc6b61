// noalloc.hip -- the paged decode step with the library's own device scratch, for callers
// that cannot allocate (code under HIP graph capture, serving loops, harnesses that forbid
// hipMalloc).
//
// The scratch is a file-scope device array: every GPU the library runs on holds its own
// copy (kNoAllocScratchBytes) until the process ends.  In host code the array's name is
// only a host-side stand-in, so its device address on each GPU is looked up once, with that
// GPU current, through hipGetSymbolAddress, and only that address is ever handed to the
// kernels.  Every call on one GPU shares that GPU's scratch: calls that overlap on one GPU
// (different streams, or host threads) race.  The decode step initialises everything it
// reads from its workspace within the call (counters and flags are reset by its own
// kernels), so nothing has to be cleared between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/dsa.h"
#include "internal.h"

#define DSA_EXPORT extern "C" __attribute__((visibility("default")))

static __device__ __align__(256) unsigned char scratch[dsa::kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current GPU's scratch (looked up on the first call on that GPU).
dsa_status_t scratch_for_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return dsa::api_fail(DSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return dsa::api_fail(DSA_ERR_UNSUPPORTED, "device %d beyond the %d this library tracks", dev,
                             kMaxDevices);
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return dsa::api_fail(DSA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                                 hipGetErrorString(e));
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return DSA_OK;
}

}  // namespace

DSA_EXPORT size_t dsa_decode_noalloc_max_workspace(void) { return dsa::kNoAllocScratchBytes; }

DSA_EXPORT dsa_status_t dsa_decode_noalloc(const void* q, const void* q_idx, const float* q_scale,
                                           const float* w, const void* kidx_cache,
                                           const float* kidx_scale, const void* k_cache,
                                           const void* v_cache, dsa_dtype_t dtype,
                                           const int32_t* block_table, const int32_t* seq_lens,
                                           int B, int num_blocks, int max_blocks, int block_size,
                                           int Hq, int G, int d, int HI, int dI, int topk,
                                           float sm_scale, void* out, int32_t* idx_out,
                                           hipStream_t stream) {
    const dsa_status_t st = dsa::decode_check_args(q, q_idx, q_scale, w, kidx_cache, kidx_scale,
                                                   k_cache, v_cache, dtype, block_table, seq_lens,
                                                   B, num_blocks, max_blocks, block_size, Hq, G,
                                                   d, HI, dI, topk, out, idx_out);
    if (st != DSA_OK || B == 0) return st;
    const size_t need = dsa_decode_workspace_size(B, max_blocks, block_size, topk, Hq, d);
    if (need > dsa::kNoAllocScratchBytes)
        return dsa::api_fail(DSA_ERR_WORKSPACE,
                             "dsa_decode_noalloc: this step needs %zu bytes of scratch, more than "
                             "the %zu the library holds per GPU; call dsa_decode with a workspace",
                             need, (size_t)dsa::kNoAllocScratchBytes);
    void* ws = nullptr;
    const dsa_status_t sst = scratch_for_current_device(&ws);
    if (sst != DSA_OK) return sst;
    return dsa_decode(q, q_idx, q_scale, w, kidx_cache, kidx_scale, k_cache, v_cache, dtype,
                      block_table, seq_lens, B, num_blocks, max_blocks, block_size, Hq, G, d, HI,
                      dI, topk, sm_scale, out, idx_out, ws, dsa::kNoAllocScratchBytes, stream);
}
