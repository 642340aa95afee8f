// moe_forward_noalloc (include/moe.h): the whole layer with its scratch in a
// fixed device array of this library instead of a caller workspace, for
// callers that cannot allocate device memory.
//
// The array lives in this file's code object.  Host code never uses its
// name as an address: on a device's first call, with that device current,
// hipGetSymbolAddress resolves the device's own copy once, and every launch
// takes that pointer (kept per device) as the workspace of moe_forward.
// Nothing here allocates; the kernels are moe_forward's own, and they do not
// rely on the scratch starting out zero (every word they read is written
// earlier in the same call).
#include <hip/hip_runtime.h>

#include <cstddef>
#include <mutex>

#include "../../include/moe.h"

namespace {

constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

void* g_scratch[kMaxDevices];
hipError_t g_status[kMaxDevices];
std::once_flag g_once[kMaxDevices];

// This device's copy of `scratch` (resolved once per device), or NULL.
void* device_scratch(int dev) {
    std::call_once(g_once[dev], [dev] {
        void* p = nullptr;
        g_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch[dev] = g_status[dev] == hipSuccess ? p : nullptr;
    });
    return g_scratch[dev];
}

}  // namespace

extern "C" moe_status moe_forward_noalloc(const moe_layer_desc* desc, const void* x, const float* W_r,
                                          const float* b, const moe_expert_weights* weights, void* out,
                                          int32_t* topk_idx, float* topk_w, int32_t* expert_counts,
                                          int32_t* expert_offsets, int32_t* sorted_token, void* stream) {
    if (!desc) return MOE_ERR_NULL;
    const size_t need = moe_workspace_size(desc, 1);
    if (need == 0)  // an invalid descriptor: moe_forward reports which check failed
        return moe_forward(desc, x, W_r, b, weights, out, topk_idx, topk_w, expert_counts, expert_offsets,
                           sorted_token, nullptr, 0, stream, nullptr);
    if (need > kScratchBytes) return MOE_ERR_SCRATCH;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    void* ws = device_scratch(dev);
    if (!ws) return MOE_ERR_HIP;
    return moe_forward(desc, x, W_r, b, weights, out, topk_idx, topk_w, expert_counts, expert_offsets,
                       sorted_token, ws, kScratchBytes, stream, nullptr);
}
