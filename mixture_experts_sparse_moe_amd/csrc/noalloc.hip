// moe_forward for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc): the
// workspace is a file-scope device array of fixed size instead of a buffer
// the caller brings.  The layer itself is moe_forward, kernel for kernel.
//
// The array lives in the code object, so every GPU the library runs on holds
// its own copy, allocated when the module loads and kept until the process
// ends.  In host code the array's name is only a stand-in for the device
// symbol, never a device address: its address on a device comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// kept per device.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe.h"
#include "moe_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // MOE_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == MOE_NOALLOC_SCRATCH_BYTES, "the header states the size");
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

struct DeviceScratch {
    std::once_flag once;
    hipError_t err = hipSuccess;
    void* ptr = nullptr;
};
DeviceScratch g_scratch[kMaxDevices];

}  // namespace

extern "C" int moe_forward_noalloc(const moe_config* cfg, const void* x, const void* w_router,
                                   const void* w_gate, const void* w_up, const void* w_down,
                                   const void* ws_gate, const void* ws_up, const void* ws_down, void* y,
                                   int32_t* topk_ids_out, float* topk_weights_out,
                                   int32_t* expert_counts_out, float* topk_gap_out, void* stream) {
    const int rc = moe::validate_config(cfg);
    if (rc != MOE_OK) return rc;
    if (moe_workspace_bytes(cfg) > kScratchBytes) return MOE_ERR_WORKSPACE;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    DeviceScratch& d = g_scratch[dev];
    // first call on this device (which is current): the array's device address
    std::call_once(d.once, [&d] { d.err = hipGetSymbolAddress(&d.ptr, HIP_SYMBOL(scratch)); });
    if (d.err != hipSuccess || d.ptr == nullptr) return MOE_ERR_HIP;
    return moe_forward(cfg, x, w_router, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, y, topk_ids_out,
                       topk_weights_out, expert_counts_out, topk_gap_out, d.ptr, kScratchBytes, stream);
}
