// The library's own device scratch: one file-scope array per device, for the
// entry point that allocates nothing (paged_attn_decode_noalloc).
//
// The array lives in this code object's global data, so every device the
// library runs on holds its own copy for as long as the process lives.  In
// host code its name is only a stand-in for the symbol, never a device
// address: the address is asked of the runtime once per device (with that
// device current) and kept, and only that address reaches kernels and
// copies.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pkv_internal.h"

namespace pkv {
namespace {

__device__ __align__(256) char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device, once known
std::mutex g_scratch_mu;

}  // namespace

int noalloc_scratch(void** ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return PKV_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return PKV_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return PKV_ERR_HIP;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    return PKV_OK;
}

}  // namespace pkv
