// Static device scratch of the allocation-free forward entry point
// (tri_attn_fwd_rows_noalloc in tri_attn_api.cpp).
//
// The array below is the workspace of that entry point: every GPU the library runs on holds
// its own copy, kScratchBytes long, from the loading of the library's code until the process
// ends.  In host code `scratch` names a host-side stand-in, not device memory, so its
// device address is looked up once per device with hipGetSymbolAddress (with that device
// current) and only that address is handed to kernels.  All calls on one device share the
// array and leave their contents in it: each call's prepass writes everything the call
// later reads (fp16 image, references, span flags, split states), and two calls that
// overlap in time on one device race on it.
#include "launch.h"

#include <mutex>

namespace tri_attn {
namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // 64 MiB
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

size_t static_scratch_bytes() { return kScratchBytes; }

hipError_t static_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_addr[dev] = p;
    }
    *out = g_addr[dev];
    return hipSuccess;
}

}  // namespace tri_attn
