// scratch.hip - the library's built-in device workspace for attn_fwd_noalloc.
//
// One file-scope device array per GPU, kScratchBytes long, 256-byte aligned,
// held from the library's load until the process ends.  In host code the
// array's name stands for a host-side shadow, not a device address: the
// device address comes from hipGetSymbolAddress, asked once per device with
// that device current, and is kept here per device.  Every attn_fwd_noalloc
// call on a device shares that device's array (calls that overlap on one
// device race; the forward writes every workspace byte it reads, so nothing
// needs clearing between calls).
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/hcattn.h"
#include "kernels.h"

namespace hc {

static_assert(kScratchBytes == ATTN_NOALLOC_WORKSPACE_BYTES, "built-in workspace size");

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

hipError_t scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace hc
