// moe_scratch.hip -- device scratch of the allocation-free forward
// (moe_decode_forward_noalloc): a file-scope device array, one copy per GPU,
// zero when the library's code object is loaded and held until the process
// ends.  Host code never uses the array's name as an address (in host code it
// is only a stand-in for the device symbol): the device address of the
// current GPU's copy is looked up once per device with hipGetSymbolAddress and
// handed out from here.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe_args.h"

namespace moe {
namespace {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_for_current_device(void** ptr, size_t* bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // this device's copy
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    *bytes = kScratchBytes;
    return hipSuccess;
}

}  // namespace moe
