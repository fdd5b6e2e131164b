// scratch.hip -- the static staging buffer of dt_bucket_allreduce_noalloc.
//
// That entry point stages its buckets (flatten -> AllReduce -> unflatten) in
// a file-scope device array instead of a caller workspace, so it allocates
// nothing.  The array lives in a translation unit of its own, with no
// kernels: the runtime loads it onto a device (and reserves its memory there
// until the process ends) only when scratch_base is first called with that
// device current, not when the library's kernels run.
//
// In host code the name `scratch` stands for a host-side shadow, not the
// device address, so it is never passed to a kernel or a copy: scratch_base
// asks the runtime for the device address once per device and hands that
// out.
#include <mutex>

#include "dt_launch.h"

namespace dt {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
}  // namespace

hipError_t scratch_base(void** ptr) {
    static std::mutex mu;
    static void* base[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (base[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        base[dev] = p;
    }
    *ptr = base[dev];
    return hipSuccess;
}

}  // namespace dt
