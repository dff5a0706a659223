// scratch.hip -- the library's static device scratch for callers that cannot allocate.
//
// One file-scope device array per GPU, created when the library's code object is loaded on that
// device and held until the process ends.  Its device address is read once per device, with that
// device current, when the first handle of the device is created (csf_create), and kept per
// device; host code only ever uses that address, never the array's own name (which on the host is
// a stand-in, not a device address).  Every call that uses the scratch on a GPU shares that GPU's
// array and finds the last call's contents in it.
#include <hip/hip_runtime.h>
#include <stddef.h>

#include <mutex>

#include "launch.hpp"

namespace csf {

namespace {

constexpr size_t kScratchBytes = size_t(8) << 20;   // 8 MiB
constexpr int kMaxScratchDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxScratchDevices] = {};

}  // namespace

size_t scratch_bytes() { return kScratchBytes; }

hipError_t scratch_init(int device)
{
    if (device < 0 || device >= kMaxScratchDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[device])
        return hipSuccess;
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess)
        return e;
    if (cur != device)
        return hipErrorInvalidDevice;     // the caller makes `device` current first
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess)
        return e;
    g_scratch_ptr[device] = p;
    return hipSuccess;
}

void *scratch_ptr(int device)
{
    if (device < 0 || device >= kMaxScratchDevices)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    return g_scratch_ptr[device];
}

}  // namespace csf
