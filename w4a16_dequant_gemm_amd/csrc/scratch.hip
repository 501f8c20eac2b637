// The library's static device scratch: one fixed-size buffer per GPU, for the entry point that
// allocates nothing (w4a16_linear_ws_noalloc).
//
// The buffer is a file-scope __device__ array, so every GPU the library runs on holds its own
// copy, at its own address, until the process ends.  In host code the array's name is only a
// stand-in for the device symbol: its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is handed to kernels.
// Every call on one GPU shares that GPU's buffer; calls that overlap on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

namespace w4a16 {

namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices] = {};
hipError_t g_err[kMaxDevices] = {};

}  // namespace

hipError_t scratch_device_ptr(float** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_once[dev], [dev] {
        void* p = nullptr;
        g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
    });
    if (g_err[dev] != hipSuccess) return g_err[dev];
    *out = static_cast<float*>(g_ptr[dev]);
    return hipSuccess;
}

}  // namespace w4a16
