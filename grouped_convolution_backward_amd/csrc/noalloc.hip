// Library-owned split-K workspace for wgrad_run_noalloc: a fixed-size device
// array that every call on a GPU shares, so that callers which cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc) can still run plans that split the
// reduction.
//
// The array is a file-scope __device__ variable: each GPU the library runs
// on holds its own copy, at its own address, from the code object's load
// until the process ends. In host code the name `scratch` is only a host-side
// stand-in for the symbol; the device address comes from hipGetSymbolAddress,
// resolved once per device with that device current and kept per device.
// Only that address is ever passed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "wgrad_internal.hpp"

namespace wgrad {
namespace {

static __device__ __align__(256) unsigned char scratch[WGRAD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

// Device address of this GPU's scratch array. device is the ordinal of the
// GPU the stream runs on. Returns a hipError_t value (0 = success).
int scratch_workspace(void* stream, void** ptr, size_t* bytes) {
    int dev = -1;
    hipError_t e;
    if (stream) {
        hipDevice_t d;
        e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &d);
        dev = (int)d;
    } else {
        e = hipGetDevice(&dev);
    }
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        int cur = -1;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return (int)e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return (int)e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t r = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess) return (int)e;
        if (r != hipSuccess) return (int)r;
        if (!p) return (int)hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    *bytes = WGRAD_NOALLOC_SCRATCH_BYTES;
    return (int)hipSuccess;
}

}  // namespace wgrad
