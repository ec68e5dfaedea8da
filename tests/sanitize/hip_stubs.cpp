// Stand-ins for the kernel launchers and the two HIP runtime calls the host
// planner and C ABI make, so that plan.cpp and abi.cpp can be built on the
// CPU with AddressSanitizer and UndefinedBehaviorSanitizer and driven without
// a GPU. Every launcher reports hipErrorNoDevice; nothing here touches
// device memory or the HIP runtime.
#include <hip/hip_runtime_api.h>

#include <cstdio>

#include "../../grouped_convolution_backward_amd/csrc/wgrad_internal.hpp"

namespace {
int g_launches = 0;
int no_device() {
    ++g_launches;
    return (int)hipErrorNoDevice;
}
}  // namespace

int stub_launch_count() { return g_launches; }

namespace wgrad {
int launch_mfma(const Plan&, const MfmaArgs&, void*) { return no_device(); }
int launch_depthwise(const Plan&, const DwArgs&, void*) { return no_device(); }
int launch_rowslab(const Plan&, const RowSlabArgs&, void*) { return no_device(); }
int launch_ring(const Plan&, const RingArgs&, void*) { return no_device(); }
int launch_depthwise2(const Plan&, const Dw2Args&, void*) { return no_device(); }
int launch_depthwise3(const Plan&, const Dw3Args&, void*) { return no_device(); }
int launch_dwtile(const Plan&, const DwTileArgs&, void*) { return no_device(); }
int launch_reduce(const ReduceArgs&, int64_t, void*) { return no_device(); }
int launch_dgrad(const Plan&, const DgradArgs&, void*) { return no_device(); }
int launch_dgrad_dw(const Plan&, const DgradDwArgs&, void*) { return no_device(); }
int launch_dgrad_dwtile(const Plan&, const DgradDwTileArgs&, void*) { return no_device(); }
int launch_dgrad_ring(const Plan&, const DgradRingArgs&, void*) { return no_device(); }
int scratch_workspace(void*, void**, size_t*) { return (int)hipErrorNoDevice; }
int launch_tr_probe(uint16_t*, void*) { return no_device(); }
}  // namespace wgrad

extern "C" const char* hipGetErrorString(hipError_t e) {
    return e == hipErrorNoDevice ? "no device (sanitizer build stub)" : "error (sanitizer build stub)";
}

extern "C" hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_t*, int) { return hipErrorNoDevice; }
