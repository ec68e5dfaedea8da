// Self-test of the CDNA4 transposed LDS read (ds_read_b64_tr_b16) lane map
// that the MFMA kernels rely on: one wave fills a 16 x 64 K-outer tile with
// codes (row << 8 | column), reads one 32x32x16 operand fragment with
// tr_frag, exactly as the kernels address it, and writes each lane's eight
// 16-bit results. The map the kernels assume: lane l receives rows
// 8*(l/32) .. 8*(l/32)+7 of column l % 32.
#include <hip/hip_runtime.h>

#include "device_common.hpp"

namespace wgrad {
namespace {

using namespace dev;

__global__ __launch_bounds__(64) void tr_probe_kernel(uint16_t* out) {
    constexpr int kPitch = 64;
    __shared__ __attribute__((aligned(16))) uint16_t tile[16 * kPitch];
    const int lane = threadIdx.x;
    for (int i = lane; i < 16 * kPitch; i += 64) tile[i] = (uint16_t)(((i / kPitch) << 8) | (i % kPitch));
    __syncthreads();
    // the fragment addressing of the MFMA kernels: rows frow and frow + 4,
    // columns fcol .. fcol + 3
    const int g16 = lane >> 4;
    const int frow = (g16 >> 1) * 8 + ((lane & 15) >> 2);
    const int fcol = (g16 & 1) * 16 + (lane & 3) * 4;
    const i16x8 f = tr_frag(tile + frow * kPitch + fcol, kPitch);
#pragma unroll
    for (int e = 0; e < 8; ++e) out[lane * 8 + e] = (uint16_t)f[e];
}

}  // namespace

int launch_tr_probe(uint16_t* out, void* stream) {
    hipLaunchKernelGGL(tr_probe_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), out);
    return (int)hipGetLastError();
}

}  // namespace wgrad
