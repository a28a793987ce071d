// Streaming-read calibration kernel (pa_bench_stream_read in include/pa_bench.h).
//
// Every thread walks the buffer in a grid-stride loop of 16-byte
// non-temporal loads, eight in flight per iteration, and folds what it
// reads with XOR.  One 256-thread workgroup per compute unit is the default:
// on MI355X that shape reads fastest (more concurrent waves lower the rate).

#include <cstdint>

#include "pa_bench.h"
#include "pa_device.h"

namespace pa {

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ buf, int64_t nvec,
                                                          uint32_t* __restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + 7 * stride < nvec; i += 8 * stride) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = ld16_stream(&buf[i + u * stride]);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= v[u];
    }
    for (; i < nvec; i += stride) acc ^= buf[i];
    const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (x == 0x9e3779b9u) sink[0] = x;
}

}  // namespace pa

extern "C" pa_status pa_bench_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t workgroups,
                                          void* stream) {
    if (!buf || !sink || (reinterpret_cast<uintptr_t>(buf) & 15u) || (bytes % 16) || workgroups < 0)
        return PA_ERR_INVALID_ARG;
    if (bytes == 0) return PA_OK;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    const int64_t nvec = (int64_t)(bytes / 16);
    int64_t wg = workgroups ? workgroups : (int64_t)cus;
    const int64_t need = (nvec + 255) / 256;
    if (wg > need) wg = need;
    hipLaunchKernelGGL(pa::stream_read_kernel, dim3((unsigned)wg), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                       reinterpret_cast<const pa::u32x4*>(buf), nvec, sink);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}
