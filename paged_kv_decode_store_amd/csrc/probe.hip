// Measurement helpers: the streaming-read rate the device sustains with the
// loads the attention kernels use (16-byte non-temporal vector loads), as a
// ceiling to hold the partial kernels' rates against, and the device's
// properties.  Neither touches the decode path.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "launch.hpp"

namespace pkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;   // loads in flight per thread per step

// Grid-stride read of n16 16-byte words; the xor of everything read is
// compared with a value it practically never equals, so that the loads stay
// (the store behind the comparison is a plain vector store).
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const u32x4 *src, size_t n16,
                                                                    uint32_t *sink)
{
    const size_t stride = (size_t)gridDim.x * kProbeThreads;
    size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
        u32x4 w[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) w[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= w[u];
    }
    for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(src + i);
    const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (x == 0x9e3779b9u && threadIdx.x == 0) sink[blockIdx.x & 63u] = x;
}

}  // namespace

hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, int32_t workgroups,
                              hipStream_t stream)
{
    const size_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    stream_read_kernel<<<(unsigned)workgroups, kProbeThreads, 0, stream>>>(
        static_cast<const u32x4 *>(buf), n16, sink);
    return hipGetLastError();
}

}  // namespace pkv
