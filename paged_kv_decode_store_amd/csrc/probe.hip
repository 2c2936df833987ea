// Measurement helper: the streaming-read rate the device sustains with the
// loads the attention kernels use (16-byte non-temporal vector loads), each
// workgroup over a contiguous share of the buffer, as a ceiling to hold the
// partial kernels' rates against.  It does not touch the decode path.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "launch.hpp"

namespace pkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;   // loads in flight per thread per step

// Each workgroup reads its own contiguous share of the n16 16-byte words,
// kProbeUnroll loads in flight per thread (this streams faster on MI355X
// than a grid-stride sweep of the same bytes: ~7.0 against ~6.3 TB/s over
// 4 GiB).  The xor of everything read is compared with a value it
// practically never equals, so that the loads stay (the store behind the
// comparison is a plain vector store).
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const u32x4 *src, size_t n16,
                                                                    uint32_t *sink)
{
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t lo = (size_t)blockIdx.x * per;
    const size_t hi = lo + per < n16 ? lo + per : n16;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (size_t i = lo + threadIdx.x; i < hi; i += kProbeUnroll * kProbeThreads) {
        u32x4 w[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            const size_t j = i + (size_t)u * kProbeThreads;
            w[u] = j < hi ? __builtin_nontemporal_load(src + j) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= w[u];
    }
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
