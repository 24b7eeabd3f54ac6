// Streaming-read probe for gfx950: the attainable HBM read rate, measured
// with a plain kernel of our own, against which the decode kernel (a pure
// weight stream) is compared next to the 8 TB/s data-sheet peak.
//
// Every thread of a grid of 8 workgroups per CU reads 16-byte words at a
// grid stride, four loads in flight per step, and folds them with XOR; the
// folded value is stored only when it equals a fixed constant, so the loads
// cannot be dropped and the probe writes (almost) nothing.

#include <stdint.h>

#include "w4a16_launch.h"

namespace w4a16 {

constexpr uint32_t kProbeKey = 0x9E3779B9u;

__global__ __launch_bounds__(256) void read_probe_kernel(const uint4 *__restrict__ p, int64_t n,
                                                         uint32_t *__restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w;
        acc ^= c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n; i += stride) {
        const uint4 a = p[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == kProbeKey) sink[0] = acc;
}

hipError_t launch_read_probe(const void *data, int64_t bytes, void *sink, hipStream_t stream,
                             int num_cus) {
    const uint4 *p = static_cast<const uint4 *>(data);
    int64_t n = bytes / 16;
    uint32_t *s = static_cast<uint32_t *>(sink);
    void *args[] = {&p, &n, &s};
    return hipLaunchKernel(reinterpret_cast<const void *>(&read_probe_kernel),
                           dim3(8 * (num_cus > 0 ? num_cus : 1)), dim3(256), args, 0, stream);
}

}  // namespace w4a16
