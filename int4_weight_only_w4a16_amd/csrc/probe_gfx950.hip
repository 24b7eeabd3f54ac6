// Streaming-read probe for gfx950: the attainable HBM read rate, measured
// with a plain kernel of our own, against which the decode kernel (a pure
// weight stream) is compared next to the 8 TB/s data-sheet peak.
//
// Every thread of a grid of 128 workgroups per CU reads 16-byte words at a
// grid stride with non-temporal loads, four in flight per step, and folds
// them with XOR; the folded value is stored only when it equals a fixed
// constant, so the loads cannot be dropped and the probe writes (almost)
// nothing.  (Of the shapes tried, 4..128 workgroups per CU, 4..16 loads in
// flight, plain or non-temporal loads, this one reads fastest.)

#include <stdint.h>

#include "w4a16_launch.h"

namespace w4a16 {

constexpr uint32_t kProbeKey = 0x9E3779B9u;
constexpr int kProbeGroupsPerCu = 128;

typedef unsigned int probe_u4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void read_probe_kernel(const probe_u4 *__restrict__ p,
                                                         int64_t n, uint32_t *__restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const probe_u4 a = __builtin_nontemporal_load(p + i);
        const probe_u4 b = __builtin_nontemporal_load(p + i + stride);
        const probe_u4 c = __builtin_nontemporal_load(p + i + 2 * stride);
        const probe_u4 d = __builtin_nontemporal_load(p + i + 3 * stride);
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w;
        acc ^= c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n; i += stride) {
        const probe_u4 a = __builtin_nontemporal_load(p + i);
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == kProbeKey) sink[0] = acc;
}

hipError_t launch_read_probe(const void *data, int64_t bytes, void *sink, hipStream_t stream,
                             int num_cus) {
    const probe_u4 *p = static_cast<const probe_u4 *>(data);
    int64_t n = bytes / 16;
    uint32_t *s = static_cast<uint32_t *>(sink);
    void *args[] = {&p, &n, &s};
    return hipLaunchKernel(reinterpret_cast<const void *>(&read_probe_kernel),
                           dim3(kProbeGroupsPerCu * (num_cus > 0 ? num_cus : 1)), dim3(256),
                           args, 0, stream);
}

}  // namespace w4a16
