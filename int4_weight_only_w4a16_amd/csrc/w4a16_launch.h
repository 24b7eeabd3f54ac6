// Internal launch interface between the C ABI and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

// Validated arguments of one linear call (shapes already checked against the
// contract, every buffer smaller than 2^31 bytes, M > 0).
struct LinearArgs {
    const void *x;
    const int32_t *qweight;
    const void *scales;
    void *y;
    int64_t M, K, N, group_size;
};

hipError_t launch_decode(const LinearArgs &a, hipStream_t stream);   // M <= 16
hipError_t launch_prefill(const LinearArgs &a, hipStream_t stream);  // any M

}  // namespace w4a16
