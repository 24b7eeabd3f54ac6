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
    bool bf16;   // x and y are bfloat16 (else fp16); scales are fp16 either way
    bool silu;   // merged gate/up: columns alternate gate and up; y[M, N/2] = silu(gate) * up
};

// Decode (M <= 16).  grid > 0 runs the stream-K kernel on `grid` workgroups
// with `workspace`, a buffer of decode_workspace_bytes(capacity) bytes laid
// out for up to `capacity` workgroups (grid <= capacity), zero-filled before
// its first use and left zeroed by every launch; grid == 0 runs the tiles
// kernel, which needs no workspace.  max_lds is the device's LDS limit per
// workgroup in bytes.
size_t decode_workspace_bytes(int capacity);
int decode_streamk_grid(const LinearArgs &a, int num_cus);   // 0: use the tiles kernel
hipError_t launch_decode(const LinearArgs &a, hipStream_t stream, void *workspace, int capacity,
                         int grid, size_t max_lds);

// Prefill (any M).  For M <= 128 the K range can be split into chunks, and
// for M > 128 a last partial round of tiles can be split along K; either
// needs `workspace` (prefill_workspace_bytes(capacity) bytes of fp32
// partials, no initial contents) when prefill_wants_workspace(a, num_cus).
// Without it (or with too small a capacity) every tile runs whole.
size_t prefill_workspace_bytes(int capacity);
bool prefill_wants_workspace(const LinearArgs &a, int num_cus);
hipError_t launch_prefill(const LinearArgs &a, hipStream_t stream, void *workspace, int capacity,
                          int num_cus);

// LoRA adapter term, added to a y the linear has already written:
// y = round(y + scale * (x . A^T) . B^T), A [r, K] and B [N, r] in the
// activation type (r % 8 == 0).  `workspace` holds lora_workspace_bytes(M, K,
// r) bytes of fp32 partial sums of x . A^T, no initial contents.
struct LoraArgs {
    const void *x, *A, *B;
    void *y;
    int64_t M, K, N, r;
    float scale;
    bool bf16;
};
size_t lora_workspace_bytes(int64_t M, int64_t K, int64_t r);
hipError_t launch_lora(const LoraArgs &a, hipStream_t stream, void *workspace);

// Stored zero points: y (the symmetric linear, already written) += the
// rank-G correction sum_g X[m,g] (8 - z[g,n]) s[g,n], X the group sums of x.
// `workspace` holds zp_workspace_bytes(M, K, N, group_size) bytes (X in fp32,
// then C^T in the activation type), no initial contents; G rounded up to 8 is
// at most kZpMaxGroups.
constexpr int kZpMaxGroups = 1536;
struct ZpArgs {
    const void *x, *scales;
    const int32_t *qzeros;
    void *y;
    int64_t M, K, N, group_size;
    bool bf16;
};
int zp_groups(int64_t K, int64_t group_size);
size_t zp_workspace_bytes(int64_t M, int64_t K, int64_t N, int64_t group_size);
hipError_t launch_zp(const ZpArgs &a, hipStream_t stream, void *workspace);

// Streaming-read probe over `bytes` (a multiple of 16) at data.
hipError_t launch_read_probe(const void *data, int64_t bytes, void *sink, hipStream_t stream,
                             int num_cus);

}  // namespace w4a16
