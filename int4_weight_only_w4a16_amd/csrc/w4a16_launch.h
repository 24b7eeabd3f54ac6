// Internal launch interface between the C ABI and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

// LoRA adapter term inside the stream-K decode launch (one kernel for the
// linear and the term): y = round(sum + delta), delta[m,n] = sum_j t'[m,j]
// B[n,j] in fp32 on the matrix cores, t' = round(scale * t) in the
// activation type, t = x . A^T summed in fp32 as Su partial slabs of
// kLoraUnitSteps 32-deep K steps each (one step per wave of a workgroup),
// added in slab order.  A null: no adapter term.
constexpr int kLoraUnitSteps = 8;        // one K step per wave of a workgroup
constexpr int kLoraMaxMR = 512;          // M * r at most
constexpr int kLoraMaxRank = 128;        // r at most (two 64-column passes per step)
constexpr int64_t kLoraMaxSlabReads = 4096;    // Su * M * r at most (16 KiB of LDS)
struct LoraTerm {
    const void *A = nullptr;     // [r, K] in the activation type
    const void *B = nullptr;     // [N, r] in the activation type
    void *tq = nullptr;          // t' [M][r] for the split reduce (caller's workspace)
    unsigned *area = nullptr;    // exit count, then the slab words (the decode workspace)
    float scale = 0.f;
    int r = 0, Su = 0;
};
// Bytes of the caller's workspace the term uses (t' for the split reduce), or
// 0 when (M, K, r) does not take this path.
size_t lora_inkernel_bytes(int64_t M, int64_t K, int64_t r);

// A low-rank term added in the prefill kernels' epilogue, before the one
// rounding of y (or into the first K chunk's fp32 partial of a split tile):
// y += ta . B^T, ta [M, r] and B [N, r] in the activation type (r % 8 == 0),
// on the matrix cores in fp32.  The LoRA adapter (ta = t' = round(s x . A^T))
// and the zero-point correction (ta = round(X), the group sums of x, and
// B = C^T = ((8 - z) s)^T) both take this form.  ta null: no term.
struct PrefillTerm {
    const void *ta = nullptr;
    const void *B = nullptr;
    int r = 0;
};

// Validated arguments of one linear call (shapes already checked against the
// contract, every buffer smaller than 2^31 bytes, M > 0).
struct LinearArgs {
    const void *x;
    const int32_t *qweight;
    const void *scales;
    void *y;
    int64_t M, K, N, group_size;
    bool bf16;   // x and y are bfloat16 (else fp16)
    bool silu;   // merged gate/up: columns alternate gate and up; y[M, N/2] = silu(gate) * up
    const int32_t *qzeros = nullptr;   // stored zero points int32 [G, N/8] (decode only), or none
    bool scales_bf16 = false;          // scales bfloat16 (requires bf16), else fp16
    int zero_bias = 0;                 // z = stored nibble + zero_bias: 0 (v2 form) or 1 (v1)
    LoraTerm lora{};                   // adapter term (stream-K decode only), or none
    PrefillTerm pterm{};               // low-rank term (prefill only), or none
};

// Decode (M <= 16).  grid > 0 runs the stream-K kernel on `grid` workgroups
// with `workspace`, a buffer of decode_workspace_bytes(capacity) bytes laid
// out for up to `capacity` workgroups (grid <= capacity), zero-filled before
// its first use and left zeroed by every launch; grid == 0 runs the tiles
// kernel, which needs no workspace.  max_lds is the device's LDS limit per
// workgroup in bytes.
constexpr size_t kDecodeWorkspacePerCu = 12 * 1024;   // exchange slots 4 KiB + partials 8 KiB
// the LoRA term's area: its exit count (256 bytes), then the slab words
constexpr size_t kDecodeLoraBytes = 256 + 4 * (size_t)kLoraMaxSlabReads;
size_t decode_workspace_bytes(int capacity);  // capacity * kDecodeWorkspacePerCu + LoRA area
int decode_streamk_grid(const LinearArgs &a, int num_cus);   // 0: use the tiles kernel
// Whether a.lora (filled but for its counters) can go inside the stream-K
// launch; launch_decode then takes it with grid = decode_streamk_grid and the
// workspace (whose counters it uses).
bool decode_lora_inkernel_ok(const LinearArgs &a, int num_cus);
hipError_t launch_decode(const LinearArgs &a, hipStream_t stream, void *workspace, int capacity,
                         int grid, size_t max_lds);

// Prefill (any M).  The 128-row kernel (M <= 128, and mid-sized M where it
// is priced cheaper) can split the K range into chunks, and the 256-row
// kernel a last partial round of tiles along K; either
// needs `workspace` (prefill_workspace_bytes(capacity) bytes of fp32
// partials, no initial contents) when prefill_wants_workspace(a, num_cus).
// A smaller capacity splits into fewer chunks; without a workspace every
// tile runs whole.
constexpr size_t kPrefillPartialTileBytes = 256 * 256 * 4;   // one 256 x 256 fp32 tile
size_t prefill_workspace_bytes(int capacity);                  // capacity partial tiles
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
// For the prefill: the shrink, then t' = round(s t) [M, r] into the
// workspace (after the partial sums), and the term for the prefill kernels.
hipError_t launch_lora_t(const LoraArgs &a, hipStream_t stream, void *workspace,
                         PrefillTerm *term);


// Stored zero points at prefill sizes: the correction sum_g X[m,g]
// (8 - z[g,n]) s[g,n] as a low-rank term of the prefill kernels, X the group
// sums of x (z = stored nibble + zero_bias).
// `workspace` holds zp_workspace_bytes(M, K, N, group_size) bytes (X, then
// C^T, both in the activation type), no initial contents; G rounded up to 8
// is at most kZpMaxGroups.
constexpr int kZpMaxGroups = 1536;
struct ZpArgs {
    const void *x, *scales;
    const int32_t *qzeros;
    void *y;
    int64_t M, K, N, group_size;
    bool bf16;
    bool scales_bf16;   // scales bfloat16, else fp16
    int zero_bias;      // z = stored nibble + zero_bias (0 or 1)
};
int zp_groups(int64_t K, int64_t group_size);
size_t zp_workspace_bytes(int64_t M, int64_t K, int64_t N, int64_t group_size);
// X rounded to the activation type [M, Gp] and C^T [N, Gp] into the
// workspace (no y yet), and the term for the prefill kernels (r = Gp).
hipError_t launch_zp_t(const ZpArgs &a, hipStream_t stream, void *workspace, PrefillTerm *term);

// Streaming-read probe over `bytes` (a multiple of 16) at data.
hipError_t launch_read_probe(const void *data, int64_t bytes, void *sink, hipStream_t stream,
                             int num_cus);

}  // namespace w4a16
