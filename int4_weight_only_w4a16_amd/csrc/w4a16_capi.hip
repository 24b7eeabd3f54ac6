// C ABI of the gfx950 W4A16 linear: argument validation, kernel dispatch and
// host-side GPTQ_V2 packing.  See include/w4a16.h for the contract.
//
// Fail-closed validation follows the pages: "Why GPTQ-Pro" (fail-closed
// support, a validated shape fallback), "Runtime contract" (group sizes,
// K % 16, N % 8), and "Installation and Quickstart", "Troubleshooting and edge
// cases" (a kernel checks bits, group size, dtype, dimensions and device
// together; packed tensors must match their metadata).  Every check runs
// before any HIP call, so an invalid call launches nothing.

#include <atomic>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>
#include <utility>

#include "../../include/w4a16.h"
#include "w4a16_launch.h"

namespace {

constexpr int64_t kMaxBufferBytes = (int64_t)1 << 31;   // buffer range checks are 32-bit

bool group_ok(int64_t g) {
    switch (g) {
        case -1: case 16: case 32: case 64: case 128: case 256: case 512: case 1024:
            return true;
        default:
            return false;
    }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int validate(const void *x, const int32_t *qweight, const void *scales, void *y, int64_t M,
             int64_t K, int64_t N, int64_t g) {
    if (M < 0 || K <= 0 || N <= 0 || K % 16 != 0 || N % 8 != 0) return W4A16_ERR_SHAPE;
    if (M >= kMaxBufferBytes || K >= kMaxBufferBytes || N >= kMaxBufferBytes)
        return W4A16_ERR_SHAPE;
    if (!group_ok(g)) return W4A16_ERR_GROUP;
    const int64_t G = g == -1 ? 1 : (K + g - 1) / g;
    // each factor < 2^31, so every product below fits in int64
    if (2 * M * K >= kMaxBufferBytes || (K / 2) * N >= kMaxBufferBytes ||
        2 * G * N >= kMaxBufferBytes || 2 * M * N >= kMaxBufferBytes)
        return W4A16_ERR_SHAPE;
    if (M == 0) return W4A16_OK;
    if (!x || !qweight || !scales || !y) return W4A16_ERR_NULL;
    if (!aligned16(x) || !aligned16(qweight) || !aligned16(scales) || !aligned16(y))
        return W4A16_ERR_ALIGN;
    return W4A16_OK;
}

// Per-device facts, queried once: is it a gfx950, and its CU count.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch[kMaxDevices];      // 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_cus[kMaxDevices];
std::atomic<size_t> g_lds[kMaxDevices];    // LDS bytes per workgroup

// Current device if it is a gfx950 (with its CU count and LDS limit), else -1.
int usable_device(int *num_cus, size_t *max_lds) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
    int state = g_arch[dev].load(std::memory_order_acquire);
    if (state == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return -1;
        state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_cus[dev].store(prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1,
                         std::memory_order_relaxed);
        g_lds[dev].store(prop.sharedMemPerBlock, std::memory_order_relaxed);
        g_arch[dev].store(state, std::memory_order_release);
    }
    *num_cus = g_cus[dev].load(std::memory_order_relaxed);
    *max_lds = g_lds[dev].load(std::memory_order_relaxed);
    return state == 1 ? dev : -1;
}

// Kernel workspaces, one per (device, stream, kind): calls on one stream run
// in stream order and calls on different streams use different workspaces,
// so eager calls never share one concurrently (a graph captured on a stream
// keeps using that stream's workspace wherever it is replayed).  Created on
// the first call on a stream that needs it (not while the stream is being
// captured into a graph), zero-filled in stream order, kept until
// w4a16_stream_release or the end of the process.
//   kind 0: decode stream-K (exchange slots and partial tiles, 3 MiB, then
//           the one-launch LoRA term's exit count and slice words, 16.25 KiB)
//   kind 1: prefill split tail (one 256 x 256 fp32 partial per CU, 64 MiB)
std::mutex g_ws_mu;
std::map<std::tuple<int, uintptr_t, int>, std::pair<void *, size_t>> g_ws;

void *stream_workspace(int dev, hipStream_t stream, int kind, size_t bytes) {
    std::lock_guard<std::mutex> lock(g_ws_mu);
    const auto key = std::make_tuple(dev, reinterpret_cast<uintptr_t>(stream), kind);
    auto it = g_ws.find(key);
    if (it != g_ws.end() && it->second.second >= bytes) return it->second.first;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone)
        return nullptr;
    if (it != g_ws.end()) {                      // grow: the old one may still be in use
        if (hipStreamSynchronize(stream) != hipSuccess) return nullptr;
        (void)hipFree(it->second.first);
        g_ws.erase(it);
    }
    void *p = nullptr;
    if (hipMalloc(&p, bytes) != hipSuccess) return nullptr;
    if (hipMemsetAsync(p, 0, bytes, stream) != hipSuccess) {
        (void)hipFree(p);
        return nullptr;
    }
    g_ws[key] = std::make_pair(p, bytes);
    return p;
}

// Frees the workspaces held for (dev, stream) after the stream has finished
// the work queued on it.
int release_stream_workspaces(int dev, hipStream_t stream) {
    std::lock_guard<std::mutex> lock(g_ws_mu);
    const uintptr_t key = reinterpret_cast<uintptr_t>(stream);
    bool synced = false;
    for (auto it = g_ws.begin(); it != g_ws.end();) {
        if (std::get<0>(it->first) != dev || std::get<1>(it->first) != key) {
            ++it;
            continue;
        }
        if (!synced) {
            if (hipStreamSynchronize(stream) != hipSuccess) return W4A16_ERR_LAUNCH;
            synced = true;
        }
        (void)hipFree(it->second.first);
        it = g_ws.erase(it);
    }
    return W4A16_OK;
}

}  // namespace

extern "C" int w4a16_stream_release(void *stream) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return W4A16_ERR_DEVICE;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (hipStreamIsCapturing(s, &cap) != hipSuccess) return W4A16_ERR_DEVICE;
    if (cap != hipStreamCaptureStatusNone) return W4A16_ERR_CAPTURE;
    return release_stream_workspaces(dev, s);
}

// linear_call's answer when it leaves a LoRA term to the caller's other path.
constexpr int kNotTaken = -1;

// One linear call, fp16 or bfloat16 (bf16) activations and outputs; silu:
// the merged gate/up projection (N % 16 == 0, y is [M, N/2]); lora: the
// adapter term inside the stream-K decode launch, or kNotTaken (nothing
// launched) when that launch cannot take it.
static int linear_call(const void *x, const int32_t *qweight, const void *scales, void *y,
                       int64_t M, int64_t K, int64_t N, int64_t group_size, void *stream,
                       int kernel, bool bf16, bool silu = false,
                       const int32_t *qzeros = nullptr, bool scales_bf16 = false,
                       int zero_bias = 0, const w4a16::LoraTerm *lora = nullptr,
                       const w4a16::PrefillTerm *pterm = nullptr) {
    const int st = validate(x, qweight, scales, y, M, K, N, group_size);
    if (st != W4A16_OK) return st;
    if (silu && N % 16 != 0) return W4A16_ERR_SHAPE;
    if (kernel == W4A16_KERNEL_AUTO)
        kernel = M <= W4A16_DECODE_MAX_M ? W4A16_KERNEL_DECODE : W4A16_KERNEL_PREFILL;
    if (kernel == W4A16_KERNEL_DECODE) {
        if (M > W4A16_DECODE_MAX_M) return W4A16_ERR_KERNEL;
    } else if (kernel != W4A16_KERNEL_PREFILL) {
        return W4A16_ERR_KERNEL;
    }
    if (M == 0) return W4A16_OK;
    int num_cus = 0;
    size_t max_lds = 0;
    const int dev = usable_device(&num_cus, &max_lds);
    if (dev < 0) return W4A16_ERR_DEVICE;
    if (scales_bf16 && !bf16) return W4A16_ERR_FLAGS;   // not reached
    w4a16::LinearArgs a{x, qweight, scales, y, M, K, N, group_size, bf16, silu, qzeros,
                        scales_bf16, zero_bias};
    if (lora) {
        if (kernel != W4A16_KERNEL_DECODE) return W4A16_ERR_KERNEL;   // not reached
        a.lora = *lora;
    }
    if (pterm) {
        if (kernel != W4A16_KERNEL_PREFILL || silu) return W4A16_ERR_KERNEL;   // not reached
        a.pterm = *pterm;
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e;
    if (qzeros && kernel != W4A16_KERNEL_DECODE) return W4A16_ERR_KERNEL;   // not reached
    if (kernel == W4A16_KERNEL_DECODE) {
        int grid = w4a16::decode_streamk_grid(a, num_cus);
        void *ws = nullptr;
        if (grid > 0) {
            ws = stream_workspace(dev, s, 0, w4a16::decode_workspace_bytes(num_cus));
            if (!ws) grid = 0;                   // under capture with no workspace yet
        }
        // the adapter term needs the stream-K launch and its counters
        if (lora && (grid == 0 || !w4a16::decode_lora_inkernel_ok(a, num_cus))) return kNotTaken;
        e = w4a16::launch_decode(a, s, ws, num_cus, grid, max_lds);
    } else {
        void *ws = nullptr;
        if (w4a16::prefill_wants_workspace(a, num_cus))   // null under capture with none yet
            ws = stream_workspace(dev, s, 1, w4a16::prefill_workspace_bytes(num_cus));
        e = w4a16::launch_prefill(a, s, ws, num_cus, num_cus);
    }
    return e == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH;
}

// ---- the allocation-free variant: scratch in a file-scope device array ----
//
// For callers that cannot allocate (graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  The array holds the decode workspace
// laid out for up to kScratchMaxCus workgroups (exchange slots, zero at load
// time and left zero by every launch; partial tiles) and kScratchPrefillTiles
// prefill partial tiles.  In host code `scratch` names a host-side stand-in,
// never the device memory: its device address comes from hipGetSymbolAddress,
// once per device, and only that address reaches the kernels.
constexpr int kScratchMaxCus = 320;
constexpr int kScratchPrefillTiles = 64;
// (the decode part omits the LoRA term's counters: this entry point has no term)
constexpr size_t kScratchDecodeBytes = (size_t)kScratchMaxCus * w4a16::kDecodeWorkspacePerCu;
constexpr size_t kScratchBytes =
    kScratchDecodeBytes + (size_t)kScratchPrefillTiles * w4a16::kPrefillPartialTileBytes;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

static std::mutex g_scratch_mu;
static void *g_scratch_ptr[kMaxDevices];    // device address of `scratch`, per device

static void *scratch_address(int dev) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

extern "C" int w4a16_linear_noalloc(const void *x, const int32_t *qweight, const void *scales,
                                    void *y, int64_t M, int64_t K, int64_t N,
                                    int64_t group_size, void *stream) {
    const int st = validate(x, qweight, scales, y, M, K, N, group_size);
    if (st != W4A16_OK) return st;
    if (M == 0) return W4A16_OK;
    int num_cus = 0;
    size_t max_lds = 0;
    const int dev = usable_device(&num_cus, &max_lds);
    if (dev < 0) return W4A16_ERR_DEVICE;
    if (num_cus > kScratchMaxCus) return W4A16_ERR_SCRATCH;
    unsigned char *base = static_cast<unsigned char *>(scratch_address(dev));
    if (!base) return W4A16_ERR_DEVICE;
    const w4a16::LinearArgs a{x, qweight, scales, y, M, K, N, group_size, false, false};
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e;
    if (M <= W4A16_DECODE_MAX_M)
        e = w4a16::launch_decode(a, s, base, kScratchMaxCus, w4a16::decode_streamk_grid(a, num_cus),
                                 max_lds);
    else
        e = w4a16::launch_prefill(a, s, base + kScratchDecodeBytes, kScratchPrefillTiles, num_cus);
    return e == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH;
}

extern "C" int w4a16_linear_ex(const void *x, const int32_t *qweight, const void *scales,
                               void *y, int64_t M, int64_t K, int64_t N, int64_t group_size,
                               void *stream, int kernel) {
    return linear_call(x, qweight, scales, y, M, K, N, group_size, stream, kernel, false);
}

extern "C" int w4a16_linear(const void *x, const int32_t *qweight, const void *scales, void *y,
                            int64_t M, int64_t K, int64_t N, int64_t group_size,
                            void *stream) {
    return linear_call(x, qweight, scales, y, M, K, N, group_size, stream, W4A16_KERNEL_AUTO,
                       false);
}

extern "C" int w4a16_linear_bf16_ex(const void *x, const int32_t *qweight, const void *scales,
                                    void *y, int64_t M, int64_t K, int64_t N,
                                    int64_t group_size, void *stream, int kernel) {
    return linear_call(x, qweight, scales, y, M, K, N, group_size, stream, kernel, true);
}

extern "C" int w4a16_linear_bf16(const void *x, const int32_t *qweight, const void *scales,
                                 void *y, int64_t M, int64_t K, int64_t N, int64_t group_size,
                                 void *stream) {
    return linear_call(x, qweight, scales, y, M, K, N, group_size, stream, W4A16_KERNEL_AUTO,
                       true);
}

extern "C" int w4a16_gate_up_silu_ex(const void *x, const int32_t *qweight, const void *scales,
                                     void *y, int64_t M, int64_t K, int64_t N,
                                     int64_t group_size, void *stream, int kernel) {
    return linear_call(x, qweight, scales, y, M, K, N, group_size, stream, kernel, false, true);
}

extern "C" int w4a16_gate_up_silu(const void *x, const int32_t *qweight, const void *scales,
                                  void *y, int64_t M, int64_t K, int64_t N, int64_t group_size,
                                  void *stream) {
    return linear_call(x, qweight, scales, y, M, K, N, group_size, stream, W4A16_KERNEL_AUTO,
                       false, true);
}

extern "C" int w4a16_gate_up_silu_bf16_ex(const void *x, const int32_t *qweight,
                                          const void *scales, void *y, int64_t M, int64_t K,
                                          int64_t N, int64_t group_size, void *stream,
                                          int kernel) {
    return linear_call(x, qweight, scales, y, M, K, N, group_size, stream, kernel, true, true);
}

extern "C" int w4a16_gate_up_silu_bf16(const void *x, const int32_t *qweight,
                                       const void *scales, void *y, int64_t M, int64_t K,
                                       int64_t N, int64_t group_size, void *stream) {
    return linear_call(x, qweight, scales, y, M, K, N, group_size, stream, W4A16_KERNEL_AUTO,
                       true, true);
}

// The linear followed by the LoRA adapter term on the same stream.
static int lora_call(const void *x, const int32_t *qweight, const void *scales,
                     const void *lora_a, const void *lora_b, float lora_scale, void *y,
                     int64_t M, int64_t K, int64_t N, int64_t group_size, int64_t rank,
                     void *workspace, size_t workspace_bytes, void *stream, bool bf16) {
    int st = validate(x, qweight, scales, y, M, K, N, group_size);
    if (st != W4A16_OK) return st;
    if (rank < 8 || rank > W4A16_LORA_MAX_RANK || rank % 8 != 0) return W4A16_ERR_RANK;
    if (2 * rank * K >= kMaxBufferBytes || 2 * N * rank >= kMaxBufferBytes) return W4A16_ERR_SHAPE;
    const size_t need = w4a16::lora_workspace_bytes(M, K, rank);
    if (need >= (size_t)kMaxBufferBytes) return W4A16_ERR_SHAPE;
    if (M == 0) return W4A16_OK;
    if (!lora_a || !lora_b || !workspace) return W4A16_ERR_NULL;
    if (!aligned16(lora_a) || !aligned16(lora_b) || !aligned16(workspace)) return W4A16_ERR_ALIGN;
    if (workspace_bytes < need) return W4A16_ERR_WORKSPACE;
    const w4a16::LoraArgs a{x, lora_a, lora_b, y, M, K, N, rank, lora_scale, bf16};
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (M <= W4A16_DECODE_MAX_M && w4a16::lora_inkernel_bytes(M, K, rank) > 0) {
        // decode: the term inside the linear's stream-K launch, when it fits
        w4a16::LoraTerm term;
        term.A = lora_a;
        term.B = lora_b;
        term.tq = workspace;
        term.scale = lora_scale;
        term.r = (int)rank;
        term.Su = (int)(((K + 31) / 32 + w4a16::kLoraUnitSteps - 1) / w4a16::kLoraUnitSteps);
        st = linear_call(x, qweight, scales, y, M, K, N, group_size, stream, W4A16_KERNEL_DECODE,
                         bf16, false, nullptr, false, 0, &term);
        if (st != kNotTaken) return st;
    }
    if (M > W4A16_DECODE_MAX_M) {
        // prefill: the shrink and t', then the linear with the term in its epilogue
        w4a16::PrefillTerm term;
        int num_cus = 0;
        size_t max_lds = 0;
        if (usable_device(&num_cus, &max_lds) < 0) return W4A16_ERR_DEVICE;
        if (w4a16::launch_lora_t(a, s, workspace, &term) != hipSuccess) return W4A16_ERR_LAUNCH;
        return linear_call(x, qweight, scales, y, M, K, N, group_size, stream,
                           W4A16_KERNEL_PREFILL, bf16, false, nullptr, false, 0, nullptr, &term);
    }
    st = linear_call(x, qweight, scales, y, M, K, N, group_size, stream, W4A16_KERNEL_AUTO, bf16);
    if (st != W4A16_OK) return st;
    const hipError_t e = w4a16::launch_lora(a, s, workspace);
    return e == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH;
}

extern "C" size_t w4a16_lora_workspace_bytes(int64_t M, int64_t K, int64_t rank) {
    if (M <= 0 || K <= 0 || K % 16 != 0 || rank < 8 || rank > W4A16_LORA_MAX_RANK ||
        rank % 8 != 0 || M >= kMaxBufferBytes || K >= kMaxBufferBytes)
        return 0;
    return w4a16::lora_workspace_bytes(M, K, rank);
}

extern "C" int w4a16_linear_lora(const void *x, const int32_t *qweight, const void *scales,
                                 const void *lora_a, const void *lora_b, float lora_scale,
                                 void *y, int64_t M, int64_t K, int64_t N, int64_t group_size,
                                 int64_t rank, void *workspace, size_t workspace_bytes,
                                 void *stream) {
    return lora_call(x, qweight, scales, lora_a, lora_b, lora_scale, y, M, K, N, group_size, rank,
                     workspace, workspace_bytes, stream, false);
}

extern "C" int w4a16_linear_lora_bf16(const void *x, const int32_t *qweight, const void *scales,
                                      const void *lora_a, const void *lora_b, float lora_scale,
                                      void *y, int64_t M, int64_t K, int64_t N,
                                      int64_t group_size, int64_t rank, void *workspace,
                                      size_t workspace_bytes, void *stream) {
    return lora_call(x, qweight, scales, lora_a, lora_b, lora_scale, y, M, K, N, group_size, rank,
                     workspace, workspace_bytes, stream, true);
}

// The linear with stored zero points on the stream: for the decode kernel in
// one launch, else the symmetric linear followed by the correction.
// workspace_always: the workspace is required even where it is not used (the
// contract of w4a16_linear_zp).
static int zp_call(const void *x, const int32_t *qweight, const void *scales,
                   const int32_t *qzeros, void *y, int64_t M, int64_t K, int64_t N,
                   int64_t group_size, void *workspace, size_t workspace_bytes, void *stream,
                   bool bf16, bool scales_bf16 = false, int zero_bias = 0,
                   int kernel = W4A16_KERNEL_AUTO, bool workspace_always = true) {
    int st = validate(x, qweight, scales, y, M, K, N, group_size);
    if (st != W4A16_OK) return st;
    if ((w4a16::zp_groups(K, group_size) + 7) / 8 * 8 > w4a16::kZpMaxGroups) return W4A16_ERR_SHAPE;
    const size_t need = w4a16::zp_workspace_bytes(M, K, N, group_size);
    if (need >= (size_t)kMaxBufferBytes) return W4A16_ERR_SHAPE;
    if (kernel == W4A16_KERNEL_AUTO)
        kernel = M <= W4A16_DECODE_MAX_M ? W4A16_KERNEL_DECODE : W4A16_KERNEL_PREFILL;
    if (kernel == W4A16_KERNEL_DECODE) {
        if (M > W4A16_DECODE_MAX_M) return W4A16_ERR_KERNEL;
    } else if (kernel != W4A16_KERNEL_PREFILL) {
        return W4A16_ERR_KERNEL;
    }
    if (M == 0) return W4A16_OK;
    const bool fused = kernel == W4A16_KERNEL_DECODE;
    const bool ws_used = !fused || workspace_always;
    if (!qzeros || (ws_used && !workspace)) return W4A16_ERR_NULL;
    if (!aligned16(qzeros) || (ws_used && !aligned16(workspace))) return W4A16_ERR_ALIGN;
    if (ws_used && workspace_bytes < need) return W4A16_ERR_WORKSPACE;
    // decode: the zero points enter the linear's own kernel (one launch)
    if (fused)
        return linear_call(x, qweight, scales, y, M, K, N, group_size, stream,
                           W4A16_KERNEL_DECODE, bf16, false, qzeros, scales_bf16, zero_bias);
    // prefill: X and C^T, then the symmetric linear with X . C^T in its epilogue
    int num_cus = 0;
    size_t max_lds = 0;
    if (usable_device(&num_cus, &max_lds) < 0) return W4A16_ERR_DEVICE;
    const w4a16::ZpArgs a{x, scales, qzeros, y, M, K, N, group_size, bf16, scales_bf16, zero_bias};
    w4a16::PrefillTerm term;
    if (w4a16::launch_zp_t(a, reinterpret_cast<hipStream_t>(stream), workspace, &term) != hipSuccess)
        return W4A16_ERR_LAUNCH;
    return linear_call(x, qweight, scales, y, M, K, N, group_size, stream, W4A16_KERNEL_PREFILL,
                       bf16, false, nullptr, scales_bf16, 0, nullptr, &term);
}

extern "C" size_t w4a16_zp_workspace_bytes(int64_t M, int64_t K, int64_t N,
                                           int64_t group_size) {
    if (M <= 0 || K <= 0 || K % 16 != 0 || N <= 0 || N % 8 != 0 || !group_ok(group_size) ||
        M >= kMaxBufferBytes || K >= kMaxBufferBytes || N >= kMaxBufferBytes)
        return 0;
    if ((w4a16::zp_groups(K, group_size) + 7) / 8 * 8 > w4a16::kZpMaxGroups) return 0;
    return w4a16::zp_workspace_bytes(M, K, N, group_size);
}

extern "C" int w4a16_linear_zp(const void *x, const int32_t *qweight, const void *scales,
                               const int32_t *qzeros, void *y, int64_t M, int64_t K, int64_t N,
                               int64_t group_size, void *workspace, size_t workspace_bytes,
                               void *stream) {
    return zp_call(x, qweight, scales, qzeros, y, M, K, N, group_size, workspace,
                   workspace_bytes, stream, false);
}

extern "C" int w4a16_linear_zp_bf16(const void *x, const int32_t *qweight, const void *scales,
                                    const int32_t *qzeros, void *y, int64_t M, int64_t K,
                                    int64_t N, int64_t group_size, void *workspace,
                                    size_t workspace_bytes, void *stream) {
    return zp_call(x, qweight, scales, qzeros, y, M, K, N, group_size, workspace,
                   workspace_bytes, stream, true);
}

extern "C" int w4a16_linear_typed(const void *x, const int32_t *qweight, const void *scales,
                                  const int32_t *qzeros, void *y, int64_t M, int64_t K, int64_t N,
                                  int64_t group_size, unsigned flags, int kernel,
                                  void *workspace, size_t workspace_bytes, void *stream) {
    constexpr unsigned kKnown = W4A16_X_BF16 | W4A16_SCALES_BF16 | W4A16_ZEROS_V1 |
                                W4A16_GATE_UP_SILU;
    const bool bf16 = (flags & W4A16_X_BF16) != 0;
    const bool scales_bf16 = (flags & W4A16_SCALES_BF16) != 0;
    const bool v1 = (flags & W4A16_ZEROS_V1) != 0;
    const bool silu = (flags & W4A16_GATE_UP_SILU) != 0;
    if ((flags & ~kKnown) != 0 || (scales_bf16 && !bf16) || (v1 && !qzeros) || (silu && qzeros))
        return W4A16_ERR_FLAGS;
    if (!qzeros)
        return linear_call(x, qweight, scales, y, M, K, N, group_size, stream, kernel, bf16, silu,
                           nullptr, scales_bf16);
    return zp_call(x, qweight, scales, qzeros, y, M, K, N, group_size, workspace, workspace_bytes,
                   stream, bf16, scales_bf16, v1 ? 1 : 0, kernel, false);
}

extern "C" int pack_gptq_v2(const uint8_t *codes, int32_t *qweight, int64_t K, int64_t N) {
    if (K <= 0 || N <= 0 || K % 8 != 0) return W4A16_ERR_SHAPE;
    if (!codes || !qweight) return W4A16_ERR_NULL;
    uint8_t seen = 0;
    for (int64_t r = 0; r < K / 8; ++r) {
        uint32_t *dst = reinterpret_cast<uint32_t *>(qweight + r * N);
        const uint8_t *src = codes + 8 * r * N;
        for (int64_t n = 0; n < N; ++n) dst[n] = 0;
        for (int j = 0; j < 8; ++j) {
            const uint8_t *row = src + j * N;
            for (int64_t n = 0; n < N; ++n) {
                seen |= row[n];
                dst[n] |= (uint32_t)row[n] << (4 * j);
            }
        }
    }
    return (seen & 0xF0u) ? W4A16_ERR_CODE : W4A16_OK;
}

extern "C" int unpack_gptq_v2(const int32_t *qweight, uint8_t *codes, int64_t K, int64_t N) {
    if (K <= 0 || N <= 0 || K % 8 != 0) return W4A16_ERR_SHAPE;
    if (!codes || !qweight) return W4A16_ERR_NULL;
    for (int64_t r = 0; r < K / 8; ++r) {
        const uint32_t *src = reinterpret_cast<const uint32_t *>(qweight + r * N);
        for (int j = 0; j < 8; ++j) {
            uint8_t *row = codes + (8 * r + j) * N;
            for (int64_t n = 0; n < N; ++n) row[n] = (uint8_t)((src[n] >> (4 * j)) & 0xFu);
        }
    }
    return W4A16_OK;
}

extern "C" int w4a16_read_probe(const void *data, int64_t bytes, void *sink, void *stream) {
    if (bytes <= 0 || bytes % 16 != 0) return W4A16_ERR_SHAPE;
    if (!data || !sink) return W4A16_ERR_NULL;
    if (!aligned16(data) || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0) return W4A16_ERR_ALIGN;
    int num_cus = 0;
    size_t max_lds = 0;
    if (usable_device(&num_cus, &max_lds) < 0) return W4A16_ERR_DEVICE;
    const hipError_t e = w4a16::launch_read_probe(data, bytes, sink,
                                                  reinterpret_cast<hipStream_t>(stream), num_cus);
    return e == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH;
}

extern "C" const char *w4a16_status_string(int status) {
    switch (status) {
        case W4A16_OK: return "ok";
        case W4A16_ERR_NULL: return "null pointer";
        case W4A16_ERR_SHAPE: return "invalid shape (need M >= 0, K > 0, K % 16 == 0, N > 0, "
                                     "N % 8 == 0, every buffer < 2^31 bytes)";
        case W4A16_ERR_GROUP: return "group_size must be one of -1, 16, 32, 64, 128, 256, 512, 1024";
        case W4A16_ERR_ALIGN: return "device pointer not 16-byte aligned";
        case W4A16_ERR_CODE: return "code above 15";
        case W4A16_ERR_DEVICE: return "no usable gfx950 device";
        case W4A16_ERR_LAUNCH: return "kernel launch failed";
        case W4A16_ERR_KERNEL: return "requested kernel cannot take this M";
        case W4A16_ERR_RANK: return "LoRA rank must be a multiple of 8 in [8, 1024]";
        case W4A16_ERR_WORKSPACE: return "workspace smaller than the size its _workspace_bytes call gives";
        case W4A16_ERR_CAPTURE: return "stream is being captured into a graph";
        case W4A16_ERR_SCRATCH: return "device has more CUs than the allocation-free scratch covers";
        case W4A16_ERR_FLAGS: return "unknown flag bit, or flags that cannot go together (bfloat16 "
                                     "scales need bfloat16 x; v1 zero points need qzeros; gate/up "
                                     "takes no qzeros)";
        default: return "unknown status";
    }
}
