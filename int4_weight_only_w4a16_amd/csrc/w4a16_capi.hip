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

// Per-device answer to "is this a gfx950?" (0 unknown, 1 yes, 2 no).
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch[kMaxDevices];

bool device_ok() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return false;
    int state = dev < kMaxDevices ? g_arch[dev].load(std::memory_order_acquire) : 0;
    if (state == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return false;
        state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        if (dev < kMaxDevices) g_arch[dev].store(state, std::memory_order_release);
    }
    return state == 1;
}

}  // namespace

extern "C" int w4a16_linear_ex(const void *x, const int32_t *qweight, const void *scales,
                               void *y, int64_t M, int64_t K, int64_t N, int64_t group_size,
                               void *stream, int kernel) {
    const int st = validate(x, qweight, scales, y, M, K, N, group_size);
    if (st != W4A16_OK) return st;
    if (kernel == W4A16_KERNEL_AUTO)
        kernel = M <= W4A16_DECODE_MAX_M ? W4A16_KERNEL_DECODE : W4A16_KERNEL_PREFILL;
    if (kernel == W4A16_KERNEL_DECODE) {
        if (M > W4A16_DECODE_MAX_M) return W4A16_ERR_KERNEL;
    } else if (kernel != W4A16_KERNEL_PREFILL) {
        return W4A16_ERR_KERNEL;
    }
    if (M == 0) return W4A16_OK;
    if (!device_ok()) return W4A16_ERR_DEVICE;
    const w4a16::LinearArgs a{x, qweight, scales, y, M, K, N, group_size};
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const hipError_t e = kernel == W4A16_KERNEL_DECODE ? w4a16::launch_decode(a, s)
                                                       : w4a16::launch_prefill(a, s);
    return e == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH;
}

extern "C" int w4a16_linear(const void *x, const int32_t *qweight, const void *scales, void *y,
                            int64_t M, int64_t K, int64_t N, int64_t group_size,
                            void *stream) {
    return w4a16_linear_ex(x, qweight, scales, y, M, K, N, group_size, stream,
                           W4A16_KERNEL_AUTO);
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
        default: return "unknown status";
    }
}
