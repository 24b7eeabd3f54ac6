// Prefill W4A16 GEMM for gfx950: any M, MFMA with fp32 accumulation.
//
// The pages' prefill path ("GPTQ-Pro" README, "Ampere kernel architecture",
// Tensor Core prefill) stages operands asynchronously, accumulates in FP32,
// handles tails and stores FP16 vectors.  The CDNA4 design:
//
//  * A workgroup of 4 waves owns a 128 (M) x 256 (N) output tile; wave w owns
//    the 128 x 64 slice of columns 64w .. 64w+63 (32 MFMA 16x16 tiles, 128
//    fp32 accumulators per lane).
//  * Activations go global -> registers -> LDS, 64 K per stage, two stages
//    (one barrier per stage).  Each 16-byte chunk is reordered on the way in
//    to the K order the nibble unpack produces, so MFMA A fragments are
//    plain ds_read_b128.
//  * Weights never touch LDS: one 128-bit load gives a lane four qweight
//    words, i.e. the 8-deep B fragments of four MFMA column sets.  They are
//    dequantised in registers to (q-8)*s in fp16 (one rounding) and each
//    fragment feeds 8 MFMAs (the 8 row tiles of the wave).  The next stage's
//    words and scales are in flight while the current stage computes.
//  * Tails: rows >= M and K >= K read as zero through buffer range checks;
//    stores are masked per row and per 4-column group (N % 8 == 0).

#include "w4a16_device.hpp"
#include "w4a16_launch.h"

namespace w4a16 {

constexpr int kPreBM = 128;               // rows per workgroup tile
constexpr int kPreBN = 256;               // columns per workgroup tile
constexpr int kPreBK = 64;                // K per LDS stage
constexpr int kPreRowBytes = 144;         // 128 B of a row + 16 B pad (bank spread)
constexpr int kPreStageBytes = kPreBM * kPreRowBytes;

template <bool PER_BLOCK_SCALE>
__global__ __launch_bounds__(256) void prefill_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, uint16_t *__restrict__ y, int M, int K, int N,
    int group_size) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[2 * kPreStageBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int kb = lane >> 4;
    const int col16 = lane & 15;
    const int m0 = blockIdx.y * kPreBM;
    const int n = blockIdx.x * kPreBN + wave * 64 + 4 * col16;
    const int G = group_size == -1 ? 1 : (K + group_size - 1) / group_size;

    const auto xr = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
    const auto qr = make_rsrc(qweight, (uint32_t)(K >> 3) * (uint32_t)N * 4u);
    const auto sr = make_rsrc(scales, (uint32_t)G * (uint32_t)N * 2u);

    // ---- activation staging: thread tid moves chunks tid + 256 i, i < 4 ----
    // chunk c: row c / 8, 8-deep K block c % 8 of the stage.
    uint32_t a_goff[4];
    bool a_row_ok[4];
    int a_kc[4];
    uint32_t a_loff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = tid + 256 * i;
        const int row = c >> 3, kc = c & 7;
        a_row_ok[i] = m0 + row < M;
        a_kc[i] = kc;
        a_goff[i] = ((uint32_t)(m0 + row) * (uint32_t)K + 8u * kc) * 2u;
        a_loff[i] = row * kPreRowBytes + kc * 16;
    }
    auto load_a = [&](u4 (&r)[4], int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = a_row_ok[i] && (k0 + 8 * a_kc[i] < K);
            r[i] = load_b128(xr, ok ? a_goff[i] + (uint32_t)k0 * 2u : kOOB);
        }
    };
    auto store_a = [&](const u4 (&r)[4], int stage) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<u4 *>(lds + stage * kPreStageBytes + a_loff[i]) = perm_x(r[i]);
    };

    // ---- weights: lane's words of packed row 4t + kb, columns n..n+3 ----
    const uint32_t q_off0 = ((uint32_t)kb * (uint32_t)N + (uint32_t)n) * 4u;
    const uint32_t q_step = (uint32_t)N * 16u;     // one 32-deep step = 4 packed rows
    auto scale_row = [&](int t) -> int {           // group of this lane's 8-deep block
        if (group_size == -1) return 0;
        return (32 * t + 8 * kb) / group_size;
    };
    auto load_b = [&](u4 (&w)[2], u2 (&s)[2], int t) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            w[h] = load_b128(qr, q_off0 + (uint32_t)(t + h) * q_step);
            s[h] = load_b64(sr, ((uint32_t)scale_row(t + h) * (uint32_t)N + (uint32_t)n) * 2u);
        }
    };

    const UnpackConsts uc = unpack_consts();
    f4 acc[8][4];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[mt][j] = f4{0.f, 0.f, 0.f, 0.f};

    const int nst = (K + kPreBK - 1) / kPreBK;
    u4 areg[4];
    u4 wcur[2], wnxt[2];
    u2 scur[2], snxt[2];

    load_a(areg, 0);
    load_b(wcur, scur, 0);
    store_a(areg, 0);
    __syncthreads();

    for (int st = 0; st < nst; ++st) {
        const int stage = st & 1;
        // next stage in flight (past the end the loads return zero; unused)
        load_a(areg, (st + 1) * kPreBK);
        load_b(wnxt, snxt, 2 * (st + 1));

#pragma unroll
        for (int h = 0; h < 2; ++h) {
            h8 b[4];
            const _Float16 s4[4] = {half_lo(scur[h].x), half_hi(scur[h].x), half_lo(scur[h].y),
                                    half_hi(scur[h].y)};
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = unpack_codes_scaled(wcur[h][j], uc, s4[j]);
            const unsigned char *abase =
                lds + stage * kPreStageBytes + col16 * kPreRowBytes + (h * 4 + kb) * 16;
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) {
                const h8 a = __builtin_bit_cast(
                    h8, *reinterpret_cast<const u4 *>(abase + mt * 16 * kPreRowBytes));
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[mt][j] = mfma16x16x32(a, b[j], acc[mt][j]);
            }
        }

        store_a(areg, stage ^ 1);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            wcur[h] = wnxt[h];
            scur[h] = snxt[h];
        }
        __syncthreads();
    }

    // ---- epilogue: rows m0 + 16 mt + 4 kb + i, columns n .. n+3 ----
    if (n < N) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = m0 + 16 * mt + 4 * kb + i;
                if (m < M) {
                    const u2 out = pack4_f16(acc[mt][0][i], acc[mt][1][i], acc[mt][2][i],
                                             acc[mt][3][i]);
                    *reinterpret_cast<u2 *>(y + (size_t)m * N + n) = out;
                }
            }
        }
    }
}

hipError_t launch_prefill(const LinearArgs &a, hipStream_t stream) {
    const int K = (int)a.K, N = (int)a.N, M = (int)a.M, g = (int)a.group_size;
    const void *xp = a.x;
    const void *qp = a.qweight;
    const void *sp = a.scales;
    void *yp = a.y;
    void *args[] = {&xp, &qp, &sp, &yp, (void *)&M, (void *)&K, (void *)&N, (void *)&g};
    dim3 grid((unsigned)((N + kPreBN - 1) / kPreBN), (unsigned)((M + kPreBM - 1) / kPreBM));
    dim3 block(256);
    return hipLaunchKernel(reinterpret_cast<const void *>(&prefill_kernel<true>), grid, block,
                           args, 0, stream);
}

}  // namespace w4a16
