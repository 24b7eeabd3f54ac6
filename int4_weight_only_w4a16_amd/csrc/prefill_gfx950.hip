// Prefill W4A16 GEMM for gfx950: any M, MFMA with fp32 accumulation.
//
// The pages' prefill path ("GPTQ-Pro" README, "Ampere kernel architecture",
// Tensor Core prefill) stages operands asynchronously, accumulates in FP32,
// handles tails and stores FP16 vectors.  The CDNA4 design:
//
//  * A workgroup of 4 waves owns a 128 (M) x 256 (N) output tile; wave w owns
//    the 128 x 64 slice of columns 64w .. 64w+63 as 4 x 2 tiles of the
//    v_mfma_f32_32x32x16_f16 instruction (128 fp32 accumulators per lane).
//    With one wave per SIMD (the accumulators and the operand pipeline use
//    most of the register file) this instruction keeps the matrix core busy;
//    the 16x16x32 one does not.
//  * Column tile j of a wave holds the columns 64w + 2c + j (c = 0..31): a
//    lane's one 64-bit load per 16-deep step brings the two adjacent qweight
//    words, the 8-deep B fragments of both column tiles, so each packed row
//    is read in 256-byte runs.  Weights never touch LDS: they are dequantised
//    in registers to (q-8)*s in fp16 (one rounding) and each fragment feeds
//    the 4 row tiles.
//  * Activations go global -> registers -> LDS, 64 K per stage.  Each 16-byte
//    chunk is reordered on the way in to the K order the nibble unpack
//    produces, so MFMA A fragments are plain ds_read_b128.
//  * Pipeline: activations are loaded four stages ahead and stored to LDS two
//    stages ahead (three LDS stages, one barrier per stage); weights and
//    scales are loaded three stages ahead into a register ring.  The loop is
//    unrolled three times so every ring index is static.
//  * Tails: rows >= M and K >= K read as zero through buffer range checks;
//    stores are masked per row and per column pair (N % 8 == 0).

#include "w4a16_device.hpp"
#include "w4a16_launch.h"

namespace w4a16 {

constexpr int kPreBM = 128;               // rows per workgroup tile
constexpr int kPreBN = 256;               // columns per workgroup tile
constexpr int kPreBK = 64;                // K per stage
constexpr int kPreRowBytes = 144;         // 128 B of a row + 16 B pad (bank spread)
constexpr int kPreStageBytes = kPreBM * kPreRowBytes;
constexpr int kPreRing = 3;               // LDS stages, register stages per operand
constexpr int kPreSteps = kPreBK / 16;    // 16-deep MFMA steps per stage

// gshift: log2(group_size), or -1 for a single group over K.
__global__ __launch_bounds__(256) void prefill_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, uint16_t *__restrict__ y, int M, int K, int N,
    int gshift) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[kPreRing * kPreStageBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int kb = lane >> 5;                 // K block (8 deep) of the 16-deep step
    const int c32 = lane & 31;                // row / column of the 32 x 32 tile
    const int m0 = blockIdx.y * kPreBM;
    const int n = blockIdx.x * kPreBN + wave * 64 + 2 * c32;   // the lane's two columns
    const int G = gshift < 0 ? 1 : ((K - 1) >> gshift) + 1;

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
    auto load_a = [&](u4 (&r)[4], int st) {
        const int k0 = st * kPreBK;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = a_row_ok[i] && (k0 + 8 * a_kc[i] < K);
            r[i] = load_b128(xr, ok ? a_goff[i] + (uint32_t)k0 * 2u : kOOB);
        }
    };
    auto store_a = [&](const u4 (&r)[4], int slot) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<u4 *>(lds + slot * kPreStageBytes + a_loff[i]) = perm_x(r[i]);
    };

    // ---- weights: words of packed row 2t + kb, columns n, n+1 (t = 16-deep step) ----
    const uint32_t q_off0 = ((uint32_t)kb * (uint32_t)N + (uint32_t)n) * 4u;
    const uint32_t q_step = (uint32_t)N * 8u;      // 2 packed rows
    auto load_b = [&](u2 (&w)[kPreSteps], uint32_t (&s)[kPreSteps], int st) {
#pragma unroll
        for (int h = 0; h < kPreSteps; ++h) {
            const int t = kPreSteps * st + h;
            const uint32_t srow = gshift < 0 ? 0u : (uint32_t)(16 * t) >> gshift;
            w[h] = load_b64(qr, q_off0 + (uint32_t)t * q_step);
            s[h] = __builtin_amdgcn_raw_buffer_load_b32(sr, (srow * (uint32_t)N + (uint32_t)n) * 2u, 0, 0);
        }
    };

    const UnpackConsts uc = unpack_consts();
    f16v acc[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[mt][j][e] = 0.f;

    // A fragments of step h of LDS slot `slot` (4 row tiles)
    auto read_a = [&](h8 (&a)[4], int slot, int h) {
        const unsigned char *abase =
            lds + slot * kPreStageBytes + c32 * kPreRowBytes + kb * 16 + h * 32;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            a[mt] = __builtin_bit_cast(h8, *reinterpret_cast<const u4 *>(abase + mt * 32 * kPreRowBytes));
    };
    // One stage: 4 steps x (4 row tiles x 2 column tiles) MFMAs.  The A
    // fragments of each step are read during the previous step's MFMAs (the
    // first step's during the previous stage), so LDS latency stays hidden
    // with one wave per SIMD.  On entry `a` holds step 0 of this stage; on
    // exit step 0 of the next stage (slot `next`, stored two stages ago).
    auto compute = [&](int slot, int next, const u2 (&w)[kPreSteps], const uint32_t (&s)[kPreSteps],
                       h8 (&a)[4]) {
#pragma unroll
        for (int h = 0; h < kPreSteps; ++h) {
            h8 an[4];
            if (h + 1 < kPreSteps) read_a(an, slot, h + 1);
            else read_a(an, next, 0);
            const h8 b0 = unpack_codes_scaled(w[h].x, uc, half_lo(s[h]));
            const h8 b1 = unpack_codes_scaled(w[h].y, uc, half_hi(s[h]));
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                acc[mt][0] = mfma32x32x16(a[mt], b0, acc[mt][0]);
                acc[mt][1] = mfma32x32x16(a[mt], b1, acc[mt][1]);
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) a[mt] = an[mt];
        }
    };

    const int nst = (K + kPreBK - 1) / kPreBK;
    u4 areg[kPreRing][4];
    u2 wreg[kPreRing][kPreSteps];
    uint32_t sreg[kPreRing][kPreSteps];

    // Prologue in the loop's issue order (stage st's loop iteration issues A
    // of st+4, then B of st+3), so the compiler's wait counts in the loop
    // stay deep.  Loads past the last stage read zero and are not used.
    load_a(areg[0], 0);
    __builtin_amdgcn_sched_barrier(0);
    load_a(areg[1], 1);
    __builtin_amdgcn_sched_barrier(0);
    load_b(wreg[0], sreg[0], 0);
    __builtin_amdgcn_sched_barrier(0);
    load_a(areg[2], 2);
    __builtin_amdgcn_sched_barrier(0);
    load_b(wreg[1], sreg[1], 1);
    __builtin_amdgcn_sched_barrier(0);
    store_a(areg[0], 0);
    load_a(areg[0], 3);
    __builtin_amdgcn_sched_barrier(0);
    load_b(wreg[2], sreg[2], 2);
    __builtin_amdgcn_sched_barrier(0);
    store_a(areg[1], 1);
    __syncthreads();
    h8 afrag[4];
    read_a(afrag, 0, 0);

    // Stages past nst (up to two, to finish a round of three) compute on
    // zeros: every load there is out of range.
    for (int st0 = 0; st0 < nst; st0 += kPreRing) {
#pragma unroll
        for (int r = 0; r < kPreRing; ++r) {
            const int st = st0 + r;
            load_a(areg[(r + 1) % kPreRing], st + 4);               // slot of stage st+1, stored
            compute(r, (r + 1) % kPreRing, wreg[r], sreg[r], afrag);
            load_b(wreg[r], sreg[r], st + 3);
            store_a(areg[(r + 2) % kPreRing], (r + 2) % kPreRing);  // stage st+2
            __syncthreads();
        }
    }

    // ---- epilogue: register i of tile (mt, j) is row m0 + 32 mt + 8 (i/4) +
    // 4 kb + i%4, column n + j; the two columns of a lane go out together ----
    if (n < N) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = m0 + 32 * mt + 8 * (i >> 2) + 4 * kb + (i & 3);
                if (m < M) {
                    const h2 v = {(_Float16)acc[mt][0][i], (_Float16)acc[mt][1][i]};
                    *reinterpret_cast<uint32_t *>(y + (size_t)m * N + n) = __builtin_bit_cast(uint32_t, v);
                }
            }
        }
    }
}

hipError_t launch_prefill(const LinearArgs &a, hipStream_t stream) {
    int K = (int)a.K, N = (int)a.N, M = (int)a.M;
    int gshift = -1;
    if (a.group_size != -1) gshift = __builtin_ctz((unsigned)a.group_size);
    const void *xp = a.x;
    const void *qp = a.qweight;
    const void *sp = a.scales;
    void *yp = a.y;
    void *args[] = {&xp, &qp, &sp, &yp, &M, &K, &N, &gshift};
    dim3 grid((unsigned)((N + kPreBN - 1) / kPreBN), (unsigned)((M + kPreBM - 1) / kPreBM));
    dim3 block(256);
    return hipLaunchKernel(reinterpret_cast<const void *>(&prefill_kernel), grid, block, args, 0,
                           stream);
}

}  // namespace w4a16
