// Small-batch (decode) W4A16 kernel for gfx950: M <= 16 rows of x.
//
// What the pages ask of this path ("GPTQ-Pro" README, "Ampere kernel
// architecture", fused decode): output tiles shared by cooperating warps,
// reuse of the native qweight across the M rows, scale residency and a
// deterministic split-K reduction; "Why GPTQ-Pro": no duplicate repacked
// weight.  The design here is for CDNA4, not a translation:
//
//  * One workgroup owns 64 output columns and every row m < M.  Its waves
//    split K into contiguous ranges of 32-deep steps (split-K inside the
//    workgroup only, so no atomics and no scratch memory).
//  * Each lane streams one 128-bit word quad per step: qweight row
//    4t + lane/16, columns n0 + 4*(lane%16) .. +3.  Sixteen lanes cover 256
//    contiguous bytes of one packed row, so every fetched line is used whole.
//  * The four words of a lane are exactly the B operands of four
//    v_mfma_f32_16x16x32_f16 instructions (one 8-deep K block of one column
//    each); the activation rows (padded to 16 with zeros) are the A operand.
//    The matrix cores do the multiply-accumulate for any M <= 16 at the same
//    cost, so the vector ALUs only unpack nibbles.
//  * For g >= 32 a step lies inside one group: the MFMA sums x*(q-8) over
//    the group in fp32 and the group's scale is applied once per group and
//    column (scale-after).  For g = 16 every 8-deep block is scaled before
//    the MFMA (scale-before, one fp16 rounding of (q-8)*s).
//  * Waves reduce their fp32 partials through LDS in wave order 0..W-1, a
//    fixed order, then round once to fp16 (8-byte stores of 4 columns).

#include "w4a16_device.hpp"
#include "w4a16_launch.h"

namespace w4a16 {

constexpr int kDecodeCols = 64;

template <int WAVES, int U, bool SCALE_AFTER>
__global__ __launch_bounds__(WAVES * 64) void decode_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, uint16_t *__restrict__ y, int M, int K, int N,
    int group_steps) {
    __shared__ f4 red[WAVES * 4 * 64];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int kb = lane >> 4;        // 8-deep K block of this lane inside a step
    const int col16 = lane & 15;     // MFMA row (A) / column (B) of this lane
    const int n = blockIdx.x * kDecodeCols + 4 * col16;

    const int steps = (K + 31) >> 5;
    const int per = (steps + WAVES - 1) / WAVES;
    const int t0 = min(steps, wave * per);
    const int t1 = min(steps, t0 + per);

    const auto xr = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
    const auto qr = make_rsrc(qweight, (uint32_t)(K >> 3) * (uint32_t)N * 4u);
    const int G = SCALE_AFTER ? (steps + group_steps - 1) / group_steps : (K + 15) >> 4;
    const auto sr = make_rsrc(scales, (uint32_t)G * (uint32_t)N * 2u);

    const uint32_t q_off0 = ((uint32_t)kb * (uint32_t)N + (uint32_t)n) * 4u;
    const uint32_t q_step = (uint32_t)N * 16u;
    const uint32_t x_off0 = ((uint32_t)col16 * (uint32_t)K + 8u * kb) * 2u;

    f4 acc[4], accg[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        acc[j] = f4{0.f, 0.f, 0.f, 0.f};
        accg[j] = f4{0.f, 0.f, 0.f, 0.f};
    }
    int cur_grp = SCALE_AFTER ? t0 / group_steps : 0;
    u2 cur_s = {0u, 0u};

    for (int t = t0; t < t1; t += U) {
        u4 wv[U], xv[U];
        u2 sv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int tt = t + u;   // past t1 the loads are in range or return zero; unused
            wv[u] = load_b128(qr, q_off0 + (uint32_t)tt * q_step);
            const bool k_ok = 32 * tt + 8 * kb < K;
            xv[u] = load_b128(xr, k_ok ? x_off0 + (uint32_t)tt * 64u : kOOB);
            const int srow = SCALE_AFTER ? tt / group_steps : 2 * tt + (kb >> 1);
            sv[u] = load_b64(sr, ((uint32_t)srow * (uint32_t)N + (uint32_t)n) * 2u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int tt = t + u;
            if (tt >= t1) break;
            const h8 a = __builtin_bit_cast(h8, perm_x(xv[u]));
            if constexpr (SCALE_AFTER) {
                const int grp = tt / group_steps;
                if (grp != cur_grp) {
                    const float s[4] = {(float)half_lo(cur_s.x), (float)half_hi(cur_s.x),
                                        (float)half_lo(cur_s.y), (float)half_hi(cur_s.y)};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        acc[j] += s[j] * accg[j];
                        accg[j] = f4{0.f, 0.f, 0.f, 0.f};
                    }
                    cur_grp = grp;
                }
                cur_s = sv[u];
#pragma unroll
                for (int j = 0; j < 4; ++j) accg[j] = mfma16x16x32(a, unpack_codes(wv[u][j]), accg[j]);
            } else {
                const _Float16 s[4] = {half_lo(sv[u].x), half_hi(sv[u].x), half_lo(sv[u].y),
                                       half_hi(sv[u].y)};
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[j] = mfma16x16x32(a, unpack_codes_scaled(wv[u][j], s[j]), acc[j]);
            }
        }
    }
    if constexpr (SCALE_AFTER) {
        const float s[4] = {(float)half_lo(cur_s.x), (float)half_hi(cur_s.x),
                            (float)half_lo(cur_s.y), (float)half_hi(cur_s.y)};
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] += s[j] * accg[j];
    }

    // Fixed-order reduction over the waves, then one fp16 rounding.
#pragma unroll
    for (int j = 0; j < 4; ++j) red[(wave * 4 + j) * 64 + lane] = acc[j];
    __syncthreads();
    if (threadIdx.x < 256) {
        const int l = threadIdx.x & 63;
        const int i = threadIdx.x >> 6;                 // row inside the lane's quad
        const int m = 4 * (l >> 4) + i;
        const int nn = blockIdx.x * kDecodeCols + 4 * (l & 15);
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        for (int w = 0; w < WAVES; ++w) {
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] += red[(w * 4 + j) * 64 + l][i];
        }
        if (m < M && nn < N) {
            const u2 out = pack4_f16(v[0], v[1], v[2], v[3]);
            *reinterpret_cast<u2 *>(y + (size_t)m * N + nn) = out;
        }
    }
}

template <int WAVES, int U, bool SCALE_AFTER>
static hipError_t launch(const LinearArgs &a, hipStream_t stream) {
    const int K = (int)a.K, N = (int)a.N, M = (int)a.M;
    const int steps = (K + 31) / 32;
    int group_steps = 0;
    if (SCALE_AFTER) group_steps = a.group_size == -1 ? steps : (int)a.group_size / 32;
    const void *xp = a.x;
    const void *qp = a.qweight;
    const void *sp = a.scales;
    void *yp = a.y;
    void *args[] = {&xp, &qp, &sp, &yp, (void *)&M, (void *)&K, (void *)&N, &group_steps};
    dim3 grid((unsigned)((N + kDecodeCols - 1) / kDecodeCols));
    dim3 block(WAVES * 64);
    return hipLaunchKernel(reinterpret_cast<const void *>(&decode_kernel<WAVES, U, SCALE_AFTER>),
                           grid, block, args, 0, stream);
}

hipError_t launch_decode(const LinearArgs &a, hipStream_t stream) {
    if (a.group_size == 16) return launch<8, 4, false>(a, stream);
    return launch<8, 4, true>(a, stream);
}

}  // namespace w4a16
