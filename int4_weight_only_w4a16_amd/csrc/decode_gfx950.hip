// Small-batch (decode) W4A16 kernels for gfx950: M <= 16 rows of x.
//
// What the pages ask of this path ("GPTQ-Pro" README, "Ampere kernel
// architecture", fused decode): output tiles shared by cooperating warps,
// reuse of the native qweight across the M rows, scale residency and a
// deterministic split-K reduction; "Why GPTQ-Pro": no duplicate repacked
// weight.  Decode streams every weight byte once, so the design is about
// keeping HBM busy on CDNA4:
//
//  * Work unit = (column tile of COLS = 16*NW columns, 32-deep K step).  Per
//    unit a lane loads NW consecutive qweight words (one 32/64/128-bit load)
//    of packed row 4t + lane/16; sixteen lanes cover one contiguous row
//    segment, so fetched lines are used whole.
//  * Each word is the 8-deep B operand of one v_mfma_f32_16x16x32_f16 (one
//    column); the activation rows, zero-padded to 16, are the A operand.  The
//    matrix cores do the multiply-accumulate for any M <= 16 at the same
//    cost, so the vector ALUs only unpack nibbles.
//  * Loads run D units ahead of the math through a ring of D register stages
//    refilled as soon as a stage is consumed.  Every load is issued
//    unconditionally so the compiler's waits count exactly the loads in
//    flight; past the wave's last unit the ring reloads that unit (a cache
//    hit, no HBM traffic).
//  * For g >= 32 a step lies inside one group: the MFMA sums x*(q-8) over the
//    group in fp32 and the group's scale multiplies the sum once per group
//    and column (scale-after).  For g = 16 each 8-deep block is scaled before
//    the MFMA (scale-before, one fp16 rounding of (q-8)*s).
//  * A CU can pull only about twice its fair share of HBM bandwidth, so the
//    work must be spread evenly over all CUs.  The stream-K kernel gives each
//    of G workgroups (G = CU count) an equal contiguous range of units in
//    tile-major order; its waves split that range contiguously and keep
//    their load rings running across tile boundaries.  A tile that lies
//    wholly inside one workgroup is finished there; a tile split between
//    two workgroups is finished by whichever comes second, through one
//    compare-and-swap per output column pair: it adds the other's fp32
//    partial to its own (one add, so the result does not depend on the
//    order of arrival).
//  * When there are many more tiles than CUs the tiles kernel (one
//    workgroup per tile, its waves splitting K) is balanced on its own and
//    needs no workspace.
//  * Within a workgroup, wave partials are added through LDS in wave order,
//    then rounded once to fp16.

#include <algorithm>

#include "w4a16_device.hpp"
#include "w4a16_launch.h"

namespace w4a16 {

constexpr int kNW = 4;                 // words per lane per unit: one 128-bit load
constexpr int kCols = 16 * kNW;        // columns per tile

template <bool XLDS>
struct Stage {
    u4 w;     // qweight words of the lane's 4 consecutive columns
    u4 x;     // 8 activations of this lane's A row / K block (unused when staged in LDS)
    u2 s;     // the 4 columns' fp16 scales
};

// Activations staged in LDS: rows m < M of x, each zero-padded to Kp = 32*S
// halves and already in unpack order (perm_x per 16-byte chunk), followed by
// one zero chunk that the lanes of rows m >= M read.  Staging is split in
// two so that the first kXPre chunks of each thread are requested before the
// weight prologue (they would otherwise queue behind it): stage_x_issue loads
// them, stage_x_finish stores them and any further chunks and returns this
// lane's byte address of step 0.
constexpr int kXPre = 2;

struct XPre {
    u4 v[kXPre];
};

__device__ __forceinline__ u4 stage_x_load(const __amdgpu_buffer_rsrc_t xr, int c, int K,
                                           int chunks_per_row) {
    const int m = c / chunks_per_row;
    const int k = 8 * (c - m * chunks_per_row);
    return load_b128(xr, k < K ? ((uint32_t)m * (uint32_t)K + (uint32_t)k) * 2u : kOOB);
}

__device__ __forceinline__ XPre stage_x_issue(const __amdgpu_buffer_rsrc_t xr, int M, int K,
                                              int S) {
    const int chunks_per_row = 4 * S;
    const int total = M * chunks_per_row;
    XPre pre;
#pragma unroll
    for (int r = 0; r < kXPre; ++r) {
        const int c = threadIdx.x + r * blockDim.x;
        pre.v[r] = stage_x_load(xr, c < total ? c : 0, K, chunks_per_row);
    }
    return pre;
}

__device__ __forceinline__ uint32_t stage_x_finish(unsigned char *xs,
                                                   const __amdgpu_buffer_rsrc_t xr, int M, int K,
                                                   int S, const XPre &pre) {
    const int Kp = 32 * S;
    const int chunks_per_row = Kp / 8;
    const int total = M * chunks_per_row;
    auto put = [&](int c, const u4 &v) {
        const int m = c / chunks_per_row;
        const int k = 8 * (c - m * chunks_per_row);
        *reinterpret_cast<u4 *>(xs + ((size_t)m * Kp + k) * 2) = perm_x(v);
    };
#pragma unroll
    for (int r = 0; r < kXPre; ++r) {
        const int c = threadIdx.x + r * blockDim.x;
        if (c < total) put(c, pre.v[r]);
    }
    for (int c = threadIdx.x + kXPre * blockDim.x; c < total; c += blockDim.x)
        put(c, stage_x_load(xr, c, K, chunks_per_row));
    if (threadIdx.x == 0) *reinterpret_cast<u4 *>(xs + (size_t)M * Kp * 2) = u4{0u, 0u, 0u, 0u};
    const int lane = threadIdx.x & 63;
    const int m = lane & 15, kb = lane >> 4;
    return m < M ? (uint32_t)(((size_t)m * Kp + 8 * kb) * 2) : (uint32_t)((size_t)M * Kp * 2);
}

__device__ __forceinline__ _Float16 scale_at(const u2 &s, int j) {
    const uint32_t d = j < 2 ? s.x : s.y;
    return (j & 1) ? half_hi(d) : half_lo(d);
}


// One wave's pass over a contiguous range [w0, w1) of units (tile-major:
// unit u = tile u / S, step u % S).  The host keeps w1 - w0 <= S, so the
// range is at most two tile segments: steps [tA0, S) or [tA0, tA0 + n) of
// tile bA, then steps [0, n - nA) of tile bA + 1.  `dump(slot, acc)` gets the
// wave's fp32 sum for each segment (slot 0, then 1): rows 4*(lane/16)+i,
// columns 4*(lane%16)+j of the tile.
//
// Per unit the scalar work is a few compares and selects: every address
// advances by a precomputed increment (a step, the jump to the next tile, or
// nothing once past the last unit: the ring's tail reloads the last unit,
// which hits in cache and moves no HBM data).
//
// XLDS: activations come from LDS staged by `after_prologue` (called once the
// first D weight loads are in flight; it returns this lane's LDS byte address
// of step 0 and ends with a workgroup barrier); otherwise from global.
// SCALE: 0 scales each 8-deep block before the MFMA (g = 16); 1 sums a
// group's products in fp32 and scales once per group (scale-after); 2 is
// scale-after with one step per group (g = 32): every MFMA starts from zero
// and its result is scaled straight into the sum.  SCALE picks which scale
// row each unit loads.
// BF: bfloat16 activations.  With SCALE 0 (g = 16) every weight is
// dequantised before the MFMA, (q - 8) * s exactly in fp32 and rounded once
// to bfloat16 (dequant_bf16).  Otherwise the MFMA sums x * (128 + q) over the
// group (codes128_bf16, exact) and a second MFMA sums x * 136 over the same
// steps; at the group's end acc += s * (sum - sum136) in fp32.  Where every
// code of a group is 8 the two sums are the same operations on the same
// values, so that group adds exactly zero, as (8 - 8) * s does.
template <int D, int SCALE, bool XLDS, bool BF, typename Dump, typename AfterPrologue>
__device__ __forceinline__ void decode_units(
    const __amdgpu_buffer_rsrc_t xr, const __amdgpu_buffer_rsrc_t qr,
    const __amdgpu_buffer_rsrc_t sr, const unsigned char *xs, int M, int K, int N, int S,
    int group_steps, int w0, int w1, Dump &&dump, AfterPrologue &&after_prologue) {
    constexpr bool SCALE_AFTER = SCALE != 0;
    const int lane = threadIdx.x & 63;
    const int kb = lane >> 4;
    const int c16 = lane & 15;

    // segments (all scalar)
    const int n = w1 > w0 ? w1 - w0 : 0;
    const int bA = n ? w0 / S : 0;
    const int tA0 = n ? w0 - bA * S : 0;
    const int nA = min(n, S - tA0);

    // per-lane byte offsets of the wave's first unit and their increments
    const uint32_t q_step = (uint32_t)N * 16u;                       // 4 packed rows
    const uint32_t q_jump = 256u - (uint32_t)S * q_step;              // to step 0 of the next tile
    uint32_t q_off = ((uint32_t)(kb + 4 * tA0) * (uint32_t)N + (uint32_t)(bA * kCols + kNW * c16)) * 4u;

    const bool ragged = (K & 31) != 0;        // the last step of a tile is half inside K
    const uint32_t x_jump = 0u - (uint32_t)S * 64u;
    uint32_t x_off = ((uint32_t)c16 * (uint32_t)K + 8u * kb) * 2u + 64u * (uint32_t)tA0;
    const bool x_tail_ok = 32 * (S - 1) + 8 * kb < K;

    // scale rows: scale-after reads the group's row (advances at group ends);
    // scale-before reads row 2t + kb/2 (advances by two rows per step)
    int lpos = SCALE_AFTER ? tA0 % group_steps : 0;
    const uint32_t s_row = (uint32_t)N * 2u;
    uint32_t s_off;
    if constexpr (SCALE_AFTER)
        s_off = ((uint32_t)(tA0 / group_steps) * (uint32_t)N + (uint32_t)(bA * kCols + kNW * c16)) * 2u;
    else
        s_off = ((uint32_t)(2 * tA0 + (kb >> 1)) * (uint32_t)N + (uint32_t)(bA * kCols + kNW * c16)) * 2u;
    const uint32_t s_tile0 = ((uint32_t)(SCALE_AFTER ? 0 : (kb >> 1)) * (uint32_t)N +
                              (uint32_t)((bA + 1) * kCols + kNW * c16)) * 2u;

    const UnpackConsts uc = unpack_consts();

    // issue side: unit index li of this wave (loads beyond n - 1 repeat the last unit)
    int li = 0;
    auto issue = [&](Stage<XLDS> &st) {
        st.w = load_b128_nt(qr, q_off);           // every weight word is read once
        if constexpr (!XLDS) {
            const int t = li < nA ? tA0 + li : li - nA;
            const uint32_t xo = (ragged && t == S - 1 && !x_tail_ok) ? kOOB : x_off;
            st.x = load_b128(xr, xo);
        }
        st.s = load_b64(sr, s_off);
        // advance to unit li + 1 (stay put at the last unit)
        const bool more = li + 1 < n;
        const bool jump = li + 1 == nA;
        q_off += more ? (jump ? q_step + q_jump : q_step) : 0u;
        if constexpr (!XLDS) x_off += more ? (jump ? 64u + x_jump : 64u) : 0u;
        if constexpr (SCALE_AFTER) {
            const bool grp_end = lpos + 1 == group_steps;
            lpos = (grp_end || jump) ? 0 : lpos + 1;
            const uint32_t s_next = s_off + (grp_end ? s_row : 0u);
            s_off = more ? (jump ? s_tile0 : s_next) : s_off;
        } else {
            s_off = more ? (jump ? s_tile0 : s_off + 2u * s_row) : s_off;
        }
        ++li;
    };

    f4 acc[kNW], accg[kNW], accx = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kNW; ++j) {
        acc[j] = f4{0.f, 0.f, 0.f, 0.f};
        accg[j] = f4{0.f, 0.f, 0.f, 0.f};
    }

    // Prologue loads in ring order: the compiler's wait counts at the loop
    // head take the stricter of the prologue's and the loop's load order, so
    // the scheduler must not reorder these.
    Stage<XLDS> ring[D];
#pragma unroll
    for (int u = 0; u < D; ++u) {
        issue(ring[u]);
        __builtin_amdgcn_sched_barrier(0);
    }
    // LDS activation address: rows < M advance 64 B per step, rows >= M stay
    // on the zero chunk
    const uint32_t xl0 = after_prologue();
    const uint32_t xl_inc = (XLDS && c16 < M) ? 64u : 0u;
    uint32_t xl = xl0 + xl_inc * (uint32_t)tA0;

    int i = 0, pos = SCALE_AFTER ? tA0 % group_steps : 0;
    // one unit of math on ring stage st (unit index i of this wave)
    auto compute = [&](Stage<XLDS> &st) {
        h8 a;
        if constexpr (XLDS)
            a = __builtin_bit_cast(h8, *reinterpret_cast<const u4 *>(xs + xl));
        else
            a = __builtin_bit_cast(h8, perm_x(st.x));
        const bool seg_end = i == nA - 1 || i == n - 1;
        if constexpr (BF && SCALE == 0) {
#pragma unroll
            for (int j = 0; j < kNW; ++j)
                acc[j] = mfma16x16x32_t<true>(__builtin_bit_cast(u4, a),
                                              dequant_bf16<false>(st.w[j], (float)scale_at(st.s, j)),
                                              acc[j]);
        } else if constexpr (BF && SCALE == 2) {
            // one step per group: both sums start from zero in the MFMA and go
            // straight into acc (no accumulators to reset)
            const u4 b136 = {0x43084308u, 0x43084308u, 0x43084308u, 0x43084308u};   // bf16 136.0
            const f4 zero = {0.f, 0.f, 0.f, 0.f};
            const f4 tx = mfma16x16x32_t<true>(__builtin_bit_cast(u4, a), b136, zero);
#pragma unroll
            for (int j = 0; j < kNW; ++j) {
                const f4 t = mfma16x16x32_t<true>(__builtin_bit_cast(u4, a), codes128_bf16(st.w[j], uc),
                                                  zero);
                const float sj = (float)scale_at(st.s, j);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[j][e] = __builtin_fmaf(sj, t[e] - tx[e], acc[j][e]);
            }
        } else if constexpr (BF) {
            const u4 b136 = {0x43084308u, 0x43084308u, 0x43084308u, 0x43084308u};   // bf16 136.0
#pragma unroll
            for (int j = 0; j < kNW; ++j)
                accg[j] = mfma16x16x32_t<true>(__builtin_bit_cast(u4, a), codes128_bf16(st.w[j], uc),
                                               accg[j]);
            accx = mfma16x16x32_t<true>(__builtin_bit_cast(u4, a), b136, accx);
            if (pos == group_steps - 1 || seg_end) {
#pragma unroll
                for (int j = 0; j < kNW; ++j) {
                    const float sj = (float)scale_at(st.s, j);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[j][e] = __builtin_fmaf(sj, accg[j][e] - accx[e], acc[j][e]);
                    accg[j] = f4{0.f, 0.f, 0.f, 0.f};
                }
                accx = f4{0.f, 0.f, 0.f, 0.f};
            }
            pos = (pos + 1 == group_steps) ? 0 : pos + 1;
        } else if constexpr (SCALE == 2) {
#pragma unroll
            for (int j = 0; j < kNW; ++j) {
                const f4 t = mfma16x16x32(a, unpack_codes(st.w[j], uc), f4{0.f, 0.f, 0.f, 0.f});
                acc[j] += (float)scale_at(st.s, j) * t;
            }
        } else if constexpr (SCALE_AFTER) {
#pragma unroll
            for (int j = 0; j < kNW; ++j)
                accg[j] = mfma16x16x32(a, unpack_codes(st.w[j], uc), accg[j]);
            if (pos == group_steps - 1 || seg_end) {
#pragma unroll
                for (int j = 0; j < kNW; ++j) {
                    acc[j] += (float)scale_at(st.s, j) * accg[j];
                    accg[j] = f4{0.f, 0.f, 0.f, 0.f};
                }
            }
            pos = (pos + 1 == group_steps) ? 0 : pos + 1;
        } else {
#pragma unroll
            for (int j = 0; j < kNW; ++j)
                acc[j] = mfma16x16x32(a, unpack_codes_scaled(st.w[j], uc, scale_at(st.s, j)),
                                      acc[j]);
        }
        if (seg_end) {
            dump(i < nA ? 0 : 1, acc);
#pragma unroll
            for (int j = 0; j < kNW; ++j) acc[j] = f4{0.f, 0.f, 0.f, 0.f};
            pos = 0;
        }
        if constexpr (XLDS) xl = seg_end ? xl0 : xl + xl_inc;   // a new segment starts at step 0
        ++i;
    };
    // full rounds: every stage holds a live unit
    for (; i + D <= n;) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            compute(ring[u]);
            issue(ring[u]);
        }
    }
    // last, partial round
#pragma unroll
    for (int u = 0; u < D; ++u) {
        if (i < n) compute(ring[u]);
    }
}

// ---------------------------------------------------------------------------
// Dynamic LDS: the staged activations (XLDS) follow the static arrays.
extern __shared__ __attribute__((aligned(16))) unsigned char decode_dyn_lds[];

// Tiles kernel: one workgroup per column tile, its waves split K.
template <int WAVES, int D, int SCALE, bool XLDS, bool BF, bool SILU>
__global__ __launch_bounds__(WAVES * 64) void decode_tiles_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, uint16_t *__restrict__ y, int M, int K, int N,
    int group_steps) {
    __shared__ f4 red[WAVES][kNW][64];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = (K + 31) >> 5;
    const int tile = blockIdx.x;
    const int per = (S + WAVES - 1) / WAVES;
    const int w0 = tile * S + min(S, wave * per);
    const int w1 = tile * S + min(S, wave * per + per);

    const int G = SCALE != 0 ? (S + group_steps - 1) / group_steps : (K + 15) >> 4;
    const auto xr = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
    const auto qr = make_rsrc(qweight, (uint32_t)(K >> 3) * (uint32_t)N * 4u);
    const auto sr = make_rsrc(scales, (uint32_t)G * (uint32_t)N * 2u);

#pragma unroll
    for (int j = 0; j < kNW; ++j) red[wave][j][lane] = f4{0.f, 0.f, 0.f, 0.f};
    XPre xpre;
    if constexpr (XLDS) xpre = stage_x_issue(xr, M, K, S);
    __builtin_amdgcn_sched_barrier(0);
    decode_units<D, SCALE, XLDS, BF>(
        xr, qr, sr, decode_dyn_lds, M, K, N, S, group_steps, w0, w1,
        [&](int, const f4(&acc)[kNW]) {
#pragma unroll
            for (int j = 0; j < kNW; ++j) red[wave][j][lane] = acc[j];
        },
        [&]() -> uint32_t {
            if constexpr (XLDS) {
                const uint32_t a = stage_x_finish(decode_dyn_lds, xr, M, K, S, xpre);
                __syncthreads();
                return a;
            }
            return 0u;
        });
    __syncthreads();
    if (threadIdx.x < 256) {
        const int l = threadIdx.x & 63;
        const int i = threadIdx.x >> 6;
        const int m = 4 * (l >> 4) + i;
        const int n = tile * kCols + kNW * (l & 15);
        float v[kNW] = {0.f, 0.f, 0.f, 0.f};
        for (int w = 0; w < WAVES; ++w) {
#pragma unroll
            for (int j = 0; j < kNW; ++j) v[j] += red[w][j][l][i];
        }
        if (m < M && n < N) store_quad<BF, SILU>(y, m, N, n, v);
    }
}

// ---------------------------------------------------------------------------
// Stream-K kernel: gridDim.x workgroups share the units evenly.
//
// Workspace for up to `capacity` workgroups (zero-filled once).  The layout
// depends only on the capacity, never on the grid of a launch, so launches
// of any grid size share it:
//   slots:    uint64[capacity][16][kCols/2] one exchange slot per (row,
//             output column pair) of a split tile, indexed by the tile's
//             later contributor; 0 when empty, and every launch leaves them 0
//   partials: float[capacity][2][16][kCols] a workgroup's sums for its first
//             (0) and last (1) tile, for launches whose tiles may have more
//             than two contributors (written before they are read)

// A slot holds two fp32 partials (adjacent columns), each XOR-ed with the bit
// pattern of a NaN; NaN partials are first replaced by the canonical NaN, so
// an occupied slot is never 0, the empty value.
constexpr uint32_t kSlotKey = 0x7FBADBADu;

__device__ __forceinline__ uint32_t slot_code(float v) {
    return (v != v ? 0x7FC00000u : __builtin_bit_cast(uint32_t, v)) ^ kSlotKey;
}

// Stream-K ranges in 32-bit arithmetic: the host keeps U * G < 2^32.
struct StreamK {
    int U, G;
    __device__ __forceinline__ int begin(int g) const {
        return (int)((uint32_t)U * (uint32_t)g / (uint32_t)G);
    }
    // workgroup whose range holds unit u
    __device__ __forceinline__ int owner(int u) const {
        int g = (int)((uint32_t)u * (uint32_t)G / (uint32_t)U);
        while (g + 1 < G && begin(g + 1) <= u) ++g;
        while (g > 0 && begin(g) > u) --g;
        return g;
    }
};

// Older waves of a workgroup are served first when several are ready to
// issue (two waves share each SIMD), so with equal shares the older half
// finishes well before the younger one: the older half of the waves takes
// this share (per mille) of the workgroup's units.
constexpr int kOldShare = 610;

// Start of wave w's share of n units, w in [0, WAVES].
template <int WAVES>
__host__ __device__ __forceinline__ int wave_share(int n, int w) {
    constexpr int H = WAVES / 2;
    const int nold = (int)((int64_t)n * kOldShare / 1000);
    if (w <= H) return nold * w / H;
    return nold + (n - nold) * (w - H) / (WAVES - H);
}

template <int WAVES, int D, int SCALE, bool XLDS, bool BF, bool SILU>
__global__ __launch_bounds__(WAVES * 64) void decode_streamk_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, uint16_t *__restrict__ y, int M, int K, int N,
    int group_steps, uint64_t *__restrict__ slots, float *__restrict__ partials) {
    constexpr int SLOT = 16 * kCols;             // floats per partial slot
    // Wave partials: block s*WAVES + w (256 f4: [lane][i]) holds wave w's
    // sums of its segment s, row i of the lane's quad, its four columns
    // together (one 16-byte read back); block 2*WAVES holds -0.0, which
    // leaves any fp32 sum unchanged when added (the stand-in for a wave that
    // has no part of a tile, so the reduction reads without branches).
    constexpr int kZeroBlock = 2 * WAVES;
    __shared__ f4 red[(2 * WAVES + 1) * 256];
    __shared__ int wtile[WAVES][2];              // each wave's first and last tile

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = (K + 31) >> 5;
    const int T = (N + kCols - 1) / kCols;
    const StreamK sk{T * S, (int)gridDim.x};
    const int g = blockIdx.x;
    const int u0 = sk.begin(g), u1 = sk.begin(g + 1);
    // the host keeps every wave's share <= S units: at most two tiles per wave
    const int w0 = u0 + wave_share<WAVES>(u1 - u0, wave);
    const int w1 = u0 + wave_share<WAVES>(u1 - u0, wave + 1);

    const int Gs = SCALE != 0 ? (S + group_steps - 1) / group_steps : (K + 15) >> 4;
    const auto xr = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
    const auto qr = make_rsrc(qweight, (uint32_t)(K >> 3) * (uint32_t)N * 4u);
    const auto sr = make_rsrc(scales, (uint32_t)Gs * (uint32_t)N * 2u);

    XPre xpre;
    if constexpr (XLDS) xpre = stage_x_issue(xr, M, K, S);
    __builtin_amdgcn_sched_barrier(0);
    decode_units<D, SCALE, XLDS, BF>(
        xr, qr, sr, decode_dyn_lds, M, K, N, S, group_steps, w0, w1,
        [&](int slot, const f4(&acc)[kNW]) {
            if (slot > 1) return;   // cannot happen: ranges hold <= S units
#pragma unroll
            for (int r = 0; r < 4; ++r)
                red[(slot * WAVES + wave) * 256 + lane * 4 + r] =
                    f4{acc[0][r], acc[1][r], acc[2][r], acc[3][r]};
        },
        [&]() -> uint32_t {
            if constexpr (XLDS) {
                const uint32_t a = stage_x_finish(decode_dyn_lds, xr, M, K, S, xpre);
                __syncthreads();
                return a;
            }
            return 0u;
        });
    // tiles of the range and of this wave's share (last < first: no units),
    // worked out once the wave's loads are done and kept before the barrier
    int b0 = u0 / S, b1 = (u1 - 1) / S;
    {
        const int wf = w0 / S;
        const int wl = w1 > w0 ? (w1 - 1) / S : wf - 1;
        if (lane == 0) {
            wtile[wave][0] = wf;
            wtile[wave][1] = wl;
        }
    }
    if (threadIdx.x < 256) red[kZeroBlock * 256 + threadIdx.x] = f4{-0.f, -0.f, -0.f, -0.f};
    asm volatile("" : "+s"(b0), "+s"(b1));
    __syncthreads();
    if (u0 >= u1) return;

    // thread: (tile phase h, row i of the lane's quad, lane l); the WAVES/4
    // groups of four waves take turns over the tiles of the range, so a
    // range with two split tiles works on both (and waits for both
    // exchanges) at the same time
    static_assert(WAVES % 4 == 0, "the epilogue takes groups of four waves");
    constexpr int kPhases = WAVES / 4;
    const int l = threadIdx.x & 63;
    const int i = (threadIdx.x >> 6) & 3;
    const int h = threadIdx.x >> 8;
    const int m = 4 * (l >> 4) + i;
    const int c = kNW * (l & 15);
    if (m >= M) return;                             // no barrier follows

    // Fixed-order sum over the waves for every tile of this range; whole
    // tiles are stored.  Without `partials`, a split tile has exactly two
    // contributors (the host keeps every range at least one tile long, or
    // makes each tile exactly two ranges), and they meet per output element
    // in the tile's exchange slots with one system-scope compare-and-swap per
    // column pair: the first deposits its partials, the second gets them
    // back, adds its own (one fp32 add each, so the result does not depend on
    // which one came first), stores y and empties the slot.  Each XCD has its
    // own L2; only system scope is coherent across them.  With `partials`
    // (tiles with more contributors), split tiles go to this workgroup's two
    // partial slots and decode_split_reduce_kernel, launched next on the same
    // stream, adds them.
    int tf[WAVES], tl[WAVES];
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
        tf[w] = wtile[w][0];
        tl[w] = wtile[w][1];
    }
    for (int tau = b0 + h; tau <= b1; tau += kPhases) {
        const int ta = tau * S, tb = ta + S;
        // every wave's part of tile tau (its segment tau - tf, or -0.0),
        // added in wave order; the reads are unconditional and issue together
        f4 rw[WAVES];
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            const int blk = tf[w] <= tau && tau <= tl[w] ? (tau - tf[w]) * WAVES + w : kZeroBlock;
            rw[w] = red[blk * 256 + l * 4 + i];
        }
        float v[kNW] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
#pragma unroll
            for (int j = 0; j < kNW; ++j) v[j] += rw[w][j];
        }
        const int n = tau * kCols + c;
        if (n >= N) continue;
        if (ta >= u0 && tb <= u1) {                 // the whole tile is here
            store_quad<BF, SILU>(y, m, N, n, v);
            continue;
        }
        if (partials) {
            float *mine = partials + ((size_t)g * 2 + (tau == b0 ? 0 : 1)) * SLOT;
            *reinterpret_cast<f4 *>(mine + m * kCols + c) = f4{v[0], v[1], v[2], v[3]};
            continue;
        }
        // the tile's later contributor: with two contributors, this workgroup
        // if the tile ends inside its range, else the next one
        const int gl = tb <= u1 ? g : g + 1;
        uint64_t *slot = slots + ((size_t)gl * 16 + m) * (kCols / 2) + c / 2;
        uint64_t got[kNW / 2];
#pragma unroll
        for (int j = 0; j < kNW / 2; ++j) {
            got[j] = 0;
            const uint64_t mine = (uint64_t)slot_code(v[2 * j]) | ((uint64_t)slot_code(v[2 * j + 1]) << 32);
            __hip_atomic_compare_exchange_strong(slot + j, &got[j], mine, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        }
        // per column pair (the two contributors' exchanges may interleave):
        // an empty slot means this one came first and deposited its values
#pragma unroll
        for (int j = 0; j < kNW / 2; ++j) {
            if (got[j] == 0) continue;
            const float r0 = __builtin_bit_cast(float, (uint32_t)got[j] ^ kSlotKey) + v[2 * j];
            const float r1 = __builtin_bit_cast(float, (uint32_t)(got[j] >> 32) ^ kSlotKey) + v[2 * j + 1];
            __hip_atomic_store(slot + j, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            store_pair<BF, SILU>(y, m, N, n + 2 * j, r0, r1);
        }
    }
}

// Adds the partials of every split tile of a stream-K launch of G workgroups
// that used partial slots, in workgroup order (fixed, so results are
// bit-reproducible), and stores y.  One workgroup per tile; thread (m, q)
// handles row m and columns 4q .. 4q+3 of the tile.  Tiles that lie whole
// inside one range were stored by the stream-K kernel.
template <bool BF, bool SILU>
__global__ __launch_bounds__(256) void decode_split_reduce_kernel(
    const float *__restrict__ partials, uint16_t *__restrict__ y, int M, int N, int S, int G) {
    constexpr int SLOT = 16 * kCols;
    const int T = (N + kCols - 1) / kCols;
    const StreamK sk{T * S, G};
    const int tau = blockIdx.x;
    const int gf = sk.owner(tau * S), gl = sk.owner(tau * S + S - 1);
    if (gf == gl) return;
    const int m = threadIdx.x >> 4, q = threadIdx.x & 15;
    const int n = tau * kCols + kNW * q;
    if (m >= M || n >= N) return;
    float r[kNW] = {0.f, 0.f, 0.f, 0.f};
    for (int h = gf; h <= gl; ++h) {
        const int hs = tau == sk.begin(h) / S ? 0 : 1;
        const f4 p = *reinterpret_cast<const f4 *>(partials + ((size_t)h * 2 + hs) * SLOT +
                                                   m * kCols + kNW * q);
#pragma unroll
        for (int j = 0; j < kNW; ++j) r[j] += p[j];
    }
    store_quad<BF, SILU>(y, m, N, n, r);
}

// ---------------------------------------------------------------------------

#ifndef W4A16_DECODE_WAVES
#define W4A16_DECODE_WAVES 8
#endif
#ifndef W4A16_DECODE_D
#define W4A16_DECODE_D 6
#endif

constexpr int kDecWaves = W4A16_DECODE_WAVES;
constexpr int kDecD = W4A16_DECODE_D;

static size_t slots_bytes(int capacity) { return (size_t)capacity * 16 * (kCols / 2) * sizeof(uint64_t); }

size_t decode_workspace_bytes(int capacity) {
    return slots_bytes(capacity) + (size_t)capacity * 2 * 16 * kCols * sizeof(float);
}

// Stream-K launches whose tiles may have more than two contributors (more
// ranges than 2T) use partial slots and the reduce kernel; so do batches of
// 15 or 16 rows, where the exchange's compare-and-swaps (one per row and
// column pair) cost more than the second kernel (measured at M = 16: -0.7
// us on K = 5120, N = 17408 and -1.5 us on N = 27648; at M = 12 +0.25 us).
// The other launches use the exchange slots.
constexpr int kPartialsMinM = 15;
static bool uses_partials(int grid, int T, int M) { return grid > 2 * T || M >= kPartialsMinM; }

// With fewer than half as many tiles as CUs, batches above two rows spread
// over every CU (a tile then has several contributors) when K is long: the
// work per range is then large enough that the extra CUs outweigh the second
// kernel.  Measured on N = 5120 (80 tiles): a gain from S = 432 at M = 4 and
// from S = 256 at M = 16, a loss at S = 256, M = 4 and none at S = 128.
static bool spread_wide(int64_t M, int64_t S) { return M > 2 && (S >= 384 || (M >= 8 && S >= 256)); }

// Stream-K grid, or 0 for the tiles kernel.  Every tile must have at most two
// contributors: either every range holds at least one tile (G <= T), or
// G = 2T and each tile is exactly two ranges.
int decode_streamk_grid(const LinearArgs &a, int num_cus) {
    const int64_t S = (a.K + 31) / 32;
    const int64_t T = (a.N + kCols - 1) / kCols;
    // the kernels compute ranges in 32-bit arithmetic (units times grid)
    if (T * S * (int64_t)num_cus >= ((int64_t)1 << 32)) return 0;
    if (T >= num_cus) {
        // every wave's share of a range must be at most S units, so that it
        // meets at most two tiles
        if (T > (int64_t)kDecWaves * num_cus) return 0;
        const int nmax = (int)((T * S + num_cus - 1) / num_cus);
        for (int n = nmax - 1; n <= nmax; ++n)      // the two range lengths
            for (int w = 0; w < kDecWaves; ++w)
                if (wave_share<kDecWaves>(n, w + 1) - wave_share<kDecWaves>(n, w) > S) return 0;
        return num_cus;
    }
    // G > 2T: partial slots (a tile may have more than two contributors)
    if (2 * T < num_cus && spread_wide(a.M, S)) return num_cus;
    if (2 * T <= num_cus && S >= 2) return (int)(2 * T);
    return (int)T;
}

// Activations are staged in LDS when they fit in this many bytes.
constexpr size_t kXStageMax = 64 * 1024;

// Static LDS of a kernel, read once from its attributes.
static size_t static_lds(const void *kernel) {
    hipFuncAttributes attr;
    if (hipFuncGetAttributes(&attr, kernel) != hipSuccess) return (size_t)-1;
    return attr.sharedSizeBytes;
}

template <int SCALE, bool XLDS, bool BF, bool SILU>
static hipError_t launch_sa(const LinearArgs &a, hipStream_t stream, void *workspace,
                            int capacity, int grid) {
    const int K = (int)a.K, N = (int)a.N, M = (int)a.M;
    const int S = (K + 31) / 32;
    int group_steps = 0;
    if (SCALE != 0) group_steps = a.group_size == -1 ? S : (int)a.group_size / 32;
    const void *xp = a.x;
    const void *qp = a.qweight;
    const void *sp = a.scales;
    void *yp = a.y;
    const dim3 block(kDecWaves * 64);
    const size_t dyn = XLDS ? (size_t)M * 32 * S * 2 + 16 : 0;
    if (grid > 0) {
        char *ws = static_cast<char *>(workspace);
        uint64_t *slots = reinterpret_cast<uint64_t *>(ws);
        const int T = (N + kCols - 1) / kCols;
        const bool part = uses_partials(grid, T, M);
        float *partials = part ? reinterpret_cast<float *>(ws + slots_bytes(capacity)) : nullptr;
        void *args[] = {&xp, &qp, &sp, &yp, (void *)&M, (void *)&K, (void *)&N,
                        &group_steps, &slots, &partials};
        hipError_t e = hipLaunchKernel(
            reinterpret_cast<const void *>(
                &decode_streamk_kernel<kDecWaves, kDecD, SCALE, XLDS, BF, SILU>),
            dim3(grid), block, args, dyn, stream);
        if (e != hipSuccess || !part) return e;
        const float *pc = partials;
        int Sv = S, G = grid;
        void *rargs[] = {&pc, &yp, (void *)&M, (void *)&N, &Sv, &G};
        return hipLaunchKernel(reinterpret_cast<const void *>(&decode_split_reduce_kernel<BF, SILU>),
                               dim3((unsigned)T), dim3(256), rargs, 0, stream);
    }
    void *args[] = {&xp, &qp, &sp, &yp, (void *)&M, (void *)&K, (void *)&N, &group_steps};
    const unsigned tiles = (unsigned)((N + kCols - 1) / kCols);
    return hipLaunchKernel(
        reinterpret_cast<const void *>(
            &decode_tiles_kernel<kDecWaves, kDecD, SCALE, XLDS, BF, SILU>),
        dim3(tiles), block, args, dyn, stream);
}

// Whether the activations can be staged in LDS: at most kXStageMax bytes,
// and the kernel's static LDS plus the staging area within the device's
// per-workgroup LDS limit (a launch beyond it is rejected by the device).
template <int SCALE, bool BF>
static bool stage_fits(const LinearArgs &a, int grid, size_t max_lds) {
    const size_t dyn = (size_t)a.M * 32 * ((a.K + 31) / 32) * 2 + 16;
    if (dyn > kXStageMax) return false;
    static const size_t sk_static = static_lds(reinterpret_cast<const void *>(
        &decode_streamk_kernel<kDecWaves, kDecD, SCALE, true, BF, false>));
    static const size_t tiles_static = static_lds(reinterpret_cast<const void *>(
        &decode_tiles_kernel<kDecWaves, kDecD, SCALE, true, BF, false>));
    const size_t st = grid > 0 ? sk_static : tiles_static;
    return st != (size_t)-1 && st + dyn <= max_lds;
}

template <int SCALE, bool BF>
static hipError_t launch_scale(const LinearArgs &a, hipStream_t stream, void *workspace,
                               int capacity, int grid, size_t max_lds) {
    const bool xlds = stage_fits<SCALE, BF>(a, grid, max_lds);
    if (a.silu)
        return xlds ? launch_sa<SCALE, true, BF, true>(a, stream, workspace, capacity, grid)
                    : launch_sa<SCALE, false, BF, true>(a, stream, workspace, capacity, grid);
    return xlds ? launch_sa<SCALE, true, BF, false>(a, stream, workspace, capacity, grid)
                : launch_sa<SCALE, false, BF, false>(a, stream, workspace, capacity, grid);
}

hipError_t launch_decode(const LinearArgs &a, hipStream_t stream, void *workspace, int capacity,
                         int grid, size_t max_lds) {
    if (grid > capacity) return hipErrorInvalidValue;
    // bfloat16: SCALE 0 dequantises before the MFMA (g = 16); 1 and 2 sum
    // 128 + q and fold the offset out per group (2: one step per group)
    const int64_t S = (a.K + 31) / 32;
    // one 32-deep step per group: g = 32, or one group over K <= 32
    const bool one_step = a.group_size == 32 || (a.group_size == -1 && S == 1);
    if (a.bf16) {
        if (a.group_size == 16) return launch_scale<0, true>(a, stream, workspace, capacity, grid, max_lds);
        if (one_step) return launch_scale<2, true>(a, stream, workspace, capacity, grid, max_lds);
        return launch_scale<1, true>(a, stream, workspace, capacity, grid, max_lds);
    }
    if (a.group_size == 16) return launch_scale<0, false>(a, stream, workspace, capacity, grid, max_lds);
    if (one_step) return launch_scale<2, false>(a, stream, workspace, capacity, grid, max_lds);
    return launch_scale<1, false>(a, stream, workspace, capacity, grid, max_lds);
}

}  // namespace w4a16
