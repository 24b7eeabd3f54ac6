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
    u4 w;       // qweight words of the lane's 4 consecutive columns
    u4 x;       // 8 activations of this lane's A row / K block (unused when staged in LDS)
    u2 s;       // the 4 columns' fp16 scales
    uint32_t z; // with stored zero points: the qzeros word holding the 4 columns' nibbles
};

// Activations staged in LDS: rows m < M of x over the S steps from step s0
// (K indices 32 s0 .. 32 (s0 + S) - 1), each row zero-padded to Kp = 32*S
// halves and already in unpack order (perm_x per 16-byte chunk), followed by
// one zero chunk that the lanes of rows m >= M read.  Staging is split in
// two so that the first kXPre chunks of each thread are requested before the
// weight prologue (they would otherwise queue behind it): stage_x_issue loads
// them, stage_x_finish stores them and any further chunks and returns this
// lane's byte address of step s0.
constexpr int kXPre = 2;

struct XPre {
    u4 v[kXPre];
};

__device__ __forceinline__ u4 stage_x_load(const __amdgpu_buffer_rsrc_t xr, int c, int K,
                                           int chunks_per_row, int k0) {
    const int m = c / chunks_per_row;
    const int k = k0 + 8 * (c - m * chunks_per_row);
    return load_b128(xr, k < K ? ((uint32_t)m * (uint32_t)K + (uint32_t)k) * 2u : kOOB);
}

__device__ __forceinline__ XPre stage_x_issue(const __amdgpu_buffer_rsrc_t xr, int M, int K,
                                              int S, int s0 = 0) {
    const int chunks_per_row = 4 * S;
    const int total = M * chunks_per_row;
    XPre pre;
#pragma unroll
    for (int r = 0; r < kXPre; ++r) {
        const int c = threadIdx.x + r * blockDim.x;
        pre.v[r] = stage_x_load(xr, c < total ? c : 0, K, chunks_per_row, 32 * s0);
    }
    return pre;
}

__device__ __forceinline__ uint32_t stage_x_finish(unsigned char *xs,
                                                   const __amdgpu_buffer_rsrc_t xr, int M, int K,
                                                   int S, const XPre &pre, int s0 = 0) {
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
        put(c, stage_x_load(xr, c, K, chunks_per_row, 32 * s0));
    if (threadIdx.x == 0) *reinterpret_cast<u4 *>(xs + (size_t)M * Kp * 2) = u4{0u, 0u, 0u, 0u};
    const int lane = threadIdx.x & 63;
    const int m = lane & 15, kb = lane >> 4;
    return m < M ? (uint32_t)(((size_t)m * Kp + 8 * kb) * 2) : (uint32_t)((size_t)M * Kp * 2);
}

__device__ __forceinline__ _Float16 scale_at(const u2 &s, int j) {
    const uint32_t d = j < 2 ? s.x : s.y;
    return (j & 1) ? half_hi(d) : half_lo(d);
}

// Scale j of the lane's quad as fp32 (exact): bfloat16 when SB, else fp16.
template <bool SB>
__device__ __forceinline__ float scale_f32(const u2 &s, int j) {
    const uint32_t d = j < 2 ? s.x : s.y;
    return (j & 1) ? hi_f32<SB>(d) : lo_f32<SB>(d);
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
// of step xstep0, the first staged step, and ends with a workgroup barrier;
// ranges that meet two tiles stage from step 0); otherwise from global.
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
// ZP: stored zero points (qzeros int32 [G, N/8], nibble j of word c = column
// 8c + j): w = (q - z) s.  Since (q - z) s = (q - 8) s + (8 - z) s, the
// symmetric sums run unchanged and one more MFMA per unit sums x itself
// (B = 1) over the group; at the group's end acc += s (8 - z) * (that sum) per
// column, in fp32.  With every z = 8 the added term is 0.  For SCALE 0 (two
// groups in a unit) the zero point enters the dequantised weight instead: fp16
// adds 8 - z to the exact q - 8 before the scale, bfloat16 takes -z s as the
// offset of its fma.  z is the stored nibble plus a bias (0 for the v2 form,
// 1 for the v1 form): z8 = 8 - bias, and 8 - z = z8 - nibble.
// SB: bfloat16 scales (with BF only), taken to fp32 exactly wherever the
// bfloat16 paths take an fp16 scale to fp32.
template <int D, int SCALE, bool XLDS, bool BF, bool ZP, bool SB, typename Dump,
          typename AfterPrologue, typename BeforeTail>
__device__ __forceinline__ void decode_units(
    const __amdgpu_buffer_rsrc_t xr, const __amdgpu_buffer_rsrc_t qr,
    const __amdgpu_buffer_rsrc_t sr, const __amdgpu_buffer_rsrc_t zr, int z8,
    const unsigned char *xs,
    int M, int K, int N, int S,
    int group_steps, int w0, int w1, Dump &&dump, AfterPrologue &&after_prologue,
    BeforeTail &&before_tail, int xstep0 = 0) {
    constexpr bool SCALE_AFTER = SCALE != 0;
    static_assert(BF || !SB, "bfloat16 scales come with bfloat16 activations");
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
        // the qzeros word of the same group row: byte (row N / 2 + col / 2) rounded
        // down to a word, i.e. the scale offset / 4 (N % 8 == 0)
        if constexpr (ZP) st.z = __builtin_amdgcn_raw_buffer_load_b32(zr, (s_off >> 2) & ~3u, 0, 0);
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

    f4 acc[kNW], accg[kNW], accx = f4{0.f, 0.f, 0.f, 0.f}, accz = f4{0.f, 0.f, 0.f, 0.f};
    const uint32_t zsh = 16u * (uint32_t)(c16 & 1);   // the lane's 4 nibbles in the qzeros word
    // 1.0 in both halves of each dword, in the activation type (B of the x sums)
    const u4 ones = BF ? u4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u}
                       : u4{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
    // zero point of column j of the lane's quad, as 8 - z
    auto zdiff = [&](const Stage<XLDS> &st, int j) -> int {
        return z8 - (int)((st.z >> (zsh + 4u * (uint32_t)j)) & 15u);
    };
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
    uint32_t xl = xl0 + xl_inc * (uint32_t)(tA0 - xstep0);   // staged from step xstep0

    int i = 0, pos = SCALE_AFTER ? tA0 % group_steps : 0;
    // one unit of math on ring stage st (unit index i of this wave)
    auto compute = [&](Stage<XLDS> &st) {
        h8 a;
        if constexpr (XLDS)
            a = __builtin_bit_cast(h8, *reinterpret_cast<const u4 *>(xs + xl));
        else
            a = __builtin_bit_cast(h8, perm_x(st.x));
        const bool seg_end = i == nA - 1 || i == n - 1;
        const f4 zero = {0.f, 0.f, 0.f, 0.f};
        if constexpr (BF && SCALE == 0) {
#pragma unroll
            for (int j = 0; j < kNW; ++j) {
                const float sj = scale_f32<SB>(st.s, j);
                const float zoff = ZP ? (float)(zdiff(st, j) - 8) * sj : -8.0f * sj;   // -z s
                acc[j] = mfma16x16x32_t<true>(__builtin_bit_cast(u4, a),
                                              dequant_bf16<false>(st.w[j], sj, zoff), acc[j]);
            }
        } else if constexpr (BF && SCALE == 2) {
            // one step per group: both sums start from zero in the MFMA and go
            // straight into acc (no accumulators to reset)
            const u4 b136 = {0x43084308u, 0x43084308u, 0x43084308u, 0x43084308u};   // bf16 136.0
            const f4 tx = mfma16x16x32_t<true>(__builtin_bit_cast(u4, a), b136, zero);
            f4 tz = zero;
            if constexpr (ZP) tz = mfma16x16x32_t<true>(__builtin_bit_cast(u4, a), ones, zero);
#pragma unroll
            for (int j = 0; j < kNW; ++j) {
                const f4 t = mfma16x16x32_t<true>(__builtin_bit_cast(u4, a), codes128_bf16(st.w[j], uc),
                                                  zero);
                const float sj = scale_f32<SB>(st.s, j);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[j][e] = __builtin_fmaf(sj, t[e] - tx[e], acc[j][e]);
                if constexpr (ZP) {
                    const float cj = sj * (float)zdiff(st, j);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[j][e] = __builtin_fmaf(cj, tz[e], acc[j][e]);
                }
            }
        } else if constexpr (BF) {
            const u4 b136 = {0x43084308u, 0x43084308u, 0x43084308u, 0x43084308u};   // bf16 136.0
#pragma unroll
            for (int j = 0; j < kNW; ++j)
                accg[j] = mfma16x16x32_t<true>(__builtin_bit_cast(u4, a), codes128_bf16(st.w[j], uc),
                                               accg[j]);
            accx = mfma16x16x32_t<true>(__builtin_bit_cast(u4, a), b136, accx);
            if constexpr (ZP) accz = mfma16x16x32_t<true>(__builtin_bit_cast(u4, a), ones, accz);
            if (pos == group_steps - 1 || seg_end) {
#pragma unroll
                for (int j = 0; j < kNW; ++j) {
                    const float sj = scale_f32<SB>(st.s, j);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[j][e] = __builtin_fmaf(sj, accg[j][e] - accx[e], acc[j][e]);
                    if constexpr (ZP) {
                        const float cj = sj * (float)zdiff(st, j);
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[j][e] = __builtin_fmaf(cj, accz[e], acc[j][e]);
                    }
                    accg[j] = zero;
                }
                accx = zero;
                accz = zero;
            }
            pos = (pos + 1 == group_steps) ? 0 : pos + 1;
        } else if constexpr (SCALE == 2) {
            f4 tz = zero;
            if constexpr (ZP) tz = mfma16x16x32_t<false>(__builtin_bit_cast(u4, a), ones, zero);
#pragma unroll
            for (int j = 0; j < kNW; ++j) {
                const f4 t = mfma16x16x32(a, unpack_codes(st.w[j], uc), zero);
                const float sj = scale_f32<SB>(st.s, j);
                acc[j] += sj * t;
                if constexpr (ZP) acc[j] += (sj * (float)zdiff(st, j)) * tz;
            }
        } else if constexpr (SCALE_AFTER) {
#pragma unroll
            for (int j = 0; j < kNW; ++j)
                accg[j] = mfma16x16x32(a, unpack_codes(st.w[j], uc), accg[j]);
            if constexpr (ZP) accz = mfma16x16x32_t<false>(__builtin_bit_cast(u4, a), ones, accz);
            if (pos == group_steps - 1 || seg_end) {
#pragma unroll
                for (int j = 0; j < kNW; ++j) {
                    const float sj = scale_f32<SB>(st.s, j);
                    acc[j] += sj * accg[j];
                    if constexpr (ZP) acc[j] += (sj * (float)zdiff(st, j)) * accz;
                    accg[j] = zero;
                }
                accz = zero;
            }
            pos = (pos + 1 == group_steps) ? 0 : pos + 1;
        } else {
#pragma unroll
            for (int j = 0; j < kNW; ++j) {
                h8 wq = unpack_codes(st.w[j], uc);                 // q - 8, exact
                if constexpr (ZP) {                                // q - z, exact
                    const _Float16 d = (_Float16)zdiff(st, j);
                    wq += h8{d, d, d, d, d, d, d, d};
                }
                const _Float16 sj = scale_at(st.s, j);
                acc[j] = mfma16x16x32(a, wq * h8{sj, sj, sj, sj, sj, sj, sj, sj}, acc[j]);
            }
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
    // last, partial round (its loads are all in flight: before_tail may add
    // loads of its own, which the round does not wait for)
    before_tail();
#pragma unroll
    for (int u = 0; u < D; ++u) {
        if (i < n) compute(ring[u]);
    }
}

// ---------------------------------------------------------------------------
// Dynamic LDS: the staged activations (XLDS) follow the static arrays.
extern __shared__ __attribute__((aligned(16))) unsigned char decode_dyn_lds[];

// Static LDS of the two kernels (bytes), for the budget check at the launch
// parameters below: the tiles kernel's wave partials, and the stream-K
// kernel's partial blocks (two segments per wave plus the -0.0 block) with
// each wave's tile bounds.
constexpr size_t tiles_static_lds(int waves) { return (size_t)waves * kNW * 64 * sizeof(f4); }
constexpr size_t streamk_static_lds(int waves) {
    return (size_t)(2 * waves + 1) * 256 * sizeof(f4) + (size_t)waves * 2 * sizeof(int) +
           4 * sizeof(int);
}

// ---------------------------------------------------------------------------
// LoRA adapter term inside the stream-K launch (LoraTerm, LK).
//
// Workgroups g < Su also own shrink unit g: each of their waves adds x . A^T
// over one 32-deep K step on the matrix cores (the loads issued ahead of the
// weight prologue, so the step waits for them only), and their last wave
// adds the eight wave partials in wave order and stores slab g
// into the slab words of the decode workspace, each value coded so that it
// is never zero (as the exchange slots code theirs).  After its main loop
// every workgroup reads all slab words (M r Su of them), waiting until none
// is zero: the owners of the units are the first workgroups of the grid,
// which the device starts first, and they wait on nothing, so the words come;
// the wait is bounded all the same, so every wave ends.  It adds each entry's
// slabs in slab order, rounds scale * t to the activation type (t' in LDS),
// and runs t' . B^T on the matrix cores with each tile it stores.  The
// workgroup that counts itself out last zeroes the words for the next launch.
// Each XCD has its own L2, so the words and the count move only through
// system-scope atomic loads and stores, which bypass it.
constexpr int kLoraStageChunks = 1024;           // 16 KiB: two chunks per thread of 512
constexpr size_t kLoraStageBytes = (size_t)kLoraStageChunks * 16;
constexpr int kLoraSpinMax = 1 << 24;            // waits of about 0.2 us: a few seconds

// This wave's shrink step (K step st of unit g, or none): x rows (A operand)
// and rows j of A (B operand) for the two 64-column passes.
struct LoraStep {
    u4 x;
    u4 a[2][4];
};

__device__ __forceinline__ LoraStep lora_step_issue(const LoraTerm &L, const __amdgpu_buffer_rsrc_t xr,
                                                    int M, int K, int st, bool own) {
    const int lane = threadIdx.x & 63, c16 = lane & 15, kb = lane >> 4;
    const auto ar = make_rsrc(L.A, (uint32_t)L.r * (uint32_t)K * 2u);
    const int k = 32 * st + 8 * kb;
    const bool in = own && k < K;               // K % 16 == 0: eight in or eight out
    LoraStep o;
    o.x = load_b128(xr, (in && c16 < M) ? (uint32_t)(c16 * K + k) * 2u : kOOB);
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
            const int j = 64 * p + 16 * jb + c16;
            o.a[p][jb] = load_b128(ar, (in && j < L.r) ? (uint32_t)(j * K + k) * 2u : kOOB);
        }
    return o;
}

// The step's products, rows m < M of this wave's partial into part[w][m][j]
// (LDS, fp32, [WAVES][M][r]).
template <bool BF>
__device__ __forceinline__ void lora_step_finish(float *part, const LoraTerm &L, const LoraStep &o,
                                                 int M, int wave) {
    const int lane = threadIdx.x & 63, c16 = lane & 15, kb = lane >> 4;
    const f4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        if (64 * p >= L.r) break;
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
            const f4 d = mfma16x16x32_t<BF>(o.x, o.a[p][jb], zero);
            const int j = 64 * p + 16 * jb + c16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = 4 * kb + e;
                if (m < M && j < L.r) part[(wave * M + m) * L.r + j] = d[e];
            }
        }
    }
}

// One wave, after a barrier that follows every wave's lora_step_finish: slab
// g = the wave partials added in wave order; publish it; the last unit's
// wave forms t' and sets the flag.
template <typename T>
__device__ __forceinline__ T sys_load(const T *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
template <typename T>
__device__ __forceinline__ void sys_store(T *p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// A slab value as a word that is never zero (NaN made canonical, then XOR
// with a NaN pattern), and back.
constexpr uint32_t kLoraKey = 0x7FBADBADu;
__device__ __forceinline__ uint32_t lora_code(float v) {
    return (v != v ? 0x7FC00000u : __builtin_bit_cast(uint32_t, v)) ^ kLoraKey;
}
__device__ __forceinline__ float lora_decode(uint32_t w) { return __builtin_bit_cast(float, w ^ kLoraKey); }

// One wave, after a barrier that follows every wave's lora_step_finish: slab
// g = the wave partials added in wave order, stored as coded words.
template <int WAVES>
__device__ __forceinline__ void lora_publish(const float *part, const LoraTerm &L, int M, int g) {
    const int lane = threadIdx.x & 63;
    const int total = M * L.r;
    unsigned *words = L.area + 64;
    for (int idx = lane; idx < total; idx += 64) {
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) acc += part[w * total + idx];
        sys_store(words + (size_t)g * total + idx, lora_code(acc));
    }
}

// Every slab value into `vals` (LDS, [Su][M r] fp32), once every word is
// set: thread t reads words t, t + 512, ... (at most eight; lora_words_issue
// requests them as soon as the thread's main loop ends), then again after a
// short sleep while any is zero, within a bounded number of rounds.  The
// values are visible to the workgroup after the next barrier.
struct LoraWords {
    uint32_t w[8];
};

__device__ __forceinline__ LoraWords lora_words_issue(const LoraTerm &L, int M) {
    const unsigned *words = L.area + 64;
    const int nw = L.Su * M * L.r;              // <= kLoraMaxSlabReads = 8 * 512
    LoraWords o;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int v = (int)threadIdx.x + 512 * k;
        o.w[k] = v < nw ? sys_load(words + v) : 1u;
    }
    return o;
}

__device__ __forceinline__ void lora_gather(float *vals, LoraWords o, const LoraTerm &L, int M) {
    const int nw = L.Su * M * L.r;
    for (int it = 0; it < kLoraSpinMax; ++it) {
        bool all = true;
#pragma unroll
        for (int k = 0; k < 8; ++k) all = all && o.w[k] != 0u;
        if (all) break;
        __builtin_amdgcn_s_sleep(8);
        o = lora_words_issue(L, M);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int v = (int)threadIdx.x + 512 * k;
        if (v < nw) vals[v] = lora_decode(o.w[k]);
    }
}

// Workgroup barrier for LDS traffic only: this wave's LDS operations complete
// first, its global loads and atomics may stay in flight across it.
__device__ __forceinline__ void lds_sync() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0) only
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// t'[e] = round(scale * sum of the Su slabs of entry e, in slab order) into
// ta (LDS, activation type) and, when tq is given, into tq as well.
template <bool BF>
__device__ __forceinline__ void lora_form_t(uint16_t *ta, uint16_t *tq, const float *vals,
                                            const LoraTerm &L, int M) {
    const int total = M * L.r;
    for (int e = threadIdx.x; e < total; e += blockDim.x) {
        float acc = 0.f;
        for (int q0 = 0; q0 < L.Su; q0 += 8) {      // eight reads in flight
            float pv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) pv[u] = q0 + u < L.Su ? vals[(q0 + u) * total + e] : 0.f;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (q0 + u < L.Su) acc += pv[u];
        }
        const uint16_t t = (uint16_t)pack2<BF>(L.scale * acc, 0.f);
        ta[e] = t;
        if (tq) tq[e] = t;
    }
}

// The workgroup counted out last (exits + 1 == grid, in `last`) zeroes the
// slab words and the count: by then every workgroup has read every word.
// After a barrier that makes `last` visible.
__device__ __forceinline__ void lora_reset(const LoraTerm &L, int M, bool last) {
    if (!last) return;
    unsigned *words = L.area + 64;
    const int nw = L.Su * M * L.r;
    for (int v = threadIdx.x; v < nw; v += blockDim.x) sys_store(words + v, 0u);
    if (threadIdx.x == 0) sys_store(L.area, 0u);
}

// Rows of B for the workgroup's first tiles, staged through registers: two
// 16-byte chunks per thread (past the staged rows: zero, no memory access),
// requested with the first weight loads and written to LDS after the main loop.
struct LoraBStage {
    u4 v[2];
    int nb;     // tiles staged, from the range's first tile
};

__device__ __forceinline__ LoraBStage lora_b_issue(const LoraTerm &L, int N, int b0, int ntiles) {
    const auto br = make_rsrc(L.B, (uint32_t)N * (uint32_t)L.r * 2u);
    const int cb = 8 * L.r;                     // chunks per tile: 64 rows of r
    LoraBStage o;
    o.nb = min(ntiles, kLoraStageChunks / cb);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = (int)threadIdx.x + 512 * i;
        const int t = c / cb, w = c - t * cb;
        const int n = (b0 + t) * kCols + w / (L.r / 8), j0 = 8 * (w % (L.r / 8));
        o.v[i] = load_b128(br, (t < o.nb && n < N) ? (uint32_t)(n * L.r + j0) * 2u : kOOB);
    }
    return o;
}

// The term for one tile on the matrix cores, in the layout of the wave sums:
// d[j][e] = sum_j' t'[m][j'] B[n][j'] for row m = 4 (lane / 16) + e and
// column n = tile * 64 + 4 (lane % 16) + j (MFMA j takes the columns 4 c + j,
// as the weight sums do).  A: t' rows (zero past M); B: the staged rows of
// the tile (`bl`, row pitch r) or global.  Every lane of the wave takes part.
// A fragments of t' (LDS, [M][r]) for the K steps of the term (r <= 128:
// four): lane (m = lane % 16, block lane / 16) holds t'[m][32 s + 8 (lane /
// 16) ..+8], zero past M and r.
struct LoraTFrag {
    u4 a[kLoraMaxRank / 32];
};

__device__ __forceinline__ LoraTFrag lora_t_frags(const uint16_t *ta, const LoraTerm &L, int M) {
    const int lane = threadIdx.x & 63, c16 = lane & 15, kb = lane >> 4;
    LoraTFrag f;
#pragma unroll
    for (int s = 0; s < kLoraMaxRank / 32; ++s) {
        const int k = 32 * s + 8 * kb;
        f.a[s] = (c16 < M && k < L.r) ? *reinterpret_cast<const u4 *>(ta + c16 * L.r + k)
                                      : u4{0u, 0u, 0u, 0u};
    }
    return f;
}

template <bool BF>
__device__ __forceinline__ void lora_tile_delta(f4 (&d)[kNW], const LoraTFrag &tf,
                                                const LoraTerm &L, int N, int tile,
                                                const uint16_t *bl) {
    const int lane = threadIdx.x & 63, c16 = lane & 15, kb = lane >> 4;
    const auto br = make_rsrc(L.B, (uint32_t)N * (uint32_t)L.r * 2u);
    const u4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < kNW; ++j) d[j] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kLoraMaxRank / 32; ++s) {
        const int j1 = 32 * s;
        if (j1 >= L.r) break;
        const int k = j1 + 8 * kb;
        const bool kin = k < L.r;               // r % 8 == 0: eight in or eight out
        const u4 a = tf.a[s];
        u4 b[kNW];
#pragma unroll
        for (int j = 0; j < kNW; ++j) {
            const int col = kNW * c16 + j;
            const int n = tile * kCols + col;
            if (bl)
                b[j] = kin ? *reinterpret_cast<const u4 *>(bl + col * L.r + k) : zero;
            else
                b[j] = load_b128(br, (kin && n < N) ? (uint32_t)(n * L.r + k) * 2u : kOOB);
        }
#pragma unroll
        for (int j = 0; j < kNW; ++j) d[j] = mfma16x16x32_t<BF>(a, b[j], d[j]);
    }
}

// v[c] += sum_j t'[m][j] B[n + c][j] for the four columns n .. n + 3, j
// ascending, t' from `tl` (fp32 values of the activation type, [M][r]); for
// the reduce kernel (one thread per row and four columns).
template <bool BF>
__device__ __forceinline__ void lora_add4(float (&v)[kNW], const float *tl, const LoraTerm &L,
                                          int m, int n, int N) {
    const auto br = make_rsrc(L.B, (uint32_t)N * (uint32_t)L.r * 2u);
    const float *trow = tl + m * L.r;
    for (int j0 = 0; j0 < L.r; j0 += 8) {
        u4 b[kNW];
#pragma unroll
        for (int c = 0; c < kNW; ++c) b[c] = load_b128(br, (uint32_t)((n + c) * L.r + j0) * 2u);
#pragma unroll
        for (int c = 0; c < kNW; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[c] = __builtin_fmaf(trow[j0 + 2 * e], lo_f32<BF>(b[c][e]), v[c]);
                v[c] = __builtin_fmaf(trow[j0 + 2 * e + 1], hi_f32<BF>(b[c][e]), v[c]);
            }
    }
}

// Dynamic LDS of the stream-K kernel: the staged activations, then (LK) a
// 16 KiB area that holds in turn the wave partials of the shrink step (M r
// <= kLoraMaxMR floats per wave) and the slab values (Su M r <= 4096
// floats), a 16 KiB area for the staged rows of B, and t' (M r <=
// kLoraMaxMR 16-bit values).
__host__ __device__ constexpr size_t lora_lds_offset(bool xlds, int M, int S) {
    return xlds ? (size_t)M * 32 * S * 2 + 16 : 0;
}
constexpr size_t kLoraLdsBytes = 2 * kLoraStageBytes + 2 * (size_t)kLoraMaxMR;
static_assert(8 * kLoraMaxMR * 4 <= kLoraStageBytes, "wave partials fit the LoRA LDS area");
static_assert(4 * kLoraMaxSlabReads <= kLoraStageBytes, "slab values fit the LoRA LDS area");

// Tiles kernel: one workgroup per column tile, its waves split K.
template <int WAVES, int D, int SCALE, bool XLDS, bool BF, bool SILU, bool ZP, bool SB>
__global__ __launch_bounds__(WAVES * 64) void decode_tiles_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, const int32_t *__restrict__ qzeros,
    uint16_t *__restrict__ y, int M, int K, int N,
    int group_steps, int z8) {
    __shared__ f4 red[WAVES][kNW][64];
    static_assert(sizeof(red) == tiles_static_lds(WAVES), "tiles kernel LDS layout");

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
    const auto zr = make_rsrc(qzeros, ZP ? (uint32_t)G * (uint32_t)N / 2u : 0u);

#pragma unroll
    for (int j = 0; j < kNW; ++j) red[wave][j][lane] = f4{0.f, 0.f, 0.f, 0.f};
    XPre xpre;
    if constexpr (XLDS) xpre = stage_x_issue(xr, M, K, S);
    __builtin_amdgcn_sched_barrier(0);
    decode_units<D, SCALE, XLDS, BF, ZP, SB>(
        xr, qr, sr, zr, z8, decode_dyn_lds, M, K, N, S, group_steps, w0, w1,
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
        },
        [] {});
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

// LK: the LoRA adapter term in the same launch (LoraTerm; SILU and ZP off).
template <int WAVES, int D, int SCALE, bool XLDS, bool BF, bool SILU, bool ZP, bool SB, bool LK>
__global__ __launch_bounds__(WAVES * 64) void decode_streamk_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, const int32_t *__restrict__ qzeros,
    uint16_t *__restrict__ y, int M, int K, int N,
    int group_steps, int z8, uint64_t *__restrict__ slots, float *__restrict__ partials,
    LoraTerm lora) {
    constexpr int SLOT = 16 * kCols;             // floats per partial slot
    // Wave partials: block s*WAVES + w (256 f4: [lane][i]) holds wave w's
    // sums of its segment s, row i of the lane's quad, its four columns
    // together (one 16-byte read back); block 2*WAVES holds -0.0, which
    // leaves any fp32 sum unchanged when added (the stand-in for a wave that
    // has no part of a tile, so the reduction reads without branches).
    constexpr int kZeroBlock = 2 * WAVES;
    __shared__ f4 red[(2 * WAVES + 1) * 256];
    __shared__ int wtile[WAVES][2];              // each wave's first and last tile
    __shared__ int lk_last[4];                   // LK: this workgroup counted out last
    static_assert(sizeof(red) + sizeof(wtile) + sizeof(lk_last) == streamk_static_lds(WAVES),
                  "stream-K kernel LDS layout");
    static_assert(!LK || (!SILU && !ZP), "the adapter term goes with the plain linear");

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = (K + 31) >> 5;
    const int T = (N + kCols - 1) / kCols;
    const StreamK sk{T * S, (int)gridDim.x};
    // three contributors per tile (each range a third of one tile)
    const bool three = partials == nullptr && (int)gridDim.x == 3 * T;
    // LK: the first Su workgroups also own a shrink unit
    const int g = blockIdx.x;
    const bool unit = LK && g < lora.Su;
    const int u0 = sk.begin(g), u1 = sk.begin(g + 1);
    // the host keeps every wave's share <= S units: at most two tiles per wave
    const int w0 = u0 + wave_share<WAVES>(u1 - u0, wave);
    const int w1 = u0 + wave_share<WAVES>(u1 - u0, wave + 1);

    const int Gs = SCALE != 0 ? (S + group_steps - 1) / group_steps : (K + 15) >> 4;
    const auto xr = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
    const auto qr = make_rsrc(qweight, (uint32_t)(K >> 3) * (uint32_t)N * 4u);
    const auto sr = make_rsrc(scales, (uint32_t)Gs * (uint32_t)N * 2u);
    const auto zr = make_rsrc(qzeros, ZP ? (uint32_t)Gs * (uint32_t)N / 2u : 0u);

    XPre xpre;
    if constexpr (XLDS) xpre = stage_x_issue(xr, M, K, S);
    u4 *img = reinterpret_cast<u4 *>(decode_dyn_lds + lora_lds_offset(XLDS, M, S));
    u4 *bst = img + kLoraStageChunks;            // LK: the staged rows of B
    LoraStep lstep{};
    // LK, unit workgroups: the shrink step's loads go ahead of the weight
    // prologue, so the step waits for them and not for the weight ring
    if constexpr (LK)
        if (unit) lstep = lora_step_issue(lora, xr, M, K, g * kLoraUnitSteps + wave, unit);
    LoraBStage lb{};
    LoraWords words{};
    __builtin_amdgcn_sched_barrier(0);
    decode_units<D, SCALE, XLDS, BF, ZP, SB>(
        xr, qr, sr, zr, z8, decode_dyn_lds, M, K, N, S, group_steps, w0, w1,
        [&](int slot, const f4(&acc)[kNW]) {
            if (slot > 1) return;   // cannot happen: ranges hold <= S units
#pragma unroll
            for (int r = 0; r < 4; ++r)
                red[(slot * WAVES + wave) * 256 + lane * 4 + r] =
                    f4{acc[0][r], acc[1][r], acc[2][r], acc[3][r]};
        },
        [&]() -> uint32_t {
            uint32_t a = 0u;
            if constexpr (LK) {
                // the rows of B; the shrink step (unit workgroups)
                lb = lora_b_issue(lora, N, u0 / S, u1 > u0 ? (u1 - 1) / S - u0 / S + 1 : 0);
                if constexpr (XLDS) a = stage_x_finish(decode_dyn_lds, xr, M, K, S, xpre);
                if (unit) lora_step_finish<BF>(reinterpret_cast<float *>(img), lora, lstep, M, wave);
                if (XLDS || unit) __syncthreads();
                if (unit && wave == WAVES - 1)
                    lora_publish<WAVES>(reinterpret_cast<const float *>(img), lora, M, g);
                return a;
            }
            if constexpr (XLDS) {
                a = stage_x_finish(decode_dyn_lds, xr, M, K, S, xpre);
                __syncthreads();
            }
            return a;
        },
        [&] {
            // LK: the slab words, requested a few units before the end of the
            // wave's range so that their round trip overlaps its last units
            if constexpr (LK) words = lora_words_issue(lora, M);
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
    LoraTFrag tfr{};
    unsigned exits = 0;
    if constexpr (LK) {
        // the slab words are requested before the barrier, their round trip
        // overlapping the other waves' last units; the barriers below order
        // LDS only.  Every wave is then past its main loop (and the shrink's
        // partials): the area takes the slab values, then the staged rows of B.
#pragma unroll
        for (int q = 0; q < 2; ++q) bst[threadIdx.x + 512 * q] = lb.v[q];
        lds_sync();
        uint16_t *ta = reinterpret_cast<uint16_t *>(bst + kLoraStageChunks);
        lora_gather(reinterpret_cast<float *>(img), words, lora, M);
        lds_sync();
        if (threadIdx.x == 0) {     // every word read here; the answer is needed at the end
            // the address in a vector register: the compiler then issues one
            // plain atomic and waits for its answer only where it is used
            __attribute__((address_space(1))) unsigned *cnt =
                (__attribute__((address_space(1))) unsigned *)lora.area;
            asm volatile("" : "+v"(cnt));
            exits = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        }
        lora_form_t<BF>(ta, (partials && g == 0) ? static_cast<uint16_t *>(lora.tq) : nullptr,
                        reinterpret_cast<const float *>(img), lora, M);
        lds_sync();
        tfr = lora_t_frags(ta, lora, M);
    } else {
        __syncthreads();
        if (u0 >= u1) return;
    }

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
    // no barrier follows, except LK's last one (every lane stays for the
    // term's MFMAs and the exit)
    if (!LK && m >= M) return;

    // Fixed-order sum over the waves for every tile of this range; whole
    // tiles are stored.  Without `partials`, a split tile has exactly two
    // contributors (the host keeps every range at least one tile long, or
    // makes each tile exactly two ranges; a grid of 3T, three, is finished in
    // two such meetings, below), and they meet per output element
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
        const int ta0 = tau * S, tb = ta0 + S;
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
        const bool whole = ta0 >= u0 && tb <= u1;   // the whole tile is here
        // the tile's later contributor: with two contributors, this workgroup
        // if the tile ends inside its range, else the next one; the adapter
        // term rides with the later contributor's sums (either arrival order
        // then adds the same two fp32 values); with `partials` the reduce
        // kernel adds it
        const int gl = tb <= u1 ? g : g + 1;
        // (with three contributors, the last one carries the term)
        if (LK && (whole || (!partials && (three ? g - 3 * tau == 2 : gl == g)))) {   // uniform
            f4 d[kNW];
            lora_tile_delta<BF>(d, tfr, lora, N, tau,
                                tau - b0 < lb.nb
                                    ? reinterpret_cast<const uint16_t *>(bst + (tau - b0) * 8 * lora.r)
                                    : nullptr);
#pragma unroll
            for (int j = 0; j < kNW; ++j) v[j] += d[j][i];
        }
        if (m >= M || n >= N) continue;
        if (whole) {
            store_quad<BF, SILU>(y, m, N, n, v);
            continue;
        }
        if (partials) {
            float *mine = partials + ((size_t)g * 2 + (tau == b0 ? 0 : 1)) * SLOT;
            *reinterpret_cast<f4 *>(mine + m * kCols + c) = f4{v[0], v[1], v[2], v[3]};
            continue;
        }
        if (three) {
            // three contributors i = g - 3 tau: 0 and 1 meet at the slot of
            // workgroup 3 tau + 1; whichever comes second carries p0 + p1 to
            // the slot of 3 tau + 2 and meets contributor 2 there.  Each
            // meeting adds two fp32 values, so y = (p0 + p1) + p2 whatever the
            // arrival order.
            const int i3 = g - 3 * tau;
            float w[kNW];
            bool live[kNW / 2];
#pragma unroll
            for (int j = 0; j < kNW; ++j) w[j] = v[j];
#pragma unroll
            for (int j = 0; j < kNW / 2; ++j) live[j] = true;
            if (i3 < 2) {
                uint64_t *s1 = slots + ((size_t)(3 * tau + 1) * 16 + m) * (kCols / 2) + c / 2;
                uint64_t got1[kNW / 2];
#pragma unroll
                for (int j = 0; j < kNW / 2; ++j) {
                    got1[j] = 0;
                    const uint64_t mine = (uint64_t)slot_code(w[2 * j]) | ((uint64_t)slot_code(w[2 * j + 1]) << 32);
                    __hip_atomic_compare_exchange_strong(s1 + j, &got1[j], mine, __ATOMIC_RELAXED,
                                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                }
#pragma unroll
                for (int j = 0; j < kNW / 2; ++j) {
                    live[j] = got1[j] != 0;
                    if (!live[j]) continue;
                    w[2 * j] = __builtin_bit_cast(float, (uint32_t)got1[j] ^ kSlotKey) + w[2 * j];
                    w[2 * j + 1] = __builtin_bit_cast(float, (uint32_t)(got1[j] >> 32) ^ kSlotKey) + w[2 * j + 1];
                    __hip_atomic_store(s1 + j, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                }
            }
            uint64_t *s2 = slots + ((size_t)(3 * tau + 2) * 16 + m) * (kCols / 2) + c / 2;
            uint64_t got2[kNW / 2];
#pragma unroll
            for (int j = 0; j < kNW / 2; ++j) {
                got2[j] = 0;
                if (!live[j]) continue;
                const uint64_t mine = (uint64_t)slot_code(w[2 * j]) | ((uint64_t)slot_code(w[2 * j + 1]) << 32);
                __hip_atomic_compare_exchange_strong(s2 + j, &got2[j], mine, __ATOMIC_RELAXED,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            }
#pragma unroll
            for (int j = 0; j < kNW / 2; ++j) {
                if (got2[j] == 0) continue;
                const float r0 = __builtin_bit_cast(float, (uint32_t)got2[j] ^ kSlotKey) + w[2 * j];
                const float r1 = __builtin_bit_cast(float, (uint32_t)(got2[j] >> 32) ^ kSlotKey) + w[2 * j + 1];
                __hip_atomic_store(s2 + j, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                store_pair<BF, SILU>(y, m, N, n + 2 * j, r0, r1);
            }
            continue;
        }
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
    if constexpr (LK) {
        asm volatile("" : "+v"(exits));   // the count's first use is here, at the end
        if (threadIdx.x == 0) lk_last[0] = exits + 1 == gridDim.x;
        lds_sync();
        lora_reset(lora, M, lk_last[0] != 0);
    }
}

// Adds the partials of every split tile of a stream-K launch of G workgroups
// that used partial slots, in workgroup order (fixed, so results are
// bit-reproducible), and stores y.  One workgroup per tile; thread (m, q)
// handles row m and columns 4q .. 4q+3 of the tile.  Tiles that lie whole
// inside one range were stored by the stream-K kernel.
template <bool BF, bool SILU>
__global__ __launch_bounds__(256) void decode_split_reduce_kernel(
    const float *__restrict__ partials, uint16_t *__restrict__ y, int M, int N, int S, int G,
    LoraTerm lora) {
    constexpr int SLOT = 16 * kCols;
    const int T = (N + kCols - 1) / kCols;
    const StreamK sk{T * S, G};
    const int tau = blockIdx.x;
    const int gf = sk.owner(tau * S), gl = sk.owner(tau * S + S - 1);
    if (gf == gl) return;
    __shared__ __attribute__((aligned(16))) float tl[kLoraMaxMR];
    if (lora.A) {                                   // t' from the stream-K launch
        const uint16_t *tq = static_cast<const uint16_t *>(lora.tq);
        for (int idx = threadIdx.x; idx < M * lora.r; idx += 256)
            tl[idx] = lo_f32<BF>((uint32_t)tq[idx]);
        __syncthreads();
    }
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
    if (lora.A) lora_add4<BF>(r, tl, lora, m, n, N);
    store_quad<BF, SILU>(y, m, N, n, r);
}

// ---------------------------------------------------------------------------

#ifndef W4A16_DECODE_WAVES
#define W4A16_DECODE_WAVES 8
#endif
#ifndef W4A16_DECODE_D
#define W4A16_DECODE_D 4
#endif
#ifndef W4A16_DECODE_DX
#define W4A16_DECODE_DX 3
#endif

constexpr int kDecWaves = W4A16_DECODE_WAVES;
// Load ring depth: with staged activations (a unit's loads are its weight
// words and scales), and with activations loaded per unit (one more 16-byte
// load per stage), where a ring of 3 measured faster than 4 at M = 4-16 on
// K = 5120 (N=17408 M = 8 / 16: 14.5 / 19.0 -> 14.4 / 18.7 us; K=N=5120 M = 4 /
// 8 / 16: 8.75 / 9.27 / 11.05 -> 8.55 / 9.03 / 10.75 us) and the same within
// 0.1 us at K = 17408; 6 was slower everywhere.
constexpr int kDecD = W4A16_DECODE_D;
constexpr int kDecDx = W4A16_DECODE_DX;

static size_t slots_bytes(int capacity) { return (size_t)capacity * 16 * (kCols / 2) * sizeof(uint64_t); }

static_assert(kDecodeWorkspacePerCu == 16 * (kCols / 2) * sizeof(uint64_t) + 2 * 16 * kCols * sizeof(float),
              "decode workspace layout");
size_t decode_workspace_bytes(int capacity) {
    return (size_t)capacity * kDecodeWorkspacePerCu + kDecodeLoraBytes;
}

// Stream-K launches whose tiles may have more than two contributors (more
// ranges than 2T) use partial slots and the reduce kernel; so do batches of
// 15 or 16 rows, where the exchange's compare-and-swaps (one per row and
// column pair) cost more than the second kernel (measured at M = 16: -0.7
// us on K = 5120, N = 17408 and -1.5 us on N = 27648; at M = 12 +0.25 us).
// The other launches use the exchange slots.
constexpr int kPartialsMinM = 15;
static bool uses_partials(int grid, int T, int M) {
    if (grid == 3 * T) return false;   // the two-level exchange, for every M
    return grid > 2 * T || M >= kPartialsMinM;
}

// With fewer than half as many tiles as CUs, batches above two rows spread
// over every CU (a tile then has several contributors) when K is long: the
// work per range is then large enough that the extra CUs outweigh the second
// kernel.  Measured on N = 5120 (80 tiles): a gain from S = 432 at M = 4 and
// from S = 256 at M = 16, a loss at S = 256, M = 4 and none at S = 128.
static bool spread_wide(int64_t M, int64_t S) { return M > 2 && (S >= 384 || (M >= 8 && S >= 256)); }

// Stream-K grid, or 0 for the tiles kernel.  With the exchange, every tile
// has at most two contributors (every range holds at least one tile, G <= T,
// or G = 2T and each tile is exactly two ranges) or exactly three (G = 3T);
// wider grids use the partial slots.
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
    // G = 3T: each tile exactly three ranges, finished by the two-level
    // exchange; its second round trip pays off with long ranges (K >= 8192)
    // or heavier units (M >= 4): down projection K=17408, M=1 15.5 -> 13.7 us,
    // M=2 16.6 -> 14.0 us, K=N=5120 M=8 9.7 -> 9.3 us; at K=5120 and M=1,
    // 0.2 us slower.  Where the wide grid below would also apply, three is
    // faster: K=17408 M = 3 / 4 / 8 / 12 / 14: 15.2 / 15.2 / 16.1 / 17.6 /
    // 18.4 -> 14.0 / 14.4 / 15.1 / 16.8 / 18.0 us; and at M = 15-16 than the
    // partial slots: K=17408 M=16 19.4 -> 18.9 us, K=N=5120 M=16 12.1 -> 11.1 us.
    if (3 * T <= num_cus && S >= 24 && (S >= 256 || a.M >= 4)) return (int)(3 * T);
    // G > 2T: partial slots (a tile may have more than two contributors)
    if (2 * T < num_cus && spread_wide(a.M, S)) return num_cus;
    // G = 2T: two ranges per tile.  With short K one workgroup per tile is
    // faster: its waves take a unit or two each and no exchange round trip
    // follows (M=1, K=N=256: 5.0 -> 4.2 us)
    if (2 * T <= num_cus && S >= 16) return (int)(2 * T);
    return (int)T;
}

// Whether the LoRA term (a.lora, counters aside) can go inside a stream-K
// launch of `grid` workgroups: rank and sizes within the LDS areas, one
// workgroup per shrink unit (the waves' shares are those of every stream-K
// launch, at most S units each).
static bool lora_inkernel_ok(const LinearArgs &a, int grid) {
    const LoraTerm &L = a.lora;
    if (L.r < 8 || L.r % 8 != 0 || L.r > kLoraMaxRank || a.M * L.r > kLoraMaxMR) return false;
    const int64_t S = (a.K + 31) / 32;
    if (grid <= 0 || L.Su != (S + kLoraUnitSteps - 1) / kLoraUnitSteps || L.Su > grid) return false;
    if ((int64_t)L.Su * a.M * L.r > kLoraMaxSlabReads) return false;
    return true;
}

bool decode_lora_inkernel_ok(const LinearArgs &a, int num_cus) {
    if (a.silu || a.qzeros) return false;
    return lora_inkernel_ok(a, decode_streamk_grid(a, num_cus));
}

// Activations are staged in LDS when they fit in this many bytes.
constexpr size_t kXStageMax = 64 * 1024;

// Every shipped instantiation fits a gfx950 workgroup's 160 KiB of LDS with
// the largest staging area (plus its zero chunk), and the LoRA kernels with
// their areas and no staging, so the launch-time check against the device's
// limit (stage_fits) only ever turns the LoRA kernels' staging off; a larger
// wave count or staging area fails here, at compile time.
constexpr size_t kGfx950LdsPerWorkgroup = 160 * 1024;
static_assert(streamk_static_lds(kDecWaves) + kXStageMax + 16 <= kGfx950LdsPerWorkgroup,
              "stream-K decode: static LDS plus staged activations exceed 160 KiB");
static_assert(streamk_static_lds(kDecWaves) + kLoraLdsBytes <= kGfx950LdsPerWorkgroup,
              "stream-K decode: static LDS plus the LoRA areas exceed 160 KiB");
static_assert(tiles_static_lds(kDecWaves) + kXStageMax + 16 <= kGfx950LdsPerWorkgroup,
              "tiles decode: static LDS plus staged activations exceed 160 KiB");
static_assert(kDecWaves * 64 == 512, "the LoRA staging takes two chunks per thread of 512");
static_assert(kDecWaves == kLoraUnitSteps, "a LoRA shrink unit is one K step per wave");

// Static LDS of a kernel, read once from its attributes.
static size_t static_lds(const void *kernel) {
    hipFuncAttributes attr;
    if (hipFuncGetAttributes(&attr, kernel) != hipSuccess) return (size_t)-1;
    return attr.sharedSizeBytes;
}

template <int SCALE, bool XLDS, bool BF, bool SILU, bool ZP, bool SB>
static hipError_t launch_sa(const LinearArgs &a, hipStream_t stream, void *workspace,
                            int capacity, int grid) {
    const int K = (int)a.K, N = (int)a.N, M = (int)a.M;
    const int S = (K + 31) / 32;
    int group_steps = 0;
    if (SCALE != 0) group_steps = a.group_size == -1 ? S : (int)a.group_size / 32;
    const void *xp = a.x;
    const void *qp = a.qweight;
    const void *sp = a.scales;
    const void *zp = a.qzeros;
    int z8 = 8 - a.zero_bias;
    void *yp = a.y;
    const dim3 block(kDecWaves * 64);
    LoraTerm lora = a.lora;
    const bool lk = lora.A != nullptr;
    const size_t dyn = lora_lds_offset(XLDS, M, S) + (lk ? kLoraLdsBytes : 0);
    if (grid > 0) {
        char *ws = static_cast<char *>(workspace);
        uint64_t *slots = reinterpret_cast<uint64_t *>(ws);
        const int T = (N + kCols - 1) / kCols;
        const bool part = uses_partials(grid, T, M);
        float *partials = part ? reinterpret_cast<float *>(ws + slots_bytes(capacity)) : nullptr;
        if (lk) lora.area = reinterpret_cast<unsigned *>(ws + capacity * kDecodeWorkspacePerCu);
        void *args[] = {&xp, &qp, &sp, &zp, &yp, (void *)&M, (void *)&K, (void *)&N,
                        &group_steps, &z8, &slots, &partials, &lora};
        const void *kern = reinterpret_cast<const void *>(
            &decode_streamk_kernel<kDecWaves, XLDS ? kDecD : kDecDx, SCALE, XLDS, BF, SILU, ZP, SB, false>);
        if constexpr (!SILU && !ZP)
            if (lk)
                kern = reinterpret_cast<const void *>(
                    &decode_streamk_kernel<kDecWaves, XLDS ? kDecD : kDecDx, SCALE, XLDS, BF, SILU, ZP, SB,
                                           true>);
        hipError_t e = hipLaunchKernel(kern, dim3(grid), block, args, dyn, stream);
        if (e != hipSuccess || !part) return e;
        const float *pc = partials;
        int Sv = S, G = grid;
        void *rargs[] = {&pc, &yp, (void *)&M, (void *)&N, &Sv, &G, &lora};
        return hipLaunchKernel(reinterpret_cast<const void *>(&decode_split_reduce_kernel<BF, SILU>),
                               dim3((unsigned)T), dim3(256), rargs, 0, stream);
    }
    void *args[] = {&xp, &qp, &sp, &zp, &yp, (void *)&M, (void *)&K, (void *)&N, &group_steps,
                    &z8};
    const unsigned tiles = (unsigned)((N + kCols - 1) / kCols);
    return hipLaunchKernel(
        reinterpret_cast<const void *>(
            &decode_tiles_kernel<kDecWaves, XLDS ? kDecD : kDecDx, SCALE, XLDS, BF, SILU, ZP, SB>),
        dim3(tiles), block, args, dyn, stream);
}

// Whether the activations are staged in LDS: one or two rows (from three
// rows on, loading them per unit is faster: K=5120, N=17408, M = 3 / 4 / 6:
// 12.7 / 13.3 / 14.3 -> 12.6 / 12.9 / 13.6 us; K=N=5120: 9.2 / 9.5 / 10.1 ->
// 8.7 / 8.7 / 9.0 us; at M = 2 staging is 0.4 us faster), at most kXStageMax
// bytes, and the kernel's static LDS plus the staging area within the
// device's per-workgroup LDS limit (a launch beyond it is rejected by the
// device).
template <int SCALE, bool BF>
static bool stage_fits(const LinearArgs &a, int grid, size_t max_lds) {
    if (a.M > 2) return false;
    const size_t stage = (size_t)a.M * 32 * ((a.K + 31) / 32) * 2 + 16;
    if (stage > kXStageMax) return false;
    const size_t dyn = stage + (a.lora.A ? kLoraLdsBytes : 0);
    static const size_t sk_static = static_lds(reinterpret_cast<const void *>(
        &decode_streamk_kernel<kDecWaves, kDecD, SCALE, true, BF, false, false, false, false>));
    static const size_t tiles_static = static_lds(reinterpret_cast<const void *>(
        &decode_tiles_kernel<kDecWaves, kDecD, SCALE, true, BF, false, false, false>));
    const size_t st = grid > 0 ? sk_static : tiles_static;
    return st != (size_t)-1 && st + dyn <= max_lds;
}

template <int SCALE, bool BF, bool SB>
static hipError_t launch_scale(const LinearArgs &a, hipStream_t stream, void *workspace,
                               int capacity, int grid, size_t max_lds) {
    const bool xlds = stage_fits<SCALE, BF>(a, grid, max_lds);
    if (a.qzeros)   // stored zero points (never with the merged gate/up epilogue)
        return xlds ? launch_sa<SCALE, true, BF, false, true, SB>(a, stream, workspace, capacity, grid)
                    : launch_sa<SCALE, false, BF, false, true, SB>(a, stream, workspace, capacity, grid);
    if (a.silu)
        return xlds ? launch_sa<SCALE, true, BF, true, false, SB>(a, stream, workspace, capacity, grid)
                    : launch_sa<SCALE, false, BF, true, false, SB>(a, stream, workspace, capacity, grid);
    return xlds ? launch_sa<SCALE, true, BF, false, false, SB>(a, stream, workspace, capacity, grid)
                : launch_sa<SCALE, false, BF, false, false, SB>(a, stream, workspace, capacity, grid);
}

template <int SCALE>
static hipError_t launch_types(const LinearArgs &a, hipStream_t stream, void *workspace,
                               int capacity, int grid, size_t max_lds) {
    if (!a.bf16)
        return launch_scale<SCALE, false, false>(a, stream, workspace, capacity, grid, max_lds);
    if (a.scales_bf16)
        return launch_scale<SCALE, true, true>(a, stream, workspace, capacity, grid, max_lds);
    return launch_scale<SCALE, true, false>(a, stream, workspace, capacity, grid, max_lds);
}

hipError_t launch_decode(const LinearArgs &a, hipStream_t stream, void *workspace, int capacity,
                         int grid, size_t max_lds) {
    if (grid > capacity || (a.scales_bf16 && !a.bf16)) return hipErrorInvalidValue;
    if (a.lora.A && (grid <= 0 || !workspace || a.silu || a.qzeros || !lora_inkernel_ok(a, grid)))
        return hipErrorInvalidValue;
    // SCALE 0 scales each 8-deep block (g = 16); 1 scales per group; 2 is one
    // 32-deep step per group: g = 32, or one group over K <= 32
    const int64_t S = (a.K + 31) / 32;
    const bool one_step = a.group_size == 32 || (a.group_size == -1 && S == 1);
    if (a.group_size == 16) return launch_types<0>(a, stream, workspace, capacity, grid, max_lds);
    if (one_step) return launch_types<2>(a, stream, workspace, capacity, grid, max_lds);
    return launch_types<1>(a, stream, workspace, capacity, grid, max_lds);
}

}  // namespace w4a16
