// Prefill W4A16 GEMM for gfx950: any M, MFMA with fp32 accumulation.
//
// The pages' prefill path ("GPTQ-Pro" README, "Ampere kernel architecture",
// Tensor Core prefill) stages operands asynchronously, accumulates in FP32,
// handles tails and stores FP16 vectors.  Two CDNA4 kernels share the
// v_mfma_f32_32x32x16_f16 instruction, one wave per SIMD (the accumulators
// fill the AGPRs) and weights that never touch registers other than their
// own lane's: each qweight word is exactly one lane's 8-deep B fragment,
// dequantised in registers to (q-8)*s in fp16 (one rounding).
//
// prefill_m256_kernel (M > 1024, and 128 < M <= 1024 where use_m256 prices it
// cheaper than the 128-row kernel): 256 x 256 output tile per workgroup.
//  * Wave w owns columns 64w .. 64w+63 of all 256 rows: 8 x 2 MFMA tiles,
//    256 fp32 accumulators per lane.  Eight row tiles share every unpacked B
//    fragment, which halves the unpack work per MFMA against 128-row tiles.
//  * Activations, codes and scales go global -> LDS by buffer loads that
//    write LDS directly (no registers), 64 K per stage, three LDS stages.
//    Activation rows are 128 bytes with the 16-byte chunks XOR-swizzled by
//    the row, so the column-major fragment reads are free of bank conflicts.
//  * Nibbles are unpacked in natural K order (v_perm_b32 spreads the byte of
//    a nibble pair into both halves of a dword), so activations need no
//    reordering and can be copied to LDS as they are.
//  * Per 16-deep step: the next step's fragments are read from LDS a few at
//    a time between the first MFMAs and its B fragments unpacked a few
//    operations at a time between the later ones; the copies for the stage
//    two ahead are issued three per step, also between the MFMAs, and the
//    main loop has no branches.  One barrier per stage.
//  * Tiles go to XCDs in blocks (workgroup id % 8 taken as the XCD).
//
// prefill_m128_kernel (M <= 128, and mid-sized M where it is priced cheaper):
//  128 x 256 tile, 4 x 2 MFMA tiles per wave, row blocks of 128 in grid y;
//  activations go global -> registers -> LDS (reordered to the nibble unpack
//  order on the way in), weights are loaded into registers three stages
//  ahead, A fragments read one step ahead.
//
// Tails: rows >= M and K >= K read as zero through buffer range checks and
// per-lane checks; stores are masked per row and per column pair (N % 8 == 0).

#include <algorithm>
#include <cmath>

#include "w4a16_device.hpp"
#include "w4a16_launch.h"

namespace w4a16 {

constexpr int kPreBM = 128;               // rows per workgroup tile (at most)
constexpr int kPreBN = 256;               // columns per workgroup tile
constexpr int kPreBK = 64;                // K per stage
constexpr int kPreRowBytes = 144;         // 128 B of a row + 16 B pad (bank spread)
constexpr int kPreRing = 3;               // LDS stages, register stages per operand
constexpr int kPreSteps = kPreBK / 16;    // 16-deep MFMA steps per stage

// The low-rank term (PrefillTerm) added to a wave's fp32 sums on the matrix
// cores: acc[mt][j] += ta[m] . B[n]^T for row m = m0 + 32 mt + (lane % 32)
// and column n = ncol + 2 (lane % 32) + j, the layout of the main sums
// (32 x 32 x 16 MFMA: A rows and B columns by lane % 32, 8-deep K blocks by
// lane / 32), over r in 16-deep steps (zero past r, M and N).  Every lane of
// the wave takes part.
template <bool BF, int MT>
__device__ __forceinline__ void prefill_term(f16v (&acc)[MT][2], const PrefillTerm &T, int M,
                                             int N, int m0, int ncol) {
    const int lane = threadIdx.x & 63;
    const int kb = lane >> 5, c32 = lane & 31;
    const auto tr = make_rsrc(T.ta, (uint32_t)M * (uint32_t)T.r * 2u);
    const auto br = make_rsrc(T.B, (uint32_t)N * (uint32_t)T.r * 2u);
    for (int s = 0; s < T.r; s += 16) {
        const int k = s + 8 * kb;
        const bool kin = k < T.r;               // r % 8 == 0: eight in or eight out
        u4 b[2], a[MT];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = ncol + 2 * c32 + j;
            b[j] = load_b128(br, (kin && n < N) ? (uint32_t)(n * T.r + k) * 2u : kOOB);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = m0 + 32 * mt + c32;
            a[mt] = load_b128(tr, (kin && m < M) ? (uint32_t)(m * T.r + k) * 2u : kOOB);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[mt][j] = mfma32x32x16_t<BF>(a[mt], b[j], acc[mt][j]);
    }
}

// gshift: log2(group_size), or -1 for a single group over K.  BF: bfloat16
// activations and output (weights dequantised by dequant_bf16); SB: bfloat16
// scales (with BF only), else fp16.
// Split K: workgroup z of `chunks` takes the 64-deep stages [sb, se) of its
// tile; with chunks > 1 it writes its fp32 sums to partials[z][M][N] and
// prefill_chunk_reduce_kernel adds the chunks, else it stores y.
template <bool BF, bool SILU, int MT, bool SB>
__global__ __launch_bounds__(256) void prefill_m128_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, uint16_t *__restrict__ y, int M, int K, int N,
    int gshift, int chunks, float *__restrict__ partials, PrefillTerm term) {
    constexpr int BM = 32 * MT;                    // rows per tile
    constexpr int kStage = BM * kPreRowBytes;      // LDS bytes per stage
    __shared__ __attribute__((aligned(16))) unsigned char lds[kPreRing * kStage];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int kb = lane >> 5;                 // K block (8 deep) of the 16-deep step
    const int c32 = lane & 31;                // row / column of the 32 x 32 tile
    const int m0 = blockIdx.y * BM;
    const int n = blockIdx.x * kPreBN + wave * 64 + 2 * c32;   // the lane's two columns
    const int G = gshift < 0 ? 1 : ((K - 1) >> gshift) + 1;
    const int nst = (K + kPreBK - 1) / kPreBK;
    const int cz = blockIdx.z;
    const int sb = (int)((int64_t)nst * cz / chunks);
    const int se = (int)((int64_t)nst * (cz + 1) / chunks);

    const auto xr = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
    const auto qr = make_rsrc(qweight, (uint32_t)(K >> 3) * (uint32_t)N * 4u);
    const auto sr = make_rsrc(scales, (uint32_t)G * (uint32_t)N * 2u);

    // ---- activation staging: thread tid moves chunks tid + 256 i, i < MT ----
    // chunk c: row c / 8, 8-deep K block c % 8 of the stage.
    uint32_t a_goff[MT];
    bool a_row_ok[MT];
    int a_kc[MT];
    uint32_t a_loff[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int c = tid + 256 * i;
        const int row = c >> 3, kc = c & 7;
        a_row_ok[i] = m0 + row < M;
        a_kc[i] = kc;
        a_goff[i] = ((uint32_t)(m0 + row) * (uint32_t)K + 8u * kc) * 2u;
        a_loff[i] = row * kPreRowBytes + kc * 16;
    }
    // stages outside [sb, se) read zero (the ring runs up to two past se)
    auto load_a = [&](u4 (&r)[MT], int st) {
        const int k0 = st * kPreBK;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const bool ok = a_row_ok[i] && st < se && (k0 + 8 * a_kc[i] < K);
            r[i] = load_b128(xr, ok ? a_goff[i] + (uint32_t)k0 * 2u : kOOB);
        }
    };
    auto store_a = [&](const u4 (&r)[MT], int slot) {
#pragma unroll
        for (int i = 0; i < MT; ++i)
            *reinterpret_cast<u4 *>(lds + slot * kStage + a_loff[i]) = perm_x(r[i]);
    };

    // ---- weights: words of packed row 2t + kb, columns n, n+1 (t = 16-deep step) ----
    const uint32_t q_off0 = ((uint32_t)kb * (uint32_t)N + (uint32_t)n) * 4u;
    const uint32_t q_step = (uint32_t)N * 8u;      // 2 packed rows
    auto load_b = [&](u2 (&w)[kPreSteps], uint32_t (&s)[kPreSteps], int st) {
#pragma unroll
        for (int h = 0; h < kPreSteps; ++h) {
            const int t = kPreSteps * st + h;
            const uint32_t srow = gshift < 0 ? 0u : (uint32_t)(16 * t) >> gshift;
            const bool in = st < se;
            w[h] = load_b64(qr, in ? q_off0 + (uint32_t)t * q_step : kOOB);
            s[h] = __builtin_amdgcn_raw_buffer_load_b32(
                sr, in ? (srow * (uint32_t)N + (uint32_t)n) * 2u : kOOB, 0, 0);
        }
    };

    const UnpackConsts uc = unpack_consts();
    f16v acc[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[mt][j][e] = 0.f;

    // A fragments of step h of LDS slot `slot` (4 row tiles)
    auto read_a = [&](h8 (&a)[MT], int slot, int h) {
        const unsigned char *abase =
            lds + slot * kStage + c32 * kPreRowBytes + kb * 16 + h * 32;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            a[mt] = __builtin_bit_cast(h8, *reinterpret_cast<const u4 *>(abase + mt * 32 * kPreRowBytes));
    };
    // One stage: 4 steps x (4 row tiles x 2 column tiles) MFMAs.  The A
    // fragments of each step are read during the previous step's MFMAs (the
    // first step's during the previous stage), so LDS latency stays hidden
    // with one wave per SIMD.  On entry `a` holds step 0 of this stage; on
    // exit step 0 of the next stage (slot `next`, stored two stages ago).
    auto compute = [&](int slot, int next, const u2 (&w)[kPreSteps], const uint32_t (&s)[kPreSteps],
                       h8 (&a)[MT]) {
#pragma unroll
        for (int h = 0; h < kPreSteps; ++h) {
            h8 an[MT];
            if (h + 1 < kPreSteps) read_a(an, slot, h + 1);
            else read_a(an, next, 0);
            u4 b0, b1;
            if constexpr (BF) {
                b0 = dequant_bf16<false>(w[h].x, lo_f32<SB>(s[h]));
                b1 = dequant_bf16<false>(w[h].y, hi_f32<SB>(s[h]));
            } else {
                b0 = __builtin_bit_cast(u4, unpack_codes_scaled(w[h].x, uc, half_lo(s[h])));
                b1 = __builtin_bit_cast(u4, unpack_codes_scaled(w[h].y, uc, half_hi(s[h])));
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                acc[mt][0] = mfma32x32x16_t<BF>(__builtin_bit_cast(u4, a[mt]), b0, acc[mt][0]);
                acc[mt][1] = mfma32x32x16_t<BF>(__builtin_bit_cast(u4, a[mt]), b1, acc[mt][1]);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) a[mt] = an[mt];
        }
    };

    u4 areg[kPreRing][MT];
    u2 wreg[kPreRing][kPreSteps];
    uint32_t sreg[kPreRing][kPreSteps];

    // Prologue in the loop's issue order (stage st's loop iteration issues A
    // of st+4, then B of st+3), so the compiler's wait counts in the loop
    // stay deep.  Loads past the last stage read zero and are not used.
    load_a(areg[0], sb);
    __builtin_amdgcn_sched_barrier(0);
    load_a(areg[1], sb + 1);
    __builtin_amdgcn_sched_barrier(0);
    load_b(wreg[0], sreg[0], sb);
    __builtin_amdgcn_sched_barrier(0);
    load_a(areg[2], sb + 2);
    __builtin_amdgcn_sched_barrier(0);
    load_b(wreg[1], sreg[1], sb + 1);
    __builtin_amdgcn_sched_barrier(0);
    store_a(areg[0], 0);
    load_a(areg[0], sb + 3);
    __builtin_amdgcn_sched_barrier(0);
    load_b(wreg[2], sreg[2], sb + 2);
    __builtin_amdgcn_sched_barrier(0);
    store_a(areg[1], 1);
    __syncthreads();
    h8 afrag[MT];
    read_a(afrag, 0, 0);

    // Stages past se (up to two, to finish a round of three) compute on
    // zeros: every load there reads zero.
    for (int st0 = sb; st0 < se; st0 += kPreRing) {
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

    // the low-rank term, once per tile: with the first K chunk
    if (term.ta && cz == 0) prefill_term<BF, MT>(acc, term, M, N, m0, n - 2 * c32);

    // ---- epilogue: register i of tile (mt, j) is row m0 + 32 mt + 8 (i/4) +
    // 4 kb + i%4, column n + j; the two columns of a lane go out together ----
    if (n < N) {
        float *pz = partials ? partials + (size_t)cz * M * N : nullptr;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = m0 + 32 * mt + 8 * (i >> 2) + 4 * kb + (i & 3);
                if (m >= M) continue;
                if (pz)
                    *reinterpret_cast<float2 *>(pz + (size_t)m * N + n) =
                        float2{acc[mt][0][i], acc[mt][1][i]};
                else
                    store_pair<BF, SILU>(y, m, N, n, acc[mt][0][i], acc[mt][1][i]);
            }
        }
    }
}

// y = the sum of the chunks' partials[c][M][N] in chunk order (fixed, so
// results are bit-reproducible); four consecutive elements per thread
// (N % 8 == 0, so they stay in one row).
template <bool BF, bool SILU>
__global__ __launch_bounds__(256) void prefill_chunk_reduce_kernel(
    const float *__restrict__ partials, uint16_t *__restrict__ y, int M, int N, int chunks) {
    const int64_t total = (int64_t)M * N;
    const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (e >= total) return;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    // eight chunks' loads in flight at a time, added in chunk order
    int c = 0;
    for (; c + 8 <= chunks; c += 8) {
        f4 p[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) p[u] = *reinterpret_cast<const f4 *>(partials + (size_t)(c + u) * total + e);
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] += p[u][j];
    }
    for (; c < chunks; ++c) {
        const f4 p = *reinterpret_cast<const f4 *>(partials + (size_t)c * total + e);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] += p[j];
    }
    store_quad<BF, SILU>(y, e / N, N, (int)(e % N), v);
}

// Row tiles of the small-M kernel: 32 * MT rows, the fewest 32-row MFMA
// tiles that cover M (up to 4), so the matrix work does not grow with the
// padding of small batches.
static int m128_mt(int64_t M) { return M <= 32 ? 1 : M <= 64 ? 2 : 4; }

// K chunks for the small-M kernel: with fewer tiles than CUs, split each
// tile's K into about CUs / tiles chunks of at least 8 stages, as long as the
// partials fit the prefill workspace (capacity x 256 KiB).
static int m128_chunks(const LinearArgs &a, int num_cus, int capacity) {
    if (num_cus <= 0) return 1;
    const int64_t bm = 32 * m128_mt(a.M);
    const int64_t tiles = ((a.N + kPreBN - 1) / kPreBN) * ((a.M + bm - 1) / bm);
    const int64_t nst = (a.K + kPreBK - 1) / kPreBK;
    int64_t chunks = std::min<int64_t>(num_cus / tiles, nst / 8);
    const int64_t fit = (int64_t)capacity * 256 * 256 / (a.M * a.N);
    chunks = std::min(chunks, fit);
    return chunks < 2 ? 1 : (int)chunks;
}

template <bool BF, bool SILU, bool SB>
static const void *m128_kernel_mt(int mt) {
    if (mt == 1) return reinterpret_cast<const void *>(&prefill_m128_kernel<BF, SILU, 1, SB>);
    if (mt == 2) return reinterpret_cast<const void *>(&prefill_m128_kernel<BF, SILU, 2, SB>);
    return reinterpret_cast<const void *>(&prefill_m128_kernel<BF, SILU, 4, SB>);
}

static const void *m128_kernel(bool bf16, bool silu, bool sbf, int mt) {
    if (bf16 && sbf)
        return silu ? m128_kernel_mt<true, true, true>(mt) : m128_kernel_mt<true, false, true>(mt);
    if (bf16)
        return silu ? m128_kernel_mt<true, true, false>(mt) : m128_kernel_mt<true, false, false>(mt);
    return silu ? m128_kernel_mt<false, true, false>(mt) : m128_kernel_mt<false, false, false>(mt);
}

static hipError_t launch_prefill_m128(const LinearArgs &a, hipStream_t stream, void *workspace,
                                      int capacity, int num_cus) {
    int K = (int)a.K, N = (int)a.N, M = (int)a.M;
    int gshift = -1;
    if (a.group_size != -1) gshift = __builtin_ctz((unsigned)a.group_size);
    int chunks = m128_chunks(a, num_cus, capacity);
    if (chunks > 1 && (!workspace ||
                       (size_t)chunks * M * N * sizeof(float) > (size_t)capacity * 256 * 256 * 4))
        chunks = 1;
    float *partials = chunks > 1 ? static_cast<float *>(workspace) : nullptr;
    const void *xp = a.x;
    const void *qp = a.qweight;
    const void *sp = a.scales;
    void *yp = a.y;
    PrefillTerm term = a.pterm;
    void *args[] = {&xp, &qp, &sp, &yp, &M, &K, &N, &gshift, &chunks, &partials, &term};
    const int mt = m128_mt(M);
    dim3 grid((unsigned)((N + kPreBN - 1) / kPreBN), (unsigned)((M + 32 * mt - 1) / (32 * mt)),
              (unsigned)chunks);
    dim3 block(256);
    const void *k = m128_kernel(a.bf16, a.silu, a.scales_bf16, mt);
    hipError_t e = hipLaunchKernel(k, grid, block, args, 0, stream);
    if (e != hipSuccess || chunks == 1) return e;
    const float *pc = partials;
    void *rargs[] = {&pc, &yp, &M, &N, &chunks};
    const void *rk =
        a.silu ? (a.bf16 ? reinterpret_cast<const void *>(&prefill_chunk_reduce_kernel<true, true>)
                         : reinterpret_cast<const void *>(&prefill_chunk_reduce_kernel<false, true>))
               : (a.bf16 ? reinterpret_cast<const void *>(&prefill_chunk_reduce_kernel<true, false>)
                         : reinterpret_cast<const void *>(&prefill_chunk_reduce_kernel<false, false>));
    const int64_t threads = ((int64_t)M * N + 3) / 4;
    return hipLaunchKernel(rk, dim3((unsigned)((threads + 255) / 256)), dim3(256), rargs, 0,
                           stream);
}

// ---------------------------------------------------------------------------
// 256 x 256 tiles

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) unsigned char lds_u8_t;

constexpr int kWBM = 256;
constexpr int kWBN = 256;
constexpr int kWBK = 64;
constexpr int kWSteps = 4;
constexpr int kWA = kWBM * 128;            // 256 rows x 64 fp16
constexpr int kWB = 8 * kWBN * 4;           // 8 packed rows x 256 columns
constexpr int kWS = kWSteps * kWBN * 2;    // 4 scale rows x 256 columns
constexpr int kWAOff = 0;
constexpr int kWBOff = 3 * kWA;
constexpr int kWSOff = 3 * kWA + 3 * kWB;
constexpr int kWLds = 3 * (kWA + kWB + kWS);

constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kLgkm0Imm = 15 | (3 << 14) | (7 << 4);     // lgkmcnt(0), no wait on vmcnt
constexpr int vmcnt_lgkm0_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
template <bool B> struct BoolC { static constexpr bool value = B; };

__device__ __forceinline__ h8 unpack_nat_scaled(uint32_t w, _Float16 s, uint32_t mask, uint32_t magic,
                                                h2 mul, h2 add) {
    u4 r;
    const h2 sv = {s, s};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t t = (__builtin_amdgcn_perm(w, w, 0x01010101u * d) & mask) | magic;
        const h2 v = __builtin_elementwise_fma(__builtin_bit_cast(h2, t), mul, add) * sv;
        r[d] = __builtin_bit_cast(uint32_t, v);
    }
    return __builtin_bit_cast(h8, r);
}

// Operands of one wide-tile call: buffer resources and sizes.
struct WideOperands {
    __amdgpu_buffer_rsrc_t xr, qr, sr, yr;
    uint16_t *ybase;
    uint32_t ybytes;
    int M, K, N, gshift;
    int nst;     // 64-deep stages: ceil(K / 64)
    int nfull;   // stages without a K tail: K / 64
};

__device__ __forceinline__ WideOperands wide_operands(const uint16_t *x, const int32_t *qweight,
                                                      const uint16_t *scales, uint16_t *y, int M,
                                                      int K, int N, int gshift) {
    const int G = gshift < 0 ? 1 : ((K - 1) >> gshift) + 1;
    WideOperands p;
    p.xr = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
    p.qr = make_rsrc(qweight, (uint32_t)(K >> 3) * (uint32_t)N * 4u);
    p.sr = make_rsrc(scales, (uint32_t)G * (uint32_t)N * 2u);
    p.yr = make_rsrc(y, (uint32_t)M * (uint32_t)N * 2u);
    p.ybase = y;
    p.ybytes = (uint32_t)M * (uint32_t)N * 2u;
    p.M = M;
    p.K = K;
    p.N = N;
    p.gshift = gshift;
    p.nst = (K + kWBK - 1) / kWBK;
    p.nfull = K / kWBK;
    return p;
}

// acc = the fp32 products of the 256 x 256 tile at (m0, n0) over the 64-deep
// stages [sb, se) of K, 0 <= sb < se <= nst.  Uses the whole LDS area L; on
// return every copy has landed, but other waves may still be reading L.
template <bool BF, bool SB>
__device__ __forceinline__ void wide_tile_range(lds_u8_t *L, const WideOperands &p, int m0, int n0,
                                                int sb, int se, f16v (&acc)[8][2]) {
    const int M = p.M, K = p.K, N = p.N, gshift = p.gshift, nfull = p.nfull;
    const auto xr = p.xr;
    const auto qr = p.qr;
    const auto sr = p.sr;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kb = lane >> 5;
    const int c32 = lane & 31;

    // ---- DMA lane offsets (stage 0) ----
    // A: instruction i moves rows 64w + 8i + lane/8; lane's physical 16-byte
    // slot is lane%8, holding logical chunk (lane%8) ^ f(row),
    // f(row) = (row & 7) ^ ((row >> 3) & 1).
    uint32_t a_voff[8];
    int a_c[8];
    bool a_ok[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = 64 * wave + 8 * i + (lane >> 3);
        const int c = (lane & 7) ^ (lane >> 3) ^ (i & 1);
        a_c[i] = c;
        a_ok[i] = m0 + r < M;
        a_voff[i] = a_ok[i] ? ((uint32_t)(m0 + r) * (uint32_t)K + 8u * c) * 2u : kOOB;
    }
    // B: instruction i moves packed rows 4i + lane/16 of the stage, columns
    // n0 + 64w + 4 (lane%16) .. +3.
    const int b_col = n0 + 64 * wave + 4 * (lane & 15);
    const bool b_ok = b_col < N;
    uint32_t b_voff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
        b_voff[i] = b_ok ? ((uint32_t)(4 * i + (lane >> 4)) * (uint32_t)N + b_col) * 4u : kOOB;
    // S: instruction i moves the scale rows of steps 2i + lane/32, columns
    // n0 + 64w + 2 (lane%32), +1.
    const int s_col = n0 + 64 * wave + 2 * (lane & 31);
    const bool s_ok = s_col < N;
    const uint32_t s_voff = s_ok ? ((gshift == 4 ? (uint32_t)(lane >> 5) * (uint32_t)N : 0u) + s_col) * 2u : kOOB;

    // DMA instruction idx (0..11) of stage st into LDS slot `slot`:
    // 0..7 activations (8 rows per instruction), 8..9 codes, 10..11 scales.
    // FULL: stage st exists and has no K tail (no per-lane K checks).
    auto dma = [&](auto fullc, int st, int slot, int idx) {
        constexpr bool FULL = decltype(fullc)::value;
        const int k0 = st * kWBK;
        if (FULL) {
            if (idx < 8) {
                lds_u8_t *la = L + kWAOff + slot * kWA + (64 * wave + 8 * idx) * 128;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void_t *)la, 16, a_voff[idx], 2u * (uint32_t)k0, 0, 0);
            } else if (idx < 10) {
                const int i = idx - 8;
                lds_u8_t *lb = L + kWBOff + slot * kWB + wave * 2048 + i * 1024;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(qr, (lds_void_t *)lb, 16, b_voff[i], (uint32_t)st * (uint32_t)N * 32u, 0, 0);
            } else {
                const int i = idx - 10;
                const uint32_t srow = gshift < 0 ? 0u : (uint32_t)(k0 + 32 * i) >> gshift;
                lds_u8_t *ls = L + kWSOff + slot * kWS + wave * 512 + i * 256;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (lds_void_t *)ls, 4, s_voff, srow * (uint32_t)N * 2u, 0, 0);
            }
        } else {
            // any stage, every lane offset checked against K
            if (idx < 8) {
                lds_u8_t *la = L + kWAOff + slot * kWA + (64 * wave + 8 * idx) * 128;
                const bool ok = a_ok[idx] && k0 + 8 * a_c[idx] < K;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void_t *)la, 16,
                                                         ok ? a_voff[idx] + 2u * (uint32_t)k0 : kOOB, 0, 0, 0);
            } else if (idx < 10) {
                const int i = idx - 8;
                lds_u8_t *lb = L + kWBOff + slot * kWB + wave * 2048 + i * 1024;
                const int prow = 8 * st + 4 * i + (lane >> 4);
                const bool ok = b_ok && prow < (K >> 3);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    qr, (lds_void_t *)lb, 16, ok ? ((uint32_t)prow * (uint32_t)N + b_col) * 4u : kOOB, 0, 0, 0);
            } else {
                const int i = idx - 10;
                lds_u8_t *ls = L + kWSOff + slot * kWS + wave * 512 + i * 256;
                const int k = k0 + 16 * (2 * i + (lane >> 5));
                const uint32_t srow = gshift < 0 ? 0u : (uint32_t)k >> gshift;
                const bool ok = s_ok && k < K;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    sr, (lds_void_t *)ls, 4, ok ? (srow * (uint32_t)N + s_col) * 2u : kOOB, 0, 0, 0);
            }
        }
    };
    // generic issue of instructions 3c .. 3c+2 of stage st (nothing past the range)
    auto dma_chunk_any = [&](int st, int slot, int c) {
        if (st < se) {
            if (st < nfull) {
                dma(BoolC<true>(), st, slot, 3 * c);
                dma(BoolC<true>(), st, slot, 3 * c + 1);
                dma(BoolC<true>(), st, slot, 3 * c + 2);
            } else {
                dma(BoolC<false>(), st, slot, 3 * c);
                dma(BoolC<false>(), st, slot, 3 * c + 1);
                dma(BoolC<false>(), st, slot, 3 * c + 2);
            }
        }
    };

    // ---- LDS fragment reads ----
    const int f = (c32 & 7) ^ ((c32 >> 3) & 1);
    uint32_t a_rd[kWSteps];
#pragma unroll
    for (int h = 0; h < kWSteps; ++h) a_rd[h] = c32 * 128 + 16 * ((2 * h + kb) ^ f);
    const uint32_t b_rd = wave * 2048 + kb * 256 + 8 * c32;
    const uint32_t s_rd = wave * 512 + 4 * c32;

    // Per step: A fragments (8 row tiles) and the unpacked, scaled B
    // fragments (2 column tiles) of the current step are in registers; the
    // next step's A fragments, words and scales are read from LDS at the start
    // and its B fragments are unpacked between the current step's MFMAs.
    h8 a_cur[8], a_nxt[8];
    h8 b_cur0, b_cur1;
    u2 w_nxt;
    uint32_t s_nxt;

    uint32_t mask = 0x00F0000Fu, magic = 0x64006400u;
    asm volatile("" : "+v"(mask), "+v"(magic));
    h2 mul = {(_Float16)1.0f, (_Float16)0.0625f};
    h2 add = {(_Float16)-1032.0f, (_Float16)-72.0f};
    {
        uint32_t mu = __builtin_bit_cast(uint32_t, mul), ad = __builtin_bit_cast(uint32_t, add);
        asm volatile("" : "+v"(mu), "+v"(ad));
        mul = __builtin_bit_cast(h2, mu);
        add = __builtin_bit_cast(h2, ad);
    }

    auto read_ws = [&](int slot, int h) {
        w_nxt = *(const __attribute__((address_space(3))) u2 *)(L + kWBOff + slot * kWB + b_rd + h * 512);
        s_nxt = *(const __attribute__((address_space(3))) uint32_t *)(L + kWSOff + slot * kWS + s_rd + h * 128);
    };
    auto read_a = [&](int slot, int h) {
        const lds_u8_t *ab = L + kWAOff + slot * kWA + a_rd[h];
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
            a_nxt[mt] = __builtin_bit_cast(h8, *(const __attribute__((address_space(3))) u4 *)(ab + mt * 4096));
    };

#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[mt][j][e] = 0.f;

    // One 16-deep step on (a_cur, b_cur), laid out as 16 MFMA slots: the next
    // step (slot, h) is read from LDS in the first slots (its words and
    // scales in slot 0, its A fragments two per slot in slots 1-4, so the
    // reads never queue up ahead of an MFMA), its B fragments are unpacked
    // three operations per slot from slot 5 on, and in the FAST form the
    // three DMA instructions of chunk dchunk of stage dst go to slots 10, 13
    // and 15.  The slow form issues the chunk up front, with its checks.
    // Fenced groups keep this order (measured against reading everything at
    // the start of the step: 5-10% faster across the prefill shapes).
    auto step = [&](auto fastc, int slot, int h, int dst, int dslot, int dchunk) {
        constexpr bool FAST = decltype(fastc)::value;
        __builtin_amdgcn_sched_barrier(0);
        if (!FAST) {
            dma_chunk_any(dst, dslot, dchunk);
            __builtin_amdgcn_sched_barrier(0);
        }
        const lds_u8_t *ab = L + kWAOff + slot * kWA + a_rd[h];
        uint32_t tw[2][4];
        h2 s_lo, s_hi;
        // bfloat16: 25 operations per word (dequant_bf16's steps, pinned one
        // by one): the fp32 scale and -8 s, the even and odd nibble bytes,
        // then per dword two byte converts, two fmas and one pack
        float bsf = 0.f, bm8 = 0.f, bqa = 0.f, bqb = 0.f;
        uint32_t blo = 0, bhi = 0;
        auto valu_bf = [&](int idx) {
            const int j = idx / 25, r = idx % 25;
            const uint32_t w = j ? w_nxt.y : w_nxt.x;
            if (r == 0) {
                bsf = j ? hi_f32<SB>(s_nxt) : lo_f32<SB>(s_nxt);
                asm volatile("" : "+v"(bsf));
            } else if (r == 1) {
                bm8 = -8.0f * bsf;
                asm volatile("" : "+v"(bm8));
            } else if (r == 2) {
                blo = w & 0x0F0F0F0Fu;
                asm volatile("" : "+v"(blo));
            } else if (r == 3) {
                bhi = w >> 4;
                asm volatile("" : "+v"(bhi));
            } else if (r == 4) {
                bhi &= 0x0F0F0F0Fu;
                asm volatile("" : "+v"(bhi));
            } else {
                const int d = (r - 5) / 5, o = (r - 5) % 5;
                if (o == 0) { bqa = ubyte_f32(blo, d); asm volatile("" : "+v"(bqa)); }
                else if (o == 1) { bqb = ubyte_f32(bhi, d); asm volatile("" : "+v"(bqb)); }
                else if (o == 2) { bqa = __builtin_fmaf(bqa, bsf, bm8); asm volatile("" : "+v"(bqa)); }
                else if (o == 3) { bqb = __builtin_fmaf(bqb, bsf, bm8); asm volatile("" : "+v"(bqb)); }
                else { tw[j][d] = pack2<true>(bqa, bqb); asm volatile("" : "+v"(tw[j][d])); }
            }
        };
        auto valu = [&](int idx) {
            const int j = idx >> 4, k = (idx >> 2) & 3, d = idx & 3;
            const uint32_t w = j ? w_nxt.y : w_nxt.x;
            if (k == 0) tw[j][d] = __builtin_amdgcn_perm(w, w, 0x01010101u * d);
            else if (k == 1) tw[j][d] = (tw[j][d] & mask) | magic;
            else if (k == 2)
                tw[j][d] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(h2, tw[j][d]), mul, add));
            else tw[j][d] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, tw[j][d]) * (j ? s_hi : s_lo));
            asm volatile("" : "+v"(tw[j][d]));   // pin the operation to this group
        };
        auto mfma = [&](int idx) {
            const int j = idx >> 3, mt = idx & 7;
            acc[mt][j] = mfma32x32x16_t<BF>(__builtin_bit_cast(u4, a_cur[mt]),
                                            __builtin_bit_cast(u4, j ? b_cur1 : b_cur0), acc[mt][j]);
        };
#pragma unroll
        for (int si = 0; si < 16; ++si) {
            mfma(si);
            if (si == 0) read_ws(slot, h);
            if (si >= 1 && si <= 4) {
#pragma unroll
                for (int mt = 2 * si - 2; mt < 2 * si; ++mt)
                    a_nxt[mt] = __builtin_bit_cast(h8, *(const __attribute__((address_space(3))) u4 *)(ab + mt * 4096));
            }
            if constexpr (BF) {
                // 50 operations over slots 5-15: five per slot, then four
                if (si >= 5) {
                    const int v0 = si <= 10 ? 5 * (si - 5) : 30 + 4 * (si - 11);
                    const int v1 = si <= 10 ? v0 + 5 : v0 + 4;
#pragma unroll
                    for (int v = v0; v < v1; ++v) valu_bf(v);
                }
            } else {
                if (si == 5) {
                    s_lo = h2{half_lo(s_nxt), half_lo(s_nxt)};
                    s_hi = h2{half_hi(s_nxt), half_hi(s_nxt)};
                }
                if (si >= 5) {
                    const int v0 = 3 * (si - 5);
#pragma unroll
                    for (int v = v0; v < v0 + 3 && v < 32; ++v) valu(v);
                }
            }
            if (FAST && (si == 10 || si == 13 || si == 15))
                dma(BoolC<true>(), dst, dslot, 3 * dchunk + (si == 10 ? 0 : si == 13 ? 1 : 2));
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) a_cur[mt] = a_nxt[mt];
        b_cur0 = __builtin_bit_cast(h8, u4{tw[0][0], tw[0][1], tw[0][2], tw[0][3]});
        b_cur1 = __builtin_bit_cast(h8, u4{tw[1][0], tw[1][1], tw[1][2], tw[1][3]});
    };

    // One stage st in slot r (r == st % 3).  DMA(s) goes to slot s % 3:
    // chunk 0 right after the barrier that frees the slot (in stage s-3),
    // chunks 1..3 during the first three steps of stage s-2.
    // FAST: stages st+2 and st+3 are in the range and have no K tail.
    auto stage = [&](auto fastc, int st, int r) {
        constexpr bool FAST = decltype(fastc)::value;
#pragma unroll
        for (int h = 0; h < kWSteps - 1; ++h) step(fastc, r, h + 1, st + 2, (r + 2) % 3, h + 1);
        // stage st+1 landed (each wave waits for its own DMA; all of stage
        // st+2's is issued after it), and every wave is done reading slot r
        if (FAST || st + 2 < se) __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(12));
        else __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(0));
        lds_barrier();
        // the last step reads step 0 of the next slot (stale after the last
        // stage: read but unused) and starts stage st+3
        step(fastc, (r + 1) % 3, 0, st + 3, r, 0);
    };

    // Prologue: stages sb and sb+1 and the first chunk of sb+2 in flight;
    // wait for stage sb.
#pragma unroll
    for (int c = 0; c < 4; ++c) dma_chunk_any(sb, 0, c);
#pragma unroll
    for (int c = 0; c < 4; ++c) dma_chunk_any(sb + 1, 1, c);
    dma_chunk_any(sb + 2, 2, 0);
    if (se - sb > 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(15));
    else if (se - sb > 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(12));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    lds_barrier();
    read_ws(0, 0);
    read_a(0, 0);
    if constexpr (BF) {
        b_cur0 = __builtin_bit_cast(h8, dequant_bf16<true>(w_nxt.x, lo_f32<SB>(s_nxt)));
        b_cur1 = __builtin_bit_cast(h8, dequant_bf16<true>(w_nxt.y, hi_f32<SB>(s_nxt)));
    } else {
        b_cur0 = unpack_nat_scaled(w_nxt.x, half_lo(s_nxt), mask, magic, mul, add);
        b_cur1 = unpack_nat_scaled(w_nxt.y, half_hi(s_nxt), mask, magic, mul, add);
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) a_cur[mt] = a_nxt[mt];

    // slot of stage st: (st - sb) % 3
    int st0 = sb;
    const int fast_end = se < nfull ? se : nfull;
    // branch-free main loop: every DMA target is a full stage of the range
    for (; st0 + 5 < fast_end; st0 += 3) {
        stage(BoolC<true>(), st0, 0);
        stage(BoolC<true>(), st0 + 1, 1);
        stage(BoolC<true>(), st0 + 2, 2);
    }
    for (; st0 < se; st0 += 3) {
        stage(BoolC<false>(), st0, 0);
        if (st0 + 1 < se) stage(BoolC<false>(), st0 + 1, 1);
        if (st0 + 2 < se) stage(BoolC<false>(), st0 + 2, 2);
    }
    // every copy of the range has landed (the last stage waited for them);
    // the last step's reads of the next slot are stale and unused.  Each
    // workgroup runs one range, so no wave waits for the others here.
}

constexpr int kWSlot = kWBM * kWBN;   // floats per partial tile

// The tile's sums pass through LDS in four passes of 64 rows (two row tiles),
// as fp32 pairs in rows of 256 floats plus 32 bytes (so that the two rows a
// wave writes at once, r and r + 4, start in different bank halves).
constexpr int kWOutRows = 64;
constexpr int kWOutPitch = kWBN * 4 + 32;
static_assert(kWOutRows * kWOutPitch <= kWLds, "a 64-row pass of the output fits the stage buffers");

// Stores the tile's sums.  Register i of lane (c32, kb) in wave w holds row
// 32 mt + 8 (i/4) + 4 kb + i%4 of the tile in column tiles v0 = acc[mt][0]
// and v1 = acc[mt][1], at columns 64w + 2 c32 + {0, 1}.  Each pass writes two
// row tiles into the stage buffers (the caller's LDS area L, no longer read
// once every wave has passed the first barrier) and reads them back as runs
// of 8 columns of a row, so that every store instruction moves 16 bytes per
// lane:
//  - y (partial == nullptr): the run rounded to the output type, one store
//    (rows >= M and columns >= N dropped); with SILU the four (gate, up)
//    pairs of the run become four values silu(gate) * up of y [M, N/2];
//  - fp32 partial tile (`partial`, row-major 256 x 256): the run as two stores.
// One body serves both: the stores that do not apply to this workgroup get an
// out-of-range offset (two bodies do not fit the register file).
template <bool BF, bool SILU>
__device__ __forceinline__ void wide_store(lds_u8_t *L, const WideOperands &p, int m0, int n0,
                                           const f16v (&acc)[8][2], float *partial) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int kb = lane >> 5;
    const int c32 = lane & 31;
    uint32_t part = partial ? ~0u : 0u;                   // uniform: this workgroup writes a partial
    part = __builtin_amdgcn_readfirstlane(part);
    asm volatile("" : "+s"(part));
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(p.ybase, p.ybytes);
    const __amdgpu_buffer_rsrc_t pr = make_rsrc(partial, (uint32_t)kWSlot * 4u & part);
    const int NY = SILU ? p.N / 2 : p.N;                  // y columns
    lds_barrier();                                        // no wave reads the stage buffers any more
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
#pragma unroll
        for (int mh = 0; mh < 2; ++mh)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = 32 * mh + 8 * (i >> 2) + 4 * kb + (i & 3);
                typedef float f2 __attribute__((ext_vector_type(2)));
                *(__attribute__((address_space(3))) f2 *)(L + r * kWOutPitch +
                                                          (64 * wave + 2 * c32) * 4) =
                    f2{acc[2 * pass + mh][0][i], acc[2 * pass + mh][1][i]};
            }
        __builtin_amdgcn_s_waitcnt(kLgkm0Imm);            // this wave's LDS writes are done
        lds_barrier();
#pragma unroll 2
        for (int it = 0; it < kWOutRows * (kWBN / 8) / 256; ++it) {
            const int id = tid + 256 * it;
            const int r = id >> 5, cc = id & 31;          // row of the pass, run of 8 columns
            const lds_u8_t *src = L + r * kWOutPitch + cc * 32;
            const f4 a = *(const __attribute__((address_space(3))) f4 *)src;
            const f4 b = *(const __attribute__((address_space(3))) f4 *)(src + 16);
            const int rt = kWOutRows * pass + r;          // row of the tile
            const int m = m0 + rt, n = n0 + 8 * cc;
            const bool in = m < p.M && n < p.N;
            if constexpr (SILU) {
                if (part) {        // a split tile: the plain fp32 sums (the reduce applies SiLU)
                    const uint32_t po = ((uint32_t)rt * kWBN + 8u * (uint32_t)cc) * 4u;
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, a), pr, po, 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, b), pr, po + 16u, 0, 0);
                } else {
                    const u2 v = {pack2<BF>(silu_f32(a[0]) * a[1], silu_f32(a[2]) * a[3]),
                                  pack2<BF>(silu_f32(b[0]) * b[1], silu_f32(b[2]) * b[3])};
                    __builtin_amdgcn_raw_buffer_store_b64(
                        v, yr, in ? ((uint32_t)m * (uint32_t)NY + (uint32_t)(n / 2)) * 2u : kOOB, 0, 0);
                }
            } else {
                const u4 h = {pack2<BF>(a[0], a[1]), pack2<BF>(a[2], a[3]), pack2<BF>(b[0], b[1]),
                              pack2<BF>(b[2], b[3])};
                const u4 fa = __builtin_bit_cast(u4, a), fb = __builtin_bit_cast(u4, b);
                const uint32_t po = ((uint32_t)rt * kWBN + 8u * (uint32_t)cc) * 4u;
                const uint32_t yo = in ? ((uint32_t)m * (uint32_t)NY + (uint32_t)n) * 2u : kOOB;
                u4 v1;
#pragma unroll
                for (int e = 0; e < 4; ++e) v1[e] = (fa[e] & part) | (h[e] & ~part);
                const uint32_t o1 = (po & part) | (yo & ~part);
                const uint32_t o2 = ((po + 16u) & part) | (kOOB & ~part);
                __builtin_amdgcn_raw_buffer_store_b128(v1, part ? pr : yr, o1, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b128(fb, pr, o2, 0, 0);
            }
        }
        if (pass < 3) lds_barrier();                      // the next pass reuses the area
    }
}

// Tile order of the wide kernel: bands of kWideBandRows row blocks, each band
// taken strip by strip (row blocks fastest).  The workgroups that run at the
// same time on one XCD take consecutive tiles of this order, so they share a
// few row blocks of activations and a few strips of codes in that XCD's L2,
// each fetched about once per round: 4 row blocks x 8 strips for the 32
// workgroups of an XCD, where all 8 row blocks of 4 strips (plain column-
// major order) fetched every activation row on every XCD.
#ifndef W4A16_PREFILL_BAND
#define W4A16_PREFILL_BAND 4
#endif
constexpr int kWideBandRows = W4A16_PREFILL_BAND;

__device__ __forceinline__ void wide_tile(int t, int tiles_m, int tiles_n, int &m0, int &n0) {
    const int band = t / (kWideBandRows * tiles_n);
    const int first = band * kWideBandRows;
    const int rows = min(tiles_m - first, kWideBandRows);    // the last band may be lower
    const int r = t - band * kWideBandRows * tiles_n;
    m0 = (first + r % rows) * kWBM;
    n0 = (r / rows) * kWBN;
}

// The wide kernel.  Workgroups [0, 8 * per_xcd) take one tile each of the
// first tiles_dp tiles (whole rounds), in XCD-blocked order: workgroup id % 8
// is taken as its XCD, and XCD x takes tiles x*per_xcd .. of the order
// above.  The remaining tiles (a last, partial round) are split along K into
// `chunks` equal stage ranges, one workgroup each, run in the same launch;
// each writes its fp32 partial tile to partials[item] (wide_store) and
// prefill_tail_reduce_kernel adds them.  Every workgroup streams K from its
// range start with the others, nothing is exchanged inside the kernel.

template <bool BF, bool SILU, bool SB>
__global__ __launch_bounds__(256) void prefill_m256_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, uint16_t *__restrict__ y, int M, int K, int N,
    int gshift, int tiles_m, int tiles_dp, int per_xcd, int chunks, float *__restrict__ partials,
    PrefillTerm term) {
    __shared__ __attribute__((aligned(16))) unsigned char lds_raw[kWLds];
    const WideOperands p = wide_operands(x, qweight, scales, y, M, K, N, gshift);
    const int id = blockIdx.x;
    const int ndp = 8 * per_xcd;
    // one call of the pipeline for both kinds of workgroup (two inlined
    // copies would not fit the register file)
    int m0, n0, sb, se, j = -1;
    if (id < ndp) {
        const int tl = (id & 7) * per_xcd + (id >> 3);
        if (tl >= tiles_dp) return;
        wide_tile(tl, tiles_m, (N + kWBN - 1) / kWBN, m0, n0);
        sb = 0;
        se = p.nst;
    } else {
        // split tail: item j = tile tiles_dp + j / chunks, K chunk j % chunks
        j = id - ndp;
        const int t = tiles_dp + j / chunks, c = j % chunks;
        wide_tile(t, tiles_m, (N + kWBN - 1) / kWBN, m0, n0);
        sb = (int)((int64_t)p.nst * c / chunks);
        se = (int)((int64_t)p.nst * (c + 1) / chunks);
    }
    f16v acc[8][2];
    wide_tile_range<BF, SB>((lds_u8_t *)lds_raw, p, m0, n0, sb, se, acc);
    // the low-rank term, once per tile: whole tiles, and the first K chunk of
    // a split one (its partial carries the term into the reduce)
    if (term.ta && (j < 0 || j % chunks == 0))
        prefill_term<BF, 8>(acc, term, M, N, m0, n0 + 64 * (int)(threadIdx.x >> 6));
    wide_store<BF, SILU>((lds_u8_t *)lds_raw, p, m0, n0, acc,
                         j < 0 ? nullptr : partials + (size_t)j * kWSlot);
}

// Sums the split tiles' partials (row-major 256 x 256 fp32 tiles, as
// wide_store writes them) in chunk order (fixed, so results are
// bit-reproducible) and stores y.  One thread per (tile, row, run of 8
// columns): 8192 per tile.  SILU: the merged gate/up projection, whose split
// tiles ran without the SiLU epilogue: each (gate, up) column pair of the
// sums becomes silu(gate) * up at column n/2 of y [M, N/2].
template <bool BF, bool SILU>
__global__ __launch_bounds__(256) void prefill_tail_reduce_kernel(
    const float *__restrict__ partials, uint16_t *__restrict__ y, int M, int N, int tiles_m,
    int tiles_dp, int chunks, int tail_tiles) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int tt = (int)(gid >> 13);
    if (tt >= tail_tiles) return;
    const int r = (int)((gid >> 5) & 255), cc = (int)(gid & 31);
    int m0, n0;
    wide_tile(tiles_dp + tt, tiles_m, (N + kWBN - 1) / kWBN, m0, n0);
    const int m = m0 + r;
    const int n = n0 + 8 * cc;
    if (m >= M || n >= N) return;
    const float *src = partials + (size_t)tt * chunks * kWSlot + (size_t)r * kWBN + 8 * cc;
    f4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < chunks; ++c) {
        a += *reinterpret_cast<const f4 *>(src + (size_t)c * kWSlot);
        b += *reinterpret_cast<const f4 *>(src + (size_t)c * kWSlot + 4);
    }
    if constexpr (SILU) {
        *reinterpret_cast<u2 *>(y + (size_t)m * (N / 2) + n / 2) =
            u2{pack2<BF>(silu_f32(a[0]) * a[1], silu_f32(a[2]) * a[3]),
               pack2<BF>(silu_f32(b[0]) * b[1], silu_f32(b[2]) * b[3])};
    } else {
        *reinterpret_cast<u4 *>(y + (size_t)m * N + n) =
            u4{pack2<BF>(a[0], a[1]), pack2<BF>(a[2], a[3]), pack2<BF>(b[0], b[1]),
               pack2<BF>(b[2], b[3])};
    }
}

// Split of the wide kernel's tiles: whole rounds of one tile per workgroup;
// a last partial round of `tail` tiles (at most half a round) split into
// `chunks` >= 2 stage ranges of at least 8 stages, so that tail * chunks
// workgroups fill up to one round, and at most `capacity` partial tiles.
// (For the merged gate/up projection the split tiles store plain fp32 sums
// and the reduce kernel applies SiLU.)
struct WidePlan {
    int tiles, tiles_dp, tail, chunks;
};

// At most six chunks per split tile: on the up-projection (M=2048, K=5120,
// N=17408: 32 tail tiles) six chunks of 13-14 stages took the step from
// 317.4 to 314.8 us against eight of 10 (four: 315.9), with 48 MiB of fp32
// partials written and read back instead of 64.
constexpr int kWideTailMaxChunks = 6;

static WidePlan wide_plan(const LinearArgs &a, int num_cus, int capacity) {
    WidePlan w;
    w.tiles = (int)(((a.M + kWBM - 1) / kWBM) * ((a.N + kWBN - 1) / kWBN));
    w.tiles_dp = w.tiles;
    w.tail = 0;
    w.chunks = 1;
    const int nst = (int)((a.K + kWBK - 1) / kWBK);
    if (num_cus <= 0) return w;
    const int tail = w.tiles % num_cus;
    if (tail == 0 || 2 * tail > num_cus) return w;
    const int chunks = std::min(std::min(std::min(num_cus / tail, nst / 8), capacity / tail),
                                kWideTailMaxChunks);
    if (chunks < 2) return w;
    w.tail = tail;
    w.chunks = chunks;
    w.tiles_dp = w.tiles - tail;
    return w;
}

static_assert(kPrefillPartialTileBytes == (size_t)kWSlot * sizeof(float), "prefill partial tile size");
size_t prefill_workspace_bytes(int capacity) { return (size_t)capacity * kPrefillPartialTileBytes; }

// Which kernel takes 128 < M <= 1024.  Both are priced with a model fitted to
// their measured times on MI355X (about microseconds): a 64-deep stage costs
// 1.15 in the 256-row kernel and 0.95 in the 128-row one, per round of
// workgroups; a K split adds its fp32 partials written and read back at
// about 4 TB/s and 3 for the reduce launch.  The 128-row kernel wins where
// the 256-row tiles leave most CUs idle or are half padding (M = 384 on the
// up-projection: 80 against 92 us; M = 192-768 at K = N = 5120: 5-7 us less)
// and loses badly where its tiles need a second round (M = 512 on the
// up-projection: 155 against 98 us).  Above 1024 rows the 256-row kernel
// always wins; at 128 rows and below only the 128-row kernel runs.
static bool use_m256(const LinearArgs &a, int num_cus) {
    if (a.M <= 128) return false;
    if (a.M > 1024 || num_cus <= 0) return true;
    const double nst = (double)((a.K + kWBK - 1) / kWBK);
    const double c256 = 1.15, c128 = 0.95, bytes_per_us = 4e6, reduce = 3.0;
    double t256;
    const WidePlan w = wide_plan(a, num_cus, num_cus);
    if (w.chunks < 2)
        t256 = (double)((w.tiles + num_cus - 1) / num_cus) * nst * c256;
    else
        t256 = (double)(w.tiles_dp / num_cus) * nst * c256 + std::ceil(nst / w.chunks) * c256 +
               (double)w.tail * w.chunks * kPrefillPartialTileBytes * 2.0 / bytes_per_us + reduce;
    double t128;
    const int64_t tiles = ((a.N + kPreBN - 1) / kPreBN) * ((a.M + kPreBM - 1) / kPreBM);
    const int chunks = m128_chunks(a, num_cus, num_cus);
    if (chunks < 2)
        t128 = (double)((tiles + num_cus - 1) / num_cus) * nst * c128;
    else
        t128 = std::ceil(nst / chunks) * c128 +
               (double)chunks * a.M * a.N * sizeof(float) * 2.0 / bytes_per_us + reduce;
    return t256 <= t128;
}

bool prefill_wants_workspace(const LinearArgs &a, int num_cus) {
    if (use_m256(a, num_cus)) return wide_plan(a, num_cus, num_cus).chunks > 1;
    return m128_chunks(a, num_cus, num_cus) > 1;
}

static hipError_t launch_prefill_m256(const LinearArgs &a, hipStream_t stream, void *workspace,
                                      int capacity, int num_cus) {
    int K = (int)a.K, N = (int)a.N, M = (int)a.M;
    int gshift = -1;
    if (a.group_size != -1) gshift = __builtin_ctz((unsigned)a.group_size);
    int tiles_m = (M + kWBM - 1) / kWBM;
    WidePlan w = wide_plan(a, num_cus, capacity);
    if (w.chunks > 1 && (!workspace || w.tail * w.chunks > capacity)) w = WidePlan{w.tiles, w.tiles, 0, 1};
    int tiles_dp = w.tiles_dp, chunks = w.chunks, tail = w.tail;
    int per_xcd = (tiles_dp + 7) / 8;
    float *partials = static_cast<float *>(workspace);
    const void *xp = a.x;
    const void *qp = a.qweight;
    const void *sp = a.scales;
    void *yp = a.y;
    PrefillTerm term = a.pterm;
    void *args[] = {&xp, &qp, &sp, &yp, &M, &K, &N, &gshift, &tiles_m, &tiles_dp, &per_xcd,
                    &chunks, &partials, &term};
    auto kernel = [&](bool silu) -> const void * {
        if (a.bf16 && a.scales_bf16)
            return silu ? reinterpret_cast<const void *>(&prefill_m256_kernel<true, true, true>)
                        : reinterpret_cast<const void *>(&prefill_m256_kernel<true, false, true>);
        if (a.bf16)
            return silu ? reinterpret_cast<const void *>(&prefill_m256_kernel<true, true, false>)
                        : reinterpret_cast<const void *>(&prefill_m256_kernel<true, false, false>);
        return silu ? reinterpret_cast<const void *>(&prefill_m256_kernel<false, true, false>)
                    : reinterpret_cast<const void *>(&prefill_m256_kernel<false, false, false>);
    };
    hipError_t e = hipLaunchKernel(kernel(a.silu), dim3(8 * per_xcd + tail * chunks), dim3(256),
                                   args, 0, stream);
    if (e != hipSuccess || tail == 0) return e;
    const float *pc = partials;
    void *rargs[] = {&pc, &yp, &M, &N, &tiles_m, &tiles_dp, &chunks, &tail};
    const void *rk =
        a.silu ? (a.bf16 ? reinterpret_cast<const void *>(&prefill_tail_reduce_kernel<true, true>)
                         : reinterpret_cast<const void *>(&prefill_tail_reduce_kernel<false, true>))
               : (a.bf16 ? reinterpret_cast<const void *>(&prefill_tail_reduce_kernel<true, false>)
                         : reinterpret_cast<const void *>(&prefill_tail_reduce_kernel<false, false>));
    return hipLaunchKernel(rk, dim3(32 * tail), dim3(256), rargs, 0, stream);
}

hipError_t launch_prefill(const LinearArgs &a, hipStream_t stream, void *workspace, int capacity,
                          int num_cus) {
    if (a.scales_bf16 && !a.bf16) return hipErrorInvalidValue;
    if (a.pterm.ta && (a.silu || a.pterm.r <= 0 || a.pterm.r % 8 != 0)) return hipErrorInvalidValue;
    if (use_m256(a, num_cus)) return launch_prefill_m256(a, stream, workspace, capacity, num_cus);
    return launch_prefill_m128(a, stream, workspace, capacity, num_cus);
}

}  // namespace w4a16
