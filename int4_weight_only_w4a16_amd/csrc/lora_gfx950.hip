// LoRA adapter term and zero-point correction kernels, gfx950.
//
// The pages list LoRA adapters on the quantised linear path in the runtime
// contract ("GPTQ-Pro" README, "Runtime contract" table) and keep an adapter
// separate from the packed weights, since a LoRA delta cannot be merged into
// them ("GPT-QModel" README, "PEFT LoRA Training and Adapter Loading"); the
// suggested ranks are 32 and 64, with 128 and 256 as larger choices ("EoRA
// Accuracy Recovery").  The update is the textbook low-rank one in PEFT's
// storage order: A [r, K] (lora_A weight) and B [N, r] (lora_B weight), both
// in the activation type, and a scaling s given as a number:
// y = x . W + s * (x . A^T) . B^T.
//
// Kernels here (all products on the matrix cores, v_mfma_f32_16x16x32_{f16,bf16}):
//   lora_shrink_kernel  t = x . A^T as fp32 partial sums over S chunks of K,
//                       one [Mp, r] slab per chunk (Mp = M rounded up to 16);
//   lora_finish_kernel  adds the slabs in chunk order and rounds t' = s * t
//                       to the activation type, for the prefill kernels to
//                       add t' . B^T in their epilogue (PrefillTerm);
//   lora_expand_kernel  the form after a linear that has already written y:
//                       sums the slabs of a 16-row block in a fixed order,
//                       rounds t to the activation type, multiplies by B^T,
//                       and writes y = round(y + s * delta), one rounding of
//                       the sum (decode calls outside the one-launch limits,
//                       and calls captured on a stream with no workspace yet).
// (Inside the limits the decode kernel runs the whole term in its own launch.)
// Both operands of every MFMA are contiguous along the contracted index (x
// and A rows along K, t rows and B rows along r), so each lane loads its
// eight values with one 16-byte load.  Results are deterministic.
//
// Stored zero points (asymmetric weights, w = (q - z) s) at prefill sizes:
// (q - z) s = (q - 8) s + (8 - z) s, so y = y_sym + sum_g X[m,g] C[g,n] with
// X the sums of x over each group and C = (8 - z) s, both formed by
// zp_prepare_kernel (X in the activation type [M, Gp], C transposed to
// [N, Gp], the layout of a low-rank term's B): the prefill kernels add X . C
// in their epilogue, a correction exactly zero where z = 8.

#include <algorithm>

#include "w4a16_device.hpp"
#include "w4a16_launch.h"

namespace w4a16 {
namespace {

constexpr int kLoraTargetGroups = 512;   // shrink workgroups aimed for (2 per CU)
constexpr int kLoraMaxSplits = 16;       // K chunks of the shrink, at most


// One workgroup (4 waves) computes the partial t of RB 16-row blocks of x
// over one K chunk, for 64 columns of t (blockIdx.z): the waves take
// alternate 32-wide K steps of the chunk (each A fragment loaded once for the
// RB blocks) and their sums are added in LDS in wave order.  Row blocks past
// the last (mblocks) are not written.
template <bool BF, int RB>
__global__ void __launch_bounds__(256) lora_shrink_kernel(const uint16_t *__restrict__ x,
                                                          const uint16_t *__restrict__ A,
                                                          float *__restrict__ tp, int M, int K,
                                                          int r, int Mp, int chunk_steps) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int mg = blockIdx.x, s = blockIdx.y, jc = blockIdx.z;
    const int nsteps = (K + 31) / 32;
    const int kb = s * chunk_steps;
    const int ke = min(kb + chunk_steps, nsteps);
    const auto xr = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
    const auto ar = make_rsrc(A, (uint32_t)r * (uint32_t)K * 2u);
    const int kofs = 8 * (lane >> 4);
    const int jbn = min(4, (r - 64 * jc + 15) / 16);   // column blocks of t present here
    f4 acc[RB][4] = {};
    // the wave's steps kb + w, kb + w + 4, ... in groups of three: the loads of
    // a group are issued together, then its products run in step order (the
    // chunks are short, so one group is usually the wave's whole share)
    constexpr int kGroup = 3;
    for (int st0 = kb + w; st0 < ke; st0 += 4 * kGroup) {
        u4 xa[kGroup][RB], av[kGroup][4];
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
            const int k = 32 * (st0 + 4 * i) + kofs;   // K % 8 == 0: eight in or eight out
            const bool kin = st0 + 4 * i < ke && k < K;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int row = 16 * (RB * mg + rb) + (lane & 15);
                xa[i][rb] = load_b128(xr, (row < M && kin) ? (uint32_t)(row * K + k) * 2u : kOOB);
            }
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) {
                if (jb < jbn) {                   // uniform across the workgroup
                    const int j = 64 * jc + 16 * jb + (lane & 15);
                    av[i][jb] = load_b128(ar, (j < r && kin) ? (uint32_t)(j * K + k) * 2u : kOOB);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
            if (st0 + 4 * i >= ke) break;         // uniform: steps past the chunk add nothing
#pragma unroll
            for (int jb = 0; jb < 4; ++jb)
                if (jb < jbn)
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
                        acc[rb][jb] = mfma16x16x32_t<BF>(xa[i][rb], av[i][jb], acc[rb][jb]);
        }
    }
    __shared__ f4 red[4][RB][4][64];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) red[w][rb][jb][lane] = acc[rb][jb];
    __syncthreads();
    // thread (w, lane) finishes column block w of the four, for every row block
    const int j = 64 * jc + 16 * w + (lane & 15);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int mb = RB * mg + rb;
        const f4 v = ((red[0][rb][w][lane] + red[1][rb][w][lane]) + red[2][rb][w][lane]) +
                     red[3][rb][w][lane];
        if (j < r && 16 * mb < Mp) {
            float *dst = tp + ((size_t)s * Mp + 16 * mb + 4 * (lane >> 4)) * r + j;
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[(size_t)i * r] = v[i];
        }
    }
}

// Two kinds of 64-thread blocks in one launch:
//  - the first `sum_blocks`: X[m, gi] = sum of x[m, k] over group gi (in fp32,
//    K for g = -1), rounded to the activation type into xs [M][Gp], columns
//    G .. Gp-1 zero.  Groups of at most 256 (per_thread): one thread
//    per (row, group) adds the group's 16-byte runs in order.  Larger groups:
//    one wave per (group, row), lane l adds the runs l, l + 64, ... in order,
//    then a fixed butterfly adds the lanes.
//  - the rest: ct[n][g0 .. g0+7] = (8 - z[g,n]) s[g,n] for eight groups per
//    thread (zero for g >= G), exact in fp32 and rounded to the activation
//    type; consecutive threads take consecutive columns, so each load of the
//    scale grid and of qzeros is coalesced.  z = stored nibble + zbias; the
//    scales are bfloat16 when sbf, else fp16.
template <bool BF>
__global__ void __launch_bounds__(64) zp_prepare_kernel(const uint16_t *__restrict__ x,
                                                        const uint16_t *__restrict__ scales,
                                                        const int32_t *__restrict__ qzeros,
                                                        uint16_t *__restrict__ xs,
                                                        uint16_t *__restrict__ ct, int M, int K,
                                                        int N, int gsz, int G, int Gp,
                                                        int per_thread, int sum_blocks, int sbf,
                                                        int zbias) {
    const int lane = threadIdx.x;
    const int b = blockIdx.x;
    if (per_thread && b < sum_blocks) {
        const int64_t i = (int64_t)b * 64 + lane;
        if (i >= (int64_t)M * Gp) return;
        const int gi = (int)(i % Gp), m = (int)(i / Gp);
        float acc = 0.f;
        if (gi < G) {
            const auto xr = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
            const int k0 = gi * gsz, k1 = min(K, k0 + gsz);   // both multiples of 16
#pragma unroll 4
            for (int k = k0; k < k1; k += 8) {
                const u4 v = load_b128(xr, (uint32_t)(m * K + k) * 2u);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc += lo_f32<BF>(v[e]);
                    acc += hi_f32<BF>(v[e]);
                }
            }
        }
        xs[(size_t)m * Gp + gi] = (uint16_t)pack2<BF>(acc, 0.f);
        return;
    }
    if (b < sum_blocks) {
        const int gi = b % Gp, m = b / Gp;
        float acc = 0.f;
        if (gi < G) {
            const auto xr = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
            const int k0 = gi * gsz, k1 = min(K, k0 + gsz);   // both multiples of 16
            for (int k = k0 + 8 * lane; k < k1; k += 512) {
                const u4 v = load_b128(xr, (uint32_t)(m * K + k) * 2u);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc += lo_f32<BF>(v[e]);
                    acc += hi_f32<BF>(v[e]);
                }
            }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
        }
        if (lane == 0) xs[(size_t)m * Gp + gi] = (uint16_t)pack2<BF>(acc, 0.f);
        return;
    }
    const int64_t tt = (int64_t)(b - sum_blocks) * 64 + lane;
    if (tt >= (int64_t)N * (Gp / 8)) return;
    const int n = (int)(tt % N), g0 = 8 * (int)(tt / N);
    float c[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int g = g0 + e;
        c[e] = 0.f;
        if (g < G) {
            const uint32_t zw = (uint32_t)qzeros[(size_t)g * (N / 8) + n / 8];
            const int z = (int)((zw >> (4 * (n % 8))) & 0xFu) + zbias;
            const uint32_t sv = scales[(size_t)g * N + n];
            c[e] = (float)(8 - z) * (sbf ? lo_f32<true>(sv) : lo_f32<false>(sv));
        }
    }
    *reinterpret_cast<u4 *>(ct + (size_t)n * Gp + g0) =
        u4{pack2<BF>(c[0], c[1]), pack2<BF>(c[2], c[3]), pack2<BF>(c[4], c[5]),
           pack2<BF>(c[6], c[7])};
}

// One workgroup (4 waves) adds the adapter term to a 16-row by 64*NB-column
// tile of y; wave w owns columns [16*NB*w, 16*NB*(w+1)) of the tile.
//  1. The tile of y is loaded first (16-byte runs, rows >= M skipped), so its
//     latency overlaps the rest.
//     The first rank step's rows of B are requested next, for the same reason.
//  2. The workgroup sums the S partial slabs of its 16 rows of t once, in
//     chunk order (kSB slabs in flight at a time), in coalesced 16-byte runs
//     spread over all threads, and
//     keeps t in LDS in the activation type ([16][r + 8], dynamic LDS).
//  3. Each wave multiplies t by its rows of B on the matrix cores.
//  4. The fp32 delta goes through LDS to the layout of the y runs, and each
//     run is written once: y = round(y + s * delta).
template <bool BF, int NB>
__global__ void __launch_bounds__(256) lora_expand_kernel(const float *__restrict__ tp,
                                                          const uint16_t *__restrict__ B,
                                                          uint16_t *__restrict__ y, float scale,
                                                          int M, int N, int r, int Mp, int S) {
    constexpr int TN = 64 * NB;
    constexpr int kRuns = TN / 8;                 // 8-column runs per row of the tile
    constexpr int kPer = (16 * kRuns + 255) / 256;
    constexpr int kSB = NB == 1 ? 8 : 4;          // partial slabs loaded per batch
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int nt = blockIdx.x, mb = blockIdx.y;

    u4 yv[kPer];
    bool yin[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int q = threadIdx.x + 256 * i;
        const int m = 16 * mb + q / kRuns, n = nt * TN + 8 * (q % kRuns);
        yin[i] = q < 16 * kRuns && m < M && n < N;   // N % 8 == 0: runs are whole
        yv[i] = yin[i] ? *reinterpret_cast<const u4 *>(y + (size_t)m * N + n) : u4{0, 0, 0, 0};
    }

    // the first rank step's rows of B, which do not depend on t
    const int n0 = nt * TN + 16 * NB * w;
    const auto br = make_rsrc(B, (uint32_t)N * (uint32_t)r * 2u);
    const int kofs = 8 * (lane >> 4);
    u4 bb0[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int n = n0 + 16 * nb + (lane & 15);
        bb0[nb] = load_b128(br, (kofs < r && n < N) ? (uint32_t)(n * r + kofs) * 2u : kOOB);
    }

    extern __shared__ u4 tsh[];                   // t of the 16 rows: [16][r + 8] 16-bit
    const int ld = r + 8;                         // row pitch in elements (16-byte multiple)
    {
        const auto tr = make_rsrc(tp, (uint32_t)S * (uint32_t)Mp * (uint32_t)r * 4u);
        const int runs = 2 * r;                   // 16 rows x r/8 runs of 8 columns
        for (int q = threadIdx.x; q < runs; q += 256) {
            const int rr = q / (r / 8), j = 8 * (q % (r / 8));
            const int m = 16 * mb + rr;
            float tv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            if (m < M) {
                for (int s0 = 0; s0 < S; s0 += kSB) {
                    f4 lo[kSB], hi[kSB];
#pragma unroll
                    for (int u = 0; u < kSB; ++u) {   // in flight together; past S: zero
                        const uint32_t o = s0 + u < S
                                               ? (uint32_t)((((s0 + u) * Mp + m) * r + j) * 4)
                                               : kOOB;
                        lo[u] = __builtin_bit_cast(f4, load_b128(tr, o));
                        hi[u] = __builtin_bit_cast(f4, load_b128(tr, o + 16u));
                    }
#pragma unroll
                    for (int u = 0; u < kSB; ++u)     // chunk order: deterministic
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            tv[i] += lo[u][i];
                            tv[4 + i] += hi[u][i];
                        }
                }
            }
            tsh[(rr * ld + j) / 8] = u4{pack2<BF>(tv[0], tv[1]), pack2<BF>(tv[2], tv[3]),
                                        pack2<BF>(tv[4], tv[5]), pack2<BF>(tv[6], tv[7])};
        }
    }
    __syncthreads();

    f4 acc[NB] = {};
    for (int kk = 0; kk < r; kk += 32) {
        const int j = kk + kofs;                  // r % 8 == 0: eight in or eight out
        const bool jin = j < r;
        u4 bb[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int n = n0 + 16 * nb + (lane & 15);
            bb[nb] = kk == 0 ? bb0[nb]
                             : load_b128(br, (jin && n < N) ? (uint32_t)(n * r + j) * 2u : kOOB);
        }
        const u4 ta = jin ? tsh[((lane & 15) * ld + j) / 8] : u4{0, 0, 0, 0};
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = mfma16x16x32_t<BF>(ta, bb[nb], acc[nb]);
    }
    // the delta tile through LDS, from the MFMA layout to 16-byte runs of rows
    __shared__ float tile[16][TN + 4];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            tile[4 * (lane >> 4) + i][16 * NB * w + 16 * nb + (lane & 15)] = acc[nb][i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        if (!yin[i]) continue;
        const int q = threadIdx.x + 256 * i;
        const int rr = q / kRuns, c = 8 * (q % kRuns);
        const int m = 16 * mb + rr, n = nt * TN + c;
        u4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            o[e] = pack2<BF>(lo_f32<BF>(yv[i][e]) + scale * tile[rr][c + 2 * e],
                             hi_f32<BF>(yv[i][e]) + scale * tile[rr][c + 2 * e + 1]);
        *reinterpret_cast<u4 *>(y + (size_t)m * N + n) = o;
    }
}

// rb: 16-row blocks per shrink workgroup: 4 from 64 blocks on (M > 1008),
// each A fragment then serving four blocks (M=2048, rank 32: 336 -> 334 us
// for the whole LoRA prefill step); 1 below (at M=512, four measured 2-4 us
// slower: too few workgroups).
struct LoraPlan {
    int mblocks, jchunks, chunk_steps, splits, Mp, rb;
};

LoraPlan lora_plan(int64_t M, int64_t K, int64_t r, int max_splits = kLoraMaxSplits) {
    LoraPlan p;
    p.mblocks = (int)((M + 15) / 16);
    p.Mp = 16 * p.mblocks;
    p.jchunks = (int)((r + 63) / 64);
    p.rb = p.mblocks >= 64 ? 4 : 1;
    const int nsteps = (int)((K + 31) / 32);
    const int groups = (p.mblocks + p.rb - 1) / p.rb * p.jchunks;
    int want = (kLoraTargetGroups + groups - 1) / groups;
    want = want < 1 ? 1 : want > max_splits ? max_splits : want;
    int per = (nsteps + want - 1) / want;
    if (per < 4) per = 4 < nsteps ? 4 : nsteps;   // every wave of a chunk gets a step
    p.chunk_steps = per;
    p.splits = (nsteps + per - 1) / per;          // every chunk non-empty
    return p;
}

}  // namespace

// The term inside the decode launch: Su = ceil(K steps / kLoraUnitSteps)
// units; the caller's workspace holds only t' [M][r] (activation type).
static int64_t lora_units(int64_t K) {
    return ((K + 31) / 32 + kLoraUnitSteps - 1) / kLoraUnitSteps;
}

size_t lora_inkernel_bytes(int64_t M, int64_t K, int64_t r) {
    if (M <= 0 || r <= 0 || r > kLoraMaxRank || M * r > kLoraMaxMR ||
        lora_units(K) * M * r > kLoraMaxSlabReads)
        return 0;
    return (size_t)M * (size_t)r * 2;
}

static size_t lora_t_offset(int64_t M, int64_t K, int64_t r);

size_t lora_workspace_bytes(int64_t M, int64_t K, int64_t r) {
    if (M <= 0) return 0;
    // the slabs and then t' (prefill), or t' alone (inside the decode launch)
    const size_t standalone = lora_t_offset(M, K, r) + (size_t)M * (size_t)r * sizeof(uint16_t);
    return std::max(standalone, lora_inkernel_bytes(M, K, r));
}

template <bool BF>
static hipError_t launch_expand(const float *tp, const uint16_t *B, uint16_t *y, float scale,
                                int M, int N, int r, int Mp, int S, int mblocks,
                                hipStream_t stream) {
    // decode-sized batches: narrow tiles for more workgroups on a short y
    const bool narrow = M <= 16;
    const int TN = narrow ? 64 : 256;
    const dim3 eg((N + TN - 1) / TN, mblocks);
    const size_t tlds = (size_t)16 * (size_t)(r + 8) * 2;   // t of 16 rows, 16-bit
    if (narrow)
        lora_expand_kernel<BF, 1><<<eg, 256, tlds, stream>>>(tp, B, y, scale, M, N, r, Mp, S);
    else
        lora_expand_kernel<BF, 4><<<eg, 256, tlds, stream>>>(tp, B, y, scale, M, N, r, Mp, S);
    return hipGetLastError();
}

static hipError_t run_shrink(const LoraArgs &a, const LoraPlan &p, hipStream_t stream,
                             float *tp) {
    const dim3 sg((p.mblocks + p.rb - 1) / p.rb, p.splits, p.jchunks);
    const auto *x = static_cast<const uint16_t *>(a.x);
    const auto *A = static_cast<const uint16_t *>(a.A);
    const int M = (int)a.M, K = (int)a.K, r = (int)a.r;
    if (p.rb == 4) {
        if (a.bf16)
            lora_shrink_kernel<true, 4><<<sg, 256, 0, stream>>>(x, A, tp, M, K, r, p.Mp, p.chunk_steps);
        else
            lora_shrink_kernel<false, 4><<<sg, 256, 0, stream>>>(x, A, tp, M, K, r, p.Mp, p.chunk_steps);
    } else {
        if (a.bf16)
            lora_shrink_kernel<true, 1><<<sg, 256, 0, stream>>>(x, A, tp, M, K, r, p.Mp, p.chunk_steps);
        else
            lora_shrink_kernel<false, 1><<<sg, 256, 0, stream>>>(x, A, tp, M, K, r, p.Mp, p.chunk_steps);
    }
    return hipGetLastError();
}

// t'[m][j] = round(s * sum of the S slabs of (m, j), in slab order), the
// activation type, one thread per entry.
template <bool BF>
__global__ void __launch_bounds__(256) lora_finish_kernel(const float *__restrict__ tp,
                                                          uint16_t *__restrict__ ta, float scale,
                                                          int M, int r, int Mp, int S) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= M * r) return;
    const int m = e / r, j = e - m * r;
    const float *src = tp + (size_t)m * r + j;
    const size_t slab = (size_t)Mp * r;
    // eight slabs' loads in flight at a time, added in slab order
    float acc = 0.f;
    int q = 0;
    for (; q + 8 <= S; q += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = src[(size_t)(q + u) * slab];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += v[u];
    }
    for (; q < S; ++q) acc += src[(size_t)q * slab];
    ta[e] = (uint16_t)pack2<BF>(scale * acc, 0.f);
}

// Byte offset of t' in the workspace: after the standalone plan's slabs.
static size_t lora_t_offset(int64_t M, int64_t K, int64_t r) {
    const LoraPlan p = lora_plan(M, K, r);
    return ((size_t)p.splits * (size_t)p.Mp * (size_t)r * sizeof(float) + 15) / 16 * 16;
}

hipError_t launch_lora_t(const LoraArgs &a, hipStream_t stream, void *workspace,
                         PrefillTerm *term) {
    const LoraPlan p = lora_plan(a.M, a.K, a.r);
    auto *tp = static_cast<float *>(workspace);
    auto *ta = reinterpret_cast<uint16_t *>(static_cast<char *>(workspace) +
                                            lora_t_offset(a.M, a.K, a.r));
    hipError_t e = run_shrink(a, p, stream, tp);
    if (e != hipSuccess) return e;
    const int M = (int)a.M, r = (int)a.r;
    const unsigned blocks = (unsigned)(((int64_t)M * r + 255) / 256);
    if (a.bf16)
        lora_finish_kernel<true><<<blocks, 256, 0, stream>>>(tp, ta, a.scale, M, r, p.Mp, p.splits);
    else
        lora_finish_kernel<false><<<blocks, 256, 0, stream>>>(tp, ta, a.scale, M, r, p.Mp, p.splits);
    term->ta = ta;
    term->B = a.B;
    term->r = r;
    return hipGetLastError();
}

hipError_t launch_lora(const LoraArgs &a, hipStream_t stream, void *workspace) {
    const LoraPlan p = lora_plan(a.M, a.K, a.r);
    const int M = (int)a.M, N = (int)a.N, r = (int)a.r;
    const auto *B = static_cast<const uint16_t *>(a.B);
    auto *y = static_cast<uint16_t *>(a.y);
    auto *tp = static_cast<float *>(workspace);
    hipError_t e = run_shrink(a, p, stream, tp);
    if (e != hipSuccess) return e;
    return a.bf16 ? launch_expand<true>(tp, B, y, a.scale, M, N, r, p.Mp, p.splits, p.mblocks,
                                        stream)
                  : launch_expand<false>(tp, B, y, a.scale, M, N, r, p.Mp, p.splits, p.mblocks,
                                         stream);
}

int zp_groups(int64_t K, int64_t group_size) {
    return group_size == -1 ? 1 : (int)((K + group_size - 1) / group_size);
}

// Workspace: X [M][Gp] in the activation type (in an area sized for fp32
// [M rounded up to 16][Gp]), then C^T [N][Gp] in the activation type.
size_t zp_workspace_bytes(int64_t M, int64_t K, int64_t N, int64_t group_size) {
    if (M <= 0) return 0;
    const int64_t Gp = (zp_groups(K, group_size) + 7) / 8 * 8;
    return (size_t)((M + 15) / 16 * 16) * (size_t)Gp * sizeof(float) +
           (size_t)N * (size_t)Gp * sizeof(uint16_t);
}

hipError_t launch_zp_t(const ZpArgs &a, hipStream_t stream, void *workspace, PrefillTerm *term) {
    const int M = (int)a.M, K = (int)a.K, N = (int)a.N;
    const int G = zp_groups(a.K, a.group_size), Gp = (G + 7) / 8 * 8;
    const int gsz = a.group_size == -1 ? K : (int)a.group_size;
    const int mblocks = (M + 15) / 16;
    const auto *x = static_cast<const uint16_t *>(a.x);
    const auto *sc = static_cast<const uint16_t *>(a.scales);
    auto *xs = static_cast<uint16_t *>(workspace);
    auto *ct = reinterpret_cast<uint16_t *>(static_cast<char *>(workspace) +
                                            (size_t)16 * mblocks * Gp * sizeof(float));
    const int64_t cthreads = (int64_t)N * (Gp / 8);
    const int per_thread = a.group_size != -1 && a.group_size <= 256;
    const int sum_blocks =
        per_thread ? (int)(((int64_t)M * Gp + 63) / 64) : (int)((int64_t)M * Gp);
    const unsigned blocks = (unsigned)(sum_blocks + (cthreads + 63) / 64);
    const int sbf = a.scales_bf16 ? 1 : 0, zbias = a.zero_bias;
    if (a.bf16)
        zp_prepare_kernel<true><<<blocks, 64, 0, stream>>>(x, sc, a.qzeros, xs, ct, M, K, N, gsz,
                                                          G, Gp, per_thread, sum_blocks, sbf, zbias);
    else
        zp_prepare_kernel<false><<<blocks, 64, 0, stream>>>(x, sc, a.qzeros, xs, ct, M, K, N, gsz,
                                                           G, Gp, per_thread, sum_blocks, sbf, zbias);
    term->ta = xs;
    term->B = ct;
    term->r = Gp;
    return hipGetLastError();
}

}  // namespace w4a16
