/*
 * CPU oracle for the W4A16 symmetric-INT4 GPTQ linear.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously-correct
 * definition that the HIP path is checked against.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it.  It shares no
 * code, header, table or helper with the product library, and it never calls
 * into it.
 *
 * What it computes (the plain definition, written out):
 *
 *   q[k,n]  = (uint32(qweight[k/8][n]) >> (4*(k mod 8))) & 0xF
 *   gidx(k) = (g == -1) ? 0 : floor(k / g)
 *   w[k,n]  = float(q[k,n] - 8) * float(scales[gidx(k)][n])        (exact in fp32)
 *   y[m,n]  = sum_{k=0..K-1} double(x[m,k]) * double(w[k,n])        (k ascending,
 *                                                                    fp64 accumulator)
 *
 * Sources on the pages:
 *  - symmetric GPTQ INT4, FP16 activations, desc_act=False only (so the group
 *    of k is floor(k/g), no g_idx), native int32 qweight, group sizes
 *    {-1,16,32,64,128,256,512,1024}, input features divisible by 16 and output
 *    features by 8: "GPTQ-Pro" README, "Runtime contract" table;
 *  - int32 is only the pack container, not the weight width: "Installation and
 *    Quickstart", "Defaults and compatibility decisions" table (pack_dtype);
 *  - g = -1 is per-output-channel (one group over all of K): "Installation and
 *    Quickstart", "Troubleshooting and edge cases" table;
 *  - the dequantise-then-matmul semantics of the portable GPTQ Torch backend:
 *    "Installation and Quickstart", "End-to-end quickstart: GPTQ W4A16".
 * The pages print neither the nibble order inside a word nor the zero point;
 * this file takes nibble j of row r = K index 8r+j, low bits first, and an
 * implicit zero point of 8 (the GPTQ_V2 layout of the benchmark spec).
 *
 * The result y is returned in float64 and is never rounded to fp16.
 *
 * bfloat16 activations (oracle_linear_ex / oracle_linear_at_ex with act = 1):
 * the same definition with x given as bfloat16 bit patterns (1 sign, 8
 * exponent, 7 fraction bits), decoded field by field below.  The scales are
 * fp16, or bfloat16 bit patterns with stype = 1 (decoded the same way): a
 * checkpoint served in bfloat16 carries its scales in that dtype too.  The
 * weight (q - 8) * s stays exact in fp32 (4 + 8 significant bits).  The
 * pages serve this checkpoint with bfloat16 activations
 * ("Qwen3.8-27B-GPTQ-Int4" model card, "4. Deployment": the verified serving
 * command runs with the bfloat16 dtype), while the GPTQ-Pro fork keeps native
 * BF16 outside its own kernels ("GPTQ-Pro" README, "Runtime contract").
 * With absval = 1 the same loops return sum_k |x[m,k]| * |w[k,n]| instead, the
 * magnitude that bounds the rounding error of any evaluation order.
 *
 * Merged gate/up projection with SiLU * mul (oracle_gate_up_silu): the
 * columns of qweight and scales alternate gate (even n) and up (odd n); with
 * g = y[m,2j] and u = y[m,2j+1] of the definition above,
 *   out[m,j] = silu(g) * u,   silu(z) = z / (1 + exp(-z))      (in fp64)
 * The pages name the merged gate_up_proj module ("GPT-QModel" README,
 * "Dynamic Quantization", "Fused Modules in Inference Engines": gate_proj
 * and up_proj merge into gate_up_proj) and serve with the fused silu_and_mul
 * custom op enabled ("Qwen3.8-27B GPTQ-Pro Hybrid INT8" model card,
 * "Text-only serving"); they print neither the column order of the merge
 * nor SiLU, which is its textbook definition here.
 * LoRA adapter on the quantised linear (oracle_lora_shrink, oracle_lora_expand,
 * oracle_linear_lora): with A [r, K] and B [N, r] in the activation type and
 * a scaling factor s,
 *   t[m,j]   = sum_{k} x[m,k] * A[j,k]                 (fp64, k ascending)
 *   d[m,n]   = s * sum_{j} t[m,j] * B[n,j]             (fp64, j ascending)
 *   out[m,n] = y[m,n] + d[m,n]                         (y the linear above)
 * The pages list LoRA adapters on the quantised linear path as part of the
 * runtime contract ("GPTQ-Pro" README, "Runtime contract" table), load an
 * adapter of a given rank (32 suggested, up to 256) beside the quantised
 * model ("GPT-QModel" README, "EoRA Accuracy Recovery") and keep it separate
 * from the packed weights, since a LoRA delta cannot be merged into them
 * ("PEFT LoRA Training and Adapter Loading").  They print no formula; this
 * file takes the textbook low-rank update in PEFT's storage order (lora_A
 * weight [r, K], lora_B weight [N, r]) with s given as a number (alpha / r
 * for plain LoRA).  With absval = 1 the functions return the magnitudes
 * sum |x| |A| and |s| sum |t| |B| instead.
 * Asymmetric weights with stored zero points (oracle_linear_zp): the same
 * definition with the zero point of (group, column) read from qzeros instead
 * of the constant 8:
 *   z[g,n]  = (uint32(qzeros[g][n/8]) >> (4*(n mod 8))) & 0xF
 *   w[k,n]  = float(q[k,n] - z[gidx(k),n]) * float(scales[gidx(k)][n])   (exact in fp32)
 * GPTQModel quantises with sym=False and stores per-group zero points, which
 * the GPTQ-Pro contract leaves out ("GPTQ-Pro" README, "Runtime contract";
 * "GPT-QModel" README), and its checkpoint formats v1 and v2 store them
 * differently without saying how.  This file takes qzeros as int32 [G, N/8]
 * packed along N, nibble j of word c = column 8c+j, low bits first, each
 * nibble the zero point itself (the v2 form).  The v1 checkpoint form
 * (zv1 = 1) is named on the pages ("GPT-QModel" README, "Quant Method /
 * Format / Backend Matrix": FORMAT.GPTQ beside FORMAT.GPTQ_V2; "Norm
 * tuning": v1 zero points read as they are decode the weights wrongly) but
 * not defined there; this file takes the published GPTQ convention that v1
 * stores z - 1 in the nibble, so z = nibble + 1, in [1, 16] (a symmetric
 * checkpoint in v1 form holds 7 in every nibble).  With every zero point 8
 * it is the symmetric definition.
 * For shapes too large for the triple loop (the 2048-row prefill case in
 * full), oracle.linear_dense (Python) takes the same fp32 dequantised W and
 * the activations decoded here (oracle_decode_act) and forms x . W with
 * numpy's float64 matmul, a library primitive: the same sums up to the order
 * of fp64 rounding, pinned against the triple loop.
 * Build: gcc -O2 -fopenmp -ffp-contract=off (no -ffast-math).  OpenMP only
 * splits rows m and column blocks of n, never the sum over k.
 */

#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_OK 0
#define OR_ERR_ARG 1

/* IEEE 754 binary16 bits -> double, decoded field by field. */
static double half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int exp = (h >> 10) & 0x1F;
    int man = h & 0x3FF;
    double v;
    if (exp == 0) {
        v = ldexp((double)man, -24);                 /* subnormal or zero */
    } else if (exp == 31) {
        v = man ? NAN : INFINITY;
    } else {
        v = ldexp((double)(man | 0x400), exp - 25);  /* (1.man) * 2^(exp-15) */
    }
    return sign ? -v : v;
}

/* bfloat16 bits -> double, decoded field by field: 1 sign bit, 8 exponent
 * bits (bias 127), 7 fraction bits. */
static double bf16_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int exp = (h >> 7) & 0xFF;
    int man = h & 0x7F;
    double v;
    if (exp == 0) {
        v = ldexp((double)man, -133);                /* subnormal or zero */
    } else if (exp == 255) {
        v = man ? NAN : INFINITY;
    } else {
        v = ldexp((double)(man | 0x80), exp - 134);  /* (1.man) * 2^(exp-127) */
    }
    return sign ? -v : v;
}

/* An activation's bits -> double: act 0 is fp16, act 1 bfloat16. */
static double act_to_double(uint16_t h, int act) {
    return act ? bf16_to_double(h) : half_to_double(h);
}

/* A scale's bits -> double: stype 0 is fp16, stype 1 bfloat16. */
static double scale_to_double(uint16_t h, int stype) {
    return stype == 1 ? bf16_to_double(h) : half_to_double(h);
}

static int type_ok(int t) { return t == 0 || t == 1; }

/* One product term, or its magnitude. */
static inline double term(double xk, double w, int absval) {
    return absval ? fabs(xk) * fabs(w) : xk * w;
}

static int group_ok(int64_t K, int64_t g) {
    (void)K;
    return g == -1 || g == 16 || g == 32 || g == 64 || g == 128 || g == 256 ||
           g == 512 || g == 1024;
}

static int shape_ok(int64_t M, int64_t K, int64_t N) {
    return M >= 0 && K > 0 && N > 0 && K % 16 == 0 && N % 8 == 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Code of weight (k, n): nibble (k mod 8) of word qweight[k/8][n], read as
 * unsigned so that words whose top nibble is >= 8 (negative int32) unpack
 * the same way as the others. */
static inline unsigned code_at(const int32_t *qweight, int64_t N, int64_t k, int64_t n) {
    uint32_t word = (uint32_t)qweight[(k / 8) * N + n];
    return (word >> (4 * (unsigned)(k % 8))) & 0xFu;
}

static inline int64_t group_of(int64_t k, int64_t g) {
    return g == -1 ? 0 : k / g;
}

/* Dequantised weight as the pages' symmetric scheme defines it:
 * (q - 8) * s, computed in fp32 (exact: at most 4 + 11 significant bits);
 * scales of type stype. */
static inline float weight_at(const int32_t *qweight, const uint16_t *scales, int stype,
                              int64_t N, int64_t g, int64_t k, int64_t n) {
    int q = (int)code_at(qweight, N, k, n);
    float s = (float)scale_to_double(scales[group_of(k, g) * N + n], stype);
    return (float)(q - 8) * s;
}

/* codes[k*N + n] <- q[k, n]. */
int oracle_unpack(const int32_t *qweight, int64_t K, int64_t N, uint8_t *codes) {
    if (!qweight || !codes || K <= 0 || N <= 0 || K % 8 != 0) return OR_ERR_ARG;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n)
            codes[k * N + n] = (uint8_t)code_at(qweight, N, k, n);
    return OR_OK;
}

/* qweight[r][n] <- sum_j codes[8r+j][n] << 4j, as a 32-bit pattern. */
int oracle_pack(const uint8_t *codes, int64_t K, int64_t N, int32_t *qweight) {
    if (!qweight || !codes || K <= 0 || N <= 0 || K % 8 != 0) return OR_ERR_ARG;
    for (int64_t r = 0; r < K / 8; ++r) {
        for (int64_t n = 0; n < N; ++n) {
            uint32_t word = 0;
            for (int j = 0; j < 8; ++j) {
                uint8_t c = codes[(8 * r + j) * N + n];
                if (c > 15) return OR_ERR_ARG;
                word |= (uint32_t)c << (4 * j);
            }
            memcpy(&qweight[r * N + n], &word, sizeof word);
        }
    }
    return OR_OK;
}

/* W[k*N + n] <- w[k, n] in fp32, scales of type stype (0 fp16, 1 bfloat16). */
int oracle_dequant_ex(const int32_t *qweight, const uint16_t *scales, int stype, int64_t K,
                      int64_t N, int64_t g, float *W) {
    if (!qweight || !scales || !W || !shape_ok(0, K, N) || !group_ok(K, g) || !type_ok(stype))
        return OR_ERR_ARG;
    #pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n)
            W[k * N + n] = weight_at(qweight, scales, stype, N, g, k, n);
    return OR_OK;
}

int oracle_dequant(const int32_t *qweight, const uint16_t *scales, int64_t K, int64_t N,
                   int64_t g, float *W) {
    return oracle_dequant_ex(qweight, scales, 0, K, N, g, W);
}

/* out[i] <- the value of activation bits x[i] (act 0 fp16, 1 bfloat16), for
 * callers that take the product with a library matmul (oracle.linear_dense). */
int oracle_decode_act(const uint16_t *x, int act, int64_t n, double *out) {
    if (n < 0 || (act != 0 && act != 1) || (n > 0 && (!x || !out))) return OR_ERR_ARG;
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = act_to_double(x[i], act);
    return OR_OK;
}

/* y[m*N + n] <- sum_k x[m,k] * w[k,n] in fp64, k ascending.  x and scales are
 * fp16 bit patterns.  The dequantised weight is built once as fp32 and reused
 * for every row; the loop runs m -> k -> n with a row of fp64 accumulators, so
 * every output still adds its K products in ascending k. */
static int linear_impl(const uint16_t *x, int act, int absval, const int32_t *qweight,
                       const uint16_t *scales, int stype, int64_t M, int64_t K, int64_t N,
                       int64_t g, double *y) {
    if (!shape_ok(M, K, N) || !group_ok(K, g) || !type_ok(act) || !type_ok(stype))
        return OR_ERR_ARG;
    if (M == 0) return OR_OK;
    if (!x || !qweight || !scales || !y) return OR_ERR_ARG;
    float *W = (float *)malloc((size_t)K * (size_t)N * sizeof(float));
    if (!W) return OR_ERR_ARG;
    oracle_dequant_ex(qweight, scales, stype, K, N, g, W);
    const int64_t NB = 256;                      /* column block per task */
    const int64_t nblocks = (N + NB - 1) / NB;
    #pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t b = 0; b < nblocks; ++b) {
            int64_t n0 = b * NB, n1 = n0 + NB < N ? n0 + NB : N;
            double acc[256];
            for (int64_t n = n0; n < n1; ++n) acc[n - n0] = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double xk = act_to_double(x[m * K + k], act);
                const float *wrow = W + k * N;
                for (int64_t n = n0; n < n1; ++n) acc[n - n0] += term(xk, (double)wrow[n], absval);
            }
            for (int64_t n = n0; n < n1; ++n) y[m * N + n] = acc[n - n0];
        }
    }
    free(W);
    return OR_OK;
}

int oracle_linear(const uint16_t *x, const int32_t *qweight, const uint16_t *scales,
                  int64_t M, int64_t K, int64_t N, int64_t g, double *y) {
    return linear_impl(x, 0, 0, qweight, scales, 0, M, K, N, g, y);
}

/* As oracle_linear, with x of type act and scales of type stype (0 fp16, 1
 * bfloat16) and, when absval is 1, sum_k |x| * |w| in place of the sum of
 * products. */
int oracle_linear_ex(const uint16_t *x, int act, int absval, const int32_t *qweight,
                     const uint16_t *scales, int stype, int64_t M, int64_t K, int64_t N,
                     int64_t g, double *y) {
    return linear_impl(x, act, absval ? 1 : 0, qweight, scales, stype, M, K, N, g, y);
}

/* out[i] <- y[ms[i], ns[i]] for sampled outputs, each from the definition
 * directly (no dequantised matrix): used at sizes where the full product is
 * too slow for a test. */
static int linear_at_impl(const uint16_t *x, int act, int absval, const int32_t *qweight,
                          const uint16_t *scales, int stype, int64_t M, int64_t K, int64_t N,
                          int64_t g, const int64_t *ms, const int64_t *ns, int64_t count,
                          double *out) {
    if (!shape_ok(M, K, N) || !group_ok(K, g) || count < 0 || !type_ok(act) || !type_ok(stype))
        return OR_ERR_ARG;
    if (count == 0) return OR_OK;
    if (!x || !qweight || !scales || !ms || !ns || !out) return OR_ERR_ARG;
    for (int64_t i = 0; i < count; ++i)
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N) return OR_ERR_ARG;
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = ms[i], n = ns[i];
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k)
            acc += term(act_to_double(x[m * K + k], act),
                        (double)weight_at(qweight, scales, stype, N, g, k, n), absval);
        out[i] = acc;
    }
    return OR_OK;
}

/* SiLU, as defined: z / (1 + exp(-z)). */
static double silu(double z) { return z / (1.0 + exp(-z)); }

/* out[m*(N/2) + j] <- silu(y[m,2j]) * y[m,2j+1], y the linear of x (type act). */
int oracle_gate_up_silu(const uint16_t *x, int act, const int32_t *qweight,
                        const uint16_t *scales, int stype, int64_t M, int64_t K, int64_t N,
                        int64_t g, double *out) {
    if (!shape_ok(M, K, N) || N % 2 != 0) return OR_ERR_ARG;
    if (M == 0) return OR_OK;
    if (!out) return OR_ERR_ARG;
    double *y = (double *)malloc((size_t)M * (size_t)N * sizeof(double));
    if (!y) return OR_ERR_ARG;
    int rc = linear_impl(x, act, 0, qweight, scales, stype, M, K, N, g, y);
    if (rc == OR_OK)
        for (int64_t m = 0; m < M; ++m)
            for (int64_t j = 0; j < N / 2; ++j)
                out[m * (N / 2) + j] = silu(y[m * N + 2 * j]) * y[m * N + 2 * j + 1];
    free(y);
    return rc;
}

int oracle_linear_at(const uint16_t *x, const int32_t *qweight, const uint16_t *scales,
                     int64_t M, int64_t K, int64_t N, int64_t g,
                     const int64_t *ms, const int64_t *ns, int64_t count, double *out) {
    return linear_at_impl(x, 0, 0, qweight, scales, 0, M, K, N, g, ms, ns, count, out);
}

int oracle_linear_at_ex(const uint16_t *x, int act, int absval, const int32_t *qweight,
                        const uint16_t *scales, int stype, int64_t M, int64_t K, int64_t N,
                        int64_t g, const int64_t *ms, const int64_t *ns, int64_t count,
                        double *out) {
    return linear_at_impl(x, act, absval ? 1 : 0, qweight, scales, stype, M, K, N, g, ms, ns,
                          count, out);
}

/* ---- LoRA adapter ---- */

/* t[m*r + j] <- sum_k x[m,k] * A[j,k] (fp64, k ascending); x and A of type act,
 * A stored [r, K].  absval: sum_k |x| * |A| instead. */
int oracle_lora_shrink(const uint16_t *x, const uint16_t *A, int act, int absval, int64_t M,
                       int64_t K, int64_t r, double *t) {
    if (M < 0 || K <= 0 || r <= 0 || (act != 0 && act != 1)) return OR_ERR_ARG;
    if (M == 0) return OR_OK;
    if (!x || !A || !t) return OR_ERR_ARG;
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t j = 0; j < r; ++j) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += term(act_to_double(x[m * K + k], act), act_to_double(A[j * K + k], act),
                            absval);
            t[m * r + j] = acc;
        }
    }
    return OR_OK;
}

/* One LoRA output: s * sum_j t[m,j] * B[n,j] (j ascending), or its magnitude. */
static double lora_delta_at(const double *t, const uint16_t *B, int act, int absval,
                            double scale, int64_t r, int64_t m, int64_t n) {
    double acc = 0.0;
    for (int64_t j = 0; j < r; ++j)
        acc += term(t[m * r + j], act_to_double(B[n * r + j], act), absval);
    return (absval ? fabs(scale) : scale) * acc;
}

/* d[m*N + n] <- s * sum_j t[m,j] * B[n,j]; t [M, r] in fp64, B [N, r] of type
 * act.  absval: |s| * sum_j |t| * |B| (t given as magnitudes then). */
int oracle_lora_expand(const double *t, const uint16_t *B, int act, int absval, double scale,
                       int64_t M, int64_t N, int64_t r, double *d) {
    if (M < 0 || N <= 0 || r <= 0 || (act != 0 && act != 1)) return OR_ERR_ARG;
    if (M == 0) return OR_OK;
    if (!t || !B || !d) return OR_ERR_ARG;
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            d[m * N + n] = lora_delta_at(t, B, act, absval, scale, r, m, n);
    return OR_OK;
}

/* out[i] <- d[ms[i], ns[i]] for sampled outputs (arguments as oracle_lora_expand). */
int oracle_lora_expand_at(const double *t, const uint16_t *B, int act, int absval,
                          double scale, int64_t M, int64_t N, int64_t r, const int64_t *ms,
                          const int64_t *ns, int64_t count, double *out) {
    if (M < 0 || N <= 0 || r <= 0 || count < 0 || (act != 0 && act != 1)) return OR_ERR_ARG;
    if (count == 0) return OR_OK;
    if (!t || !B || !ms || !ns || !out) return OR_ERR_ARG;
    for (int64_t i = 0; i < count; ++i)
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N) return OR_ERR_ARG;
    for (int64_t i = 0; i < count; ++i)
        out[i] = lora_delta_at(t, B, act, absval, scale, r, ms[i], ns[i]);
    return OR_OK;
}

/* out[m*N + n] <- linear(x)[m,n] + s * sum_j t[m,j] * B[n,j], t = x . A^T. */
int oracle_linear_lora(const uint16_t *x, int act, const int32_t *qweight,
                       const uint16_t *scales, int stype, const uint16_t *A, const uint16_t *B,
                       double scale, int64_t M, int64_t K, int64_t N, int64_t g, int64_t r,
                       double *out) {
    if (!shape_ok(M, K, N) || !group_ok(K, g) || r <= 0) return OR_ERR_ARG;
    if (M == 0) return OR_OK;
    if (!out) return OR_ERR_ARG;
    double *t = (double *)malloc((size_t)M * (size_t)r * sizeof(double));
    double *d = (double *)malloc((size_t)M * (size_t)N * sizeof(double));
    int rc = (t && d) ? OR_OK : OR_ERR_ARG;
    if (rc == OR_OK) rc = linear_impl(x, act, 0, qweight, scales, stype, M, K, N, g, out);
    if (rc == OR_OK) rc = oracle_lora_shrink(x, A, act, 0, M, K, r, t);
    if (rc == OR_OK) rc = oracle_lora_expand(t, B, act, 0, scale, M, N, r, d);
    if (rc == OR_OK)
        for (int64_t i = 0; i < M * N; ++i) out[i] += d[i];
    free(t);
    free(d);
    return rc;
}

/* ---- asymmetric weights: stored zero points ---- */

/* Stored nibble of (group gi, column n): nibble (n mod 8) of qzeros[gi][n/8]. */
static inline unsigned zero_at(const int32_t *qzeros, int64_t N, int64_t gi, int64_t n) {
    uint32_t word;
    memcpy(&word, &qzeros[gi * (N / 8) + n / 8], sizeof word);
    return (word >> (4 * (unsigned)(n % 8))) & 0xFu;
}

/* Zero point of (group gi, column n): the stored nibble (v2 form), or the
 * nibble plus one (v1 form, zv1 = 1). */
static inline int zero_point(const int32_t *qzeros, int zv1, int64_t N, int64_t gi, int64_t n) {
    return (int)zero_at(qzeros, N, gi, n) + (zv1 ? 1 : 0);
}

/* y[m*N + n] <- sum_k x[m,k] * (q[k,n] - z[gidx(k),n]) * s[gidx(k),n] in fp64,
 * k ascending, x of type act, scales of type stype, zero points in the v2
 * (zv1 = 0) or v1 (zv1 = 1) form; absval: sum_k |x| |w| instead. */
int oracle_linear_zp(const uint16_t *x, int act, int absval, const int32_t *qweight,
                     const uint16_t *scales, int stype, const int32_t *qzeros, int zv1,
                     int64_t M, int64_t K, int64_t N, int64_t g, double *y) {
    if (!shape_ok(M, K, N) || !group_ok(K, g) || !type_ok(act) || !type_ok(stype) ||
        !type_ok(zv1))
        return OR_ERR_ARG;
    if (M == 0) return OR_OK;
    if (!x || !qweight || !scales || !qzeros || !y) return OR_ERR_ARG;
    float *W = (float *)malloc((size_t)K * (size_t)N * sizeof(float));
    if (!W) return OR_ERR_ARG;
    #pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) {
            const int64_t gi = group_of(k, g);
            const int q = (int)code_at(qweight, N, k, n), z = zero_point(qzeros, zv1, N, gi, n);
            W[k * N + n] = (float)(q - z) * (float)scale_to_double(scales[gi * N + n], stype);
        }
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += term(act_to_double(x[m * K + k], act), (double)W[k * N + n], absval);
            y[m * N + n] = acc;
        }
    free(W);
    return OR_OK;
}

/* out[i] <- y[ms[i], ns[i]] of oracle_linear_zp for sampled outputs, each from
 * the definition directly (no dequantised matrix). */
int oracle_linear_zp_at(const uint16_t *x, int act, const int32_t *qweight,
                        const uint16_t *scales, int stype, const int32_t *qzeros, int zv1,
                        int64_t M, int64_t K, int64_t N, int64_t g, const int64_t *ms,
                        const int64_t *ns, int64_t count, double *out) {
    if (!shape_ok(M, K, N) || !group_ok(K, g) || count < 0 || !type_ok(act) || !type_ok(stype) ||
        !type_ok(zv1))
        return OR_ERR_ARG;
    if (count == 0) return OR_OK;
    if (!x || !qweight || !scales || !qzeros || !ms || !ns || !out) return OR_ERR_ARG;
    for (int64_t i = 0; i < count; ++i)
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N) return OR_ERR_ARG;
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < count; ++i) {
        const int64_t m = ms[i], n = ns[i];
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const int64_t gi = group_of(k, g);
            const int q = (int)code_at(qweight, N, k, n), z = zero_point(qzeros, zv1, N, gi, n);
            const float w = (float)(q - z) * (float)scale_to_double(scales[gi * N + n], stype);
            acc += act_to_double(x[m * K + k], act) * (double)w;
        }
        out[i] = acc;
    }
    return OR_OK;
}
