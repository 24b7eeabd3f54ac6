/*
 * w4a16.h - C ABI of the MI355X (gfx950) W4A16 symmetric-INT4 GPTQ linear.
 *
 * The operation is the GPTQ weight-only linear layer described by the
 * "GPTQ-Pro" README ("Runtime contract" table and "Ampere kernel
 * architecture" section): FP16 activations, symmetric INT4 weights stored as
 * native int32 qweight, one FP16 scale per (group, output column), group
 * sizes {-1, 16, 32, 64, 128, 256, 512, 1024}, input features divisible by
 * 16 and output features divisible by 8, desc_act=False only.  For every
 * row m < M and column n < N:
 *
 *     q[k,n] = (uint32(qweight[k/8][n]) >> 4*(k mod 8)) & 0xF
 *     w[k,n] = (q[k,n] - 8) * scales[gidx(k)][n],   gidx(k) = (g == -1) ? 0 : k / g
 *     y[m,n] = sum_k x[m,k] * w[k,n]                (fp32 accumulation, fp16 result)
 *
 * g = -1 is one group over all of K (per output channel): "Installation and
 * Quickstart" page, "Troubleshooting and edge cases" table.  int32 is only
 * the container of eight 4-bit codes: same page, "Defaults and compatibility
 * decisions" table (pack_dtype).  The nibble order (nibble j of row r holds K
 * index 8r+j, low bits first) and the zero point 8 are the GPTQ_V2 layout
 * this library implements; the pages print neither.
 *
 * Layouts (all row-major, contiguous, caller-owned):
 *   x        fp16  [M, K]
 *   qweight  int32 [K/8, N]
 *   scales   fp16  [G, N]   with G = 1 for g = -1, else ceil(K/g); a partial
 *                           last group (K % g != 0) and g > K are allowed
 *   y        fp16  [M, N]   must not overlap the inputs
 *
 * Common rules:
 *   - Every argument is validated before any HIP call.  On error nothing is
 *     launched, y is untouched and a nonzero w4a16_status is returned.
 *   - The library keeps no copy of the weights (dense, dequantised or
 *     repacked).  Its only state is a per-device cache of the device's
 *     architecture and up to two workspaces per (device, stream), each
 *     allocated (hipMalloc) and zero-filled on the first call on that stream
 *     that needs it and kept until w4a16_stream_release(stream) frees them
 *     or the process exits (a caller that creates and destroys streams
 *     releases each one before destroying it, else its workspaces stay
 *     held).  They exist because a split-K reduction across workgroups needs
 *     device scratch for its partial sums:
 *       decode: 3 MiB + 16.25 KiB on a 256-CU device (per CU: 16x32
 *         64-bit exchange slots, left zeroed by every launch, and two 16x64
 *         fp32 partial tiles, written before they are read; then the LoRA
 *         term's exit count and slice words, also left zeroed);
 *       prefill: 64 MiB on a 256-CU device (one 256x256 fp32 partial tile
 *         per CU), used when a last partial round of 256-row tiles is split
 *         along K and when fewer 128-row tiles than CUs are split along K
 *         (fp32 partials of y, one per K chunk).  The 128-row kernel takes
 *         M <= 128, the 256-row kernel M > 1024; in between the library
 *         prices both and takes the cheaper.
 *     A call on a stream that is being captured into a graph and has no
 *     workspace yet allocates nothing and runs a kernel that needs none.
 *     Calls on one stream share its workspaces in stream order; calls on
 *     different streams never share one.  A graph captured on a stream keeps
 *     that stream's workspaces: replay it in that stream's order (on the
 *     stream itself, or while nothing else uses that stream's workspaces),
 *     never beside eager calls on that stream.  Thread-safe and reentrant.
 *   - Device calls are asynchronous on the given stream (a hipStream_t; 0 is
 *     the null stream); results are valid once the stream is synchronised.
 *     No call synchronises the device and nothing is printed.
 *   - Results are deterministic: the same inputs give bit-identical y on
 *     a given device.  (A call under capture on a stream with no workspace
 *     yet runs a kernel that needs none, whose summation order, and so
 *     whose last bits, may differ.)
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    W4A16_OK = 0,
    W4A16_ERR_NULL = 1,    /* a required pointer is null (M > 0) */
    W4A16_ERR_SHAPE = 2,   /* M < 0, K <= 0, N <= 0, K % 16 != 0, N % 8 != 0, or a
                              buffer reaches 2^31 bytes */
    W4A16_ERR_GROUP = 3,   /* group_size not in {-1,16,32,64,128,256,512,1024} */
    W4A16_ERR_ALIGN = 4,   /* a device pointer is not 16-byte aligned */
    W4A16_ERR_CODE = 5,    /* pack_gptq_v2: a code above 15 */
    W4A16_ERR_DEVICE = 6,  /* no usable HIP device, or the current one is not gfx950 */
    W4A16_ERR_LAUNCH = 7,  /* the kernel launch reported an error */
    W4A16_ERR_KERNEL = 8,  /* w4a16_linear_ex: the requested kernel cannot take this M */
    W4A16_ERR_RANK = 9,    /* LoRA rank not a multiple of 8 in [8, W4A16_LORA_MAX_RANK] */
    W4A16_ERR_WORKSPACE = 10, /* workspace smaller than w4a16_lora_workspace_bytes or
                                 w4a16_zp_workspace_bytes gives */
    W4A16_ERR_CAPTURE = 11,   /* w4a16_stream_release: the stream is being captured */
    W4A16_ERR_SCRATCH = 12,   /* w4a16_linear_noalloc: the device has more CUs than its
                                 scratch covers */
    W4A16_ERR_FLAGS = 13      /* w4a16_linear_typed: an unknown flag bit, or flags that
                                 cannot go together */
} w4a16_status;

/* Largest M the small-batch (decode) kernel takes; larger M runs the MFMA
 * GEMM (prefill) kernel.  The split follows the pages' separate fused-decode
 * and Tensor-Core prefill paths ("GPTQ-Pro" README, "Ampere kernel
 * architecture"). */
#define W4A16_DECODE_MAX_M 16

/* y = x . dequant(qweight, scales) on the current HIP device.
 *   x, qweight, scales, y : device pointers, each 16-byte aligned
 *   M >= 0 rows of x (M == 0 returns W4A16_OK and does nothing);
 *   K > 0, K % 16 == 0 input features; N > 0, N % 8 == 0 output features;
 *   group_size in {-1, 16, 32, 64, 128, 256, 512, 1024};
 *   stream : hipStream_t to enqueue on (0 = null stream).
 * Dispatch: M <= W4A16_DECODE_MAX_M runs the decode kernel, larger M the
 * prefill kernel.  Returns a w4a16_status. */
int w4a16_linear(const void *x, const int32_t *qweight, const void *scales, void *y,
                 int64_t M, int64_t K, int64_t N, int64_t group_size, void *stream);

/* w4a16_linear for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, layouts, kernels and errors as w4a16_linear (fp16), plus
 * W4A16_ERR_SCRATCH on a device with more than 320 CUs.  It calls no
 * allocating routine: the split-K scratch lives in one file-scope device
 * array of 20,709,376 bytes (the decode workspace laid out for 320
 * workgroups, 3.75 MiB, and 64 prefill partial tiles of 256 KiB), which
 * every device the library runs on holds until the process ends.  Prefill
 * plans that would need more than 64 partial tiles split K into fewer chunks
 * (the result stays within the same bar; its last bits can differ from
 * w4a16_linear's for such shapes).  Every call on a device shares that
 * device's array: calls that overlap in time on one device (two streams, or
 * a graph replayed beside eager calls) race and give wrong results; calls in
 * one stream's order do not.  Graph-capturable from the first call. */
int w4a16_linear_noalloc(const void *x, const int32_t *qweight, const void *scales, void *y,
                         int64_t M, int64_t K, int64_t N, int64_t group_size, void *stream);

/* Kernel selectors for w4a16_linear_ex. */
#define W4A16_KERNEL_AUTO 0     /* same choice as w4a16_linear */
#define W4A16_KERNEL_DECODE 1   /* small-batch kernel; requires M <= W4A16_DECODE_MAX_M */
#define W4A16_KERNEL_PREFILL 2  /* MFMA GEMM kernel; any M */

/* As w4a16_linear, with the kernel chosen by the caller (tests and crossover
 * measurements).  Same arguments, layouts and errors, plus W4A16_ERR_KERNEL
 * when `kernel` is unknown or cannot take M. */
int w4a16_linear_ex(const void *x, const int32_t *qweight, const void *scales, void *y,
                    int64_t M, int64_t K, int64_t N, int64_t group_size, void *stream,
                    int kernel);

/* y = x . dequant(qweight, scales) with bfloat16 activations and output: the
 * dtype the pages serve this checkpoint with ("Qwen3.8-27B-GPTQ-Int4" model
 * card, "4. Deployment": the verified serving command passes the bfloat16
 * dtype; the "GPTQ-Pro" README's "Runtime contract" keeps native BF16
 * outside its own kernels).
 *   x : device bfloat16 [M, K];  y : device bfloat16 [M, N];
 *   qweight, scales (fp16), shapes, group sizes, alignment, stream, dispatch,
 *   errors and workspaces exactly as for w4a16_linear.
 * Arithmetic: products accumulate in fp32 and y is rounded once to bfloat16
 * (nearest even).  Prefill, and decode with g = 16, form every weight
 * (q - 8) * s exactly in fp32 and round it once to bfloat16 for the bfloat16
 * matrix instructions; decode with g >= 32 (or -1) sums x * (128 + q), exact
 * in bfloat16, and x * 136 over each group and takes s * (the difference) in
 * fp32 (a group whose codes are all 8 adds exactly zero).
 * Hence, per element, |y - y_exact| <= 2^-8 |y_exact|
 *   + (2^-8 + K 2^-24) sum_k |x||w| + 35 K 2^-24 * 8 sum_k |x| s
 * (each rounding at most half a bfloat16 ulp; fp32 accumulation, including
 * the cancellation of the 128 offset).
 * Results are deterministic, as for fp16. */
int w4a16_linear_bf16(const void *x, const int32_t *qweight, const void *scales, void *y,
                      int64_t M, int64_t K, int64_t N, int64_t group_size, void *stream);

/* As w4a16_linear_bf16 with the kernel chosen by the caller, as in
 * w4a16_linear_ex. */
int w4a16_linear_bf16_ex(const void *x, const int32_t *qweight, const void *scales, void *y,
                         int64_t M, int64_t K, int64_t N, int64_t group_size, void *stream,
                         int kernel);

/* Merged gate/up projection with the SiLU * mul epilogue fused: the pages'
 * engines merge gate_proj and up_proj into one gate_up_proj module ("GPT-QModel"
 * README, "Dynamic Quantization": "Fused Modules in Inference Engines") and
 * serve with the fused silu_and_mul op ("Qwen3.8-27B GPTQ-Pro Hybrid INT8"
 * model card, "Text-only serving").
 *   qweight int32 [K/8, N], scales fp16 [G, N]: the columns alternate gate
 *     (even n) and up (odd n), each column in the GPTQ_V2 layout above (the
 *     caller merges gate_proj and up_proj by interleaving their columns);
 *   y : device [M, N/2], y[m,j] = silu(g) * u with g, u the fp32 sums of
 *     columns 2j and 2j+1 (never rounded), silu(z) = z / (1 + e^-z) in fp32,
 *     rounded once to the output type;
 *   N % 16 == 0 (else W4A16_ERR_SHAPE), everything else as for w4a16_linear.
 * The _bf16 forms take bfloat16 x and write bfloat16 y (arithmetic as in
 * w4a16_linear_bf16); the _ex forms choose the kernel as w4a16_linear_ex.
 * Prefill splits K as the linear does; split tiles' fp32 sums are added in
 * a fixed order and SiLU * mul is applied to the sums, as above. */
int w4a16_gate_up_silu(const void *x, const int32_t *qweight, const void *scales, void *y,
                       int64_t M, int64_t K, int64_t N, int64_t group_size, void *stream);
int w4a16_gate_up_silu_ex(const void *x, const int32_t *qweight, const void *scales, void *y,
                          int64_t M, int64_t K, int64_t N, int64_t group_size, void *stream,
                          int kernel);
int w4a16_gate_up_silu_bf16(const void *x, const int32_t *qweight, const void *scales, void *y,
                            int64_t M, int64_t K, int64_t N, int64_t group_size, void *stream);
int w4a16_gate_up_silu_bf16_ex(const void *x, const int32_t *qweight, const void *scales,
                               void *y, int64_t M, int64_t K, int64_t N, int64_t group_size,
                               void *stream, int kernel);

/* LoRA adapter on the quantised linear: y = x . dequant(qweight, scales)
 * + s * (x . A^T) . B^T.  The pages list LoRA adapters on the quantised
 * linear path in the runtime contract ("GPTQ-Pro" README, "Runtime contract"
 * table), keep the adapter beside the packed weights rather than merged into
 * them ("GPT-QModel" README, "PEFT LoRA Training and Adapter Loading") and
 * suggest ranks 32 and 64, with 128 and 256 as larger choices ("EoRA Accuracy
 * Recovery").  The update is the textbook low-rank one in PEFT's storage
 * order:
 *   lora_a : device [rank, K], the activation type (lora_A weight)
 *   lora_b : device [N, rank], the activation type (lora_B weight)
 *   lora_scale : s (alpha / rank for plain LoRA), applied in fp32
 *   rank : a multiple of 8 in [8, W4A16_LORA_MAX_RANK] (else W4A16_ERR_RANK)
 *   workspace : device buffer of at least w4a16_lora_workspace_bytes(M, K,
 *     rank) bytes, 16-byte aligned, no initial contents, owned by the caller;
 *     calls that overlap in time must not share one (else a race).  Too small:
 *     W4A16_ERR_WORKSPACE.
 *   x, qweight, scales, y, shapes, group sizes, stream and the other errors
 *   as for w4a16_linear (the _bf16 form: bfloat16 x, A, B and y, as for
 *   w4a16_linear_bf16).  All checks run before any HIP call.
 * Steps on the stream:
 *   - M <= W4A16_DECODE_MAX_M with rank <= 128, M * rank <= 512 and
 *     ceil(K / 256) * M * rank <= 4096, when the decode runs its stream-K
 *     launch (a stream that already holds its workspace, or one that may
 *     create it): one launch.  Its first ceil(K / 256) workgroups also sum
 *     t = x . A^T over 256-deep slices of K in fp32 on the matrix cores; after
 *     its main loop every workgroup adds the slices in slice order, rounds
 *     s * t to the activation type (t') and adds t' . B^T (fp32, matrix
 *     cores) to its fp32 sums before the one rounding of y.  The slices pass
 *     through the library's workspace for the stream, which the launch leaves
 *     as it found it; the caller's workspace holds t' for the split-K reduce.
 *   - M > W4A16_DECODE_MAX_M: a shrink kernel forms t = x . A^T as fp32
 *     partial sums over chunks of K; a second adds the chunks in a fixed
 *     order and rounds s * t to the activation type (t'); the prefill linear
 *     adds t' . B^T (fp32, matrix cores) to its fp32 sums before the one
 *     rounding of y (for a tile split along K, to the first chunk's partial);
 *   - otherwise (a decode outside the one-launch limits, or captured on a
 *     stream with no workspace yet): the linear writes y; a shrink kernel
 *     forms t = x . A^T as fp32 partial sums over chunks of K; an expand
 *     kernel adds the chunks in a fixed order, rounds t to the activation
 *     type, forms delta = t . B^T in fp32 on the matrix cores and writes
 *     y = round(y + s * delta).
 * Hence, per element and beyond the linear's own bound (u = 2^-11 for fp16,
 * 2^-8 for bfloat16): u |y_lin| + u |y| + |s| sum_j |B[n,j]| (u |t_j|
 * + K 2^-24 sum_k |x[m,k]| |A[j,k]|) + rank 2^-24 |s| sum_j |t_j| |B[n,j]|,
 * to first order (the one-launch form rounds s t_j, and y once: within the
 * same terms); fp16 needs every t_j inside the fp16 range.
 * Deterministic, as w4a16_linear. */
#define W4A16_LORA_MAX_RANK 1024
int w4a16_linear_lora(const void *x, const int32_t *qweight, const void *scales,
                      const void *lora_a, const void *lora_b, float lora_scale, void *y,
                      int64_t M, int64_t K, int64_t N, int64_t group_size, int64_t rank,
                      void *workspace, size_t workspace_bytes, void *stream);
int w4a16_linear_lora_bf16(const void *x, const int32_t *qweight, const void *scales,
                           const void *lora_a, const void *lora_b, float lora_scale, void *y,
                           int64_t M, int64_t K, int64_t N, int64_t group_size, int64_t rank,
                           void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace w4a16_linear_lora needs for (M, K, rank): fp32 partial
 * sums of x . A^T, at most 16 chunks of [M rounded up to 16, rank] (and room
 * for t' of the one-launch form).  0 for M <= 0 or arguments the linear
 * would reject. */
size_t w4a16_lora_workspace_bytes(int64_t M, int64_t K, int64_t rank);

/* Asymmetric weights with stored zero points: w[k,n] = (q[k,n] - z[k/g, n]) *
 * scales[k/g][n] in place of the symmetric (q - 8) * s.  GPTQModel quantises
 * with sym=False and stores per-group zero points, which the GPTQ-Pro contract
 * leaves out ("GPTQ-Pro" README, "Runtime contract"); the pages say only that
 * the v1 and v2 checkpoint formats store them differently.
 *   qzeros : device int32 [G, N/8], 16-byte aligned: nibble j (bits 4j..4j+3)
 *     of word [g][c] is the zero point of column 8c + j, read as unsigned and
 *     used as stored (the v2 form; w4a16_linear_typed with W4A16_ZEROS_V1
 *     takes the v1 form).  It is pack_gptq_v2 applied to the transposed [N, G] zero
 *     points, transposed back.
 *   workspace : device buffer of at least w4a16_zp_workspace_bytes(M, K, N,
 *     group_size) bytes, 16-byte aligned, no initial contents, owned by the
 *     caller; calls that overlap in time must not share one.
 *   ceil(G / 8) * 8 <= 1536 (else W4A16_ERR_SHAPE); everything else as for
 *   w4a16_linear (the _bf16 form: bfloat16 x and y, as w4a16_linear_bf16).
 * Steps on the stream: since (q - z) s = (q - 8) s + (8 - z) s,
 *   - M <= W4A16_DECODE_MAX_M: one launch of the decode kernel, which sums x
 *     over each group on the matrix cores beside the symmetric sums and adds
 *     s (8 - z) times that sum per group and column in fp32 (for g = 16 the
 *     zero point enters the dequantised weight: fp16 (q - z) s rounded once,
 *     bfloat16 (q - z) s exact in fp32 and rounded once); the workspace is
 *     not touched;
 *   - larger M: one kernel sums x over each group in fp32 (X[m, g], rounded
 *     to the activation type) and forms C[g, n] = (8 - z) s exactly in
 *     fp32, rounded to the activation type; the symmetric prefill linear adds
 *     X . C (fp32, matrix cores) to its fp32 sums before the one rounding of
 *     y (for a tile split along K, to the first chunk's partial).
 * Where every zero point is 8 the correction is 0 and y is the symmetric
 * result (bit for bit, up to the sign of a zero).
 * Hence, per element and beyond the symmetric linear's own bound (u = 2^-11
 * for fp16, 2^-8 for bfloat16): u |y_sym| + u |y| + (2u + K 2^-24) P, to
 * first order, with P = sum_k |x[m,k]| |8 - z| s (the magnitude of the
 * correction).  Deterministic, as w4a16_linear. */
int w4a16_linear_zp(const void *x, const int32_t *qweight, const void *scales,
                    const int32_t *qzeros, void *y, int64_t M, int64_t K, int64_t N,
                    int64_t group_size, void *workspace, size_t workspace_bytes, void *stream);
int w4a16_linear_zp_bf16(const void *x, const int32_t *qweight, const void *scales,
                         const int32_t *qzeros, void *y, int64_t M, int64_t K, int64_t N,
                         int64_t group_size, void *workspace, size_t workspace_bytes,
                         void *stream);

/* Bytes of workspace w4a16_linear_zp needs: an area of (M rounded up to 16)
 * x Gp fp32 values for the group sums of x (stored in the activation type),
 * then the correction matrix C^T [N, Gp] in the activation type, Gp = G
 * rounded up to 8.  0 for M <= 0 or arguments it rejects. */
size_t w4a16_zp_workspace_bytes(int64_t M, int64_t K, int64_t N, int64_t group_size);

/* Flags of w4a16_linear_typed. */
#define W4A16_X_BF16 0x1u        /* x and y bfloat16, else fp16 */
#define W4A16_SCALES_BF16 0x2u   /* scales bfloat16, else fp16; needs W4A16_X_BF16 */
#define W4A16_ZEROS_V1 0x4u      /* qzeros in the v1 checkpoint form; needs qzeros */
#define W4A16_GATE_UP_SILU 0x8u  /* merged gate/up with SiLU * mul; not with qzeros */

/* Every variant of the linear behind one call, chosen by flags (bitwise OR of
 * the W4A16_ flags above) and by whether qzeros is null:
 *   - qzeros null: w4a16_linear_ex (no flags), w4a16_linear_bf16_ex
 *     (W4A16_X_BF16), w4a16_gate_up_silu_ex / _bf16_ex (W4A16_GATE_UP_SILU);
 *     workspace is not used and may be null;
 *   - qzeros given: w4a16_linear_zp / _bf16, steps as there, with `kernel`
 *     choosing them: W4A16_KERNEL_AUTO as w4a16_linear_zp, W4A16_KERNEL_DECODE
 *     the one-launch decode path (M <= W4A16_DECODE_MAX_M, else
 *     W4A16_ERR_KERNEL), W4A16_KERNEL_PREFILL the symmetric prefill linear
 *     followed by the correction.  The workspace (w4a16_zp_workspace_bytes,
 *     as for w4a16_linear_zp) is needed only on the correction path and may
 *     be null on the one-launch path.
 * W4A16_SCALES_BF16: scales are bfloat16 bit patterns.  A checkpoint served
 * in bfloat16 carries its scales in that dtype ("Qwen3.8-27B-GPTQ-Int4" model
 * card, "4. Deployment": the verified serving command uses the bfloat16
 * dtype).  Each scale enters the arithmetic exactly where an fp16 scale does
 * on the bfloat16 path (both convert to fp32 exactly), so the error bounds of
 * the bfloat16 forms hold unchanged.  fp16 activations take fp16 scales only
 * (W4A16_ERR_FLAGS).
 * W4A16_ZEROS_V1: the nibble holds z - 1, so z = nibble + 1, in [1, 16].  The
 * pages name a GPTQ v1 checkpoint form beside v2 ("GPT-QModel" README, "Quant
 * Method / Format / Backend Matrix"; "Norm tuning": v1 zero points read as
 * they are decode the weights wrongly) but print no rule; this is the
 * published GPTQ one, under which a symmetric checkpoint stores 7 in every
 * nibble.
 * Everything else (pointers, shapes, group sizes, alignment, determinism,
 * the bounds) as for the entry point each combination names above.  Returns
 * W4A16_ERR_FLAGS for an unknown bit, W4A16_SCALES_BF16 without
 * W4A16_X_BF16, W4A16_ZEROS_V1 without qzeros, or W4A16_GATE_UP_SILU with
 * qzeros, before any HIP call. */
int w4a16_linear_typed(const void *x, const int32_t *qweight, const void *scales,
                       const int32_t *qzeros, void *y, int64_t M, int64_t K, int64_t N,
                       int64_t group_size, unsigned flags, int kernel, void *workspace,
                       size_t workspace_bytes, void *stream);

/* Frees the workspaces the library holds for `stream` on the current device
 * (a hipStream_t, 0 = null stream), after waiting for the work queued on it.
 * The next call on that stream creates them again.  Returns W4A16_OK (also
 * when none are held), W4A16_ERR_CAPTURE while the stream is being captured
 * (nothing is freed), W4A16_ERR_DEVICE without a usable device, or
 * W4A16_ERR_LAUNCH when waiting for the stream fails. */
int w4a16_stream_release(void *stream);

/* Host-side packing into the GPTQ_V2 layout (native int32 qweight, "GPTQ-Pro"
 * README, "Runtime contract"):
 *   qweight[r][n] = sum_{j=0..7} codes[8r+j][n] << 4j   (as a 32-bit pattern)
 *   codes   : host uint8 [K, N], every value in 0..15
 *   qweight : host int32 [K/8, N]
 * Requires K > 0, K % 8 == 0, N > 0.  Returns W4A16_ERR_CODE (and leaves
 * qweight unspecified) when a code exceeds 15. */
int pack_gptq_v2(const uint8_t *codes, int32_t *qweight, int64_t K, int64_t N);

/* Exact inverse of pack_gptq_v2: host int32 [K/8, N] -> host uint8 [K, N]. */
int unpack_gptq_v2(const int32_t *qweight, uint8_t *codes, int64_t K, int64_t N);

/* Streaming-read probe, a measurement aid beside the linear (the pages ask
 * for achieved HBM bandwidth against peak for decode; this gives the
 * attainable read rate on the device, measured with a plain kernel):
 * reads `bytes` bytes at `data` once with 16-byte non-temporal loads spread
 * over the whole device.
 *   data   : device pointer, 16-byte aligned; bytes > 0, bytes % 16 == 0
 *   sink   : device pointer to 4 writable bytes, 4-byte aligned (written
 *            only when the XOR of the words one thread read equals a fixed
 *            constant; its contents mean nothing)
 *   stream : hipStream_t to enqueue on (0 = null stream)
 * Returns W4A16_ERR_SHAPE, _NULL, _ALIGN, _DEVICE or _LAUNCH on failure,
 * before any HIP call for the first three. */
int w4a16_read_probe(const void *data, int64_t bytes, void *sink, void *stream);

/* Static, human-readable name of a status code (never null). */
const char *w4a16_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
