// Device-side building blocks shared by the gfx950 W4A16 kernels.
//
// The operation is the symmetric-INT4 GPTQ linear of the "GPTQ-Pro" README
// ("Runtime contract" table): y = x . W with W[k,n] = (q[k,n] - 8) * s[k/g, n],
// FP16 activations, int32-packed codes (nibble j of qweight row r = K index
// 8r+j, low bits first) and fp32 accumulation ("Ampere kernel architecture":
// the prefill path accumulates in FP32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b2 __attribute__((ext_vector_type(2)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// Raw (stride-0) buffer resources, gfx9 family: a load whose byte offset is at
// or past the record count returns zero, a store there is dropped.  Every
// buffer handed to the kernels is smaller than 2^31 bytes (the host checks),
// so kOOB is out of range for all of them.
constexpr int kRsrcWord3 = 0x00020000;
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                             kRsrcWord3);
}

__device__ __forceinline__ u4 load_b128(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

// 16-byte load with the non-temporal hint (data read once, streamed past the
// caches): cache policy bit 1 is "nt" on gfx950.
__device__ __forceinline__ u4 load_b128_nt(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 2));
}

__device__ __forceinline__ u2 load_b64(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0));
}

// Register-resident constants of the nibble unpack.  gfx9 VOP3 encodings take
// no literal operands, so the masks and the fp16 bias live in VGPRs; the
// empty asm makes them opaque so every unpack step stays one v_and_or_b32.
struct UnpackConsts {
    uint32_t lo;      // 0x000F000F: nibbles 0 and 4 of a (shifted) word
    uint32_t hi;      // 0x00F000F0: nibbles 1 and 5
    uint32_t magic;   // 0x64006400: fp16 1024.0 in both halves
};

__device__ __forceinline__ UnpackConsts unpack_consts() {
    UnpackConsts c{0x000F000Fu, 0x00F000F0u, 0x64006400u};
    asm volatile("" : "+v"(c.lo), "+v"(c.hi), "+v"(c.magic));
    return c;
}

// The eight 4-bit codes of one qweight word as eight fp16 values (q - 8), in
// the order (q0, q4, q1, q5, q2, q6, q3, q7).  OR-ing a nibble into the low
// mantissa bits of fp16 1024.0 (0x6400) makes the half read as 1024 + q, and
// subtracting 1032 leaves q - 8 exactly (the int->fp16 "magic number"
// conversion published by Kim et al. (2022), "Who Says Elephants Can't Run?").
// Nibbles 1/5 (and 3/7 after one shift) are taken in place at bits 4..7, so
// they read as 1024 + 16q; one fma by 1/16 with -72 maps them to q - 8, also
// exactly.  Cost per word: 5 bit operations and 4 packed fp16 operations.
__device__ __forceinline__ h8 unpack_codes(uint32_t w, const UnpackConsts &c) {
    const h2 bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2 bias16 = {(_Float16)-72.0f, (_Float16)-72.0f};
    const uint32_t w8 = w >> 8;
    const h2 p0 = __builtin_bit_cast(h2, (w & c.lo) | c.magic) + bias;
    const h2 p1 = __builtin_elementwise_fma(__builtin_bit_cast(h2, (w & c.hi) | c.magic),
                                            sixteenth, bias16);
    const h2 p2 = __builtin_bit_cast(h2, (w8 & c.lo) | c.magic) + bias;
    const h2 p3 = __builtin_elementwise_fma(__builtin_bit_cast(h2, (w8 & c.hi) | c.magic),
                                            sixteenth, bias16);
    const u4 r = {__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                  __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
    return __builtin_bit_cast(h8, r);
}

// Same, each value multiplied by the fp16 scale s (one rounding: RNE((q-8)*s)).
__device__ __forceinline__ h8 unpack_codes_scaled(uint32_t w, const UnpackConsts &c,
                                                  _Float16 s) {
    const h8 v = unpack_codes(w, c);
    const h8 sv = {s, s, s, s, s, s, s, s};
    return v * sv;
}

// Eight consecutive fp16 activations k0..k7 (one 16-byte load, dwords
// (k0,k1),(k2,k3),(k4,k5),(k6,k7)) reordered to (k0,k4,k1,k5,k2,k6,k3,k7),
// the order unpack_codes gives the weights.  Applying the same permutation
// to both MFMA operands leaves every dot product unchanged.  v_perm_b32
// picks bytes 0-3 from its second operand and 4-7 from its first.
__device__ __forceinline__ u4 perm_x(u4 d) {
    u4 r;
    r.x = __builtin_amdgcn_perm(d.z, d.x, 0x05040100u);
    r.y = __builtin_amdgcn_perm(d.z, d.x, 0x07060302u);
    r.z = __builtin_amdgcn_perm(d.w, d.y, 0x05040100u);
    r.w = __builtin_amdgcn_perm(d.w, d.y, 0x07060302u);
    return r;
}

// Four consecutive fp16 scales (one 8-byte load) as floats / halves.
__device__ __forceinline__ _Float16 half_lo(uint32_t v) {
    return __builtin_bit_cast(h2, v).x;
}
__device__ __forceinline__ _Float16 half_hi(uint32_t v) {
    return __builtin_bit_cast(h2, v).y;
}

// The low / high 16-bit value of a dword as fp32: bfloat16 (BF: the top half
// of an fp32, exact) or fp16 (converted, exact).
template <bool BF>
__device__ __forceinline__ float lo_f32(uint32_t v) {
    if constexpr (BF) return __uint_as_float(v << 16);
    else return (float)half_lo(v);
}
template <bool BF>
__device__ __forceinline__ float hi_f32(uint32_t v) {
    if constexpr (BF) return __uint_as_float(v & 0xFFFF0000u);
    else return (float)half_hi(v);
}

// D(16x16, fp32) += A(16x32, fp16) * B(32x16, fp16) on the matrix cores.
// Lane l supplies A row (l % 16) and B column (l % 16), each as 8 values of
// K-block (l / 16); it receives D rows 4*(l/16) .. 4*(l/16)+3 of column l % 16.
__device__ __forceinline__ f4 mfma16x16x32(h8 a, h8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// D(32x32, fp32) += A(32x16, fp16) * B(16x32, fp16) on the matrix cores.
// Lane l supplies A row (l % 32) and B column (l % 32), each as 8 values of
// K-block (l / 32); register i of lane l receives D row
// 8*(i/4) + 4*(l/32) + i%4 of column l % 32.  One wave per SIMD keeps the
// matrix core busy with this instruction, which it does not with 16x16x32.
__device__ __forceinline__ f16v mfma32x32x16(h8 a, h8 b, f16v c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Four fp32 values -> four fp16 (round to nearest even) packed in 8 bytes.
__device__ __forceinline__ u2 pack4_f16(float a, float b, float c, float d) {
    h2 lo = {(_Float16)a, (_Float16)b};
    h2 hi = {(_Float16)c, (_Float16)d};
    u2 r = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
    return r;
}

// ---- the activation type: fp16, or bfloat16 when BF ----
// bfloat16 activations and outputs are the pages' serving dtype for this
// checkpoint ("Qwen3.8-27B-GPTQ-Int4" model card, "4. Deployment"); scales
// stay fp16 and accumulation fp32.

// Two fp32 values rounded to nearest even in the activation type, packed
// low-first in one dword (bfloat16: one v_cvt_pk_bf16_f32).
template <bool BF>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    if constexpr (BF) {
        const b2 v = {(__bf16)a, (__bf16)b};
        return __builtin_bit_cast(uint32_t, v);
    } else {
        const h2 v = {(_Float16)a, (_Float16)b};
        return __builtin_bit_cast(uint32_t, v);
    }
}

template <bool BF>
__device__ __forceinline__ u2 pack4(float a, float b, float c, float d) {
    return u2{pack2<BF>(a, b), pack2<BF>(c, d)};
}

// v rounded to the activation type (nearest even), as fp32.
template <bool BF>
__device__ __forceinline__ float round_act(float v) {
    return lo_f32<BF>(pack2<BF>(v, 0.f));
}

// ---- final stores: plain, or the merged gate/up projection's SiLU * mul ----
// With SILU the columns alternate gate (even) and up (odd) and the pair
// (gate, up) becomes one value silu(gate) * up at column n/2 of a y with N/2
// columns (vLLM's silu_and_mul, which the pages serve with: "Qwen3.8-27B
// GPTQ-Pro Hybrid INT8" model card, "Text-only serving"), taken from the fp32
// sums before any rounding.  SiLU(z) = z / (1 + e^-z).
__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + __expf(-z)); }

// Columns n, n + 1 (n even) of row m.
template <bool BF, bool SILU>
__device__ __forceinline__ void store_pair(uint16_t *y, int64_t m, int N, int n, float a,
                                           float b) {
    if constexpr (SILU)
        y[m * (N / 2) + n / 2] = (uint16_t)pack2<BF>(silu_f32(a) * b, 0.f);
    else
        *reinterpret_cast<uint32_t *>(y + m * N + n) = pack2<BF>(a, b);
}

// Columns n .. n + 3 (n % 4 == 0) of row m.
template <bool BF, bool SILU>
__device__ __forceinline__ void store_quad(uint16_t *y, int64_t m, int N, int n,
                                           const float (&v)[4]) {
    if constexpr (SILU)
        *reinterpret_cast<uint32_t *>(y + m * (N / 2) + n / 2) =
            pack2<BF>(silu_f32(v[0]) * v[1], silu_f32(v[2]) * v[3]);
    else
        *reinterpret_cast<u2 *>(y + m * N + n) = pack4<BF>(v[0], v[1], v[2], v[3]);
}

// The MFMAs above on 16-bit operands given as raw bits (eight values each).
template <bool BF>
__device__ __forceinline__ f4 mfma16x16x32_t(u4 a, u4 b, f4 c) {
    if constexpr (BF)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, a),
                                                       __builtin_bit_cast(b8, b), c, 0, 0, 0);
    else
        return mfma16x16x32(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c);
}

template <bool BF>
__device__ __forceinline__ f16v mfma32x32x16_t(u4 a, u4 b, f16v c) {
    if constexpr (BF)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(b8, a),
                                                       __builtin_bit_cast(b8, b), c, 0, 0, 0);
    else
        return mfma32x32x16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c);
}

// One byte of a dword as fp32 (v_cvt_f32_ubyte<d>).
__device__ __forceinline__ float ubyte_f32(uint32_t v, int d) {
    return (float)((v >> (8 * d)) & 0xFFu);
}

// The eight codes of word w as bfloat16 128 + q, exactly (q in the low
// mantissa bits of 128.0 = 0x4300), in the fp16 unpack order (q0, q4, q1,
// q5, q2, q6, q3, q7): one v_and_or_b32 per pair.  A sum of x * (128 + q)
// minus the sum of x * 136 is the sum of x * (q - 8).
__device__ __forceinline__ u4 codes128_bf16(uint32_t w, const UnpackConsts &c) {
    const uint32_t magic = 0x43004300u;
    u4 r;
    r[0] = (w & c.lo) | magic;
    r[1] = ((w >> 4) & c.lo) | magic;
    r[2] = ((w >> 8) & c.lo) | magic;
    r[3] = ((w >> 12) & c.lo) | magic;
    return r;
}

// The eight weights of word w as bfloat16: (q - 8) * s computed in fp32 as
// fma(q, s, -8 s), exact there (a 4-bit integer times an fp16 scale), then
// rounded once to nearest even.  gfx950 has no packed bfloat16 arithmetic,
// so the magic-number trick of the fp16 path does not carry over.  lo holds
// the even nibbles in its bytes (q0, q2, q4, q6), hi the odd ones.
// NATURAL: order (q0, q1, ..., q7), else the fp16 unpack order (q0, q4, q1,
// q5, q2, q6, q3, q7).
// With a stored zero point z the offset term is -z s instead of -8 s (exact
// in fp32 as well): pass zoff = -z s.
template <bool NATURAL>
__device__ __forceinline__ u4 dequant_bf16(uint32_t w, float s, float zoff) {
    const float m8s = zoff;
    uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    // opaque, so that each nibble is one v_cvt_f32_ubyte<d> of the masked
    // word rather than a bit-field extract and a convert
    asm volatile("" : "+v"(lo), "+v"(hi));
    auto wq = [&](uint32_t src, int d) { return __builtin_fmaf(ubyte_f32(src, d), s, m8s); };
    u4 r;
    if constexpr (NATURAL) {
#pragma unroll
        for (int d = 0; d < 4; ++d) r[d] = pack2<true>(wq(lo, d), wq(hi, d));
    } else {
        r[0] = pack2<true>(wq(lo, 0), wq(lo, 2));
        r[1] = pack2<true>(wq(hi, 0), wq(hi, 2));
        r[2] = pack2<true>(wq(lo, 1), wq(lo, 3));
        r[3] = pack2<true>(wq(hi, 1), wq(hi, 3));
    }
    return r;
}

template <bool NATURAL>
__device__ __forceinline__ u4 dequant_bf16(uint32_t w, float s) {
    return dequant_bf16<NATURAL>(w, s, -8.0f * s);
}

}  // namespace w4a16
