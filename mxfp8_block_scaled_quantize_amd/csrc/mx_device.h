// Device helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Streaming (non-temporal) global stores and loads: data written or read once
// in a pass (the GEMM's output tile; the tile quantizer's inputs and row codes).
__device__ __forceinline__ void store_nt16(void* p, uint4 d) {
  const u32x4 v = {d.x, d.y, d.z, d.w};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void store_nt8(void* p, uint2 d) {
  const u32x2 v = {d.x, d.y};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
}
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Packed per-halfword unsigned max / min (v_pk_max_u16 / v_pk_min_u16).
// Non-negative BF16 values order like their bit patterns, so |x| max is an
// integer max on bits & 0x7FFF.
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}
__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}

__device__ __forceinline__ uint32_t abs_bits2(uint32_t w) { return w & 0x7FFF7FFFu; }

// BF16 halves of a dword as fp32 (exact: BF16 is the top half of binary32).
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// BF16 value t (0..3) of four packed in two dwords (little-endian), as fp32.
__device__ __forceinline__ float bf16_half2(u32x2 w, int t) {
  const uint32_t d = t < 2 ? w.x : w.y;
  return (t & 1) ? bf_hi(d) : bf_lo(d);
}

// E8M0 byte of a block from the 15-bit magnitude pattern of its amax.
// floor(log2 amax) - 8 + 127 is (biased exponent field - 8); subnormal or zero
// amax (exponent field 0) and anything below 2^-118 clamp to byte 0.
__device__ __forceinline__ uint32_t scale_byte_from_amax(uint32_t amax_bits) {
  int e = (int)(amax_bits >> 7);
  return (uint32_t)(e > 8 ? e - 8 : 0);
}

// BF16 magnitude pattern of 448 * 2^(byte - 127), the largest value a block
// with this scale byte encodes (1.75 * 2^(byte - 119): exponent field
// byte + 8, mantissa 0x60).  Always a normal finite BF16 for bytes 0..246.
__device__ __forceinline__ uint32_t sat_limit_bits(uint32_t byte) { return ((byte + 8u) << 7) | 0x60u; }

// Clamp the magnitudes of two BF16 values to the packed limits, keeping the
// signs.  RNE sends (448, 464] * 2^X to 448 * 2^X anyway, so clamping to
// 448 * 2^X changes no code except that values the convert would turn into
// NaN (above 464 * 2^X) saturate.
__device__ __forceinline__ uint32_t clamp_bf16x2(uint32_t w, uint32_t lim2) {
  return (w & 0x80008000u) | pk_min_u16(abs_bits2(w), lim2);
}

// Four BF16 values (two dwords, already clamped) -> four E4M3 bytes of
// x / 2^(byte - 127).  v_cvt_scalef32_pk_fp8_bf16 divides by two to the power
// of the exponent field of its fp32 scale operand (the fp32 with bits
// byte << 23, i.e. the E8M0 scale itself, byte 0 included) and rounds to
// nearest even with E4M3 subnormals; this was measured on every BF16 pattern
// for every scale byte 0..254.
__device__ __forceinline__ uint32_t cvt4_scaled(uint32_t c0, uint32_t c1, uint32_t byte) {
  const float f = __uint_as_float(byte << 23);
  i16x2 r = {0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2, c0), f, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2, c1), f, true);
  return __builtin_bit_cast(uint32_t, r);
}

// Eight consecutive BF16 values of one block -> eight E4M3 codes.
__device__ __forceinline__ uint2 quantize8(uint4 v, uint32_t byte) {
  uint32_t lim = sat_limit_bits(byte);
  lim |= lim << 16;
  uint2 o;
  o.x = cvt4_scaled(clamp_bf16x2(v.x, lim), clamp_bf16x2(v.y, lim), byte);
  o.y = cvt4_scaled(clamp_bf16x2(v.z, lim), clamp_bf16x2(v.w, lim), byte);
  return o;
}

// GELU(x) = x Phi(x) and GELU'(a) = Phi(a) + a phi(a), Phi / phi the
// standard normal distribution / density, in fp32 without branches.  Both
// come from the normal tail Phi(-t) = exp(-t^2 / 2) Q(t), t = |x|, where
// Q(t) = 0.5 erfcx(t / sqrt 2) (a scaled Mills ratio: smooth, Q(0) = 1/2,
// Q(t) ~ 1 / (t sqrt(2 pi))) is a (4, 5) rational fitted for this library by
// least squares on the relative error, reweighted toward the minimax, on
// [0, 14]: 3.1e-8 relative with the coefficients rounded to fp32, all of
// them positive, so Horner's rule stays accurate.  The tail keeps its
// relative accuracy where 1 + erf(x / sqrt 2) would cancel; Phi(x) for x > 0
// is 1 - Phi(-x).  t is clamped to 16 (exp(-128) is 0 in fp32, so nothing
// changes there but t^2 cannot overflow): huge inputs give GELU = x or -0 and
// GELU' = 1 or 0.
// Measured on every BF16 input against fp64: GELU within 0.87 (4 + 1.5 x^2)
// ulp, at most 64 (the rounding of the exponent -t^2 log2(e) / 2 grows with
// t^2); GELU' within 3.9 ulp of |Phi(a)| + |a phi(a)| for |a| <= 13 (the
// exponent is split into a rounded part and its exact residual, applied to
// first order; beyond 13 exp(-t^2 / 2) leaves fp32's normal range).  On
// arbitrary fp32 inputs (where t^2 itself rounds) GELU stays within
// 1.16 (4 + 1.5 x^2) ulp.  Each evaluation is about 25 VALU operations with
// one v_exp_f32 and one v_rcp_f32, without branches.
__device__ __forceinline__ float normal_tail_q(float t) {   // t in [0, 16]
  const float n = fmaf(fmaf(fmaf(fmaf(4.077574238e-03f, t, 4.037233070e-02f), t, 1.824611872e-01f), t,
                            4.372501075e-01f), t, 0.5f);
  const float d = fmaf(fmaf(fmaf(fmaf(fmaf(1.022083405e-02f, t, 1.012052298e-01f), t, 4.674274027e-01f), t,
                                 1.199288130e+00f), t, 1.672385097e+00f), t, 1.0f);
  return n * __builtin_amdgcn_rcpf(d);
}
constexpr float kNegHalfLog2e = -0.72134752044448170f;   // -log2(e) / 2, rounded to fp32
constexpr float kNegHalfLog2eLo = -9.6298149e-09f;       // -log2(e) / 2 - kNegHalfLog2e

__device__ __forceinline__ float gelu_f32(float x) {
  const float t = fminf(fabsf(x), 16.0f);
  const float p = __builtin_amdgcn_exp2f(t * t * kNegHalfLog2e) * normal_tail_q(t);   // Phi(-|x|)
  return x < 0.0f ? x * p : fmaf(-x, p, x);
}
__device__ __forceinline__ float dgelu_f32(float a) {
  const float t = fminf(fabsf(a), 16.0f);
  const float y = t * t;
  const float zh = y * kNegHalfLog2e;
  const float zl = fmaf(y, kNegHalfLog2eLo, fmaf(y, kNegHalfLog2e, -zh));   // exact residual + constant's tail
  float e = __builtin_amdgcn_exp2f(zh);
  e = fmaf(e * zl, 0.69314718055994531f, e);                                 // exp(-t^2 / 2)
  const float p = e * normal_tail_q(t);                                      // Phi(-|a|)
  return fmaf(a * 0.39894228040143268f, e, a < 0.0f ? p : 1.0f - p);
}

// SiLU(z) = z sigma(z) = z / (1 + exp(-z)) in fp32: one v_exp_f32 and one
// v_rcp_f32.  Measured on every BF16 input and 4M random fp32 inputs against
// fp64: within 1.14 (4 + |z|) ulp for |z| < 87.3.  Below z = -87.3 the
// reciprocal of 1 + exp(-z) leaves fp32's normal range and is flushed, so the
// result is -0 (the exact value there is below 1e-36); exp(-z) = +inf below
// -88.7 gives -0 as well, never a NaN.
__device__ __forceinline__ float silu_f32(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.44269504088896341f));
}

// Cross-lane max inside a quad of lanes via DPP quad permutes.
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  uint32_t t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);  // lane ^ 1
  v = v > t ? v : t;
  t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);           // lane ^ 2
  return v > t ? v : t;
}

}  // namespace mx
