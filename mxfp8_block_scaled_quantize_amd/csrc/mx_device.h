// Device helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) 16-byte global accesses for data touched once.
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_nt16(void* p, uint4 d) {
  const u32x4 v = {d.x, d.y, d.z, d.w};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// Packed per-halfword unsigned max (v_pk_max_u16).  Non-negative BF16 values
// order like their bit patterns, so |x| max is an integer max on bits & 0x7FFF.
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}

__device__ __forceinline__ uint32_t abs_bits2(uint32_t w) { return w & 0x7FFF7FFFu; }

// BF16 halves of a dword as fp32 (exact: BF16 is the top half of binary32).
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// E8M0 byte of a block from the 15-bit magnitude pattern of its amax.
// floor(log2 amax) - 8 + 127 is (biased exponent field - 8); subnormal or zero
// amax (exponent field 0) and anything below 2^-119 clamp to byte 0.
__device__ __forceinline__ uint32_t scale_byte_from_amax(uint32_t amax_bits) {
  int e = (int)(amax_bits >> 7);
  return (uint32_t)(e > 8 ? e - 8 : 0);
}

// 2^-(byte-127) as fp32: always a normal number for bytes 0..246.
__device__ __forceinline__ float inv_scale(uint32_t byte) {
  return __uint_as_float((254u - byte) << 23);
}

// v_cvt_pk_fp8_f32 rounds to nearest even and handles E4M3 subnormals, but it
// turns magnitudes above 464 into NaN: clamp to the saturation value first.
__device__ __forceinline__ float sat448(float v) { return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f); }

// Four fp32 values (already multiplied by the inverse scale) -> four E4M3 bytes.
__device__ __forceinline__ uint32_t cvt4_e4m3(float a, float b, float c, float d) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(c), sat448(d), r, true);
  return (uint32_t)r;
}

// Cross-lane max inside a quad of lanes via DPP quad permutes.
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  uint32_t t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);  // lane ^ 1
  v = v > t ? v : t;
  t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);           // lane ^ 2
  return v > t ? v : t;
}

// fp32 -> bf16 round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

}  // namespace mx
