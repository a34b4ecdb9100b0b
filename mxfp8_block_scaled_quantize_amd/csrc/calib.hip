// Measurement aid, not part of the MXFP8 library: the rate of the gfx950
// scaled FP8 MFMA when its operands never leave the registers, i.e. the
// ceiling of a GEMM that still had to move its operands from memory.
//
// Each workgroup has the GEMM kernel's shape: 4 waves, one per SIMD, each
// holding 16 blocks of 32 x 32 fp32 accumulators (256 AGPRs) and two sets of
// four A and four B E4M3 fragments (128 VGPRs) with their scale words.  An
// iteration issues the 16 block MFMAs of one fragment set and then of the
// other, so consecutive MFMAs see different operands, as in the GEMM's two
// K halves.  The operands come from a device buffer of random codes, and the
// accumulator sums are written out, so the compiler can neither fold nor drop
// the work.  FLOPs per launch: blocks * 4 * iters * 32 * 2 * 32 * 32 * 64.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace mxcal {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kCodeWords = 4096;   // random operand words read by the kernel

__global__ __launch_bounds__(256) void mfma_ceiling_kernel(const uint32_t* __restrict__ codes,
                                                           const uint32_t* __restrict__ scales,
                                                           float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  v8i fa[2][4], fb[2][4];
#pragma unroll
  for (int s = 0; s < 2; s++)
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int k = 0; k < 8; k++) {
        fa[s][i][k] = (int)codes[((((s * 4 + i) * 8 + k) * 64 + lane) * 7 + wave) % kCodeWords];
        fb[s][i][k] = (int)codes[((((s * 4 + i) * 8 + k) * 64 + lane) * 11 + 3 * wave + 1) % kCodeWords];
      }
  const int sa = (int)scales[lane], sb = (int)scales[64 + lane];
  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = v16f{};
  for (int it = 0; it < iters; it++) {
    // set 0 with scale byte 0 of the words, set 1 with byte 1 (op_sel)
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[0][j], fa[0][i], acc[i][j], 0, 0, 0, sb, 0,
                                                                    sa);
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[1][j], fa[1][i], acc[i][j], 0, 0, 1, sb, 1,
                                                                    sa);
  }
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) sum += acc[i][j][r];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = sum;
}

}  // namespace mxcal

// codes: kCodeWords (4096) uint32 words of E4M3 codes; scales: 128 uint32
// words of E8M0 bytes; out: blocks * 256 floats.  All device pointers.
// Returns the hipError_t of the launch.
extern "C" int mxfp8_calib_mfma_ceiling(const uint32_t* codes, const uint32_t* scales, float* out, int blocks,
                                        int iters, void* stream) {
  if (!codes || !scales || !out || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mxcal::mfma_ceiling_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), codes, scales, out, iters);
  return (int)hipGetLastError();
}

extern "C" int mxfp8_calib_code_words(void) { return mxcal::kCodeWords; }
