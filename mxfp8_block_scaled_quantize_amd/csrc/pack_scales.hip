// E8M0 scale packing for the block-scaled GEMM (gfx950).
//
// s[dim][ld_s] bytes -> packed[k/128][dim] uint32: word (t, r) holds the four
// scale bytes of K-blocks 4t .. 4t+3 of row r.  The four bytes are already
// contiguous in s, so packing is a transpose of a [dim][k/128] matrix of
// 32-bit words, done through a padded 64 x 64 LDS tile with coalesced
// 256-byte reads (along k) and writes (along dim).
#include "mx_device.h"
#include "launch.h"

namespace mx {

constexpr int PK_T = 64;

__global__ __launch_bounds__(256) void pack_scales_kernel(const uint8_t* __restrict__ s, int64_t dim,
                                                          int64_t kw, int64_t ld_s,
                                                          uint32_t* __restrict__ packed, int64_t tiles_k) {
  __shared__ uint32_t t[PK_T][PK_T + 1];
  const int tid = threadIdx.x;
  const int64_t bid = blockIdx.x;
  const int64_t tr = bid / tiles_k;
  const int64_t tk = bid - tr * tiles_k;
  const int64_t r0 = tr * PK_T, w0 = tk * PK_T;
  const int wl = tid & 63;
#pragma unroll
  for (int i = 0; i < 16; i++) {
    const int rl = (tid >> 6) + 4 * i;
    const int64_t r = r0 + rl, wd = w0 + wl;
    uint32_t val = 0;
    if (r < dim && wd < kw) val = *reinterpret_cast<const uint32_t*>(s + r * ld_s + 4 * wd);
    t[rl][wl] = val;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; i++) {
    const int wl2 = (tid >> 6) + 4 * i;
    const int rl = tid & 63;
    const int64_t r = r0 + rl, wd = w0 + wl2;
    if (r < dim && wd < kw) packed[wd * dim + r] = t[rl][wl2];
  }
}

bool pack_scales_grid_fits(int64_t dim, int64_t k) {
  const int64_t kw = k / 128;
  return grid_fits((dim + PK_T - 1) / PK_T, (kw + PK_T - 1) / PK_T, 256);
}

hipError_t launch_pack_scales(const uint8_t* s, int64_t dim, int64_t k, int64_t ld_s, uint32_t* packed,
                              hipStream_t stream) {
  const int64_t kw = k / 128;
  const int64_t tiles_k = (kw + PK_T - 1) / PK_T;
  const int64_t blocks = ((dim + PK_T - 1) / PK_T) * tiles_k;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_scales_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, s, dim, kw, ld_s,
                     packed, tiles_k);
  return hipGetLastError();
}

}  // namespace mx
