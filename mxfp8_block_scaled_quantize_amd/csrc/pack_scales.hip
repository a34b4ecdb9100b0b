// E8M0 scale packing for the block-scaled GEMM (gfx950).
//
// s[dim][ld_s] bytes -> packed[k/128][dim] uint32: word (t, r) holds the four
// scale bytes of K-blocks 4t .. 4t+3 of row r.  The four bytes are already
// contiguous in s, so packing is a transpose of a [dim][k/128] matrix of
// 32-bit words, done through an LDS tile: 16-byte reads along k and writes
// along dim where the shapes allow it, else a padded 64 x 64 tile of 4-byte
// accesses (256 bytes per wave instruction).
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

// 16-byte form, used when every row holds whole groups of four words and
// whole groups of four rows exist (kw % 4 == 0, dim % 4 == 0, 16-byte aligned
// rows and output): a workgroup moves a 64-row x 16-word tile with one
// 16-byte load (four words of one row) and one 16-byte store (one word of
// four consecutive rows) per thread, so a wave reads and writes 1 KB per
// instruction instead of 256 bytes.
constexpr int PV_R = 64;
constexpr int PV_W = 16;

__global__ __launch_bounds__(256) void pack_scales_vec_kernel(const uint8_t* __restrict__ s, int64_t dim,
                                                              int64_t kw, int64_t ld_s,
                                                              uint32_t* __restrict__ packed, int64_t tiles_w) {
  __shared__ uint32_t t[PV_W][PV_R + 4];   // [word][row]
  const int tid = threadIdx.x;
  const int64_t bid = blockIdx.x;
  const int64_t tr = bid / tiles_w;
  const int64_t tw = bid - tr * tiles_w;
  const int64_t r0 = tr * PV_R, w0 = tw * PV_W;
  {
    const int rl = tid >> 2, wq = 4 * (tid & 3);
    const int64_t r = r0 + rl, wd = w0 + wq;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r < dim && wd < kw) v = *reinterpret_cast<const uint4*>(s + r * ld_s + 4 * wd);
    t[wq][rl] = v.x;
    t[wq + 1][rl] = v.y;
    t[wq + 2][rl] = v.z;
    t[wq + 3][rl] = v.w;
  }
  __syncthreads();
  {
    const int wl = tid >> 4, rq = 4 * (tid & 15);
    const int64_t r = r0 + rq, wd = w0 + wl;
    if (r < dim && wd < kw)
      *reinterpret_cast<uint4*>(packed + wd * dim + r) = make_uint4(t[wl][rq], t[wl][rq + 1], t[wl][rq + 2],
                                                                     t[wl][rq + 3]);
  }
}

static bool pack_vec_ok(const uint8_t* s, int64_t dim, int64_t kw, int64_t ld_s, const uint32_t* packed) {
  return kw % 4 == 0 && dim % 4 == 0 && ld_s % 16 == 0 && (reinterpret_cast<uintptr_t>(s) & 15) == 0 &&
         (reinterpret_cast<uintptr_t>(packed) & 15) == 0;
}

bool pack_scales_grid_fits(int64_t dim, int64_t k) {
  // the 16-byte form's grid ((dim / 64) x (kw / 16) tiles) is the larger one
  const int64_t kw = k / 128;
  return grid_fits((dim + PV_R - 1) / PV_R, (kw + PV_W - 1) / PV_W, 256);
}

hipError_t launch_pack_scales(const uint8_t* s, int64_t dim, int64_t k, int64_t ld_s, uint32_t* packed,
                              hipStream_t stream) {
  const int64_t kw = k / 128;
  if (pack_vec_ok(s, dim, kw, ld_s, packed)) {
    const int64_t tiles_w = (kw + PV_W - 1) / PV_W;
    const int64_t blocks = ((dim + PV_R - 1) / PV_R) * tiles_w;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_scales_vec_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, s, dim, kw, ld_s,
                       packed, tiles_w);
    return hipGetLastError();
  }
  const int64_t tiles_k = (kw + PK_T - 1) / PK_T;
  const int64_t blocks = ((dim + PK_T - 1) / PK_T) * tiles_k;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_scales_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, s, dim, kw, ld_s,
                     packed, tiles_k);
  return hipGetLastError();
}

}  // namespace mx
