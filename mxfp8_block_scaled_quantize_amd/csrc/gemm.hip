// Block-scaled MXFP8 GEMM (TN) on the gfx950 scaled FP8 MFMA.
//
//   C[m][n] = bf16_rne( sum_k dq(A)[m][k] * dq(B)[n][k] ), fp32 accumulation.
//
// Operand register layout of V_MFMA_SCALE_F32_16X16X128_F8F6F4 (E4M3 both
// sides), as measured on gfx950: lane l holds row (l % 16) of the 16-row
// block; its bytes 0..15 are K = 16*(l/16) + [0,16) and bytes 16..31 are
// K = 64 + 16*(l/16) + [0,16) of the 128-wide K slab.  The scale operand of
// lane l (byte chosen by op_sel) scales row (l % 16), K-block (l / 16).  The
// fp32 result of lane l, register i, is row 4*(l/16) + i, column l % 16.
//
// v1 tiling: a 128 x 128 output tile per workgroup of 4 waves (2 x 2, each
// 64 x 64 = 4 x 4 MFMA blocks), K in 128-byte slabs staged through LDS
// (16-byte chunks XOR-swizzled by row so fragment reads are conflict free),
// next slab prefetched into registers while the current one is multiplied.
// Scales come straight from the packed [K/128][rows] words: one 32-bit load
// per lane per 16-row block per slab, shifted so byte 0 is the lane's block.
#include "mx_device.h"
#include "launch.h"

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int GB_M = 128;
constexpr int GB_N = 128;
constexpr int GB_K = 128;  // bytes of K per slab (= elements)

__device__ __forceinline__ int swz_chunk(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

template <bool GROUPED>
__global__ __launch_bounds__(256) void gemm_v1_kernel(const uint8_t* __restrict__ A, const uint32_t* __restrict__ Ap,
                                                      const uint8_t* __restrict__ B, const uint32_t* __restrict__ Bp,
                                                      uint16_t* __restrict__ Cm, int64_t ldc, int64_t M, int64_t N,
                                                      int64_t K, const int32_t* __restrict__ offsets, int32_t G,
                                                      int64_t tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[GB_M * GB_K];
  __shared__ __attribute__((aligned(16))) uint8_t sB[GB_N * GB_K];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const int64_t bid = blockIdx.x;
  const int64_t tn = bid % tiles_n;
  int64_t tm = bid / tiles_n;

  int64_t m_lo, m_hi;       // rows [m_lo, m_hi) of A / C belong to this tile's group
  int64_t b_row0 = 0;       // first row of this group's B in the stacked [G*N] rows
  if (GROUPED) {
    int64_t found = -1;
    m_lo = 0;
    m_hi = 0;
    for (int g = 0; g < G; g++) {
      int64_t lo = offsets[g], hi = offsets[g + 1];
      lo = lo < 0 ? 0 : (lo > M ? M : lo);
      hi = hi < lo ? lo : (hi > M ? M : hi);
      const int64_t nt = (hi - lo + GB_M - 1) / GB_M;
      if (tm < nt) {
        found = g;
        m_lo = lo + tm * GB_M;
        m_hi = hi;
        break;
      }
      tm -= nt;
    }
    if (found < 0) return;  // uniform for the whole workgroup
    b_row0 = found * N;
  } else {
    m_lo = tm * GB_M;
    m_hi = M;
  }
  const int64_t n0 = tn * GB_N;
  const int64_t brows = GROUPED ? (int64_t)G * N : N;  // rows of the packed B scale matrix
  const uint8_t* Bg = B + b_row0 * K;

  const int nk = (int)(K / GB_K);

  // Global -> register staging: 1024 16-byte chunks per operand tile, 4 per thread.
  uint4 ra[4], rb[4];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int q = tid + 256 * i;
      const int r = q >> 3, c = q & 7;
      const int64_t am = m_lo + r;
      ra[i] = am < m_hi ? *reinterpret_cast<const uint4*>(A + am * K + (int64_t)kt * GB_K + 16 * c)
                        : make_uint4(0u, 0u, 0u, 0u);
      const int64_t bn = n0 + r;
      rb[i] = bn < N ? *reinterpret_cast<const uint4*>(Bg + bn * K + (int64_t)kt * GB_K + 16 * c)
                     : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int q = tid + 256 * i;
      const int r = q >> 3, c = q & 7;
      *reinterpret_cast<uint4*>(sA + r * GB_K + 16 * swz_chunk(r, c)) = ra[i];
      *reinterpret_cast<uint4*>(sB + r * GB_K + 16 * swz_chunk(r, c)) = rb[i];
    }
  };

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int lr = lane & 15;   // row within a 16-row MFMA block
  const int lg = lane >> 4;   // K group of this lane
  if (nk > 0) gload(0);
  for (int kt = 0; kt < nk; kt++) {
    // scales for this slab (one word per 16-row block, byte lg moved to byte 0)
    uint32_t sa[4], sb[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int64_t am = m_lo + wm * 64 + 16 * i + lr;
      sa[i] = am < m_hi ? (Ap[(int64_t)kt * M + am] >> (8 * lg)) : 0u;
      const int64_t bn = n0 + wn * 64 + 16 * i + lr;
      sb[i] = bn < N ? (Bp[(int64_t)kt * brows + b_row0 + bn] >> (8 * lg)) : 0u;
    }
    __syncthreads();
    lstore();
    __syncthreads();
    if (kt + 1 < nk) gload(kt + 1);

    v8i fa[4], fb[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int r = wm * 64 + 16 * i + lr;
      const uint4 lo = *reinterpret_cast<const uint4*>(sA + r * GB_K + 16 * swz_chunk(r, lg));
      const uint4 hi = *reinterpret_cast<const uint4*>(sA + r * GB_K + 16 * swz_chunk(r, 4 + lg));
      fa[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      const int rn = wn * 64 + 16 * i + lr;
      const uint4 blo = *reinterpret_cast<const uint4*>(sB + rn * GB_K + 16 * swz_chunk(rn, lg));
      const uint4 bhi = *reinterpret_cast<const uint4*>(sB + rn * GB_K + 16 * swz_chunk(rn, 4 + lg));
      fb[i] = v8i{(int)blo.x, (int)blo.y, (int)blo.z, (int)blo.w, (int)bhi.x, (int)bhi.y, (int)bhi.z, (int)bhi.w};
    }
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, 0,
                                                                     (int)sa[i], 0, (int)sb[j]);
  }

  // Epilogue: lane l, register q of block (i, j) -> row 16i + 4(l/16) + q, column 16j + l%16.
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int64_t m = m_lo + wm * 64 + 16 * i + 4 * lg + q;
        const int64_t n = n0 + wn * 64 + 16 * j + lr;
        if (m < m_hi && n < N) Cm[m * ldc + n] = (uint16_t)f32_to_bf16_rne(acc[i][j][q]);
      }
}

int64_t gemm_blocks(int64_t M, int64_t N, int32_t G, bool grouped) {
  const int64_t tn = (N + GB_N - 1) / GB_N;
  const int64_t tm = (M + GB_M - 1) / GB_M + (grouped ? (int64_t)G : 0);
  return tm * tn;
}

hipError_t launch_gemm(const uint8_t* a, const uint32_t* ap, const uint8_t* b, const uint32_t* bp,
                       uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K,
                       const int32_t* offsets, int32_t G, hipStream_t stream) {
  const bool grouped = offsets != nullptr;
  const int64_t tiles_n = (N + GB_N - 1) / GB_N;
  const int64_t blocks = gemm_blocks(M, N, G, grouped);
  if (blocks == 0) return hipSuccess;
  if (grouped)
    hipLaunchKernelGGL(gemm_v1_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, a, ap, b, bp, c, ldc, M,
                       N, K, offsets, G, tiles_n);
  else
    hipLaunchKernelGGL(gemm_v1_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, a, ap, b, bp, c, ldc,
                       M, N, K, offsets, G, tiles_n);
  return hipGetLastError();
}

}  // namespace mx
