// MXFP8 quantization kernels for gfx950.
//
// One workgroup (256 threads = 4 wave64) owns a 128 x 128 BF16 tile.  Wave w
// owns rows [32w, 32w + 32) of the tile; lane (rg = lane / 16, cg = lane % 16)
// owns the 8 x 8 sub-block rows 32w + 8rg + [0, 8), columns 8cg + [0, 8), read
// with eight 16-byte loads (each load instruction of a wave covers four rows
// of 256 contiguous bytes).  Plain (cached) loads measured faster here than
// non-temporal ones; the transposed copy is stored non-temporally.
//
//  - rowwise 32-blocks are 4 consecutive lanes (a DPP quad) in one row;
//  - columnwise 32-blocks are the 4 lanes cg, cg+16, cg+32, cg+48 of a wave
//    (8 rows each), so every colwise block is reduced inside one wave;
//  - the columnwise codes are converted column-major in registers (pairs of
//    rows of one column per convert), written to a transposed 16 KB LDS tile
//    and streamed out as full 128-byte rows of q_colT;
//  - dbias partial sums are reduced lane -> wave -> workgroup and written once
//    per (row tile, column); a second kernel sums the row tiles.
//
// The arithmetic is exact integer scale selection (amax on BF16 bit patterns)
// and exact power-of-two scaling in fp32, followed by the hardware
// round-to-nearest-even E4M3 convert after clamping to +-448.
#include "mx_device.h"
#include "launch.h"

namespace mx {

constexpr int QT_R = 128;
constexpr int QT_C = 128;
constexpr int Q_THREADS = 256;

template <bool ROW, bool COL, bool DBIAS>
__global__ __launch_bounds__(Q_THREADS) void quantize_tile_kernel(
    const uint16_t* __restrict__ x, int64_t R, int64_t C, int64_t ldx,
    uint8_t* __restrict__ q_row, uint8_t* __restrict__ s_row,
    uint8_t* __restrict__ q_colT, uint8_t* __restrict__ s_colT,
    float* __restrict__ dbias_part, int64_t tiles_c) {
  // Transposed FP8 tile: [column][row] bytes, 8-byte row units XOR-swizzled
  // by the column group to spread the transposing writes over the banks.
  __shared__ __attribute__((aligned(16))) uint8_t lds_t[COL ? QT_C * QT_R : 16];
  __shared__ float lds_db[DBIAS ? 4 * QT_C : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int cg = lane & 15;
  const int rg = lane >> 4;
  int64_t tr, tc;
  if (ROW && !COL) {
    // Rowwise only: workgroup ids are dealt round-robin to the 8 XCDs; remap
    // them so each XCD walks its own share in groups of 8 x 8 tiles.  The 8
    // column tiles of a group write 8 x 4 = 32 contiguous scale bytes per row
    // from one L2, instead of 4-byte pieces from 8 different L2s.
    const int64_t ntile = gridDim.x;
    const int64_t bid = blockIdx.x;
    const int64_t full = (ntile / 8) * 8;
    const int64_t lid = bid < full ? (bid & 7) * (full >> 3) + (bid >> 3) : bid;
    const int64_t tiles_r = ntile / tiles_c;
    const int64_t per_band = 8 * tiles_c;                          // tiles in 8 row tiles
    const int64_t band = lid / per_band;
    const int64_t hb = (tiles_r - 8 * band) < 8 ? (tiles_r - 8 * band) : 8;
    const int64_t inb = lid - band * per_band;
    const int64_t grp = inb / (8 * hb);
    const int64_t wg = (tiles_c - 8 * grp) < 8 ? (tiles_c - 8 * grp) : 8;
    const int64_t ing = inb - grp * 8 * hb;
    tr = 8 * band + ing / wg;
    tc = 8 * grp + ing % wg;
  } else {
    tr = (int64_t)blockIdx.x / tiles_c;
    tc = (int64_t)blockIdx.x - tr * tiles_c;
  }
  const int64_t r0 = tr * QT_R;
  const int64_t c0 = tc * QT_C;
  const int64_t rb = r0 + 32 * w + 8 * rg;  // first row of this lane
  const int64_t cb = c0 + 8 * cg;           // first column of this lane
  const bool cval = cb < C;                 // C % 32 == 0: whole quads are valid

  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    if (cval && rb + i < R)
      v[i] = *reinterpret_cast<const uint4*>(x + (rb + i) * ldx + cb);
    else
      v[i] = make_uint4(0u, 0u, 0u, 0u);
  }

  if (ROW) {
    const int64_t ncb = C >> 5;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      uint32_t m = pk_max_u16(pk_max_u16(abs_bits2(v[i].x), abs_bits2(v[i].y)),
                              pk_max_u16(abs_bits2(v[i].z), abs_bits2(v[i].w)));
      m = max(m & 0xFFFFu, m >> 16);
      m = quad_max(m);
      const uint32_t byte = scale_byte_from_amax(m);
      const float sc = inv_scale(byte);
      uint2 o;
      o.x = cvt4_e4m3(bf_lo(v[i].x) * sc, bf_hi(v[i].x) * sc, bf_lo(v[i].y) * sc, bf_hi(v[i].y) * sc);
      o.y = cvt4_e4m3(bf_lo(v[i].z) * sc, bf_hi(v[i].z) * sc, bf_lo(v[i].w) * sc, bf_hi(v[i].w) * sc);
      const int64_t r = rb + i;
      if (cval && r < R) {
        *reinterpret_cast<uint2*>(q_row + r * C + cb) = o;
        if ((cg & 3) == 0) s_row[r * ncb + (cb >> 5)] = (uint8_t)byte;
      }
    }
  }

  if (COL) {
    // Per-column amax over this lane's 8 rows, then across the 4 row groups.
    uint32_t cm[4];
    cm[0] = abs_bits2(v[0].x);
    cm[1] = abs_bits2(v[0].y);
    cm[2] = abs_bits2(v[0].z);
    cm[3] = abs_bits2(v[0].w);
#pragma unroll
    for (int i = 1; i < 8; i++) {
      cm[0] = pk_max_u16(cm[0], abs_bits2(v[i].x));
      cm[1] = pk_max_u16(cm[1], abs_bits2(v[i].y));
      cm[2] = pk_max_u16(cm[2], abs_bits2(v[i].z));
      cm[3] = pk_max_u16(cm[3], abs_bits2(v[i].w));
    }
#pragma unroll
    for (int j = 0; j < 4; j++) {
      cm[j] = pk_max_u16(cm[j], (uint32_t)__shfl_xor((int)cm[j], 16, 64));
      cm[j] = pk_max_u16(cm[j], (uint32_t)__shfl_xor((int)cm[j], 32, 64));
    }
    const bool wval = (r0 + 32 * w) < R;  // R % 32 == 0: the wave's 32 rows are all valid or not
    const int64_t nrb = R >> 5;
    const int u = 4 * w + rg;             // 8-row unit of this lane inside the tile
    const int swz = 2 * (cg & 7);         // even XOR keeps 16-byte pairs of units adjacent
#pragma unroll
    for (int k = 0; k < 8; k++) {
      const uint32_t amax = (k & 1) ? (cm[k >> 1] >> 16) : (cm[k >> 1] & 0xFFFFu);
      const uint32_t byte = scale_byte_from_amax(amax);
      const float sc = inv_scale(byte);
      float e[8];
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const uint32_t d = (k >> 1) == 0 ? v[i].x : (k >> 1) == 1 ? v[i].y : (k >> 1) == 2 ? v[i].z : v[i].w;
        e[i] = ((k & 1) ? bf_hi(d) : bf_lo(d)) * sc;
      }
      uint2 o;
      o.x = cvt4_e4m3(e[0], e[1], e[2], e[3]);
      o.y = cvt4_e4m3(e[4], e[5], e[6], e[7]);
      const int cl = 8 * cg + k;
      *reinterpret_cast<uint2*>(lds_t + cl * QT_R + 8 * (u ^ swz)) = o;
      if (rg == 0 && cval && wval) s_colT[(cb + k) * nrb + ((r0 >> 5) + w)] = (uint8_t)byte;
    }
  }

  if (DBIAS) {
    float cs[8];
#pragma unroll
    for (int k = 0; k < 8; k++) {
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const uint32_t d = (k >> 1) == 0 ? v[i].x : (k >> 1) == 1 ? v[i].y : (k >> 1) == 2 ? v[i].z : v[i].w;
        s += (k & 1) ? bf_hi(d) : bf_lo(d);
      }
      s += __shfl_xor(s, 16, 64);
      s += __shfl_xor(s, 32, 64);
      cs[k] = s;
    }
    if (rg == 0) {
#pragma unroll
      for (int k = 0; k < 8; k++) lds_db[w * QT_C + 8 * cg + k] = cs[k];
    }
  }

  if (COL || DBIAS) __syncthreads();

  if (COL) {
    // Thread t streams 16-byte chunk (t % 8) of transposed rows t/8 + 32j.
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int cl = (tid >> 3) + 32 * j;
      const int ch = tid & 7;
      const int swz = 2 * ((cl >> 3) & 7);
      const uint4 d = *reinterpret_cast<const uint4*>(lds_t + cl * QT_R + 8 * ((2 * ch) ^ swz));
      const int64_t col = c0 + cl;
      const int64_t row = r0 + 16 * ch;
      if (col < C && row < R) store_nt16(q_colT + col * R + row, d);
    }
  }

  if (DBIAS) {
    if (tid < QT_C && c0 + tid < C) {
      const float s = ((lds_db[tid] + lds_db[QT_C + tid]) + lds_db[2 * QT_C + tid]) + lds_db[3 * QT_C + tid];
      dbias_part[tr * C + c0 + tid] = s;
    }
  }
}

// Rowwise copy of a contiguous input (ld_x == cols): blocks never cross rows
// (cols % 32 == 0), so the tensor is one flat stream of 32-element blocks and
// the scales [rows][cols/32] are the flat block index.  Each wave quantizes
// FL_ELEMS contiguous elements: load u of lane l covers elements
// 512u + 8l + [0, 8), i.e. every load instruction reads 1 KB contiguous, each
// DPP quad holds one block, codes go out (non-temporally) as 512-byte runs and
// the wave's 32 scale bytes are contiguous.  Two loads per lane measured best
// (more waves in flight than with four or eight).
constexpr int FL_LOADS = 2;
constexpr int64_t FL_ELEMS = 512 * FL_LOADS;  // per wave

__global__ __launch_bounds__(Q_THREADS) void quantize_rowwise_flat_kernel(const uint16_t* __restrict__ x,
                                                                         int64_t total,
                                                                         uint8_t* __restrict__ q,
                                                                         uint8_t* __restrict__ s) {
  const int lane = threadIdx.x & 63;
  const int64_t base = ((int64_t)blockIdx.x * (Q_THREADS / 64) + (threadIdx.x >> 6)) * FL_ELEMS;
  uint4 v[FL_LOADS];
#pragma unroll
  for (int u = 0; u < FL_LOADS; u++) {
    const int64_t e = base + 512 * u + 8 * lane;
    v[u] = e < total ? *reinterpret_cast<const uint4*>(x + e) : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int u = 0; u < FL_LOADS; u++) {
    const int64_t e = base + 512 * u + 8 * lane;
    uint32_t m = pk_max_u16(pk_max_u16(abs_bits2(v[u].x), abs_bits2(v[u].y)),
                            pk_max_u16(abs_bits2(v[u].z), abs_bits2(v[u].w)));
    m = max(m & 0xFFFFu, m >> 16);
    m = quad_max(m);
    const uint32_t byte = scale_byte_from_amax(m);
    const float sc = inv_scale(byte);
    uint2 o;
    o.x = cvt4_e4m3(bf_lo(v[u].x) * sc, bf_hi(v[u].x) * sc, bf_lo(v[u].y) * sc, bf_hi(v[u].y) * sc);
    o.y = cvt4_e4m3(bf_lo(v[u].z) * sc, bf_hi(v[u].z) * sc, bf_lo(v[u].w) * sc, bf_hi(v[u].w) * sc);
    if (e < total) {  // total % 32 == 0: a quad is entirely in or out
      __builtin_nontemporal_store(o.x, reinterpret_cast<uint32_t*>(q + e));
      __builtin_nontemporal_store(o.y, reinterpret_cast<uint32_t*>(q + e) + 1);
      if ((lane & 3) == 0) s[e >> 5] = (uint8_t)byte;
    }
  }
}

// dbias[c] = sum over row tiles of the partial sums, in four interleaved
// chains combined pairwise (a fixed order: the result is deterministic).
__global__ __launch_bounds__(256) void dbias_reduce_kernel(const float* __restrict__ part, int64_t tiles,
                                                           int64_t C, float* __restrict__ out) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= C) return;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  int64_t t = 0;
  for (; t + 4 <= tiles; t += 4) {
    a0 += part[(t + 0) * C + c];
    a1 += part[(t + 1) * C + c];
    a2 += part[(t + 2) * C + c];
    a3 += part[(t + 3) * C + c];
  }
  if (t < tiles) a0 += part[t * C + c];
  if (t + 1 < tiles) a1 += part[(t + 1) * C + c];
  if (t + 2 < tiles) a2 += part[(t + 2) * C + c];
  out[c] = (a0 + a1) + (a2 + a3);
}

__global__ __launch_bounds__(256) void fill_zero_f32_kernel(float* __restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = 0.0f;
}

int64_t quantize_row_tiles(int64_t R) { return (R + QT_R - 1) / QT_R; }
int64_t quantize_col_tiles(int64_t C) { return (C + QT_C - 1) / QT_C; }

hipError_t launch_quantize(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, uint32_t flags,
                           uint8_t* q_row, uint8_t* s_row, uint8_t* q_colT, uint8_t* s_colT,
                           float* dbias, float* dbias_part, hipStream_t stream) {
  const bool row = flags & 1u, col = flags & 2u, db = flags & 4u;
  const int64_t tr = quantize_row_tiles(R), tc = quantize_col_tiles(C);
  const int64_t tiles = tr * tc;
  if (row && !col && !db && ldx == C) {
    const int64_t total = R * C;
    const int64_t blocks = (total + FL_ELEMS * (Q_THREADS / 64) - 1) / (FL_ELEMS * (Q_THREADS / 64));
    if (blocks > 0)
      hipLaunchKernelGGL(quantize_rowwise_flat_kernel, dim3((unsigned)blocks), dim3(Q_THREADS), 0, stream, x, total,
                         q_row, s_row);
    return hipGetLastError();
  }
  if (tiles > 0) {
    const dim3 grid((unsigned)tiles), block(Q_THREADS);
#define MX_Q_LAUNCH(RW, CL, DB)                                                                   \
  hipLaunchKernelGGL((quantize_tile_kernel<RW, CL, DB>), grid, block, 0, stream, x, R, C, ldx, q_row, \
                     s_row, q_colT, s_colT, dbias_part, tc)
    if (row && col && db) MX_Q_LAUNCH(true, true, true);
    else if (row && col) MX_Q_LAUNCH(true, true, false);
    else if (row && db) MX_Q_LAUNCH(true, false, true);
    else if (row) MX_Q_LAUNCH(true, false, false);
    else if (col && db) MX_Q_LAUNCH(false, true, true);
    else MX_Q_LAUNCH(false, true, false);
#undef MX_Q_LAUNCH
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (db && C > 0) {
    const dim3 grid((unsigned)((C + 255) / 256)), block(256);
    if (tiles > 0)
      hipLaunchKernelGGL(dbias_reduce_kernel, grid, block, 0, stream, dbias_part, tr, C, dbias);
    else
      hipLaunchKernelGGL(fill_zero_f32_kernel, grid, block, 0, stream, dbias, C);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace mx
