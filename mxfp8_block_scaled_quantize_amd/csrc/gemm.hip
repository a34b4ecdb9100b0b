// Block-scaled MXFP8 GEMM (TN) on the gfx950 scaled FP8 MFMA.
//
//   C[m][n] = bf16_rne( sum_k dq(A)[m][k] * dq(B)[n][k] ), fp32 accumulation.
//
// Operand layout of V_MFMA_SCALE_F32_32X32X64_F8F6F4 with E4M3 on both sides,
// as measured on gfx950: lane l holds row (l % 32) of the 32-row block; its
// bytes 0..15 are K = 16*(l/32) + [0,16) and bytes 16..31 are
// K = 32 + 16*(l/32) + [0,16) of the 64-wide K step.  The scale operand of
// lane l (byte chosen by op_sel) scales row (l % 32), K-block (l / 32) of the
// step.  Result register i of lane l is row 8*(i/4) + 4*(l/32) + (i%4),
// column l % 32.
//
// Tiling: one workgroup of 4 waves computes a 256 x 256 tile; wave (wm, wn)
// owns 128 x 128 = 4 x 4 MFMA blocks (256 fp32 accumulators per lane).  K is
// consumed in 64-byte steps through a 4-slot LDS ring (34 KB per slot: A and
// B 256 x 64 bytes each, plus the packed scale words of a 128-wide K slab).
// Slots are filled by buffer->LDS DMA (16 bytes per lane, rows past the end
// of the matrix read as zero) issued four steps ahead; operand fragments of
// step s+1 are read from LDS while the MFMAs of step s run.  16-byte chunks
// of each 64-byte LDS row are XOR-swizzled by (row >> 2) & 3, which makes
// every fragment read conflict free.  Workgroup ids are remapped so that the
// tiles resident on one XCD (ids are dealt round-robin to the 8 XCDs) form
// compact groups of 4 row tiles, sharing A and B in that XCD's L2.
#include "mx_device.h"
#include "launch.h"

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) const uint32_t lds_u32;

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;                  // K bytes per pipeline step
constexpr int NSLOT = 4;
constexpr int A_BYTES = BM * BK;        // 16 KB
constexpr int B_BYTES = BN * BK;        // 16 KB
constexpr int SA_OFF = A_BYTES + B_BYTES;
constexpr int SB_OFF = SA_OFF + BM * 4;
constexpr int SLOT_BYTES = SB_OFF + BN * 4;          // 34 KB
constexpr int LDS_BYTES = NSLOT * SLOT_BYTES;        // 136 KB
constexpr int GROUP_M = 4;              // row tiles per L2 group
constexpr int C_LDS_STRIDE = 2 * BN + 16;            // BF16 output tile row in LDS, padded (528 B)
static_assert(BM * C_LDS_STRIDE <= LDS_BYTES, "output tile must fit in the ring");
constexpr uint32_t RSRC_FLAGS = 0x00020000u;         // raw buffer, 32-bit data format

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // s_waitcnt with vmcnt = N (6 bits: [3:0] and [15:14]); expcnt and lgkmcnt left at max.
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

template <int V>
struct ic {
  static constexpr int value = V;
};

template <bool GROUPED>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void gemm_kernel(const uint8_t* __restrict__ A, const uint32_t* __restrict__ Ap,
                 const uint8_t* __restrict__ B, const uint32_t* __restrict__ Bp,
                 uint16_t* __restrict__ Cm, int64_t ldc, int64_t M, int64_t N, int64_t K,
                 const int32_t* __restrict__ offsets, int32_t G, int64_t tiles_m, int64_t tiles_n) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
  lds_u8* smem = (lds_u8*)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- tile selection: XCD-aware remap, then groups of GROUP_M row tiles
  const int64_t nblk = tiles_m * tiles_n;
  const int64_t bid = blockIdx.x;
  const int64_t full = (nblk / 8) * 8;
  const int64_t lid = bid < full ? (bid & 7) * (full >> 3) + (bid >> 3) : bid;
  const int64_t per_group = (int64_t)GROUP_M * tiles_n;
  const int64_t grp = lid / per_group;
  const int64_t first_m = grp * GROUP_M;
  const int64_t gm = (tiles_m - first_m) < GROUP_M ? (tiles_m - first_m) : GROUP_M;
  const int64_t rem = lid - grp * per_group;
  int64_t tm = first_m + rem % gm;
  const int64_t tn = rem / gm;

  int64_t m_lo, m_hi, b_row0 = 0;
  if (GROUPED) {
    int64_t found = -1;
    m_lo = m_hi = 0;
    for (int g = 0; g < G; g++) {
      int64_t lo = offsets[g], hi = offsets[g + 1];
      lo = lo < 0 ? 0 : (lo > M ? M : lo);
      hi = hi < lo ? lo : (hi > M ? M : hi);
      const int64_t nt = (hi - lo + BM - 1) / BM;
      if (tm < nt) {
        found = g;
        m_lo = lo + tm * BM;
        m_hi = hi;
        break;
      }
      tm -= nt;
    }
    if (found < 0) return;  // whole workgroup leaves together
    b_row0 = found * N;
  } else {
    m_lo = tm * BM;
    m_hi = M;
  }
  const int64_t n0 = tn * BN;
  const int64_t brows = GROUPED ? (int64_t)G * N : N;
  const int rows_a = (int)((m_hi - m_lo) < BM ? (m_hi - m_lo) : BM);
  const int rows_b = (int)((N - n0) < BN ? (N - n0) : BN);

  // ---- DMA sources.  Data: raw buffers over the tile's rows (out-of-range rows read 0).
  const __amdgpu_buffer_rsrc_t rs_a =
      __builtin_amdgcn_make_buffer_rsrc((void*)(A + m_lo * K), 0, (int)((int64_t)rows_a * K), RSRC_FLAGS);
  const __amdgpu_buffer_rsrc_t rs_b = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(B + (b_row0 + n0) * K), 0, (int)((int64_t)rows_b * K), RSRC_FLAGS);
  // lane's 4 DMA row/chunk offsets (same for A and B): LDS rows 16*(4w+i) + lane/4, slot lane%4
  uint32_t dma_off[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int r = 16 * (4 * wave + i) + (lane >> 2);
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    dma_off[i] = (uint32_t)r * (uint32_t)K + 16u * (uint32_t)c;
  }
  // scale words: wave w brings rows 64w + lane (clamped into the valid rows)
  const int sra = (64 * wave + lane) < rows_a ? (64 * wave + lane) : rows_a - 1;
  const int srb = (64 * wave + lane) < rows_b ? (64 * wave + lane) : rows_b - 1;
  const uint32_t* sa_src = Ap + m_lo + sra;
  const uint32_t* sb_src = Bp + b_row0 + n0 + srb;

  const int nk = (int)(K / BK);  // even: K % 128 == 0

  // DMA of one K step into its ring slot: 8 data loads per lane, plus the
  // scale words of the 128-wide slab on even steps (2 more loads per lane).
  auto issue_step = [&](int s, auto EVEN) {
    lds_u8* base = smem + (s & (NSLOT - 1)) * SLOT_BYTES;
    const uint32_t k0 = (uint32_t)s * BK;
#pragma unroll
    for (int i = 0; i < 4; i++)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_a, (lds_void*)(base + 1024 * (4 * wave + i)), 16,
                                               dma_off[i] + k0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; i++)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_b, (lds_void*)(base + A_BYTES + 1024 * (4 * wave + i)), 16,
                                               dma_off[i] + k0, 0, 0, 0);
    if constexpr (decltype(EVEN)::value) {
      const int64_t t = s >> 1;
      __builtin_amdgcn_global_load_lds((const void*)(sa_src + t * M), (lds_void*)(base + SA_OFF + 256 * wave), 4,
                                       0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(sb_src + t * brows), (lds_void*)(base + SB_OFF + 256 * wave),
                                       4, 0, 0);
    }
  };

  // ---- fragment addressing inside a slot
  const int lr = lane & 31;
  const int lg = lane >> 5;
  const int swz = (lane >> 2) & 3;
  const int a_row_off = (wm * 128 + lr) * BK;
  const int b_row_off = A_BYTES + (wn * 128 + lr) * BK;
  const int c0 = 16 * (lg ^ swz);
  const int c1 = 16 * ((2 + lg) ^ swz);

  v8i fa[2][4], fb[2][4];
  uint32_t sa[2][4], sb[2][4];
  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = v16f{};

  // LDS -> registers: operand fragments of step s into register set SET; on
  // even steps also the slab's scale words into scale set T2.  At use the
  // words are shifted right by 8 * (lane / 32), so that byte 0 is this lane's
  // K block of the even step and byte 2 that of the odd step.
  const uint32_t sh = 8u * (uint32_t)lg;
  auto read_frags = [&](int s, auto SET, auto EVEN, auto T2) {
    constexpr int set = decltype(SET)::value;
    const lds_u8* base = smem + (s & (NSLOT - 1)) * SLOT_BYTES;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const u32x4 lo = *(lds_u32x4*)(base + a_row_off + i * 32 * BK + c0);
      const u32x4 hi = *(lds_u32x4*)(base + a_row_off + i * 32 * BK + c1);
      fa[set][i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      const u32x4 blo = *(lds_u32x4*)(base + b_row_off + i * 32 * BK + c0);
      const u32x4 bhi = *(lds_u32x4*)(base + b_row_off + i * 32 * BK + c1);
      fb[set][i] = v8i{(int)blo.x, (int)blo.y, (int)blo.z, (int)blo.w, (int)bhi.x, (int)bhi.y, (int)bhi.z, (int)bhi.w};
    }
    if constexpr (decltype(EVEN)::value) {
      constexpr int t2 = decltype(T2)::value;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        sa[t2][i] = *(lds_u32*)(base + SA_OFF + 4 * (wm * 128 + 32 * i + lr));
        sb[t2][i] = *(lds_u32*)(base + SB_OFF + 4 * (wn * 128 + 32 * i + lr));
      }
    }
  };

  auto mfma_step = [&](auto SET, auto T2, auto OPSEL) {
    constexpr int set = decltype(SET)::value;
    constexpr int t2 = decltype(T2)::value;
    constexpr int op = decltype(OPSEL)::value;
    int xa[4], xb[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      xa[i] = (int)(sa[t2][i] >> sh);
      xb[i] = (int)(sb[t2][i] >> sh);
    }
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[set][i], fb[set][j], acc[i][j], 0, 0, op,
                                                                    xa[i], op, xb[j]);
  };

  // One pipeline step st (register set SET, scale set T2, op_sel OP): make
  // step st+1 resident (the DMA of steps st+2, st+3 may stay in flight: 18
  // loads per lane, one even and one odd step), refill the slot of step st
  // with step st+4, read the fragments of st+1, multiply step st.
  auto substep = [&](int st, auto SET, auto T2, auto OP, auto EVEN) {
    constexpr bool even = decltype(EVEN)::value;
    if (st + 1 < nk) {
      if (st + 3 < nk) wait_vmcnt<18>();
      else if (st + 2 < nk) wait_vmcnt<even ? 10 : 8>();
      else wait_vmcnt<0>();
    }
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    if (st + 4 < nk) issue_step(st + 4, EVEN);
    // Fragments of st+1 are read unconditionally (after the last step they
    // read a stale slot and are never used) so that the reads and the MFMAs
    // share one basic block and can be interleaved: one MFMA, then up to two
    // LDS reads, keeping the MFMA pipe fed while the LDS queue drains.
    read_frags(st + 1, ic<1 - decltype(SET)::value>{}, ic<!even>{}, ic<1 - decltype(T2)::value>{});
    mfma_step(SET, T2, OP);
    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);   // scale shifts
#pragma unroll
    for (int i = 0; i < 16; i++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
    }
  };

  if (nk > 0) {
    // prologue: steps 0..3 in flight, step 0 resident, its fragments read
    issue_step(0, ic<1>{});
    if (1 < nk) issue_step(1, ic<0>{});
    if (2 < nk) issue_step(2, ic<1>{});
    if (3 < nk) issue_step(3, ic<0>{});
    if (nk >= 4) wait_vmcnt<8 + 10 + 8>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    read_frags(0, ic<0>{}, ic<1>{}, ic<0>{});

    for (int s = 0; s < nk; s += 4) {
      substep(s, ic<0>{}, ic<0>{}, ic<0>{}, ic<1>{});
      if (s + 1 < nk) substep(s + 1, ic<1>{}, ic<0>{}, ic<2>{}, ic<0>{});
      if (s + 2 < nk) substep(s + 2, ic<0>{}, ic<1>{}, ic<0>{}, ic<1>{});
      if (s + 3 < nk) substep(s + 3, ic<1>{}, ic<1>{}, ic<2>{}, ic<0>{});
    }
  }

  // ---- epilogue: fp32 -> BF16 (RNE) into a padded row-major LDS tile (the
  // ring is free once every wave is past its last step), then 16-byte
  // stores that cover whole 512-byte row segments of C.  Lane pairs swap
  // values so each LDS write is one 32-bit word (two adjacent columns).
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  {
    const bool odd = lane & 1;
    const int rb = wm * 128 + 4 * lg;
    const int cb = wn * 128 + lr - (odd ? 1 : 0);
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const uint32_t a = f32_to_bf16_rne(acc[i][j][r]);
          const uint32_t b = f32_to_bf16_rne(acc[i][j][r + 1]);
          const uint32_t x = odd ? a : b;
          const uint32_t y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, true);  // lane ^ 1
          const uint32_t word = odd ? (y | (b << 16)) : (a | (y << 16));
          const int row = rb + 32 * i + 8 * (r >> 2) + (r & 3) + (odd ? 1 : 0);
          *(__attribute__((address_space(3))) uint32_t*)(smem + row * C_LDS_STRIDE + 2 * (cb + 32 * j)) = word;
        }
  }
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  {
    const int ch = tid & 31;           // 16-byte chunk of a 512-byte tile row
    const int64_t col = n0 + 8 * ch;
    if (col < N) {
#pragma unroll 8
      for (int k = 0; k < 32; k++) {
        const int row = (tid >> 5) + 8 * k;
        const int64_t grow = m_lo + row;
        const u32x4 v = *(lds_u32x4*)(smem + row * C_LDS_STRIDE + 16 * ch);
        if (grow < m_hi) store_nt16(Cm + grow * ldc + col, make_uint4(v.x, v.y, v.z, v.w));
      }
    }
  }
}

int64_t gemm_blocks(int64_t M, int64_t N, int32_t G, bool grouped) {
  const int64_t tn = (N + BN - 1) / BN;
  const int64_t tm = (M + BM - 1) / BM + (grouped ? (int64_t)G : 0);
  return tm * tn;
}

hipError_t launch_gemm(const uint8_t* a, const uint32_t* ap, const uint8_t* b, const uint32_t* bp,
                       uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K,
                       const int32_t* offsets, int32_t G, hipStream_t stream) {
  const bool grouped = offsets != nullptr;
  const int64_t tiles_n = (N + BN - 1) / BN;
  const int64_t tiles_m = (M + BM - 1) / BM + (grouped ? (int64_t)G : 0);
  const int64_t blocks = tiles_m * tiles_n;
  if (blocks == 0) return hipSuccess;
  static bool attr_done[2] = {false, false};
  if (!attr_done[grouped]) {
    hipError_t e = grouped ? hipFuncSetAttribute((const void*)gemm_kernel<true>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES)
                           : hipFuncSetAttribute((const void*)gemm_kernel<false>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_done[grouped] = true;
  }
  if (grouped)
    hipLaunchKernelGGL(gemm_kernel<true>, dim3((unsigned)blocks), dim3(256), LDS_BYTES, stream, a, ap, b, bp, c,
                       ldc, M, N, K, offsets, G, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL(gemm_kernel<false>, dim3((unsigned)blocks), dim3(256), LDS_BYTES, stream, a, ap, b, bp, c,
                       ldc, M, N, K, offsets, G, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace mx
