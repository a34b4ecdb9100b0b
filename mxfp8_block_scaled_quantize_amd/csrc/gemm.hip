// Block-scaled MXFP8 GEMM (TN) on the gfx950 scaled FP8 MFMA.
//
//   C[m][n] = bf16_rne( sum_k dq(A)[m][k] * dq(B)[n][k] ), fp32 accumulation.
//
// Operand layout of V_MFMA_SCALE_F32_32X32X64_F8F6F4 with E4M3 on both sides,
// as measured on gfx950: lane l holds row (l % 32) of the 32-row block; its
// bytes 0..15 are K = 16*(l/32) + [0,16) and bytes 16..31 are
// K = 32 + 16*(l/32) + [0,16) of the 64-wide K step.  Bytes 0..15 of every
// lane are scaled by the scale operand of lane (l % 32) and bytes 16..31 by
// that of lane 32 + (l % 32) (byte chosen by op_sel): lane l supplies the
// scale of K-block l / 32.  Result register i of lane l is row
// 8*(i/4) + 4*(l/32) + (i%4), column l % 32 of the product of the first
// operand's rows with the second's.  The kernel passes B first, so it holds
// C^T: lane l has C[l % 32][8*(i/4) + 4*(l/32) + (i%4)], four consecutive
// columns of one row of C in registers 4g .. 4g + 3.
//
// Tiling: one workgroup of 4 waves computes a 256 x 256 tile; wave (wm, wn)
// owns 128 x 128 = 4 x 4 MFMA blocks (256 fp32 accumulators per lane, in
// AGPRs).  K moves in 128-byte steps through a 2-slot LDS ring (66 KB per
// slot: A and B 256 x 128 bytes, plus the step's packed scale words), filled
// by buffer->LDS DMA of whole 128-byte row segments (rows past the end of the
// operand read as zero).  A step runs as two 64-wide halves with their own
// fragment registers: the first half's MFMAs overlap the LDS reads of the
// second half; then one barrier makes step t+1 resident and frees this
// step's slot; the second half's MFMAs overlap the DMA of step t+2 and the
// LDS reads of step t+1.  Each MFMA is issued together with one 16-byte LDS
// read and (second half) one DMA, in a fixed order pinned by scheduling
// barriers; reads come in the order the next MFMAs consume them.  Two steps
// are unrolled so both slots sit at constant LDS offsets (an odd step count
// runs one extra all-zero step).  The scale words are laid out in LDS so
// that the four a lane needs are one 16-byte read.  16-byte chunks of each
// 128-byte LDS row are XOR-swizzled by (row >> 1) & 7, which makes the
// fragment reads conflict free.  Workgroup ids are remapped so the tiles
// resident on one XCD (ids are dealt round-robin to the 8 XCDs) form groups of
// 4 tiles sharing A and B in that XCD's L2, with the XCDs splitting the larger
// of M and N.
//
// Epilogues (template EPI): none, relu(acc)^2, GELU(acc), each applied to the
// fp32 sum before the one BF16 rounding; SwiGLU, where B holds gate rows then
// up rows and a tile covers 128 output columns whose gate and up sums end in
// the same wave (see the SwiGLU DMA and epilogue below).  Accumulate (ACC)
// adds the old C before the rounding; BIAS adds a BF16 value per B row (per
// expert row for the grouped GEMM) to the fp32 sum before the activation.
// MXO writes the output as MXFP8 instead of BF16: the staged BF16 tile (the
// values the BF16 output would hold) is quantized row by row in 32-column
// blocks on its way out, with the scales as packed words [N/128][M].
#include <atomic>

#include "mx_device.h"
#include "launch.h"

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 128;                 // K bytes per pipeline step
constexpr int NSLOT = 2;
constexpr int A_BYTES = BM * BK;        // 32 KB
constexpr int B_BYTES = BN * BK;        // 32 KB
constexpr int SA_OFF = A_BYTES + B_BYTES;
constexpr int SB_OFF = SA_OFF + BM * 4;
constexpr int SLOT_BYTES = SB_OFF + BN * 4;          // 66 KB (67584 B)
constexpr int LDS_BYTES = NSLOT * SLOT_BYTES;        // 132 KB (135168 B)
constexpr int GROUP = 4;                // tiles per L2 group
constexpr int C_LDS_STRIDE = 2 * BN + 16;            // BF16 output tile row in LDS, padded (528 B)
// The staged output tile (256 x 528 B = 135168 B) fills the ring exactly: a
// wider row stride needs a larger ring.
static_assert(BM * C_LDS_STRIDE <= LDS_BYTES, "output tile must fit in the ring");
// SwiGLU epilogue: a tile covers 128 output columns (its 256 B rows are the
// gate and up rows of those columns), staged as 256 x 272 B.
constexpr int SW_TN = 128;
constexpr int SW_LDS_STRIDE = 2 * SW_TN + 16;
static_assert(BM * SW_LDS_STRIDE <= LDS_BYTES, "SwiGLU output tile must fit in the ring");
static_assert(LDS_BYTES <= 160 * 1024, "LDS");
constexpr uint32_t RSRC_FLAGS = 0x00020000u;         // raw buffer, 32-bit data format

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // s_waitcnt with vmcnt = N (6 bits: [3:0] and [15:14]); expcnt and lgkmcnt left at max.
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// Workgroup barrier that the compiler may not move LDS (or any memory)
// accesses across.  The hardware side (which loads and DMAs must have landed)
// is handled by the explicit waits in front of each use.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int V>
struct ic {
  static constexpr int value = V;
};

// MXFP8 output of one 16-byte chunk of a staged BF16 output row: four
// consecutive lanes hold a 32-column block, sixteen consecutive lanes (a DPP
// row) the 128 columns of one packed scale word.  The block amax is the
// integer max of the BF16 magnitudes over the quad, the scale byte and the
// codes follow the quantizer's rowwise rule (the same device functions), and
// the first lane of each 16-lane row assembles the word from the bytes of
// lanes +4, +8, +12 (DPP row shifts).  Every lane of a 16-lane row must execute this (the
// reductions read the other lanes); row_ok only gates the stores.
__device__ __forceinline__ void mx_out_chunk(u32x4 v, bool row_ok, uint8_t* q, uint32_t* word, bool word_lane) {
  uint32_t m = pk_max_u16(pk_max_u16(abs_bits2(v.x), abs_bits2(v.y)), pk_max_u16(abs_bits2(v.z), abs_bits2(v.w)));
  m = max(m & 0xFFFFu, m >> 16);
  m = quad_max(m);
  const uint32_t byte = scale_byte_from_amax(m);
  const uint2 o = quantize8(make_uint4(v.x, v.y, v.z, v.w), byte);
  // DPP row_shl:n (lane i reads lane i + n of its 16-lane row)
  const uint32_t b1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)byte, 0x104, 0xF, 0xF, true);
  const uint32_t b2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)byte, 0x108, 0xF, 0xF, true);
  const uint32_t b3 = (uint32_t)__builtin_amdgcn_mov_dpp((int)byte, 0x10C, 0xF, 0xF, true);
  if (row_ok) {
    *reinterpret_cast<uint2*>(q) = o;
    if (word_lane) *word = byte | (b1 << 8) | (b2 << 16) | (b3 << 24);
  }
}

template <bool GROUPED, bool ACC, int EPI, bool BIAS, bool MXO>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void gemm_kernel(const uint8_t* __restrict__ A, const uint32_t* __restrict__ Ap,
                 const uint8_t* __restrict__ B, const uint32_t* __restrict__ Bp,
                 uint16_t* __restrict__ Cm, int64_t ldc, int64_t M, int64_t N, int64_t K,
                 const int32_t* __restrict__ offsets, int32_t G, int64_t tiles_m, int64_t tiles_n,
                 const uint16_t* __restrict__ bias, uint8_t* __restrict__ Q, int64_t ldq,
                 uint32_t* __restrict__ Qp) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
  lds_u8* smem = (lds_u8*)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS DMA targets stay scalar
  const int wm = wave >> 1, wn = wave & 1;
  // EPI 3 (SwiGLU): B holds 2N rows, gate rows [0, N) then up rows [N, 2N)
  // (per group when grouped); a tile covers SW_TN output columns.
  constexpr bool SW = EPI == 3;
  constexpr int64_t BMUL = SW ? 2 : 1;

  // ---- tile selection: XCD-aware remap (each XCD gets a contiguous range of
  // ids), then groups of GROUP tiles along one dimension walked across the
  // other.  Each XCD streams its own share of one operand and all of the
  // other, so the shares are taken along the larger dimension: N when
  // tiles_n > tiles_m and for the grouped GEMM (every expert's B is read once
  // instead of once per XCD), M otherwise.
  const int64_t nblk = tiles_m * tiles_n;
  const int64_t bid = blockIdx.x;
  const int64_t full = (nblk / 8) * 8;
  const int64_t lid = bid < full ? (bid & 7) * (full >> 3) + (bid >> 3) : bid;
  int64_t tm, tn;
  if (!(GROUPED || tiles_n > tiles_m)) {
    const int64_t per_group = (int64_t)GROUP * tiles_n;
    const int64_t grp = lid / per_group;
    const int64_t first_m = grp * GROUP;
    const int64_t gm = (tiles_m - first_m) < GROUP ? (tiles_m - first_m) : GROUP;
    const int64_t rem = lid - grp * per_group;
    tm = first_m + rem % gm;
    tn = rem / gm;
  } else {
    const int64_t per_group = (int64_t)GROUP * tiles_m;
    const int64_t grp = lid / per_group;
    const int64_t first_n = grp * GROUP;
    const int64_t gn = (tiles_n - first_n) < GROUP ? (tiles_n - first_n) : GROUP;
    const int64_t rem = lid - grp * per_group;
    tn = first_n + rem % gn;
    tm = rem / gn;
  }

  int64_t m_lo, m_hi, b_row0 = 0;
  if (GROUPED) {
    // Row tile tm counts the groups' tiles in order.  Each wave looks at 64
    // groups at a time: lane g loads its group's bounds, a wave prefix sum of
    // the tile counts finds the group holding tile tm, and the result is
    // broadcast from that lane.  Every wave of the workgroup computes the
    // same answer.  Bounds are clamped into [0, M] and then replaced by the
    // running maximum of all bounds so far (carried across 64-group chunks),
    // so groups never overlap even for decreasing offsets (such a group is
    // empty) and the tile count stays within ceil(M / 256) + G.
    int found = -1;
    m_lo = m_hi = 0;
    int carry = 0;   // running maximum of the clamped bounds of earlier chunks
    for (int g0 = 0; g0 < G; g0 += 64) {
      const int g = g0 + lane;
      int lo = 0, hi = 0;
      if (g < G) {
        const int64_t l = offsets[g], h = offsets[g + 1];
        lo = (int)(l < 0 ? 0 : (l > M ? M : l));
        hi = (int)(h < 0 ? 0 : (h > M ? M : h));
      }
      lo = lo > carry ? lo : carry;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {   // inclusive prefix max of the lower bounds
        const int t = __shfl_up(lo, d, 64);
        if (lane >= d) lo = lo > t ? lo : t;
      }
      hi = hi > lo ? hi : lo;
      carry = __builtin_amdgcn_readlane(hi, 63);
      const int nt = (hi - lo + BM - 1) / BM;
      int incl = nt;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_up(incl, d, 64);
        if (lane >= d) incl += t;
      }
      const int total = __builtin_amdgcn_readlane(incl, 63);
      if (tm < total) {
        const int fl = __builtin_ctzll(__ballot(incl > tm));
        const int before = __builtin_amdgcn_readlane(incl - nt, fl);
        found = g0 + fl;
        m_lo = (int64_t)__builtin_amdgcn_readlane(lo, fl) + (tm - before) * BM;
        m_hi = (int64_t)__builtin_amdgcn_readlane(hi, fl);
        break;
      }
      tm -= total;
    }
    if (found < 0) return;  // whole workgroup leaves together
    b_row0 = (int64_t)found * N * BMUL;
  } else {
    m_lo = tm * BM;
    m_hi = M;
  }
  const int64_t n0 = tn * (SW ? SW_TN : BN);
  const int64_t brows = (GROUPED ? (int64_t)G : 1) * N * BMUL;
  const int rows_a = (int)((m_hi - m_lo) < BM ? (m_hi - m_lo) : BM);
  const int rows_b = (int)((N - n0) < BN ? (N - n0) : BN);

  // ---- DMA addressing (same for A and B).  Data goes through raw buffers
  // over the tile's rows, so rows past the end of the operand read as zero.
  // DMA instruction i of wave w covers LDS rows 8(8w + i) + lane/8, chunk
  // slot lane%8; the swizzle (row >> 1) & 7 is (4i + lane/16) & 7.  The step's
  // K offset goes into the scalar offset field.
  uint32_t dma_off[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int r = 64 * wave + 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ ((4 * i + (lane >> 4)) & 7);
    dma_off[i] = (uint32_t)r * (uint32_t)K + 16u * (uint32_t)c;
  }
  // Scale words are stored so that the four words a lane needs (rows
  // 32i + lr of its wave's 128-row half, i = 0..3) are one 16-byte LDS read:
  // word position p = 128 * half + 4 * lr + i holds row 128 * half + 32i + lr.
  // Wave w brings positions 64w + lane (rows past the end are clamped into the
  // valid rows: their data rows are zero, so any scale will do).
  const int sp = 64 * wave + lane;
  const int srow = (sp & ~127) + 32 * (sp & 3) + ((sp & 127) >> 2);
  const int sra = srow < rows_a ? srow : rows_a - 1;
  // SwiGLU: slab row srow lies in 64-row segment s = srow / 64, which holds
  // the gate (s even) or up (s odd) rows of output columns n0 + 64 (s / 2) +
  // [0, 64); rows past N are clamped to the half's last row (their data rows
  // read as zero, so any scale will do).
  int srb;
  if (SW) {
    const int s = srow >> 6;
    const int64_t oc = n0 + 64 * (s >> 1) + (srow & 63);
    srb = (int)((s & 1) * N + (oc < N ? oc : N - 1));
  } else {
    srb = srow < rows_b ? srow : rows_b - 1;
  }

  const int nk = (int)(K / BK);

  // DMA of one 128-wide K step into its slot: 16 data loads per lane (8 rows x
  // 128 B per instruction) plus the step's two scale words, 18 per lane.  It is
  // branch-free: a step past the end gets zero-length buffer ranges, so its
  // loads touch no memory and write zeros to a slot nobody reads.
  const uint32_t a_rec = (uint32_t)((int64_t)rows_a * K);
  const uint32_t b_rec = (uint32_t)((int64_t)rows_b * K);
  const __amdgpu_buffer_rsrc_t ra_v = __builtin_amdgcn_make_buffer_rsrc((void*)(A + m_lo * K), 0, (int)a_rec, RSRC_FLAGS);
  // B: the plain tile is rows b_row0 + n0 + [0, 256).  SwiGLU: wave w DMAs
  // slab rows 64w + [0, 64) (segment w: gate rows for even w, up rows for odd
  // w, of output columns n0 + 64 (w / 2) + [0, 64)); its resource starts 64w
  // rows before that segment's first B row, so the shared row offsets (which
  // include 64w rows) land on it, and ends after the segment's valid rows.
  // Every access is at or after the segment's first row.
  __amdgpu_buffer_rsrc_t rb_v;
  if (SW) {
    const int64_t oc0 = n0 + 64 * (wave >> 1);
    const int64_t seg_rows = N - oc0 < 0 ? 0 : (N - oc0 < 64 ? N - oc0 : 64);
    const int64_t src = b_row0 + (wave & 1) * N + oc0;
    rb_v = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((uintptr_t)B + (uintptr_t)((src - 64 * wave) * K)), 0, (int)((64 * wave + seg_rows) * K), RSRC_FLAGS);
  } else {
    rb_v = __builtin_amdgcn_make_buffer_rsrc((void*)(B + (b_row0 + n0) * K), 0, (int)b_rec, RSRC_FLAGS);
  }
  const __amdgpu_buffer_rsrc_t r_none = __builtin_amdgcn_make_buffer_rsrc((void*)A, 0, 0, RSRC_FLAGS);
  // DMA piece q of step s into SLOT: 0..7 A rows, 8..15 B rows, 16/17 the
  // scale words of A / B.  A step past the end gets zero-length buffer ranges.
  auto dma_piece = [&](int s, auto SLOT, int q) {
    lds_u8* base = smem + decltype(SLOT)::value * SLOT_BYTES;
    const bool valid = s < nk;
    const int k0 = valid ? s * BK : 0;
    const int64_t sv = valid ? s : 0;
    if (q < 8) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(valid ? ra_v : r_none, (lds_void*)(base + 1024 * (8 * wave + q)), 16,
                                               dma_off[q], k0, 0, 0);
    } else if (q < 16) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(valid ? rb_v : r_none,
                                               (lds_void*)(base + A_BYTES + 1024 * (8 * wave + q - 8)), 16,
                                               dma_off[q - 8], k0, 0, 0);
    } else if (q == 16) {
      const __amdgpu_buffer_rsrc_t rsa =
          __builtin_amdgcn_make_buffer_rsrc((void*)(Ap + sv * M + m_lo), 0, valid ? rows_a * 4 : 0, RSRC_FLAGS);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_void*)(base + SA_OFF + 256 * wave), 4, 4u * (uint32_t)sra, 0,
                                               0, 0);
    } else {
      const __amdgpu_buffer_rsrc_t rsb =
          SW ? __builtin_amdgcn_make_buffer_rsrc((void*)(Bp + sv * brows + b_row0), 0, valid ? (int)(8 * N) : 0,
                                                 RSRC_FLAGS)
             : __builtin_amdgcn_make_buffer_rsrc((void*)(Bp + sv * brows + b_row0 + n0), 0, valid ? rows_b * 4 : 0,
                                                 RSRC_FLAGS);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_void*)(base + SB_OFF + 256 * wave), 4, 4u * (uint32_t)srb, 0,
                                               0, 0);
    }
  };
  auto issue_step = [&](int s, auto SLOT) {
#pragma unroll
    for (int q = 0; q < 18; q++) dma_piece(s, SLOT, q);
  };

  // Fragment of lane (row lr, group lg) for K half h: bytes 0..15 are
  // K = 64h + 16lg + [0,16) and bytes 16..31 are K = 64h + 32 + 16lg + [0,16):
  // the MFMA scales bytes 0..15 of every lane with the scale of lane lr and
  // bytes 16..31 with that of lane 32 + lr.
  const int lr = lane & 31;
  const int lg = lane >> 5;
  const int swz = (lr >> 1) & 7;
  const int a_row_off = (wm * 128 + lr) * BK;
  const int b_row_off = A_BYTES + (wn * 128 + lr) * BK;
  const uint32_t sh = 8u * (uint32_t)lg;

  v8i fa[2][4], fb[2][4];
  uint32_t sa[4], sb[4], na[4], nb[4];   // scale words of the current / next step
  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = v16f{};

  // One 16-byte piece q of the fragments: frag q/2 (A blocks 0..3, then B
  // blocks 0..3), low (K block 2h) or high (block 2h+1) half.
  auto read_piece = [&](auto SLOT, auto H, auto SET, int qq) {
    // order: A0, B0..B3, A1..A3 (the operands of MFMA (i, j) in i-major order)
    constexpr int order[16] = {0, 1, 8, 9, 10, 11, 12, 13, 14, 15, 2, 3, 4, 5, 6, 7};
    const int q = order[qq];
    constexpr int h = decltype(H)::value;
    constexpr int set = decltype(SET)::value;
    const lds_u8* base = smem + decltype(SLOT)::value * SLOT_BYTES;
    const int f = q >> 1;
    const int p = (q & 1) ? 16 * ((4 * h + 2 + lg) ^ swz) : 16 * ((4 * h + lg) ^ swz);
    const int off = (f < 4 ? a_row_off + f * 32 * BK : b_row_off + (f - 4) * 32 * BK) + p;
    const v4i v = __builtin_bit_cast(v4i, *(lds_u32x4*)(base + off));
    if (f < 4) {
      if (q & 1) fa[set][f].hi = v; else fa[set][f].lo = v;
    } else {
      if (q & 1) fb[set][f - 4].hi = v; else fb[set][f - 4].lo = v;
    }
  };
  // The four scale words of a step (one 16-byte read each for A and B), read
  // one half before the MFMAs that use them.  They are shifted right by
  // 8 * (lane / 32) when the step starts (the same shift serves both halves;
  // op_sel then picks byte 0 or 2): lane l supplies the scale of K-block l / 32.
  auto read_scales = [&](auto SLOT, uint32_t* ra, uint32_t* rb) {
    const lds_u8* base = smem + decltype(SLOT)::value * SLOT_BYTES;
    const u32x4 a4 = *(lds_u32x4*)(base + SA_OFF + 16 * (wm * 32 + lr));
    const u32x4 b4 = *(lds_u32x4*)(base + SB_OFF + 16 * (wn * 32 + lr));
    ra[0] = a4.x; ra[1] = a4.y; ra[2] = a4.z; ra[3] = a4.w;
    rb[0] = b4.x; rb[1] = b4.y; rb[2] = b4.z; rb[3] = b4.w;
  };
  auto mfma_one = [&](auto SET, auto OPSEL, int q) {
    constexpr int set = decltype(SET)::value;
    constexpr int op = decltype(OPSEL)::value;
    const int i = q >> 2, j = q & 3;
    // B first: the block of C^T, so a lane's registers are consecutive columns of C
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[set][j], fa[set][i], acc[i][j], 0, 0, op,
                                                                (int)sb[j], op, (int)sa[i]);
  };
  // One K step: first half from register set 0 while the second half's
  // fragments load; then make step t+1 resident, refill this step's slot with
  // step t+2, and run the second half while the first-half fragments and the
  // scales of step t+1 load.  Slots alternate, so two steps are unrolled and
  // every LDS address is a constant offset.
  auto kstep = [&](int t, auto SLOT) {
    constexpr int slot = decltype(SLOT)::value;
#pragma unroll
    for (int q = 0; q < 16; q++) {
      mfma_one(ic<0>{}, ic<0>{}, q);
      read_piece(SLOT, ic<1>{}, ic<1>{}, q);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vmcnt<0>();
    wait_lgkm0();
    lds_barrier();
    dma_piece(t + 2, SLOT, 16);
    dma_piece(t + 2, SLOT, 17);
    read_scales(ic<1 - slot>{}, na, nb);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 16; q++) {
      mfma_one(ic<1>{}, ic<2>{}, q);
      read_piece(ic<1 - slot>{}, ic<0>{}, ic<0>{}, q);
      dma_piece(t + 2, SLOT, q);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
      sa[i] = na[i] >> sh;
      sb[i] = nb[i] >> sh;
    }
  };

  if (nk > 0) {
    issue_step(0, ic<0>{});
    issue_step(1, ic<1>{});
    wait_vmcnt<18>();
    lds_barrier();
    // Scale words first, then the fragments in the loop's own read order:
    // on loop entry the outstanding LDS reads are then in the same order as
    // on the back edge, so the wait in front of the first MFMA only covers
    // the reads it needs (otherwise every iteration starts with a full
    // drain of the LDS read queue).
    read_scales(ic<0>{}, sa, sb);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 16; q++) {
      read_piece(ic<0>{}, ic<0>{}, ic<0>{}, q);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
      sa[i] >>= sh;
      sb[i] >>= sh;
    }
    // An odd step count runs one extra all-zero step (its DMA ranges are
    // empty, so its codes and scales read as zero and add nothing).
    for (int t = 0; t < nk; t += 2) {
      kstep(t, ic<0>{});
      kstep(t + 1, ic<1>{});
    }
  }

  wait_vmcnt<0>();   // the tail's empty DMA must land before the ring is reused
  // ---- epilogue: fp32 -> BF16 (RNE, v_cvt_pk_bf16_f32) into a padded
  // row-major LDS tile (the ring is free once every wave is past its last
  // step), then 16-byte stores that cover whole 512-byte row segments of C.
  // Registers 4g .. 4g + 3 of block (i, j) are four consecutive columns of one
  // row: one 8-byte LDS write each.  With ACCUMULATE the current C tile is
  // staged first and each lane adds the old values at its own positions.
  wait_lgkm0();
  lds_barrier();
  // Lane-derived values are re-derived from the lane id here so that none of
  // them stays live (or spills) across the main loop.
  const int elane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const bool full_rows = m_lo + BM <= m_hi;
  // Four BF16 bias values at element offset `at` of the bias array, for the
  // output columns col .. col + 3 (col % 4 == 0, N % 32 == 0: all four are
  // inside N or none is); zeros past N.  One 8-byte load (the bias is
  // 16-byte aligned).
  auto bias4 = [&](int64_t at, int64_t col) -> u32x2 {
    if (col < N) return *reinterpret_cast<const u32x2*>(bias + at);
    return u32x2{0u, 0u};
  };
  if constexpr (SW) {
    // SwiGLU: blocks j = 0, 1 of a wave hold the gate and blocks j + 2 the up
    // products of the same 64 output columns wn * 64 + [0, 64), so each output
    // is SiLU(gate) * up of two registers of the lane, in fp32, rounded once.
    {
      const int lr = elane & 31, lg = elane >> 5;
      // BIAS: the gate bias of output column n is bias[n], the up bias
      // bias[N + n] (per group: the bias rows follow B's rows).
      u32x2 bgate[2][4], bup[2][4];
      if (BIAS) {
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
          for (int g = 0; g < 4; g++) {
            const int64_t col = n0 + wn * 64 + 32 * j + 8 * g + 4 * lg;
            bgate[j][g] = bias4(b_row0 + col, col);
            bup[j][g] = bias4(b_row0 + N + col, col);
          }
      }
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int row = wm * 128 + 32 * i + lr;
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
          for (int g = 0; g < 4; g++) {
            const int col = wn * 64 + 32 * j + 8 * g + 4 * lg;
            float v[4];
#pragma unroll
            for (int t = 0; t < 4; t++) {
              float gt = acc[i][j][4 * g + t], ut = acc[i][j + 2][4 * g + t];
              if (BIAS) {
                gt += bf16_half2(bgate[j][g], t);
                ut += bf16_half2(bup[j][g], t);
              }
              v[t] = silu_f32(gt) * ut;
            }
            const bf16x2 h0 = {(__bf16)v[0], (__bf16)v[1]};
            const bf16x2 h1 = {(__bf16)v[2], (__bf16)v[3]};
            *(__attribute__((address_space(3))) u32x2*)(smem + row * SW_LDS_STRIDE + 2 * col) =
                u32x2{__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1)};
          }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    wait_lgkm0();
    lds_barrier();
    // 16 chunks of 16 bytes per 256-byte output row: 16 rows per pass
    const int ech = elane & 15;
    const int erow0 = 4 * wave + (elane >> 4);
    const int64_t ecol = n0 + 8 * ech;
    if (ecol < N) {
      u32x4 v[16];
#pragma unroll
      for (int k = 0; k < 16; k++) v[k] = *(lds_u32x4*)(smem + (erow0 + 16 * k) * SW_LDS_STRIDE + 16 * ech);
#pragma unroll
      for (int k = 0; k < 16; k++) {
        const int64_t grow = m_lo + erow0 + 16 * k;
        if constexpr (MXO)   // a 16-lane row is one output row's 128 columns: one scale word
          mx_out_chunk(v[k], full_rows || grow < m_hi, Q + grow * ldq + ecol, Qp + (n0 >> 7) * M + grow, ech == 0);
        else if (full_rows || grow < m_hi)
          store_nt16(Cm + grow * ldc + ecol, make_uint4(v[k].x, v[k].y, v[k].z, v[k].w));
      }
    }
    return;
  }
  const int ech = elane & 31;                    // 16-byte chunk of a tile row
  const int erow0 = 2 * wave + (elane >> 5);     // rows erow0 + 8 k
  const int64_t ecol = n0 + 8 * ech;
  if (ACC) {
    // all 32 loads of a thread are issued before the first LDS write, so the
    // tile costs one memory latency (rows / columns outside C read as 0)
    u32x4 v[32];
#pragma unroll
    for (int k = 0; k < 32; k++) {
      const int64_t grow = m_lo + erow0 + 8 * k;
      v[k] = u32x4{0u, 0u, 0u, 0u};
      if (ecol < N && grow < m_hi)
        v[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Cm + grow * ldc + ecol));
    }
#pragma unroll
    for (int k = 0; k < 32; k++)
      *(__attribute__((address_space(3))) u32x4*)(smem + (erow0 + 8 * k) * C_LDS_STRIDE + 16 * ech) = v[k];
    wait_lgkm0();
    lds_barrier();
  }
  {
    const int lr = elane & 31, lg = elane >> 5;
    u32x2 bv[4][4];   // BIAS: the bias of the lane's four columns per (j, g)
    if (BIAS) {
#pragma unroll
      for (int j = 0; j < 4; j++)
#pragma unroll
        for (int g = 0; g < 4; g++) {
          const int64_t gcol = n0 + wn * 128 + 32 * j + 8 * g + 4 * lg;
          bv[j][g] = bias4(b_row0 + gcol, gcol);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int row = wm * 128 + 32 * i + lr;
#pragma unroll
      for (int j = 0; j < 4; j++)
#pragma unroll
        for (int g = 0; g < 4; g++) {
          const int col = wn * 128 + 32 * j + 8 * g + 4 * lg;
          __attribute__((address_space(3))) u32x2* p =
              (__attribute__((address_space(3))) u32x2*)(smem + row * C_LDS_STRIDE + 2 * col);
          float v0 = acc[i][j][4 * g], v1 = acc[i][j][4 * g + 1];
          float v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
          if (ACC) {
            const u32x2 o = *p;
            v0 += __uint_as_float(o.x << 16);
            v1 += __uint_as_float(o.x & 0xFFFF0000u);
            v2 += __uint_as_float(o.y << 16);
            v3 += __uint_as_float(o.y & 0xFFFF0000u);
          }
          if (BIAS) {   // the bias joins the fp32 sum before any activation
            v0 += bf16_half2(bv[j][g], 0);
            v1 += bf16_half2(bv[j][g], 1);
            v2 += bf16_half2(bv[j][g], 2);
            v3 += bf16_half2(bv[j][g], 3);
          }
          if (EPI == 1) {   // relu(acc)^2 in fp32, then the one BF16 rounding
            v0 = fmaxf(v0, 0.0f);
            v1 = fmaxf(v1, 0.0f);
            v2 = fmaxf(v2, 0.0f);
            v3 = fmaxf(v3, 0.0f);
            v0 *= v0;
            v1 *= v1;
            v2 *= v2;
            v3 *= v3;
          }
          if (EPI == 2) {   // GELU(acc) in fp32, then the one BF16 rounding
            v0 = gelu_f32(v0);
            v1 = gelu_f32(v1);
            v2 = gelu_f32(v2);
            v3 = gelu_f32(v3);
          }
          const bf16x2 h0 = {(__bf16)v0, (__bf16)v1};
          const bf16x2 h1 = {(__bf16)v2, (__bf16)v3};
          *p = u32x2{__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1)};
        }
      __builtin_amdgcn_sched_barrier(0);   // bounds the registers the batched AGPR reads take
    }
  }
  wait_lgkm0();
  lds_barrier();
  if (ecol < N) {
    // all LDS reads of a batch before its stores (one LDS latency per batch)
#pragma unroll
    for (int kb = 0; kb < 32; kb += 16) {
      u32x4 v[16];
#pragma unroll
      for (int k = 0; k < 16; k++) v[k] = *(lds_u32x4*)(smem + (erow0 + 8 * (kb + k)) * C_LDS_STRIDE + 16 * ech);
#pragma unroll
      for (int k = 0; k < 16; k++) {
        const int64_t grow = m_lo + erow0 + 8 * (kb + k);
        if constexpr (MXO)   // lanes 16 t .. 16 t + 15 of a row: scale word n0 / 128 + t
          mx_out_chunk(v[k], full_rows || grow < m_hi, Q + grow * ldq + ecol,
                       Qp + ((n0 >> 7) + (ech >> 4)) * M + grow, (ech & 15) == 0);
        else if (full_rows || grow < m_hi)
          store_nt16(Cm + grow * ldc + ecol, make_uint4(v[k].x, v[k].y, v[k].z, v[k].w));
      }
    }
  }
}

bool gemm_grid_fits(int64_t M, int64_t N, int32_t G, bool grouped, bool swiglu) {
  const int64_t tn = swiglu ? (N + SW_TN - 1) / SW_TN : (N + BN - 1) / BN;
  const int64_t tm = (M + BM - 1) / BM + (grouped ? (int64_t)G : 0);
  return grid_fits(tm, tn, 256);
}

template <bool GROUPED, bool ACC, int EPI, bool BIAS, bool MXO>
static hipError_t launch_gemm_t(const uint8_t* a, const uint32_t* ap, const uint8_t* b, const uint32_t* bp,
                                uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K, const int32_t* offsets,
                                int32_t G, int64_t tiles_m, int64_t tiles_n, const uint16_t* bias, MxOut mxo,
                                hipStream_t stream) {
  // The dynamic-LDS opt-in is set once per device (bit d of the mask, for
  // device ids below 64; others set it on every launch), race-free across
  // host threads.  The device is the stream's (the current device for the
  // null stream), made current while the attribute is set.
  static std::atomic<uint64_t> attr_done{0};
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
  if (!bit || !(attr_done.load(std::memory_order_acquire) & bit)) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel<GROUPED, ACC, EPI, BIAS, MXO>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess) return e;
    attr_done.fetch_or(bit, std::memory_order_release);
  }
  hipLaunchKernelGGL((gemm_kernel<GROUPED, ACC, EPI, BIAS, MXO>), dim3((unsigned)(tiles_m * tiles_n)), dim3(256),
                     LDS_BYTES, stream, a, ap, b, bp, c, ldc, M, N, K, offsets, G, tiles_m, tiles_n, bias, mxo.q,
                     mxo.ldq, mxo.qp);
  return hipGetLastError();
}

// One launch for an (epilogue, bias, output format) choice of a dense or
// grouped GEMM.
template <bool GROUPED, bool MXO>
static hipError_t launch_gemm_o(const uint8_t* a, const uint32_t* ap, const uint8_t* b, const uint32_t* bp,
                                uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K, const int32_t* offsets,
                                int32_t G, int64_t tiles_m, int64_t tiles_n, bool accumulate, int epilogue,
                                const uint16_t* bias, MxOut mxo, hipStream_t stream) {
#define MX_G_LAUNCH(AC, EP, BI) \
  launch_gemm_t<GROUPED, AC, EP, BI, MXO>(a, ap, b, bp, c, ldc, M, N, K, offsets, G, tiles_m, tiles_n, bias, mxo, \
                                          stream)
  // accumulate, the epilogues and the bias: the API rejects accumulate
  // together with any of the others, and with the MXFP8 output
  if constexpr (!MXO)
    if (accumulate) return MX_G_LAUNCH(true, 0, false);
  if (bias)
    return epilogue == 1 ? MX_G_LAUNCH(false, 1, true)
         : epilogue == 2 ? MX_G_LAUNCH(false, 2, true)
         : epilogue == 3 ? MX_G_LAUNCH(false, 3, true)
                         : MX_G_LAUNCH(false, 0, true);
  return epilogue == 1 ? MX_G_LAUNCH(false, 1, false)
       : epilogue == 2 ? MX_G_LAUNCH(false, 2, false)
       : epilogue == 3 ? MX_G_LAUNCH(false, 3, false)
                       : MX_G_LAUNCH(false, 0, false);
#undef MX_G_LAUNCH
}

template <bool GROUPED>
static hipError_t launch_gemm_g(const uint8_t* a, const uint32_t* ap, const uint8_t* b, const uint32_t* bp,
                                uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K, const int32_t* offsets,
                                int32_t G, int64_t tiles_m, int64_t tiles_n, bool accumulate, int epilogue,
                                const uint16_t* bias, MxOut mxo, hipStream_t stream) {
  return mxo.q ? launch_gemm_o<GROUPED, true>(a, ap, b, bp, c, ldc, M, N, K, offsets, G, tiles_m, tiles_n,
                                               accumulate, epilogue, bias, mxo, stream)
               : launch_gemm_o<GROUPED, false>(a, ap, b, bp, c, ldc, M, N, K, offsets, G, tiles_m, tiles_n,
                                                accumulate, epilogue, bias, mxo, stream);
}

hipError_t launch_gemm(const uint8_t* a, const uint32_t* ap, const uint8_t* b, const uint32_t* bp,
                       uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K,
                       const int32_t* offsets, int32_t G, bool accumulate, int epilogue, const uint16_t* bias,
                       MxOut mxo, hipStream_t stream) {
  const bool grouped = offsets != nullptr;
  const int64_t tiles_n = epilogue == 3 ? (N + SW_TN - 1) / SW_TN : (N + BN - 1) / BN;
  const int64_t tiles_m = (M + BM - 1) / BM + (grouped ? (int64_t)G : 0);
  if (tiles_m * tiles_n == 0) return hipSuccess;
  return grouped ? launch_gemm_g<true>(a, ap, b, bp, c, ldc, M, N, K, offsets, G, tiles_m, tiles_n, accumulate,
                                       epilogue, bias, mxo, stream)
                 : launch_gemm_g<false>(a, ap, b, bp, c, ldc, M, N, K, offsets, G, tiles_m, tiles_n, accumulate,
                                        epilogue, bias, mxo, stream);
}

}  // namespace mx
