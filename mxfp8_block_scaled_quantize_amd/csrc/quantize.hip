// MXFP8 quantization kernels for gfx950.
//
// Tile kernel: one workgroup of QW waves owns a (32 * QW) x 128 BF16 tile.
// Wave w owns rows [32w, 32w + 32) of the tile; lane (rg = lane / 16,
// cg = lane % 16) owns the 8 x 8 sub-block rows 32w + 8rg + [0, 8), columns
// 8cg + [0, 8), read with eight 16-byte loads (each load instruction of a wave
// covers four rows of 256 contiguous bytes).
//
//  - rowwise 32-blocks are 4 consecutive lanes (a DPP quad) in one row;
//  - columnwise 32-blocks are the 4 lanes cg, cg+16, cg+32, cg+48 of a wave
//    (8 rows each), so every colwise block is reduced inside one wave;
//  - conversion is exact integer scale selection (amax on BF16 bit patterns),
//    a clamp of the BF16 magnitudes to 448 * 2^X, and the hardware scaled
//    convert, which divides by 2^X and rounds to nearest even;
//  - the columnwise codes are built column-major in registers (a byte permute
//    pairs two rows of one column per convert), written to a transposed LDS
//    tile and streamed out as full (32 * QW)-byte rows of q_colT;
//  - the scale bytes of a tile are gathered in LDS and stored as one word per
//    row (rowwise) and one QW-byte group per column (columnwise) instead of
//    single bytes;
//  - dbias partial sums are reduced lane -> wave -> workgroup and written once
//    per (row tile, column); a second kernel sums the row tiles.
//
//  - with a fused activation (squared ReLU, GELU or their backward) the tile
//    kernel quantizes the fp32 activation values by the same block rule.
//
// Flat kernel: the rowwise copy of a contiguous input is one stream of
// 32-element blocks (see quantize_rowwise_flat_kernel).  Panel kernel: the
// rowwise copy with its scales written as packed words (see
// quantize_rowwise_packed_kernel).
#include <mutex>

#include "mx_device.h"
#include "launch.h"

namespace mx {

// Device scratch of the allocation-free quantize entry point: the dbias
// partial sums (one fp32 per row tile and column) live here instead of in a
// caller workspace.  Each GPU holds its own copy for the life of the process;
// host code reaches it only through the address hipGetSymbolAddress returns
// for that device (the array's name is not a device address on the host).
static __device__ __align__(256) float scratch[kNoallocScratchBytes / sizeof(float)];

hipError_t noalloc_scratch(hipStream_t stream, float** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float* addr[kMaxDevices];
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    // once per device, with that device current
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = static_cast<float*>(p);
  }
  *out = addr[dev];
  return hipSuccess;
}

// Options of one quantize call that only change where results go: all
// uniform across the grid.
struct QuantOpts {
  uint32_t* amax;        // non-null: atomic max of |x| (fp32 bit patterns order like the values)
  const int32_t* noop;   // non-null and *noop != 0: write nothing
  int packed;            // scales in the packed word layout instead of bytes
};

__device__ __forceinline__ bool skip_call(const QuantOpts& o) { return o.noop != nullptr && *o.noop != 0; }

// Fold a per-lane amax (fp32 bit pattern of |x|) into the tensor amax: wave
// maximum, then one atomic per wave, skipped when the stored value is already
// at least as large (max is order independent: the result is exact).
__device__ __forceinline__ void fold_amax(const QuantOpts& o, uint32_t m) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const uint32_t t = (uint32_t)__shfl_xor((int)m, d, 64);
    m = m > t ? m : t;
  }
  if ((threadIdx.x & 63) == 0) {
    if (m > __hip_atomic_load(o.amax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(o.amax, m);
  }
}

// Activation fused into the quantizer: none, squared ReLU relu(x)^2 or its
// backward grad * 2 relu(a), GELU x Phi(x) or its backward grad * GELU'(a).
// Values are fp32 and are quantized with the fp32 form of the scaled convert.
// The squared-ReLU values are exact in fp32 (products of two BF16 values
// inside its normal range); the GELU values are within the error bounds
// stated with gelu_f32 / dgelu_f32 in mx_device.h.
enum { ACT_NONE = 0, ACT_SQRELU = 1, DACT_SQRELU = 2, ACT_GELU = 3, DACT_GELU = 4 };

// relu of two BF16 values on their bits: every negative value (-0 included)
// is a negative signed halfword, so a signed max with 0 (v_pk_max_i16) gives
// +0 for it and leaves non-negative values unchanged.
__device__ __forceinline__ uint32_t relu_bf16x2(uint32_t w) {
  const i16x2 z = {0, 0};
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(i16x2, w), z));
}

// Exact doubling of two non-negative BF16 values on their bits: a normal
// value gains one in the exponent field (+0x80); a zero or subnormal one
// (bits < 0x80) doubles its bit pattern, carrying into the exponent field
// when it becomes normal.  Both cases are bits + min(bits, 0x80).  Values of
// 2^127 and above overflow to the infinity / NaN patterns, as 2a does in fp32.
__device__ __forceinline__ uint32_t twice_bf16x2(uint32_t w) {
  const u16x2 h = __builtin_bit_cast(u16x2, w);
  const u16x2 c = {0x80, 0x80};
  return __builtin_bit_cast(uint32_t, h + __builtin_elementwise_min(h, c));
}

__device__ __forceinline__ float bf_half(uint4 v, int k) {
  const uint32_t d = (k >> 1) == 0 ? v.x : (k >> 1) == 1 ? v.y : (k >> 1) == 2 ? v.z : v.w;
  return (k & 1) ? bf_hi(d) : bf_lo(d);
}

// E8M0 byte of a block from the fp32 bit pattern of its amax (same rule as the
// BF16 form: biased exponent - 8, clamped at 0).
__device__ __forceinline__ uint32_t scale_byte_from_amax_f32(uint32_t amax_bits) {
  const int e = (int)(amax_bits >> 23);
  return (uint32_t)(e > 8 ? e - 8 : 0);
}

// Four fp32 values -> four E4M3 codes of v / 2^(byte - 127), magnitudes first
// clamped to 448 * 2^(byte - 127) (fp32 pattern (byte + 8) << 23 | 0x600000).
__device__ __forceinline__ uint32_t cvt4_scaled_f32(float a, float b, float c, float d, uint32_t byte) {
  const float lim = __uint_as_float(((byte + 8u) << 23) | 0x600000u);
  const float f = __uint_as_float(byte << 23);
  const float ca = __builtin_amdgcn_fmed3f(a, -lim, lim);
  // both halves of the result are written below: any register serves as the
  // initial contents (a dead one saves a move)
  i16x2 r = __builtin_bit_cast(i16x2, ca);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, ca, __builtin_amdgcn_fmed3f(b, -lim, lim), f, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, __builtin_amdgcn_fmed3f(c, -lim, lim),
                                               __builtin_amdgcn_fmed3f(d, -lim, lim), f, true);
  return __builtin_bit_cast(uint32_t, r);
}

constexpr int QT_C = 128;            // tile columns
constexpr int QT_R_MIN = 128;        // rows of the smallest tile (4 waves)

template <bool ROW, bool COL, bool DBIAS, int QW, int ACT>
__global__ __launch_bounds__(64 * QW) void quantize_tile_kernel(
    const uint16_t* __restrict__ x, int64_t R, int64_t C, int64_t ldx,
    uint8_t* __restrict__ q_row, uint8_t* __restrict__ s_row,
    uint8_t* __restrict__ q_colT, uint8_t* __restrict__ s_colT,
    float* __restrict__ dbias_part, int64_t tiles_c, QuantOpts opt, const uint16_t* __restrict__ act_in) {
  constexpr int TR = 32 * QW;   // tile rows
  constexpr int NT = 64 * QW;   // threads
  constexpr int TGR = QW == 8 ? 8 : 1;   // row tiles per group of the tile order (1: plain row-major)
  // Transposed FP8 tile [column][row]; 8-byte row units XOR-swizzled by the
  // column group to spread the transposing writes over the banks.
  __shared__ __attribute__((aligned(16))) uint8_t lds_t[COL ? QT_C * TR : 16];
  __shared__ __attribute__((aligned(16))) uint8_t lds_sc[COL ? QT_C * QW : 16];  // [column][wave]
  __shared__ __attribute__((aligned(16))) uint8_t lds_sr[ROW ? TR * 4 : 16];     // [row][block]
  __shared__ float lds_db[DBIAS ? QW * QT_C : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int cg = lane & 15;
  const int rg = lane >> 4;
  if (skip_call(opt)) return;   // uniform: the whole grid leaves
  // Tile order: groups of TGR row tiles walked row tile fastest, so the 8
  // XCDs (workgroup ids are dealt to them round-robin) each take one row band
  // of a group across all its column tiles: contiguous input rows and
  // row-code rows per XCD, and the transposed codes of a column band written
  // as 8 adjacent row runs at once.
  const int64_t tiles_r = (R + TR - 1) / TR;
  const int64_t per_g = (int64_t)TGR * tiles_c;
  const int64_t gq = (int64_t)blockIdx.x / per_g;
  const int64_t first_r = gq * TGR;
  const int64_t gr = (tiles_r - first_r) < TGR ? (tiles_r - first_r) : TGR;
  const int64_t remq = (int64_t)blockIdx.x - gq * per_g;
  const int64_t tr = first_r + remq % gr;
  const int64_t tc = remq / gr;
  const int64_t r0 = tr * TR;
  const int64_t c0 = tc * QT_C;
  const int64_t rb = r0 + 32 * w + 8 * rg;  // first row of this lane
  const int64_t cb = c0 + 8 * cg;           // first column of this lane
  const bool cval = cb < C;                 // C % 32 == 0: whole quads are valid

  // Tiles entirely inside the tensor (uniform test) load without per-row
  // guards; edge tiles read zeros outside it.
  const bool full_tile = r0 + TR <= R && c0 + QT_C <= C;
  // Inputs are read once: non-temporal loads.
  auto load_rows = [&](const uint16_t* __restrict__ src, uint4 (&d)[8]) {
    if (full_tile) {
#pragma unroll
      for (int i = 0; i < 8; i++) d[i] = load_nt16(src + (rb + i) * ldx + cb);
    } else {
#pragma unroll
      for (int i = 0; i < 8; i++)
        d[i] = (cval && rb + i < R) ? load_nt16(src + (rb + i) * ldx + cb) : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  uint4 v[8];
  load_rows(x, v);

  uint32_t lane_amax = 0;
  if constexpr (ACT != ACT_NONE) {
    // ---- activation path.  relu is applied to the BF16 bits in place.  For
    // the squared ReLU and its backward the fp32 value of row i, column k of
    // the lane is recomputed where it is needed (a few operations; keeping 64
    // fp32 values live would halve the waves per SIMD); GELU keeps them (see
    // below).  Squared ReLU: max r^2 = (max r)^2, so block amaxes come from
    // integer maxima of the relu'd BF16 bits, as in the plain path.
    constexpr bool DACT = ACT == DACT_SQRELU || ACT == DACT_GELU;
    uint4 a[8];
    if (ACT == DACT_SQRELU) {
      load_rows(act_in, a);
#pragma unroll
      for (int i = 0; i < 8; i++)
        a[i] = make_uint4(twice_bf16x2(relu_bf16x2(a[i].x)), twice_bf16x2(relu_bf16x2(a[i].y)),
                          twice_bf16x2(relu_bf16x2(a[i].z)), twice_bf16x2(relu_bf16x2(a[i].w)));
    } else if (ACT == DACT_GELU) {
      load_rows(act_in, a);
    } else if (ACT == ACT_SQRELU) {
#pragma unroll
      for (int i = 0; i < 8; i++)
        v[i] = make_uint4(relu_bf16x2(v[i].x), relu_bf16x2(v[i].y), relu_bf16x2(v[i].z), relu_bf16x2(v[i].w));
    }
    // GELU (about 20 VALU operations, one v_exp and one v_rcp a value) is
    // evaluated once and its 64 results are kept for both passes.  Right
    // after a GEMM, where an MLP runs it and the clock is power-limited, that
    // is a third faster than recomputing (8192 x 14336 row + col: 116 against
    // 175 us); alone at full clock recomputing is faster (103 against 121 us,
    // more waves per SIMD), but that is not where the launch runs.
    constexpr bool KEEP = ACT == ACT_GELU || ACT == DACT_GELU;
    float fv[KEEP ? 8 : 1][8];
    if constexpr (KEEP) {
#pragma unroll
      for (int i = 0; i < 8; i++)
#pragma unroll
        for (int k = 0; k < 8; k++)
          fv[i][k] = ACT == ACT_GELU ? gelu_f32(bf_half(v[i], k))
                                     : bf_half(v[i], k) * dgelu_f32(bf_half(a[i], k));
    }
    auto val = [&](int i, int k) -> float {
      if (KEEP) return fv[KEEP ? i : 0][k];
      const float xv = bf_half(v[i], k);
      if (ACT == ACT_SQRELU) return xv * xv;
      return xv * bf_half(a[i], k);   // a holds 2 relu(a)
    };
    // |value| bits -> block amax bits (squared ReLU: from the max relu'd input)
    auto sq_bits = [](uint32_t r15) -> uint32_t {
      const float r = __uint_as_float(r15 << 16);
      return __float_as_uint(r * r);
    };
    if (ROW) {
#pragma unroll
      for (int i = 0; i < 8; i++) {
        float f[8];
        uint32_t m = 0;
        if (ACT == ACT_SQRELU) {
          uint32_t h = pk_max_u16(pk_max_u16(v[i].x, v[i].y), pk_max_u16(v[i].z, v[i].w));
          m = sq_bits(quad_max(max(h & 0xFFFFu, h >> 16)));
#pragma unroll
          for (int k = 0; k < 8; k++) f[k] = val(i, k);
        } else {
          float fm = 0.0f;
#pragma unroll
          for (int k = 0; k < 8; k++) {
            f[k] = val(i, k);
            fm = fmaxf(fm, fabsf(f[k]));
          }
          m = quad_max(__float_as_uint(fm));
        }
        lane_amax = max(lane_amax, m);
        const uint32_t byte = scale_byte_from_amax_f32(m);
        uint2 o;
        o.x = cvt4_scaled_f32(f[0], f[1], f[2], f[3], byte);
        o.y = cvt4_scaled_f32(f[4], f[5], f[6], f[7], byte);
        const int64_t r = rb + i;
        if (cval && r < R) store_nt8(q_row + r * C + cb, o);
        if ((cg & 3) == 0) lds_sr[(32 * w + 8 * rg + i) * 4 + (cg >> 2)] = (uint8_t)byte;
      }
    }
    if (!KEEP && ROW && (COL || DBIAS)) {
      // Opaque to the optimiser: the column pass recomputes its values
      // instead of keeping the row pass's 64 fp32 results alive.
#pragma unroll
      for (int i = 0; i < 8; i++) {
        asm volatile("" : "+v"(v[i].x), "+v"(v[i].y), "+v"(v[i].z), "+v"(v[i].w));
        if (DACT) asm volatile("" : "+v"(a[i].x), "+v"(a[i].y), "+v"(a[i].z), "+v"(a[i].w));
      }
    }
    if (COL || DBIAS) {
      const int u = 4 * w + rg;
      const int swz = 2 * (cg & 7);
      uint32_t cm[4] = {0u, 0u, 0u, 0u};
      if (ACT == ACT_SQRELU && COL) {
#pragma unroll
        for (int i = 0; i < 8; i++) {
          cm[0] = pk_max_u16(cm[0], v[i].x);
          cm[1] = pk_max_u16(cm[1], v[i].y);
          cm[2] = pk_max_u16(cm[2], v[i].z);
          cm[3] = pk_max_u16(cm[3], v[i].w);
        }
#pragma unroll
        for (int j = 0; j < 4; j++) {
          cm[j] = pk_max_u16(cm[j], (uint32_t)__shfl_xor((int)cm[j], 16, 64));
          cm[j] = pk_max_u16(cm[j], (uint32_t)__shfl_xor((int)cm[j], 32, 64));
        }
      }
      float cs[8];
#pragma unroll
      for (int k = 0; k < 8; k++) {
        float f[8];
        float fm = 0.0f;
        float t = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; i++) {
          f[i] = val(i, k);
          if (ACT != ACT_SQRELU) fm = fmaxf(fm, fabsf(f[i]));
          if (DBIAS) t += f[i];
        }
        uint32_t m = __float_as_uint(fm);
        if (DBIAS) {
          t += __shfl_xor(t, 16, 64);
          t += __shfl_xor(t, 32, 64);
          cs[k] = t;
        }
        if (COL) {
          if (ACT == ACT_SQRELU) {
            m = sq_bits((k & 1) ? (cm[k >> 1] >> 16) : (cm[k >> 1] & 0xFFFFu));
          } else {
            m = max(m, (uint32_t)__shfl_xor((int)m, 16, 64));
            m = max(m, (uint32_t)__shfl_xor((int)m, 32, 64));
          }
          if (!ROW) lane_amax = max(lane_amax, m);
          const uint32_t byte = scale_byte_from_amax_f32(m);
          uint2 o;
          o.x = cvt4_scaled_f32(f[0], f[1], f[2], f[3], byte);
          o.y = cvt4_scaled_f32(f[4], f[5], f[6], f[7], byte);
          const int cl = 8 * cg + k;
          *reinterpret_cast<uint2*>(lds_t + cl * TR + 8 * (u ^ swz)) = o;
          if (rg == 0) lds_sc[cl * QW + w] = (uint8_t)byte;
        }
      }
      if (DBIAS && rg == 0) {
#pragma unroll
        for (int k = 0; k < 8; k++) lds_db[w * QT_C + 8 * cg + k] = cs[k];
      }
    }
  } else {
  if (ROW) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      uint32_t m = pk_max_u16(pk_max_u16(abs_bits2(v[i].x), abs_bits2(v[i].y)),
                              pk_max_u16(abs_bits2(v[i].z), abs_bits2(v[i].w)));
      m = max(m & 0xFFFFu, m >> 16);
      m = quad_max(m);
      lane_amax = max(lane_amax, m);
      const uint32_t byte = scale_byte_from_amax(m);
      const uint2 o = quantize8(v[i], byte);
      const int64_t r = rb + i;
      if (cval && r < R) store_nt8(q_row + r * C + cb, o);
      if ((cg & 3) == 0) lds_sr[(32 * w + 8 * rg + i) * 4 + (cg >> 2)] = (uint8_t)byte;
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
    if (!ROW) {
#pragma unroll
      for (int j = 0; j < 4; j++) lane_amax = max(lane_amax, max(cm[j] & 0xFFFFu, cm[j] >> 16));
    }
    // Dword j of every row holds columns 2j (low half) and 2j + 1 (high half):
    // clamp both halves with their own column's limit.
    uint32_t cbyte[8], cw[8][4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      cbyte[2 * j] = scale_byte_from_amax(cm[j] & 0xFFFFu);
      cbyte[2 * j + 1] = scale_byte_from_amax(cm[j] >> 16);
      const uint32_t lim2 = sat_limit_bits(cbyte[2 * j]) | (sat_limit_bits(cbyte[2 * j + 1]) << 16);
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const uint32_t d = j == 0 ? v[i].x : j == 1 ? v[i].y : j == 2 ? v[i].z : v[i].w;
        cw[i][j] = clamp_bf16x2(d, lim2);
      }
    }
    const int u = 4 * w + rg;             // 8-row unit of this lane inside the tile
    const int swz = 2 * (cg & 7);         // even XOR keeps 16-byte pairs of units adjacent
#pragma unroll
    for (int k = 0; k < 8; k++) {
      // rows 2p and 2p + 1 of column k side by side: bytes 0-1 / 2-3 of each dword
      const uint32_t sel = (k & 1) ? 0x07060302u : 0x05040100u;
      uint32_t d[4];
#pragma unroll
      for (int p = 0; p < 4; p++) d[p] = __builtin_amdgcn_perm(cw[2 * p + 1][k >> 1], cw[2 * p][k >> 1], sel);
      uint2 o;
      o.x = cvt4_scaled(d[0], d[1], cbyte[k]);
      o.y = cvt4_scaled(d[2], d[3], cbyte[k]);
      const int cl = 8 * cg + k;
      *reinterpret_cast<uint2*>(lds_t + cl * TR + 8 * (u ^ swz)) = o;
      if (rg == 0) lds_sc[cl * QW + w] = (uint8_t)cbyte[k];
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
  }   // activation / plain

  if (opt.amax) fold_amax(opt, ACT ? lane_amax : lane_amax << 16);   // uniform branch

  __syncthreads();

  if (COL) {
    // Transposed rows are TR bytes: CH 16-byte chunks each.
    constexpr int CH = TR / 16;
#pragma unroll
    for (int j = 0; j < (QT_C * CH) / NT; j++) {
      const int t = tid + NT * j;
      const int cl = t / CH;
      const int ch = t % CH;
      const int swz = 2 * ((cl >> 3) & 7);
      const uint4 d = *reinterpret_cast<const uint4*>(lds_t + cl * TR + 8 * ((2 * ch) ^ swz));
      const int64_t col = c0 + cl;
      const int64_t row = r0 + 16 * ch;
      if (col < C && row < R) *reinterpret_cast<uint4*>(q_colT + col * R + row) = d;
    }
    // The QW scale bytes of a column: QW consecutive row blocks of s_colT
    // (packed layout: QW / 4 words (t, col), t = 128-row slab, R % 128 == 0).
    if (opt.packed && tid < QT_C) {
      const int64_t col = c0 + tid;
      if (col < C) {
#pragma unroll
        for (int k = 0; k < QW / 4; k++) {
          const int64_t t = (r0 >> 7) + k;
          if (t < (R >> 7))
            reinterpret_cast<uint32_t*>(s_colT)[t * C + col] =
                *reinterpret_cast<const uint32_t*>(lds_sc + tid * QW + 4 * k);
        }
      }
    } else if (tid < QT_C) {
      const int64_t col = c0 + tid;
      const int64_t nrb = R >> 5;
      const int64_t b0 = r0 >> 5;
      if (col < C) {
        uint8_t* dst = s_colT + col * nrb + b0;
        const bool whole = b0 + QW <= nrb && (reinterpret_cast<uintptr_t>(dst) & (QW - 1)) == 0;
        if (QW == 8 && whole) {
          *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(lds_sc + tid * QW);
        } else if (QW == 4 && whole) {
          *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(lds_sc + tid * QW);
        } else {
          for (int j = 0; j < QW && b0 + j < nrb; j++) dst[j] = lds_sc[tid * QW + j];
        }
      }
    }
  }
  if (ROW && tid >= NT - TR) {
    // The 4 scale bytes of a row of the tile (one per 32-column block).
    const int rl = tid - (NT - TR);
    const int64_t row = r0 + rl;
    if (row < R && opt.packed) {
      // packed layout: word (tc, row) of uint32 [C / 128][R] (C % 128 == 0)
      reinterpret_cast<uint32_t*>(s_row)[tc * R + row] = *reinterpret_cast<const uint32_t*>(lds_sr + 4 * rl);
    } else if (row < R) {
      const int64_t ncb = C >> 5;
      const uint32_t word = *reinterpret_cast<const uint32_t*>(lds_sr + 4 * rl);
      uint8_t* dst = s_row + row * ncb + 4 * tc;
      const int64_t nb = ncb - 4 * tc;
      if (nb >= 4 && (reinterpret_cast<uintptr_t>(dst) & 3) == 0) {
        *reinterpret_cast<uint32_t*>(dst) = word;
      } else {
        for (int j = 0; j < 4 && j < nb; j++) dst[j] = (uint8_t)(word >> (8 * j));
      }
    }
  }
  if (DBIAS) {
    if (tid < QT_C && c0 + tid < C) {
      // pairwise over the waves (QW is 4 or 8)
      float t[QW];
#pragma unroll
      for (int q = 0; q < QW; q++) t[q] = lds_db[q * QT_C + tid];
#pragma unroll
      for (int h = QW / 2; h >= 1; h /= 2)
#pragma unroll
        for (int q = 0; q < h; q++) t[q] = t[q] + t[q + h];
      dbias_part[tr * C + c0 + tid] = t[0];
    }
  }
}

// Rowwise copy of a contiguous input (ld_x == cols): blocks never cross rows
// (cols % 32 == 0), so the tensor is one flat stream of 32-element blocks and
// the scales [rows][cols/32] are the flat block index.  Each wave quantizes
// FL_ELEMS contiguous elements: load u of lane l covers elements
// 512u + 8l + [0, 8), i.e. every load instruction reads 1 KB contiguous, each
// DPP quad holds one block, codes go out as 512-byte runs and
// the wave's 32 scale bytes are contiguous.  Two loads per lane measured best
// (more waves in flight than with four or eight).
constexpr int FL_THREADS = 256;
constexpr int FL_LOADS = 2;
constexpr int64_t FL_ELEMS = 512 * FL_LOADS;  // per wave

__global__ __launch_bounds__(FL_THREADS) void quantize_rowwise_flat_kernel(const uint16_t* __restrict__ x,
                                                                          int64_t total,
                                                                          uint8_t* __restrict__ q,
                                                                          uint8_t* __restrict__ s, QuantOpts opt) {
  if (skip_call(opt)) return;
  const int lane = threadIdx.x & 63;
  uint32_t lane_amax = 0;
  const int64_t base = ((int64_t)blockIdx.x * (FL_THREADS / 64) + (threadIdx.x >> 6)) * FL_ELEMS;
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
    lane_amax = max(lane_amax, m);
    const uint32_t byte = scale_byte_from_amax(m);
    const uint2 o = quantize8(v[u], byte);
    if (e < total) {  // total % 32 == 0: a quad is entirely in or out
      *reinterpret_cast<uint2*>(q + e) = o;
      if ((lane & 3) == 0) s[e >> 5] = (uint8_t)byte;
    }
  }
  if (opt.amax) fold_amax(opt, lane_amax << 16);
}

// Rowwise copy with scales in the packed word layout (C % 128 == 0): a
// workgroup owns a panel of 8 rows x 512 columns; wave w holds rows 2w, 2w+1
// and lane l columns 8l + [0, 8) of each, so every load instruction still
// reads 1 KB contiguous and each DPP quad holds one block.  The panel's 8 x 4
// packed words (slab = 128 columns) are gathered in LDS and written as four
// 32-byte runs; panels are ordered rows-fastest inside an XCD's id range, so
// the four panels that fill one 128-byte line of a slab run back to back on
// one XCD.
constexpr int PN_ROWS = 8;
constexpr int PN_COLS = 512;

__global__ __launch_bounds__(256) void quantize_rowwise_packed_kernel(const uint16_t* __restrict__ x, int64_t R,
                                                                      int64_t C, int64_t ldx,
                                                                      uint8_t* __restrict__ q,
                                                                      uint32_t* __restrict__ packed, QuantOpts opt) {
  if (skip_call(opt)) return;
  __shared__ __attribute__((aligned(16))) uint8_t lds_s[PN_ROWS * 4 * 4];   // [row][slab][block]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int64_t n_rb = (R + PN_ROWS - 1) / PN_ROWS;
  const int64_t nwg = gridDim.x;
  const int64_t bid = blockIdx.x;
  const int64_t full = (nwg / 8) * 8;
  const int64_t lid = bid < full ? (bid & 7) * (full >> 3) + (bid >> 3) : bid;
  const int64_t cbk = lid / n_rb;
  const int64_t r0 = (lid - cbk * n_rb) * PN_ROWS;
  const int64_t c0 = cbk * PN_COLS;
  const int64_t col = c0 + 8 * lane;
  const bool cval = col < C;            // C % 128 == 0: whole quads (and slabs) are valid
  uint4 v[2];
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const int64_t r = r0 + 2 * w + u;
    v[u] = (cval && r < R) ? *reinterpret_cast<const uint4*>(x + r * ldx + col) : make_uint4(0u, 0u, 0u, 0u);
  }
  uint32_t lane_amax = 0;
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const int64_t r = r0 + 2 * w + u;
    uint32_t m = pk_max_u16(pk_max_u16(abs_bits2(v[u].x), abs_bits2(v[u].y)),
                            pk_max_u16(abs_bits2(v[u].z), abs_bits2(v[u].w)));
    m = max(m & 0xFFFFu, m >> 16);
    m = quad_max(m);
    lane_amax = max(lane_amax, m);
    const uint32_t byte = scale_byte_from_amax(m);
    const uint2 o = quantize8(v[u], byte);
    if (cval && r < R) *reinterpret_cast<uint2*>(q + r * C + col) = o;
    // lane 16k + 4b holds block b of slab k
    if ((lane & 3) == 0) lds_s[((2 * w + u) * 4 + (lane >> 4)) * 4 + ((lane >> 2) & 3)] = (uint8_t)byte;
  }
  if (opt.amax) fold_amax(opt, lane_amax << 16);
  __syncthreads();
  if (tid < PN_ROWS * 4) {
    const int slab = tid >> 3, row = tid & 7;
    const int64_t t = (c0 >> 7) + slab;
    const int64_t r = r0 + row;
    if (t < (C >> 7) && r < R)
      packed[t * R + r] = *reinterpret_cast<const uint32_t*>(lds_s + (row * 4 + slab) * 4);
  }
}

// dbias[c] = sum over row tiles of the partial sums.  A workgroup owns 32
// columns; its 8 thread groups sum the row tiles g, g + 8, g + 16, ... of a
// column and the 8 sums are combined pairwise (a fixed order: the result is
// deterministic).
constexpr int DB_COLS = 32;
constexpr int DB_PARTS = 8;

__global__ __launch_bounds__(DB_COLS * DB_PARTS) void dbias_reduce_kernel(const float* __restrict__ part,
                                                                          int64_t tiles, int64_t C,
                                                                          float* __restrict__ out,
                                                                          const int32_t* __restrict__ noop) {
  if (noop != nullptr && *noop != 0) return;
  __shared__ float lds[DB_PARTS][DB_COLS];
  const int cl = threadIdx.x % DB_COLS;
  const int g = threadIdx.x / DB_COLS;
  const int64_t c = (int64_t)blockIdx.x * DB_COLS + cl;
  float s = 0.0f;
  if (c < C)
    for (int64_t t = g; t < tiles; t += DB_PARTS) s += part[t * C + c];
  lds[g][cl] = s;
  __syncthreads();
  if (g == 0 && c < C) {
    float q[DB_PARTS];
#pragma unroll
    for (int p = 0; p < DB_PARTS; p++) q[p] = lds[p][cl];
#pragma unroll
    for (int h = DB_PARTS / 2; h >= 1; h /= 2)
#pragma unroll
      for (int p = 0; p < h; p++) q[p] = q[p] + q[p + h];
    out[c] = q[0];
  }
}

__global__ __launch_bounds__(256) void fill_zero_f32_kernel(float* __restrict__ out, int64_t n,
                                                            const int32_t* __restrict__ noop) {
  if (noop != nullptr && *noop != 0) return;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = 0.0f;
}

int64_t quantize_row_tiles(int64_t R) { return (R + QT_R_MIN - 1) / QT_R_MIN; }
int64_t quantize_col_tiles(int64_t C) { return (C + QT_C - 1) / QT_C; }

// Which kernel a call runs: the packed-scale rowwise panel kernel, the flat
// rowwise kernel (contiguous rows, byte scales) or the tile kernel (every
// other copy set, dbias, activations).
enum QuantPath { QP_PACKED_ROW, QP_FLAT, QP_TILES };
static QuantPath quantize_path(int64_t C, int64_t ldx, uint32_t flags) {
  const bool row = flags & 1u, col = flags & 2u, db = flags & 4u, packed = flags & 16u;
  const bool act = flags & (32u | 64u | 128u | 256u);
  if (row && !col && !db && packed && !act) return QP_PACKED_ROW;
  if (row && !col && !db && !packed && !act && ldx == C) return QP_FLAT;
  return QP_TILES;
}
// Waves of the tile kernel: 8 when the rowwise copy is written or for the
// rowwise copy alone, 4 for the columnwise copy alone.
constexpr int tile_waves(bool row, bool col) { return (row || !col) ? 8 : 4; }

bool quantize_grids_fit(int64_t R, int64_t C, int64_t ldx, uint32_t flags) {
  bool ok;
  switch (quantize_path(C, ldx, flags)) {
    case QP_PACKED_ROW:
      ok = grid_fits((R + PN_ROWS - 1) / PN_ROWS, (C + PN_COLS - 1) / PN_COLS, 256);
      break;
    case QP_FLAT: {
      const int64_t per_block = FL_ELEMS * (FL_THREADS / 64);
      ok = grid_fits((R * C + per_block - 1) / per_block, 1, FL_THREADS);
      break;
    }
    default: {
      const int qw = tile_waves(flags & 1u, flags & 2u);
      ok = grid_fits((R + 32 * qw - 1) / (32 * qw), quantize_col_tiles(C), 64 * qw);
    }
  }
  // the dbias reduce (one 32-column group per workgroup; the zero fill of an
  // empty dbias needs fewer work-items)
  if (flags & 4u) ok = ok && grid_fits((C + DB_COLS - 1) / DB_COLS, 1, DB_COLS * DB_PARTS);
  return ok;
}

// Tile configuration per copy set (measured on MI355X with the stress,
// backward and columnwise-only shapes): 8 waves when the rowwise copy is
// written, 4 for the columnwise copy alone (4-wave row + col tiles were 1-5 %
// faster on 60-240 MB tensors, where the last round of 8-wave tiles is
// partly empty, but 7 % slower on 1 GB and 3 % slower with dbias).  Inputs
// are read and row codes written non-temporally; the transposed codes, which
// a later wgrad reads, are written cached.
template <bool ROW, bool COL, bool DBIAS, int ACT>
static hipError_t launch_tiles(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, uint8_t* q_row,
                               uint8_t* s_row, uint8_t* q_colT, uint8_t* s_colT, float* dbias_part,
                               const QuantOpts& opt, const uint16_t* act_in, int64_t* row_tiles,
                               hipStream_t stream) {
  constexpr int QW = tile_waves(ROW, COL);
  const int64_t tr = (R + 32 * QW - 1) / (32 * QW);
  const int64_t tc = quantize_col_tiles(C);
  *row_tiles = tr;
  if (tr * tc == 0) return hipSuccess;
  hipLaunchKernelGGL((quantize_tile_kernel<ROW, COL, DBIAS, QW, ACT>), dim3((unsigned)(tr * tc)),
                     dim3(64 * QW), 0, stream, x, R, C, ldx, q_row, s_row, q_colT, s_colT, dbias_part, tc, opt,
                     act_in);
  return hipGetLastError();
}

// One tile launch for a copy set, with the activation ACT fused in.
template <int ACT>
static hipError_t launch_tiles_act(bool row, bool col, bool db, const uint16_t* x, int64_t R, int64_t C,
                                   int64_t ldx, uint8_t* q_row, uint8_t* srow, uint8_t* q_colT, uint8_t* scol,
                                   float* dbias_part, const QuantOpts& opt, const uint16_t* act_in,
                                   int64_t* tiles_r, hipStream_t stream) {
#define MX_Q_LAUNCH(RW, CL, DB) \
  launch_tiles<RW, CL, DB, ACT>(x, R, C, ldx, q_row, srow, q_colT, scol, dbias_part, opt, act_in, tiles_r, stream)
  if (row && col && db) return MX_Q_LAUNCH(true, true, true);
  if (row && col) return MX_Q_LAUNCH(true, true, false);
  if (row && db) return MX_Q_LAUNCH(true, false, true);
  if (row) return MX_Q_LAUNCH(true, false, false);
  if (col && db) return MX_Q_LAUNCH(false, true, true);
  return MX_Q_LAUNCH(false, true, false);
#undef MX_Q_LAUNCH
}

hipError_t launch_quantize(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, uint32_t flags,
                           uint8_t* q_row, void* s_row, uint8_t* q_colT, void* s_colT,
                           float* dbias, float* dbias_part, float* amax, const int32_t* noop,
                           const uint16_t* act_in, hipStream_t stream) {
  const bool row = flags & 1u, col = flags & 2u, db = flags & 4u, want_amax = flags & 8u, packed = flags & 16u;
  const int act = (flags & 32u)    ? ACT_SQRELU
                  : (flags & 64u)  ? DACT_SQRELU
                  : (flags & 128u) ? ACT_GELU
                  : (flags & 256u) ? DACT_GELU
                                   : ACT_NONE;
  const QuantOpts opt{want_amax ? reinterpret_cast<uint32_t*>(amax) : nullptr, noop, packed ? 1 : 0};
  if (want_amax) {   // max starts from 0 (also the amax of an empty tensor)
    hipLaunchKernelGGL(fill_zero_f32_kernel, dim3(1), dim3(256), 0, stream, amax, (int64_t)1, noop);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  uint8_t* srow = static_cast<uint8_t*>(s_row);
  uint8_t* scol = static_cast<uint8_t*>(s_colT);
  const QuantPath path = quantize_path(C, ldx, flags);
  if (path == QP_PACKED_ROW) {
    const int64_t blocks = ((R + PN_ROWS - 1) / PN_ROWS) * ((C + PN_COLS - 1) / PN_COLS);
    if (blocks > 0)
      hipLaunchKernelGGL(quantize_rowwise_packed_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, R, C, ldx,
                         q_row, static_cast<uint32_t*>(s_row), opt);
    return hipGetLastError();
  }
  if (path == QP_FLAT) {
    const int64_t total = R * C;
    const int64_t per_block = FL_ELEMS * (FL_THREADS / 64);
    const int64_t blocks = (total + per_block - 1) / per_block;
    if (blocks > 0)
      hipLaunchKernelGGL(quantize_rowwise_flat_kernel, dim3((unsigned)blocks), dim3(FL_THREADS), 0, stream, x, total,
                         q_row, srow, opt);
    return hipGetLastError();
  }
  int64_t tiles_r = 0;
  hipError_t e;
  if (act == ACT_SQRELU)
    e = launch_tiles_act<ACT_SQRELU>(row, col, db, x, R, C, ldx, q_row, srow, q_colT, scol, dbias_part, opt, act_in,
                                     &tiles_r, stream);
  else if (act == DACT_SQRELU)
    e = launch_tiles_act<DACT_SQRELU>(row, col, db, x, R, C, ldx, q_row, srow, q_colT, scol, dbias_part, opt,
                                      act_in, &tiles_r, stream);
  else if (act == ACT_GELU)
    e = launch_tiles_act<ACT_GELU>(row, col, db, x, R, C, ldx, q_row, srow, q_colT, scol, dbias_part, opt, act_in,
                                   &tiles_r, stream);
  else if (act == DACT_GELU)
    e = launch_tiles_act<DACT_GELU>(row, col, db, x, R, C, ldx, q_row, srow, q_colT, scol, dbias_part, opt,
                                    act_in, &tiles_r, stream);
  else
    e = launch_tiles_act<ACT_NONE>(row, col, db, x, R, C, ldx, q_row, srow, q_colT, scol, dbias_part, opt, act_in,
                                   &tiles_r, stream);
  if (e != hipSuccess) return e;
  if (db && C > 0) {
    const dim3 grid((unsigned)((C + DB_COLS - 1) / DB_COLS));
    if (tiles_r > 0)
      hipLaunchKernelGGL(dbias_reduce_kernel, grid, dim3(DB_COLS * DB_PARTS), 0, stream, dbias_part, tiles_r, C,
                         dbias, noop);
    else
      hipLaunchKernelGGL(fill_zero_f32_kernel, dim3((unsigned)((C + 255) / 256)), dim3(256), 0, stream, dbias, C,
                         noop);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace mx
