// C ABI of the MXFP8 library: host-side validation, then one launch sequence
// on the caller's stream.  See include/mxfp8.h for the contract.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mxfp8.h"
#include "launch.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxDim = int64_t(1) << 40; // keeps every element offset well inside int64
constexpr int64_t kMaxGemmK = int64_t(1) << 22; // a 256-row operand tile stays below 2^31 bytes

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

mxfp8_status hip_status(hipError_t e) {
  if (e == hipSuccess) return MXFP8_OK;
  g_last_hip_error = static_cast<int>(e);
  return MXFP8_ERR_HIP;
}

mxfp8_status check_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld_x, uint32_t flags,
                            const uint8_t* q_row, const void* s_row, const uint8_t* q_colT,
                            const void* s_colT, const float* dbias, const float* amax, const int32_t* noop,
                            const void* act_in, const void* ws, size_t ws_bytes) {
  constexpr uint32_t kActs = MXFP8_ACT_SQRELU | MXFP8_DACT_SQRELU | MXFP8_ACT_GELU | MXFP8_DACT_GELU;
  constexpr uint32_t kDacts = MXFP8_DACT_SQRELU | MXFP8_DACT_GELU;
  if (flags & ~(MXFP8_ROWWISE | MXFP8_COLWISE | MXFP8_DBIAS | MXFP8_AMAX | MXFP8_PACKED_SCALES | kActs))
    return MXFP8_ERR_FLAGS;
  if (!(flags & (MXFP8_ROWWISE | MXFP8_COLWISE))) return MXFP8_ERR_FLAGS;
  if (__builtin_popcount(flags & kActs) > 1) return MXFP8_ERR_FLAGS;   // at most one activation
  if ((flags & MXFP8_AMAX) && !amax) return MXFP8_ERR_NULL;
  if ((flags & MXFP8_AMAX) && !aligned(amax, 4)) return MXFP8_ERR_MISALIGNED;
  if (noop && !aligned(noop, 4)) return MXFP8_ERR_MISALIGNED;
  if (flags & MXFP8_PACKED_SCALES) {
    if ((flags & MXFP8_ROWWISE) && cols % 128) return MXFP8_ERR_SHAPE;
    if ((flags & MXFP8_COLWISE) && rows % 128) return MXFP8_ERR_SHAPE;
  }
  if (rows < 0 || cols < 0 || ld_x < cols) return MXFP8_ERR_SHAPE;
  if (rows > kMaxDim || ld_x > kMaxDim || (rows > 0 && ld_x > kMaxDim / rows)) return MXFP8_ERR_LIMIT;
  if (cols % 32) return MXFP8_ERR_SHAPE;
  if ((flags & MXFP8_COLWISE) && rows % 32) return MXFP8_ERR_SHAPE;
  const bool any = rows > 0 && cols > 0;
  if (any && !x) return MXFP8_ERR_NULL;
  if (any && (flags & MXFP8_ROWWISE) && (!q_row || !s_row)) return MXFP8_ERR_NULL;
  if (any && (flags & MXFP8_COLWISE) && (!q_colT || !s_colT)) return MXFP8_ERR_NULL;
  if (any && (flags & kDacts) && !act_in) return MXFP8_ERR_NULL;
  if ((flags & MXFP8_DBIAS) && cols > 0 && !dbias) return MXFP8_ERR_NULL;
  if (any) {
    if (!aligned(x, 16) || ld_x % 8) return MXFP8_ERR_MISALIGNED;
    if ((flags & kDacts) && !aligned(act_in, 16)) return MXFP8_ERR_MISALIGNED;
    if ((flags & MXFP8_ROWWISE) && !aligned(q_row, 16)) return MXFP8_ERR_MISALIGNED;
    if ((flags & MXFP8_COLWISE) && !aligned(q_colT, 16)) return MXFP8_ERR_MISALIGNED;
    if ((flags & MXFP8_PACKED_SCALES) && (flags & MXFP8_ROWWISE) && !aligned(s_row, 4)) return MXFP8_ERR_MISALIGNED;
    if ((flags & MXFP8_PACKED_SCALES) && (flags & MXFP8_COLWISE) && !aligned(s_colT, 4))
      return MXFP8_ERR_MISALIGNED;
  }
  if ((flags & MXFP8_DBIAS) && cols > 0 && !aligned(dbias, 4)) return MXFP8_ERR_MISALIGNED;
  if (!mx::quantize_grids_fit(rows, cols, ld_x, flags)) return MXFP8_ERR_LIMIT;
  const size_t need = mxfp8_quantize_workspace_bytes(rows, cols, flags);
  if (need > 0) {
    if (!ws || ws_bytes < need) return MXFP8_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return MXFP8_ERR_MISALIGNED;
  }
  return MXFP8_OK;
}

// c / ldc: the output and its row stride in elements of out_bytes bytes (2 for
// BF16, 1 for MXFP8 codes); rows must start 16-byte aligned.
mxfp8_status check_gemm_common(const uint8_t* a, const uint32_t* ap, const uint8_t* b, const uint32_t* bp,
                               const void* c, int64_t ldc, int64_t M, int64_t N, int64_t K, int out_bytes = 2) {
  if (M < 0 || N < 0 || K < 0) return MXFP8_ERR_SHAPE;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim || ldc > kMaxDim) return MXFP8_ERR_LIMIT;
  if (K > kMaxGemmK) return MXFP8_ERR_LIMIT;
  if (N % 32 || K % 128 || ldc < N) return MXFP8_ERR_SHAPE;
  if (M == 0 || N == 0) return MXFP8_OK;
  if (!c) return MXFP8_ERR_NULL;
  if (K > 0 && (!a || !ap || !b || !bp)) return MXFP8_ERR_NULL;
  if (!aligned(c, 16) || (ldc * out_bytes) % 16) return MXFP8_ERR_MISALIGNED;
  if (K > 0 && (!aligned(a, 16) || !aligned(b, 16) || !aligned(ap, 4) || !aligned(bp, 4)))
    return MXFP8_ERR_MISALIGNED;
  return MXFP8_OK;
}

// GEMM options: known bits only, at most one of accumulate / relu^2 / GELU / SwiGLU.
bool gemm_flags_ok(uint32_t flags) {
  constexpr uint32_t kAll = MXFP8_GEMM_ACCUMULATE | MXFP8_GEMM_SQRELU | MXFP8_GEMM_GELU | MXFP8_GEMM_SWIGLU;
  return !(flags & ~kAll) && __builtin_popcount(flags) <= 1;
}
int gemm_epilogue(uint32_t flags) {
  return (flags & MXFP8_GEMM_SQRELU) ? 1 : (flags & MXFP8_GEMM_GELU) ? 2 : (flags & MXFP8_GEMM_SWIGLU) ? 3 : 0;
}
// SwiGLU reads 2N rows of B: their scale-word offsets (8N bytes) stay below 2^31.
constexpr int64_t kMaxSwigluN = int64_t(1) << 27;

// Every GEMM entry point: flags, shapes, pointers, grid; then one launch.
// Dense when offsets == nullptr and G == 0.  with_bias: the bias entry points
// (a bias is required, accumulate is rejected).  mxo.q set: the MXFP8-output
// entry points (c unused; the bias is optional, accumulate is rejected).
mxfp8_status gemm_entry(const uint8_t* a, const uint32_t* a_packed, const uint8_t* b, const uint32_t* b_packed,
                        const int32_t* offsets, int32_t G, const void* bias, bool with_bias, void* c, int64_t ldc,
                        int64_t M, int64_t N, int64_t K, uint32_t flags, void* stream,
                        mx::MxOut mxo = mx::MxOut{nullptr, 0, nullptr}, bool mx_out = false) {
  if (!gemm_flags_ok(flags)) return MXFP8_ERR_FLAGS;
  if ((with_bias || mx_out) && (flags & MXFP8_GEMM_ACCUMULATE)) return MXFP8_ERR_FLAGS;
  const bool grouped = G > 0;
  const mxfp8_status st = mx_out ? check_gemm_common(a, a_packed, b, b_packed, mxo.q, mxo.ldq, M, N, K, 1)
                                 : check_gemm_common(a, a_packed, b, b_packed, c, ldc, M, N, K);
  if (st != MXFP8_OK) return st;
  if (mx_out && N % 128) return MXFP8_ERR_SHAPE;   // whole packed scale words per row
  const bool swiglu = (flags & MXFP8_GEMM_SWIGLU) != 0;
  if (swiglu && N > kMaxSwigluN) return MXFP8_ERR_LIMIT;
  if (M == 0 || N == 0) return MXFP8_OK;
  if (grouped && !offsets) return MXFP8_ERR_NULL;
  if (grouped && !aligned(offsets, 4)) return MXFP8_ERR_MISALIGNED;
  if (with_bias && !bias) return MXFP8_ERR_NULL;
  if (with_bias && !aligned(bias, 16)) return MXFP8_ERR_MISALIGNED;
  if (mx_out && !mxo.qp) return MXFP8_ERR_NULL;
  if (mx_out && !aligned(mxo.qp, 4)) return MXFP8_ERR_MISALIGNED;
  if (!mx::gemm_grid_fits(M, N, G, grouped, swiglu)) return MXFP8_ERR_LIMIT;
  return hip_status(mx::launch_gemm(a, a_packed, b, b_packed, static_cast<uint16_t*>(c), ldc, M, N, K,
                                    grouped ? offsets : nullptr, G, (flags & MXFP8_GEMM_ACCUMULATE) != 0,
                                    gemm_epilogue(flags), with_bias ? static_cast<const uint16_t*>(bias) : nullptr,
                                    mx_out ? mxo : mx::MxOut{nullptr, 0, nullptr}, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

const char* mxfp8_status_string(mxfp8_status s) {
  switch (s) {
    case MXFP8_OK: return "MXFP8_OK";
    case MXFP8_ERR_NULL: return "MXFP8_ERR_NULL: a required pointer is NULL";
    case MXFP8_ERR_SHAPE: return "MXFP8_ERR_SHAPE: negative size or divisibility rule violated";
    case MXFP8_ERR_MISALIGNED: return "MXFP8_ERR_MISALIGNED: pointer or leading dimension misaligned";
    case MXFP8_ERR_FLAGS: return "MXFP8_ERR_FLAGS: unknown flag bits or no copy requested";
    case MXFP8_ERR_WORKSPACE: return "MXFP8_ERR_WORKSPACE: workspace missing or too small";
    case MXFP8_ERR_HIP: return "MXFP8_ERR_HIP: the HIP runtime reported an error";
    case MXFP8_ERR_LIMIT: return "MXFP8_ERR_LIMIT: problem too large for one launch grid";
  }
  return "unknown mxfp8_status";
}

int mxfp8_last_hip_error(void) { return g_last_hip_error; }

size_t mxfp8_quantize_workspace_bytes(int64_t rows, int64_t cols, uint32_t flags) {
  if (!(flags & MXFP8_DBIAS) || rows <= 0 || cols <= 0) return 0;
  return (size_t)mx::quantize_row_tiles(rows) * (size_t)cols * sizeof(float);
}

mxfp8_status mxfp8_quantize_ex(const void* x, int64_t rows, int64_t cols, int64_t ld_x, uint32_t flags,
                               uint8_t* q_row, void* s_row, uint8_t* q_colT, void* s_colT, float* dbias,
                               float* amax, const int32_t* noop, const void* act_in, void* workspace,
                               size_t workspace_bytes, void* stream) {
  const mxfp8_status st = check_quantize(x, rows, cols, ld_x, flags, q_row, s_row, q_colT, s_colT, dbias, amax,
                                         noop, act_in, workspace, workspace_bytes);
  if (st != MXFP8_OK) return st;
  const bool empty = rows == 0 || cols == 0;
  if (empty && !(flags & MXFP8_AMAX) && !((flags & MXFP8_DBIAS) && cols > 0)) return MXFP8_OK;
  return hip_status(mx::launch_quantize(static_cast<const uint16_t*>(x), rows, cols, ld_x, flags, q_row, s_row,
                                        q_colT, s_colT, dbias, static_cast<float*>(workspace), amax, noop,
                                        static_cast<const uint16_t*>(act_in), static_cast<hipStream_t>(stream)));
}

mxfp8_status mxfp8_quantize_ex_noalloc(const void* x, int64_t rows, int64_t cols, int64_t ld_x, uint32_t flags,
                                       uint8_t* q_row, void* s_row, uint8_t* q_colT, void* s_colT, float* dbias,
                                       float* amax, const int32_t* noop, const void* act_in, void* stream) {
  static_assert(MXFP8_NOALLOC_SCRATCH_BYTES == mx::kNoallocScratchBytes, "scratch size");
  const size_t need = mxfp8_quantize_workspace_bytes(rows, cols, flags);
  // every other rule as mxfp8_quantize_ex (a stand-in workspace of the right
  // size passes its workspace checks), then the scratch limit
  void* const stand_in = need ? reinterpret_cast<void*>(uintptr_t(256)) : nullptr;
  const mxfp8_status st = check_quantize(x, rows, cols, ld_x, flags, q_row, s_row, q_colT, s_colT, dbias, amax,
                                         noop, act_in, stand_in, need);
  if (st != MXFP8_OK) return st;
  if (need > MXFP8_NOALLOC_SCRATCH_BYTES) return MXFP8_ERR_WORKSPACE;
  const bool empty = rows == 0 || cols == 0;
  if (empty && !(flags & MXFP8_AMAX) && !((flags & MXFP8_DBIAS) && cols > 0)) return MXFP8_OK;
  float* ws = nullptr;
  if (need) {
    const hipError_t e = mx::noalloc_scratch(static_cast<hipStream_t>(stream), &ws);
    if (e != hipSuccess) return hip_status(e);
  }
  return hip_status(mx::launch_quantize(static_cast<const uint16_t*>(x), rows, cols, ld_x, flags, q_row, s_row,
                                        q_colT, s_colT, dbias, ws, amax, noop,
                                        static_cast<const uint16_t*>(act_in), static_cast<hipStream_t>(stream)));
}

mxfp8_status mxfp8_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld_x, uint32_t flags,
                            uint8_t* q_row, uint8_t* s_row, uint8_t* q_colT, uint8_t* s_colT, float* dbias,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (flags & ~(MXFP8_ROWWISE | MXFP8_COLWISE | MXFP8_DBIAS)) return MXFP8_ERR_FLAGS;
  return mxfp8_quantize_ex(x, rows, cols, ld_x, flags, q_row, s_row, q_colT, s_colT, dbias, nullptr, nullptr,
                           nullptr, workspace, workspace_bytes, stream);
}

size_t mxfp8_packed_scale_bytes(int64_t dim, int64_t k) {
  if (dim <= 0 || k <= 0) return 0;
  return (size_t)(k / 128) * (size_t)dim * 4u;
}

mxfp8_status mxfp8_pack_scales(const uint8_t* s, int64_t dim, int64_t k, int64_t ld_s, uint32_t* packed,
                               void* stream) {
  if (dim < 0 || k < 0 || k % 128 || ld_s < k / 32) return MXFP8_ERR_SHAPE;
  if (dim > kMaxDim || ld_s > kMaxDim || k > kMaxDim) return MXFP8_ERR_LIMIT;
  if (dim == 0 || k == 0) return MXFP8_OK;
  if (!s || !packed) return MXFP8_ERR_NULL;
  if (!aligned(s, 4) || ld_s % 4 || !aligned(packed, 4)) return MXFP8_ERR_MISALIGNED;
  if (!mx::pack_scales_grid_fits(dim, k)) return MXFP8_ERR_LIMIT;
  return hip_status(mx::launch_pack_scales(s, dim, k, ld_s, packed, static_cast<hipStream_t>(stream)));
}

mxfp8_status mxfp8_gemm_ex(const uint8_t* a, const uint32_t* a_packed, const uint8_t* b, const uint32_t* b_packed,
                           void* c, int64_t ldc, int64_t M, int64_t N, int64_t K, uint32_t flags, void* stream) {
  return gemm_entry(a, a_packed, b, b_packed, nullptr, 0, nullptr, false, c, ldc, M, N, K, flags, stream);
}

mxfp8_status mxfp8_gemm(const uint8_t* a, const uint32_t* a_packed, const uint8_t* b, const uint32_t* b_packed,
                        void* c, int64_t ldc, int64_t M, int64_t N, int64_t K, void* stream) {
  return mxfp8_gemm_ex(a, a_packed, b, b_packed, c, ldc, M, N, K, 0u, stream);
}

mxfp8_status mxfp8_gemm_bias(const uint8_t* a, const uint32_t* a_packed, const uint8_t* b, const uint32_t* b_packed,
                             const void* bias, void* c, int64_t ldc, int64_t M, int64_t N, int64_t K, uint32_t flags,
                             void* stream) {
  return gemm_entry(a, a_packed, b, b_packed, nullptr, 0, bias, true, c, ldc, M, N, K, flags, stream);
}

mxfp8_status mxfp8_grouped_gemm_ex(const uint8_t* a, const uint32_t* a_packed, const uint8_t* b,
                                   const uint32_t* b_packed, const int32_t* offsets, int32_t G, void* c, int64_t ldc,
                                   int64_t M_total, int64_t N, int64_t K, uint32_t flags, void* stream) {
  if (G < 1 || G > 65536) return gemm_flags_ok(flags) ? MXFP8_ERR_SHAPE : MXFP8_ERR_FLAGS;
  return gemm_entry(a, a_packed, b, b_packed, offsets, G, nullptr, false, c, ldc, M_total, N, K, flags, stream);
}

mxfp8_status mxfp8_grouped_gemm(const uint8_t* a, const uint32_t* a_packed, const uint8_t* b,
                                const uint32_t* b_packed, const int32_t* offsets, int32_t G, void* c, int64_t ldc,
                                int64_t M_total, int64_t N, int64_t K, void* stream) {
  return mxfp8_grouped_gemm_ex(a, a_packed, b, b_packed, offsets, G, c, ldc, M_total, N, K, 0u, stream);
}

mxfp8_status mxfp8_grouped_gemm_bias(const uint8_t* a, const uint32_t* a_packed, const uint8_t* b,
                                     const uint32_t* b_packed, const int32_t* offsets, int32_t G, const void* bias,
                                     void* c, int64_t ldc, int64_t M_total, int64_t N, int64_t K, uint32_t flags,
                                     void* stream) {
  if (G < 1 || G > 65536) return gemm_flags_ok(flags) ? MXFP8_ERR_SHAPE : MXFP8_ERR_FLAGS;
  return gemm_entry(a, a_packed, b, b_packed, offsets, G, bias, true, c, ldc, M_total, N, K, flags, stream);
}

mxfp8_status mxfp8_gemm_mxfp8_out(const uint8_t* a, const uint32_t* a_packed, const uint8_t* b,
                                  const uint32_t* b_packed, const void* bias, uint8_t* q_out, int64_t ldq,
                                  uint32_t* q_out_packed, int64_t M, int64_t N, int64_t K, uint32_t flags,
                                  void* stream) {
  return gemm_entry(a, a_packed, b, b_packed, nullptr, 0, bias, bias != nullptr, nullptr, 0, M, N, K, flags, stream,
                    mx::MxOut{q_out, ldq, q_out_packed}, true);
}

mxfp8_status mxfp8_grouped_gemm_mxfp8_out(const uint8_t* a, const uint32_t* a_packed, const uint8_t* b,
                                          const uint32_t* b_packed, const int32_t* offsets, int32_t G,
                                          const void* bias, uint8_t* q_out, int64_t ldq, uint32_t* q_out_packed,
                                          int64_t M_total, int64_t N, int64_t K, uint32_t flags, void* stream) {
  if (G < 1 || G > 65536) return gemm_flags_ok(flags) ? MXFP8_ERR_SHAPE : MXFP8_ERR_FLAGS;
  return gemm_entry(a, a_packed, b, b_packed, offsets, G, bias, bias != nullptr, nullptr, 0, M_total, N, K, flags,
                    stream, mx::MxOut{q_out, ldq, q_out_packed}, true);
}

}  // extern "C"
