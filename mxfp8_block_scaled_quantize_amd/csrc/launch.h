// Internal launchers (host side) of the gfx950 kernels.  The public C ABI in
// include/mxfp8.h validates every argument before calling these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

int64_t quantize_row_tiles(int64_t R);
int64_t quantize_col_tiles(int64_t C);

// An AQL dispatch packet holds the grid size in work-items as a 32-bit
// field: a launch of `a * b` workgroups of `threads` work-items fits when the
// product is at most 2^32 - 1 (checked without overflow; a or b == 0 fits).
constexpr int64_t kMaxWorkItems = 0xFFFFFFFFll;
inline bool grid_fits(int64_t a, int64_t b, int64_t threads) {
  if (a <= 0 || b <= 0) return true;
  return a <= kMaxWorkItems / threads / b;
}

// Whether every launch of mxfp8_quantize_ex with these sizes and flags fits
// in one grid (R, C >= 0, R * C <= 2^40).
bool quantize_grids_fit(int64_t R, int64_t C, int64_t ldx, uint32_t flags);

// flags: rowwise 1, colwise 2, dbias 4, amax 8, packed scales 16, squared-ReLU
// activation 32, its backward 64, GELU 128, its backward 256 (act_in: the
// activation's input, same shape and leading dimension as x).  noop may be
// null (always run).
hipError_t launch_quantize(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, uint32_t flags,
                           uint8_t* q_row, void* s_row, uint8_t* q_colT, void* s_colT,
                           float* dbias, float* dbias_part, float* amax, const int32_t* noop,
                           const uint16_t* act_in, hipStream_t stream);

// Bytes of the static device scratch behind the allocation-free quantize
// entry point (equal to MXFP8_NOALLOC_SCRATCH_BYTES of the C ABI).
constexpr size_t kNoallocScratchBytes = size_t(8) << 20;
// Device address of that scratch on the device of `stream` (looked up once per
// device with hipGetSymbolAddress, that device current).
hipError_t noalloc_scratch(hipStream_t stream, float** out);

hipError_t launch_pack_scales(const uint8_t* s, int64_t dim, int64_t k, int64_t ld_s, uint32_t* packed,
                              hipStream_t stream);
bool pack_scales_grid_fits(int64_t dim, int64_t k);

// MXFP8 output of the GEMM (rowwise copy): codes q [M][ldq] bytes and packed
// scale words qp [N/128][M]; q == nullptr selects the BF16 output c.
struct MxOut {
  uint8_t* q;
  int64_t ldq;
  uint32_t* qp;
};

// Dense (offsets == nullptr) or grouped GEMM; accumulate adds the product to C; epilogue 1 writes
// relu(product)^2, 2 writes GELU(product), 3 writes SiLU(gate) * up with B holding 2N rows (gate rows,
// then up rows; per group when grouped) and N the output columns (none together with accumulate).
// bias (optional, BF16, one value per B row, per group when grouped) is added to the fp32 sum before
// the epilogue (not together with accumulate).  mxo.q set: the output is written as MXFP8 (N % 128 == 0,
// not together with accumulate) instead of to c.
hipError_t launch_gemm(const uint8_t* a, const uint32_t* ap, const uint8_t* b, const uint32_t* bp,
                       uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K,
                       const int32_t* offsets, int32_t G, bool accumulate, int epilogue, const uint16_t* bias,
                       MxOut mxo, hipStream_t stream);
bool gemm_grid_fits(int64_t M, int64_t N, int32_t G, bool grouped, bool swiglu);

}  // namespace mx
