/*
 * mxfp8.h - C ABI of the MI355X (gfx950) MXFP8 library.
 *
 * MXFP8 block-scaled quantization (BF16 -> E4M3 codes + one E8M0 scale per
 * 32 consecutive elements along the reduction direction, rowwise and
 * columnwise, optional fused dbias) and the block-scaled MXFP8 GEMM
 * (fp32 accumulation, BF16 output or its rowwise MXFP8 copy; dense and
 * ragged grouped; optional accumulate, bias and activation epilogues).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers on the device that owns
 *    `stream`.  The caller allocates and owns every buffer (inputs, outputs,
 *    workspace); the library never allocates, frees or synchronises, and
 *    never reads device data on the host.
 *  - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *    Work is enqueued asynchronously; a returned MXFP8_OK means "validated
 *    and launched", not "finished".
 *  - Sizes are int64_t element counts; matrices are row-major.
 *  - Arguments are validated on the host BEFORE anything is launched; an
 *    invalid call returns an error code and enqueues nothing.  Unsupported
 *    requests are rejected, never silently changed.  There is no fallback
 *    path.  Launch failures return MXFP8_ERR_HIP (the HIP error code is
 *    available from mxfp8_last_hip_error()).
 *  - Empty problems (a zero dimension) are valid no-ops, except that
 *    outputs that are mathematically defined (a dbias over zero rows, a GEMM
 *    with K = 0) are written: zeros, or the epilogue of the bias for a GEMM
 *    with a bias.
 *
 * Numerics (OCP MX reading of the pages: the block size, E8M0 scales, E4M3
 * data and the rowwise / columnwise / dbias options come from the page
 * "[Common] Experimental CuTeDSL MXFP8 backends in C++ via TVM-FFI",
 * config-struct review and Greptile summary; the scale rule is OCP MX):
 *  - block amax over 32 BF16 values; shared exponent X = floor(log2 amax) - 8
 *    clamped to [-127, 127]; scale byte = X + 127 (0 for an all-zero block);
 *  - code = E4M3(x * 2^-X) rounded to nearest even, saturated to +-448, sign
 *    of zero kept;
 *  - dequantized value = E4M3 value * 2^(byte - 127).
 */
#ifndef MXFP8_H
#define MXFP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mxfp8_status {
    MXFP8_OK = 0,
    MXFP8_ERR_NULL = 1,        /* a required pointer is NULL                       */
    MXFP8_ERR_SHAPE = 2,       /* negative size or a divisibility rule violated     */
    MXFP8_ERR_MISALIGNED = 3,  /* pointer / leading dimension alignment violated    */
    MXFP8_ERR_FLAGS = 4,       /* unknown flag bits or no copy requested            */
    MXFP8_ERR_WORKSPACE = 5,   /* DBIAS workspace missing or too small              */
    MXFP8_ERR_HIP = 6,         /* the HIP runtime reported an error at launch       */
    MXFP8_ERR_LIMIT = 7        /* a size exceeds what one launch grid can cover:
                                * a kernel of the call would need more than
                                * 2^32 - 1 work-items (the 32-bit grid field of
                                * an AQL dispatch packet), a dimension or
                                * rows * ld exceeds 2^40, or GEMM K exceeds 2^22 */
} mxfp8_status;

/* Flags of mxfp8_quantize (the rowwise / colwise / with_dbias options of the
 * quantization config in "[Common] Experimental CuTeDSL MXFP8 backends in C++
 * via TVM-FFI", review of the config key). */
#define MXFP8_ROWWISE 1u /* blocks along rows:    q_row[rows][cols], s_row[rows][cols/32]    */
#define MXFP8_COLWISE 2u /* blocks along columns, stored transposed:
                            q_colT[cols][rows], s_colT[cols][rows/32]                       */
#define MXFP8_DBIAS 4u   /* dbias[cols] = fp32 column sums of the BF16 input                 */

/* Human-readable name of a status code (static storage). */
const char *mxfp8_status_string(mxfp8_status s);

/* HIP error code (hipError_t as int) of the last MXFP8_ERR_HIP returned on
 * the calling thread; 0 if none. */
int mxfp8_last_hip_error(void);

/* ------------------------------------------------------------------------
 * Quantization
 *
 * Defining passage: MXFP8 quantization with rowwise and/or columnwise output
 * and an optional fused dbias whose partial sums go to a caller workspace and
 * are then reduced ("[Common] Experimental CuTeDSL MXFP8 backends in C++ via
 * TVM-FFI", Greptile summary and config struct); columnwise storage is the
 * materialised transpose ("Experimental FlyDSL GEMM backend for TE PyTorch
 * (BF16/FP16/FP32/FP8/MXFP8)", commit notes on TN/NN/NT storage selection).
 * ------------------------------------------------------------------------ */

/* Extra flags of mxfp8_quantize_ex (the with_amax option and the swizzled
 * scale-output option of the quantization config in "[Common] Experimental
 * CuTeDSL MXFP8 backends in C++ via TVM-FFI", review of the config key; the
 * packed layout is the one mxfp8_pack_scales writes, so the GEMM can consume
 * the quantizer's scales without a separate packing launch). */
#define MXFP8_AMAX 8u            /* amax[0] = max |x| over the tensor (fp32)   */
#define MXFP8_PACKED_SCALES 16u  /* s_row / s_colT in the packed word layout:
                                    s_row  uint32 [cols/128][rows] (cols % 128 == 0),
                                    s_colT uint32 [rows/128][cols] (rows % 128 == 0) */
/* Activation fused into mxfp8_quantize_ex (the with_act / with_dact /
 * activation keys of the quantization config, "[Common] Experimental CuTeDSL
 * MXFP8 backends in C++ via TVM-FFI", config key listing; squared ReLU is the
 * FC1 activation of "gemm(cutedsl): add standalone Lightning W4A16 grouped
 * GEMM - #811", section "API and compatibility impact").  The value that is
 * quantized (and summed by DBIAS, and measured by AMAX) is then fp32:       */
#define MXFP8_ACT_SQRELU 32u     /* relu(x)^2                                  */
#define MXFP8_DACT_SQRELU 64u    /* x * 2 relu(act_in): backward of relu(a)^2,
                                    x = incoming gradient, act_in = a           */
/* GELU, the activation that the config key's activation field names besides
 * the ReLU family and that the GEMM review finds silently dropped from the
 * FlyDSL path ("Experimental FlyDSL GEMM backend for TE PyTorch
 * (BF16/FP16/FP32/FP8/MXFP8)", review of the gelu / grad epilogue
 * arguments).  The pages fix no formula; this library uses the exact form
 * GELU(a) = a * Phi(a) = 0.5 a erfc(-a / sqrt 2), evaluated in fp32:       */
#define MXFP8_ACT_GELU 128u      /* GELU(x)                                    */
#define MXFP8_DACT_GELU 256u     /* x * GELU'(act_in), GELU'(a) = Phi(a) +
                                    a phi(a) (phi the standard normal density) */

/* Bytes of workspace mxfp8_quantize needs for `flags` at this shape (0 when
 * DBIAS is not requested). */
size_t mxfp8_quantize_workspace_bytes(int64_t rows, int64_t cols, uint32_t flags);

/*
 * x       BF16 input [rows][ld_x] (row-major, only the first `cols` of each
 *         row are read).  16-byte aligned; ld_x >= cols and ld_x % 8 == 0.
 * rows    >= 0; a multiple of 32 when MXFP8_COLWISE is set.
 * cols    >= 0; a multiple of 32.
 * flags   a non-empty combination of MXFP8_ROWWISE / MXFP8_COLWISE, plus
 *         MXFP8_DBIAS optionally.
 * q_row   ROWWISE: E4M3 codes [rows][cols], 16-byte aligned.   Else ignored.
 * s_row   ROWWISE: E8M0 scales [rows][cols/32].                Else ignored.
 * q_colT  COLWISE: E4M3 codes [cols][rows], 16-byte aligned.   Else ignored.
 * s_colT  COLWISE: E8M0 scales [cols][rows/32].                Else ignored.
 * dbias   DBIAS: fp32 [cols], 4-byte aligned.                  Else ignored.
 * workspace, workspace_bytes
 *         DBIAS: device scratch of at least
 *         mxfp8_quantize_workspace_bytes(rows, cols, flags) bytes, 16-byte
 *         aligned, used for per-row-tile partial sums (the result is
 *         deterministic: no atomics).  Else ignored.
 * Errors: NULL (a required pointer is NULL), SHAPE, MISALIGNED, FLAGS,
 *         WORKSPACE, LIMIT, HIP.  Inputs with NaN/Inf are outside the
 *         contract (the codes are then unspecified; nothing faults).
 */
mxfp8_status mxfp8_quantize(const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                            uint32_t flags,
                            uint8_t *q_row, uint8_t *s_row,
                            uint8_t *q_colT, uint8_t *s_colT,
                            float *dbias,
                            void *workspace, size_t workspace_bytes,
                            void *stream);

/*
 * mxfp8_quantize with the fused extras.  Defining passage: the with_amax,
 * swizzled and noop options of the quantization config and the device-side
 * noop check, which must also cover the dbias reduction ("[Common]
 * Experimental CuTeDSL MXFP8 backends in C++ via TVM-FFI", review of the
 * config key, commit "Perform noop tensor check on device", Greptile summary
 * on the noop + dbias interaction).
 * flags   as mxfp8_quantize, plus MXFP8_AMAX, MXFP8_PACKED_SCALES and at most
 *         one of MXFP8_ACT_SQRELU / MXFP8_DACT_SQRELU / MXFP8_ACT_GELU /
 *         MXFP8_DACT_GELU.  With an activation the quantized value v is the
 *         fp32 result of the activation (for squared ReLU each product of two
 *         BF16 values is exact in fp32; GELU is evaluated in fp32 from the
 *         normal tail exp(-t^2/2) Q(t) with a fitted rational Q, within
 *         (8 + 3 a^2) fp32 ulp of GELU(a) and 8 ulp of |Phi(a)| + |a phi(a)|
 *         for its derivative); its block scale follows the same
 *         rule (exponent of the block amax - 8), codes are RNE of
 *         v / 2^(scale - 127) saturated to +-448.
 * s_row, s_colT  byte scales as in mxfp8_quantize, or (PACKED_SCALES) uint32
 *         words in the mxfp8_pack_scales layout, 4-byte aligned.
 * amax    AMAX: fp32 [1], 4-byte aligned: the largest |v| of the tensor (v = x,
 *         or the activation's output; exact; 0 for an empty tensor).  Else
 *         ignored.
 * noop    optional DEVICE int32 flag, 4-byte aligned.  When non-NULL and
 *         nonzero at the time the work executes, nothing is written (codes,
 *         scales, dbias and amax keep their old contents).  NULL: always run.
 * act_in  DACT_SQRELU / DACT_GELU: BF16 [rows][ld_x], the forward
 *         activation's input, same layout as x, 16-byte aligned.  Else
 *         ignored.
 * Errors: as mxfp8_quantize; SHAPE also for PACKED_SCALES with cols (rowwise)
 *         or rows (columnwise) not a multiple of 128; NULL for AMAX without
 *         amax or a DACT flag without act_in; FLAGS for two activations at
 *         once.  Activation results that overflow fp32 or fall below its
 *         normal range are outside the contract.  mxfp8_quantize(...) rejects
 *         the extra flags (FLAGS).
 */
mxfp8_status mxfp8_quantize_ex(const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                               uint32_t flags,
                               uint8_t *q_row, void *s_row,
                               uint8_t *q_colT, void *s_colT,
                               float *dbias, float *amax, const int32_t *noop,
                               const void *act_in,
                               void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * mxfp8_quantize_ex without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  The dbias partial sums go to a static device
 * buffer of MXFP8_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it
 * runs on until the process ends; nothing is allocated or freed by the call.
 * Arguments, results and errors are those of mxfp8_quantize_ex without
 * workspace / workspace_bytes, plus:
 *  - MXFP8_ERR_WORKSPACE when DBIAS needs more partial-sum space than the
 *    buffer holds, i.e. mxfp8_quantize_workspace_bytes(rows, cols, flags) >
 *    MXFP8_NOALLOC_SCRATCH_BYTES (e.g. 8 MiB covers 16384 rows x 16384
 *    columns); nothing is launched then;
 *  - MXFP8_ERR_HIP when the buffer's device address cannot be obtained (it is
 *    looked up once per device, on the first call that needs it there).
 * Every call on one GPU shares that GPU's buffer and leaves its contents
 * behind: calls that can overlap on one GPU (e.g. on two streams) race and
 * must be ordered by the caller.  Every partial sum is written before it is
 * read, so nothing needs clearing between calls.
 */
#define MXFP8_NOALLOC_SCRATCH_BYTES 8388608u
mxfp8_status mxfp8_quantize_ex_noalloc(const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                                       uint32_t flags,
                                       uint8_t *q_row, void *s_row,
                                       uint8_t *q_colT, void *s_colT,
                                       float *dbias, float *amax, const int32_t *noop,
                                       const void *act_in,
                                       void *stream);

/* ------------------------------------------------------------------------
 * Scale packing
 *
 * Defining passage: one fused launch per GEMM operand converts the E8M0
 * scales into the MFMA-ready [K/128, dim] packed word layout, from rowwise
 * or columnwise scale storage with its actual strides ("Experimental FlyDSL
 * GEMM backend for TE PyTorch (BF16/FP16/FP32/FP8/MXFP8)", commit notes on
 * the fused scale-pack kernel).
 *
 * Layout: packed is uint32 [k/128][dim]; byte j (little-endian) of word
 * (t, r) is the scale of K-block 4t + j of row r, i.e. of
 * K = [128t + 32j, 128t + 32j + 32).
 * ------------------------------------------------------------------------ */

/* Bytes of the packed layout for a [dim][k] operand: 4 * (k/128) * dim. */
size_t mxfp8_packed_scale_bytes(int64_t dim, int64_t k);

/*
 * s       E8M0 scales [dim][ld_s] bytes (K-block index fastest), 4-byte
 *         aligned; ld_s >= k/32 and ld_s % 4 == 0.
 * dim     >= 0 rows of the operand (M for A, N -- or G*N stacked -- for B).
 * k       >= 0, a multiple of 128.
 * packed  uint32 [k/128][dim], 4-byte aligned; must not overlap s.
 * Errors: NULL, SHAPE, MISALIGNED, LIMIT, HIP.
 */
mxfp8_status mxfp8_pack_scales(const uint8_t *s, int64_t dim, int64_t k, int64_t ld_s,
                               uint32_t *packed, void *stream);

/* ------------------------------------------------------------------------
 * Block-scaled GEMM (TN)
 *
 * Defining passage: MXFP8 x MXFP8 -> BF16 on the gfx950 scaled FP8 MFMA,
 * where the FlyDSL backend supports only alpha = 1 and beta = 0 (no
 * accumulate, bias or output quantization), TN layout with both operands
 * K-major ("Experimental FlyDSL GEMM backend for TE PyTorch
 * (BF16/FP16/FP32/FP8/MXFP8)", Summary and the review of the epilogue
 * validation).  mxfp8_gemm is that operation; the _ex, _bias and _mxfp8_out
 * entry points below add the options the review finds missing.
 *
 *   C[m][n] = bf16_rne( sum_k dq(A)[m][k] * dq(B)[n][k] ),  fp32 accumulation.
 * ------------------------------------------------------------------------ */

/*
 * a         E4M3 codes A [M][K] (row-major, K contiguous), 16-byte aligned.
 * a_packed  packed scales of A, uint32 [K/128][M] (mxfp8_pack_scales layout).
 * b         E4M3 codes B [N][K], 16-byte aligned.
 * b_packed  packed scales of B, uint32 [K/128][N].
 * c         BF16 output [M][ldc], 16-byte aligned; ldc >= N, ldc % 8 == 0.
 * M >= 0; N >= 0 and N % 32 == 0; K >= 0, K % 128 == 0 and K <= 2^22.
 * K == 0 writes zeros.  The output must not overlap the inputs.
 * Overflow beyond BF16 range gives +-inf, like the fp32->BF16 rounding.
 * Errors: NULL, SHAPE, MISALIGNED, LIMIT, HIP.
 */
mxfp8_status mxfp8_gemm(const uint8_t *a, const uint32_t *a_packed,
                        const uint8_t *b, const uint32_t *b_packed,
                        void *c, int64_t ldc,
                        int64_t M, int64_t N, int64_t K, void *stream);

/* Flags of mxfp8_gemm_ex / mxfp8_grouped_gemm_ex (at most one of them). */
#define MXFP8_GEMM_ACCUMULATE 1u /* C = bf16_rne( float(C) + sum_k dq(A) dq(B) ): beta = 1 */
#define MXFP8_GEMM_SQRELU 2u     /* C = bf16_rne( relu(acc)^2 ), acc = the fp32 sum and
                                    relu(acc)^2 formed in fp32: the squared-ReLU
                                    epilogue of an MLP's first projection */
#define MXFP8_GEMM_GELU 4u       /* C = bf16_rne( GELU(acc) ), GELU in fp32 as for
                                    MXFP8_ACT_GELU: the fused GELU epilogue that the
                                    FlyDSL review asks for ("Experimental FlyDSL GEMM
                                    backend for TE PyTorch (BF16/FP16/FP32/FP8/MXFP8)",
                                    review of the gelu / grad arguments) */
#define MXFP8_GEMM_SWIGLU 8u     /* C[m][n] = bf16_rne( SiLU(g) * u ), g = the fp32 sum
                                    over B row n, u = over B row N + n, SiLU(z) =
                                    z / (1 + exp(-z)) in fp32: B holds 2N rows (the
                                    gate projection, then the up projection; per
                                    expert for the grouped GEMM), N is the output
                                    width.  The block-scale matmul and MoE grouped
                                    forward with a SwiGLU epilogue of "frost(gemm):
                                    Add Rubin kernel pipelines" (its test and
                                    benchmark list) */

/*
 * mxfp8_gemm with options.  Defining passage: the accumulate option that the
 * FlyDSL backend still rejects (wgrad accumulation into an existing gradient,
 * "Experimental FlyDSL GEMM backend for TE PyTorch (BF16/FP16/FP32/FP8/MXFP8)",
 * review of the epilogue validation and of the fallback exceptions).
 * flags   0, MXFP8_GEMM_ACCUMULATE, MXFP8_GEMM_SQRELU, MXFP8_GEMM_GELU or
 *         MXFP8_GEMM_SWIGLU.  With ACCUMULATE, C
 *         is read and the sum is rounded once (fp32 accumulator + the old BF16
 *         value, then BF16 round-to-nearest-even); K == 0 leaves C unchanged.
 *         With SQRELU the fp32 accumulator goes through relu(v)^2 before the
 *         BF16 rounding (the FC1 "squared_relu" epilogue of "gemm(cutedsl):
 *         add standalone Lightning W4A16 grouped GEMM - #811", section "API
 *         and compatibility impact"); K == 0 writes zeros.  GELU likewise
 *         (GELU(0) = 0).  With SWIGLU, b is [2N][K] and b_packed
 *         [K/128][2N] (rows 0..N-1 the gate, N..2N-1 the up projection), C
 *         is [M][N]; K == 0 writes zeros; N > 2^27 -> LIMIT.
 * Other arguments and errors as mxfp8_gemm; unknown flag bits or two flags
 * -> FLAGS.
 * mxfp8_gemm(...) is mxfp8_gemm_ex(..., 0, stream).
 */
mxfp8_status mxfp8_gemm_ex(const uint8_t *a, const uint32_t *a_packed,
                           const uint8_t *b, const uint32_t *b_packed,
                           void *c, int64_t ldc,
                           int64_t M, int64_t N, int64_t K, uint32_t flags, void *stream);

/*
 * mxfp8_gemm_ex with a bias epilogue.  Defining passage: the fused bias that
 * the FlyDSL backend leaves as a TODO, so that te.Linear(bias=True) fails on
 * its first forward pass ("Experimental FlyDSL GEMM backend for TE PyTorch
 * (BF16/FP16/FP32/FP8/MXFP8)", review of the fallback exceptions and of the
 * epilogue validation).
 *
 *   C[m][n] = bf16_rne( epi( sum_k dq(A)[m][k] dq(B)[n][k] + bias[n] ) ),
 *
 * the BF16 bias added to the fp32 sum, epi the relu^2 / GELU epilogue or the
 * identity.  With MXFP8_GEMM_SWIGLU the bias has 2N values, one per B row:
 * C[m][n] = SiLU(g + bias[n]) * (u + bias[N + n]).
 * bias    BF16 [N] ([2N] with SWIGLU), 16-byte aligned, not NULL.
 * flags   0, MXFP8_GEMM_SQRELU, MXFP8_GEMM_GELU or MXFP8_GEMM_SWIGLU
 *         (ACCUMULATE -> FLAGS).  K == 0 writes epi(bias).
 * Other arguments and errors as mxfp8_gemm_ex; NULL for a NULL bias,
 * MISALIGNED for a bias not 16-byte aligned.
 */
mxfp8_status mxfp8_gemm_bias(const uint8_t *a, const uint32_t *a_packed,
                             const uint8_t *b, const uint32_t *b_packed,
                             const void *bias, void *c, int64_t ldc,
                             int64_t M, int64_t N, int64_t K, uint32_t flags, void *stream);

/* ------------------------------------------------------------------------
 * Grouped (ragged expert) GEMM
 *
 * Defining passages: per group g the A operand's row base moves to the
 * group's first row and its row extent shrinks to the group size ("frost
 * (gemm): Add Rubin kernel pipelines", review of the MoE grouped template);
 * expert boundaries are int32 offsets that stay on the device, empty groups
 * are legal and an empty total is a no-op, one launch per call, no host
 * synchronisation and no workspace ("gemm(cutedsl): add standalone Lightning
 * W4A16 grouped GEMM", PR body and review of the zero-token case).
 *
 *   for g < G, for m in [offsets[g], offsets[g+1]):
 *       C[m][n] = bf16_rne( sum_k dq(A)[m][k] * dq(B_g)[n][k] ).
 * ------------------------------------------------------------------------ */

/*
 * a          E4M3 codes [M_total][K], 16-byte aligned.
 * a_packed   uint32 [K/128][M_total].
 * b          E4M3 codes of the G experts [G][N][K], 16-byte aligned.
 * b_packed   uint32 [K/128][G*N]: the experts' scales stacked as G*N rows and
 *            packed in one mxfp8_pack_scales call (expert g, row n is packed
 *            row g*N + n).
 * offsets    DEVICE int32 [G+1]: offsets[0] = 0, non-decreasing,
 *            offsets[G] <= M_total.  Rows of C outside every group are not
 *            written.  Values are read on the device only.  Invalid offsets
 *            cannot make an access leave the buffers: each bound is clamped
 *            into [0, M_total] and then raised to the largest bound before
 *            it, i.e. group g covers rows [e_g, e_{g+1}) with
 *            e_i = max_{j <= i} clamp(offsets[j], 0, M_total).  Groups
 *            therefore never overlap, and a group whose offsets decrease is
 *            empty (for valid offsets e_i = offsets[i]).
 * G          1 <= G <= 65536.
 * c          BF16 [M_total][ldc]; ldc >= N, ldc % 8 == 0.
 * M_total >= 0; N >= 0 and N % 32 == 0; K >= 0, K % 128 == 0 and K <= 2^22.
 * Errors: NULL, SHAPE, MISALIGNED, LIMIT, HIP.
 */
mxfp8_status mxfp8_grouped_gemm(const uint8_t *a, const uint32_t *a_packed,
                                const uint8_t *b, const uint32_t *b_packed,
                                const int32_t *offsets, int32_t G,
                                void *c, int64_t ldc,
                                int64_t M_total, int64_t N, int64_t K, void *stream);

/* mxfp8_grouped_gemm with options (flags as mxfp8_gemm_ex; rows outside every
 * group are neither read nor written).  With MXFP8_GEMM_SWIGLU each expert
 * holds 2N rows: b is [G][2N][K], b_packed [K/128][G*2N] (expert g, row r is
 * packed row 2gN + r), the gate projection in rows 0..N-1 of an expert and
 * the up projection in rows N..2N-1; C is [M_total][N]. */
mxfp8_status mxfp8_grouped_gemm_ex(const uint8_t *a, const uint32_t *a_packed,
                                   const uint8_t *b, const uint32_t *b_packed,
                                   const int32_t *offsets, int32_t G,
                                   void *c, int64_t ldc,
                                   int64_t M_total, int64_t N, int64_t K, uint32_t flags, void *stream);

/* mxfp8_grouped_gemm_ex with the bias epilogue of mxfp8_gemm_bias, one bias
 * per expert: bias BF16 [G][N] ([G][2N] with SWIGLU), expert g's bias at
 * bias + g * N (g * 2N), 16-byte aligned.  Flags and errors as
 * mxfp8_gemm_bias and mxfp8_grouped_gemm_ex. */
mxfp8_status mxfp8_grouped_gemm_bias(const uint8_t *a, const uint32_t *a_packed,
                                     const uint8_t *b, const uint32_t *b_packed,
                                     const int32_t *offsets, int32_t G, const void *bias,
                                     void *c, int64_t ldc,
                                     int64_t M_total, int64_t N, int64_t K, uint32_t flags, void *stream);

/*
 * GEMM with an MXFP8 output: the output quantization that the FlyDSL backend
 * rejects ("Experimental FlyDSL GEMM backend for TE PyTorch
 * (BF16/FP16/FP32/FP8/MXFP8)", review of the fallback exceptions: a quantizer
 * for the GEMM output, reachable from te.Linear's output quantization
 * parameters, and of the epilogue validation, which raises for it).
 *
 * The output of mxfp8_gemm_bias (bias given) or mxfp8_gemm_ex (bias NULL)
 * with the same flags, i.e. the BF16 values C that those would write, is
 * written as its rowwise MXFP8 copy instead: codes q_out[m][n] and, per row
 * and 32-column block, the scale byte of the quantizer's rowwise rule, in the
 * packed word layout of the GEMM operands, so the result is the A operand of
 * a following GEMM.  The codes and scales equal those of mxfp8_quantize_ex
 * (ROWWISE | PACKED_SCALES) applied to C.
 * q_out         E4M3 codes [M][ldq]; ldq >= N, ldq % 16 == 0, 16-byte aligned.
 * q_out_packed  uint32 [N/128][M] (word (t, m): scale bytes of blocks
 *               4t .. 4t+3 of row m), 4-byte aligned, not NULL.
 * bias          as mxfp8_gemm_bias, or NULL for none.
 * N             the output columns (SWIGLU: B holds 2N rows); N % 128 == 0.
 * flags         0, MXFP8_GEMM_SQRELU, MXFP8_GEMM_GELU or MXFP8_GEMM_SWIGLU
 *               (ACCUMULATE -> FLAGS).
 * Other arguments and errors as mxfp8_gemm_ex.
 */
mxfp8_status mxfp8_gemm_mxfp8_out(const uint8_t *a, const uint32_t *a_packed,
                                  const uint8_t *b, const uint32_t *b_packed, const void *bias,
                                  uint8_t *q_out, int64_t ldq, uint32_t *q_out_packed,
                                  int64_t M, int64_t N, int64_t K, uint32_t flags, void *stream);

/* The grouped GEMM (mxfp8_grouped_gemm_ex / mxfp8_grouped_gemm_bias, bias per
 * expert or NULL) with the MXFP8 output of mxfp8_gemm_mxfp8_out: q_out
 * [M_total][ldq], q_out_packed [N/128][M_total]; rows outside every group are
 * not written (codes nor scale words). */
mxfp8_status mxfp8_grouped_gemm_mxfp8_out(const uint8_t *a, const uint32_t *a_packed,
                                          const uint8_t *b, const uint32_t *b_packed,
                                          const int32_t *offsets, int32_t G, const void *bias,
                                          uint8_t *q_out, int64_t ldq, uint32_t *q_out_packed,
                                          int64_t M_total, int64_t N, int64_t K, uint32_t flags,
                                          void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFP8_H */
