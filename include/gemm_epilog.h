/*
 * gemm_epilog.h -- fused GEMM + bias/activation epilogue for AMD MI355X (gfx950).
 *
 *   D = epilogue(scale_a*scale_b * A*B + bias)
 *
 * computed in ONE kernel: the bias broadcast-add, the activation (ReLU or
 * GELU) and the optional ReLU sign-mask output are applied to the fp32
 * accumulators while they are still in registers, so the pre-activation
 * matrix is never written to memory and read back.
 *
 * Pages cited:
 *   [cuBLASLt page] "PyTorch inference: cuBLASLt bias fusion optimization"
 *                   (blog.hotdry.top, 2025-09-22)
 *   [nvmath page]   "nvmath-python cuBLASLt bias fusion for PyTorch inference"
 *                   (blog.hotdry.top, 2025-09-22)
 *   [epilog page]   "Explaining how nvmath-python's epilog mechanism
 *                   configures parameters to fuse the bias add into the
 *                   cuBLASLt matmul kernel" (blog.hotdry.top, 2025-09-22)
 *   [NVGEMM page]   "PyTorch 2.14 NVGEMM epilogue fusion" (zdabc.icu)
 *
 * Life cycle (the stateful create -> plan -> execute -> free object of the
 * nvmath page, paragraph on the workflow, and of the epilog page, paragraphs
 * on Matmul.plan's epilog and epilog_inputs arguments):
 *
 *   gemm_epilog_create   describe the problem (shapes, dtypes, layouts)
 *   gemm_epilog_plan     choose the epilogue and bias axis; the planner picks
 *                        the kernel, tile and launch shape (host-only work,
 *                        done once, kept apart from the steady-state calls)
 *   gemm_epilog_execute  launch asynchronously on a HIP stream (any number of
 *                        times, from any thread, on any stream)
 *   gemm_epilog_free     release the host-side plan
 *
 * Conventions, all calls:
 *   - Matrices are row-major.  A is m x k with leading dimension lda.  B is
 *     k x n (op_b = GE_OP_N, ldb >= n) or, for a Linear layer's weight, n x k
 *     (op_b = GE_OP_T, ldb >= k).  D is m x n with leading dimension ldd.
 *     Leading dimensions are in elements.
 *   - Every buffer passed to execute is a DEVICE pointer owned by the caller.
 *     The library never allocates, frees, copies or synchronises.
 *   - Status codes are returned, never thrown; a call that fails leaves no
 *     state behind and launches nothing.  All validation happens before any
 *     HIP runtime call.
 *   - A planned handle is immutable: concurrent executes on different
 *     streams are safe.  free() touches only host memory and is safe while
 *     kernels launched from the handle are still running.
 *
 * Environment, read by gemm_epilog_plan:
 *   GE_LOG=1           print each successful plan's description to stderr
 *   GE_K_STAGGER=<n>   the tile path takes its full K steps in a rotated
 *                      order, each tile starting n steps further in per tile
 *                      row and column of its launch group, so that tiles
 *                      sharing a panel of A or B do not fetch the same lines
 *                      at once; overrides the planner's choice (0 = off).
 *                      The K summation order, and so the rounding of float
 *                      results, depends on it; results stay bitwise
 *                      reproducible for a given plan.
 */
#ifndef GEMM_EPILOG_H
#define GEMM_EPILOG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
enum {
    GE_OK = 0,
    GE_ERR_NULL = 1,      /* a required pointer is NULL                         */
    GE_ERR_SHAPE = 2,     /* m, n or k < 0, a leading dimension too small, a
                             dimension beyond 2^31-1, or an unknown plan option */
    GE_ERR_DTYPE = 3,     /* unsupported or mismatched dtype combination        */
    GE_ERR_EPILOG = 4,    /* unknown epilogue / axis, or aux buffer missing for
                             RELU_AUX_BIAS / given for any other epilogue, or
                             bias missing when the epilogue needs one           */
    GE_ERR_ALIGN = 5,     /* a pointer or a row stride is not 16-byte aligned   */
    GE_ERR_STATE = 6,     /* execute on a handle that has not been planned      */
    GE_ERR_WORKSPACE = 7, /* workspace NULL or smaller than workspace_size      */
    GE_ERR_HIP = 8,       /* the kernel launch failed (HIP error)               */
    GE_ERR_ALLOC = 9,     /* host memory for the handle could not be allocated  */
    GE_ERR_STATIC_LIMIT = 10 /* execute_static: the plan needs more workspace than
                                GE_STATIC_WORKSPACE_BYTES                         */
};

/* Size of the workspace array the library holds on each GPU for
 * gemm_epilog_execute_static (16 MiB). */
#define GE_STATIC_WORKSPACE_BYTES (16u << 20)

/* ---- element types ---------------------------------------------------------
 * fp16 = IEEE binary16; bf16 = bfloat16; e4m3 = OCP 8-bit float E4M3 (max
 * 448, no infinities), the fp8 format of gfx950's matrix cores.  All products
 * accumulate in fp32 (the 32-bit compute type of the cuBLASLt page,
 * paragraph 3).
 * GE_MXF8_E4M3: E4M3 elements in MX block-scaled form (OCP Microscaling):
 * every run of 32 consecutive K values of a row of A, or of a column of B,
 * shares one E8M0 scale (an unsigned 8-bit exponent, scale = 2^(e - 127),
 * 0xFF = NaN); the element's value is its E4M3 value times that scale.  The
 * nvmath page names FP8 among the input types and, in its closing
 * paragraph, low-precision formats as where the fused epilogue is heading.
 * Such handles are executed with gemm_epilog_execute_mx, which takes the
 * scales. */
typedef enum { GE_F32 = 0, GE_F16 = 1, GE_BF16 = 2, GE_F8_E4M3 = 3, GE_MXF8_E4M3 = 4 } ge_dtype;

typedef enum { GE_OP_N = 0, GE_OP_T = 1 } ge_op;

/* Epilogues, as the epilog page's paragraph on the epilog enum lists them
 * (BIAS, RELU_BIAS, RELU_AUX_BIAS), plus NONE and GELU_BIAS (GELU is named
 * as a fused activation on the cuBLASLt page, paragraph 2, and in the NVGEMM
 * page's section on why epilogue fusion matters).  With C = s*A*B the scaled
 * product (s = scale_a * scale_b, see execute) and P the pre-activation (C
 * plus bias):
 *   NONE           D = C                            (no bias read)
 *   BIAS           D = P
 *   RELU_BIAS      D = max(P, 0)
 *   RELU_AUX_BIAS  D = max(P, 0), and aux bit (i,j) = (P[i][j] > 0)
 *   GELU_BIAS      D = GELU(P) = 0.5 P (1 + tanh(sqrt(2/pi) (P + 0.044715 P^3)))
 *   TANH_BIAS      D = tanh(P)  (Tanh is among the predefined epilogues the
 *                  nvmath page lists in its paragraph on limitations)
 * The training-side epilogues serve the backward pass, which needs what the
 * forward activation saw (nvmath page, paragraph on limitations: RELU_AUX_BIAS
 * produces the mask backward needs; its closing paragraph names GELU and the
 * bias gradient as the next fusions):
 *   GELU_AUX_BIAS  D = GELU(P), and aux[i][j] = P[i][j] in D's dtype (output)
 *   DRELU          D = C * ReLU'(P): C where mask bit (i,j) of aux is set,
 *                  else 0; aux is an input, the bit matrix RELU_AUX_BIAS wrote
 *   DGELU          D = C * GELU'(P), P read from aux (an input, the matrix
 *                  GELU_AUX_BIAS wrote); GELU' is the derivative of the tanh
 *                  form above
 *   DRELU_BGRAD, DGELU_BGRAD
 *                  D as DRELU / DGELU, and the bias gradient written to the
 *                  bias pointer (an output here, D's dtype): the fp32 values
 *                  of D summed along the other axis, g[i] = sum_j D[i][j]
 *                  (ROW, m values) or g[j] = sum_i D[i][j] (COL, n values);
 *                  the unfused pair sums the stored, rounded D instead
 * The backward epilogues read no bias (C is the gradient arriving from the
 * next layer's product).  Conversion of the fp32 result to D's dtype rounds
 * to nearest even. */
typedef enum {
    GE_EPILOG_NONE = 0,
    GE_EPILOG_BIAS = 1,
    GE_EPILOG_RELU_BIAS = 2,
    GE_EPILOG_RELU_AUX_BIAS = 3,
    GE_EPILOG_GELU_BIAS = 4,
    GE_EPILOG_GELU_AUX_BIAS = 5,
    GE_EPILOG_DRELU = 6,
    GE_EPILOG_DGELU = 7,
    GE_EPILOG_DRELU_BGRAD = 8,
    GE_EPILOG_DGELU_BGRAD = 9,
    GE_EPILOG_TANH_BIAS = 10
} ge_epilog;

/* Bias broadcast axis.
 * ROW: m values (shape (m,) or (m,1)); bias[i] is added to every column of
 *      row i -- the epilog page's paragraph on epilog_inputs.
 * COL: n values (shape (1,n)); bias[j] is added to every row of column j --
 *      the nvmath page's paragraph on shape constraints; a Linear layer. */
typedef enum { GE_BIAS_ROW = 0, GE_BIAS_COL = 1 } ge_bias_axis;

/* Problem description.  Supported dtype combinations (a_type == b_type):
 *   F32  inputs -> d_type F32
 *   F16  inputs -> d_type F16, F32 or E4M3
 *   BF16 inputs -> d_type BF16, F32 or E4M3
 *   E4M3 inputs -> d_type BF16, F16, F32 or E4M3
 *   MXF8_E4M3 inputs -> d_type BF16, F16, F32 or E4M3 (the 128 x 128 tile)
 * bias_type must equal d_type (for every epilogue): there is no implicit
 * conversion (nvmath page, paragraph on dtype agreement); with an E4M3 D
 * the bias is BF16.  E4M3 output: D = E4M3(y * scale_d), y the activated
 * fp32 value, rounded to nearest even and saturated to +-448 (NaN stays
 * NaN); see gemm_epilog_set_fp8_output for scale_d and the amax output.
 * It serves the inference epilogues (NONE, BIAS, RELU_BIAS, RELU_AUX_BIAS,
 * GELU_BIAS, TANH_BIAS) in the fused kernel: the plan refuses the others,
 * the unfused pair and execute_c with GE_ERR_DTYPE.
 * batch: 0 or 1 for one product; B > 1 (at most 65535) for B independent
 * products of the same shape and epilogue in one launch.  By default their
 * buffers are packed back to back: product b reads A + b*m*lda, B + b*k*ldb
 * (N) or b*n*ldb (T), the bias (or writes the bias gradient) at b*len (len =
 * m for ROW, n for COL), writes D + b*m*ldd and aux + b*m*(aux_ld_bits/8)
 * bytes (all offsets in elements of the buffer's dtype unless stated);
 * gemm_epilog_set_batch_strides sets other strides per operand.  The fp8
 * scales are shared.  The workspace scales with B. */
typedef struct {
    int64_t m, n, k;
    int32_t a_type, b_type, d_type, bias_type; /* ge_dtype */
    int32_t op_b;                              /* ge_op (op_a is always N) */
    int32_t batch;                             /* independent products, 0 = 1 */
    int64_t lda, ldb, ldd;                     /* in elements */
} ge_desc;

/* Planner preferences (all 0 = automatic).
 * path:    0 auto, 1 tile kernel, 2 small-m (batch <= 16) streaming kernel
 * unfused: 1 = run the unfused pair instead of the fused kernel: the GEMM
 *          with no epilogue writes the product, rounded to d_type, into the
 *          workspace; a second, elementwise kernel reads it back, adds the
 *          bias, applies the activation and writes D (and the mask).  This is
 *          the two-kernel sequence that fusion removes (epilog page, first
 *          body paragraph), kept for measurement and cross-checking.
 * tile:    0 auto, else a tile id: 1..4 the register-staged kernel (any
 *          dtype; 64x64, 128x128, 256x256, 256x128), 5..8 the pipelined
 *          direct-to-LDS kernel (fp16/bf16/fp8 inputs, not fp32; 256x256
 *          with 4 waves, 256x256 with 8 waves, 256x128, 128x128), 9..10
 *          the same kernel with register-staged copies (256x256 with 8 or
 *          4 waves), 11..12 with 128-byte K steps (256x256 with 8 or 4
 *          waves), 13 a 64x64 tile of it (fp16/bf16 only), 14 that tile with
 *          split-K (fp16/bf16 only; K slices in parallel, fp32 partials in
 *          the workspace summed in slice order by the tile's last slice before
 *          the epilogue; not with the bias-gradient epilogues).  An id the
 *          input dtype does not support gives GE_ERR_SHAPE.  The automatic
 *          choice takes 14 for fp16/bf16 problems of at most 64 such tiles
 *          with k >= 4096.  15: the pipelined kernel at 256x128 with 8 waves.
 * split_k: 0 auto, else the number of K slices (small-m path, or tile 14)
 * group_m: 0 auto, else the tile rows per group of the tile kernels' launch
 *          order (tiles are taken a group of rows at a time, column by
 *          column; a group of g rows keeps g row panels of A and the column
 *          panels of B in flight per die's L2).  Small-m path: 1, 2 or 4
 *          groups of 16 rows of W per wave, which share each fragment of x
 *          (a workgroup then covers 16, 32 or 64 output columns); any other
 *          value gives GE_ERR_SHAPE */
typedef struct {
    int32_t path;
    int32_t unfused;
    int32_t tile;
    int32_t split_k;
    int32_t group_m;
} ge_pref;

typedef struct ge_plan_s* ge_handle;

/* Create a handle for a problem.  Degenerate sizes are valid: m == 0 or
 * n == 0 makes execute a validated no-op; k == 0 gives D = act(bias) (the
 * product of empty operands is zero).  Validates shapes (m, n, k >= 0; lda >= k;
 * ldb >= n for N or >= k for T; ldd >= n), dtypes, and that every row
 * stride is a multiple of 16 bytes (epilog page, paragraph on epilog_inputs:
 * tensors must be 16-byte aligned).  On success *h owns host memory only.
 * Errors: GE_ERR_NULL, GE_ERR_SHAPE, GE_ERR_DTYPE, GE_ERR_ALIGN,
 * GE_ERR_ALLOC. */
int gemm_epilog_create(ge_handle* h, const ge_desc* desc);

/* Choose the epilogue and bias axis and plan the launch (kernel, tile, grid,
 * workspace).  p may be NULL.  May be called again to re-plan.  The bias
 * axis is validated for every epilogue but only used by those with a bias.
 * The small-m kernel serves the inference epilogues (NONE .. GELU_BIAS and
 * TANH_BIAS); the automatic path takes the tile kernel for the others.
 * Errors: GE_ERR_NULL (h), GE_ERR_EPILOG (unknown epilogue or axis, or the
 * small-m path forced with a training-side epilogue), GE_ERR_SHAPE (an
 * unknown tile id, split or group in p; or a forced pipelined tile whose
 * rows of A, or rows of B given n x k, span 4 GiB or more: its copies
 * address them as 32-bit offsets from the tile's first row, so the
 * automatic choice takes the register-staged kernel then), GE_ERR_ALIGN (batch > 1 with a COL bias
 * read by the epilogue and n * element size not a multiple of 16 bytes:
 * product b's bias, b*n values in, would not be 16-byte aligned). */
int gemm_epilog_plan(ge_handle h, int32_t epilog, int32_t bias_axis, const ge_pref* p);

/* Bytes of device workspace execute() needs: 0 for most fused launches; the
 * unfused pair's intermediate (m*ldd elements of d_type); the small-m path's
 * split-K partials and counters; the bias-gradient epilogues' fp32 partial
 * sums (one per tile row or column and gradient entry).  Each part is rounded
 * up to 256 bytes.
 * Errors: GE_ERR_NULL, GE_ERR_STATE (not planned). */
int gemm_epilog_workspace_size(ge_handle h, size_t* bytes);

/* Row stride of the aux buffer in bits.
 * Mask epilogues (RELU_AUX_BIAS writes it, DRELU and DRELU_BGRAD read it), and any handle
 * not planned with a pre-activation epilogue: round_up(n, 128), so each row
 * starts 16-byte aligned.  The mask is a row-major bit matrix of m rows: bit
 * (i,j) is bit j%32 of the little-endian 32-bit word at word index
 * i*(ld_bits/32) + j/32.  RELU_AUX_BIAS writes bits j >= n of a row as 0.
 * Pre-activation epilogues (GELU_AUX_BIAS writes it, DGELU and DGELU_BGRAD read it):
 * round_up(n, 128) elements of D's dtype, i.e. that many times 32 or 16 bits;
 * a row-major m-row matrix whose padding columns are never written.
 * The buffer must hold m*ld_bits/8 bytes.  Errors: GE_ERR_NULL. */
int gemm_epilog_aux_ld(ge_handle h, int64_t* ld_bits);

/* Launch the planned computation on `stream` (a hipStream_t; NULL = the
 * null stream).  Asynchronous: returns once the kernel(s) are queued.
 *   A, B     device operands (see ge_desc)
 *   bias     device vector of m (ROW) or n (COL) bias_type values; NULL
 *            only for NONE, DRELU and DGELU (which read no bias); for
 *            DRELU_BGRAD and DGELU_BGRAD the bias gradient is written here
 *   D        device output, m x n with leading dimension ldd
 *   aux      device aux buffer (see gemm_epilog_aux_ld); required for
 *            RELU_AUX_BIAS and GELU_AUX_BIAS (written) and for the backward
 *            epilogues (read), must be NULL otherwise
 *   scale_a, scale_b
 *            device pointers to one fp32 each; the product is scaled by
 *            s = scale_a * scale_b before the bias (D uses s*A*B): the
 *            per-tensor dequantisation factors of fp8 inputs, or an arbitrary
 *            alpha for any input dtype.  NULL means 1.0.
 *   workspace, workspace_bytes
 *            device scratch of at least gemm_epilog_workspace_size bytes
 *            (may be NULL/0 when that size is 0)
 * A pointer may be NULL only when its buffer holds no elements (e.g. A and B
 * when k == 0).  Every non-NULL pointer must be 16-byte aligned (scales:
 * 4-byte).  The
 * output and aux buffers must not overlap the inputs.
 * Errors: GE_ERR_NULL, GE_ERR_STATE, GE_ERR_EPILOG, GE_ERR_ALIGN,
 * GE_ERR_WORKSPACE, GE_ERR_HIP. */
int gemm_epilog_execute(ge_handle h, const void* A, const void* B, const void* bias,
                        void* D, void* aux, const float* scale_a, const float* scale_b,
                        void* workspace, size_t workspace_bytes, void* stream);

/* execute with a further input term: the product becomes s*A*B + beta*C
 * before the bias, activation or derivative, i.e. D = epilogue(s*A*B +
 * beta*C + bias) -- the general alpha/beta form that the cuBLASLt page's
 * paragraph on compute and scale types implies (alpha = s, see execute).
 *   C     device matrix, m x n in D's dtype, row stride ldc >= n elements
 *         (ldc * element size a multiple of 16 bytes); may be D itself (an
 *         in-place update: every element is read before it is written, by
 *         the same thread); with batch > 1, product b reads C + b*m*ldc
 *   beta  device pointer to one fp32, 4-byte aligned; when it holds 0, C is
 *         not read (it may hold anything, NaN included)
 * The other arguments, the asynchrony and the errors are as for execute, plus
 * GE_ERR_NULL (beta NULL, or C NULL with m*n > 0) and GE_ERR_SHAPE (ldc < n). */
int gemm_epilog_execute_c(ge_handle h, const void* A, const void* B, const void* C, int64_t ldc,
                          const float* beta, const void* bias, void* D, void* aux, const float* scale_a,
                          const float* scale_b, void* workspace, size_t workspace_bytes, void* stream);

/* execute for callers that cannot allocate device memory -- code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc: the
 * same kernels as gemm_epilog_execute, with the workspace taken from an
 * array the library itself holds on each GPU (GE_STATIC_WORKSPACE_BYTES, a
 * file-scope device array, resident until the process ends) instead of a
 * caller buffer.  The caller still passes every input and output.
 *   - Nothing is allocated or freed, by the library or anything it calls.
 *   - The array serves the current device (hipGetDevice); `stream` must
 *     belong to it.  The first call on a device looks up that device's copy
 *     of the array (one hipGetSymbolAddress, after all validation); later
 *     calls reuse the address.
 *   - Every call on a GPU shares that GPU's array, which keeps the last
 *     call's contents; what must start at zero (split-K arrival counters) is
 *     cleared by a kernel on `stream` at each call.  Calls on one stream are
 *     ordered; calls that overlap in time on one GPU (different streams, or
 *     different threads) race on the array and must not be made.
 * Arguments and errors as for gemm_epilog_execute (there is no workspace
 * argument), plus GE_ERR_STATIC_LIMIT when gemm_epilog_workspace_size exceeds
 * GE_STATIC_WORKSPACE_BYTES (e.g. the unfused pair's intermediate of a large
 * product), and GE_ERR_HIP when the array's device address cannot be had.
 * A plan whose workspace size is 0 never touches the array. */
int gemm_epilog_execute_static(ge_handle h, const void* A, const void* B, const void* bias,
                               void* D, void* aux, const float* scale_a, const float* scale_b,
                               void* stream);

/* fp8 (E4M3) output of a handle whose d_type is GE_F8_E4M3.  The nvmath page
 * lists FP8 among the supported dtypes and, in its closing paragraph, names
 * fp8 epilogues as where fusion is going; it gives no output-scaling rule,
 * and this one is the common fp8 inference reading.  scale_d (device, one
 * fp32, NULL = 1) multiplies y before the conversion; amax_d (device, one
 * fp32 per product of the batch, or NULL) receives max |y| over the
 * product's outputs (before the scale; NaN values do not count; 0 for a
 * product with no outputs), for a caller that derives the next scale from
 * it (delayed scaling).  The
 * library clears amax_d with a small kernel on the stream before each
 * execute, and the kernel combines the waves' maxima with atomic max on
 * the float's bits, so the result does not depend on the order.  The
 * pointers are kept in the handle and used by every later execute.
 * Errors: GE_ERR_NULL (h), GE_ERR_DTYPE (d_type is not E4M3), GE_ERR_ALIGN
 * (a pointer not 4-byte aligned). */
int gemm_epilog_set_fp8_output(ge_handle h, const float* scale_d, float* amax_d);

/* Per-product strides of a batched handle (batch > 1), in elements of each
 * buffer's type (aux: 32-bit words for the mask, D's dtype for the
 * pre-activation matrix): product z uses A + z*a, B + z*b, bias + z*bias,
 * D + z*d, aux + z*aux.  This is the strided-batch layout of the pages'
 * batched matmul (nvmath page, batched and strided operands; cuBLASLt page,
 * batch count and strides).  An input's stride may be anything >= 0; 0
 * shares one operand (a weight, a bias) between all products.  Outputs must
 * not overlap: d >= (m-1)*ldd + n, aux >= m * aux_ld_bits/32 words (the
 * mask's or pre-activation's rows as the plan lays them out), and a bias
 * gradient's stride >= its length.  Every stride times the element size
 * must keep 16-byte alignment (the operands' rows are read 16 bytes at a
 * time), except a ROW bias's, which is read one element at a time.  The
 * C input of execute_c stays packed (m*ldc elements per product).
 * s = NULL returns to the packed layout.  Strides are checked when execute
 * runs (they depend on the plan's epilogue).
 * Errors: GE_ERR_NULL (h), GE_ERR_SHAPE (a negative stride); at execute:
 * GE_ERR_ALIGN (a misaligned stride), GE_ERR_SHAPE (overlapping outputs). */
typedef struct {
    int64_t a, b, bias, d, aux;
} ge_batch_strides;
int gemm_epilog_set_batch_strides(ge_handle h, const ge_batch_strides* s);

/* execute with m rows, 0 <= m <= the m the handle was created with (the
 * dynamic-shape case of the NVGEMM page's upgrade checklist: one plan
 * serves every batch of rows up to its maximum, with no re-planning).  The
 * planned kernel, tile and launch order are kept; only the grid follows m.
 * A, D, the ROW bias and the aux rows hold m rows; with batch > 1 the
 * products stay where the planned m puts them (product z at z*m_max*lda,
 * ...), or at the strides set.  The workspace size of the plan suffices.
 * Errors: those of execute; GE_ERR_SHAPE (m < 0 or above the planned m);
 * GE_ERR_DTYPE for block-scaled handles (their scales come with
 * execute_mx). */
int gemm_epilog_execute_m(ge_handle h, int64_t m, const void* A, const void* B, const void* bias,
                          void* D, void* aux, const float* scale_a, const float* scale_b,
                          void* workspace, size_t workspace_bytes, void* stream);

/* execute for GE_MXF8_E4M3 handles (block-scaled fp8).  Arguments as for
 * execute, plus the block scales:
 *   a_scales  device, m rows of GE_MX_SCALE_LD(k) bytes: byte b of row i is
 *             the E8M0 scale of A[i][32b .. 32b+31]
 *   b_scales  device, n rows of GE_MX_SCALE_LD(k) bytes: byte b of row j is
 *             the scale of B's column j at K values 32b .. 32b+31, whichever
 *             layout B has (for B given n x k, its rows' scales)
 * Only the first ceil(k/32) bytes of a row are read; the rest is padding
 * that keeps every row 16-byte aligned.  With batch > 1, product z reads
 * a_scales + z*m*ld and b_scales + z*n*ld.  scale_a and scale_b keep their
 * meaning (a further per-tensor factor, NULL = 1).
 * Errors: those of execute, GE_ERR_DTYPE (the handle is not MXF8_E4M3),
 * GE_ERR_NULL (a scale array NULL while its operand holds elements),
 * GE_ERR_ALIGN (a scale array not 16-byte aligned).  execute, execute_c,
 * execute_static and autotune on an MXF8_E4M3 handle return GE_ERR_NULL
 * (the scales are missing). */
#define GE_MX_SCALE_LD(k) ((((k) + 31) / 32 + 15) / 16 * 16)
/* (batched MX: the scale arrays stay packed, z*m*ld and z*n*ld bytes, with
 * or without gemm_epilog_set_batch_strides) */
int gemm_epilog_execute_mx(ge_handle h, const void* A, const void* B, const void* a_scales,
                           const void* b_scales, const void* bias, void* D, void* aux,
                           const float* scale_a, const float* scale_b, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Release the handle (NULL is accepted).  Host-only. */
int gemm_epilog_free(ge_handle h);

/* Human-readable text for a status code (static storage). */
const char* gemm_epilog_status_string(int status);

/* Write a one-line description of the plan (path, tile, grid, workspace)
 * into buf (always NUL-terminated when cap > 0).  Errors: GE_ERR_NULL. */
int gemm_epilog_describe(ge_handle h, char* buf, size_t cap);

/* Autotune a planned handle on the caller's buffers (the cuBLASLt page's
 * paragraph on limitations and the nvmath page's paragraph on timing both
 * suggest letting the library try its kernels when the default choice is not
 * fast enough).  Every candidate the plan's path and input dtype allow -- the
 * tile ids of the tile path, or the row groups 1, 2, 4 times the K splits
 * 1, 2, 4, ... of the small-m path -- is re-planned with the same epilogue, bias axis and unfused
 * choice, run once, then `iters` times between two HIP events on `stream`;
 * the fastest replaces the plan (the shape heuristic's own choice is among
 * the candidates, so the result is never slower than it as measured).
 * Candidates whose workspace would exceed workspace_bytes are skipped.
 * Arguments as for execute, which this calls: it overwrites D, aux (and, for
 * the bias-gradient epilogues, bias) like execute does.  Unlike execute it
 * synchronises `stream` and creates and destroys two HIP events; nothing is
 * allocated on the device.  *best_ms (may be NULL) receives the winner's mean
 * time per call.  Errors: those of execute, GE_ERR_SHAPE (iters < 1), and
 * GE_ERR_HIP if event creation or timing fails (the plan is then unchanged). */
int gemm_epilog_autotune(ge_handle h, const void* A, const void* B, const void* bias,
                         void* D, void* aux, const float* scale_a, const float* scale_b,
                         void* workspace, size_t workspace_bytes, int32_t iters, void* stream,
                         float* best_ms);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_EPILOG_H */
