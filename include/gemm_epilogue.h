/*
 * gemm_epilogue.h -- fused GEMM + epilogue for AMD Instinct MI355X (gfx950).
 *
 * One operation:  Y = epilogue(A @ B [, A @ B2])  with bf16 operands, fp32
 * accumulation, and an epilogue that runs on the fp32 output tile while it is
 * still in registers, followed by the only store of Y to HBM.
 *
 * Where the operation is defined (pages as titled):
 *   - The tiled GEMM with the output tile kept in register fragments and the
 *     bias + GELU epilogue applied before the final write: "Optimising GPU
 *     kernels with TileLang: from GEMM to FlashAttention", tiled-matmul and
 *     fused-epilogue paragraphs; "Lean4-TileLang Tensor Program
 *     Superoptimizer" write-up, section 8 (Matmul): W is laid out [d, N].
 *   - The epilogue primitive set (scaling, reductions, pairwise transforms,
 *     accumulation) running while the GEMM output tile is on chip: "CODA:
 *     GEMM-epilogue for Transformer blocks", section "How CODA works".
 *   - Host-scalar alpha, bias, activation and an AMAX reduction on the result
 *     in the same kernel, feeding the next fp8 quantisation: "NVIDIA cuDNN
 *     Graph API" tutorial, batched-matmul paragraph; build-then-execute over
 *     a pack of device pointers: same tutorial, opening paragraph.
 *   - The pairwise SwiGLU epilogue out = silu(X@W_gate) * (X@W_up):
 *     superoptimizer write-up, section 7 (SwiGLU).
 *   - The per-row RMS scale 1/sqrt(mean(x^2) + eps) applied after the GEMM via
 *     (X*S)@W == (X@W)*S: superoptimizer write-up, section 9 (RMSNorm).
 *   - fp8 operands with delayed scaling: the AMAX of one pass sets the fp8 scale
 *     of the next (cuDNN tutorial, batched-matmul paragraph); a GEMM that
 *     consumes such fp8 tensors multiplies their e4m3 codes and dequantises the
 *     accumulator with alpha = 1 / (scale_A * scale_B).
 *
 * Layout (all row-major, leading dimensions and batch strides in ELEMENTS):
 *   A  [batch][M][K] bf16, element (b,m,k) at A + b*stride_a + m*lda + k
 *   B  b_layout GE_LAYOUT_KN (default): [batch][K][N] bf16, element (b,k,n) at
 *      B + b*stride_b + k*ldb + n (ldb >= N), as the pages lay W out;
 *      b_layout GE_LAYOUT_NK: [batch][N][K] bf16, element (b,k,n) at B + b*stride_b +
 *      n*ldb + k (ldb >= K) -- the product A @ B^T of a backward pass, dY @ W^T with W
 *      stored [K][N] (CODA news item, "How CODA works": forward and backward epilogues)
 *   B2 same layout, leading dimension and batch stride as B (pairwise only)
 *   Y  [batch][M][N] bf16 or fp8-e4m3 (OCP "e4m3fn"), at Y + b*stride_y + m*ldy + n
 *   R  [batch][M][N] bf16 residual, at R + b*stride_r + m*ldr + n
 *   Z  [batch][M][N] bf16 saved pre-activation (ACT_GRAD), at aux + b*stride_z + m*ldz + n
 *   col_sum [N] fp32 (COL_SUM)
 *   bias [N] bf16, shared by every row and batch
 *   row_scale [batch][M] fp32, at row_scale + b*M + m
 *   amax: one fp32 in device memory
 *   A batch stride of 0 broadcasts that operand over the batch.
 *   fp8 operands: a_type == b_type == GE_DT_FP8_E4M3 makes A, B (and B2) one-byte OCP e4m3
 *   ("e4m3fn") codes in the same element layout; B must then be GE_LAYOUT_NK, K, lda, ldb
 *   and the A/B batch strides multiples of 16, and ROW_RMS and ACT_GRAD are unsupported.
 *   The products are summed by the fp8 matrix-core instruction into fp32 accumulators
 *   (its own summation of each 64 products is less exact than fp32).
 *
 * Epilogue chain (descriptor order must be this canonical order; each op at
 * most once):
 *   SCALE            t = alpha * acc                      (alpha: host scalar)
 *   ROW_RMS(eps)     t = t / sqrt(mean_k A[b,m,k]^2 + eps) (statistic gathered in the mainloop)
 *   ROW_SCALE        t = t * row_scale[b,m]               (exclusive with ROW_RMS)
 *   BIAS_COL         t = t + bias[n]                      (not with PAIRWISE_ACT_MUL)
 *   ACT(act)         y = act(t)
 *   PAIRWISE_ACT_MUL(act)  y = act(t_gate) * t_up, gate from B, up from B2; the
 *                    linear ops above apply to both accumulators (exclusive with ACT)
 *   ACT_GRAD(act)    y = t * act'(Z[b,m,n]) -- the activation-gradient step of a backward
 *                    pass, dZ = (dY @ W^T) * act'(Z) (CODA news item, "How CODA works":
 *                    epilogues for the forward and the backward pass); exclusive with ACT
 *                    and PAIRWISE_ACT_MUL
 *   RESIDUAL         y = y + R[b,m,n]
 *   COL_SUM          col_sum[n] = sum over b, m of y[b,m,n] in fp32, before any rounding --
 *                    the column reduction that gives a bias gradient (same item, the
 *                    "reductions" primitive); overwritten, not accumulated; needs the
 *                    workspace; deterministic (fixed summation order)
 *   AMAX             *amax = max |y| over all outputs, before any rounding (needs the workspace);
 *                    the maximum is taken on the bit patterns of |y|, so a NaN y gives a NaN
 *   QUANT_FP8        Y = e4m3(clamp(y * quant_scale, -448, 448)), round to
 *                    nearest even; requires y_type == GE_DT_FP8_E4M3 and must be last.
 *                    Overflow saturates to +-448; a NaN y * quant_scale is written as the
 *                    e4m3 NaN code 0x7F (OCP: S.1111.111, no infinities)
 *   Without QUANT_FP8, Y = bf16(y), round to nearest even (y_type == GE_DT_BF16); NaN
 *   stays NaN and overflow becomes +-inf.
 *   Activations: RELU max(t,0); GELU_TANH 0.5 t (1 + tanh(sqrt(2/pi)(t + 0.044715 t^3)));
 *   SILU t / (1 + e^-t).
 *
 * Supported shapes: batch >= 0, M >= 0, N >= 0, K >= 0 (K >= 1 with ROW_RMS);
 * N, K, lda, ldb, ldy (and ldr, ldz) multiples of 8; lda >= K, ldb >= N ([K][N] B) or
 * ldb >= K ([N][K] B), ldy >= N, ldr >= N, ldz >= N; every device pointer 16-byte aligned
 * (col_sum and amax: 4-byte).  Ragged M, N and K tails (not multiples of the tile) are
 * handled inside the kernels.
 *
 * Ownership: the caller owns every device buffer and the stream.  The
 * library borrows the pointers until the work enqueued by gemm_epilogue_run
 * has completed.  A handle owns host memory only; the library never
 * allocates or frees device memory and never synchronises the stream.
 *
 * Errors: every call returns a status; nothing aborts and there is no global
 * error state.  Calls on one handle are safe from several threads because
 * run() reads the handle only.
 */
#ifndef GEMM_EPILOGUE_H
#define GEMM_EPILOGUE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GE_MAX_OPS 8

typedef enum {
  GE_OK = 0,
  GE_ERR_INVALID_ARG = 1,   /* null pointer, negative size, bad stride, bad op order */
  GE_ERR_UNSUPPORTED = 2,   /* well-formed but outside the supported set */
  GE_ERR_DEVICE = 3,        /* no HIP device, or the current device is not gfx950 */
  GE_ERR_HIP = 4,           /* a HIP runtime call or kernel launch failed */
  GE_ERR_SCRATCH = 5        /* gemm_epilogue_run_noalloc: the plan needs more scratch than
                               GE_NOALLOC_SCRATCH_BYTES */
} ge_status_t;

/* Size of the static device scratch behind gemm_epilogue_run_noalloc (per GPU). */
#define GE_NOALLOC_SCRATCH_BYTES (4u << 20)

typedef enum { GE_DT_BF16 = 0, GE_DT_FP8_E4M3 = 1, GE_DT_FP32 = 2 } ge_dtype_t;

typedef enum { GE_ACT_NONE = 0, GE_ACT_RELU = 1, GE_ACT_GELU_TANH = 2, GE_ACT_SILU = 3 } ge_act_t;

typedef enum { GE_LAYOUT_KN = 0, GE_LAYOUT_NK = 1 } ge_layout_t;

/* Kernel instances (output tile shapes).  The first five run 4 waves of 64 lanes (2 x 2 over the
 * tile, one wave per SIMD); the _2W ones run 8 waves (2 x 4, two waves per SIMD that alternate
 * between memory work and matrix-core work) and need K to be a multiple of 64 (bf16 operands) or
 * 128 (fp8 operands); other descriptors that request them get GE_ERR_UNSUPPORTED.  The pairwise instances hold two accumulators (gate and up).  With
 * tile = 0 the library takes a _2W instance where it applies and the grid has >= 256
 * workgroups of its shape. */
typedef enum {
  GE_TILE_256x256 = 0,
  GE_TILE_256x128_PAIR = 1,
  GE_TILE_128x128 = 2,
  GE_TILE_64x64 = 3,
  GE_TILE_128x128_PAIR = 4,
  GE_TILE_256x256_2W = 5,
  GE_TILE_256x128_PAIR_2W = 6,
  GE_TILE_COUNT = 7
} ge_tile_t;

/* Static facts of one instance: tile rows and columns, whether it is a pairwise instance,
 * workgroup size, and the LDS bytes one workgroup allocates with B given [K][N] (the [N][K]
 * and fp8-operand variants allocate within 32 bytes of it); a tile-config search filters
 * candidates by this against the 160 KiB of LDS per compute unit. */
typedef struct {
  int32_t bm, bn, pairwise, threads, lds_bytes;
} ge_tile_info_t;

typedef enum {
  GE_OP_SCALE = 0,
  GE_OP_ROW_RMS = 1,
  GE_OP_ROW_SCALE = 2,
  GE_OP_BIAS_COL = 3,
  GE_OP_ACT = 4,
  GE_OP_PAIRWISE_ACT_MUL = 5,
  GE_OP_RESIDUAL = 6,
  GE_OP_AMAX = 7,
  GE_OP_QUANT_FP8 = 8,
  GE_OP_ACT_GRAD = 9,
  GE_OP_COL_SUM = 10
} ge_op_kind_t;

typedef struct {
  int32_t kind;     /* ge_op_kind_t */
  int32_t act;      /* ge_act_t, for ACT, PAIRWISE_ACT_MUL and ACT_GRAD; else 0 */
  float eps;        /* for ROW_RMS; else 0 */
} ge_op_t;

typedef struct {
  int64_t batch, M, N, K;
  int64_t lda, ldb, ldy, ldr;                   /* leading dimensions, elements */
  int64_t stride_a, stride_b, stride_y, stride_r; /* batch strides, elements (0 = broadcast) */
  int32_t a_type, b_type, y_type;               /* ge_dtype_t: A and B both bf16 or both fp8_e4m3;
                                                   Y bf16 | fp8_e4m3 */
  int32_t n_ops;
  ge_op_t ops[GE_MAX_OPS];
  int32_t b_layout;                             /* ge_layout_t of B and B2 (0 = [K][N]) */
  int32_t tile;                                 /* kernel instance: 0 = chosen by create (the
                                                   largest tile that still gives >= 256
                                                   workgroups), 1 + ge_tile_t = that instance
                                                   (a tuned choice, e.g. from a tile-config
                                                   sweep); its pairwise-ness must match the chain */
  int64_t ldz, stride_z;                        /* ACT_GRAD: Z leading dimension and batch stride */
} ge_desc_t;

/* The per-execution "variant pack": borrowed device pointers plus host scalars.
 * Pointers an op does not use may be NULL. */
typedef struct {
  const void* A;
  const void* B;
  const void* B2;          /* PAIRWISE_ACT_MUL: the "up" weight */
  const void* bias;        /* BIAS_COL */
  const float* row_scale;  /* ROW_SCALE */
  const void* residual;    /* RESIDUAL */
  void* Y;
  float* amax;             /* AMAX: overwritten with max|y| */
  void* workspace;         /* AMAX, COL_SUM, shared ROW_RMS: device scratch of gemm_epilogue_workspace_size bytes,
                              16-byte aligned, ZERO-FILLED before its first use; each run leaves
                              it zeroed again when it completes.  Runs that share a workspace
                              must not overlap (order them on one stream). */
  size_t workspace_bytes;
  float alpha;             /* SCALE */
  float quant_scale;       /* QUANT_FP8 */
  const void* aux;         /* ACT_GRAD: Z, the saved pre-activation */
  float* col_sum;          /* COL_SUM: N floats, overwritten */
} ge_args_t;

typedef struct ge_plan* ge_handle_t;

/* Checks a descriptor without touching any device: the validation step of the cuDNN
 * tutorial's five-step build (opening paragraph: validate, build the operation graph, create
 * execution plans, check support, build the plan; then execute over a variant pack of
 * pointers); the op set and its order are the CODA news item's epilogue primitives ("How
 * CODA works").
 *   desc: host pointer, read only, not retained.
 * Returns GE_OK, GE_ERR_INVALID_ARG (NULL desc, negative size or stride, a leading dimension
 * below the row length, unknown op or dtype, ops out of the canonical order or repeated) or
 * GE_ERR_UNSUPPORTED (well formed but outside the supported set: alignment, extents beyond
 * 31-bit byte offsets, fp8 operands with B given [K][N], ...).  Never aborts. */
ge_status_t gemm_epilogue_validate(const ge_desc_t* desc);

/* Builds a plan: validation, the support check against the current device and the choice
 * of a kernel instance -- the support-check and plan-building steps of the cuDNN tutorial's
 * five-step build (opening paragraph), done once so that execution only binds pointers.
 *   desc: host pointer, copied into the plan (the caller may free it afterwards).
 *   out:  receives the handle; set to NULL on any failure.
 * Returns the status of gemm_epilogue_validate, GE_ERR_DEVICE when no HIP device is current or
 * it is not gfx950, GE_ERR_HIP when host memory for the plan cannot be had.  Launches nothing
 * and allocates no device memory; the handle owns host memory only. */
ge_status_t gemm_epilogue_create(const ge_desc_t* desc, ge_handle_t* out);

/* Device scratch the plan needs from the caller, in bytes -- the plan-specific workspace of
 * the cuDNN tutorial (set-up paragraph: a helper allocates the workspace; engine-autotuning
 * paragraph: each candidate plan is built, given a workspace of the size it reports, and
 * timed); 0 without AMAX, COL_SUM and a shared row statistic.
 * AMAX: nine ticket counters on their own cache lines plus one partial-maximum slot per
 * workgroup.  COL_SUM: one ticket counter per column tile plus one fp32 partial column sum
 * per row tile, batch and column.  ROW_RMS on the two-wave instances with more than one
 * tile column: per row tile and batch, a published flag and a ticket counter plus the tile's
 * fp32 sums of squares, so that tiles of a tile row that start after one of them has
 * published the statistic read it instead of recomputing it (no tile waits for another).
 * The workspace must be zero-filled before its first use, and every run that completes leaves
 * its counters at zero again.  HAZARD: a workspace whose counters are not zero -- never
 * cleared, or shared by two runs that overlap in time (two streams, or a run that did not
 * complete) -- makes AMAX, COL_SUM and ROW_RMS silently wrong: a counter holding d > 0 elects
 * a "last" workgroup d arrivals early, and a flag left set makes tiles read stale sums.  Clear it again (e.g. hipMemset) after any such event, and give
 * concurrent runs separate workspaces.  Returns GE_ERR_INVALID_ARG for a NULL handle or bytes. */
ge_status_t gemm_epilogue_workspace_size(ge_handle_t handle, size_t* bytes);

/* Executes a plan against a "variant pack" of borrowed device pointers and host scalars --
 * the execution step of the cuDNN tutorial's build-then-execute model (opening paragraph:
 * execution over a variant pack; batched-matmul paragraph: alpha is a host scalar and AMAX is
 * reduced on the result in the same kernel; closing paragraph: the stream is set per
 * execution, e.g. to a graph-capturing stream).  Computes the operation of the header
 * comment: the tiled GEMM with its output tile kept on chip while the epilogue runs, then one
 * store (TileLang tutorial, tiled-matmul and fused-epilogue paragraphs; CODA news item, "How
 * CODA works").
 *   handle: from gemm_epilogue_create; read only, so concurrent runs of one handle are safe
 *           when they use separate outputs and workspaces.
 *   args:   host pointer, read during the call only; the device pointers it holds are borrowed
 *           until the enqueued kernel completes.
 *   stream: a hipStream_t (NULL = the null stream).
 * Enqueues ONE kernel launch and returns without waiting.  With AMAX in the chain, *amax is
 * overwritten with max|y| when the kernel completes (the last workgroup to finish reduces the
 * per-workgroup maxima and publishes it).  Returns GE_ERR_INVALID_ARG for a NULL handle or
 * args, for a pointer an op needs that is NULL or misaligned, or for a workspace smaller than
 * gemm_epilogue_workspace_size (nothing is enqueued then), GE_ERR_HIP if the launch fails.  An
 * empty problem (batch, M or N zero) launches only a one-thread kernel that writes *amax = 0
 * (and, with COL_SUM, a kernel that zeroes col_sum). */
ge_status_t gemm_epilogue_run(ge_handle_t handle, const ge_args_t* args, void* stream);

/* For callers that cannot allocate device memory -- code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc: gemm_epilogue_run without a caller-given
 * workspace.  Same plan, same kernels, same results as gemm_epilogue_run; args->workspace and
 * args->workspace_bytes are ignored.  The AMAX / COL_SUM / row-statistic scratch comes from a static device
 * array of GE_NOALLOC_SCRATCH_BYTES (4 MiB) that the library's code object holds on every GPU
 * it runs on until the process ends; its device address is looked up once per device
 * (hipGetSymbolAddress, on the first call made with that device current).  Each call first
 * enqueues a small kernel that zeroes the ticket counters the plan uses (the array keeps the
 * previous call's contents), then the fused kernel: two launches on `stream`, no hipMalloc,
 * hipFree, memset node or other allocating call.  Plans without AMAX, COL_SUM and a shared
 * row statistic use no scratch and enqueue the fused kernel alone.
 * Returns GE_ERR_SCRATCH, enqueueing nothing, when gemm_epilogue_workspace_size exceeds
 * GE_NOALLOC_SCRATCH_BYTES (e.g. COL_SUM over more than about a million row-tile x column
 * partials); otherwise the statuses of gemm_epilogue_run, plus GE_ERR_HIP when the scratch
 * address cannot be looked up.
 * RACE: every call on one GPU shares that GPU's array, so calls that overlap in time on one
 * GPU (two streams, two host threads) corrupt each other's AMAX, COL_SUM and ROW_RMS; order them. */
ge_status_t gemm_epilogue_run_noalloc(ge_handle_t handle, const ge_args_t* args, void* stream);

/* Frees the plan's host memory (the end of a plan's life in the cuDNN tutorial's plan-reuse
 * model, closing paragraphs: a plan is built once and executed many times).  NULL is a no-op.  Work
 * already enqueued with the handle is unaffected: run() copies what the kernel needs. */
void gemm_epilogue_destroy(ge_handle_t handle);

/* Static, NUL-terminated description of a status code (never NULL; "unknown status" for a
 * value outside ge_status_t). */
const char* gemm_epilogue_status_string(ge_status_t status);

/* Fills *info for instance `tile` (a ge_tile_t).  GE_ERR_INVALID_ARG for an unknown tile or a
 * NULL info.  Pure host, no device needed.  For a tile-config search: the TileLang tutorial's
 * schedule-exploration paragraph autotunes over tile sizes and drops candidates beyond the
 * shared-memory budget; the cuDNN tutorial's engine-autotuning paragraph times every candidate
 * plan instead of trusting the heuristic.  The chosen instance goes in ge_desc_t.tile. */
ge_status_t gemm_epilogue_tile_info(int32_t tile, ge_tile_info_t* info);

/* Writes a one-line description of the plan's kernel instance (tile shape,
 * waves, grid) into buf (NUL-terminated, truncated to len). */
ge_status_t gemm_epilogue_describe(ge_handle_t handle, char* buf, size_t len);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_EPILOGUE_H */
