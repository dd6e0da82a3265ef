/* Comparators and calibration probes for the fused GEMM-epilogue library (gfx950).
 *
 * libge_baselines.so is measurement infrastructure, not part of the fused path:
 *
 *  - The unfused sequence.  The pages' point is that the memory-bound operations around a GEMM
 *    (scale, bias, activation, gating, normalisation statistics, residual, reductions) each move
 *    a whole intermediate through HBM when they run as separate kernels ("Optimising GPU kernels
 *    with TileLang", fused-epilogue paragraph; superoptimizer write-up, sections 7 and 9: the
 *    two-kernel RMSNorm that lost for its extra launch and round trip of S; CODA news item, "How
 *    CODA works"; cuDNN tutorial, graph with an AMAX node).  These kernels run that sequence
 *    literally -- one kernel per operation, bf16 in and bf16 out (fp8 for the quantiser), the
 *    GEMM itself being libgemm_epilogue.so with an empty chain -- so that the bytes the fused
 *    kernel saves and its speed-up can be measured, not assumed.
 *  - Calibration probes: a matrix-core loop and a streaming copy, giving the MFMA throughput and
 *    HBM bandwidth this GPU sustains, next to the published peaks.
 *
 * Conventions.  Every pointer is a device pointer owned by the caller; arrays are dense and
 * row-major; bf16 values are passed as their 16-bit patterns, fp8 as OCP e4m3 bytes.  Work is
 * enqueued on `stream` (a hipStream_t, NULL = the legacy default stream) and nothing
 * synchronises.  Return value: 0 on success, 1 for an invalid argument (null pointer with a
 * non-zero size, negative size, unknown activation), 2 when the launch itself failed (the HIP
 * error is cleared).  Sizes of zero enqueue nothing (AMAX then stores 0).  Rounding: every
 * bf16 result is rounded to nearest even from the fp32 value the operation computes.
 */
#ifndef GE_BASELINES_H
#define GE_BASELINES_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* y[i] = bf16(alpha * x[i]), i < n. */
int ge_unfused_scale(const uint16_t* x, uint16_t* y, int64_t n, float alpha, void* stream);

/* y[r][c] = bf16(x[r][c] + bias[c]) for rows x cols (bias has cols entries, shared by rows);
 * cols % 8 == 0 and rows * cols / 8 < 2^32, else 1. */
int ge_unfused_bias_col(const uint16_t* x, const uint16_t* bias, uint16_t* y, int64_t rows, int64_t cols,
                        void* stream);

/* y[i] = bf16(act(x[i])); act as ge_act_t: 0 none, 1 ReLU, 2 GELU (tanh form), 3 SiLU. */
int ge_unfused_act(const uint16_t* x, uint16_t* y, int64_t n, int act, void* stream);

/* y[i] = bf16(act(g[i]) * u[i]) -- the pairwise gate over two GEMM outputs. */
int ge_unfused_act_mul(const uint16_t* g, const uint16_t* u, uint16_t* y, int64_t n, int act, void* stream);

/* s[r] = 1 / sqrt(sum_k x[r][k]^2 / cols + eps) in fp32, for rows x cols bf16 x (the separate
 * statistic kernel of the superoptimizer's two-kernel RMSNorm). */
int ge_unfused_row_rms(const uint16_t* x, float* s, int64_t rows, int64_t cols, float eps, void* stream);

/* y[r][c] = bf16(x[r][c] * s[r]) -- normalisation of the rows by an fp32 row scale; same size
 * limits as ge_unfused_bias_col. */
int ge_unfused_row_scale(const uint16_t* x, const float* s, uint16_t* y, int64_t rows, int64_t cols,
                         void* stream);

/* y[i] = bf16(x[i] * act'(z[i])) -- the backward activation gradient with the saved
 * pre-activation z; act as in ge_unfused_act. */
int ge_unfused_act_grad(const uint16_t* x, const uint16_t* z, uint16_t* y, int64_t n, int act, void* stream);

/* out[c] = sum over r of x[r][c] in fp32 (rows x cols bf16 x; rows summed in order) -- the
 * bias-gradient column reduction. */
int ge_unfused_col_sum(const uint16_t* x, float* out, int64_t rows, int64_t cols, void* stream);

/* y[i] = bf16(x[i] + r[i]) -- residual add. */
int ge_unfused_add(const uint16_t* x, const uint16_t* r, uint16_t* y, int64_t n, void* stream);

/* *amax = max_i |x[i]| over bf16 x, as fp32 (NaN propagates as the largest pattern). */
int ge_unfused_amax(const uint16_t* x, int64_t n, float* amax, void* stream);

/* y[i] = e4m3(clamp(x[i] * scale, -448, 448)), round to nearest even. */
int ge_unfused_quant_fp8(const uint16_t* x, uint8_t* y, int64_t n, float scale, void* stream);

/* Matrix-core probe: `workgroups` workgroups of 4 waves, each wave running 16 independent
 * chains of `iters` v_mfma_f32_32x32x16_bf16 on random register operands (four sets per
 * source, so consecutive instructions see different bits, as in a GEMM -- the matrix core's
 * power, and so its sustained rate, depends on the data); `sink` receives workgroups * 256
 * floats (keeps the work live).  Floating-point work per launch:
 * workgroups * 4 * 16 * iters * 32768. */
int ge_probe_mfma(float* sink, int workgroups, int iters, void* stream);

/* The same probe on the other matrix-core forms: variant 0 is ge_probe_mfma; variant 1 runs 16
 * chains of v_mfma_f32_16x16x32_bf16 on the same random bf16 operand sets (work per launch:
 * workgroups * 4 * 16 * iters * 16384); variant 2 runs 8 chains of v_mfma_f32_32x32x64_f8f6f4
 * on random e4m3 codes without NaN codes, the fp8-operand mainloop's instruction (work per
 * launch: workgroups * 4 * 8 * iters * 131072).  Returns 1 for an unknown variant or invalid
 * arguments. */
int ge_probe_mfma_variant(float* sink, int workgroups, int iters, int variant, void* stream);

/* fp8 matrix-core probe: `waves` single-wave workgroups, each running ONE
 * v_mfma_f32_32x32x64_f8f6f4 with e4m3 codes in both sources and no block scales on its own
 * register contents.  Lane l of wave w reads 32 bytes of src0 and of src1 at byte offset
 * (64*w + l)*32 and 16 fp32 accumulator values of c at float offset (64*w + l)*16, and writes its
 * 16 result values to d at the same offsets.  All pointers 64-byte aligned.  Used to measure
 * how the instruction sums its 64 products (the accuracy of fp8-operand GEMMs). */
int ge_probe_mfma_f8(const uint8_t* src0, const uint8_t* src1, const float* c, float* d, int waves, void* stream);

/* L2 -> LDS probe, the fused kernels' operand path alone: `workgroups` workgroups of 4 waves,
 * each wave issuing `iters` rounds of eight direct global->LDS loads (16 bytes per lane, 1 KB
 * per instruction; up to sixteen in flight) from the first `src_kb` KiB of `src` (8 to 2^20;
 * small enough to stay in L2 for the rate of L2 hits) into the workgroup's 64 KiB of LDS;
 * `sink` receives workgroups * 256 floats.  Bytes moved per launch: workgroups * iters * 32768. */
int ge_probe_lds_load(const void* src, int src_kb, float* sink, int workgroups, int iters, void* stream);

/* LDS read probe, the fused kernels' fragment reads alone: `workgroups` workgroups of 8 waves
 * (two per SIMD) holding 96 KiB of LDS each, so one per CU; each wave reads its own 12 KiB with
 * 16-byte-per-lane reads free of bank conflicts, `iters` rounds of eight 1 KiB reads.  `sink`
 * receives workgroups * 512 words (the folded data); `clocks` receives per workgroup two words:
 * the shader-clock cycles (s_memtime) and the constant-rate counter ticks (s_memrealtime) of
 * wave 0 around the loop.  Bytes read per workgroup: iters * 65536. */
int ge_probe_lds_read(uint32_t* sink, uint64_t* clocks, int workgroups, int iters, void* stream);

/* Streaming copy of `bytes` (a multiple of 16, 16-byte aligned pointers): reads and writes each
 * byte once. */
int ge_probe_copy(const void* src, void* dst, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GE_BASELINES_H */
