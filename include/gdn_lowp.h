/*
 * gdn_lowp.h -- FP8 (OCP E4M3) projection GEMMs of the GDN block, gfx950.
 *
 * The pages run the block's projections (q, k, v, gates, output) in mixed precision (the Chinese summary,
 * "Results", Table 2 and Figure 6: projections that keep quality in low precision; the Korean review,
 * section 1 "Key Terms", MPQ).  They print neither the formats' details nor a scaling policy; this interface
 * takes E4M3 with one float32 scale per row:
 *     quantise:  s[r] = max_c |x[r][c]| / 448,  code[r][c] = E4M3(x[r][c] * (448 / max_c |x[r][c]|))
 *                (all in float32; round to nearest, ties to even; saturating at +-448; a zero row gives s = 0
 *                and codes 0)
 *     GEMM:      y[m][n] = s_x[m] s_w[n] sum_k E4M3^-1(x[m][k]) E4M3^-1(w[n][k])
 *                (float32 accumulation, bf16 result rounded to nearest even)
 * Activations are quantised per token (rows of x), weights per output feature (rows of w), so a projection is
 * one gdn_quantize_rows_e4m3 of its input and one gdn_gemm_e4m3 against pre-quantised weights.
 *
 * Conventions: return GDN_OK (0) or a negative GDN_E_* code from gdn_stream.h with gdn_last_error() set;
 * on error nothing is enqueued.  Device pointers are caller-owned, on the current HIP device; work is
 * enqueued on hip_stream (NULL = null stream).  No handle and no allocation.
 */
#ifndef GDN_LOWP_H
#define GDN_LOWP_H

#include <stdint.h>

#include "gdn_stream.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Per-row E4M3 quantisation.  x: [rows][cols] of x_dtype (GDN_BF16 or GDN_F32) with row stride x_stride
 * elements (>= cols); codes: [rows][codes_stride] bytes (>= cols); scales: [rows] float32.  rows, cols >= 0.
 * Errors: GDN_E_INVAL (NULL pointer with rows > 0, stride below cols), GDN_E_DTYPE, GDN_E_SHAPE (an extent of
 * 2^40 bytes or more), GDN_E_HIP. */
GDN_API int gdn_quantize_rows_e4m3(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t x_stride,
                                   uint8_t* codes, int64_t codes_stride, float* scales, void* hip_stream);

/* y = diag(x_scales) dec(x) dec(w)^T diag(w_scales) as bf16.  x: [M][K] codes, row stride x_stride bytes;
 * w: [N][K] codes, row stride w_stride bytes; y: [M][N] bf16, row stride y_stride elements.  Requirements:
 * K a multiple of 16; N a multiple of 4; x, w, w_scales 16-byte aligned, y 8-byte aligned; x_stride and
 * w_stride multiples of 16 and >= K; y_stride a multiple of 4 and >= N; (M - 1) x_stride + K and
 * (N - 1) w_stride + K below 2^31.  M = 0 or N = 0 enqueues nothing; K = 0 writes y = 0 and reads neither x nor
 * w (which may then be NULL).  x_scales, w_scales and y are caller-owned device memory, as are x and w; the call
 * is asynchronous on hip_stream.  Errors: GDN_E_INVAL (NULL pointer, alignment, strides), GDN_E_SHAPE (sizes),
 * GDN_E_HIP. */
GDN_API int gdn_gemm_e4m3(const uint8_t* x, int64_t x_stride, const float* x_scales, const uint8_t* w,
                          int64_t w_stride, const float* w_scales, int64_t M, int64_t N, int64_t K, void* y,
                          int64_t y_stride, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_LOWP_H */
