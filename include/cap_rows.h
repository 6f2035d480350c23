/*
 * cap_rows.h -- wide-row reduction-reuse workloads in libcap: softmax over
 * rows of logits and LayerNorm over rows, FP32, on AMD MI355X (gfx950).
 *
 * Source of the operation class: the CREDIT summary, section III.B
 * ("Reduction-Reuse Transformation": each row's elements are reduced to
 * scalar statistics that an elementwise function then reuses for every
 * output element) and section V.A ("Experimental Setup": FP32 workloads,
 * softmax-logits and LayerNorm among them, rows 4K to 64K wide).  The pages
 * give no formulas; these are the standard ones:
 *   softmax:   y_i = exp(x_i - max_j x_j) / sum_j exp(x_j - max_j x_j)
 *   LayerNorm: mu = mean_j x_j, var = mean_j (x_j - mu)^2 (biased),
 *              y_i = (x_i - mu) / sqrt(var + eps) * gamma_i + beta_i
 *
 * Conventions as in cap.h: the return code is the only error channel
 * (cap_last_error() for the message), a call that fails validation launches
 * nothing, all pointers are caller-owned DEVICE pointers, one launch on
 * `stream` (a hipStream_t; NULL = the null stream), no synchronisation.
 *
 * Layout: x and y are [rows][width] row-major FP32; y may be the same buffer
 * as x (in place) but may not overlap it otherwise.  gamma and beta are
 * [width] FP32.  Rows whose width is a multiple of 4 with 16-byte aligned
 * buffers use 16-byte accesses; other shapes use 4-byte accesses.
 *
 * mode: 0 = auto (3 for LayerNorm with 8192 <= width <= 16384, 16-byte
 * accesses and rows >= 1024; else 1 for width <= 65536 with 16-byte accesses
 * or <= 16384 with 4-byte accesses; else 2); 1 = retained: one workgroup
 * keeps its whole row in registers, so the row is read from HBM once
 * (width <= 65536, CAP_ERR_UNSUPPORTED above); 2 = two passes: a statistics
 * pass, then a second read of the row for the output (any width; the
 * non-retaining baseline); 3 = retained, pipelined: one round of resident
 * workgroups, each taking rows / (workgroups the GPU holds at once) rows (at
 * least 2) in turn, keeping each in registers and loading the next while it
 * reduces and writes the current one (LayerNorm: gamma and beta stay in
 * registers across its rows); HBM traffic as for 1 (width <= 65536,
 * CAP_ERR_UNSUPPORTED above; rows too wide to be held twice run as 1).
 * Results are deterministic for a given (mode, width); modes 1 and 3 may
 * differ in the last bits, since they may split a row over a different
 * number of lanes.
 *
 * Errors: CAP_ERR_INVALID_ARG (NULL pointer, rows < 0, width < 1, bad mode,
 * partial overlap of x and y, eps negative or not finite), CAP_ERR_UNSUPPORTED
 * (rows >= 2^31, width > 2^24, mode 1 above 65536), CAP_ERR_HIP (launch).
 * rows = 0 launches nothing.
 */
#ifndef CAP_ROWS_H
#define CAP_ROWS_H

#include "cap.h"

#ifdef __cplusplus
extern "C" {
#endif

cap_status cap_rows_softmax(const float *x, float *y, int64_t rows, int64_t width, int32_t mode,
                            cap_stream_t stream);

cap_status cap_rows_layernorm(const float *x, const float *gamma, const float *beta, float *y,
                              int64_t rows, int64_t width, float eps, int32_t mode,
                              cap_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* CAP_ROWS_H */
