/*
 * rowred_oracle.c -- plain FP64 CPU oracle for the fused row reductions.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file or the library built from it.  Only the test suite,
 * the package smoke check and the benchmark's CPU-baseline leg use it.  It
 * shares no code, header, table or constant with the HIP library.
 *
 * Every function takes FP32 inputs (widened exactly to double), computes in
 * FP64 with plain sequential loops in the order the definition states, and
 * writes FP64 outputs.  Rows are independent; the caller may split the row
 * range over threads by offsetting the pointers.  No state is kept.
 *
 * Sources (the pages' titles and sections):
 *  - "Residual LayerNorm shared-Tile materialization search", section
 *    "Structural finding": the residual LayerNorm program -- combined input
 *    x + residual, mean over the row, centred values, biased variance of the
 *    centred values, output centred / sqrt(variance + eps).
 *  - "Immutable input reuse in Metal reductions", section "What the
 *    transformation actually preserves": RMSNorm is one sum-of-squares
 *    reduction followed by an output map over the same input; softmax is a
 *    max phase followed by an exp-sum phase over a computed stripe and a
 *    normalising map.  The pages print no formula for either, so the plain
 *    definitions are used: RMSNorm y = x / sqrt(mean(x^2) + eps) with no
 *    weight; softmax y = exp(x - max) / sum(exp(x - max)).
 *  - "Cooperating-program packing: implementation and fixed-plan evidence",
 *    section "Validation": the operator list includes sum and paired
 *    min/max row reductions; "Immutable input reuse in Metal reductions",
 *    section "Fixed-width GPU and dispatch results", times plain (no
 *    residual) LayerNorm next to softmax and RMSNorm.
 *
 * IEEE special values propagate with no special case: a row whose entries
 * are all -inf gives NaN in softmax (-inf - -inf), a NaN input poisons its
 * row's sums, and a zero-variance row with eps = 0 gives 0/0 = NaN.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

/* Residual LayerNorm without affine parameters.  r may be NULL, which gives
 * plain LayerNorm of x.  gamma and beta may be NULL; when given they are the
 * per-column scale and shift applied after normalisation (y * gamma + beta).
 * y receives rows*width doubles.  eps is the FP32 eps widened to double. */
void rowred_oracle_layernorm(const float *x, const float *r, const float *gamma,
                             const float *beta, double *y, int64_t rows,
                             int64_t width, double eps) {
  for (int64_t i = 0; i < rows; ++i) {
    const float *xi = x + i * width;
    const float *ri = r ? r + i * width : NULL;
    double *yi = y + i * width;
    /* combined = x + residual */
    for (int64_t j = 0; j < width; ++j)
      yi[j] = (double)xi[j] + (ri ? (double)ri[j] : 0.0);
    /* mean = sum(combined) / width */
    double sum = 0.0;
    for (int64_t j = 0; j < width; ++j) sum += yi[j];
    double mean = sum / (double)width;
    /* centered = combined - mean */
    for (int64_t j = 0; j < width; ++j) yi[j] = yi[j] - mean;
    /* variance = sum(centered^2) / width  (biased, second pass) */
    double sq = 0.0;
    for (int64_t j = 0; j < width; ++j) sq += yi[j] * yi[j];
    double var = sq / (double)width;
    /* y = centered / sqrt(variance + eps) */
    double denom = sqrt(var + eps);
    for (int64_t j = 0; j < width; ++j) {
      double v = yi[j] / denom;
      if (gamma) v = v * (double)gamma[j];
      if (beta) v = v + (double)beta[j];
      yi[j] = v;
    }
  }
}

/* RMSNorm: y = x / sqrt(sum(x^2) / width + eps). */
void rowred_oracle_rmsnorm(const float *x, double *y, int64_t rows,
                           int64_t width, double eps) {
  for (int64_t i = 0; i < rows; ++i) {
    const float *xi = x + i * width;
    double *yi = y + i * width;
    double sq = 0.0;
    for (int64_t j = 0; j < width; ++j) sq += (double)xi[j] * (double)xi[j];
    double ms = sq / (double)width;
    double denom = sqrt(ms + eps);
    for (int64_t j = 0; j < width; ++j) yi[j] = (double)xi[j] / denom;
  }
}

/* Softmax with max subtraction: m = max x, e = exp(x - m), y = e / sum(e). */
void rowred_oracle_softmax(const float *x, double *y, int64_t rows,
                           int64_t width) {
  for (int64_t i = 0; i < rows; ++i) {
    const float *xi = x + i * width;
    double *yi = y + i * width;
    double m = -INFINITY;
    for (int64_t j = 0; j < width; ++j) m = fmax(m, (double)xi[j]);
    double s = 0.0;
    for (int64_t j = 0; j < width; ++j) {
      yi[j] = exp((double)xi[j] - m);
      s += yi[j];
    }
    for (int64_t j = 0; j < width; ++j) yi[j] = yi[j] / s;
  }
}

/* Row sum: out[i] = sum_j x[i][j]. */
void rowred_oracle_row_sum(const float *x, double *out, int64_t rows,
                           int64_t width) {
  for (int64_t i = 0; i < rows; ++i) {
    const float *xi = x + i * width;
    double s = 0.0;
    for (int64_t j = 0; j < width; ++j) s += (double)xi[j];
    out[i] = s;
  }
}

/* Paired row min/max: out_min[i] = min_j x[i][j], out_max[i] = max_j x[i][j].
 * NaN entries are skipped (fmin/fmax semantics); an empty row gives
 * (+inf, -inf), the identities of the two reductions. */
void rowred_oracle_row_minmax(const float *x, double *out_min, double *out_max,
                              int64_t rows, int64_t width) {
  for (int64_t i = 0; i < rows; ++i) {
    const float *xi = x + i * width;
    double lo = INFINITY, hi = -INFINITY;
    for (int64_t j = 0; j < width; ++j) {
      lo = fmin(lo, (double)xi[j]);
      hi = fmax(hi, (double)xi[j]);
    }
    out_min[i] = lo;
    out_max[i] = hi;
  }
}
