/*
 * mhcpb_oracle.c -- CPU oracle for the DSv4.1 mHC projection/RMS backward.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow FP64 definition
 * that the GPU library is checked against.  Only the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark may load it; the library
 * never does, and the two share no code, headers or tables.
 *
 * What it follows ("DSv4.1 mHC projection/RMS backward", cuDNN Frontend
 * page, introduction and "Requirements and tensor contract"):
 *
 *   P  = grad_proj[:, :24]          (the last 8 of 32 columns are never read)
 *   dX = P W + grad_r / (r K) * X   (rank-24 product plus the RMS term)
 *   dW = P^T X
 *
 * The page says the two products take TF32 operands and accumulate in FP32,
 * while the RMS term is FP32 arithmetic.  The oracle evaluates everything in
 * FP64 with no final rounding, in one of two modes:
 *   mode 0 (exact): the FP32 inputs are widened exactly;
 *   mode 1 (tf32):  P, W (for dX) and P, X (for dW) are first rounded to
 *                   TF32 (the 23-bit FP32 fraction rounded to nearest-even at
 *                   10 bits, the carry allowed into the exponent).
 * In both modes the RMS term uses the unrounded x.  The optional BF16
 * grad_x_addend (prime-kernels pull request 15, "FP8 weight cache, split
 * backward, fused mHC stream gradient" section) is added to dX exactly.
 *
 * oracle_forward is the map whose gradient these are: the 24 gate logits
 * X W^T (TF32 operands in mode 1) and the row RMS sqrt(mean(x^2) + eps) in
 * FP32-range arithmetic on the raw x (see its own comment).
 *
 * oracle_rmsnorm_backward is a second workload (see its own comment).
 *
 * Rounding here is done arithmetically (frexp / ldexp / nearbyint under
 * round-to-nearest-even), deliberately not by bit manipulation.
 *
 * Parity pins: every function below is pinned by tests/test_oracle.py
 * (finite-difference VJP of the forward map, a float64 autograd cross-check,
 * hand-derived TF32/BF16 bit tables in tests/golden/, one-hot cases,
 * invariants).  The general FP32 bits of the GPU result (its accumulation
 * order) are "parity unpinned": they are covered only by tolerances.
 */
#include <fenv.h>
#include <float.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_PROJ_COLS 24      /* columns of grad_proj that take part     */
#define ORACLE_PROJ_STRIDE 32    /* row length of grad_proj                  */

/* Round a finite FP32 value, given as a double, to `bits` significant bits of
 * an FP32-style format whose fraction field is cut to (bits - 1) bits:
 * normal values keep `bits` significant bits, subnormal values keep the
 * quantum of the cut fraction field (2^(-149 + 24 - bits)).  Ties go to even.
 * A result at or above 2^128 overflows to infinity.  NaN and infinities pass
 * through unchanged. */
static double round_fp32_format(double v, int bits)
{
    if (isnan(v) || isinf(v) || v == 0.0)
        return v;
    double a = fabs(v);
    double quantum;
    if (a < 0x1p-126) {
        quantum = ldexp(1.0, -149 + 24 - bits);
    } else {
        int e;
        (void)frexp(a, &e);          /* a = m * 2^e with 0.5 <= m < 1 */
        quantum = ldexp(1.0, e - bits);
    }
    double q = nearbyint(v / quantum) * quantum;  /* v / quantum is exact */
    if (fabs(q) >= 0x1p128)
        q = copysign(INFINITY, v);
    return q;
}

/* TF32 value of an FP32 input: 11 significant bits (10 fraction bits). */
static double tf32_of(float v)
{
    return round_fp32_format((double)v, 11);
}

double oracle_tf32(float v)
{
    fesetround(FE_TONEAREST);
    return tf32_of(v);
}

/* BF16 value of an FP32 input: 8 significant bits (7 fraction bits),
 * round to nearest even.  Returned as a float (every BF16 value is one). */
float oracle_bf16(float v)
{
    fesetround(FE_TONEAREST);
    if (isnan(v))
        return v;
    return (float)round_fp32_format((double)v, 8);
}

/* Widen BF16 bits to a double. */
static double bf16_bits_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double operand(float v, int mode)
{
    return mode == 1 ? tf32_of(v) : (double)v;
}

/*
 * dX for `rows` tokens and `cols` columns of the full K-wide row.
 *   x        [rows, cols]  FP32, the columns of X being checked
 *   w        [24, cols]    FP32, the same columns of W
 *   grad_proj[rows, 32]    FP32, only columns 0..23 are read
 *   grad_r   [rows], r [rows]
 *   addend   [rows, cols]  BF16 bits, or NULL
 *   K        full row width (streams * hidden) used in grad_r / (r K)
 *   dx       [rows, cols]  FP64 out
 */
int oracle_dx(int mode, int64_t rows, int64_t cols, int64_t K,
              const float *x, const float *w, const float *grad_proj,
              const float *grad_r, const float *r, const uint16_t *addend,
              double *dx)
{
    if (mode != 0 && mode != 1)
        return -1;
    if (rows < 0 || cols < 0 || K <= 0)
        return -1;
    fesetround(FE_TONEAREST);
    for (int64_t t = 0; t < rows; ++t) {
        /* RMS coefficient grad_r / (r K), in FP64 */
        double c = (double)grad_r[t] / ((double)r[t] * (double)K);
        for (int64_t k = 0; k < cols; ++k) {
            double s = 0.0;
            for (int j = 0; j < ORACLE_PROJ_COLS; ++j)
                s += operand(grad_proj[t * ORACLE_PROJ_STRIDE + j], mode) *
                     operand(w[(int64_t)j * cols + k], mode);
            s += c * (double)x[t * cols + k];   /* raw x: the RMS term */
            if (addend)
                s += bf16_bits_to_double(addend[t * cols + k]);
            dx[t * cols + k] = s;
        }
    }
    return 0;
}

/*
 * dW for `cols` columns, summed over all `rows` tokens in ascending order.
 *   x         [rows, cols] FP32
 *   grad_proj [rows, 32]   FP32, only columns 0..23 are read
 *   dw        [24, cols]   FP64 out
 */
int oracle_dw(int mode, int64_t rows, int64_t cols,
              const float *x, const float *grad_proj, double *dw)
{
    if (mode != 0 && mode != 1)
        return -1;
    if (rows < 0 || cols < 0)
        return -1;
    fesetround(FE_TONEAREST);
    for (int j = 0; j < ORACLE_PROJ_COLS; ++j) {
        for (int64_t k = 0; k < cols; ++k) {
            double s = 0.0;
            for (int64_t t = 0; t < rows; ++t)
                s += operand(grad_proj[t * ORACLE_PROJ_STRIDE + j], mode) *
                     operand(x[t * cols + k], mode);
            dw[(int64_t)j * cols + k] = s;
        }
    }
    return 0;
}

/*
 * The forward map of the stage: the 24 gate logits and the RMS of each row,
 * in one pass over X.
 *
 * The backward page ("DSv4.1 mHC projection/RMS backward", introduction and
 * "Requirements and tensor contract") takes r as the RMS "from forward" and
 * defines dX = P W + grad_r / (r K) X and dW = P^T X: exactly the gradient of
 *
 *   proj[t, j] = sum_k X[t, k] W[j, k]            (j < 24)
 *   r[t]       = sqrt(sum_k X[t, k]^2 / K + eps)
 *
 * with respect to X and W, since d r / d X[t, k] = X[t, k] / (r K).  The
 * prime-kernels pull request 15 page (its list of kernels, "mhc_projection")
 * computes the RMS and the gate logits of the streams in one read.  Where
 * the normalisation by r is applied to the logits is not printed; the
 * backward's separate grad_proj and grad_r mean the logits leave this map
 * unnormalised, and that is the reading taken here.  As in the backward the
 * product takes TF32 operands (mode 1) or the exact FP32 inputs (mode 0);
 * the RMS always uses the raw FP32 x.  Everything is evaluated in FP64 with
 * no final rounding, except one fact of the FP32 arithmetic the RMS is
 * defined in: a sum of squares beyond the FP32 range makes r infinite.
 *
 *   x    [rows, K]  FP32
 *   w    [24, K]    FP32
 *   eps  the RMS epsilon (finite, >= 0)
 *   proj [rows, 24] FP64 out
 *   r    [rows]     FP64 out
 */
int oracle_forward(int mode, int64_t rows, int64_t K, const float *x,
                   const float *w, double eps, double *proj, double *r)
{
    if (mode != 0 && mode != 1)
        return -1;
    if (rows < 0 || K <= 0 || !(eps >= 0.0) || isinf(eps))
        return -1;
    fesetround(FE_TONEAREST);
    for (int64_t t = 0; t < rows; ++t) {
        const float *xt = x + t * K;
        for (int j = 0; j < ORACLE_PROJ_COLS; ++j) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k)
                s += operand(xt[k], mode) * operand(w[(int64_t)j * K + k], mode);
            proj[t * ORACLE_PROJ_COLS + j] = s;
        }
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k)
            ss += (double)xt[k] * (double)xt[k];
        if (ss > (double)FLT_MAX)
            ss = INFINITY;
        r[t] = sqrt(ss / (double)K + eps);
    }
    return 0;
}

/*
 * A second workload: the backward of a BF16 RMSNorm, y = x * rstd * w per
 * row, rstd = 1 / sqrt(mean(x^2) + eps) given by the forward
 * ("flashinfer.cake_rmsnorm_det_train.cake_rmsnorm_det_train_backward" page,
 * its signature and parameter list: BF16 g and x, BF16 or FP32 w, FP32 rstd,
 * optional BF16 g_residual added once, BF16 dx and FP32 dw).  The page does
 * not print the formula; this is the textbook gradient of that map with rstd
 * taken as the forward gave it:
 *
 *   c1[t]   = sum_h w[h] g[t,h] x[t,h] / H
 *   dx[t,h] = rstd[t] w[h] g[t,h] - rstd[t]^3 c1[t] x[t,h]  [+ g_residual]
 *   dw[h]   = sum_t g[t,h] x[t,h] rstd[t]
 *
 * (rstd depends on x: d rstd / d x[t,h] = -rstd^3 x[t,h] / H.)  Evaluated in
 * FP64 from the exact input values, no final rounding.
 *
 *   g, x, res  [rows, H] BF16 bits (res may be NULL)
 *   w          [H] the weight's values (BF16 or FP32, widened exactly)
 *   rstd       [rows]
 *   dx         [rows, H] FP64 out;  dw [H] FP64 out (summed over the rows)
 */
int oracle_rmsnorm_backward(int64_t rows, int64_t H, const uint16_t *g, const uint16_t *x,
                            const float *w, const float *rstd, const uint16_t *res,
                            double *dx, double *dw)
{
    if (rows < 0 || H <= 0)
        return -1;
    for (int64_t h = 0; h < H; ++h)
        dw[h] = 0.0;
    for (int64_t t = 0; t < rows; ++t) {
        const uint16_t *gt = g + t * H, *xt = x + t * H;
        double c1 = 0.0;
        for (int64_t h = 0; h < H; ++h)
            c1 += (double)w[h] * bf16_bits_to_double(gt[h]) * bf16_bits_to_double(xt[h]);
        c1 /= (double)H;
        const double rs = (double)rstd[t];
        for (int64_t h = 0; h < H; ++h) {
            const double gv = bf16_bits_to_double(gt[h]), xv = bf16_bits_to_double(xt[h]);
            double v = rs * (double)w[h] * gv - rs * rs * rs * c1 * xv;
            if (res)
                v += bf16_bits_to_double(res[t * H + h]);
            dx[t * H + h] = v;
            dw[h] += gv * xv * rs;
        }
    }
    return 0;
}
