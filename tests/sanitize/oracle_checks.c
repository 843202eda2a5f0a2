/* Host build of the CPU oracle under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitizers.py): every entry point on
 * small shapes, empty ones and rejected arguments, plus closed forms that a
 * memory or indexing error would break (grad_proj = 0 leaves the RMS term;
 * a one-hot P copies a row of X into dW).  Exits non-zero on a failure. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

double oracle_tf32(float v);
float oracle_bf16(float v);
int oracle_dx(int mode, int64_t rows, int64_t cols, int64_t K, const float *x, const float *w,
              const float *grad_proj, const float *grad_r, const float *r,
              const uint16_t *addend, double *dx);
int oracle_dw(int mode, int64_t rows, int64_t cols, const float *x, const float *grad_proj,
              double *dw);
int oracle_forward(int mode, int64_t rows, int64_t K, const float *x, const float *w,
                   double eps, double *proj, double *r);
int oracle_rmsnorm_backward(int64_t rows, int64_t H, const uint16_t *g, const uint16_t *x,
                            const float *w, const float *rstd, const uint16_t *res, double *dx,
                            double *dw);

static int fail = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); fail = 1; } } while (0)

static uint32_t lcg = 12345u;
static float rnd(void) { lcg = lcg * 1664525u + 1013904223u; return (float)((lcg >> 8) & 0xFFFF) / 32768.0f - 1.0f; }

int main(void) {
    for (int mode = 0; mode < 2; ++mode) {
        for (int64_t rows = 0; rows < 6; ++rows) {
            for (int64_t cols = 0; cols < 40; cols += 13) {
                float *x = malloc(sizeof(float) * (rows * cols + 1));
                float *w = malloc(sizeof(float) * (24 * cols + 1));
                float *gp = malloc(sizeof(float) * (rows * 32 + 1));
                float *gr = malloc(sizeof(float) * (rows + 1));
                float *r = malloc(sizeof(float) * (rows + 1));
                uint16_t *ad = malloc(sizeof(uint16_t) * (rows * cols + 1));
                double *dx = malloc(sizeof(double) * (rows * cols + 1));
                double *dw = malloc(sizeof(double) * (24 * cols + 1));
                double *proj = malloc(sizeof(double) * (rows * 24 + 1));
                double *rr = malloc(sizeof(double) * (rows + 1));
                for (int64_t i = 0; i < rows * cols; ++i) { x[i] = rnd(); ad[i] = (uint16_t)(lcg >> 16); }
                for (int64_t i = 0; i < 24 * cols; ++i) w[i] = rnd();
                for (int64_t i = 0; i < rows * 32; ++i) gp[i] = (i % 32) < 24 ? 0.0f : NAN;
                for (int64_t i = 0; i < rows; ++i) { gr[i] = rnd(); r[i] = 1.0f + fabsf(rnd()); }
                const int64_t K = cols > 0 ? cols : 1;
                CHECK(oracle_dx(mode, rows, cols, K, x, w, gp, gr, r, NULL, dx) == 0);
                for (int64_t t = 0; t < rows; ++t)
                    for (int64_t k = 0; k < cols; ++k)
                        CHECK(dx[t * cols + k] == (double)gr[t] / ((double)r[t] * (double)K) * (double)x[t * cols + k]);
                CHECK(oracle_dx(mode, rows, cols, K, x, w, gp, gr, r, ad, dx) == 0);
                /* one-hot P in column 5 of row 0: dW[5, :] = x[0, :] (rounded in mode 1) */
                if (rows > 0) gp[5] = 1.0f;
                CHECK(oracle_dw(mode, rows, cols, x, gp, dw) == 0);
                for (int64_t k = 0; k < cols && rows > 0; ++k)
                    CHECK(dw[5 * cols + k] == (mode ? oracle_tf32(x[k]) : (double)x[k]));
                if (cols > 0) CHECK(oracle_forward(mode, rows, cols, x, w, 1e-6, proj, rr) == 0);
                free(x); free(w); free(gp); free(gr); free(r); free(ad); free(dx); free(dw);
                free(proj); free(rr);
            }
        }
    }
    CHECK(oracle_dx(2, 1, 1, 1, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == -1);
    CHECK(oracle_dw(-1, 1, 1, NULL, NULL, NULL) == -1);
    CHECK(oracle_forward(0, 1, 0, NULL, NULL, 0.0, NULL, NULL) == -1);
    CHECK(oracle_forward(0, 1, 1, NULL, NULL, -1.0, NULL, NULL) == -1);
    /* RMSNorm backward: small rows with and without the residual */
    for (int64_t rows = 0; rows < 4; ++rows) {
        const int64_t H = 24;
        uint16_t *g = malloc(2 * (rows * H + 1)), *xb = malloc(2 * (rows * H + 1)), *res = malloc(2 * (rows * H + 1));
        float *w = malloc(4 * H), *rstd = malloc(4 * (rows + 1));
        double *dx = malloc(8 * (rows * H + 1)), *dw = malloc(8 * H);
        for (int64_t i = 0; i < rows * H; ++i) { g[i] = 0x3F80; xb[i] = 0x3F80; res[i] = 0x0000; }
        for (int64_t h = 0; h < H; ++h) w[h] = 1.0f;
        for (int64_t t = 0; t < rows; ++t) rstd[t] = 1.0f;
        CHECK(oracle_rmsnorm_backward(rows, H, g, xb, w, rstd, NULL, dx, dw) == 0);
        /* constant rows of ones with rstd = 1: dx = 1 - 1 = 0, dw = rows */
        for (int64_t i = 0; i < rows * H; ++i) CHECK(dx[i] == 0.0);
        for (int64_t h = 0; h < H; ++h) CHECK(dw[h] == (double)rows);
        CHECK(oracle_rmsnorm_backward(rows, H, g, xb, w, rstd, res, dx, dw) == 0);
        free(g); free(xb); free(res); free(w); free(rstd); free(dx); free(dw);
    }
    CHECK(oracle_rmsnorm_backward(1, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == -1);
    CHECK(oracle_bf16(1.0f) == 1.0f && oracle_tf32(1.0f) == 1.0);
    printf(fail ? "oracle checks FAILED\n" : "oracle checks passed\n");
    return fail;
}
