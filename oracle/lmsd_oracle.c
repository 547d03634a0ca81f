/*
 * HSTU LMSD oracle: a plain, slow fp64 CPU implementation.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or load
 * this file; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark use it.  It shares no code with the HIP kernels.
 *
 * What it computes is the definition on the "HSTU LayerNorm-Multiply-SiLU-
 * Dropout (LMSD)" page ("Overview", the displayed equations), per row of x and
 * u (N rows of D values), with dropout off (ratio 0, where the page says the
 * dropout work is compiled out):
 *
 *     mean = sum_d x_d / D,   var = sum_d (x_d - mean)^2 / D,
 *     rstd = 1 / sqrt(var + eps),   xh = (x - mean) rstd,
 *     l = xh * weight + bias,   a = SiLU(u) or u,
 *     y = [a if concat_u, x if concat_x, l * a]          (segments of D)
 *
 * and the page's explicit backward (its inputs: dy, x, u, weight, bias and the
 * saved mean and rstd), by the chain rule on those equations, with g the
 * gradient of the l * a segment, ga of the a segment and gx of the x segment:
 *
 *     dl = g a,   da = g l (+ ga),   du = da SiLU'(u) or da,
 *     dweight = sum_rows dl xh,   dbias = sum_rows dl,
 *     dxh = dl weight,
 *     dx = rstd (dxh - mean_d(dxh) - xh mean_d(dxh xh)) (+ gx).
 *
 * Readings where the page is silent (each is listed in the design notes): the
 * variance is the biased (1/D) one of LayerNorm; the backward recomputes xh
 * from the saved mean and rstd (it is given those, not xh).  Rows are
 * independent and spread over OpenMP threads; the column sums of dweight and
 * dbias run over rows in order, in fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>

static inline double silu(double s) { return s / (1.0 + exp(-s)); }
static inline double dsilu(double s) {
    const double sg = 1.0 / (1.0 + exp(-s));
    return sg * (1.0 + s * (1.0 - sg));
}

/* Forward.  x, u: (n, d) with row strides xs, us; w, b: (d); y: (n, s d)
 * contiguous, s = 1 + concat_u + concat_x; mean, rstd: (n). */
void oracle_lmsd_fwd(int64_t n, int64_t d, const double* x, int64_t xs, const double* u, int64_t us,
                     const double* w, const double* b, double eps, int silu_u, int concat_u, int concat_x,
                     double* y, double* mean, double* rstd) {
    const int64_t s = 1 + (concat_u != 0) + (concat_x != 0);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        const double* xr = x + r * xs;
        const double* ur = u + r * us;
        double m = 0.0;
        for (int64_t j = 0; j < d; ++j) m += xr[j];
        m /= (double)d;
        double v = 0.0;
        for (int64_t j = 0; j < d; ++j) v += (xr[j] - m) * (xr[j] - m);
        v /= (double)d;
        const double rs = 1.0 / sqrt(v + eps);
        mean[r] = m;
        rstd[r] = rs;
        double* yr = y + r * s * d;
        int64_t seg = 0;
        if (concat_u) {
            for (int64_t j = 0; j < d; ++j) yr[j] = silu_u ? silu(ur[j]) : ur[j];
            ++seg;
        }
        if (concat_x) {
            for (int64_t j = 0; j < d; ++j) yr[seg * d + j] = xr[j];
            ++seg;
        }
        for (int64_t j = 0; j < d; ++j) {
            const double l = (xr[j] - m) * rs * w[j] + b[j];
            const double a = silu_u ? silu(ur[j]) : ur[j];
            yr[seg * d + j] = l * a;
        }
    }
}

/* Backward.  dy: (n, s d) with row stride dys; mean, rstd as saved by the
 * forward; dx, du: (n, d) contiguous; dw, db: (d). */
void oracle_lmsd_bwd(int64_t n, int64_t d, const double* dy, int64_t dys, const double* x, int64_t xs,
                     const double* u, int64_t us, const double* w, const double* b, const double* mean,
                     const double* rstd, int silu_u, int concat_u, int concat_x, double* dx, double* du,
                     double* dw, double* db) {
    const int64_t gseg = (concat_u != 0) + (concat_x != 0);  /* index of the l * a segment */
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        const double* xr = x + r * xs;
        const double* ur = u + r * us;
        const double* g = dy + r * dys + gseg * d;
        double s1 = 0.0, s2 = 0.0;  /* sum dxh, sum dxh xh */
        for (int64_t j = 0; j < d; ++j) {
            const double xh = (xr[j] - mean[r]) * rstd[r];
            const double a = silu_u ? silu(ur[j]) : ur[j];
            const double dxh = g[j] * a * w[j];
            s1 += dxh;
            s2 += dxh * xh;
        }
        for (int64_t j = 0; j < d; ++j) {
            const double xh = (xr[j] - mean[r]) * rstd[r];
            const double l = xh * w[j] + b[j];
            const double a = silu_u ? silu(ur[j]) : ur[j];
            const double dxh = g[j] * a * w[j];
            double gx = dxh - s1 / (double)d - xh * s2 / (double)d;
            gx *= rstd[r];
            double da = g[j] * l;
            if (concat_u) da += dy[r * dys + j];
            if (concat_x) gx += dy[r * dys + (concat_u ? d : 0) + j];
            dx[r * d + j] = gx;
            du[r * d + j] = silu_u ? da * dsilu(ur[j]) : da;
        }
    }
    for (int64_t j = 0; j < d; ++j) {
        double sw = 0.0, sb = 0.0;
        for (int64_t r = 0; r < n; ++r) {
            const double xh = (x[r * xs + j] - mean[r]) * rstd[r];
            const double a = silu_u ? silu(u[r * us + j]) : u[r * us + j];
            const double dl = dy[r * dys + gseg * d + j] * a;
            sw += dl * xh;
            sb += dl;
        }
        dw[j] = sw;
        db[j] = sb;
    }
}
