/*
 * Plain fp64 CPU oracle for In-Place Activated BatchNorm (InPlace-ABN).
 *
 * TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's CPU
 * baseline call it; the product library never does.  It shares no code, header,
 * table or constant with the HIP implementation.
 *
 * Source pages: "In-Place Activated BatchNorm for Memory-Optimized Training of
 * DNNs" (Rota Bulo, Porzi, Kontschieder), read from the paperlayer summary of
 * arXiv 1712.02616v3, section 3 ("In-Place Activated Batch Normalization") and
 * the Appendix ("Derivation of Gradient"), plus the abstract on the
 * codewithpapers and cochat pages.  Batch normalisation itself is the method of
 * Ioffe & Szegedy, which the cochat page lists among the works cited.
 *
 * Every tensor here is logical NCHW, fp64, contiguous: element (n, c, i), with
 * i = h*W + w, sits at index (n*C + c)*HW + i.  Every loop runs in the order of
 * the definition it implements; the only parallelism is one OpenMP thread per
 * channel, which does not change any channel's arithmetic.
 *
 * Readings taken where the pages are silent:
 *   - the normalising variance is the biased one, 1/m (section 3, "Batch
 *     Normalization Review": "empirical mean and variance");
 *   - eps sits inside the root: invstd = 1/sqrt(var + eps);
 *   - running statistics: new = (1 - momentum)*old + momentum*batch, with the
 *     unbiased variance var*m/(m-1) for the running variance;
 *   - the activation branches on z > 0 going forward and on y > 0 going
 *     backward; at exactly zero both inverses give z = 0;
 *   - the ELU inverse clamps y/alpha to at least -1 + 2^-24 (only reachable
 *     through rounding of the stored y).
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_ACT_IDENTITY 0
#define ORC_ACT_LEAKY_RELU 1
#define ORC_ACT_ELU 2

#define ORC_STORE_F64 0
#define ORC_STORE_F32 1
#define ORC_STORE_BF16 2
#define ORC_STORE_F16 3

/* ---------------------------------------------------------------------------
 * Invertible activations (section 3, "INPLACE-ABN": the activation must be
 * invertible; section 4, "Experimental setup": leaky ReLU with slope 0.01).
 * ELU is not on the pages; it is the second strictly monotone activation the
 * workloads ask for.
 */

/* y = act(z) */
static double act_forward(int act, double p, double z)
{
    switch (act) {
    case ORC_ACT_LEAKY_RELU: return z > 0.0 ? z : p * z;
    case ORC_ACT_ELU:        return z > 0.0 ? z : p * expm1(z);
    default:                 return z;
    }
}

/* z = act^-1(y): recover the pre-activation from the stored output. */
static double act_inverse(int act, double p, double y)
{
    switch (act) {
    case ORC_ACT_LEAKY_RELU: return y > 0.0 ? y : y / p;
    case ORC_ACT_ELU: {
        if (y > 0.0) return y;
        double u = y / p;
        const double lo = -1.0 + 5.9604644775390625e-08; /* -1 + 2^-24 */
        if (u < lo) u = lo;
        return log1p(u);
    }
    default: return y;
    }
}

/* act'(z), written as a function of y = act(z). */
static double act_derivative_from_y(int act, double p, double y)
{
    switch (act) {
    case ORC_ACT_LEAKY_RELU: return y > 0.0 ? 1.0 : p;
    case ORC_ACT_ELU:        return y > 0.0 ? 1.0 : y + p;   /* p*exp(z) = y + p */
    default:                 return 1.0;
    }
}

/* act'(z), written as a function of z (the conventional block keeps z). */
static double act_derivative_from_z(int act, double p, double z)
{
    switch (act) {
    case ORC_ACT_LEAKY_RELU: return z > 0.0 ? 1.0 : p;
    case ORC_ACT_ELU:        return z > 0.0 ? 1.0 : p * exp(z);
    default:                 return 1.0;
    }
}

static int act_valid(int act, double p)
{
    if (act == ORC_ACT_IDENTITY) return 1;
    if (act == ORC_ACT_LEAKY_RELU || act == ORC_ACT_ELU) return p > 0.0 && isfinite(p);
    return 0;
}

#define AT(n, c, i) ((((int64_t)(n)) * C + (c)) * HW + (i))

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Statistics of channel c (section 3, "Batch Normalization Review"): the mean,
 * the biased variance (two passes) and 1/sqrt(var + eps). */
static void channel_stats(int64_t N, int64_t C, int64_t HW, const double *x, int64_t c,
                          double eps, double *mu_out, double *v_out, double *is_out)
{
    const int64_t m = N * HW;
    double sum = 0.0;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t i = 0; i < HW; ++i) sum += x[AT(n, c, i)];
    const double mu = sum / (double)m;

    double ss = 0.0;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t i = 0; i < HW; ++i) {
            const double d = x[AT(n, c, i)] - mu;
            ss += d * d;
        }
    const double v = ss / (double)m;
    const double is = 1.0 / sqrt(v + eps);
    *mu_out = mu;
    *v_out = v;
    *is_out = is;
}

/* The running statistics of channel c after one training step (when given). */
static void update_running(int64_t c, int64_t m, double momentum, double mu, double v,
                           double *running_mean, double *running_var)
{
    if (running_mean)
        running_mean[c] = (1.0 - momentum) * running_mean[c] + momentum * mu;
    if (running_var)
        running_var[c] = (1.0 - momentum) * running_var[c]
                       + momentum * v * (double)m / (double)(m - 1);
}

/* ---------------------------------------------------------------------------
 * Training forward (section 3, "Batch Normalization Review" and "INPLACE-ABN"):
 *   mu_c = (1/m) sum x,   var_c = (1/m) sum (x - mu_c)^2   (two passes),
 *   xhat = (x - mu_c) / sqrt(var_c + eps),   z = gamma_c xhat + beta_c,
 *   y = act(z).
 * Outputs y (fp64, not rounded), mean, var (biased), invstd; updates the running
 * statistics when they are given.  Returns 0, or -1 for invalid arguments.
 */
int orc_forward_train(int64_t N, int64_t C, int64_t HW,
                      const double *x, const double *gamma, const double *beta,
                      int act, double p, double eps, double momentum,
                      double *y, double *mean, double *var, double *invstd,
                      double *running_mean, double *running_var)
{
    const int64_t m = N * HW;
    if (C < 0 || m < 2 || !act_valid(act, p) || !(eps >= 0.0)) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < C; ++c) {
        double mu, v, is;
        channel_stats(N, C, HW, x, c, eps, &mu, &v, &is);
        for (int64_t n = 0; n < N; ++n)
            for (int64_t i = 0; i < HW; ++i) {
                const double xhat = (x[AT(n, c, i)] - mu) * is;
                const double z = gamma[c] * xhat + beta[c];
                y[AT(n, c, i)] = act_forward(act, p, z);
            }
        if (mean) mean[c] = mu;
        if (var) var[c] = v;
        if (invstd) invstd[c] = is;
        update_running(c, m, momentum, mu, v, running_mean, running_var);
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Inference forward: the same scale-and-shift and activation, with the running
 * statistics in place of the batch statistics.
 *   y = act(gamma_c (x - rm_c) / sqrt(rv_c + eps) + beta_c)
 */
int orc_forward_eval(int64_t N, int64_t C, int64_t HW,
                     const double *x, const double *gamma, const double *beta,
                     const double *running_mean, const double *running_var,
                     int act, double p, double eps, double *y)
{
    if (C < 0 || N < 0 || HW < 0 || !act_valid(act, p) || !(eps >= 0.0)) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < C; ++c) {
        const double is = 1.0 / sqrt(running_var[c] + eps);
        for (int64_t n = 0; n < N; ++n)
            for (int64_t i = 0; i < HW; ++i) {
                const double xhat = (x[AT(n, c, i)] - running_mean[c]) * is;
                y[AT(n, c, i)] = act_forward(act, p, gamma[c] * xhat + beta[c]);
            }
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Backward from the stored output y alone (section 3, "INPLACE-ABN": invert the
 * activation and the scale-and-shift; Appendix: discarded buffers are rebuilt
 * during the backward pass).  Form I:
 *   z = act^-1(y),  dz = act'(z) dy,  xhat = (z - beta_c) / gamma_c,
 *   dbeta_c = sum dz,  dgamma_c = sum dz xhat,
 *   dx = gamma_c invstd_c (dz - dbeta_c/m - xhat dgamma_c/m).
 * invstd is an input: the value the forward pass saved.  xhat_out (nullable)
 * receives the reconstructed xhat.
 */
int orc_backward_from_y(int64_t N, int64_t C, int64_t HW,
                        const double *y, const double *dy,
                        const double *gamma, const double *beta, const double *invstd,
                        int act, double p,
                        double *dx, double *dgamma, double *dbeta, double *xhat_out)
{
    const int64_t m = N * HW;
    if (C < 0 || m < 1 || !act_valid(act, p)) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < C; ++c) {
        double sdz = 0.0, sdzx = 0.0;
        for (int64_t n = 0; n < N; ++n)
            for (int64_t i = 0; i < HW; ++i) {
                const double yy = y[AT(n, c, i)];
                const double z = act_inverse(act, p, yy);
                const double dz = act_derivative_from_y(act, p, yy) * dy[AT(n, c, i)];
                const double xhat = (z - beta[c]) / gamma[c];
                sdz += dz;
                sdzx += dz * xhat;
            }
        dbeta[c] = sdz;
        dgamma[c] = sdzx;
        const double k = gamma[c] * invstd[c];
        for (int64_t n = 0; n < N; ++n)
            for (int64_t i = 0; i < HW; ++i) {
                const double yy = y[AT(n, c, i)];
                const double z = act_inverse(act, p, yy);
                const double dz = act_derivative_from_y(act, p, yy) * dy[AT(n, c, i)];
                const double xhat = (z - beta[c]) / gamma[c];
                dx[AT(n, c, i)] = k * (dz - sdz / (double)m - xhat * sdzx / (double)m);
                if (xhat_out) xhat_out[AT(n, c, i)] = xhat;
            }
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Backward through the inference forward, with the normalisation statistics
 * frozen: the running mean and variance are constants of the layer, as in the
 * "Eval mode" of a pre-trained network being fine-tuned (the "Problem" section
 * of the page "Efficient ConvBN Blocks for Transfer Learning and Beyond").  It is
 * the chain rule of orc_forward_eval, taken from the stored output y:
 *   z = act^-1(y),  dz = act'(z) dy,  xhat = (z - beta_c) / gamma_c,
 *   dx = gamma_c dz / sqrt(running_var_c + eps),
 *   dbeta_c = sum dz,  dgamma_c = sum dz xhat.
 * No term through the batch statistics: here they are not functions of x.
 */
int orc_backward_eval(int64_t N, int64_t C, int64_t HW,
                      const double *y, const double *dy,
                      const double *gamma, const double *beta, const double *running_var,
                      double eps, int act, double p,
                      double *dx, double *dgamma, double *dbeta)
{
    if (C < 0 || N < 0 || HW < 0 || !act_valid(act, p) || !(eps >= 0.0)) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < C; ++c) {
        const double k = gamma[c] / sqrt(running_var[c] + eps);
        double sdz = 0.0, sdzx = 0.0;
        for (int64_t n = 0; n < N; ++n)
            for (int64_t i = 0; i < HW; ++i) {
                const double yy = y[AT(n, c, i)];
                const double z = act_inverse(act, p, yy);
                const double dz = act_derivative_from_y(act, p, yy) * dy[AT(n, c, i)];
                sdz += dz;
                sdzx += dz * (z - beta[c]) / gamma[c];
                dx[AT(n, c, i)] = k * dz;
            }
        dbeta[c] = sdz;
        dgamma[c] = sdzx;
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Form II (section 3, "INPLACE-ABN" II): the gradients written directly in
 * terms of z = act^-1(y), so the affine recovery becomes per-channel constants:
 *   dbeta_c = sum dz,
 *   dgamma_c = (sum dz z - beta_c sum dz) / gamma_c,
 *   dx = invstd_c (gamma_c dz - z dgamma_c/m + (beta_c dgamma_c - gamma_c dbeta_c)/m).
 * Equal to form I in exact arithmetic.
 */
int orc_backward_from_y_form2(int64_t N, int64_t C, int64_t HW,
                              const double *y, const double *dy,
                              const double *gamma, const double *beta, const double *invstd,
                              int act, double p,
                              double *dx, double *dgamma, double *dbeta)
{
    const int64_t m = N * HW;
    if (C < 0 || m < 1 || !act_valid(act, p)) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < C; ++c) {
        double sdz = 0.0, sdzz = 0.0;
        for (int64_t n = 0; n < N; ++n)
            for (int64_t i = 0; i < HW; ++i) {
                const double yy = y[AT(n, c, i)];
                const double z = act_inverse(act, p, yy);
                const double dz = act_derivative_from_y(act, p, yy) * dy[AT(n, c, i)];
                sdz += dz;
                sdzz += dz * z;
            }
        const double db = sdz;
        const double dg = (sdzz - beta[c] * sdz) / gamma[c];
        dbeta[c] = db;
        dgamma[c] = dg;
        const double k0 = (beta[c] * dg - gamma[c] * db) / (double)m;
        for (int64_t n = 0; n < N; ++n)
            for (int64_t i = 0; i < HW; ++i) {
                const double yy = y[AT(n, c, i)];
                const double z = act_inverse(act, p, yy);
                const double dz = act_derivative_from_y(act, p, yy) * dy[AT(n, c, i)];
                dx[AT(n, c, i)] = invstd[c] * (gamma[c] * dz - z * dg / (double)m + k0);
            }
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Conventional backward of a BN + activation block that keeps x (section 3,
 * "Standard and Checkpointed Computation"): recompute the statistics, xhat and
 * z from x, take dz = act'(z) dy, then the same BN gradient as form I.
 */
int orc_backward_from_x(int64_t N, int64_t C, int64_t HW,
                        const double *x, const double *dy,
                        const double *gamma, const double *beta,
                        int act, double p, double eps,
                        double *dx, double *dgamma, double *dbeta)
{
    const int64_t m = N * HW;
    if (C < 0 || m < 2 || !act_valid(act, p) || !(eps >= 0.0)) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < C; ++c) {
        double sum = 0.0;
        for (int64_t n = 0; n < N; ++n)
            for (int64_t i = 0; i < HW; ++i) sum += x[AT(n, c, i)];
        const double mu = sum / (double)m;
        double ss = 0.0;
        for (int64_t n = 0; n < N; ++n)
            for (int64_t i = 0; i < HW; ++i) {
                const double d = x[AT(n, c, i)] - mu;
                ss += d * d;
            }
        const double is = 1.0 / sqrt(ss / (double)m + eps);

        double sdz = 0.0, sdzx = 0.0;
        for (int64_t n = 0; n < N; ++n)
            for (int64_t i = 0; i < HW; ++i) {
                const double xhat = (x[AT(n, c, i)] - mu) * is;
                const double z = gamma[c] * xhat + beta[c];
                const double dz = act_derivative_from_z(act, p, z) * dy[AT(n, c, i)];
                sdz += dz;
                sdzx += dz * xhat;
            }
        dbeta[c] = sdz;
        dgamma[c] = sdzx;
        const double k = gamma[c] * is;
        for (int64_t n = 0; n < N; ++n)
            for (int64_t i = 0; i < HW; ++i) {
                const double xhat = (x[AT(n, c, i)] - mu) * is;
                const double z = gamma[c] * xhat + beta[c];
                const double dz = act_derivative_from_z(act, p, z) * dy[AT(n, c, i)];
                dx[AT(n, c, i)] = k * (dz - sdz / (double)m - xhat * sdzx / (double)m);
            }
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Optimized checkpointing (section 3, "Proposed Checkpointing"): the block
 * keeps the normalised value xhat instead of its input x.  The backward gets
 * y back by the scale-and-shift followed by the activation, and the BN
 * backward uses the stored xhat directly instead of recomputing it from x.
 *
 * Forward: the statistics as in orc_forward_train, then
 *   xhat = (x - mu_c) / sqrt(var_c + eps)   (the stored buffer),
 *   y = act(gamma_c xhat + beta_c)          (the layer output).
 * Both outputs are fp64, not rounded.  Returns 0, or -1 for invalid arguments.
 */
int orc_forward_train_ckpt(int64_t N, int64_t C, int64_t HW,
                           const double *x, const double *gamma, const double *beta,
                           int act, double p, double eps, double momentum,
                           double *xhat, double *y, double *mean, double *var, double *invstd,
                           double *running_mean, double *running_var)
{
    const int64_t m = N * HW;
    if (C < 0 || m < 2 || !act_valid(act, p) || !(eps >= 0.0)) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < C; ++c) {
        double mu, v, is;
        channel_stats(N, C, HW, x, c, eps, &mu, &v, &is);
        for (int64_t n = 0; n < N; ++n)
            for (int64_t i = 0; i < HW; ++i) {
                const double xh = (x[AT(n, c, i)] - mu) * is;
                xhat[AT(n, c, i)] = xh;
                y[AT(n, c, i)] = act_forward(act, p, gamma[c] * xh + beta[c]);
            }
        if (mean) mean[c] = mu;
        if (var) var[c] = v;
        if (invstd) invstd[c] = is;
        update_running(c, m, momentum, mu, v, running_mean, running_var);
    }
    return 0;
}

/* The layer output rebuilt from the checkpoint, before the following layer's
 * backward needs it: y = act(gamma_c xhat + beta_c). */
int orc_recompute_from_xhat(int64_t N, int64_t C, int64_t HW,
                            const double *xhat, const double *gamma, const double *beta,
                            int act, double p, double *y)
{
    if (C < 0 || N < 0 || HW < 0 || !act_valid(act, p)) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < C; ++c)
        for (int64_t n = 0; n < N; ++n)
            for (int64_t i = 0; i < HW; ++i)
                y[AT(n, c, i)] = act_forward(act, p, gamma[c] * xhat[AT(n, c, i)] + beta[c]);
    return 0;
}

/* Backward from the checkpoint:
 *   z = gamma_c xhat + beta_c,  dz = act'(z) dy,
 *   dbeta_c = sum dz,  dgamma_c = sum dz xhat,
 *   dx = gamma_c invstd_c (dz - dbeta_c/m - xhat dgamma_c/m).
 * invstd is the value the forward saved.  z is formed with one rounding (a
 * fused multiply-add), so the side of the activation's kink it falls on is that
 * of the exact gamma_c xhat + beta_c (a rounding never flips a sign); the leaky
 * ReLU's slope jumps from a to 1 there, so the branch must not depend on how z
 * is rounded. */
static double ckpt_z(double gamma, double xhat, double beta)
{
    return fma(gamma, xhat, beta);   /* one rounding: the sign of the exact value */
}

int orc_backward_from_xhat(int64_t N, int64_t C, int64_t HW,
                           const double *xhat, const double *dy,
                           const double *gamma, const double *beta, const double *invstd,
                           int act, double p,
                           double *dx, double *dgamma, double *dbeta)
{
    const int64_t m = N * HW;
    if (C < 0 || m < 1 || !act_valid(act, p)) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < C; ++c) {
        double sdz = 0.0, sdzx = 0.0;
        for (int64_t n = 0; n < N; ++n)
            for (int64_t i = 0; i < HW; ++i) {
                const double xh = xhat[AT(n, c, i)];
                const double z = ckpt_z(gamma[c], xh, beta[c]);
                const double dz = act_derivative_from_z(act, p, z) * dy[AT(n, c, i)];
                sdz += dz;
                sdzx += dz * xh;
            }
        dbeta[c] = sdz;
        dgamma[c] = sdzx;
        const double k = gamma[c] * invstd[c];
        for (int64_t n = 0; n < N; ++n)
            for (int64_t i = 0; i < HW; ++i) {
                const double xh = xhat[AT(n, c, i)];
                const double z = ckpt_z(gamma[c], xh, beta[c]);
                const double dz = act_derivative_from_z(act, p, z) * dy[AT(n, c, i)];
                dx[AT(n, c, i)] = k * (dz - sdz / (double)m - xh * sdzx / (double)m);
            }
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Storage rounding: the forward keeps y in the storage dtype, so the stored
 * value is the exact result rounded to nearest, ties to even.
 *   ORC_STORE_F64: unchanged; ORC_STORE_F32: IEEE binary32;
 *   ORC_STORE_BF16: 8 significant bits, binary32 exponent range, subnormal
 *   quantum 2^-133, overflow to infinity;
 *   ORC_STORE_F16: IEEE binary16, 11 significant bits, normal range down to
 *   2^-14, subnormal quantum 2^-24, largest finite 65504, overflow to infinity.
 */
static double round_bf16(double v)
{
    if (!isfinite(v) || v == 0.0) return v;
    const double min_normal = ldexp(1.0, -126);
    double r;
    if (fabs(v) < min_normal) {
        r = ldexp(nearbyint(ldexp(v, 133)), -133);
    } else {
        int e;
        const double f = frexp(v, &e);          /* v = f 2^e, 0.5 <= |f| < 1 */
        r = ldexp(nearbyint(ldexp(f, 8)), e - 8);
    }
    const double max_finite = ldexp(255.0, 120);  /* (2 - 2^-7) 2^127 */
    if (fabs(r) > max_finite) r = copysign(INFINITY, v);
    return r;
}

static double round_f16(double v)
{
    if (!isfinite(v) || v == 0.0) return v;
    double r;
    if (fabs(v) < ldexp(1.0, -14)) {
        r = ldexp(nearbyint(ldexp(v, 24)), -24);
    } else {
        int e;
        const double f = frexp(v, &e);          /* v = f 2^e, 0.5 <= |f| < 1 */
        r = ldexp(nearbyint(ldexp(f, 11)), e - 11);
    }
    if (fabs(r) > 65504.0) r = copysign(INFINITY, v);
    return r;
}

int orc_round_storage(double *v, int64_t count, int storage)
{
    if (storage == ORC_STORE_F64) return 0;
    if (storage != ORC_STORE_F32 && storage != ORC_STORE_BF16 && storage != ORC_STORE_F16)
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        if (storage == ORC_STORE_F32) v[i] = (double)(float)v[i];
        else if (storage == ORC_STORE_BF16) v[i] = round_bf16(v[i]);
        else v[i] = round_f16(v[i]);
    }
    return 0;
}
