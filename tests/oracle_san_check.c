/*
 * The fp64 oracle's C source under AddressSanitizer and UndefinedBehaviorSanitizer
 * (CPU only; built by tests/test_sanitizers.py).  It includes oracle/iabn_oracle.c
 * itself and calls every exported function on small random problems, the
 * degenerate sizes (m = 1, 2, empty), invalid arguments and the storage rounding
 * of special values, so that any out-of-bounds index, overflow or other undefined
 * behaviour in the oracle stops the run.  Exit status 0 when every call returned
 * what it should and every result is finite where it must be.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "../oracle/iabn_oracle.c"

static int failures = 0;
#define CHECK(cond, what)                                     \
    do {                                                      \
        if (!(cond)) {                                        \
            ++failures;                                       \
            printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, what); \
        }                                                     \
    } while (0)

static unsigned long long rng = 88172645463325252ull;
static double uni(void)   /* xorshift64, in (-1, 1) */
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (double)(rng >> 11) / 4503599627370496.0 - 1.0;
}

static double *vec(int64_t n, double lo, double hi)
{
    double *v = malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) v[i] = lo + (hi - lo) * 0.5 * (uni() + 1.0);
    return v;
}

static int all_finite(const double *v, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(v[i])) return 0;
    return 1;
}

static void run(int64_t N, int64_t C, int64_t HW, int act, double p)
{
    const int64_t n = N * C * HW, m = N * HW;
    double *x = vec(n, -3.0, 3.0), *dy = vec(n, -1.0, 1.0);
    double *g = vec(C, 0.5, 1.5), *b = vec(C, -0.3, 0.3);
    double *y = vec(n, 0, 0), *xh = vec(n, 0, 0), *dx = vec(n, 0, 0);
    double *mean = vec(C, 0, 0), *var = vec(C, 0, 0), *inv = vec(C, 0, 0);
    double *rm = vec(C, 0, 0), *rv = vec(C, 1, 1), *dg = vec(C, 0, 0), *db = vec(C, 0, 0);
    const int ok = m >= 2;
    CHECK(orc_forward_train(N, C, HW, x, g, b, act, p, 1e-5, 0.1, y, mean, var, inv, rm, rv)
          == (ok ? 0 : -1), "forward_train status");
    if (ok) {
        CHECK(all_finite(y, n) && all_finite(inv, C), "forward_train finite");
        CHECK(orc_backward_from_y(N, C, HW, y, dy, g, b, inv, act, p, dx, dg, db, xh) == 0,
              "backward_from_y");
        CHECK(all_finite(dx, n), "backward_from_y finite");
        CHECK(orc_backward_from_y_form2(N, C, HW, y, dy, g, b, inv, act, p, dx, dg, db) == 0,
              "form2");
        CHECK(orc_backward_from_x(N, C, HW, x, dy, g, b, act, p, 1e-5, dx, dg, db) == 0,
              "backward_from_x");
        CHECK(orc_forward_train_ckpt(N, C, HW, x, g, b, act, p, 1e-5, 0.1, xh, y, mean, var, inv,
                                     rm, rv) == 0, "forward_train_ckpt");
        CHECK(orc_backward_from_xhat(N, C, HW, xh, dy, g, b, inv, act, p, dx, dg, db) == 0,
              "backward_from_xhat");
        CHECK(all_finite(dx, n), "backward_from_xhat finite");
    }
    CHECK(orc_forward_eval(N, C, HW, x, g, b, rm, rv, act, p, 1e-5, y) == 0, "forward_eval");
    CHECK(orc_backward_eval(N, C, HW, y, dy, g, b, rv, 1e-5, act, p, dx, dg, db) == 0,
          "backward_eval");
    CHECK(orc_recompute_from_xhat(N, C, HW, x, g, b, act, p, y) == 0, "recompute");
    for (int s = 0; s <= 3; ++s) CHECK(orc_round_storage(y, n, s) == 0, "round_storage");
    free(x); free(dy); free(g); free(b); free(y); free(xh); free(dx);
    free(mean); free(var); free(inv); free(rm); free(rv); free(dg); free(db);
}

int main(void)
{
    const int64_t shapes[][3] = {{2, 4, 64}, {1, 1, 2}, {2, 3, 1}, {3, 5, 7}, {1, 2, 1},
                                 {4, 1, 9}, {1, 7, 13}};
    for (size_t k = 0; k < sizeof shapes / sizeof shapes[0]; ++k)
        for (int act = 0; act < 3; ++act)
            run(shapes[k][0], shapes[k][1], shapes[k][2], act, act == 2 ? 0.7 : 0.01);
    /* invalid arguments are refused, never read */
    double d = 0.0;
    CHECK(orc_forward_train(1, 1, 1, &d, &d, &d, 1, 0.01, 1e-5, 0.1, &d, 0, 0, 0, 0, 0) == -1,
          "m = 1");
    CHECK(orc_forward_train(2, 1, 1, &d, &d, &d, 9, 0.01, 1e-5, 0.1, &d, 0, 0, 0, 0, 0) == -1,
          "bad activation");
    CHECK(orc_forward_train(2, 1, 1, &d, &d, &d, 1, -1.0, 1e-5, 0.1, &d, 0, 0, 0, 0, 0) == -1,
          "bad slope");
    CHECK(orc_forward_train(2, 1, 1, &d, &d, &d, 1, 0.01, -1.0, 0.1, &d, 0, 0, 0, 0, 0) == -1,
          "bad eps");
    CHECK(orc_round_storage(&d, 1, 7) == -1, "bad storage");
    /* storage rounding of special values */
    double sp[] = {NAN, INFINITY, -INFINITY, 0.0, -0.0, 1e-45, 6e-8, 65519.0, 65520.0, 3.4e38,
                   1e300, -1e-300, 5.9604644775390625e-08};
    const int64_t ns = (int64_t)(sizeof sp / sizeof sp[0]);
    for (int s = 1; s <= 3; ++s) {
        double t[sizeof sp / sizeof sp[0]];
        for (int64_t i = 0; i < ns; ++i) t[i] = sp[i];
        CHECK(orc_round_storage(t, ns, s) == 0, "special values");
        CHECK(isnan(t[0]) && t[1] == INFINITY && t[2] == -INFINITY, "specials kept");
    }
    CHECK(orc_num_threads() >= 1, "threads");
    if (failures) {
        printf("FAILED %d checks\n", failures);
        return 1;
    }
    printf("OK\n");
    return 0;
}
