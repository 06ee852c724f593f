/* The fp64 oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (host code
 * only): every form of the map and the backward pass on small seeded problems, ragged
 * sequences, groups, both decays, with and without D and h0.  The recurrence (O1), the
 * materialised quadratic form (O2) and the chunked form (O3) must agree to 1e-10, so a
 * sanitizer build that still computes the right numbers is checked, not only one that
 * does not crash.  Exit status 0 on success, 1 on a mismatch or a refused shape. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_recurrence(int64_t b, int64_t T, int64_t H, int64_t P, int64_t N, int64_t G, int diag,
                      const double* x, const double* dt, const double* A, const double* B, const double* C,
                      const double* D, const double* h0, double* y, double* hT, int nthreads);
int oracle_quadratic(int64_t b, int64_t T, int64_t H, int64_t P, int64_t N, int64_t G, int diag,
                     const double* x, const double* dt, const double* A, const double* B, const double* C,
                     const double* D, const double* h0, double* y, double* hT, double* M, int nthreads);
int oracle_chunked(int64_t b, int64_t T, int64_t H, int64_t P, int64_t N, int64_t G, int diag, int64_t Q,
                   const double* x, const double* dt, const double* A, const double* B, const double* C,
                   const double* D, const double* h0, double* y, double* hT, double* cdt, double* Gm, double* S,
                   double* Hc, double* ydiag, double* yoff, int nthreads);
int oracle_recurrence_bwd(int64_t b, int64_t T, int64_t H, int64_t P, int64_t N, int64_t G, int diag,
                          const double* x, const double* dt, const double* A, const double* B, const double* C,
                          const double* D, const double* h0, const double* dy, const double* dhT, double* dx,
                          double* ddt, double* dA, double* dB, double* dC, double* dD, double* dh0, int nthreads);

static uint64_t st = 7u;
static double uni(void) { /* splitmix64 -> [0, 1) */
    uint64_t z = (st += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) * (1.0 / 9007199254740992.0);
}
static double* fill(size_t n, double lo, double hi) {
    double* a = (double*)malloc((n ? n : 1) * sizeof(double));
    for (size_t i = 0; i < n; ++i) a[i] = lo + (hi - lo) * uni();
    return a;
}
static double maxrel(const double* a, const double* r, size_t n) {
    double e = 0.0, m = 0.0;
    for (size_t i = 0; i < n; ++i) {
        e = fmax(e, fabs(a[i] - r[i]));
        m = fmax(m, fabs(r[i]));
    }
    return m > 0.0 ? e / m : e;
}

static int one(int64_t b, int64_t T, int64_t H, int64_t P, int64_t N, int64_t G, int diag, int64_t Q, int withD,
               int withh0) {
    const size_t nx = (size_t)(b * T * H * P), nbc = (size_t)(b * T * G * N), nh = (size_t)(b * H * P * N);
    double *x = fill(nx, -1, 1), *dt = fill((size_t)(b * T * H), 1e-3, 0.1), *A = fill((size_t)(diag ? H * N : H), -4, -0.2);
    double *Bm = fill(nbc, -0.5, 0.5), *Cm = fill(nbc, -0.5, 0.5);
    double *D = withD ? fill((size_t)H, -1, 1) : NULL, *h0 = withh0 ? fill(nh, -0.1, 0.1) : NULL;
    double *y1 = fill(nx, 0, 0), *y2 = fill(nx, 0, 0), *y3 = fill(nx, 0, 0);
    double *h1 = fill(nh, 0, 0), *h2 = fill(nh, 0, 0), *h3 = fill(nh, 0, 0);
    int bad = 0;
    bad |= oracle_recurrence(b, T, H, P, N, G, diag, x, dt, A, Bm, Cm, D, h0, y1, h1, 2);
    bad |= oracle_quadratic(b, T, H, P, N, G, diag, x, dt, A, Bm, Cm, D, h0, y2, h2, NULL, 2);
    bad |= oracle_chunked(b, T, H, P, N, G, diag, Q, x, dt, A, Bm, Cm, D, h0, y3, h3, NULL, NULL, NULL, NULL, NULL,
                          NULL, 2);
    const double e = fmax(fmax(maxrel(y2, y1, nx), maxrel(y3, y1, nx)), fmax(maxrel(h2, h1, nh), maxrel(h3, h1, nh)));
    /* backward: every gradient buffer written, finite */
    double *dy = fill(nx, -1, 1), *dhT = fill(nh, -0.1, 0.1);
    double *dx = fill(nx, 0, 0), *ddt = fill((size_t)(b * T * H), 0, 0), *dA = fill((size_t)(diag ? H * N : H), 0, 0);
    double *dB = fill(nbc, 0, 0), *dC = fill(nbc, 0, 0), *dD = fill((size_t)H, 0, 0), *dh0 = fill(nh, 0, 0);
    bad |= oracle_recurrence_bwd(b, T, H, P, N, G, diag, x, dt, A, Bm, Cm, D, h0, dy, dhT, dx, ddt, dA, dB, dC, dD,
                                 dh0, 2);
    double s = 0.0;
    for (size_t i = 0; i < nx; ++i) s += dx[i];
    for (size_t i = 0; i < nbc; ++i) s += dB[i] + dC[i];
    printf("b%lld T%lld H%lld P%lld N%lld G%lld diag%d Q%lld: O2/O3 vs O1 %.2e, backward checksum %s\n", (long long)b,
           (long long)T, (long long)H, (long long)P, (long long)N, (long long)G, diag, (long long)Q, e,
           isfinite(s) ? "finite" : "NOT FINITE");
    free(x); free(dt); free(A); free(Bm); free(Cm); free(D); free(h0);
    free(y1); free(y2); free(y3); free(h1); free(h2); free(h3);
    free(dy); free(dhT); free(dx); free(ddt); free(dA); free(dB); free(dC); free(dD); free(dh0);
    return bad || !(e < 1e-10) || !isfinite(s);
}

int main(void) {
    int bad = 0;
    bad |= one(1, 1, 1, 1, 1, 1, 0, 1, 0, 0);
    bad |= one(2, 37, 4, 3, 5, 2, 0, 8, 1, 1);
    bad |= one(1, 64, 2, 4, 6, 1, 1, 16, 1, 0);
    bad |= one(3, 29, 6, 2, 3, 3, 1, 7, 0, 1);
    bad |= one(1, 50, 2, 2, 2, 2, 0, 64, 1, 1);  /* one chunk holds the whole sequence */
    bad |= one(2, 0, 2, 3, 4, 1, 0, 4, 1, 1);    /* empty sequence */
    printf(bad ? "FAILED\n" : "OK\n");
    return bad;
}
