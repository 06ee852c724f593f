/* The library used from plain C: no Python, no PyTorch.  Device memory and copies come
 * from the HIP runtime; the scan is libssd.so through include/ssd.h alone.  One float32
 * forward (scalar decay, ragged last chunk, groups), one decode step continuing it, and
 * one backward pass, each compared with the fp64 oracle (oracle/ssd_oracle.c, linked in
 * for this check only) on the same seeded inputs.  Exit status 0 when every output is
 * within 1e-4 (max-norm relative), 1 on a mismatch, 2 on a library or runtime error.
 *
 * Inputs: a splitmix64 stream (Steele, Lea and Flood, "Fast splittable pseudorandom
 * number generators") mapped to uniforms; dt in [1e-3, 0.1], A = -exp(U[0, ln 16]),
 * x ~ U[-1, 1], B and C ~ U[-1, 1] / sqrt(N), D ~ U[-1, 1], h0 ~ 0.1 U[-1, 1]. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "ssd.h"

int oracle_recurrence(int64_t b, int64_t T, int64_t H, int64_t P, int64_t N, int64_t G, int diag,
                      const double* x, const double* dt, const double* A, const double* B, const double* C,
                      const double* D, const double* h0, double* y, double* hT, int nthreads);
int oracle_recurrence_bwd(int64_t b, int64_t T, int64_t H, int64_t P, int64_t N, int64_t G, int diag,
                          const double* x, const double* dt, const double* A, const double* B, const double* C,
                          const double* D, const double* h0, const double* dy, const double* dhT, double* dx,
                          double* ddt, double* dA, double* dB, double* dC, double* dD, double* dh0, int nthreads);

static uint64_t rng_state = 20261203u;
static double uniform(void) { /* splitmix64 -> [0, 1) */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) * (1.0 / 9007199254740992.0);
}
static double sym(void) { return 2.0 * uniform() - 1.0; }

#define CHECK_HIP(e)                                                           \
    do {                                                                       \
        hipError_t err_ = (e);                                                 \
        if (err_ != hipSuccess) {                                              \
            fprintf(stderr, "HIP error %d at line %d\n", (int)err_, __LINE__); \
            exit(2);                                                           \
        }                                                                      \
    } while (0)
#define CHECK_SSD(e)                                                                                   \
    do {                                                                                               \
        int st_ = (e);                                                                                 \
        if (st_ != SSD_OK) {                                                                           \
            fprintf(stderr, "libssd status %d (%s) at line %d\n", st_, ssd_status_string(st_), __LINE__); \
            exit(2);                                                                                   \
        }                                                                                              \
    } while (0)

static float* to_dev(const double* h, size_t n) {
    float* f = (float*)malloc(n * sizeof(float));
    for (size_t i = 0; i < n; ++i) f[i] = (float)h[i];
    void* d = NULL;
    CHECK_HIP(hipMalloc(&d, n * sizeof(float) + 16));
    CHECK_HIP(hipMemcpy(d, f, n * sizeof(float), hipMemcpyHostToDevice));
    free(f);
    return (float*)d;
}
static float* dev_alloc(size_t n) {
    void* d = NULL;
    CHECK_HIP(hipMalloc(&d, n * sizeof(float) + 16));
    return (float*)d;
}
static double* from_dev(const float* d, size_t n) {
    float* f = (float*)malloc(n * sizeof(float));
    CHECK_HIP(hipMemcpy(f, d, n * sizeof(float), hipMemcpyDeviceToHost));
    double* h = (double*)malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) h[i] = (double)f[i];
    free(f);
    return h;
}
/* max |got - ref| / max |ref| over the whole tensor */
static double rel(const double* got, const double* ref, size_t n) {
    double e = 0.0, m = 0.0;
    for (size_t i = 0; i < n; ++i) {
        const double d = fabs(got[i] - ref[i]);
        if (d != d) return INFINITY; /* a NaN anywhere fails */
        if (d > e) e = d;
        if (fabs(ref[i]) > m) m = fabs(ref[i]);
    }
    return m > 0.0 ? e / m : e;
}

int main(void) {
    const int64_t b = 2, T = 300, H = 4, P = 32, N = 64, G = 2, Q = 128;
    const size_t nx = (size_t)(b * T * H * P), nd = (size_t)(b * T * H), nb = (size_t)(b * T * G * N),
                 ns = (size_t)(b * H * P * N);
    double *x = malloc(nx * 8), *dt = malloc(nd * 8), *A = malloc(H * 8), *B = malloc(nb * 8),
           *C = malloc(nb * 8), *D = malloc(H * 8), *h0 = malloc(ns * 8), *dy = malloc(nx * 8),
           *dhT = malloc(ns * 8);
    for (size_t i = 0; i < nx; ++i) x[i] = sym();
    for (size_t i = 0; i < nd; ++i) dt[i] = 1e-3 * exp(uniform() * log(100.0));
    for (int64_t h = 0; h < H; ++h) A[h] = -exp(uniform() * log(16.0));
    for (size_t i = 0; i < nb; ++i) B[i] = sym() / sqrt((double)N);
    for (size_t i = 0; i < nb; ++i) C[i] = sym() / sqrt((double)N);
    for (int64_t h = 0; h < H; ++h) D[h] = sym();
    for (size_t i = 0; i < ns; ++i) h0[i] = 0.1 * sym();
    for (size_t i = 0; i < nx; ++i) dy[i] = sym();
    for (size_t i = 0; i < ns; ++i) dhT[i] = 0.1 * sym();

    float *dx_ = to_dev(x, nx), *ddt_ = to_dev(dt, nd), *dA_ = to_dev(A, H), *dB_ = to_dev(B, nb),
          *dC_ = to_dev(C, nb), *dD_ = to_dev(D, H), *dh0_ = to_dev(h0, ns), *ddy_ = to_dev(dy, nx),
          *ddhT_ = to_dev(dhT, ns);
    int bad = 0;

    /* ---- forward ---- */
    ssd_problem p = {b, T, H, P, N, G, Q, SSD_F32, 0};
    const size_t wsb = ssd_workspace_bytes(&p, 0);
    void* ws = NULL;
    CHECK_HIP(hipMalloc(&ws, wsb));
    float *y_ = dev_alloc(nx), *hT_ = dev_alloc(ns);
    CHECK_SSD(ssd_scan_fwd(&p, dx_, ddt_, dA_, dB_, dC_, dD_, dh0_, y_, hT_, ws, wsb, NULL));
    CHECK_HIP(hipDeviceSynchronize());
    double *y = from_dev(y_, nx), *hT = from_dev(hT_, ns);
    double *yr = malloc(nx * 8), *hr = malloc(ns * 8);
    if (oracle_recurrence(b, T, H, P, N, G, 0, x, dt, A, B, C, D, h0, yr, hr, 0)) return 2;
    const double ey = rel(y, yr, nx), eh = rel(hT, hr, ns);
    printf("forward: y %.3e hT %.3e\n", ey, eh);
    bad |= !(ey < 1e-4 && eh < 1e-4);

    /* ---- one decode step continuing from hT ---- */
    ssd_problem ps = {b, 1, H, P, N, G, Q, SSD_F32, 0};
    double *x1 = malloc((size_t)(b * H * P) * 8), *dt1 = malloc((size_t)(b * H) * 8),
           *B1 = malloc((size_t)(b * G * N) * 8), *C1 = malloc((size_t)(b * G * N) * 8);
    for (int64_t i = 0; i < b * H * P; ++i) x1[i] = sym();
    for (int64_t i = 0; i < b * H; ++i) dt1[i] = 0.05;
    for (int64_t i = 0; i < b * G * N; ++i) B1[i] = sym() / sqrt((double)N);
    for (int64_t i = 0; i < b * G * N; ++i) C1[i] = sym() / sqrt((double)N);
    float *x1_ = to_dev(x1, (size_t)(b * H * P)), *dt1_ = to_dev(dt1, (size_t)(b * H)),
          *B1_ = to_dev(B1, (size_t)(b * G * N)), *C1_ = to_dev(C1, (size_t)(b * G * N)),
          *y1_ = dev_alloc((size_t)(b * H * P));
    CHECK_SSD(ssd_step(&ps, x1_, dt1_, dA_, B1_, C1_, dD_, hT_, y1_, NULL));
    CHECK_HIP(hipDeviceSynchronize());
    double *y1 = from_dev(y1_, (size_t)(b * H * P)), *h1 = from_dev(hT_, ns);
    double *y1r = malloc((size_t)(b * H * P) * 8), *h1r = malloc(ns * 8);
    /* the oracle's reference: one token from the oracle's own final state */
    if (oracle_recurrence(b, 1, H, P, N, G, 0, x1, dt1, A, B1, C1, D, hr, y1r, h1r, 0)) return 2;
    const double ey1 = rel(y1, y1r, (size_t)(b * H * P)), eh1 = rel(h1, h1r, ns);
    printf("step: y %.3e h %.3e\n", ey1, eh1);
    bad |= !(ey1 < 1e-4 && eh1 < 1e-4);

    /* ---- backward ---- */
    const size_t bwsb = ssd_bwd_workspace_bytes(&p);
    void* bws = NULL;
    CHECK_HIP(hipMalloc(&bws, bwsb));
    float *gx_ = dev_alloc(nx), *gdt_ = dev_alloc(nd), *gA_ = dev_alloc(H), *gB_ = dev_alloc(nb),
          *gC_ = dev_alloc(nb), *gD_ = dev_alloc(H), *gh0_ = dev_alloc(ns);
    CHECK_SSD(ssd_scan_bwd(&p, dx_, ddt_, dA_, dB_, dC_, dD_, dh0_, ddy_, ddhT_, gx_, gdt_, gA_, gB_, gC_, gD_, gh0_,
                           bws, bwsb, NULL));
    CHECK_HIP(hipDeviceSynchronize());
    double *rx = malloc(nx * 8), *rdt = malloc(nd * 8), *rA = malloc(H * 8), *rB = malloc(nb * 8),
           *rC = malloc(nb * 8), *rD = malloc(H * 8), *rh0 = malloc(ns * 8);
    if (oracle_recurrence_bwd(b, T, H, P, N, G, 0, x, dt, A, B, C, D, h0, dy, dhT, rx, rdt, rA, rB, rC, rD, rh0, 0))
        return 2;
    const double e[6] = {rel(from_dev(gx_, nx), rx, nx), rel(from_dev(gdt_, nd), rdt, nd),
                         rel(from_dev(gB_, nb), rB, nb), rel(from_dev(gC_, nb), rC, nb),
                         rel(from_dev(gD_, H), rD, H), rel(from_dev(gh0_, ns), rh0, ns)};
    printf("backward: dx %.3e ddt %.3e dB %.3e dC %.3e dD %.3e dh0 %.3e\n", e[0], e[1], e[2], e[3], e[4], e[5]);
    for (int i = 0; i < 6; ++i) bad |= !(e[i] < 1e-4);
    /* dA: each entry sums dt dl over every token (cancellation); gate against the
     * sum of |terms| bound, sum_b max_t |dl| sum_t |dt| with dl = ddt / A */
    double* gA = from_dev(gA_, H);
    for (int64_t h = 0; h < H; ++h) {
        double bound = 0.0;
        for (int64_t bi = 0; bi < b; ++bi) {
            double mdl = 0.0, sdt = 0.0;
            for (int64_t t = 0; t < T; ++t) {
                const double dl = rdt[(bi * T + t) * H + h] / A[h];
                if (fabs(dl) > mdl) mdl = fabs(dl);
                sdt += fabs(dt[(bi * T + t) * H + h]);
            }
            bound += mdl * sdt;
        }
        const double err = fabs(gA[h] - rA[h]);
        if (!(err <= 1e-4 * bound)) bad = 1;
    }
    printf("%s\n", bad ? "MISMATCH" : "ok");
    return bad ? 1 : 0;
}
