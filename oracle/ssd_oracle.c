/*
 * ssd_oracle.c -- plain, slow, fp64 CPU oracle for the SSD (structured state
 * space duality) scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or load
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline leg
 * use it.  It shares no code, header, table or helper with the HIP library.
 *
 * Sources (web pages, cited by title and section):
 *   [SSD]  "Structured State Space Duality" concept page:
 *          sections "The recurrence as one matrix", "The chunked algorithm takes
 *          both", "What the duality gives up", "When it breaks".
 *   [DIAG] "Diagonal Equivalence in State Space Models: Characterization,
 *          Retrieval Rank, and Selective Extensions", abstract (state-mediated
 *          kernels = unnormalised scalar-mode linear attention with
 *          multiplicative masks).
 *   [SEMI] "Semiseparable Matrix Transformations" keyword page, definition.
 *
 * Readings taken where the pages are silent (all fp64):
 *   - decay a_t = exp(dt_t * A_h) (scalar), a_{t,n} = exp(dt_t * A_{h,n}) (diagonal);
 *   - the input term is B_t x_t^T (dt enters only through the decay);
 *   - h0 is the state before token 0 (decayed by a_0); h_T the state after T-1;
 *   - y_t reads the state after token t's update (diagonal of M included);
 *   - optional per-head skip D_h * x_t;
 *   - P channels of a head are independent SSMs sharing a_t, B_t, C_t;
 *   - head h uses B/C group g = floor(h * G / H).
 *
 * Layouts (row-major, contiguous):
 *   x, y [b,T,H,P]; dt [b,T,H]; A [H] (scalar) or [H,N] (diagonal);
 *   B, C [b,T,G,N]; D [H]; h0, hT [b,H,P,N].
 *
 * Parity pins: every function here is checked by the CPU test suite against
 * hand-derived values, closed forms and structural invariants (see the oracle
 * pin tests); none of them is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int64_t b, T, H, P, N, G;
    int diag;
} dims_t;

static int64_t group_of(const dims_t* d, int64_t h) { return h * d->G / d->H; }

static double decay_log(const dims_t* d, const double* A, int64_t h, int64_t n, double dt) {
    /* log of the per-token decay: dt * A_h, or dt * A_{h,n} in the diagonal case */
    return dt * (d->diag ? A[h * d->N + n] : A[h]);
}

static int check_dims(const dims_t* d) {
    if (d->b < 0 || d->T < 0 || d->H <= 0 || d->P <= 0 || d->N <= 0 || d->G <= 0) return 1;
    if (d->H % d->G != 0) return 1;
    return 0;
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* ------------------------------------------------------------------------- *
 * O1: the selective recurrence stepped token by token.
 * [SSD] "The recurrence as one matrix": h_t = Abar_t h_{t-1} + Bbar_t x_t,
 * y_t = C_t^T h_t, with Abar_t = a_t I (scalar) or diag(a_{t,n}) ([SSD] "What the
 * duality gives up"; [DIAG]).  State per head is P x N (one N-vector per channel).
 * Work items are (b, h, channel block) so that few heads still use every core.
 * ------------------------------------------------------------------------- */
int oracle_recurrence(int64_t b, int64_t T, int64_t H, int64_t P, int64_t N, int64_t G, int diag,
                      const double* x, const double* dt, const double* A, const double* B,
                      const double* C, const double* D, const double* h0, double* y, double* hT,
                      int nthreads) {
    dims_t d = {b, T, H, P, N, G, diag};
    if (check_dims(&d)) return 1;
    set_threads(nthreads);
    int64_t pblocks = 1;
#ifdef _OPENMP
    {
        int64_t want = 2 * (int64_t)omp_get_max_threads();
        while (b * H * pblocks < want && pblocks < P) pblocks *= 2;
        if (pblocks > P) pblocks = P;
    }
#endif
    const int64_t pstep = (P + pblocks - 1) / pblocks;
    const int64_t items = b * H * pblocks;
#pragma omp parallel
    {
        double* S = (double*)malloc(sizeof(double) * (size_t)(pstep * N));
        double* a = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
        for (int64_t it = 0; it < items; ++it) {
            const int64_t bi = it / (H * pblocks);
            const int64_t h = (it / pblocks) % H;
            const int64_t p0 = (it % pblocks) * pstep;
            const int64_t p1 = p0 + pstep < P ? p0 + pstep : P;
            const int64_t g = group_of(&d, h);
            for (int64_t p = p0; p < p1; ++p)
                for (int64_t n = 0; n < N; ++n)
                    S[(p - p0) * N + n] = h0 ? h0[((bi * H + h) * P + p) * N + n] : 0.0;
            for (int64_t t = 0; t < T; ++t) {
                const double dtv = dt[(bi * T + t) * H + h];
                for (int64_t n = 0; n < N; ++n) a[n] = exp(decay_log(&d, A, h, n, dtv));
                const double* Bt = B + ((bi * T + t) * G + g) * N;
                const double* Ct = C + ((bi * T + t) * G + g) * N;
                for (int64_t p = p0; p < p1; ++p) {
                    const double xv = x[((bi * T + t) * H + h) * P + p];
                    double* s = S + (p - p0) * N;
                    double acc = 0.0;
                    for (int64_t n = 0; n < N; ++n) {
                        s[n] = a[n] * s[n] + xv * Bt[n];
                        acc += Ct[n] * s[n];
                    }
                    y[((bi * T + t) * H + h) * P + p] = acc + (D ? D[h] * xv : 0.0);
                }
            }
            if (hT)
                for (int64_t p = p0; p < p1; ++p)
                    for (int64_t n = 0; n < N; ++n)
                        hT[((bi * H + h) * P + p) * N + n] = S[(p - p0) * N + n];
        }
        free(S);
        free(a);
    }
    return 0;
}

/* ------------------------------------------------------------------------- *
 * O2: the materialised quadratic form y = M x ([SSD] "The recurrence as one
 * matrix": the sequence map is one lower-triangular matrix M; with a_k I the
 * product of transitions collapses to a product of scalars and M is a causal
 * attention matrix C_i^T B_j times a decay mask, no softmax).  Diagonal case:
 * M = sum_n L^(n) o (c_n b_n^T), a sum of N scalar-mode masked attentions
 * ([DIAG] abstract).
 *
 *   M_ij = sum_n C_in B_jn prod_{k=j+1..i} a_{k,n}          (i >= j, else 0)
 *   y_i  = sum_{j<=i} M_ij x_j + sum_n (prod_{k=0..i} a_{k,n}) C_in h0[:,n] + D x_i
 *   hT   = (prod_{k=0..T-1} a_k) h0 + sum_j (prod_{k=j+1..T-1} a_k) x_j B_j^T
 *
 * Every decay product is formed by explicit multiplication of the a_k (no
 * logarithms, no cumulative sums), so this form shares no numerical path with
 * O1 or O3.  O(T^2 N) per head: for small inputs only.  If M_out is given it
 * receives M as [b,H,T,T].
 * ------------------------------------------------------------------------- */
int oracle_quadratic(int64_t b, int64_t T, int64_t H, int64_t P, int64_t N, int64_t G, int diag,
                     const double* x, const double* dt, const double* A, const double* B,
                     const double* C, const double* D, const double* h0, double* y, double* hT,
                     double* M_out, int nthreads) {
    dims_t d = {b, T, H, P, N, G, diag};
    if (check_dims(&d)) return 1;
    set_threads(nthreads);
    const int64_t items = b * H;
#pragma omp parallel
    {
        double* M = (double*)malloc(sizeof(double) * (size_t)(T * T > 0 ? T * T : 1));
        double* a = (double*)malloc(sizeof(double) * (size_t)((T > 0 ? T : 1) * N));
        double* prod = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
        for (int64_t it = 0; it < items; ++it) {
            const int64_t bi = it / H, h = it % H, g = group_of(&d, h);
            for (int64_t t = 0; t < T; ++t) {
                const double dtv = dt[(bi * T + t) * H + h];
                for (int64_t n = 0; n < N; ++n) a[t * N + n] = exp(decay_log(&d, A, h, n, dtv));
            }
            /* M, row by row; prod[n] = prod_{k=j+1..i} a_{k,n} as j walks down from i */
            for (int64_t i = 0; i < T; ++i) {
                const double* Ci = C + ((bi * T + i) * G + g) * N;
                for (int64_t n = 0; n < N; ++n) prod[n] = 1.0;
                for (int64_t j = i; j >= 0; --j) {
                    const double* Bj = B + ((bi * T + j) * G + g) * N;
                    double m = 0.0;
                    for (int64_t n = 0; n < N; ++n) m += Ci[n] * Bj[n] * prod[n];
                    M[i * T + j] = m;
                    for (int64_t n = 0; n < N; ++n) prod[n] *= a[j * N + n];
                }
                for (int64_t j = i + 1; j < T; ++j) M[i * T + j] = 0.0;
                /* here prod[n] = prod_{k=0..i} a_{k,n}: the decay applied to h0 */
                for (int64_t p = 0; p < P; ++p) {
                    double acc = 0.0;
                    for (int64_t j = 0; j <= i; ++j) acc += M[i * T + j] * x[((bi * T + j) * H + h) * P + p];
                    if (h0) {
                        const double* hp = h0 + ((bi * H + h) * P + p) * N;
                        for (int64_t n = 0; n < N; ++n) acc += prod[n] * Ci[n] * hp[n];
                    }
                    const double xv = x[((bi * T + i) * H + h) * P + p];
                    y[((bi * T + i) * H + h) * P + p] = acc + (D ? D[h] * xv : 0.0);
                }
            }
            if (M_out) memcpy(M_out + (bi * H + h) * T * T, M, sizeof(double) * (size_t)(T * T));
            if (hT) {
                /* prod[n] = prod_{k=j+1..T-1} a_{k,n} as j walks down from T-1 */
                for (int64_t p = 0; p < P; ++p)
                    for (int64_t n = 0; n < N; ++n) hT[((bi * H + h) * P + p) * N + n] = 0.0;
                for (int64_t n = 0; n < N; ++n) prod[n] = 1.0;
                for (int64_t j = T - 1; j >= 0; --j) {
                    const double* Bj = B + ((bi * T + j) * G + g) * N;
                    for (int64_t p = 0; p < P; ++p) {
                        const double xv = x[((bi * T + j) * H + h) * P + p];
                        double* hp = hT + ((bi * H + h) * P + p) * N;
                        for (int64_t n = 0; n < N; ++n) hp[n] += prod[n] * xv * Bj[n];
                    }
                    for (int64_t n = 0; n < N; ++n) prod[n] *= a[j * N + n];
                }
                if (h0)
                    for (int64_t p = 0; p < P; ++p)
                        for (int64_t n = 0; n < N; ++n)
                            hT[((bi * H + h) * P + p) * N + n] +=
                                prod[n] * h0[((bi * H + h) * P + p) * N + n];
            }
        }
        free(M);
        free(a);
        free(prod);
    }
    return 0;
}

/* ------------------------------------------------------------------------- *
 * O3: the chunked algorithm ([SSD] "The chunked algorithm takes both"), in fp64,
 * step by step, with optional dumps of every intermediate:
 *
 *   split T into chunks of Q (the last one may be shorter);
 *   cdt_i   = sum_{k=c0..i} dt_k     chunk-local cumulative step ("accumulated
 *                                    decay"; log-decay is A * cdt, kept in fp64 here);
 *   G_c     = C_c B_c^T              per (batch, chunk, group), Q x Q;
 *   Ydiag_i = sum_{j=c0..i} G_ij exp(A (cdt_i - cdt_j)) x_j   quadratic form on the
 *                                    diagonal block ("one masked matmul");
 *   S_c     = sum_j exp(A (cdt_last - cdt_j)) x_j B_j^T      chunk input projection;
 *   H_0 = h0, H_{c+1} = exp(A cdt_last) H_c + S_c            one recurrence step
 *                                    per chunk carries the state;
 *   Yoff_i  = exp(A cdt_i) H_c C_i   chunk output projection times accumulated
 *                                    decay (the factored off-diagonal blocks);
 *   y       = Ydiag + Yoff + D x;  hT = H_nc.
 *
 * Diagonal case: every A above becomes A_{h,n} inside the sum over n, and the
 * masked block is G^(h)_ij = sum_n C_in B_jn exp(A_n (cdt_i - cdt_j)), formed per
 * head.
 *
 * Dumps (each may be NULL; nc = ceil(T/Q)):
 *   cdt_out  [b,H,nc,Q]   positions past T hold the chunk's final value
 *   G_out    [b,nc,G,Q,Q] scalar case only (rows/cols past T are 0; upper part too)
 *   S_out    [b,H,nc,P,N] chunk states S_c
 *   Hc_out   [b,H,nc,P,N] state entering chunk c (H_c)
 *   ydiag_out, yoff_out [b,T,H,P]
 * ------------------------------------------------------------------------- */
int oracle_chunked(int64_t b, int64_t T, int64_t H, int64_t P, int64_t N, int64_t G, int diag,
                   int64_t Q, const double* x, const double* dt, const double* A,
                   const double* B, const double* C, const double* D, const double* h0,
                   double* y, double* hT, double* cdt_out, double* G_out, double* S_out,
                   double* Hc_out, double* ydiag_out, double* yoff_out, int nthreads) {
    dims_t d = {b, T, H, P, N, G, diag};
    if (check_dims(&d) || Q <= 0) return 1;
    set_threads(nthreads);
    const int64_t nc = (T + Q - 1) / Q;

    /* G_c = C_c B_c^T per (batch, chunk, group): independent of the head */
    if (G_out && !diag) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t it = 0; it < b * nc * G; ++it) {
            const int64_t bi = it / (nc * G), c = (it / G) % nc, g = it % G;
            double* Gc = G_out + it * Q * Q;
            for (int64_t i = 0; i < Q; ++i)
                for (int64_t j = 0; j < Q; ++j) {
                    const int64_t ti = c * Q + i, tj = c * Q + j;
                    double m = 0.0;
                    if (ti < T && tj < T && j <= i)
                        for (int64_t n = 0; n < N; ++n)
                            m += C[((bi * T + ti) * G + g) * N + n] * B[((bi * T + tj) * G + g) * N + n];
                    Gc[i * Q + j] = m;
                }
        }
    }

    const int64_t items = b * H;
#pragma omp parallel
    {
        double* cdt = (double*)malloc(sizeof(double) * (size_t)Q);
        double* Hs = (double*)malloc(sizeof(double) * (size_t)(P * N));
        double* Sc = (double*)malloc(sizeof(double) * (size_t)(P * N));
        double* An = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
        for (int64_t it = 0; it < items; ++it) {
            const int64_t bi = it / H, h = it % H, g = group_of(&d, h);
            for (int64_t n = 0; n < N; ++n) An[n] = diag ? A[h * N + n] : A[h];
            for (int64_t k = 0; k < P * N; ++k) Hs[k] = h0 ? h0[(bi * H + h) * P * N + k] : 0.0;
            for (int64_t c = 0; c < nc; ++c) {
                const int64_t c0 = c * Q;
                const int64_t len = (T - c0) < Q ? (T - c0) : Q;
                /* chunk-local cumulative step; positions past T repeat the total */
                double run = 0.0;
                for (int64_t i = 0; i < Q; ++i) {
                    if (i < len) run += dt[(bi * T + c0 + i) * H + h];
                    cdt[i] = run;
                }
                if (cdt_out) memcpy(cdt_out + ((bi * H + h) * nc + c) * Q, cdt, sizeof(double) * (size_t)Q);
                const double last = cdt[len - 1];

                /* entering state H_c */
                if (Hc_out) memcpy(Hc_out + ((bi * H + h) * nc + c) * P * N, Hs, sizeof(double) * (size_t)(P * N));

                for (int64_t i = 0; i < len; ++i) {
                    const int64_t ti = c0 + i;
                    const double* Ci = C + ((bi * T + ti) * G + g) * N;
                    for (int64_t p = 0; p < P; ++p) {
                        /* diagonal block: masked quadratic form */
                        double yd = 0.0;
                        for (int64_t j = 0; j <= i; ++j) {
                            const int64_t tj = c0 + j;
                            const double* Bj = B + ((bi * T + tj) * G + g) * N;
                            double m = 0.0;
                            if (diag) {
                                for (int64_t n = 0; n < N; ++n)
                                    m += Ci[n] * Bj[n] * exp(An[n] * (cdt[i] - cdt[j]));
                            } else {
                                for (int64_t n = 0; n < N; ++n) m += Ci[n] * Bj[n];
                                m *= exp(An[0] * (cdt[i] - cdt[j]));
                            }
                            yd += m * x[((bi * T + tj) * H + h) * P + p];
                        }
                        /* off-diagonal blocks: output projection of the carried state */
                        double yo = 0.0;
                        for (int64_t n = 0; n < N; ++n) yo += Ci[n] * exp(An[n] * cdt[i]) * Hs[p * N + n];
                        const double xv = x[((bi * T + ti) * H + h) * P + p];
                        const int64_t yi = ((bi * T + ti) * H + h) * P + p;
                        if (ydiag_out) ydiag_out[yi] = yd;
                        if (yoff_out) yoff_out[yi] = yo;
                        y[yi] = yd + yo + (D ? D[h] * xv : 0.0);
                    }
                }

                /* chunk state S_c (input projection, decayed to the chunk end) */
                for (int64_t k = 0; k < P * N; ++k) Sc[k] = 0.0;
                for (int64_t j = 0; j < len; ++j) {
                    const int64_t tj = c0 + j;
                    const double* Bj = B + ((bi * T + tj) * G + g) * N;
                    for (int64_t p = 0; p < P; ++p) {
                        const double xv = x[((bi * T + tj) * H + h) * P + p];
                        for (int64_t n = 0; n < N; ++n)
                            Sc[p * N + n] += exp(An[n] * (last - cdt[j])) * xv * Bj[n];
                    }
                }
                if (S_out) memcpy(S_out + ((bi * H + h) * nc + c) * P * N, Sc, sizeof(double) * (size_t)(P * N));

                /* one recurrence step per chunk */
                for (int64_t p = 0; p < P; ++p)
                    for (int64_t n = 0; n < N; ++n)
                        Hs[p * N + n] = exp(An[n] * last) * Hs[p * N + n] + Sc[p * N + n];
            }
            if (hT) memcpy(hT + (bi * H + h) * P * N, Hs, sizeof(double) * (size_t)(P * N));
        }
        free(cdt);
        free(Hs);
        free(Sc);
        free(An);
    }
    return 0;
}

/* ------------------------------------------------------------------------- *
 * O4: gradients of the recurrence (the backward pass), by reverse-mode
 * differentiation of O1 written out by hand.  The loss is any L whose gradients
 * with respect to the outputs are given: dy = dL/dy [b,T,H,P] and dhT = dL/dhT
 * [b,H,P,N] (NULL = 0).  The pages give no backward algorithm; their speed claims
 * are about training ([SSD] "The chunked algorithm takes both").  This follows the
 * recurrence of [SSD] "The recurrence as one matrix" step by step, in reverse:
 *
 *   g_t   = dL/dh_t (through y_t and every later state)
 *         = r_t + dy_t C_t^T,        r_{T-1} = dhT,  r_{t-1} = a_t o g_t
 *   dx_t  = D_h dy_t + g_t B_t                      (sum over n)
 *   dB_t += g_t^T x_t,  dC_t += h_t^T dy_t          (sum over p and over the heads of the group)
 *   dl_t  = sum_p g_t o (a_t h_{t-1})               (per n: dL / d(dt_t A_{h,n}))
 *   ddt_t = sum_n A_{h(,n)} dl_{t,n},  dA_{h(,n)} += dt_t dl_{t,n},  dD_h += dy_t . x_t
 *   dh0   = r_{-1} = a_0 o g_0
 *
 * Two passes, so that every sum has one fixed order and no two threads write one
 * element:
 *   pass A, one item per (b, h): the state sequence is rebuilt segment by segment
 *     from checkpoints every ~sqrt(T) tokens, the adjoint runs backward over the
 *     full P x N state; dx, ddt, dh0 and per-(b, h) partials of dA and dD;
 *   pass B, one item per (b, g, n): every state column n evolves on its own (the
 *     decay is a_t or a_{t,n}), so h_t[:, n] forward and g_t[:, n] backward give
 *     dC_t[n] and dB_t[n] summed over the group's heads in head order.
 * dA and dD are then summed over b in order.
 * ------------------------------------------------------------------------- */
int oracle_recurrence_bwd(int64_t b, int64_t T, int64_t H, int64_t P, int64_t N, int64_t G, int diag,
                          const double* x, const double* dt, const double* A, const double* B,
                          const double* C, const double* D, const double* h0, const double* dy,
                          const double* dhT, double* dx, double* ddt, double* dA, double* dB, double* dC,
                          double* dD, double* dh0, int nthreads) {
    dims_t d = {b, T, H, P, N, G, diag};
    if (check_dims(&d)) return 1;
    set_threads(nthreads);
    const int64_t PN = P * N;
    const int64_t nA = diag ? N : 1;  /* dA entries per head */
    int64_t SEG = 1;
    while (SEG * SEG < T) ++SEG;
    const int64_t nseg = T > 0 ? (T + SEG - 1) / SEG : 0;
    double* dApart = (double*)calloc((size_t)(b * H * nA + 1), sizeof(double));
    double* dDpart = (double*)calloc((size_t)(b * H + 1), sizeof(double));
    if (!dApart || !dDpart) {
        free(dApart);
        free(dDpart);
        return 2;
    }

    /* pass A: one (b, h) per item */
#pragma omp parallel
    {
        double* ck = (double*)malloc(sizeof(double) * (size_t)((nseg > 0 ? nseg : 1) * PN));
        double* buf = (double*)malloc(sizeof(double) * (size_t)(SEG * PN));
        double* S = (double*)malloc(sizeof(double) * (size_t)PN);
        double* r = (double*)malloc(sizeof(double) * (size_t)PN);
        double* a = (double*)malloc(sizeof(double) * (size_t)N);
        double* dl = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(static)
        for (int64_t it = 0; it < b * H; ++it) {
            const int64_t bi = it / H, h = it % H, g = group_of(&d, h);
            const double Dh = D ? D[h] : 0.0;
            double* dAp = dApart + it * nA;
            double dDp = 0.0;
            /* forward, keeping the state before every SEG-th token */
            for (int64_t e = 0; e < PN; ++e) S[e] = h0 ? h0[(bi * H + h) * PN + e] : 0.0;
            for (int64_t t = 0; t < T; ++t) {
                if (t % SEG == 0) memcpy(ck + (t / SEG) * PN, S, sizeof(double) * (size_t)PN);
                const double dtv = dt[(bi * T + t) * H + h];
                for (int64_t n = 0; n < N; ++n) a[n] = exp(decay_log(&d, A, h, n, dtv));
                const double* Bt = B + ((bi * T + t) * G + g) * N;
                for (int64_t p = 0; p < P; ++p) {
                    const double xv = x[((bi * T + t) * H + h) * P + p];
                    for (int64_t n = 0; n < N; ++n) S[p * N + n] = a[n] * S[p * N + n] + xv * Bt[n];
                }
            }
            /* backward: r holds dL/dh_t through the later tokens (dhT after the last) */
            for (int64_t e = 0; e < PN; ++e) r[e] = dhT ? dhT[(bi * H + h) * PN + e] : 0.0;
            for (int64_t k = nseg - 1; k >= 0; --k) {
                const int64_t t0 = k * SEG, t1 = (t0 + SEG < T) ? t0 + SEG : T;
                memcpy(S, ck + k * PN, sizeof(double) * (size_t)PN);
                for (int64_t t = t0; t < t1; ++t) {
                    const double dtv = dt[(bi * T + t) * H + h];
                    for (int64_t n = 0; n < N; ++n) a[n] = exp(decay_log(&d, A, h, n, dtv));
                    const double* Bt = B + ((bi * T + t) * G + g) * N;
                    for (int64_t p = 0; p < P; ++p) {
                        const double xv = x[((bi * T + t) * H + h) * P + p];
                        for (int64_t n = 0; n < N; ++n) S[p * N + n] = a[n] * S[p * N + n] + xv * Bt[n];
                    }
                    memcpy(buf + (t - t0) * PN, S, sizeof(double) * (size_t)PN);
                }
                for (int64_t t = t1 - 1; t >= t0; --t) {
                    const double* hprev = (t == t0) ? ck + k * PN : buf + (t - 1 - t0) * PN;
                    const double dtv = dt[(bi * T + t) * H + h];
                    for (int64_t n = 0; n < N; ++n) a[n] = exp(decay_log(&d, A, h, n, dtv));
                    const double* Bt = B + ((bi * T + t) * G + g) * N;
                    const double* Ct = C + ((bi * T + t) * G + g) * N;
                    const double* dyt = dy + ((bi * T + t) * H + h) * P;
                    const double* xt = x + ((bi * T + t) * H + h) * P;
                    for (int64_t n = 0; n < N; ++n) dl[n] = 0.0;
                    for (int64_t p = 0; p < P; ++p) {
                        double* gp = r + p * N;  /* becomes g_t, then r_{t-1} */
                        double acc = 0.0;
                        for (int64_t n = 0; n < N; ++n) {
                            gp[n] += dyt[p] * Ct[n];
                            acc += gp[n] * Bt[n];
                            dl[n] += gp[n] * a[n] * hprev[p * N + n];
                        }
                        dx[((bi * T + t) * H + h) * P + p] = Dh * dyt[p] + acc;
                        dDp += dyt[p] * xt[p];
                    }
                    double dd = 0.0;
                    for (int64_t n = 0; n < N; ++n) {
                        const double An = diag ? A[h * N + n] : A[h];
                        dd += An * dl[n];
                        dAp[diag ? n : 0] += dtv * dl[n];
                    }
                    ddt[(bi * T + t) * H + h] = dd;
                    for (int64_t p = 0; p < P; ++p)
                        for (int64_t n = 0; n < N; ++n) r[p * N + n] *= a[n];
                }
            }
            if (dh0)
                for (int64_t e = 0; e < PN; ++e) dh0[(bi * H + h) * PN + e] = r[e];
            dDpart[it] = dDp;
        }
        free(ck);
        free(buf);
        free(S);
        free(r);
        free(a);
        free(dl);
    }

    /* pass B: one (b, g, n) per item; the group's heads in order */
    const int64_t hpg = H / G;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)P);
        double* accB = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
        double* accC = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
#pragma omp for schedule(static)
        for (int64_t it = 0; it < b * G * N; ++it) {
            const int64_t bi = it / (G * N), g = (it / N) % G, n = it % N;
            for (int64_t t = 0; t < T; ++t) accB[t] = accC[t] = 0.0;
            for (int64_t h = g * hpg; h < (g + 1) * hpg; ++h) {
                for (int64_t p = 0; p < P; ++p) s[p] = h0 ? h0[((bi * H + h) * P + p) * N + n] : 0.0;
                for (int64_t t = 0; t < T; ++t) {
                    const double at = exp(decay_log(&d, A, h, n, dt[(bi * T + t) * H + h]));
                    const double Bn = B[((bi * T + t) * G + g) * N + n];
                    const double* xt = x + ((bi * T + t) * H + h) * P;
                    const double* dyt = dy + ((bi * T + t) * H + h) * P;
                    double acc = 0.0;
                    for (int64_t p = 0; p < P; ++p) {
                        s[p] = at * s[p] + xt[p] * Bn;
                        acc += dyt[p] * s[p];
                    }
                    accC[t] += acc;
                }
                for (int64_t p = 0; p < P; ++p) s[p] = dhT ? dhT[((bi * H + h) * P + p) * N + n] : 0.0;
                for (int64_t t = T - 1; t >= 0; --t) {
                    const double at = exp(decay_log(&d, A, h, n, dt[(bi * T + t) * H + h]));
                    const double Cn = C[((bi * T + t) * G + g) * N + n];
                    const double* xt = x + ((bi * T + t) * H + h) * P;
                    const double* dyt = dy + ((bi * T + t) * H + h) * P;
                    double acc = 0.0;
                    for (int64_t p = 0; p < P; ++p) {
                        s[p] += dyt[p] * Cn;   /* g_t[p][n] */
                        acc += s[p] * xt[p];
                        s[p] *= at;            /* r_{t-1}[p][n] */
                    }
                    accB[t] += acc;
                }
            }
            for (int64_t t = 0; t < T; ++t) {
                dB[((bi * T + t) * G + g) * N + n] = accB[t];
                dC[((bi * T + t) * G + g) * N + n] = accC[t];
            }
        }
        free(s);
        free(accB);
        free(accC);
    }

    for (int64_t h = 0; h < H; ++h) {
        for (int64_t k = 0; k < nA; ++k) {
            double v = 0.0;
            for (int64_t bi = 0; bi < b; ++bi) v += dApart[(bi * H + h) * nA + k];
            dA[h * nA + k] = v;
        }
        if (dD) {
            double v = 0.0;
            for (int64_t bi = 0; bi < b; ++bi) v += dDpart[bi * H + h];
            dD[h] = v;
        }
    }
    free(dApart);
    free(dDpart);
    return 0;
}

int oracle_abi_version(void) { return 1; }
