// bwd.hpp -- the backward pass of the SSD chunked scan (scalar decay): the gradients
// of a loss with respect to x, dt, A, B, C, D and h0, given its gradients dy and dhT
// with respect to y and the final state.
//
// The pages give the forward map only ("Structured State Space Duality" concept
// page, sections "The recurrence as one matrix" and "The chunked algorithm takes
// both"); the gradients below follow from differentiating that recurrence.  Per
// (batch, head), with a_t = exp(dt_t A), states h_t (P x N) and g_t = dL/dh_t:
//
//   g_t   = dy_t C_t^T + a_{t+1} g_{t+1},   g_{T-1} = dy_{T-1} C_{T-1}^T + dhT
//   dx_t  = g_t B_t + D dy_t                dB_t = sum_heads g_t^T x_t
//   dC_t  = sum_heads h_t^T dy_t            dh0  = a_0 g_0
//
// The adjoint g runs the same linear recurrence backward in time with C in place of
// B, so it is chunked the same way: per chunk an adjoint input
// S'_c = sum_i exp(A cdt_i) dy_i C_i^T (k_state with ADJ), a reverse scan over chunks
// R_{c-1} = exp(A cdt_last) R_c + S'_c from R_{nc-1} = dhT (k_scan_rev; R_c is the
// adjoint arriving at chunk c's last token from the chunks after it), and within a
// chunk
//   dx_j = sum_{i >= j} exp(A (cdt_i - cdt_j)) (C_i . B_j) dy_i + exp(A (cdt_last - cdt_j)) R_c B_j + D dy_j
//   dC_i = sum_h [ sum_{j <= i} W_ij B_j + exp(A cdt_i) H_c^T dy_i ]
//   dB_j = sum_h [ sum_{i >= j} W_ij C_i + exp(A (cdt_last - cdt_j)) R_c^T x_j ]
// with W_ij = exp(A (cdt_i - cdt_j)) (dy_i . x_j) for i >= j, H_c the forward state
// entering the chunk.  B and C are shared by the heads of a group, so the head sum of
// W is formed first and multiplied by B and C once per group.
//
// The decay gradient.  With s_t the running sum of log-decays, the loss depends on
// s through y and hT only, and
//   dL/ds_t = dy_t . (y_t - D x_t) - x_t . (dx_t - D dy_t)    (+ <dhT, hT> at t = T-1)
// (each pair i >= j of the quadratic form contributes +W_ij at its row and -W_ij at its
// column); the log-decay of token t enters every s_u with u >= t, so
//   dL/d(dt_t A) = sum_{u >= t} dL/ds_u,   ddt_t = A dL/d(dt_t A),   dA = sum dt_t dL/d(dt_t A).
// k_bwd_x forms the per-token term from the fp32 accumulators of y - D x (recomputed)
// and dx - D dy; k_bwd_dt takes the reverse running sum.
//
// Kernels, in launch order after k_bprep (the forward's cumsum, C B^T in both
// orientations, B^T and C^T per chunk, in one launch) and the entering states H_c and
// final state hT (k_state + k_scan, or with many (b, h) chains k_states walking each
// chain's chunks with the state in registers):
//   k_state<ADJ>  adjoint chunk inputs S'_c                        -> states (reused)
//   k_scan_rev    R_c per chunk, dh0, partials of <R_c, H_{c+1}>     -> rin, dh0, kpart
//   k_bwd_x       dx, per-token decay term, D partial sums, per (b, h, c)
//   k_bwd_bc      dB and dC per (b, c, group, 64-row slab, n range)
//   k_bwd_dt      reverse running sums within each chunk from the boundary values
//                 <R_c, H_{c+1}> -> ddt, per-(b, h, c) A partial sums
//   k_bwd_reduce  dA, dD
#pragma once

#include "kernels.hpp"

namespace ssd {

// ---------------------------------------------------------------------------
// k_bprep: the tables a backward pass rebuilds, in one launch (the forward's k_prep does
// the same for its three).  They do not depend on one another, so one grid (chunks,
// tasks) runs them side by side, each task the work one block of the separate kernel
// does (the same arithmetic, so the same tables bit for bit):
//   y in [0, nh)                          k_cumsum's work for heads 16 y .. 16 y + 15
//   y in [nh, + npair G)                  k_cb's work, C B^T, block pair y % npair, group y / npair
//   y in [nh + npair G, + npair G)        the same transposed (B C^T, the input gradient's operand)
//   y in [nh + 2 npair G, + nslab G)      k_bt's work for B: B^T per chunk, and B by token if bcp
//   y in [nh + 2 npair G + nslab G, ...)  the same for C: C^T, and C by token if ccp
// (nh = ceil(H / 16), npair = nb (nb + 1) / 2 with nb = Q / 64, nslab = Q / 64.)
// ---------------------------------------------------------------------------
template <typename T, int N, int Q>
__global__ __launch_bounds__(kThreads) void k_bprep(const float* __restrict__ dt, float* __restrict__ cdt,
                                                    const T* __restrict__ Bm, const T* __restrict__ Cm,
                                                    T* __restrict__ cb, T* __restrict__ cbt, T* __restrict__ bt,
                                                    T* __restrict__ ct, T* __restrict__ bcp, T* __restrict__ ccp,
                                                    Rows rows, int G) {
    constexpr int nb = Q / 64, npair = nb * (nb + 1) / 2, nslab = Q / 64;
    constexpr size_t s1 = cumsum_smem<Q>(), s2 = cb_smem<T, N>(), s3 = bt_smem<T, N>();
    constexpr size_t SB = s1 > s2 ? (s1 > s3 ? s1 : s3) : (s2 > s3 ? s2 : s3);
    __shared__ __attribute__((aligned(16))) unsigned char smem[SB];
    const int nh = (rows.H + kCumsumHeads - 1) / kCumsumHeads;
    const int k = blockIdx.x;
    int y = blockIdx.y;
    if (y < nh) {
        cumsum_body<Q>(dt, cdt, rows, k, y, reinterpret_cast<float(*)[Q + 1]>(smem));
        return;
    }
    y -= nh;
    if (y < 2 * npair * G) {
        const bool tr = y >= npair * G;
        const int t = tr ? y - npair * G : y;
        if (tr) cb_body<T, N, true>(Bm, Cm, cbt, rows, G, Q, k, t % npair, t / npair, reinterpret_cast<T*>(smem));
        else cb_body<T, N, false>(Bm, Cm, cb, rows, G, Q, k, t % npair, t / npair, reinterpret_cast<T*>(smem));
        return;
    }
    y -= 2 * npair * G;
    const bool isc = y >= nslab * G;
    const int t = isc ? y - nslab * G : y;
    T* cp = isc ? ccp : bcp;
    const T* src = isc ? Cm : Bm;
    bt_body<T, N>(src, isc ? ct : bt, cp ? src : nullptr, cp, rows, G, Q, k, (t % nslab) * 64, t / nslab,
                  reinterpret_cast<T*>(smem));
}

// sum over the four lanes l16, l16 + 16, l16 + 32, l16 + 48 (one matrix-core column)
__device__ __forceinline__ float sum_q(float v) {
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}
__device__ __forceinline__ float sum_wave(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// ---------------------------------------------------------------------------
// k_scan_rev: the adjoint carried across chunks, last chunk first:
//   R = dhT;  for c = nc-1 .. 0: rin[c] = R;  R = exp(A cdt_last(c)) R + S'_c;  dh0 = R
// Parallel over b x H x P x N like k_scan (4 consecutive elements per thread), loads
// issued 8 chunks ahead.  On the way it forms the decay gradient's value at the start of
// chunk c + 1, <R_c, H_{c+1}> (H_nc = hT, the forward's final state, when dhT is given):
// each wave reduces its elements' share and writes one partial per chunk,
// kpart[b, h, c, (block part) * 4 + wave], summed in that order by k_bwd_dt.  (P N / 4
// is a multiple of 64, so every wave is either whole or absent.)  DIAG: each element
// decays at its own rate exp(A_{h,n} cdt_last); no boundary products (the diagonal
// backward forms them per dimension itself).
// ---------------------------------------------------------------------------
template <typename T, bool DIAG = false>
__global__ __launch_bounds__(kThreads) void k_scan_rev(const float* __restrict__ S, T* __restrict__ rin,
                                                       float* __restrict__ dh0, const float* __restrict__ dhT,
                                                       const float* __restrict__ A, const float* __restrict__ cdt,
                                                       const T* __restrict__ hin, const float* __restrict__ hTf,
                                                       float* __restrict__ kpart, int H, int PN, int N, int Q,
                                                       int nc, int per_head) {
    typedef typename V4<T>::type v4;
    const int64_t bh = blockIdx.x / per_head;
    const int part = (int)(blockIdx.x - bh * per_head);
    const int h = (int)(bh % H);
    const int e0 = (part * kThreads + threadIdx.x) * 4;
    if (e0 >= PN) return;
    const int lane = threadIdx.x & 63, slot = part * 4 + (int)(threadIdx.x >> 6), nslot = per_head * 4;
    // decay rate of each of the thread's 4 elements (4 consecutive n of one p)
    float a4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) a4[r] = DIAG ? A[(int64_t)h * N + (e0 + r) % N] : A[h];
    f32x4 st = dhT ? ld4(dhT + bh * PN + e0) : f32x4{0.f, 0.f, 0.f, 0.f};
    const float* cl = cdt + bh * (int64_t)nc * Q + (Q - 1);
    const float* sp = S + bh * (int64_t)nc * PN + e0;
    T* rp = rin + bh * (int64_t)nc * PN + e0;
    const T* hp = hin + bh * (int64_t)nc * PN + e0;
    float* kp = DIAG ? nullptr : kpart + bh * (int64_t)nc * nslot + slot;
    constexpr int DEPTH = 8;
    for (int c0 = nc - 1; c0 >= 0; c0 -= DEPTH) {
        f32x4 s[DEPTH];
        float Lc[DEPTH];
        f32x4 hn[DEPTH];  // H_{c+1}: the state entering the next chunk
#pragma unroll
        for (int k = 0; k < DEPTH; ++k) {
            const int c = c0 - k;
            if (c >= 0) {
                s[k] = ld4(sp + (int64_t)c * PN);
                Lc[k] = cl[(int64_t)c * Q];
                if (DIAG) {
                    hn[k] = f32x4{0.f, 0.f, 0.f, 0.f};
                } else if (c + 1 < nc) {
                    const v4 hv = ld4(hp + (int64_t)(c + 1) * PN);
#pragma unroll
                    for (int r = 0; r < 4; ++r) hn[k][r] = to_f(hv[r]);
                } else {
                    hn[k] = dhT ? ld4(hTf + bh * PN + e0) : f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
#pragma unroll
        for (int k = 0; k < DEPTH; ++k) {
            const int c = c0 - k;
            if (c >= 0) {
                v4 o;
#pragma unroll
                for (int r = 0; r < 4; ++r) o[r] = from_f<T>(st[r]);
                st4(rp + (int64_t)c * PN, o);
                if (!DIAG) {
                    float dot = 0.f;
#pragma unroll
                    for (int r = 0; r < 4; ++r) dot += st[r] * hn[k][r];
                    dot = sum_wave(dot);
                    if (lane == 0) kp[(int64_t)c * nslot] = dot;
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) st[r] = exp_f(a4[r] * Lc[k]) * st[r] + s[k][r];
            }
        }
    }
    if (dh0) st4(dh0 + bh * PN + e0, st);
}

// ---------------------------------------------------------------------------
// k_states: the forward state recurrence of one (b, h), walked chunk by chunk with the
// state held in registers: what k_state + k_scan compute, without the float32 chunk
// states going to HBM and back.
//   H = h0;  for c = 0 .. nc-1:  Hout[c] = H;  H = e^{A cdt_last} H + sum_j e^{A (cdt_last - cdt_j)} x_j B_j^T
//   fin = H (the final state)
// One work-group per (b, h), so it pays only with many (b, h) chains.  Within a chunk,
// 64-token slabs of x (weight applied while staging) and of B go through LDS as in
// k_state; the next slab's loads, across chunk boundaries too, are in flight during the
// current slab's matrix-core work.  (Walking the adjoint this way, with the boundary
// products, spilled and measured slower than k_state<ADJ> + k_scan_rev.)
// ---------------------------------------------------------------------------
template <typename T, int P, int N>
__global__ __launch_bounds__(kThreads, P * N <= 8192 ? 3 : 1) void k_states(const T* __restrict__ xin,
                                                                            const T* __restrict__ Bm,
                                                                            const float* __restrict__ A,
                                                                            const float* __restrict__ cdt,
                                                                            const float* __restrict__ init,
                                                                            T* __restrict__ Hout, float* __restrict__ fin,
                                                                            int64_t Tn, int H, int G, int Q, int nc) {
    typedef typename V8<T>::type v8;
    typedef typename V4<T>::type v4;
    typedef StateTiling<P, N> TL;
    constexpr int JB = 64, LDX = P + 8, LDB = N + 8, PN = P * N;
    constexpr int XV = JB * P / 8, BV = JB * N / 8;
    constexpr int XR = (XV + kThreads - 1) / kThreads, BR = (BV + kThreads - 1) / kThreads;
    __shared__ __attribute__((aligned(16))) T Xs[JB * LDX];
    __shared__ __attribute__((aligned(16))) T Bs[JB * LDB];
    __shared__ float cds[256];
    const int64_t bh = blockIdx.x;
    const int h = (int)(bh % H);
    const int64_t bi = bh / H;
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, q = lane >> 4;
    const float ah2 = A[h] * 1.4426950408889634f;
    const bool wact = TL::active(w);
    const int wn0 = TL::n0(w), wp0 = TL::p0(w);
    auto len_of = [&](int c) { return (int)((Tn - (int64_t)c * Q) < Q ? (Tn - (int64_t)c * Q) : Q); };

    // the state, in k_state's tile layout: lane holds S^T[n][p] for its tiles
    f32x4 acc[TL::WN][TL::WP];
#pragma unroll
    for (int a = 0; a < TL::WN; ++a)
#pragma unroll
        for (int b = 0; b < TL::WP; ++b) {
            const int p = (wp0 + b) * 16 + l16, n = (wn0 + a) * 16 + 4 * q;
            acc[a][b] = (wact && init) ? ld4(init + bh * PN + p * N + n) : f32x4{0.f, 0.f, 0.f, 0.f};
        }

    v8 xv[XR], bv[BR];
    float cdv = 0.f;
    auto prefetch = [&](int c, int j0) {
        const int64_t tok0 = (int64_t)c * Q;
        const int len = len_of(c);
        const T* xb = xin + ((bi * Tn + tok0) * H + h) * P;
        const T* bb = Bm + ((bi * Tn + tok0) * G + g) * N;
#pragma unroll
        for (int r = 0; r < XR; ++r) {
            const int v = tid + r * kThreads;
            const int jj = v / (P / 8), p0 = (v - jj * (P / 8)) * 8;
            const int jr = j0 + jj < len ? j0 + jj : len - 1;
            xv[r] = sel8(v < XV && j0 + jj < len, ld8(xb + (int64_t)jr * H * P + p0));
        }
#pragma unroll
        for (int r = 0; r < BR; ++r) {
            const int v = tid + r * kThreads;
            const int jj = v / (N / 8), n0 = (v - jj * (N / 8)) * 8;
            const int jr = j0 + jj < len ? j0 + jj : len - 1;
            bv[r] = sel8(v < BV && j0 + jj < len, ld8(bb + (int64_t)jr * G * N + n0));
        }
        if (j0 == 0 && tid < Q) cdv = cdt[(bh * nc + c) * (int64_t)Q + tid];
    };

    if (nc > 0) prefetch(0, 0);
    for (int c = 0; c < nc; ++c) {
        const int len = len_of(c);
        __syncthreads();  // the previous chunk is done with cds, Xs and Bs
        if (tid < Q) cds[tid] = cdv;
        // the state entering chunk c
        if (wact) {
            T* ho = Hout + (bh * nc + c) * (int64_t)PN;
#pragma unroll
            for (int a = 0; a < TL::WN; ++a)
#pragma unroll
                for (int b = 0; b < TL::WP; ++b) {
                    v4 o;
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] = from_f<T>(acc[a][b][r]);
                    st4(ho + ((wp0 + b) * 16 + l16) * N + (wn0 + a) * 16 + 4 * q, o);
                }
        }
        __syncthreads();  // cds in place
        const float last = cds[Q - 1];
        const float dch = exp2f_fast(ah2 * last);
#pragma unroll
        for (int a = 0; a < TL::WN; ++a)
#pragma unroll
            for (int b = 0; b < TL::WP; ++b) acc[a][b] *= dch;
        for (int j0 = 0; j0 < len; j0 += JB) {
            // slab j0 -> LDS, the weight of each token applied to its input row
#pragma unroll
            for (int r = 0; r < XR; ++r) {
                const int v = tid + r * kThreads;
                if (v < XV) {
                    const int jj = v / (P / 8), p0 = (v - jj * (P / 8)) * 8;
                    v8 o = xv[r];
                    const float wj = exp2f_fast(ah2 * (last - cds[j0 + jj]));
#pragma unroll
                    for (int e = 0; e < 8; ++e) o[e] = from_f<T>(to_f(o[e]) * wj);
                    st8(&Xs[jj * LDX + p0], o);
                }
            }
#pragma unroll
            for (int r = 0; r < BR; ++r) {
                const int v = tid + r * kThreads;
                if (v < BV) {
                    const int jj = v / (N / 8), n0 = (v - jj * (N / 8)) * 8;
                    st8(&Bs[jj * LDB + n0], bv[r]);
                }
            }
            __syncthreads();
            // the next slab: this chunk's, else the next chunk's first
            if (j0 + JB < len) prefetch(c, j0 + JB);
            else if (c + 1 < nc) prefetch(c + 1, 0);
            if (wact) {
#pragma unroll
                for (int kk = 0; kk < JB; kk += 32) {
                    v8 bf[TL::WP];
#pragma unroll
                    for (int b = 0; b < TL::WP; ++b) bf[b] = frag_rows(Xs, LDX, kk, (wp0 + b) * 16, lane);
#pragma unroll
                    for (int a = 0; a < TL::WN; ++a) {
                        const v8 af = frag_rows(Bs, LDB, kk, (wn0 + a) * 16, lane);
#pragma unroll
                        for (int b = 0; b < TL::WP; ++b) acc[a][b] = mma(acc[a][b], af, bf[b]);
                    }
                }
            }
            __syncthreads();
        }
    }
    if (fin && wact) {
#pragma unroll
        for (int a = 0; a < TL::WN; ++a)
#pragma unroll
            for (int b = 0; b < TL::WP; ++b)
                st4(fin + bh * PN + ((wp0 + b) * 16 + l16) * N + (wn0 + a) * 16 + 4 * q, acc[a][b]);
    }
}

// ---------------------------------------------------------------------------
// k_bwd_x: one (b, h, c) chunk of the input gradient and of the decay term.
//   phase 1  yhat^T[p][i] = sum_{j <= i} (L o C B^T)_ij x_j[p] + exp(A cdt_i) (H_c C_i)[p]
//            (y without the D term, fp32), then dy_i . yhat_i and dy_i . x_i.  (Not the
//            forward's stored y: y - D x from a bf16 y loses the bits of the state-space
//            part whenever D x dominates y.)
//   phase 2  dxhat^T[p][j] = sum_{i >= j} (L o C B^T)_ij dy_i[p] + exp(A (cdt_last - cdt_j)) (R_c B_j)[p]
//            then x_j . dxhat_j; ds_j = dy_j . yhat_j - x_j . dxhat_j; dx = dxhat + D dy
// One 64-token-major LDS tile holds x in phase 1 and dy in phase 2 (both read back as
// token-contiguous fragments by the LDS transpose read).  Phase 1 is k_out's output
// without D.  Phase 2 reads the transposed table cbt[j][i] = B_j . C_i so a lane's
// fragment holds 8 consecutive i of one column j; off the diagonal k-step the mask
// factors as exp(A (cdt_i - cdt_r)) exp(A (cdt_r - cdt_j)) with r the first token of
// the k-step (both <= 1).  Each wave owns the same row tiles in both phases (paired
// k, 7-k: the forward's causal work on a tile grows with its index and the backward's
// shrinks, so every tile costs the same), so the per-token sum needs no exchange.
// ---------------------------------------------------------------------------
template <typename T, int P>
struct BxSmem {
    static constexpr int LDX = P + 8;
    __host__ __device__ static size_t bytes(int Q) {
        return (size_t)Q * LDX * sizeof(T) + (size_t)3 * Q * sizeof(float) + 4 * sizeof(float);
    }
};

template <typename T, int P, int N>
__global__ __launch_bounds__(kThreads) void k_bwd_x(const T* __restrict__ x, const T* __restrict__ dy,
                                                    const T* __restrict__ Bm, const T* __restrict__ Cm,
                                                    const T* __restrict__ cb, const T* __restrict__ cbt,
                                                    const T* __restrict__ hin, const T* __restrict__ rin,
                                                    const float* __restrict__ A, const float* __restrict__ D,
                                                    const float* __restrict__ cdt, T* __restrict__ dx,
                                                    float* __restrict__ ds, float* __restrict__ dDp, int64_t Tn,
                                                    int H, int G, int Q, int nc) {
    typedef typename V8<T>::type v8;
    typedef typename V4<T>::type v4;
    constexpr int LDX = P + 8, PT = P / 16;
    constexpr float LOG2E = 1.4426950408889634f;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    T* Ts = reinterpret_cast<T*>(smem_raw);
    float* cds = reinterpret_cast<float*>(Ts + Q * LDX);
    float* u2 = cds + Q;   // exp(A (cdt_{j|31} - cdt_j)): from j to the end of its 32-token block
    float* v2 = u2 + Q;    // exp(A (cdt_i - cdt_{i&~31})): from the start of i's 32-token block to i
    float* red = v2 + Q;   // one partial sum per wave

    const int64_t blk = blockIdx.x;
    const int c = (int)(blk % nc);
    const int64_t bh = blk / nc;
    const int h = (int)(bh % H);
    const int64_t bi = bh / H;
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, q = lane >> 4;
    const int64_t tok0 = (int64_t)c * Q;
    const int len = (int)((Tn - tok0) < Q ? (Tn - tok0) : Q);
    const int rpw = Q / 64;
    const int KS = Q / 32;
    const T* xb = x + ((bi * Tn + tok0) * H + h) * P;     // row j at + j * H * P
    const T* dyb = dy + ((bi * Tn + tok0) * H + h) * P;
    const T* crow = Cm + ((bi * Tn + tok0) * G + g) * N;  // row i at + i * G * N
    const T* brow = Bm + ((bi * Tn + tok0) * G + g) * N;
    const T* hbase = hin + (bh * nc + c) * (int64_t)(P * N);
    const T* rbase = rin + (bh * nc + c) * (int64_t)(P * N);
    const float* cd = cdt + (bh * nc + c) * (int64_t)Q;
    const float ah2 = A[h] * LOG2E;
    const float Dh = D ? D[h] : 0.f;

    auto row_tile = [&](int k) { return (rpw == 1) ? w : ((k & 1) ? 8 * (k >> 1) + 7 - w : 8 * (k >> 1) + w); };

    constexpr int XR = (256 * P / 8 + kThreads - 1) / kThreads;  // enough for Q = 256
    const int XV = Q * P / 8;
    v8 rv[XR];
    auto load_rows = [&](const T* base) {
#pragma unroll
        for (int r = 0; r < XR; ++r) {
            const int v = tid + r * kThreads;
            const int jj = v / (P / 8), p0 = (v - jj * (P / 8)) * 8;
            const int jr = jj < len ? jj : len - 1;
            rv[r] = sel8(v < XV && jj < len, ld8(base + (int64_t)jr * H * P + p0));
        }
    };
    auto store_rows = [&]() {
#pragma unroll
        for (int r = 0; r < XR; ++r) {
            const int v = tid + r * kThreads;
            if (v < XV) {
                const int jj = v / (P / 8), p0 = (v - jj * (P / 8)) * 8;
                st8(&Ts[jj * LDX + p0], rv[r]);
            }
        }
    };
    // state term, raw: acc^T[p][t] += sum_n S[p][n] V_t[n] for the wave's row tiles t
    // (S = H_c with V = C in phase 1, S = R_c with V = B in phase 2)
    f32x4 acc[4][PT];
    auto state_term = [&](const T* sbase, const T* vrow) {
#pragma unroll
        for (int n0 = 0; n0 < N; n0 += 32) {
            const int nn = n0 + 8 * q;
            const bool nv = (N % 32 == 0) || (nn < N);  // N = 16: half the k-step is padding
            v8 hf[PT], cf[4];
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) hf[pt] = sel8(nv, ld8(sbase + (pt * 16 + l16) * N + (nv ? nn : 0)));
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = row_tile(k) * 16 + l16;
                const int ir = i < len ? i : len - 1;
                cf[k] = sel8(k < rpw && nv && i < len, ld8(vrow + (int64_t)ir * G * N + (nv ? nn : 0)));
            }
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (k < rpw)
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) acc[k][pt] = mma(acc[k][pt], hf[pt], cf[k]);
        }
    };

    float p1[4];
    float dd = 0.f;
    // ---- phase 1: yhat ----
    load_rows(xb);
    const float cdv = tid < Q ? cd[tid] : 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[k][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
    state_term(hbase, crow);
    store_rows();
    if (tid < Q) cds[tid] = cdv;
    __syncthreads();
    if (tid < Q) {
        u2[tid] = exp2f_fast(ah2 * (cds[tid | 31] - cds[tid]));
        v2[tid] = exp2f_fast(ah2 * (cds[tid] - cds[tid & ~31]));
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k)
        if (k < rpw) {
            const float sc = exp2f_fast(ah2 * cds[row_tile(k) * 16 + l16]);
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) acc[k][pt] *= sc;
        }
    const T* cbb = cb + ((bi * nc + c) * G + g) * (int64_t)Q * Q;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (k < rpw) {
            const int rt = row_tile(k);
            const int i = rt * 16 + l16;
            const int nks = rt / 2 + 1;  // k-steps of 32 tokens up to this row tile
            v8 gf[8];
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) gf[ks] = ld8(cbb + tfrag(i, (ks < nks ? ks : nks - 1) * 32 + 8 * q, Q));
            const float ci = cds[i];
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                if (ks < nks) {
                    const int j0 = ks * 32 + 8 * q;
                    v8 mf;
                    if (ks < nks - 1) {
                        const float vi = exp2f_fast(ah2 * (ci - cds[ks * 32 + 31]));
#pragma unroll
                        for (int e = 0; e < 8; ++e) mf[e] = from_f<T>(to_f(gf[ks][e]) * (u2[j0 + e] * vi));
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int j = j0 + e;
                            const float m = to_f(gf[ks][e]) * exp2f_fast(fminf(ah2 * (ci - cds[j]), 0.f));
                            mf[e] = from_f<T>(j <= i ? m : 0.f);
                        }
                    }
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt)
                        acc[k][pt] = mma(acc[k][pt], frag_rows(Ts, LDX, ks * 32, pt * 16, lane), mf);
                }
            }
        }
    }
    // dy_i . yhat_i per row (lane (i, q) holds p = 16 pt + 4 q + r), and dy . x for dD
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        p1[k] = 0.f;
        if (k < rpw) {
            const int i = row_tile(k) * 16 + l16;
            float s = 0.f;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                v4 dv;
                if (i < len) dv = ld4(dyb + (int64_t)i * H * P + pt * 16 + 4 * q);
                else
#pragma unroll
                    for (int r = 0; r < 4; ++r) dv[r] = from_f<T>(0.f);
                const v4 xv = ld4(&Ts[i * LDX + pt * 16 + 4 * q]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    s += to_f(dv[r]) * acc[k][pt][r];
                    dd += to_f(dv[r]) * to_f(xv[r]);
                }
            }
            p1[k] = sum_q(s);
        }
    }
    __syncthreads();  // every wave is done with the x tile

    // ---- phase 2: dxhat ----
    load_rows(dyb);
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[k][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
    state_term(rbase, brow);
    store_rows();
    __syncthreads();
    const float clast = cds[Q - 1];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        if (k < rpw) {
            const float sc = exp2f_fast(ah2 * (clast - cds[row_tile(k) * 16 + l16]));
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) acc[k][pt] *= sc;
        }
    const T* cbtb = cbt + ((bi * nc + c) * G + g) * (int64_t)Q * Q;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (k < rpw) {
            const int rt = row_tile(k);
            const int j = rt * 16 + l16;
            const int kd = rt / 2;  // the k-step holding row tile rt
            v8 gf[8];
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) gf[ks] = ld8(cbtb + tfrag(j, ((ks >= kd && ks < KS) ? ks : kd) * 32 + 8 * q, Q));
            const float cj = cds[j];
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                if (ks >= kd && ks < KS) {
                    const int i0 = ks * 32 + 8 * q;
                    v8 mf;
                    if (ks > kd) {
                        const float wj = exp2f_fast(ah2 * (cds[ks * 32] - cj));
#pragma unroll
                        for (int e = 0; e < 8; ++e) mf[e] = from_f<T>(to_f(gf[ks][e]) * (v2[i0 + e] * wj));
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int i = i0 + e;
                            const float m = to_f(gf[ks][e]) * exp2f_fast(fminf(ah2 * (cds[i] - cj), 0.f));
                            mf[e] = from_f<T>(i >= j ? m : 0.f);
                        }
                    }
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt)
                        acc[k][pt] = mma(acc[k][pt], frag_rows(Ts, LDX, ks * 32, pt * 16, lane), mf);
                }
            }
        }
    }
    // ds_j = dy_j . yhat_j - x_j . dxhat_j; then dx = dxhat + D dy
    float* dsb = ds + (bh * nc + c) * (int64_t)Q;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (k < rpw) {
            const int j = row_tile(k) * 16 + l16;
            float s = 0.f;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                v4 xv;
                if (j < len) xv = ld4(xb + (int64_t)j * H * P + pt * 16 + 4 * q);
                else
#pragma unroll
                    for (int r = 0; r < 4; ++r) xv[r] = from_f<T>(0.f);
                const v4 dv = ld4(&Ts[j * LDX + pt * 16 + 4 * q]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    s += to_f(xv[r]) * acc[k][pt][r];
                    acc[k][pt][r] += Dh * to_f(dv[r]);
                }
            }
            s = sum_q(s);
            if (q == 0) dsb[j] = p1[k] - s;
        }
    }
    dd = sum_wave(dd);
    if (lane == 0) red[w] = dd;
    __syncthreads();  // every wave is done with the dy tile
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (k < rpw) {
            const int j = row_tile(k) * 16 + l16;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                v4 o;
#pragma unroll
                for (int r = 0; r < 4; ++r) o[r] = from_f<T>(acc[k][pt][r]);
                st4(&Ts[j * LDX + pt * 16 + 4 * q], o);
            }
        }
    }
    __syncthreads();
    if (tid == 0) dDp[bh * nc + c] = (red[0] + red[1]) + (red[2] + red[3]);
    T* dxb = dx + ((bi * Tn + tok0) * H + h) * P;
    for (int v = tid; v < len * (P / 8); v += kThreads) {
        const int jj = v / (P / 8), p0 = (v - jj * (P / 8)) * 8;
        st8(dxb + (int64_t)jj * H * P + p0, ld8(&Ts[jj * LDX + p0]));
    }
}

// ---------------------------------------------------------------------------
// k_bwd_xs: what k_bwd_x computes, for bfloat16 at headdim 64 and dstate 64 or 128, laid
// out like the fused forward kernel: the chunk's x (then dy) rows and its entering state
// H_c (then the adjoint R_c) go straight into swizzled LDS tiles by direct transfers, so no
// register holds them in flight; each wave then takes its row tiles one at a time (one
// tile's accumulators live, not four), its state term from the LDS state tile and its
// diagonal block from the C B^T (or transposed) table in L2, and dx leaves in whole rows.
// Its LDS fits three work-groups per CU.  Per row tile, phase 1 keeps only dy_i . yhat_i (a
// scalar per row) for phase 2's decay term.
// ---------------------------------------------------------------------------
template <int Q, int N>
struct BxsCfg {
    static constexpr int P = 64;
    static constexpr int RPW = Q / 64;          // row tiles per wave
    static constexpr int KS = Q / 32;           // 32-token k-steps per chunk
    static constexpr int NF = N / 32;           // 32-wide n-steps of the state term
};

// Registers: at chunk 256 two work-groups per CU (226 registers, no spills; within the 168
// that a third allows it spilled 49 per lane, which measured 150 us slower at the 2.7B layer
// shape); smaller chunks fit three.
template <int Q, int N>
__global__ __launch_bounds__(kThreads, Q >= 256 ? 2 : 3) void k_bwd_xs(const bf16* __restrict__ x, const bf16* __restrict__ dy,
                                                     const bf16* __restrict__ Bf, const bf16* __restrict__ Cf,
                                                     const bf16* __restrict__ cb, const bf16* __restrict__ cbt,
                                                     const bf16* __restrict__ hin, const bf16* __restrict__ rin,
                                                     const float* __restrict__ A, const float* __restrict__ D,
                                                     const float* __restrict__ cdt, bf16* __restrict__ dx,
                                                     float* __restrict__ ds, float* __restrict__ dDp, int64_t Tn,
                                                     int H, int G, int nc) {
    typedef BxsCfg<Q, N> CF;
    constexpr int P = 64, RPW = CF::RPW, KS = CF::KS, NF = CF::NF;
    constexpr int PN = P * N;
    constexpr float LOG2E = 1.4426950408889634f;
    __shared__ __attribute__((aligned(16))) bf16 Ts[Q * P];   // x rows, then dy rows (swizzled)
    __shared__ __attribute__((aligned(16))) bf16 Hs[P * N];   // H_c, then R_c (chunks swizzled by row)
    __shared__ float cds[Q], u2[Q], v2[Q], red[4];

    const int64_t blk = blockIdx.x;
    const int c = (int)(blk % nc);
    const int64_t bh = blk / nc;
    const int h = (int)(bh % H);
    const int64_t bi = bh / H;
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), l16 = lane & 15, q = lane >> 4;
    const float ah2 = A[h] * LOG2E;
    const float Dh = D ? D[h] : 0.f;

    // buffer resources based at this batch row (rows past T read as zero, stores dropped),
    // the group's tables and this chain's states
    const int XS = H * P * 2;  // x / dy / dx row stride in bytes
    const uint32_t xbytes = (uint32_t)(Tn * H * P * 2);
    const brsrc rx = make_rsrc(x + bi * Tn * H * P, xbytes);
    const brsrc rdy = make_rsrc(dy + bi * Tn * H * P, xbytes);
    const brsrc rdx = make_rsrc(dx + bi * Tn * H * P, xbytes);
    // B and C per chunk by token, in fragment order (tokens past T hold zeros)
    const uint32_t fbytes = (uint32_t)((int64_t)nc * G * Q * N * 2);
    const brsrc rc = make_rsrc(Cf + bi * nc * G * Q * N, fbytes);
    const brsrc rb = make_rsrc(Bf + bi * nc * G * Q * N, fbytes);
    const uint32_t tbytes = (uint32_t)((int64_t)nc * G * Q * Q * 2);
    const brsrc rcb = make_rsrc(cb + bi * nc * G * Q * Q, tbytes);
    const brsrc rcbt = make_rsrc(cbt + bi * nc * G * Q * Q, tbytes);
    const uint32_t sbytes = (uint32_t)((int64_t)nc * PN * 2);
    const brsrc rh = make_rsrc(hin + bh * nc * PN, sbytes);
    const brsrc rr = make_rsrc(rin + bh * nc * PN, sbytes);
    const int hcol = h * P * 2;
    const int tab0 = (c * G + g) * Q * Q * 2;                    // this chunk's table, bytes

    // the chunk's rows (x or dy) and a state tile (H_c or R_c) into LDS, this wave's share
    auto stage = [&](brsrc rrows, brsrc rstate) {
        dma_rows_state<Q, N>(Ts, Hs, rrows, c * Q * XS, XS, hcol, rstate, c * PN * 2, w);
    };
    auto row_tile = [&](int k) { return (RPW == 1) ? w : ((k & 1) ? 8 * (k >> 1) + 7 - w : 8 * (k >> 1) + w); };
    // state term of one row tile: acc^T[p][t] = sum_n S[p][n] V_t[n] (S in Hs, V = C or B
    // rows; each 16 x 32 fragment one contiguous 1 KB run)
    auto state_term = [&](f32x4* acc, brsrc rv, int rt) {
        bf16x8 vf[NF];
        const int sv = __builtin_amdgcn_readfirstlane(((c * G + g) * Q * N + rt * (N / 32) * 512) * 2);
#pragma unroll
        for (int n = 0; n < NF; ++n) vf[n] = bload8(rv, lane * 16, sv + n * 1024);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int n = 0; n < NF; ++n)
#pragma unroll
            for (int pt = 0; pt < 4; ++pt)
                acc[pt] = mma(acc[pt], ld8(Hs + hs_off<N>(pt * 16 + l16, n * 32 + 8 * q)), vf[n]);
    };

    // ---- phase 1: yhat ----
    stage(rx, rh);
    if (tid < Q) {
        const float* cd = cdt + (bh * nc + c) * (int64_t)Q;
        const float cv = cd[tid], cr = cd[tid | 31], cs = cd[tid & ~31];
        cds[tid] = cv;
        u2[tid] = exp2f_fast(ah2 * (cr - cv));  // exp(A (cdt_{j|31} - cdt_j))
        v2[tid] = exp2f_fast(ah2 * (cv - cs));  // exp(A (cdt_i - cdt_{i&~31}))
    }
    __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): this wave's transfers have landed
    __syncthreads();                    // ... every wave's, and the tables are in place
    float p1[RPW];
    float dd = 0.f;
#pragma unroll
    for (int k = 0; k < RPW; ++k) {
        const int rt = row_tile(k), i = rt * 16 + l16, nks = rt / 2 + 1;
        bf16x8 gf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            if (ks < nks) gf[ks] = bload8(rcb, lane * 16, __builtin_amdgcn_readfirstlane(tab0 + (rt * (Q / 32) + ks) * 1024));
        // the tile's dy rows for dy_i . yhat_i, requested with the tile's other operands
        const int sy = __builtin_amdgcn_readfirstlane((c * Q + rt * 16) * XS);
        bf16x4 dv[4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
            dv[pt] = __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(
                                                    rdy, l16 * XS + hcol + (pt * 16 + 4 * q) * 2, sy, 0));
        f32x4 acc[4];
        state_term(acc, rc, rt);
        const float ci = cds[i];
        const float sc = exp2f_fast(ah2 * ci);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc[pt] *= sc;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks < nks) {
                const int j0 = ks * 32 + 8 * q;
                bf16x8 mf;
                if (ks < nks - 1) {
                    const float vi = exp2f_fast(ah2 * (ci - cds[ks * 32 + 31]));
#pragma unroll
                    for (int e = 0; e < 8; ++e) mf[e] = (bf16)((float)gf[ks][e] * (u2[j0 + e] * vi));
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int j = j0 + e;
                        const float m = (float)gf[ks][e] * exp2f_fast(fminf(ah2 * (ci - cds[j]), 0.f));
                        mf[e] = (bf16)(j <= i ? m : 0.f);
                    }
                }
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) acc[pt] = mma(acc[pt], frag_xs(Ts, ks * 32, pt * 16, lane), mf);
                __builtin_amdgcn_sched_barrier(0);  // (hoisting every k-step's reads spills)
            }
        }
        // dy_i . yhat_i (lane (i, q) holds p = 16 pt + 4 q + r), and dy . x for dD
        float s = 0.f;
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
            const bf16x4 xv = ld4(Ts + xs_off(i, pt * 16 + 4 * q));
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                s += (float)dv[pt][r] * acc[pt][r];
                dd += (float)dv[pt][r] * (float)xv[r];
            }
        }
        p1[k] = sum_q(s);
        __builtin_amdgcn_sched_barrier(0);  // one row tile's operands in flight at a time
    }
    // dD's partial now (left for the end, its operands would stay live through phase 2)
    dd = sum_wave(dd);
    if (lane == 0) red[w] = dd;
    __syncthreads();  // every wave is done with the x rows and H_c

    // ---- phase 2: dxhat, the decay term, dx ----
    stage(rdy, rr);
    __builtin_amdgcn_s_waitcnt(0xF70);
    __syncthreads();
    const float clast = cds[Q - 1];
    float* dsb = ds + (bh * nc + c) * (int64_t)Q;
#pragma unroll
    for (int k = 0; k < RPW; ++k) {
        const int rt = row_tile(k), j = rt * 16 + l16, kd = rt / 2;  // kd: the k-step holding the tile
        bf16x8 gf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            if (ks >= kd) gf[ks] = bload8(rcbt, lane * 16, __builtin_amdgcn_readfirstlane(tab0 + (rt * (Q / 32) + ks) * 1024));
        // the tile's x rows for x_j . dxhat_j, requested with the tile's other operands
        const int sx = __builtin_amdgcn_readfirstlane((c * Q + rt * 16) * XS);
        bf16x4 xv[4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
            xv[pt] = __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(
                                                    rx, l16 * XS + hcol + (pt * 16 + 4 * q) * 2, sx, 0));
        f32x4 acc[4];
        state_term(acc, rb, rt);
        const float cj = cds[j];
        const float sc = exp2f_fast(ah2 * (clast - cj));
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc[pt] *= sc;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks >= kd) {
                const int i0 = ks * 32 + 8 * q;
                bf16x8 mf;
                if (ks > kd) {
                    const float wj = exp2f_fast(ah2 * (cds[ks * 32] - cj));
#pragma unroll
                    for (int e = 0; e < 8; ++e) mf[e] = (bf16)((float)gf[ks][e] * (v2[i0 + e] * wj));
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int i = i0 + e;
                        const float m = (float)gf[ks][e] * exp2f_fast(fminf(ah2 * (cds[i] - cj), 0.f));
                        mf[e] = (bf16)(i >= j ? m : 0.f);
                    }
                }
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) acc[pt] = mma(acc[pt], frag_xs(Ts, ks * 32, pt * 16, lane), mf);
                __builtin_amdgcn_sched_barrier(0);  // (hoisting every k-step's reads spills)
            }
        }
        // ds_j = dy_j . yhat_j - x_j . dxhat_j; dx = dxhat + D dy
        float s = 0.f;
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
            const bf16x4 dv = ld4(Ts + xs_off(j, pt * 16 + 4 * q));
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                s += (float)xv[pt][r] * acc[pt][r];
                acc[pt][r] += Dh * (float)dv[r];
            }
        }
        s = sum_q(s);
        if (q == 0) dsb[j] = p1[k] - s;
        store_tile16(acc, rdx, sx, XS, hcol);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (tid == 0) dDp[bh * nc + c] = (red[0] + red[1]) + (red[2] + red[3]);
}

// ---------------------------------------------------------------------------
// k_bwd_bc: dB and dC of one (b, c, group) chunk, for the 64-row slab s of tokens and
// the n range [n0, n0 + NB).  Loop over the group's heads:
//   W   += L^h o (dy^h x^h^T)  on the tiles a slab needs: rows i in the slab with
//          j <= i (for dC) and columns j in the slab with i >= j (for dB); fp32, each
//          16x16 tile owned by one wave (u = w, w + 4, ...).  Off the diagonal tile
//          the decay factors as exp(A(cdt_i - cdt_I0)) exp(A(cdt_I0 - cdt_J15))
//          exp(A(cdt_J15 - cdt_j)) (I0 first row of i's tile, J15 last of j's), all <= 1.
//   dC^T[n][i] += sum_p H_c^h[p][n] exp(A cdt_i) dy_i^h[p]          (wave w: rows of tile 4s + w)
//   dB^T[n][j] += sum_p R_c^h[p][n] exp(A (cdt_last - cdt_j)) x_j^h[p]
// then, once per group: dC^T += B^T W^T (W rows of the slab, k over j), dB^T += C^T W
// (W columns of the slab, k over i), with W staged in LDS in the operand dtype and
// B^T, C^T from the per-chunk transposed tables.  H_c^h and R_c^h are staged in LDS per
// head (the next head's prefetched into registers meanwhile) and read with the
// transpose read, p running down the rows.
// ---------------------------------------------------------------------------
constexpr int kBcThreads = 512;  // k_bwd_bc work-groups: 8 waves (16 measured slower: spills at 128 VGPRs)

template <typename T, int P, int NB>
struct BcSmem {
    static constexpr int PR = P < 32 ? 32 : P;  // rows past P stay zero (k-step padding)
    static constexpr int LDH = NB + 8;
    static constexpr int LDY = PR + 8;          // dy / x rows of one head
    static constexpr int LDW = 72;              // W columns of the slab
    __host__ __device__ static constexpr int ldc(int Q) { return Q + 8; }  // W rows of the slab
    // H and R tiles, then the head's dy rows [64 s, Q) and x rows [0, 64 s + 64)
    __host__ __device__ static constexpr size_t phase1(int Q) {
        return ((size_t)2 * PR * LDH + (size_t)(Q + 64) * LDY) * sizeof(T);
    }
    __host__ __device__ static constexpr size_t phase2(int Q) {
        return ((size_t)64 * ldc(Q) + (size_t)Q * LDW) * sizeof(T);
    }
    __host__ __device__ static constexpr size_t region(int Q) { return phase1(Q) > phase2(Q) ? phase1(Q) : phase2(Q); }
    __host__ __device__ static constexpr size_t bytes(int Q) { return region(Q) + (size_t)5 * Q * sizeof(float); }
};

// n range of one k_bwd_bc work-group: the widest (up to 128) whose LDS fits one CU at
// chunk 256, else at chunk 128 (larger chunks are then reported unsupported)
template <typename T, int P, int N>
constexpr int bc_nb() {
    constexpr size_t lim = 160 * 1024;
    for (int Q = 256; Q >= 128; Q /= 2) {
        if (N >= 128 && BcSmem<T, P, 128>::bytes(Q) <= lim) return 128;
        if (N >= 64 && BcSmem<T, P, 64>::bytes(Q) <= lim) return 64;
        if (N >= 32 && BcSmem<T, P, 32>::bytes(Q) <= lim) return 32;
        if (BcSmem<T, P, 16>::bytes(Q) <= lim) return 16;
    }
    return 16;
}

template <typename T, int P, int N, int NB>
__global__ __launch_bounds__(kBcThreads) void k_bwd_bc(const T* __restrict__ x, const T* __restrict__ dy,
                                                     const T* __restrict__ bt, const T* __restrict__ ct,
                                                     const T* __restrict__ hin, const T* __restrict__ rin,
                                                     const float* __restrict__ A, const float* __restrict__ cdt,
                                                     T* __restrict__ dB, T* __restrict__ dC, int64_t Tn, int H,
                                                     int G, int Q, int nc) {
    typedef typename V8<T>::type v8;
    typedef typename V4<T>::type v4;
    typedef BcSmem<T, P, NB> SM;
    constexpr int PR = SM::PR, LDH = SM::LDH, LDY = SM::LDY, LDW = SM::LDW, NBT = NB / 16, NR = N / NB;
    constexpr int NW = kBcThreads / 64;           // 8 waves
    constexpr int NTW = (58 + NW - 1) / NW;       // W tiles per wave at Q = 256 (58 tiles)
    // state terms and products: wave w takes row tile w % 4 of the slab and n tiles
    // [nb0, nb0 + NBH) of the range, NBH = NBT / NSP (one tile when NBT < NSP)
    constexpr int NSP = NW / 4;                   // n-tile splits
    constexpr int NBH = NBT >= NSP ? NBT / NSP : 1;
    constexpr float LOG2E = 1.4426950408889634f;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    T* Hs = reinterpret_cast<T*>(smem_raw);
    T* Rs = Hs + PR * LDH;
    T* Ys = Rs + PR * LDH;  // dy row i at Ys[(i - 64 s) * LDY], i in [64 s, Q)
    T* Wc = reinterpret_cast<T*>(smem_raw);  // phase 2: [64][Q + 8]  W rows i of the slab, all j
    T* Wb = Wc + 64 * SM::ldc(Q);            //          [Q][72]      W rows i >= slab start, columns of the slab
    float* cdh = reinterpret_cast<float*>(smem_raw + SM::region(Q));
    float* es = cdh + Q;   // exp(A (cdt_i - cdt_{i & ~15}))
    float* ee = es + Q;    // exp(A (cdt_{j | 15} - cdt_j))
    float* sci = ee + Q;   // exp(A cdt_i)
    float* scj = sci + Q;  // exp(A (cdt_last - cdt_j))

    const int nslab = Q / 64;
    // blocks k, k+8, k+16, ... run on one XCD: give each XCD a contiguous range of the
    // (b, c, g, slab, n range) grid, so that the slabs of one chunk, which stage the same
    // heads' H, R, dy and x tiles, share an L2
    int64_t blk = blockIdx.x;
    if (gridDim.x % 8 == 0) blk = (blk % 8) * (gridDim.x / 8) + blk / 8;
    const int nr = (int)(blk % NR);
    blk /= NR;
    const int s = (int)(blk % nslab);
    blk /= nslab;
    const int g = (int)(blk % G);
    blk /= G;
    const int c = (int)(blk % nc);
    const int64_t bi = blk / nc;
    const int n0 = nr * NB;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, q = lane >> 4;
    const int64_t tok0 = (int64_t)c * Q;
    const int len = (int)((Tn - tok0) < Q ? (Tn - tok0) : Q);
    const int hpg = H / G, hbeg = g * hpg;
    const int NT = 16 * nslab - 6;  // W tiles the slab needs
    const int s64 = 64 * s;
    T* Xs = Ys + (Q - s64) * LDY;  // x row j at Xs[j * LDY], j in [0, 64 s + 64)
    const int NY = Q - s64, NX = s64 + 64;  // staged dy rows, x rows

    // tile u -> (I, J): first the rows of the slab (J <= I), then the columns of the slab
    // below it
    auto tile_ij = [&](int u, int& I, int& J) {
        const int nA = 16 * s + 10;
        if (u < nA) {
            int a = 0, base = 0;
            while (a < 3 && u >= base + 4 * s + a + 1) {
                base += 4 * s + a + 1;
                ++a;
            }
            I = 4 * s + a;
            J = u - base;
        } else {
            const int v = u - nA;
            I = 4 * s + 4 + v / 4;
            J = 4 * s + (v & 3);
        }
    };

    // rows past P of the staged tiles and columns past P of the staged rows stay zero
    for (int v = tid; v < (PR - P) * LDH; v += kBcThreads) {
        Hs[P * LDH + v] = from_f<T>(0.f);
        Rs[P * LDH + v] = from_f<T>(0.f);
    }
    if (PR > P)
        for (int v = tid; v < (NY + NX) * (PR - P); v += kBcThreads)
            Ys[(v / (PR - P)) * LDY + P + v % (PR - P)] = from_f<T>(0.f);

    constexpr int HV = P * NB / 8;
    constexpr int HR = (HV + kBcThreads - 1) / kBcThreads;
    constexpr int RV = (256 + 64) * P / 8;          // dy + x row vectors at Q = 256 (at most)
    constexpr int RR = (RV + kBcThreads - 1) / kBcThreads;
    const int nrv = (NY + NX) * (P / 8);
    v8 hv[HR], rv[HR], yv[RR];
    float cv = 0.f, c0v = 0.f, c15v = 0.f, clv = 0.f;
    auto prefetch = [&](int hh) {
        const int64_t bhh = bi * H + hh;
        const T* hb = hin + (bhh * nc + c) * (int64_t)(P * N) + n0;
        const T* rb = rin + (bhh * nc + c) * (int64_t)(P * N) + n0;
#pragma unroll
        for (int r = 0; r < HR; ++r) {
            const int v = tid + r * kBcThreads;
            const int pp = v / (NB / 8), nn = (v - pp * (NB / 8)) * 8;
            if (v < HV) {
                hv[r] = ld8(hb + pp * N + nn);
                rv[r] = ld8(rb + pp * N + nn);
            }
        }
        // the head's dy rows [64 s, Q), then its x rows [0, 64 s + 64); rows past T are zero
        const T* xh = x + ((bi * Tn + tok0) * H + hh) * P;
        const T* dyh = dy + ((bi * Tn + tok0) * H + hh) * P;
#pragma unroll
        for (int r = 0; r < RR; ++r) {
            const int v = tid + r * kBcThreads;
            const int row = v / (P / 8), pp = (v - row * (P / 8)) * 8;
            const bool isy = row < NY;
            const int tok = isy ? s64 + row : row - NY;
            const bool ok = v < nrv && tok < len;
            const T* src = (isy ? dyh : xh) + (int64_t)(ok ? tok : 0) * H * P + pp;
            yv[r] = sel8(ok, ld8(src));
        }
        const float* cd = cdt + (bhh * nc + c) * (int64_t)Q;
        if (tid < Q) {
            cv = cd[tid];
            c0v = cd[tid & ~15];
            c15v = cd[tid | 15];
            clv = cd[Q - 1];
        }
    };
    float ah2 = 0.f;
    auto stage = [&](int hh) {
#pragma unroll
        for (int r = 0; r < HR; ++r) {
            const int v = tid + r * kBcThreads;
            const int pp = v / (NB / 8), nn = (v - pp * (NB / 8)) * 8;
            if (v < HV) {
                st8(&Hs[pp * LDH + nn], hv[r]);
                st8(&Rs[pp * LDH + nn], rv[r]);
            }
        }
#pragma unroll
        for (int r = 0; r < RR; ++r) {
            const int v = tid + r * kBcThreads;
            const int row = v / (P / 8), pp = (v - row * (P / 8)) * 8;
            if (v < nrv) st8(&Ys[row * LDY + pp], yv[r]);  // Xs follows Ys row for row
        }
        ah2 = A[hh] * LOG2E;
        if (tid < Q) {
            cdh[tid] = cv;
            es[tid] = exp2f_fast(ah2 * (cv - c0v));
            ee[tid] = exp2f_fast(ah2 * (c15v - cv));
            sci[tid] = exp2f_fast(ah2 * cv);
            scj[tid] = exp2f_fast(ah2 * (clv - cv));
        }
    };

    f32x4 accW[NTW], accC[NBH], accB[NBH];
#pragma unroll
    for (int m = 0; m < NTW; ++m) accW[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < NBH; ++nt) accC[nt] = accB[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int rt = w & 3, nh = w >> 2;             // row tile, n-tile split
    const bool sact = nh < NBT / NBH;              // (fewer n tiles than splits: the rest idle)
    const int nb0 = nh * NBH;                      // first n tile of this wave
    const int iw = s64 + rt * 16 + l16;            // this wave's row (dC) and column (dB) token

    prefetch(hbeg);
    for (int hh = hbeg; hh < hbeg + hpg; ++hh) {
        __syncthreads();  // the previous head's tiles and tables are no longer read
        stage(hh);
        __syncthreads();
        if (hh + 1 < hbeg + hpg) prefetch(hh + 1);

        // W tiles of this head, decay-masked, summed into accW
#pragma unroll
        for (int m = 0; m < NTW; ++m) {
            const int u = w + NW * m;
            if (u < NT) {
                int I, J;
                tile_ij(u, I, J);
                const int i = I * 16 + l16, j = J * 16 + l16;
                f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int p0 = 0; p0 < PR; p0 += 32)
                    t = mma(t, ld8(&Ys[(i - s64) * LDY + p0 + 8 * q]), ld8(&Xs[j * LDY + p0 + 8 * q]));
                // lane: W[I*16 + 4q + r][J*16 + l16]
                if (I > J) {
                    const float f = exp2f_fast(ah2 * (cdh[I * 16] - cdh[J * 16 + 15])) * ee[J * 16 + l16];
#pragma unroll
                    for (int r = 0; r < 4; ++r) accW[m][r] += t[r] * (es[I * 16 + 4 * q + r] * f);
                } else {
                    const float cj = cdh[J * 16 + l16];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int ii = I * 16 + 4 * q + r;
                        const float L = exp2f_fast(fminf(ah2 * (cdh[ii] - cj), 0.f));
                        accW[m][r] += (ii >= J * 16 + l16) ? t[r] * L : 0.f;
                    }
                }
            }
        }

        // state terms: this wave's 16 tokens, its half of the n tiles of the range
        const float si = sci[iw], sj = scj[iw];
#pragma unroll
        for (int p0 = 0; p0 < PR; p0 += 32) {
            if (!sact) break;
            v8 yb = ld8(&Ys[(iw - s64) * LDY + p0 + 8 * q]);
            v8 xb8 = ld8(&Xs[iw * LDY + p0 + 8 * q]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                yb[e] = from_f<T>(to_f(yb[e]) * si);
                xb8[e] = from_f<T>(to_f(xb8[e]) * sj);
            }
#pragma unroll
            for (int nt = 0; nt < NBH; ++nt) {
                accC[nt] = mma(accC[nt], frag_rows(Hs, LDH, p0, (nb0 + nt) * 16, lane), yb);
                accB[nt] = mma(accB[nt], frag_rows(Rs, LDH, p0, (nb0 + nt) * 16, lane), xb8);
            }
        }
    }

    // ---- once per group: W through LDS, then the products with B^T and C^T ----
    __syncthreads();  // every wave is done with the staged H and R tiles
    {
        const int nvec = (int)(SM::phase2(Q) / 16);
        u32x4v* z = reinterpret_cast<u32x4v*>(smem_raw);
        for (int v = tid; v < nvec; v += kBcThreads) z[v] = u32x4v{0u, 0u, 0u, 0u};
    }
    __syncthreads();
    const int ldc = SM::ldc(Q);
#pragma unroll
    for (int m = 0; m < NTW; ++m) {
        const int u = w + NW * m;
        if (u < NT) {
            int I, J;
            tile_ij(u, I, J);
            const int j = J * 16 + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = I * 16 + 4 * q + r;
                const T v = from_f<T>(accW[m][r]);
                if (I >= 4 * s && I < 4 * s + 4) Wc[(i - s64) * ldc + j] = v;
                if (J >= 4 * s && J < 4 * s + 4) Wb[(i - s64) * LDW + (j - s64)] = v;
            }
        }
    }
    __syncthreads();
    const T* btb = bt + ((bi * nc + c) * G + g) * (int64_t)N * Q;  // [n][j], fragment order
    const T* ctb = ct + ((bi * nc + c) * G + g) * (int64_t)N * Q;
    if (!sact) return;
    for (int j0 = 0; j0 < s64 + 64; j0 += 32) {
        const v8 wf = ld8(&Wc[(iw - s64) * ldc + j0 + 8 * q]);
#pragma unroll
        for (int nt = 0; nt < NBH; ++nt)
            accC[nt] = mma(accC[nt], ld8(btb + tfrag(n0 + (nb0 + nt) * 16 + l16, j0 + 8 * q, Q)), wf);
    }
    for (int i0 = s64; i0 < Q; i0 += 32) {
        const v8 wf = frag_rows(Wb, LDW, i0 - s64, rt * 16, lane);
#pragma unroll
        for (int nt = 0; nt < NBH; ++nt)
            accB[nt] = mma(accB[nt], ld8(ctb + tfrag(n0 + (nb0 + nt) * 16 + l16, i0 + 8 * q, Q)), wf);
    }
    if (iw < len) {
        T* dCr = dC + ((bi * Tn + tok0 + iw) * G + g) * N + n0;
        T* dBr = dB + ((bi * Tn + tok0 + iw) * G + g) * N + n0;
#pragma unroll
        for (int nt = 0; nt < NBH; ++nt) {
            v4 oc, ob;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                oc[r] = from_f<T>(accC[nt][r]);
                ob[r] = from_f<T>(accB[nt][r]);
            }
            st4(dCr + (nb0 + nt) * 16 + 4 * q, oc);
            st4(dBr + (nb0 + nt) * 16 + 4 * q, ob);
        }
    }
}

// ---------------------------------------------------------------------------
// k_bwd_bcs: what k_bwd_bc computes, for bfloat16 at headdim 64 (n range NB = 64 or 128),
// with each head's operands -- its dy rows [64 s, Q) and x rows [0, 64 s + 64), its H_c and
// R_c tiles over the n range, its cdt row -- brought straight into LDS by direct transfers,
// into one of two buffers: while the work-group computes one head from a buffer, the next
// head's transfers land in the other.  (k_bwd_bc stages each head through registers one
// head ahead, so it waits for every head's loads.)  The rows sit in xs_off's swizzled
// layout; the H and R tiles in 64-column sub-tiles of the same layout (rows p), read as
// transposed fragments.  The two buffers are separate arrays, so reads of one never wait
// for the transfers into the other.
// ---------------------------------------------------------------------------
constexpr int kBcsThreads = 1024;  // k_bwd_bcs work-groups: 16 waves

template <int Q, int NB>
struct BcsCfg {
    static constexpr int ROWS = Q + 64;                        // staged rows per head
    static constexpr int RT = ROWS / 8;                        // 1 KB row transfers per head
    static constexpr int NSUB = NB / 64;                       // 64-column sub-tiles of H (and of R)
    static constexpr int ST = 2 * NSUB * 8;                    // state transfers per head
    static constexpr int TPW = (RT + ST + 15) / 16;            // transfers per wave (16 waves)
    static constexpr int BUF = ROWS * 64 + 2 * NSUB * 64 * 64; // bf16 elements of one buffer
    static constexpr int LDC = Q + 8, LDW = 72;                // W rows of the slab, W columns of the slab
    static_assert(64 * LDC <= BUF && Q * LDW <= BUF, "the W staging fits one buffer each");
};

template <int Q, int N, int NB>
__global__ __launch_bounds__(kBcsThreads) void k_bwd_bcs(const bf16* __restrict__ x, const bf16* __restrict__ dy,
                                                      const bf16* __restrict__ bt, const bf16* __restrict__ ct,
                                                      const bf16* __restrict__ hin, const bf16* __restrict__ rin,
                                                      const float* __restrict__ A, const float* __restrict__ cdt,
                                                      bf16* __restrict__ dB, bf16* __restrict__ dC, int64_t Tn,
                                                      int H, int G, int nc) {
    typedef BcsCfg<Q, NB> CF;
    constexpr int P = 64, ROWS = CF::ROWS, RT = CF::RT, NSUB = CF::NSUB, TPW = CF::TPW, BUF = CF::BUF;
    constexpr int LDC = CF::LDC, LDW = CF::LDW, NBT = NB / 16, NR = N / NB, PN = P * N;
    constexpr int NW = kBcsThreads / 64;                 // 16 waves
    constexpr int nslab = Q / 64;
    constexpr int NTMAX = 16 * nslab - 6;                // W tiles a slab needs
    constexpr int NTW = (NTMAX + NW - 1) / NW;
    constexpr int NSP = NW / 4;                          // n-tile splits of the state terms
    constexpr int NBH = NBT >= NSP ? NBT / NSP : 1;
    constexpr float LOG2E = 1.4426950408889634f;
    __shared__ __attribute__((aligned(16))) bf16 buf0[BUF];
    __shared__ __attribute__((aligned(16))) bf16 buf1[BUF];
    __shared__ __attribute__((aligned(16))) float cdq0[Q];
    __shared__ __attribute__((aligned(16))) float cdq1[Q];
    __shared__ float cdh[Q], es[Q], ee[Q], sci[Q], scj[Q];

    // work item (b, c, g, slab, n range); each XCD takes a contiguous range, so the slabs
    // of one chunk, which stage the same heads' rows and tiles, share an L2
    int64_t blk = blockIdx.x;
    if (gridDim.x % 8 == 0) blk = (blk % 8) * (gridDim.x / 8) + blk / 8;
    const int nr = (int)(blk % NR);
    blk /= NR;
    const int s = (int)(blk % nslab);
    blk /= nslab;
    const int g = (int)(blk % G);
    blk /= G;
    const int c = (int)(blk % nc);
    const int64_t bi = blk / nc;
    const int n0 = nr * NB;
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), l16 = lane & 15, q = lane >> 4;
    const int64_t tok0 = (int64_t)c * Q;
    const int len = (int)((Tn - tok0) < Q ? (Tn - tok0) : Q);
    const int hpg = H / G, hbeg = g * hpg, hend = hbeg + hpg;
    const int s64 = 64 * s, NY = Q - s64;  // dy row i at tile row i - 64 s; x row j at tile row NY + j

    // buffer resources based at this batch row: rows past T read as zero
    const int XS = H * P * 2;
    const uint32_t xbytes = (uint32_t)(Tn * H * P * 2);
    const brsrc rx = make_rsrc(x + bi * Tn * H * P, xbytes);
    const brsrc rdy = make_rsrc(dy + bi * Tn * H * P, xbytes);
    const uint32_t sbytes = (uint32_t)((int64_t)H * nc * PN * 2);
    const brsrc rh = make_rsrc(hin + bi * H * nc * PN, sbytes);
    const brsrc rr = make_rsrc(rin + bi * H * nc * PN, sbytes);
    const brsrc rcd = make_rsrc(cdt + bi * H * nc * Q, (uint32_t)((int64_t)H * nc * Q * 4));

    // head hh's transfers into buffer bb and its cdt row into cq; the caller waits (vmcnt)
    // and synchronises before reading them
    auto issue = [&](int hh, bf16* bb, float* cq) {
        int ln = lane_now();  // rebuilt per call, not kept live
        const int hcol = hh * P * 2;
        const int vr0 = xs_dma_lane(ln, 0, XS, hcol), vr1 = xs_dma_lane(ln, 1, XS, hcol);
        const int vs0 = xs_dma_lane(ln, 0, N * 2, n0 * 2), vs1 = xs_dma_lane(ln, 1, N * 2, n0 * 2);
        const int st0 = (hh * nc + c) * PN * 2;  // the head's state tile within the batch row, bytes
#pragma unroll
        for (int r = 0; r < TPW; ++r) {
            const int m = w * TPW + r;
            if (m >= RT + CF::ST) {
            } else if (m < RT) {
                // rows 8 m .. 8 m + 7 of the row tile: dy rows first, then x rows (NY is a
                // multiple of 64, so no transfer mixes the two)
                const bool isy = 8 * m < NY;
                const int tok = isy ? s64 + 8 * m : 8 * m - NY;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(isy ? rdy : rx,
                                                         (__attribute__((address_space(3))) void*)(bb + m * 512), 16,
                                                         xs_dma_bit(m) ? vr1 : vr0,
                                                         __builtin_amdgcn_readfirstlane((c * Q + tok) * XS), 0, 0);
            } else {
                // state transfer k: tensor k / (8 NSUB) (H, R), sub-tile (k / 8) % NSUB, rows 8 (k % 8) ..
                const int k = m - RT, t = k / (8 * NSUB), sub = (k / 8) % NSUB, mm = k % 8;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    t ? rr : rh,
                    (__attribute__((address_space(3))) void*)(bb + ROWS * 64 + (t * NSUB + sub) * 4096 + mm * 512), 16,
                    (xs_dma_bit(mm) ? vs1 : vs0) + sub * 128,
                    __builtin_amdgcn_readfirstlane(st0 + 8 * mm * N * 2), 0, 0);
            }
        }
        if (w == 0 && ln * 4 < Q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rcd, (__attribute__((address_space(3))) void*)cq, 16, ln * 16,
                                                     __builtin_amdgcn_readfirstlane((hh * nc + c) * Q * 4), 0, 0);
    };
    // the head's decay tables from its cdt row
    auto tables = [&](int hh, const float* cq) {
        if (tid < Q) {
            const float ah2 = A[hh] * LOG2E;
            const float cv = cq[tid], c0v = cq[tid & ~15], c15v = cq[tid | 15], clv = cq[Q - 1];
            cdh[tid] = cv;
            es[tid] = exp2f_fast(ah2 * (cv - c0v));
            ee[tid] = exp2f_fast(ah2 * (c15v - cv));
            sci[tid] = exp2f_fast(ah2 * cv);
            scj[tid] = exp2f_fast(ah2 * (clv - cv));
        }
    };

    // tile u -> (I, J): first the rows of the slab (J <= I), then the columns of the slab
    // below it
    auto tile_ij = [&](int u, int& I, int& J) {
        const int nA = 16 * s + 10;
        if (u < nA) {
            int a = 0, base = 0;
            while (a < 3 && u >= base + 4 * s + a + 1) {
                base += 4 * s + a + 1;
                ++a;
            }
            I = 4 * s + a;
            J = u - base;
        } else {
            const int v = u - nA;
            I = 4 * s + 4 + v / 4;
            J = 4 * s + (v & 3);
        }
    };

    f32x4 accW[NTW], accC[NBH], accB[NBH];
#pragma unroll
    for (int m = 0; m < NTW; ++m) accW[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < NBH; ++nt) accC[nt] = accB[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int rt = w & 3, nh = w >> 2;  // row tile of the slab, n-tile split
    const bool sact = nh < NBT / NBH;   // (fewer n tiles than splits: the rest idle)
    const int nb0 = nh * NBH;           // first n tile of this wave
    const int iw = s64 + rt * 16 + l16; // this wave's row (dC) and column (dB) token

    // this wave's W tiles (the same for every head; wave-uniform)
    int tI[NTW], tJ[NTW];
#pragma unroll
    for (int m = 0; m < NTW; ++m) {
        tI[m] = tJ[m] = 0;
        if (w + NW * m < NTMAX) tile_ij(w + NW * m, tI[m], tJ[m]);
    }

    // one head from buffer bb: W tiles, decay-masked, into accW; the state terms
    auto compute = [&](int hh, const bf16* bb) {
        const float ah2 = A[hh] * LOG2E;
        const bf16* Ys = bb;                 // the staged rows
        const bf16* Hs = bb + ROWS * 64;     // H sub-tiles, then R sub-tiles
        const bf16* Rs = Hs + NSUB * 4096;
#pragma unroll
        for (int m = 0; m < NTW; ++m) {
            const int u = w + NW * m;
            if (u < NTMAX) {
                const int I = tI[m], J = tJ[m];
                const int i = I * 16 + l16, j = J * 16 + l16;
                f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int p0 = 0; p0 < P; p0 += 32)
                    t = mma(t, ld8(Ys + xs_off(i - s64, p0 + 8 * q)), ld8(Ys + xs_off(NY + j, p0 + 8 * q)));
                // lane: W[I*16 + 4q + r][J*16 + l16]
                if (I > J) {
                    const float f = exp2f_fast(ah2 * (cdh[I * 16] - cdh[J * 16 + 15])) * ee[J * 16 + l16];
#pragma unroll
                    for (int r = 0; r < 4; ++r) accW[m][r] += t[r] * (es[I * 16 + 4 * q + r] * f);
                } else {
                    const float cj = cdh[J * 16 + l16];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int ii = I * 16 + 4 * q + r;
                        const float L = exp2f_fast(fminf(ah2 * (cdh[ii] - cj), 0.f));
                        accW[m][r] += (ii >= J * 16 + l16) ? t[r] * L : 0.f;
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);  // one tile's fragments in flight at a time
        }
        // state terms: this wave's 16 tokens, its share of the n tiles of the range
        if (sact) {
            const float si = sci[iw], sj = scj[iw];
#pragma unroll
            for (int p0 = 0; p0 < P; p0 += 32) {
                bf16x8 yb = ld8(Ys + xs_off(iw - s64, p0 + 8 * q));
                bf16x8 xb8 = ld8(Ys + xs_off(NY + iw, p0 + 8 * q));
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    yb[e] = (bf16)((float)yb[e] * si);
                    xb8[e] = (bf16)((float)xb8[e] * sj);
                }
#pragma unroll
                for (int nt = 0; nt < NBH; ++nt) {
                    const int nn = (nb0 + nt) * 16, sub = nn / 64, cc = nn % 64;
                    accC[nt] = mma(accC[nt], frag_xs(Hs + sub * 4096, p0, cc, lane), yb);
                    accB[nt] = mma(accB[nt], frag_xs(Rs + sub * 4096, p0, cc, lane), xb8);
                }
            }
        }
    };

    issue(hbeg, buf0, cdq0);
    for (int hh = hbeg; hh < hend; hh += 2) {
        __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): this wave's transfers of head hh
        __syncthreads();                    // ... every wave's; every wave is done with head hh - 1
        tables(hh, cdq0);
        __syncthreads();
        if (hh + 1 < hend) issue(hh + 1, buf1, cdq1);
        __builtin_amdgcn_sched_barrier(0);
        compute(hh, buf0);
        __builtin_amdgcn_sched_barrier(0);
        if (hh + 1 < hend) {
            __builtin_amdgcn_s_waitcnt(0xF70);
            __syncthreads();
            tables(hh + 1, cdq1);
            __syncthreads();
            if (hh + 2 < hend) issue(hh + 2, buf0, cdq0);
            __builtin_amdgcn_sched_barrier(0);
            compute(hh + 1, buf1);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // ---- once per group: W through LDS (W rows of the slab in buf0, W columns of the slab
    //      in buf1), then the products with B^T and C^T ----
    bf16* Wc = buf0;  // [64][Q + 8]  W rows i of the slab, all j
    bf16* Wb = buf1;  // [Q][72]      W rows i >= slab start, columns of the slab
    __syncthreads();  // every wave is done with the last head's buffer
    for (int v = tid; v < 64 * LDC / 8; v += kBcsThreads) reinterpret_cast<u32x4v*>(Wc)[v] = u32x4v{0u, 0u, 0u, 0u};
    for (int v = tid; v < Q * LDW / 8; v += kBcsThreads) reinterpret_cast<u32x4v*>(Wb)[v] = u32x4v{0u, 0u, 0u, 0u};
    __syncthreads();
    const int NT = NTMAX;
#pragma unroll
    for (int m = 0; m < NTW; ++m) {
        const int u = w + NW * m;
        if (u < NT) {
            int I, J;
            tile_ij(u, I, J);
            const int j = J * 16 + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = I * 16 + 4 * q + r;
                const bf16 v = (bf16)accW[m][r];
                if (I >= 4 * s && I < 4 * s + 4) Wc[(i - s64) * LDC + j] = v;
                if (J >= 4 * s && J < 4 * s + 4) Wb[(i - s64) * LDW + (j - s64)] = v;
            }
        }
    }
    __syncthreads();
    const bf16* btb = bt + ((bi * nc + c) * G + g) * (int64_t)N * Q;  // [n][j], fragment order
    const bf16* ctb = ct + ((bi * nc + c) * G + g) * (int64_t)N * Q;
    if (!sact) return;
    for (int j0 = 0; j0 < s64 + 64; j0 += 32) {
        const bf16x8 wf = ld8(&Wc[(iw - s64) * LDC + j0 + 8 * q]);
#pragma unroll
        for (int nt = 0; nt < NBH; ++nt)
            accC[nt] = mma(accC[nt], ld8(btb + tfrag(n0 + (nb0 + nt) * 16 + l16, j0 + 8 * q, Q)), wf);
    }
    for (int i0 = s64; i0 < Q; i0 += 32) {
        const bf16x8 wf = frag_rows(Wb, LDW, i0 - s64, rt * 16, lane);
#pragma unroll
        for (int nt = 0; nt < NBH; ++nt)
            accB[nt] = mma(accB[nt], ld8(ctb + tfrag(n0 + (nb0 + nt) * 16 + l16, i0 + 8 * q, Q)), wf);
    }
    if (iw < len) {
        bf16* dCr = dC + ((bi * Tn + tok0 + iw) * G + g) * N + n0;
        bf16* dBr = dB + ((bi * Tn + tok0 + iw) * G + g) * N + n0;
#pragma unroll
        for (int nt = 0; nt < NBH; ++nt) {
            bf16x4 oc, ob;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                oc[r] = (bf16)accC[nt][r];
                ob[r] = (bf16)accB[nt][r];
            }
            st4(dCr + (nb0 + nt) * 16 + 4 * q, oc);
            st4(dBr + (nb0 + nt) * 16 + 4 * q, ob);
        }
    }
}

// ---------------------------------------------------------------------------
// k_bwd_dt: dl_t = dL/d(dt_t A) = sum_{u >= t} ds_u + <dhT, hT>, ddt_t = A dl_t, and
// partials sum_t dt_t dl_t of dA.
// The running sum restarts at every chunk: at the first token of chunk c + 1, dl equals
// the inner product of the adjoint arriving at the end of chunk c from later tokens with
// the state entering chunk c + 1, <R_c, H_{c+1}> (H_nc = hT, R_{nc-1} = dhT), so within
// chunk c dl_t = <R_c, H_{c+1}> + sum_{u = t}^{chunk end} ds_u.  Rounding of the
// per-token terms then accumulates over at most one chunk instead of the whole sequence.
// k_scan_rev leaves the boundary products as per-wave partials.  One work-group per
// (batch, chunk), one thread per head walking the chunk backward, so each step writes
// the heads of one token side by side.
// ---------------------------------------------------------------------------
template <int BLOCK = 128>
__global__ __launch_bounds__(BLOCK) void k_bwd_dt(const float* __restrict__ ds, const float* __restrict__ dt,
                                                  const float* __restrict__ A, const float* __restrict__ kpart,
                                                  float* __restrict__ ddt, float* __restrict__ dAp, int64_t Tn,
                                                  int H, int Q, int nc, int nslot, int nvalid) {
    const int c = (int)(blockIdx.x % nc);
    const int64_t bi = blockIdx.x / nc;
    const int64_t t0 = (int64_t)c * Q;
    const int len = (int)((Tn - t0) < Q ? (Tn - t0) : Q);
    for (int h = threadIdx.x; h < H; h += BLOCK) {
        const int64_t bh = bi * H + h;
        const float* kp = kpart + (bh * nc + c) * (int64_t)nslot;
        float run = 0.f;
        for (int i = 0; i < nvalid; ++i) run += kp[i];
        const float* d = ds + (bh * nc + c) * (int64_t)Q;
        const float Ah = A[h];
        float da = 0.f;
        // the running sum is serial; its operands are requested DEPTH tokens at a time
        constexpr int DEPTH = 16;
        for (int i0 = len - 1; i0 >= 0; i0 -= DEPTH) {
            float dv[DEPTH], tv[DEPTH];
#pragma unroll
            for (int k = 0; k < DEPTH; ++k) {
                const int i = i0 - k >= 0 ? i0 - k : 0;
                dv[k] = d[i];
                tv[k] = dt[(bi * Tn + t0 + i) * H + h];
            }
#pragma unroll
            for (int k = 0; k < DEPTH; ++k) {
                if (i0 - k >= 0) {
                    run += dv[k];
                    const int64_t o = (bi * Tn + t0 + i0 - k) * H + h;
                    ddt[o] = Ah * run;
                    da += tv[k] * run;
                }
            }
        }
        dAp[bh * nc + c] = da;
    }
}

// dA[h] = sum_{b, c} dAp[b, h, c];  dD[h] = sum_{b, c} dDp[b, h, c].  One work-group per
// head; each thread sums a fixed strided subset, then a fixed reduction tree, so the
// result does not depend on scheduling.
__device__ __forceinline__ float block_sum(float v, float* part) {  // part: >= 16 floats
    v = sum_wave(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
    __syncthreads();
    float t = 0.f;
    for (int k = 0; k < (int)(blockDim.x >> 6); ++k) t += part[k];
    return t;
}

template <int BLOCK = kThreads>
__global__ __launch_bounds__(BLOCK) void k_bwd_reduce(const float* __restrict__ dAp,
                                                         const float* __restrict__ dDp, float* __restrict__ dA,
                                                         float* __restrict__ dD, int64_t b, int H, int nc) {
    __shared__ float part[16];
    const int h = blockIdx.x;
    const int64_t n = b * nc;  // (batch, chunk) terms of this head
    float a = 0.f, d = 0.f;
    for (int64_t k = threadIdx.x; k < n; k += BLOCK) {
        const int64_t bi = k / nc, c = k - bi * nc;
        a += dAp[(bi * H + h) * nc + c];
        d += dDp[(bi * H + h) * nc + c];
    }
    a = block_sum(a, part);
    d = block_sum(d, part);
    if (threadIdx.x == 0) {
        dA[h] = a;
        if (dD) dD[h] = d;
    }
}

}  // namespace ssd
