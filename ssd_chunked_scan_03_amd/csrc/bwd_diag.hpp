// bwd_diag.hpp -- backward pass of the diagonal-decay SSD scan (a_{t,n} = exp(dt_t A_{h,n})).
//
// "Structured State Space Duality" concept page, the diagonal generalisation: every state
// dimension n of a head is its own scalar-decay recurrence over the head's P channels,
//   h_t[:, n] = a_{t,n} h_{t-1}[:, n] + x_t B_{t,n},   y_t = sum_n C_{t,n} h_t[:, n] + D x_t.
// The pages give no backward algorithm; this one follows the chunked evaluation of the
// forward.  Across chunks it uses the forward's chunk states and their scan (H_c entering
// chunk c, hT), and the same scan run backward for the adjoint (R_c: the gradient of the
// state after chunk c's last token coming from the tokens after it, R_{nc-1} = dhT).
// Within a chunk each (batch, head) walks its tokens: forward from H_c, and backward from
// R_c with the adjoint g_t = dy_t C_t^T + a_{t+1} g_{t+1}, so that per token
//   Zh_{t,n} = dy_t . h_t[:, n]      (h_t the state after token t)
//   Yh_{t,n} = x_t . g_t[:, n]       (g_t the gradient of h_t)
//   dx_t     = sum_n g_t[:, n] B_{t,n} + D dy_t
// and, summed over the heads of a group, dC = sum_h Zh, dB = sum_h Yh.
//
// Decay gradient.  With s_{t,n} the running sum of log-decays of dimension n, every pair
// i >= j of the quadratic form contributes at its row and, with the opposite sign, at its
// column (the per-dimension form of the scalar identity), so
//   dL/ds_{t,n} = C_{t,n} Zh_{t,n} - B_{t,n} Yh_{t,n}    (+ <dhT, hT>_n at t = T-1),
// and the log-decay of token t enters s_{u,n} for every u >= t:
//   dl_{t,n} = <R_c[:, n], H_{c+1}[:, n]> + sum_{u >= t in chunk c} dL/ds_{u,n}
// (the first term is the sum over every later token, and <dhT, hT>_n, written as the
// chunk boundary's product), ddt_t = sum_n A_{h,n} dl_{t,n}, dA_{h,n} = sum_t dt_t dl_{t,n}.
//
// Kernels, after k_cumsum, k_state + k_scan (H_c, hT) and k_state<ADJ> + k_scan_rev<DIAG>
// (R_c, dh0):
//   k_bwd_diag         one wave per (batch, head, chunk, slice of dstate): both walks of
//                      the chunk, writing Zh, Yh, dx (or per-slice partials), ddt (or
//                      per-slice partials) and per-chunk partial sums of dA and dD
//   k_bwd_diag_bc      dB, dC: head sums of Yh, Zh per group, in head order
//   k_bwd_diag_fin     dx and ddt from the per-slice partials (dstate split over waves)
//   k_bwd_diag_reduce  dA [H, N] and dD [H]: sums over (batch, chunk) in a fixed order
#pragma once

#include "kernels.hpp"

namespace ssd {

// K consecutive elements at p (16-byte aligned when K * sizeof(T) is a multiple of 16,
// else aligned to K * sizeof(T)) as floats
template <int K>
__device__ __forceinline__ void ldk(const bf16* p, float* o) {
    if constexpr (K % 8 == 0) {
#pragma unroll
        for (int v = 0; v < K / 8; ++v) {
            const bf16x8 t = ld8(p + 8 * v);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[8 * v + e] = (float)t[e];
        }
    } else if constexpr (K == 4) {
        const bf16x4 t = ld4(p);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (float)t[e];
    } else {
        static_assert(K == 2, "ldk: K in {2, 4, 8k}");
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 t = *reinterpret_cast<const bf16x2*>(p);
        o[0] = (float)t[0];
        o[1] = (float)t[1];
    }
}
template <int K>
__device__ __forceinline__ void ldk(const float* p, float* o) {
    if constexpr (K % 4 == 0) {
#pragma unroll
        for (int v = 0; v < K / 4; ++v) {
            const f32x4 t = ld4(p + 4 * v);
#pragma unroll
            for (int e = 0; e < 4; ++e) o[4 * v + e] = t[e];
        }
    } else {
        static_assert(K == 2, "ldk: K in {2, 4k}");
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        const f32x2 t = *reinterpret_cast<const f32x2*>(p);
        o[0] = t[0];
        o[1] = t[1];
    }
}
template <int K>
__device__ __forceinline__ void stk(float* p, const float* v) {
    if constexpr (K % 4 == 0) {
#pragma unroll
        for (int u = 0; u < K / 4; ++u) st4(p + 4 * u, f32x4{v[4 * u], v[4 * u + 1], v[4 * u + 2], v[4 * u + 3]});
    } else {
        static_assert(K == 2, "stk: K in {2, 4k}");
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        *reinterpret_cast<f32x2*>(p) = f32x2{v[0], v[1]};
    }
}
template <int K>
__device__ __forceinline__ void stk(bf16* p, const float* v) {
    if constexpr (K % 4 == 0) {
#pragma unroll
        for (int u = 0; u < K / 4; ++u)
            st4(p + 4 * u, bf16x4{(bf16)v[4 * u], (bf16)v[4 * u + 1], (bf16)v[4 * u + 2], (bf16)v[4 * u + 3]});
    } else {
        static_assert(K == 2, "stk: K in {2, 4k}");
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        *reinterpret_cast<bf16x2*>(p) = bf16x2{(bf16)v[0], (bf16)v[1]};
    }
}

// Work split of one (batch, head, chunk): a wave holds a P x NS block of the state, NS =
// dstate or a slice of it so that every lane holds at most 64 elements and at most 8
// dimensions (each dimension costs a lane its decay rate, running sums and row values).
// Lane (pg, ng) = (lane / 8, lane % 8) holds channels pg PP .. +PP and dimensions
// ng NN .. +NN of the slice.
template <int P, int N>
struct DiagSplit {
    static constexpr int NS = N < 64 ? (N < 4096 / P ? N : 4096 / P) : (64 < 4096 / P ? 64 : 4096 / P);
    static constexpr int NSL = N / NS;
    static constexpr int PP = P / 8, NN = NS / 8;
    static_assert(NS % 16 == 0 && NSL * NS == N && PP >= 2, "dstate slice");
};

// Lane sums without LDS memory: DPP moves within a row of 16 lanes (quad_perm [1,0,3,2]
// and [2,3,0,1] pair lanes l ^ 1 and l ^ 2; row_half_mirror pairs the two quads of each
// 8-lane half, whose quad sums are by then uniform; row_ror:8 pairs l ^ 8), a ds_swizzle
// for l ^ 16 within each 32-lane half, and a cross-half permute for l ^ 32.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// sum over the 8 lanes of one dimension group (lanes ng, ng + 8, ..., ng + 56)
__device__ __forceinline__ float sum_pg(float v) {
    v += dpp_f<0x128>(v);  // row_ror:8
    v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));  // l ^ 16
    return v + __shfl_xor(v, 32, 64);
}
// sum over the 8 lanes of one channel group (lanes 8 pg .. 8 pg + 7)
__device__ __forceinline__ float sum_ng(float v) {
    v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
    return v + dpp_f<0x141>(v);  // row_half_mirror
}

// ---------------------------------------------------------------------------
// k_bwd_diag: one wave per (batch, head, chunk, dstate slice); waves are independent
// (no LDS, no barriers).  Wave index order: slice, head, chunk, batch (fastest first),
// so the waves of a work-group share the chunk's B and C rows in the caches.
//   zh, yh  [b, H, nc, Q, N] float32  (Zh, Yh of every token)
//   dx      [b, T, H, P] (problem dtype; NSL == 1) or dxp [NSL, b, T, H, P] float32 partials
//   ddt     [b, T, H] (NSL == 1) or ddtp [NSL, b, T, H] float32 partials
//   dAp     [b, H, nc, N], dDp [b, H, nc]: per-chunk partial sums
// hin / rin hold H_c / R_c in the problem dtype; hTf is the forward's final state (read
// when dhT is given: the last chunk's boundary product is <dhT, hT>).
// ---------------------------------------------------------------------------
template <typename T, int P, int N>
__global__ __launch_bounds__(kThreads) void k_bwd_diag(
    const T* __restrict__ x, const T* __restrict__ dy, const T* __restrict__ Bm, const T* __restrict__ Cm,
    const float* __restrict__ dt, const float* __restrict__ A, const float* __restrict__ D,
    const T* __restrict__ hin, const T* __restrict__ rin, const float* __restrict__ hTf, bool have_dhT,
    float* zh, float* yh, T* __restrict__ dx, float* __restrict__ dxp, float* __restrict__ ddt,
    float* __restrict__ ddtp, float* __restrict__ dAp, float* __restrict__ dDp, int64_t nb, int64_t Tn, int H, int G,
    int Q, int nc, int64_t nwaves) {
    typedef DiagSplit<P, N> S;
    constexpr int PP = S::PP, NN = S::NN, NS = S::NS, NSL = S::NSL;
    constexpr float LOG2E = 1.4426950408889634f;
    const int64_t wv = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (wv >= nwaves) return;  // whole waves only: no barrier below
    const int lane = threadIdx.x & 63, pg = lane >> 3, ng = lane & 7;
    const int sl = (int)(wv % NSL);
    const int h = (int)((wv / NSL) % H);
    const int c = (int)((wv / ((int64_t)NSL * H)) % nc);
    const int64_t bi = wv / ((int64_t)NSL * H * nc);
    const int g = h / (H / G);
    const int64_t bh = bi * H + h, bhc = bh * nc + c;
    const int64_t tok0 = (int64_t)c * Q;
    const int len = (int)((Tn - tok0) < Q ? (Tn - tok0) : Q);
    const int p0 = pg * PP, n0 = sl * NS + ng * NN;  // this lane's first channel and dimension

    float an2[NN], An[NN];
#pragma unroll
    for (int k = 0; k < NN; ++k) {
        An[k] = A[(int64_t)h * N + n0 + k];
        an2[k] = An[k] * LOG2E;
    }
    const int64_t rowx = H * P, rowb = (int64_t)G * N;
    const T* xr = x + ((bi * Tn + tok0) * H + h) * P + p0;    // token t at + t * rowx
    const T* dyr = dy + ((bi * Tn + tok0) * H + h) * P + p0;
    const T* br = Bm + ((bi * Tn + tok0) * G + g) * N + n0;   // token t at + t * rowb
    const T* cr = Cm + ((bi * Tn + tok0) * G + g) * N + n0;
    const float* dtr = dt + (bi * Tn + tok0) * H + h;          // token t at + t * H
    float* zr = zh + bhc * Q * N + n0;                         // token t at + t * N
    float* yr = yh + bhc * Q * N + n0;
    const int64_t PN = (int64_t)P * N;

    float st[PP][NN];
    // ---- forward walk from H_c: Zh_t = dy_t . h_t ----
#pragma unroll
    for (int i = 0; i < PP; ++i) ldk<NN>(hin + bhc * PN + (int64_t)(p0 + i) * N + n0, st[i]);
    for (int t = 0; t < len; ++t) {
        float xv[PP], dv[PP], bv[NN];
        ldk<PP>(xr + t * rowx, xv);
        ldk<PP>(dyr + t * rowx, dv);
        ldk<NN>(br + t * rowb, bv);
        const float dtv = dtr[(int64_t)t * H];
        float z[NN];
#pragma unroll
        for (int k = 0; k < NN; ++k) {
            const float a = exp2f_fast(an2[k] * dtv);
            z[k] = 0.f;
#pragma unroll
            for (int i = 0; i < PP; ++i) {
                st[i][k] = a * st[i][k] + xv[i] * bv[k];
                z[k] += dv[i] * st[i][k];
            }
        }
#pragma unroll
        for (int k = 0; k < NN; ++k) z[k] = sum_pg(z[k]);
        if (pg == 0) stk<NN>(zr + (int64_t)t * N, z);
    }

    // ---- backward walk from R_c ----
#pragma unroll
    for (int i = 0; i < PP; ++i) ldk<NN>(rin + bhc * PN + (int64_t)(p0 + i) * N + n0, st[i]);
    // boundary product <R_c[:, n], H_{c+1}[:, n]> (H_nc = hT; zero without dhT)
    float dl[NN];
    {
        float hn[PP][NN];
        const bool last = c + 1 == nc;
#pragma unroll
        for (int i = 0; i < PP; ++i) {
            if (!last) ldk<NN>(hin + (bhc + 1) * PN + (int64_t)(p0 + i) * N + n0, hn[i]);
            else if (have_dhT) ldk<NN>(hTf + bh * PN + (int64_t)(p0 + i) * N + n0, hn[i]);
            else
#pragma unroll
                for (int k = 0; k < NN; ++k) hn[i][k] = 0.f;
        }
#pragma unroll
        for (int k = 0; k < NN; ++k) {
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < PP; ++i) s += st[i][k] * hn[i][k];
            dl[k] = sum_pg(s);
        }
    }
    float dAacc[NN];
#pragma unroll
    for (int k = 0; k < NN; ++k) dAacc[k] = 0.f;
    float dd = 0.f;
    const float Dh = D ? D[h] : 0.f;
    for (int t = len - 1; t >= 0; --t) {
        float xv[PP], dv[PP], bv[NN], cv[NN], zv[NN];
        ldk<PP>(xr + t * rowx, xv);
        ldk<PP>(dyr + t * rowx, dv);
        ldk<NN>(br + t * rowb, bv);
        ldk<NN>(cr + t * rowb, cv);
        // Zh of this token: written above by this same lane (pg == 0) -- others skip it
        if (pg == 0) ldk<NN>(zr + (int64_t)t * N, zv);
        else
#pragma unroll
            for (int k = 0; k < NN; ++k) zv[k] = 0.f;
        const float dtv = dtr[(int64_t)t * H];
        float y[NN], dxa[PP];
#pragma unroll
        for (int i = 0; i < PP; ++i) dxa[i] = 0.f;
#pragma unroll
        for (int k = 0; k < NN; ++k) {
            y[k] = 0.f;
#pragma unroll
            for (int i = 0; i < PP; ++i) {
                st[i][k] += dv[i] * cv[k];  // g_t
                y[k] += xv[i] * st[i][k];
                dxa[i] += st[i][k] * bv[k];
            }
        }
#pragma unroll
        for (int k = 0; k < NN; ++k) y[k] = sum_pg(y[k]);
#pragma unroll
        for (int i = 0; i < PP; ++i) dxa[i] = sum_ng(dxa[i]);
        // decay gradient of this token (lanes with pg == 0 hold Zh)
        float dsum = 0.f;
#pragma unroll
        for (int k = 0; k < NN; ++k) {
            dl[k] += cv[k] * zv[k] - bv[k] * y[k];
            dsum += An[k] * dl[k];
            dAacc[k] += dtv * dl[k];
        }
        dsum = sum_ng(dsum);
        const int64_t tk = bi * Tn + tok0 + t;
        if (pg == 0) {
            stk<NN>(yr + (int64_t)t * N, y);
            if (ng == 0) {
                if (NSL == 1) ddt[tk * H + h] = dsum;
                else ddtp[((int64_t)sl * nb * Tn + tk) * H + h] = dsum;
            }
        }
        if (ng == 0) {
            if (NSL == 1) {
                float o[PP];
#pragma unroll
                for (int i = 0; i < PP; ++i) o[i] = dxa[i] + Dh * dv[i];
                stk<PP>(dx + (tk * H + h) * P + p0, o);
            } else {
                stk<PP>(dxp + (((int64_t)sl * nb * Tn + tk) * H + h) * P + p0, dxa);
            }
            if (sl == 0)
#pragma unroll
                for (int i = 0; i < PP; ++i) dd += xv[i] * dv[i];
        }
#pragma unroll
        for (int k = 0; k < NN; ++k) {
            const float a = exp2f_fast(an2[k] * dtv);
#pragma unroll
            for (int i = 0; i < PP; ++i) st[i][k] *= a;  // a_t g_t: the part of g_{t-1} from t on
        }
    }
    if (pg == 0) stk<NN>(dAp + bhc * N + n0, dAacc);
    if (sl == 0) {
        dd = sum_pg(dd);  // lanes with ng == 0 hold the channel groups' shares
        if (lane == 0) dDp[bhc] = dd;
    }
}

// dB[b,t,g,n] = sum_{h in g} Yh, dC = sum_{h in g} Zh, heads in order; one thread per
// (b, t, g, 4 consecutive n)
template <typename T>
__global__ __launch_bounds__(kThreads) void k_bwd_diag_bc(const float* __restrict__ zh, const float* __restrict__ yh,
                                                          T* __restrict__ dB, T* __restrict__ dC, int64_t Tn,
                                                          int H, int G, int N, int Q, int nc, int64_t total4) {
    const int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (v >= total4) return;
    const int n4 = N / 4;
    const int n = (int)(v % n4) * 4;
    const int g = (int)((v / n4) % G);
    const int64_t bt = v / ((int64_t)n4 * G);  // b * Tn + t
    const int64_t bi = bt / Tn, t = bt - bi * Tn;
    const int c = (int)(t / Q), r = (int)(t - (int64_t)c * Q);
    const int hpg = H / G;
    f32x4 sb = f32x4{0.f, 0.f, 0.f, 0.f}, sc = sb;
    for (int j = 0; j < hpg; ++j) {
        const int64_t bhc = (bi * H + g * hpg + j) * nc + c;
        const int64_t o = (bhc * Q + r) * N + n;
        sb += ld4(yh + o);
        sc += ld4(zh + o);
    }
    const int64_t out = (bt * G + g) * N + n;
    typedef typename V4<T>::type v4;
    v4 ob, oc;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        ob[e] = from_f<T>(sb[e]);
        oc[e] = from_f<T>(sc[e]);
    }
    st4(dB + out, ob);
    st4(dC + out, oc);
}

// dx = sum_s dxp[s] + D dy and ddt = sum_s ddtp[s] when dstate is split over NSL waves;
// one thread per (b, t, h, 4 consecutive p), slices in order
template <typename T>
__global__ __launch_bounds__(kThreads) void k_bwd_diag_fin(const float* __restrict__ dxp,
                                                           const float* __restrict__ ddtp,
                                                           const T* __restrict__ dy, const float* __restrict__ D,
                                                           T* __restrict__ dx, float* __restrict__ ddt, int H, int P,
                                                           int nsl, int64_t total4) {
    const int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (v >= total4) return;
    const int64_t e = v * 4;  // element of [b, T, H, P]
    const int h = (int)((e / P) % H);
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < nsl; ++k) s += ld4(dxp + (int64_t)k * total4 * 4 + e);
    const float Dh = D ? D[h] : 0.f;
    typedef typename V4<T>::type v4;
    const v4 dv = ld4(dy + e);
    v4 o;
#pragma unroll
    for (int r = 0; r < 4; ++r) o[r] = from_f<T>(s[r] + Dh * to_f(dv[r]));
    st4(dx + e, o);
    if (e % P == 0) {  // one thread per (b, t, h)
        const int64_t bth = e / P, nbth = total4 * 4 / P;
        float d = 0.f;
        for (int k = 0; k < nsl; ++k) d += ddtp[(int64_t)k * nbth + bth];
        ddt[bth] = d;
    }
}

// dA[h, n] = sum over (batch, chunk) of dAp, dD[h] = sum of dDp; one work-group per head.
// The (batch, chunk) list is cut into RP contiguous parts, each summed by its own thread
// with eight loads in flight, and the parts are added in part order: a fixed order.
template <int BLOCK>
__global__ __launch_bounds__(BLOCK) void k_bwd_diag_reduce(const float* __restrict__ dAp,
                                                           const float* __restrict__ dDp, float* __restrict__ dA,
                                                           float* __restrict__ dD, int64_t nb, int H, int N, int nc) {
    __shared__ float part[BLOCK];
    const int h = blockIdx.x;
    const int64_t nbc = nb * nc;  // (batch, chunk) pairs, index bi * nc + c
    // columns: n = 0 .. N-1 for dA, and one more for dD
    const int cols = N + 1;
    const int RP = BLOCK / cols > 0 ? BLOCK / cols : 1;
    for (int c0 = 0; c0 < cols; c0 += BLOCK / RP) {
        const int col = c0 + (int)threadIdx.x % (BLOCK / RP), rp = (int)threadIdx.x / (BLOCK / RP);
        float s = 0.f;
        if (col < cols && rp < RP) {
            const int64_t lo = nbc * rp / RP, hi = nbc * (rp + 1) / RP;
            auto at = [&](int64_t k) {
                const int64_t bi = k / nc, c = k - bi * nc;
                const int64_t bhc = (bi * H + h) * nc + c;
                return col < N ? dAp[bhc * N + col] : (dDp ? dDp[bhc] : 0.f);
            };
            int64_t k = lo;
            for (; k + 8 <= hi; k += 8) {
                float v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] = at(k + u);
#pragma unroll
                for (int u = 0; u < 8; ++u) s += v[u];
            }
            for (; k < hi; ++k) s += at(k);
        }
        part[threadIdx.x] = s;
        __syncthreads();
        if (rp == 0 && col < cols) {
            float t = 0.f;
            for (int r = 0; r < RP; ++r) t += part[r * (BLOCK / RP) + (int)threadIdx.x];
            if (col < N) dA[(int64_t)h * N + col] = t;
            else if (dD) dD[h] = t;
        }
        __syncthreads();
    }
}

}  // namespace ssd
