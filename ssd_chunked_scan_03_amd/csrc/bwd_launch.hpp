// bwd_launch.hpp -- enqueue the kernel sequence of one SSD backward pass on a stream.
#pragma once

#include "bwd.hpp"
#include "bwd_diag.hpp"
#include "walk.hpp"

#include <type_traits>

namespace ssd {

// Everything one backward launch sequence needs; validated by the C ABI beforehand.
struct BwdArgs {
    int64_t b, T, H, P, N, G, Q, nc;
    const void* x;
    const float* dt;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const float* h0;
    const void* dy;
    const float* dhT;
    void* dx;
    float* ddt;
    float* dA;
    void* dB;
    void* dC;
    float* dD;
    float* dh0;
    // workspace regions
    float* cdt;     // [b,H,nc,Q]
    void* cb;       // [b,nc,G,Q,Q]  C_c B_c^T, blocks on and below the diagonal
    void* cbt;      // [b,nc,G,Q,Q]  its transpose, cbt[j][i] = B_j . C_i
    void* bt;       // [b,nc,G,N,Q]  B per chunk, tokens contiguous
    void* ct;       // [b,nc,G,N,Q]  C per chunk, tokens contiguous
    void* bcp;      // [b,nc,G,Q,N]  B per chunk by token (k_bwd_xs's state-term operand), or null
    void* ccp;      // [b,nc,G,Q,N]  C per chunk by token, or null
    float* states;  // [b,H,nc,P,N]  chunk states, then adjoint chunk inputs
    void* hin;      // [b,H,nc,P,N]  forward state entering each chunk
    void* rin;      // [b,H,nc,P,N]  adjoint arriving at each chunk's last token
    float* hTf;     // [b,H,P,N]     forward final state (when dhT is given)
    float* ds;      // [b,H,nc,Q]    per-token decay term
    float* dDp;     // [b,H,nc]      D partial sums
    float* dAp;     // [b,H,nc]      A partial sums
    float* kpart;   // [b,H,nc,4 * ceil(P N / 1024)]  per-wave partials of <R_c, H_{c+1}>
    // diagonal decay only (dAp is then [b,H,nc,N])
    float* zh;      // [b,H,nc,Q,N]  dy_t . h_t per dimension
    float* yh;      // [b,H,nc,Q,N]  x_t . g_t per dimension
    float* dxp;     // [nsl,b,T,H,P] per-slice partials of dx (dstate split over nsl waves)
    float* ddtp;    // [nsl,b,T,H]   per-slice partials of ddt
    hipStream_t stream;
};

// The chunk-pipelined walks (walk.hpp) take both state recurrences when there are enough
// (batch, head) chains to occupy every CU and the shape is theirs: bfloat16, headdim 64,
// dstate 64 or 128, and buffer offsets of a batch row within 32 bits.  (The workspace
// layout takes the same decision: the walks need no chunk-state region.)
// Whether the backward's dx runs k_bwd_xs (bfloat16, headdim 64, dstate 64 or 128, buffer
// offsets of a batch row within 32 bits); it then reads B and C per chunk by token in
// fragment order (two more workspace regions).
inline bool xs_applies(bool bf16_dtype, int64_t T, int64_t H, int64_t P, int64_t N, int64_t G, int64_t Q) {
    const int64_t lim = (int64_t)1 << 31, nc = (T + Q - 1) / Q;
    return bf16_dtype && P == 64 && (N == 64 || N == 128) && T * H * P * 2 < lim && nc * G * N * Q * 2 < lim &&
           nc * G * Q * Q * 2 < lim && nc * P * N * 2 < lim;
}

inline bool walks_apply(bool bf16_dtype, int64_t b, int64_t T, int64_t H, int64_t P, int64_t N, int64_t G,
                        int64_t Q) {
    const int64_t lim = (int64_t)1 << 31, nc = (T + Q - 1) / Q;
    return bf16_dtype && P == 64 && (N == 64 || N == 128) && b * H >= 512 && T * H * P * 2 < lim &&
           nc * G * N * Q * 2 < lim;
}
template <typename T, int P, int N>
bool walk_applies(const BwdArgs& a) {
    return walks_apply(std::is_same<T, bf16>::value, a.b, a.T, a.H, P, N, a.G, a.Q);
}

template <int Q, int N>
void launch_walks(const BwdArgs& a, const bf16* x, const bf16* dy, const bf16* bt, const bf16* ct, bf16* hin,
                  bf16* rin, int nslot) {
    const unsigned nb = (unsigned)(a.b * a.H);
    const int H = (int)a.H, G = (int)a.G, nc = (int)a.nc, nrows = (int)a.b;
    k_walk<Q, N, false><<<nb, kThreads, 0, a.stream>>>(x, bt, a.A, a.cdt, a.h0, hin, a.dhT ? a.hTf : nullptr,
                                                       nullptr, nullptr, nullptr, 0, a.T, nrows, H, G, nc);
    k_walk<Q, N, true><<<nb, kThreads, 0, a.stream>>>(dy, ct, a.A, a.cdt, a.dhT, rin, a.dh0, hin,
                                                      a.dhT ? a.hTf : nullptr, a.kpart, nslot, a.T, nrows, H, G, nc);
}

template <typename T, int P, int N>
int run_bwd(const BwdArgs& a) {
    constexpr int NB = bc_nb<T, P, N>();
    const int Q = (int)a.Q, nc = (int)a.nc, H = (int)a.H, G = (int)a.G;
    const size_t sx = BxSmem<T, P>::bytes(Q), sbc = BcSmem<T, P, NB>::bytes(Q);
    if (sx > 160 * 1024 || sbc > 160 * 1024) return 3;
    hipStream_t s = a.stream;
    const T* x = static_cast<const T*>(a.x);
    const T* dy = static_cast<const T*>(a.dy);
    const T* Bm = static_cast<const T*>(a.B);
    const T* Cm = static_cast<const T*>(a.C);
    T* cb = static_cast<T*>(a.cb);
    T* cbt = static_cast<T*>(a.cbt);
    T* bt = static_cast<T*>(a.bt);
    T* ct = static_cast<T*>(a.ct);
    T* hin = static_cast<T*>(a.hin);
    T* rin = static_cast<T*>(a.rin);

    Rows rows;
    rows.ts = nullptr;
    rows.kb = nullptr;
    rows.T = a.T;
    rows.nc = nc;
    rows.nrows = (int)a.b;
    rows.H = H;
    rows.kcap = (int)(a.b * a.nc);
    const unsigned kc = (unsigned)rows.kcap;

    // the forward's tables (cdt, C B^T in both orientations, B^T and C^T per chunk; with
    // a.bcp / a.ccp also B and C per chunk by token) in one launch, then the entering states
    const int nb = Q / 64;
    const dim3 gp(kc, (unsigned)((H + 15) / 16 + 2 * (nb * (nb + 1) / 2) * G + 2 * nb * G));
    T* bcp = static_cast<T*>(a.bcp);
    T* ccp = static_cast<T*>(a.ccp);
    switch (Q) {
        case 64: k_bprep<T, N, 64><<<gp, kThreads, 0, s>>>(a.dt, a.cdt, Bm, Cm, cb, cbt, bt, ct, bcp, ccp, rows, G); break;
        case 128: k_bprep<T, N, 128><<<gp, kThreads, 0, s>>>(a.dt, a.cdt, Bm, Cm, cb, cbt, bt, ct, bcp, ccp, rows, G); break;
        case 256: k_bprep<T, N, 256><<<gp, kThreads, 0, s>>>(a.dt, a.cdt, Bm, Cm, cb, cbt, bt, ct, bcp, ccp, rows, G); break;
        default: return 3;
    }
    const dim3 g3((unsigned)(a.b * H * nc));
    const int per_head = (int)((a.P * a.N / 4 + kThreads - 1) / kThreads);
    int nvalid = (int)(a.P * a.N / 4 / 64);  // partials of <R_c, H_{c+1}> per chunk
    bool walked = false;
    if constexpr (std::is_same<T, bf16>::value && P == 64 && (N == 64 || N == 128)) {
        if (walk_applies<T, P, N>(a)) {
            // both recurrences walked chunk by chunk, the states on chip
            switch (Q) {
                case 64: launch_walks<64, N>(a, x, dy, bt, ct, hin, rin, per_head * 4); break;
                case 128: launch_walks<128, N>(a, x, dy, bt, ct, hin, rin, per_head * 4); break;
                case 256: launch_walks<256, N>(a, x, dy, bt, ct, hin, rin, per_head * 4); break;
                default: return 3;
            }
            nvalid = 4;  // one partial per wave
            walked = true;
        }
    }
    // otherwise the forward states: with many (b, h) chains, each chain's chunks walked with
    // the state in registers; else chunk states, then the scan
    if (!walked && a.b * H >= 512) {
        k_states<T, P, N><<<(unsigned)(a.b * H), kThreads, 0, s>>>(x, Bm, a.A, a.cdt, a.h0, hin,
                                                                   a.dhT ? a.hTf : nullptr, a.T, H, G, Q, nc);
    } else if (!walked) {
        k_state<T, P, N, false, false><<<g3, kThreads, 0, s>>>(x, Bm, a.A, a.cdt, a.states, a.T, H, G, Q, nc);
        const int64_t BHPN = a.b * H * a.P * a.N;
        const dim3 g4((unsigned)(a.b * H * per_head));
        k_scan<T, false, 0><<<g4, kThreads, 0, s>>>(a.states, hin, a.dhT ? a.hTf : nullptr, a.h0, a.A, a.cdt,
                                                    nullptr, nullptr, H, (int)(a.P * a.N), (int)a.N, Q, nc,
                                                    per_head, nc, BHPN);
    }
    // the adjoint: chunk inputs (into the chunk-state buffer), reverse scan
    if (!walked) {
        const dim3 g4((unsigned)(a.b * H * per_head));
        k_state<T, P, N, false, true><<<g3, kThreads, 0, s>>>(dy, Cm, a.A, a.cdt, a.states, a.T, H, G, Q, nc);
        k_scan_rev<T><<<g4, kThreads, 0, s>>>(a.states, rin, a.dh0, a.dhT, a.A, a.cdt, hin, a.hTf, a.kpart, H,
                                              (int)(a.P * a.N), (int)a.N, Q, nc, per_head);
    }
    const int nslot = per_head * 4;  // partials' stride per chunk
    // gradients: dx and the per-token decay term (LDS-staged kernel where it applies)
    bool xs_done = false;
    if constexpr (std::is_same<T, bf16>::value && P == 64 && (N == 64 || N == 128)) {
        if (a.bcp && a.ccp) {  // (the workspace has the copies exactly where xs_applies)
            bf16* dxp = static_cast<bf16*>(a.dx);
            const bf16* Bf = static_cast<const bf16*>(a.bcp);
            const bf16* Cf = static_cast<const bf16*>(a.ccp);
            switch (Q) {
                case 64: k_bwd_xs<64, N><<<g3, kThreads, 0, s>>>(x, dy, Bf, Cf, cb, cbt, hin, rin, a.A, a.D, a.cdt,
                                                                 dxp, a.ds, a.dDp, a.T, H, G, nc); break;
                case 128: k_bwd_xs<128, N><<<g3, kThreads, 0, s>>>(x, dy, Bf, Cf, cb, cbt, hin, rin, a.A, a.D, a.cdt,
                                                                   dxp, a.ds, a.dDp, a.T, H, G, nc); break;
                case 256: k_bwd_xs<256, N><<<g3, kThreads, 0, s>>>(x, dy, Bf, Cf, cb, cbt, hin, rin, a.A, a.D, a.cdt,
                                                                   dxp, a.ds, a.dDp, a.T, H, G, nc); break;
                default: return 3;
            }
            xs_done = true;
        }
    }
    if (!xs_done) {
        (void)hipFuncSetAttribute((const void*)k_bwd_x<T, P, N>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sx);
        k_bwd_x<T, P, N><<<g3, kThreads, sx, s>>>(x, dy, Bm, Cm, cb, cbt, hin, rin, a.A, a.D, a.cdt,
                                                  static_cast<T*>(a.dx), a.ds, a.dDp, a.T, H, G, Q, nc);
    }
    bool bc_done = false;
    if constexpr (std::is_same<T, bf16>::value && P == 64 && (N == 64 || N == 128)) {
        // the double-buffered variant: buffer offsets of a batch row within 32 bits
        const int64_t lim = (int64_t)1 << 31;
        if (a.T * H * P * 2 < lim && H * a.nc * P * N * 2 < lim && H * a.nc * Q * 4 < lim) {
            const dim3 g7((unsigned)(a.b * nc * G * (Q / 64)));
            const bf16* xb = x;
            switch (Q) {
                case 64: k_bwd_bcs<64, N, N><<<g7, kBcsThreads, 0, s>>>(xb, dy, bt, ct, hin, rin, a.A, a.cdt,
                                                                      static_cast<T*>(a.dB), static_cast<T*>(a.dC),
                                                                      a.T, H, G, nc); break;
                case 128: k_bwd_bcs<128, N, N><<<g7, kBcsThreads, 0, s>>>(xb, dy, bt, ct, hin, rin, a.A, a.cdt,
                                                                        static_cast<T*>(a.dB), static_cast<T*>(a.dC),
                                                                        a.T, H, G, nc); break;
                case 256: k_bwd_bcs<256, N, N><<<g7, kBcsThreads, 0, s>>>(xb, dy, bt, ct, hin, rin, a.A, a.cdt,
                                                                        static_cast<T*>(a.dB), static_cast<T*>(a.dC),
                                                                        a.T, H, G, nc); break;
                default: return 3;
            }
            bc_done = true;
        }
    }
    if (!bc_done) {
        (void)hipFuncSetAttribute((const void*)k_bwd_bc<T, P, N, NB>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)sbc);
        const dim3 g7((unsigned)(a.b * nc * G * (Q / 64) * (N / NB)));
        k_bwd_bc<T, P, N, NB><<<g7, kBcThreads, sbc, s>>>(x, dy, bt, ct, hin, rin, a.A, a.cdt, static_cast<T*>(a.dB),
                                                        static_cast<T*>(a.dC), a.T, H, G, Q, nc);
    }
    k_bwd_dt<128><<<(unsigned)(a.b * nc), 128, 0, s>>>(a.ds, a.dt, a.A, a.kpart, a.ddt, a.dAp, a.T, H, Q, nc,
                                                       nslot, nvalid);
    k_bwd_reduce<kThreads><<<(unsigned)H, kThreads, 0, s>>>(a.dAp, a.dDp, a.dA, a.dD, a.b, H, nc);
    return hipGetLastError() == hipSuccess ? 0 : 7;
}

// The diagonal-decay backward (bwd_diag.hpp): forward chunk states and their scan, the
// adjoint's chunk inputs and reverse scan, the per-chunk walks, then the head and
// (batch, chunk) reductions.
template <typename T, int P, int N>
int run_bwd_diag(const BwdArgs& a) {
    typedef DiagSplit<P, N> SP;
    const int Q = (int)a.Q, nc = (int)a.nc, H = (int)a.H, G = (int)a.G;
    hipStream_t s = a.stream;
    const T* x = static_cast<const T*>(a.x);
    const T* dy = static_cast<const T*>(a.dy);
    const T* Bm = static_cast<const T*>(a.B);
    const T* Cm = static_cast<const T*>(a.C);
    T* hin = static_cast<T*>(a.hin);
    T* rin = static_cast<T*>(a.rin);

    Rows rows;
    rows.ts = nullptr;
    rows.kb = nullptr;
    rows.T = a.T;
    rows.nc = nc;
    rows.nrows = (int)a.b;
    rows.H = H;
    rows.kcap = (int)(a.b * a.nc);
    const dim3 g1((unsigned)rows.kcap, 1, (H + 15) / 16);
    switch (Q) {
        case 64: k_cumsum<64><<<g1, kThreads, 0, s>>>(a.dt, a.cdt, rows); break;
        case 128: k_cumsum<128><<<g1, kThreads, 0, s>>>(a.dt, a.cdt, rows); break;
        case 256: k_cumsum<256><<<g1, kThreads, 0, s>>>(a.dt, a.cdt, rows); break;
        default: return 3;
    }
    const dim3 g3((unsigned)(a.b * H * nc));
    const int PN = (int)(a.P * a.N);
    const int per_head = (PN / 4 + kThreads - 1) / kThreads;
    const dim3 g4((unsigned)(a.b * H * per_head));
    const int64_t BHPN = a.b * H * a.P * a.N;
    // entering states H_c and the final state
    k_state<T, P, N, true, false><<<g3, kThreads, 0, s>>>(x, Bm, a.A, a.cdt, a.states, a.T, H, G, Q, nc);
    k_scan<T, true, 0><<<g4, kThreads, 0, s>>>(a.states, hin, a.dhT ? a.hTf : nullptr, a.h0, a.A, a.cdt, nullptr,
                                               nullptr, H, PN, N, Q, nc, per_head, nc, BHPN);
    // the adjoint: chunk inputs sum_i e^{A_n cdt_i} dy_i C_i^T, reverse scan -> R_c, dh0
    k_state<T, P, N, true, true><<<g3, kThreads, 0, s>>>(dy, Cm, a.A, a.cdt, a.states, a.T, H, G, Q, nc);
    k_scan_rev<T, true><<<g4, kThreads, 0, s>>>(a.states, rin, a.dh0, a.dhT, a.A, a.cdt, hin, a.hTf, nullptr, H,
                                                PN, N, Q, nc, per_head);
    // the walks of every chunk
    const int64_t nwaves = a.b * H * nc * SP::NSL;
    k_bwd_diag<T, P, N><<<(unsigned)((nwaves + 3) / 4), kThreads, 0, s>>>(
        x, dy, Bm, Cm, a.dt, a.A, a.D, hin, rin, a.hTf, a.dhT != nullptr, a.zh, a.yh, static_cast<T*>(a.dx), a.dxp,
        a.ddt, a.ddtp, a.dAp, a.dDp, a.b, a.T, H, G, Q, nc, nwaves);
    const int64_t bc4 = a.b * a.T * G * N / 4;
    k_bwd_diag_bc<T><<<(unsigned)((bc4 + kThreads - 1) / kThreads), kThreads, 0, s>>>(
        a.zh, a.yh, static_cast<T*>(a.dB), static_cast<T*>(a.dC), a.T, H, G, N, Q, nc, bc4);
    if (SP::NSL > 1) {
        const int64_t x4 = a.b * a.T * H * a.P / 4;
        k_bwd_diag_fin<T><<<(unsigned)((x4 + kThreads - 1) / kThreads), kThreads, 0, s>>>(
            a.dxp, a.ddtp, dy, a.D, static_cast<T*>(a.dx), a.ddt, H, (int)a.P, SP::NSL, x4);
    }
    k_bwd_diag_reduce<kThreads><<<(unsigned)H, kThreads, 0, s>>>(a.dAp, a.dDp, a.dA, a.dD, a.b, H, N, nc);
    return hipGetLastError() == hipSuccess ? 0 : 7;
}

// dstate slices of the diagonal backward's walks (host side of DiagSplit)
inline int diag_bwd_slices(int64_t P, int64_t N) {
    const int64_t ns = N < 64 ? (N < 4096 / P ? N : 4096 / P) : (64 < 4096 / P ? 64 : 4096 / P);
    return (int)(N / ns);
}

int run_bwd_bf16(const BwdArgs& a);
int run_bwd_f32(const BwdArgs& a);
int run_bwd_diag_bf16(const BwdArgs& a);
int run_bwd_diag_f32(const BwdArgs& a);

}  // namespace ssd
