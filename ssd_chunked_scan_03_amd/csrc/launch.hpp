// launch.hpp -- enqueue the kernel sequence of one SSD forward on a stream.
#pragma once

#include "fused.hpp"

#include <type_traits>

namespace ssd {

// Everything one launch sequence needs; validated by the C ABI beforehand.
struct RunArgs {
    int64_t b, T, H, P, N, G, Q, nc;
    int diag;
    const void* x;
    const float* dt;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const float* h0;
    void* y;
    float* hT;
    float* cdt;     // [b,H,nc,Q]
    void* cb;       // [b,nc,G,Q,Q] (scalar decay); [b,H,nc,Q,Q] (diagonal decay, table path)
    void* states;   // [b,H,nc,P,N] chunk states, in the input type
    void* hin;      // [b,H,nc,P,N]
    void* bt;       // [b,nc,G,N,Q]  (scalar decay only)
    // packed variable-length rows (nullptr: dense).  b rows share the token axis of T
    // tokens; ts / kb (b + 1 entries, in the workspace) are each row's first token and
    // first chunk, kcap bounds the chunk axis, nc is the most chunks any row can have.
    // Packed rows run only on the fused schedule; cdt is then [H][kcap][Q] and cb / bt
    // are [kcap, G, ...].
    const int* ts;
    const int* kb;
    int64_t kcap;
    float* carry;   // [nseg, b, H, P, N] then [b, H, nseg] when the state scan runs in
                    // segments (entering states, then each segment's summed cdt totals)
    hipStream_t stream;
    int stages;       // 0: the whole schedule; else a mask of kernels to enqueue
                      // (1 cumsum, 2 cb, 4 state, 8 scan, 16 out, 32 bt, 64 fused)
    bool force_split;
    bool force_fused;
};

// Segments of the split schedule's state scan: 1 (one sequential pass) unless b H P N / 4
// threads cannot fill the GPU; then enough segments of at least 4 chunks, at most 64,
// that the parallel scan has about 128 K threads.  Returns the segment length in chunks
// (nc for one segment); the segment count is ceil(nc / length).
inline int64_t scan_segment_len(int64_t b, int64_t H, int64_t P, int64_t N, int64_t nc) {
    const int64_t want = 131072, threads = b * H * P * N / 4;
    if (threads >= want || nc < 8) return nc > 0 ? nc : 1;
    int64_t S = (want + threads - 1) / threads;
    if (S > nc / 4) S = nc / 4;
    if (S > 64) S = 64;
    if (S < 2) return nc;
    return (nc + S - 1) / S;
}

// The fused per-(batch, head) schedule: bf16, scalar decay, P = 64, N in {64, 128},
// and enough (batch, head) chains to occupy every CU several times over.
inline bool fused_supported(const RunArgs& a, bool bf16_dtype) {
    // the fused kernel addresses a batch row's x / y, C, C B^T and B^T tables through
    // buffer resources with 32-bit offsets: each must span less than 2 GiB
    const int64_t lim = (int64_t)1 << 31;
    const bool fits = a.T * a.H * a.P * 2 < lim && a.T * a.G * a.N * 2 < lim &&
                      a.nc * a.G * a.Q * a.Q * 2 < lim && a.nc * a.G * a.N * a.Q * 2 < lim;
    return bf16_dtype && !a.diag && a.P == 64 && (a.N == 64 || a.N == 128) && fits;
}
inline bool fused_applies(const RunArgs& a, bool bf16_dtype) {
    return fused_supported(a, bf16_dtype) && !a.force_split && (a.ts || a.force_fused || a.b * a.H >= 512);
}

// The split schedule's scalar-decay output kernel in the fused layout (k_outs): bfloat16,
// headdim 64, dstate 64 to 256, dense rows, buffer offsets of a batch row within 32 bits.
// Enqueues it and returns true where it applies; false leaves the output to k_out.
template <typename T, int P, int N>
bool launch_outs(const RunArgs& a, dim3 g3, hipStream_t s, const T* x, const T* Cm, const T* cb, const T* hin,
                 T* y) {
    if constexpr (std::is_same<T, bf16>::value && P == 64 && (N == 64 || N == 128 || N == 256)) {
        const int64_t lim = (int64_t)1 << 31;
        if (a.ts || !(a.T * a.H * a.P * 2 < lim && a.T * a.G * a.N * 2 < lim && a.nc * a.G * a.Q * a.Q * 2 < lim &&
                      a.nc * a.P * a.N * 2 < lim))
            return false;
        const int H = (int)a.H, G = (int)a.G, nc = (int)a.nc;
        switch (a.Q) {
            case 64: k_outs<64, N><<<g3, kThreads, 0, s>>>(x, Cm, cb, hin, a.A, a.D, a.cdt, y, a.T, H, G, nc); return true;
            case 128: k_outs<128, N><<<g3, kThreads, 0, s>>>(x, Cm, cb, hin, a.A, a.D, a.cdt, y, a.T, H, G, nc); return true;
            case 256: k_outs<256, N><<<g3, kThreads, 0, s>>>(x, Cm, cb, hin, a.A, a.D, a.cdt, y, a.T, H, G, nc); return true;
            default: return false;
        }
    }
    return false;
}

inline Rows rows_of(const RunArgs& a) {
    Rows r;
    r.ts = a.ts;
    r.kb = a.kb;
    r.T = a.T;
    r.nc = (int)a.nc;
    r.nrows = (int)a.b;
    r.H = (int)a.H;
    r.kcap = a.ts ? (int)a.kcap : (int)(a.b * a.nc);
    return r;
}

// The diagonal decay's output kernel keeps a chunk's x rows and its rescaled C and B rows
// in LDS (OutSmem<T, P, N, true>).  Where they do not fit one CU's 160 KiB, k_gtab forms
// each (b, h, c)'s decay-weighted query-key block as a table in the workspace (the cb
// region) and the output kernel reads it instead.
inline bool diag_uses_table(int64_t Q, int64_t P, int64_t N, size_t es) {
    const size_t bytes = (size_t)(Q * (P + 8) + 2 * Q * (N + 8)) * es + (size_t)(2 * Q + N) * 4;
    return bytes > 160 * 1024;
}

template <int Q, int N>
void launch_fused(const RunArgs& a) {
    const int BH = (int)(a.b * a.H);
    const Rows rows = rows_of(a);
    const bf16* bt = static_cast<const bf16*>(a.bt);  // B^T per chunk, then C per chunk
    k_fused<Q, N><<<BH, kThreads, 0, a.stream>>>(
        static_cast<const bf16*>(a.x), bt + (int64_t)rows.kcap * a.G * N * Q, static_cast<const bf16*>(a.cb), bt,
        a.A, a.D, a.cdt, a.h0, static_cast<bf16*>(a.y), a.hT, rows, (int)a.G);
}

template <typename T, int P, int N>
int run(const RunArgs& a) {
    constexpr bool kBF16 = sizeof(T) == 2;
    if (a.force_fused && !fused_supported(a, kBF16)) return 3;
    const bool fused = fused_applies(a, kBF16);
    if (a.ts && (!fused || a.force_split)) return 3;  // packed rows: fused schedule only
    // a stage mask may name only kernels of the schedule that runs: the workspace holds
    // that schedule's regions only
    const int sched_bits = fused ? (1 | 2 | 32 | 64) : (1 | 2 | 4 | 8 | 16);
    if (a.stages & ~sched_bits) return 3;
    int st = a.stages ? a.stages : sched_bits;
    const int Q = (int)a.Q, nc = (int)a.nc, H = (int)a.H, G = (int)a.G;
    hipStream_t s = a.stream;
    const T* x = static_cast<const T*>(a.x);
    const T* Bm = static_cast<const T*>(a.B);
    const T* Cm = static_cast<const T*>(a.C);
    T* cb = static_cast<T*>(a.cb);
    T* hin = static_cast<T*>(a.hin);
    T* y = static_cast<T*>(a.y);

    // the output kernel's LDS must fit one CU (160 KiB); checked before any launch
    const bool tab = a.diag && diag_uses_table(Q, P, N, sizeof(T));
    // the diagonal decay's swizzled tiles where they fit one more work-group per CU (the
    // kernel's registers allow at most 3)
    const auto per_cu = [](size_t bytes) { const size_t n = (160 * 1024) / bytes; return n < 3 ? n : (size_t)3; };
    const bool swzr = a.diag && !tab && sizeof(T) == 2 &&
                      per_cu(OutSmem<T, P, N, true, false, true>::bytes(Q)) > per_cu(OutSmem<T, P, N, true>::bytes(Q));
    const size_t smem = !a.diag ? OutSmem<T, P, N, false>::bytes(Q)
                        : tab   ? OutSmem<T, P, N, true, true>::bytes(Q)
                        : swzr  ? OutSmem<T, P, N, true, false, true>::bytes(Q)
                                : OutSmem<T, P, N, true>::bytes(Q);
    if (smem > 160 * 1024) return 3;

    // the prep kernels run over the global chunk axis (blocks past the last chunk exit)
    const Rows rows = rows_of(a);
    const unsigned kc = (unsigned)rows.kcap;
    // the whole preparation of a forward (cumsum, C B^T, and B^T for the fused schedule)
    // in one launch; a stage mask that asks for part of it runs the separate kernels
    const int prep_bits = fused ? (1 | 2 | 32) : (1 | 2);
    if (!a.diag && (st & prep_bits) == prep_bits) {
        const int nb = Q / 64;
        const dim3 gp(kc, (unsigned)((H + 15) / 16 + prep_cb_tasks<T, N>(nb) * G + (fused ? nb * G : 0)));
        switch (Q * 2 + (fused ? 1 : 0)) {
#define SSD_PREP(QQ, F) \
    case QQ * 2 + F: k_prep<T, N, QQ, F><<<gp, kThreads, 0, s>>>(a.dt, a.cdt, Bm, Cm, cb, static_cast<T*>(a.bt), rows, G); break;
            SSD_PREP(64, 0) SSD_PREP(64, 1) SSD_PREP(128, 0) SSD_PREP(128, 1) SSD_PREP(256, 0) SSD_PREP(256, 1)
#undef SSD_PREP
            default: return 3;
        }
        st &= ~prep_bits;
    }
    const dim3 g1(kc, 1, (H + 15) / 16);
    if (st & 1) switch (Q) {
        case 64: k_cumsum<64><<<g1, kThreads, 0, s>>>(a.dt, a.cdt, rows); break;
        case 128: k_cumsum<128><<<g1, kThreads, 0, s>>>(a.dt, a.cdt, rows); break;
        case 256: k_cumsum<256><<<g1, kThreads, 0, s>>>(a.dt, a.cdt, rows); break;
        default: return 3;
    }
    if (!a.diag && (st & 2)) {
        const int nb = Q / 64;
        const dim3 g2(kc, nb * (nb + 1) / 2, (unsigned)G);
        k_cb<T, N><<<g2, kThreads, 0, s>>>(Bm, Cm, cb, rows, G, Q);
    } else if (tab && (st & 2)) {
        const int nb = Q / 64;
        const size_t gsm = gtab_smem<T, N>();
        hipFuncSetAttribute((const void*)k_gtab<T, N>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)gsm);
        k_gtab<T, N><<<dim3((unsigned)(a.b * H * nc), (unsigned)(nb * (nb + 1) / 2)), kThreads, gsm, s>>>(
            Bm, Cm, a.A, a.D, a.cdt, cb, a.T, H, G, Q, nc);
    }
    const dim3 g3((unsigned)(a.b * H * nc));
    T* Sc = static_cast<T*>(a.states);
    if (!(st & 4)) {
    } else if (a.diag)
        k_state<T, P, N, true, false, T><<<g3, kThreads, 0, s>>>(x, Bm, a.A, a.cdt, Sc, a.T, H, G, Q, nc);
    else
        k_state<T, P, N, false, false, T><<<g3, kThreads, 0, s>>>(x, Bm, a.A, a.cdt, Sc, a.T, H, G, Q, nc);

    const int per_head = (P * N / 4 + kThreads - 1) / kThreads;
    const int L = (int)scan_segment_len(a.b, H, P, N, nc);
    const int nseg = (nc + L - 1) / L;
    const int64_t BHPN = a.b * H * P * N;
    const dim3 g4((unsigned)(a.b * H * per_head)), g4s((unsigned)(a.b * H * per_head), (unsigned)nseg);
    float* segsum = a.carry ? a.carry + nseg * BHPN : nullptr;  // [b, H, nseg]
    if (!(st & 8)) {
    } else if (nseg <= 1) {
        if (a.diag)
            k_scan<T, true, 0, T><<<g4, kThreads, 0, s>>>(Sc, hin, a.hT, a.h0, a.A, a.cdt, nullptr, nullptr, H,
                                                      P * N, N, Q, nc, per_head, nc, BHPN);
        else
            k_scan<T, false, 0, T><<<g4, kThreads, 0, s>>>(Sc, hin, a.hT, a.h0, a.A, a.cdt, nullptr, nullptr, H,
                                                       P * N, N, Q, nc, per_head, nc, BHPN);
    } else if (a.diag) {
        k_scan<T, true, 1, T><<<g4s, kThreads, 0, s>>>(Sc, hin, a.hT, a.h0, a.A, a.cdt, a.carry, segsum, H,
                                                    P * N, N, Q, nc, per_head, L, BHPN);
        k_scan_carry<true><<<g4, kThreads, 0, s>>>(a.h0, a.A, segsum, a.carry, H, P * N, N, per_head, nseg, BHPN);
        k_scan<T, true, 2, T><<<g4s, kThreads, 0, s>>>(Sc, hin, a.hT, a.h0, a.A, a.cdt, a.carry, segsum, H,
                                                    P * N, N, Q, nc, per_head, L, BHPN);
    } else {
        k_scan<T, false, 1, T><<<g4s, kThreads, 0, s>>>(Sc, hin, a.hT, a.h0, a.A, a.cdt, a.carry, segsum, H,
                                                     P * N, N, Q, nc, per_head, L, BHPN);
        k_scan_carry<false><<<g4, kThreads, 0, s>>>(a.h0, a.A, segsum, a.carry, H, P * N, N, per_head, nseg, BHPN);
        k_scan<T, false, 2, T><<<g4s, kThreads, 0, s>>>(Sc, hin, a.hT, a.h0, a.A, a.cdt, a.carry, segsum, H,
                                                     P * N, N, Q, nc, per_head, L, BHPN);
    }

    if (!(st & 16)) {
    } else if (tab) {
        hipFuncSetAttribute((const void*)k_out<T, P, N, true, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)smem);
        k_out<T, P, N, true, true><<<g3, kThreads, smem, s>>>(x, Bm, Cm, cb, hin, a.A, a.D, a.cdt, y, a.T, H, G, Q, nc);
    } else if (a.diag) {
        if (swzr) {
            hipFuncSetAttribute((const void*)k_out<T, P, N, true, false, true>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
            k_out<T, P, N, true, false, true><<<g3, kThreads, smem, s>>>(x, Bm, Cm, nullptr, hin, a.A, a.D, a.cdt, y,
                                                                         a.T, H, G, Q, nc);
        } else {
            hipFuncSetAttribute((const void*)k_out<T, P, N, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)smem);
            k_out<T, P, N, true><<<g3, kThreads, smem, s>>>(x, Bm, Cm, nullptr, hin, a.A, a.D, a.cdt, y, a.T, H, G,
                                                            Q, nc);
        }
    } else if (launch_outs<T, P, N>(a, g3, s, x, Cm, cb, hin, y)) {
    } else {
        hipFuncSetAttribute((const void*)k_out<T, P, N, false>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        k_out<T, P, N, false><<<g3, kThreads, smem, s>>>(x, Bm, Cm, cb, hin, a.A, a.D, a.cdt, y, a.T, H, G, Q, nc);
    }
    if (!a.diag && (st & 32)) {
        const dim3 g6(kc * (unsigned)(Q / 64), (unsigned)G);
        T* btp = static_cast<T*>(a.bt);
        k_bt<T, N><<<g6, kThreads, 0, s>>>(Bm, btp, Cm, btp + (int64_t)rows.kcap * G * N * Q, rows, G, Q);
    }
    if (st & 64) {
        if constexpr (kBF16 && P == 64 && (N == 64 || N == 128)) {
            if (a.diag) return 3;
            switch (Q) {
                case 64: launch_fused<64, N>(a); break;
                case 128: launch_fused<128, N>(a); break;
                case 256: launch_fused<256, N>(a); break;
                default: return 3;
            }
        } else {
            return 3;
        }
    }
    return hipGetLastError() == hipSuccess ? 0 : 7;
}

int run_bf16(const RunArgs& a);
int run_f32(const RunArgs& a);

// The (headdim, dstate) pairs with compiled kernels.
#define SSD_FOR_EACH_PN(X)                                                              \
    X(16, 16) X(16, 32) X(16, 64) X(16, 128) X(16, 256) X(32, 16) X(32, 32) X(32, 64)   \
    X(32, 128) X(32, 256) X(64, 16) X(64, 32) X(64, 64) X(64, 128) X(64, 256)           \
    X(128, 16) X(128, 32) X(128, 64) X(128, 128) X(128, 256)

}  // namespace ssd
