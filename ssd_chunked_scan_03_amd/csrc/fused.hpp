// fused.hpp -- the whole chunked scan of one (batch, head) pair in one work-group,
// with the state kept on chip across chunks (scalar decay, bfloat16 x/B/C/y, P = 64).
//
// "The chunked algorithm takes both" ("Structured State Space Duality" concept page):
// the quadratic form on each diagonal block, one recurrence step per chunk for the
// carried state.  The split schedule writes the chunk states and the entering states
// to HBM and reads them back; here the state never leaves the work-group:
//
//   for each chunk c of this (b, h):
//     Hs   <- H_c (bf16 copy of the fp32 state accumulators, LDS)
//     y_c  = (L o C B^T) x_c + exp(A cdt) C H_c^T + D x_c      (as in k_out)
//     H_{c+1} = exp(A cdt_last) H_c + Bt_c diag(w) x_c      w_j = exp(A (cdt_last - cdt_j))
//
// so HBM sees x once, y once, and the small per-chunk tables (cdt, C B^T, C, B^T) that
// every head of a group shares through L2.  The next chunk's x rows are loaded into
// registers while the current chunk computes.
//
// Tiling (4 waves): state tiles S^T[n][p] -- wave w owns n-tiles [w N/64, (w+1) N/64)
// x all 4 p-tiles; output tiles y^T[p][i] -- wave w owns Q/64 row tiles (paired
// (k, 7-k) for causal balance) x all 4 p-tiles, done two row tiles at a time.
// LDS: x tile Q x 64 (16-byte chunks XOR-swizzled by row so the transpose reads of a
// 16-lane group hit disjoint banks), H_c 64 x N (chunks swizzled by row), three
// per-chunk float tables.  Blocks are numbered so that the heads of one batch row
// share an XCD (and its L2 copy of the per-chunk tables).
#pragma once

#include "kernels.hpp"

namespace ssd {

template <int Q, int N>
struct FusedCfg {
    static constexpr int P = 64;
    static constexpr int RPW = Q / 64;  // row tiles per wave
    static constexpr int SN = N / 64;   // state n-tiles per wave
    static constexpr int XR = Q / 32;   // 16-byte x vectors per thread and chunk
    static constexpr int HSW = (N / 8) < 16 ? (N / 8) : 16;
    static constexpr size_t lds_bytes = (size_t)Q * P * 2 + (size_t)P * N * 2 + 3 * Q * 4;
};

// element offset of x(j, p) in the swizzled x tile (64 bf16 = 128 B per row, 16-byte
// chunks).  A transpose read touches 4 consecutive rows x 32 B per 16-lane group, and two
// groups 8 (or 16) rows apart are serviced together: the 32-byte slot of a row is XORed
// with (j & 3) and with bit 3 ^ bit 4 of j, so all 8 rows of a serviced pair land in
// distinct bank ranges.  Rows j and j + 32 k share a swizzle.
__device__ __forceinline__ int xs_swz(int j) { return (j & 3) ^ (((j >> 3) ^ (j >> 4)) & 1); }
__device__ __forceinline__ int xs_off(int j, int p) {
    const int ch = p >> 3;
    return j * 64 + (((((ch >> 1) ^ xs_swz(j)) << 1) | (ch & 1)) << 3) + (p & 7);
}

// MFMA fragment of the swizzled x tile: lane l holds x(k0 + 8 (l/16) + e, c0 + l % 16)
__device__ __forceinline__ bf16x8 frag_xs(const bf16* Xs, int k0, int c0, int lane) {
    const int s = lane & 15;
    const int r = k0 + 8 * (lane >> 4) + (s >> 2);
    const int col = c0 + 4 * (s & 3);
    const s16x4 a = ds_tr16(Xs + xs_off(r, col));
    const s16x4 b = ds_tr16(Xs + xs_off(r + 4, col));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Same fragment from a lane-constant base: xo = xs_off(8 (l/16) + (l%16)/4, c0 + 4 (l%4)).
// k0 is a multiple of 32, so the row swizzle (j & 3) is unchanged and k0 adds k0 * 64.
__device__ __forceinline__ bf16x8 frag_xs_o(const bf16* Xs, int xo, int k0) {
    const s16x4 a = ds_tr16(Xs + xo + k0 * 64);
    const s16x4 b = ds_tr16(Xs + xo + k0 * 64 + 256);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int N>
__device__ __forceinline__ int hs_off(int p, int n) {
    constexpr int HSW = (N / 8) < 16 ? (N / 8) : 16;
    return p * N + ((((n >> 3) ^ (p % HSW))) << 3) + (n & 7);
}

template <int Q, int N>
__global__ __launch_bounds__(kThreads, 3) void k_fused(const bf16* __restrict__ x, const bf16* __restrict__ Cm,
                                                    const bf16* __restrict__ cb, const bf16* __restrict__ Bt,
                                                    const float* __restrict__ A, const float* __restrict__ D,
                                                    const float* __restrict__ cdt, const float* __restrict__ h0,
                                                    bf16* __restrict__ y, float* __restrict__ hT, int64_t Tn,
                                                    int H, int G, int nc, int BH) {
    typedef FusedCfg<Q, N> CF;
    constexpr int P = 64, RPW = CF::RPW, SN = CF::SN, XR = CF::XR;
    constexpr float LOG2E = 1.4426950408889634f;
    __shared__ __attribute__((aligned(16))) bf16 Xs[Q * P];
    __shared__ __attribute__((aligned(16))) bf16 Hs[P * N];
    __shared__ float cds[Q], w2[Q], u2[Q];

    // blocks k, k+8, k+16, ... run on one XCD: give each XCD a contiguous range of (b, h)
    const int k = blockIdx.x;
    const int64_t bh = (BH % 8 == 0) ? (int64_t)(k % 8) * (BH / 8) + k / 8 : k;
    const int h = (int)(bh % H);
    const int64_t bi = bh / H;
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), l16 = lane & 15, q = lane >> 4;
    const float ah2 = A[h] * LOG2E;
    const float Dh = D ? D[h] : 0.f;
    // one buffer resource per tensor, based at this batch row; rows t >= T fall outside
    // it, so they read as zero and their stores are dropped
    const uint32_t xbytes = (uint32_t)(Tn * H * P * 2);
    const brsrc rx = make_rsrc(x + bi * Tn * H * P, xbytes);
    const brsrc ry = make_rsrc(y + bi * Tn * H * P, xbytes);
    const brsrc rc = make_rsrc(Cm + bi * Tn * G * N, (uint32_t)(Tn * G * N * 2));
    const brsrc rcb = make_rsrc(cb + bi * (int64_t)nc * G * Q * Q, (uint32_t)((int64_t)nc * G * Q * Q * 2));
    const brsrc rbt = make_rsrc(Bt + bi * (int64_t)nc * G * N * Q, (uint32_t)((int64_t)nc * G * N * Q * 2));
    const int XS = H * P * 2, CS = G * N * 2;                     // row strides in bytes
    // per-lane byte offsets, the same for every unit
    const int vx = (tid >> 3) * XS + h * P * 2 + (tid & 7) * 16;  // x prefetch: row tid/8, 8 p
    const int vc = l16 * CS + g * N * 2 + q * 16;                  // C row l16 of a row tile
    const int vq = (l16 * Q + 8 * q) * 2;                          // cb / Bt row l16, k-group q
    const int vy = l16 * XS + h * P * 2 + q * 8;                   // y row l16, p 4q..4q+3

    auto row_tile = [&](int kk) { return (RPW == 1) ? w : ((kk & 1) ? 8 * (kk >> 1) + 7 - w : 8 * (kk >> 1) + w); };
    int rts[RPW];  // this wave's row tiles
#pragma unroll
    for (int t = 0; t < RPW; ++t) rts[t] = row_tile(t);
    // lane-constant LDS offsets: x fragments per p-tile, H rows per 32-wide n-step
    int xo[4], ho[N / 32];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) xo[pt] = xs_off(8 * q + ((lane & 15) >> 2), pt * 16 + 4 * (lane & 3));
#pragma unroll
    for (int n = 0; n < N / 32; ++n) ho[n] = hs_off<N>(l16, n * 32 + 8 * q);

    // state accumulators: lane holds H^T[n = (w SN + a) 16 + 4q + r][p = pt 16 + l16]
    f32x4 acc_h[SN][4];
#pragma unroll
    for (int a = 0; a < SN; ++a)
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
            const int p = pt * 16 + l16, n = (w * SN + a) * 16 + 4 * q;
            acc_h[a][pt] = h0 ? ld4(h0 + (bh * P + p) * N + n) : f32x4{0.f, 0.f, 0.f, 0.f};
        }

    bf16x8 xv[XR];
    float cdv = 0.f, cdr = 0.f, cdl = 0.f;
    // next chunk's x rows (zero past T) and cdt -> registers
    auto prefetch_x = [&](int c) {
        const int s0 = __builtin_amdgcn_readfirstlane(c * Q * XS);
#pragma unroll
        for (int r = 0; r < XR; ++r) xv[r] = bload8(rx, vx, s0 + r * 32 * XS);
        const float* cd = cdt + (bh * nc + c) * (int64_t)Q;
        if (tid < Q) {
            cdv = cd[tid];
            cdr = cd[tid | 31];
        }
        cdl = cd[Q - 1];
    };

    // ---- the chunk's output in passes of up to two row tiles; pass 0 also carries the state
    //      update over every k-step.  Per k-step operands (C B^T rows of the pass's tiles, B^T
    //      rows of the state) are requested one k-step ahead. ----
    constexpr int KS = Q / 32;
    constexpr int NPASS = (RPW + 1) / 2;
    constexpr int TPP = RPW < 2 ? RPW : 2;  // row tiles per pass
    const int vq1 = vq + 16 * Q * 2;        // Bt rows of the second n-tile
    struct KOps {
        bf16x8 gb[TPP];   // C B^T row fragment of each of the pass's row tiles
        bf16x8 bt[SN];    // B^T fragments of the wave's n-tiles (pass 0)
    };

    prefetch_x(0);

    for (int c = 0; c < nc; ++c) {
        const int64_t t0 = (int64_t)c * Q;
        __syncthreads();  // the previous chunk is done with Xs, Hs and the tables
#pragma unroll
        for (int r = 0; r < XR; ++r) {
            const int v = tid + r * kThreads;
            const int jj = v >> 3, ch = v & 7;
            st8(Xs + xs_off(jj, ch * 8), xv[r]);
        }
        if (tid < Q) {
            cds[tid] = cdv;
            w2[tid] = exp2f_fast(ah2 * (cdl - cdv));
            u2[tid] = exp2f_fast(ah2 * (cdr - cdv));
        }
        // entering state H_c -> Hs (bf16), read by the state term
#pragma unroll
        for (int a = 0; a < SN; ++a)
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                const int p = pt * 16 + l16, n = (w * SN + a) * 16 + 4 * q;
                st4(Hs + hs_off<N>(p, n),
                    bf16x4{(bf16)acc_h[a][pt][0], (bf16)acc_h[a][pt][1], (bf16)acc_h[a][pt][2], (bf16)acc_h[a][pt][3]});
            }
        const float dch = exp2f_fast(ah2 * cdl);  // decay over the whole chunk
        __syncthreads();
#pragma unroll
        for (int a = 0; a < SN; ++a)
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) acc_h[a][pt] *= dch;

#pragma unroll
        for (int pass = 0; pass < NPASS; ++pass) {
            const bool su = pass == 0;  // the state update rides on the first pass
            if (pass == NPASS - 1 && NPASS > 1 && c + 1 < nc) prefetch_x(c + 1);  // long lead
            int prt[TPP];               // the pass's row tiles
#pragma unroll
            for (int t = 0; t < TPP; ++t) prt[t] = rts[pass * 2 + t];
            int kend = 0;  // k-steps this pass needs
#pragma unroll
            for (int t = 0; t < TPP; ++t) kend = max(kend, prt[t] / 2 + 1);
            if (su) kend = KS;

            auto load_kops = [&](KOps& o, int ks) {
                const int sbq = __builtin_amdgcn_readfirstlane(((c * G + g) * Q * Q + ks * 32) * 2);
#pragma unroll
                for (int t = 0; t < TPP; ++t)
                    if (ks <= prt[t] / 2) o.gb[t] = bload8(rcb, vq, sbq + prt[t] * 16 * Q * 2);
                if (su) {
                    const int sbt = __builtin_amdgcn_readfirstlane(((c * G + g) * N * Q + w * SN * 16 * Q + ks * 32) * 2);
#pragma unroll
                    for (int a = 0; a < SN; ++a) o.bt[a] = bload8(rbt, a == 0 ? vq : vq1, sbt);
                }
            };
            KOps ops[2];
            load_kops(ops[0], 0);

            // state term: y^T[p][i] = exp(A cdt_i) sum_n H_c[p][n] C_i[n]
            f32x4 acc[TPP][4];
#pragma unroll
            for (int t = 0; t < TPP; ++t) {
                bf16x8 cf[N / 32];
                const int sb = __builtin_amdgcn_readfirstlane((c * Q + prt[t] * 16) * CS);
#pragma unroll
                for (int n = 0; n < N / 32; ++n) cf[n] = bload8(rc, vc, sb + n * 64);
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) acc[t][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int n = 0; n < N / 32; ++n)
#pragma unroll
                    for (int pt = 0; pt < 4; ++pt)
                        acc[t][pt] = mma(acc[t][pt], ld8(Hs + ho[n] + pt * 16 * N), cf[n]);
                const float sc = exp2f_fast(ah2 * cds[prt[t] * 16 + l16]);
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) acc[t][pt] *= sc;
            }

            // k-steps: one read of each x fragment feeds the state update and the pass's tiles
            auto kstep = [&](KOps& o, KOps& nxt, int ks) {
                __builtin_amdgcn_sched_barrier(0);
                if (ks + 1 < kend) load_kops(nxt, ks + 1);
                __builtin_amdgcn_sched_barrier(0);
                const int j0 = ks * 32 + 8 * q;
                bf16x8* mf = o.gb;  // masked in place
                bf16x8* af = o.bt;  // weighted in place
#pragma unroll
                for (int t = 0; t < TPP; ++t) {
                    const int rt = prt[t], i = rt * 16 + l16, nks = rt / 2 + 1;
                    if (ks < nks) {
                        const float ci = cds[i];
                        if (ks < nks - 1) {
                            const float vi = exp2f_fast(ah2 * (ci - cds[ks * 32 + 31]));
#pragma unroll
                            for (int e = 0; e < 8; ++e) mf[t][e] = (bf16)((float)mf[t][e] * (u2[j0 + e] * vi));
                        } else {
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                const int j = j0 + e;
                                // exponent clamped to <= 0 so the unused (j > i) slots stay finite
                                float m = (float)mf[t][e] * exp2f_fast(fminf(ah2 * (ci - cds[j]), 0.f));
                                m = (j <= i) ? m : 0.f;
                                m += (j == i) ? Dh : 0.f;
                                mf[t][e] = (bf16)m;
                            }
                        }
                    }
                }
                if (su)
#pragma unroll
                    for (int a = 0; a < SN; ++a)
#pragma unroll
                        for (int e = 0; e < 8; ++e) af[a][e] = (bf16)((float)af[a][e] * w2[j0 + e]);
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    const bf16x8 xf = frag_xs_o(Xs, xo[pt], ks * 32);
                    if (su)
#pragma unroll
                        for (int a = 0; a < SN; ++a) acc_h[a][pt] = mma(acc_h[a][pt], af[a], xf);
#pragma unroll
                    for (int t = 0; t < TPP; ++t)
                        if (ks <= prt[t] / 2) acc[t][pt] = mma(acc[t][pt], xf, mf[t]);
                }
            };
#pragma unroll 1
            for (int ks = 0; ks < kend; ks += 2) {
                kstep(ops[0], ops[1], ks);
                if (ks + 1 < kend) kstep(ops[1], ops[0], ks + 1);
            }

            // y rows (dropped past T), non-temporal: this lane has 4 consecutive p per p-tile
#pragma unroll
            for (int t = 0; t < TPP; ++t) {
                const int sy = __builtin_amdgcn_readfirstlane((int)((t0 + prt[t] * 16) * XS));
#pragma unroll
                for (int pt = 0; pt < 4; ++pt)
                    __builtin_amdgcn_raw_buffer_store_b64(
                        __builtin_bit_cast(u32x2, bf16x4{(bf16)acc[t][pt][0], (bf16)acc[t][pt][1],
                                                         (bf16)acc[t][pt][2], (bf16)acc[t][pt][3]}),
                        ry, vy, sy + pt * 32, 2);
            }
        }
        if (NPASS == 1 && c + 1 < nc) prefetch_x(c + 1);
    }
    if (hT) {
#pragma unroll
        for (int a = 0; a < SN; ++a)
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                const int p = pt * 16 + l16, n = (w * SN + a) * 16 + 4 * q;
                st4(hT + (bh * P + p) * N + n, acc_h[a][pt]);
            }
    }
}

}  // namespace ssd
