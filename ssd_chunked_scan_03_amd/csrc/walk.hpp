// walk.hpp -- the state recurrence of one (batch, head) chain walked chunk by chunk with the
// state on chip, for the backward pass (bfloat16 x/dy/B/C, headdim 64).
//
// "The chunked algorithm takes both" ("Structured State Space Duality" concept page): one
// recurrence step per chunk carries the state across chunks.  The backward needs it twice:
//
//   forward  H_0 = h0,   H_{c+1} = exp(A cdt_last) H_c + sum_j exp(A (cdt_last - cdt_j)) x_j B_j^T
//            -> hin[c] = H_c (each chunk's entering state), hT = H_nc
//   adjoint  R = dhT,    for c = nc-1 .. 0:  rin[c] = R,  R <- exp(A cdt_last) R + sum_i exp(A cdt_i) dy_i C_i^T
//            -> rin, dh0 = R, and the decay gradient's boundary values <R_c, H_{c+1}>
//
// (the adjoint g_t = dL/dh_t runs the same recurrence backward in time with C for B; see
// bwd.hpp).  One work-group of 4 waves per chain.  Per chunk the B^T (C^T) table rows come
// from the per-chunk transposed tables as matrix-core fragments and the chunk's x (dy) rows
// sit in LDS weighted by their decay.  Loads run half a chunk to a chunk ahead of use, in
// an order that lets the in-order memory counter wait for each without waiting for later
// ones: at the top of chunk c the fragments of c's second half are requested, then c+1's
// rows (into registers), then c+1's cumulative decays and, for the adjoint, the forward
// state H_{c+1} of c+1's boundary value (both straight into LDS, once every wave is past
// the reads of the current ones); at the middle, the fragments of c+1's first half.  So
// the first half computes from fragments already in registers, the second half waits only
// for its own, and everything c+1 needs at its top has had half a chunk or more to arrive.
// Every load is issued on every iteration (the last one re-reads a chunk) so that the
// counter's bookkeeping is the same on every path through the loop.  The state
// tiles follow the fused forward kernel's layout: wave w owns n-tiles
// [w N/64, (w+1) N/64) x all 4 p-tiles, lane (l16, q) holding S^T[n = 16 a + 4 q + r][p = 16 pt + l16].
#pragma once

#include "bwd.hpp"

namespace ssd {

template <int Q, int N>
struct WalkCfg {
    static constexpr int P = 64;
    static constexpr int SN = N / 64;    // state n-tiles per wave
    static constexpr int KS = Q / 32;    // k-steps per chunk
    static constexpr int KH = KS / 2;    // k-steps per half chunk
    static constexpr int XR = Q / 32;    // 16-byte row vectors per thread and chunk (Q rows x 8)
    static constexpr int NW = 16 * SN;   // state columns n per wave
    static constexpr int CPR = NW / 8;   // 16-byte pieces per state row of a wave
    static constexpr int RPI = 64 / CPR; // state rows per 64-lane transfer
};

template <int Q, int N, bool ADJ>
__global__ __launch_bounds__(kThreads, 3) void k_walk(const bf16* __restrict__ xin, const bf16* __restrict__ tab,
                                                   const float* __restrict__ A, const float* __restrict__ cdt,
                                                   const float* __restrict__ init, bf16* __restrict__ sout,
                                                   float* __restrict__ fin, const bf16* __restrict__ hin,
                                                   const float* __restrict__ hTf, float* __restrict__ kpart,
                                                   int nslot, int64_t Tn, int nrows, int H, int G, int nc) {
    typedef WalkCfg<Q, N> CF;
    constexpr int P = 64, SN = CF::SN, KS = CF::KS, KH = CF::KH, XR = CF::XR, PN = P * N;
    constexpr int NW = CF::NW, CPR = CF::CPR, RPI = CF::RPI;
    constexpr float LOG2E = 1.4426950408889634f;
    __shared__ __attribute__((aligned(16))) bf16 Xs[Q * P];
    __shared__ __attribute__((aligned(16))) float cdq[Q];                 // the chunk's cumulative decays
    __shared__ __attribute__((aligned(16))) bf16 Hb[ADJ ? P * N : 8];     // adjoint: H_{c+1}, wave w's columns at w P NW

    // blocks k, k+8, k+16, ... run on one XCD: each XCD takes a contiguous range of chains,
    // so the heads of a batch row share its L2 copy of the per-chunk tables
    const int BH = nrows * H;
    const int k = blockIdx.x;
    const int64_t bh = (BH % 8 == 0) ? (int64_t)(k % 8) * (BH / 8) + k / 8 : k;
    const int h = (int)(bh % H);
    const int64_t bi = bh / H;
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), l16 = lane & 15, q = lane >> 4;
    const float ah2 = A[h] * LOG2E;

    // buffer resources based at this batch row / chain; rows past T read as zero
    const int XS = H * P * 2;  // row stride in bytes
    const brsrc rx = make_rsrc(xin + bi * Tn * H * P, (uint32_t)(Tn * H * P * 2));
    const brsrc rt = make_rsrc(tab + bi * nc * G * N * Q, (uint32_t)((int64_t)nc * G * N * Q * 2));
    const brsrc rcd = make_rsrc(cdt + bh * (int64_t)nc * Q, (uint32_t)((int64_t)nc * Q * 4));
    const brsrc rh = make_rsrc(ADJ ? hin + bh * (int64_t)nc * PN : hin, ADJ ? (uint32_t)((int64_t)nc * PN * 2) : 0u);
    // thread's row vectors: v = tid + 256 r -> row v / 8, columns 8 (v % 8) .. + 8
    const int vrow = tid >> 3, vcol = (tid & 7) * 8;

    int xo[4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) xo[pt] = xs_off(8 * q + ((lane & 15) >> 2), pt * 16 + 4 * (lane & 3));

    f32x4 acc[SN][4];
#pragma unroll
    for (int a = 0; a < SN; ++a)
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
            const int p = pt * 16 + l16, n = (w * SN + a) * 16 + 4 * q;
            acc[a][pt] = init ? ld4(init + (bh * P + p) * N + n) : f32x4{0.f, 0.f, 0.f, 0.f};
        }

    // chunk c's rows into registers
    bf16x8 xv[XR];
    auto prefetch = [&](int c) {
#pragma unroll
        for (int r = 0; r < XR; ++r)
            xv[r] = bload8(rx, vrow * XS + vcol * 2 + (int)h * P * 2,
                           __builtin_amdgcn_readfirstlane((c * Q + 32 * r) * XS));
    };
    // chunk c's cumulative decays into cdq (wave 0), and for the adjoint H_{c+1} into Hb,
    // each wave its own columns, read back by the same wave
    auto stage_lds = [&](int c) {
        if (w == 0 && lane_now() * 4 < Q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rcd, (__attribute__((address_space(3))) void*)cdq, 16,
                                                     lane_now() * 16, __builtin_amdgcn_readfirstlane(c * Q * 4), 0, 0);
        if (ADJ) {
            const int cn = c + 1 < nc ? c + 1 : c;  // (the last chunk's value is formed before the loop)
#pragma unroll
            for (int m = 0; m < CPR; ++m) {
                const int ln = lane_now(), p = m * RPI + ln / CPR, piece = ln % CPR;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rh, (__attribute__((address_space(3))) void*)(Hb + w * P * NW + m * RPI * NW), 16,
                    (p * N + w * NW + piece * 8) * 2, __builtin_amdgcn_readfirstlane(cn * PN * 2), 0, 0);
            }
        }
    };
    // table fragments of half e of chunk c: k-steps [e KH, e KH + KH)
    bf16x8 bt[2][KH][SN];
    auto load_half = [&](int c, int e) {
        const int sbt = __builtin_amdgcn_readfirstlane(((c * G + g) * N * Q + w * SN * (Q / 32) * 512) * 2);
#pragma unroll
        for (int kk = 0; kk < KH; ++kk)
#pragma unroll
            for (int a = 0; a < SN; ++a) bt[e][kk][a] = bload8(rt, lane * 16, sbt + (a * (Q / 32) + e * KH + kk) * 1024);
    };

    // adjoint: the last chunk's boundary value <R_{nc-1}, H_nc> = <dhT, hT> (zero without dhT)
    if (ADJ && nc > 0) {
        float s = 0.f;
        if (init && hTf) {
#pragma unroll
            for (int a = 0; a < SN; ++a)
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    const int p = pt * 16 + l16, n = (w * SN + a) * 16 + 4 * q;
                    const f32x4 hq = ld4(hTf + (bh * P + p) * N + n);
#pragma unroll
                    for (int r = 0; r < 4; ++r) s += acc[a][pt][r] * hq[r];
                }
        }
        s = sum_wave(s);
        if (lane == 0) kpart[(bh * nc + nc - 1) * (int64_t)nslot + w] = s;
    }

    const int c_first = ADJ ? nc - 1 : 0, c_step = ADJ ? -1 : 1;
    if (nc > 0) {
        prefetch(c_first);
        stage_lds(c_first);
        load_half(c_first, 0);
    }
    for (int it = 0; it < nc; ++it) {
        const int c = c_first + c_step * it;
        // the next chunk, or this one again on the last iteration
        const int cn = it + 1 < nc ? c + c_step : c;
        __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): this chunk's rows, decays and H_{c+1} have landed
        __syncthreads();  // ... for every wave; every wave is done with the previous chunk's rows
        // this chunk's rows, weighted by their decay, into LDS
        const float clv = cdq[Q - 1];
        const float dch = exp2f_fast(ah2 * clv);
#pragma unroll
        for (int r = 0; r < XR; ++r) {
            const float cvr = cdq[vrow + 32 * r];
            const float wgt = exp2f_fast(ah2 * (ADJ ? cvr : clv - cvr));
            bf16x8 o = xv[r];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = (bf16)((float)o[e] * wgt);
            st8(Xs + xs_off(vrow + 32 * r, vcol), o);
        }
        if (ADJ) {
            // <R_c, H_{c+1}> (R_c the adjoint before this chunk's step); on the last chunk
            // it lands in an unused slot (the value there is formed before the loop)
            float s = 0.f;
#pragma unroll
            for (int a = 0; a < SN; ++a)
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    const bf16x4 hv = ld4(Hb + w * P * NW + (pt * 16 + l16) * NW + a * 16 + 4 * q);
#pragma unroll
                    for (int r = 0; r < 4; ++r) s += acc[a][pt][r] * (float)hv[r];
                }
            s = sum_wave(s);
            kpart[(bh * nc + c) * (int64_t)nslot + w + (c + 1 < nc ? 0 : 4)] = s;  // every lane: one address
        }
        // the second half's fragments, then the next chunk's rows
        load_half(c, 1);
        prefetch(cn);
        __syncthreads();  // the chunk's rows are in place; every wave is past cdq and Hb
        stage_lds(cn);
        // the state entering this chunk's step (forward: H_c; adjoint: R_c) leaves as bf16,
        // after every load the chunk waits for (stores retire in the same order as loads, so
        // a store ahead of a fragment would hold up its wait)
        bf16* so = sout + (bh * nc + c) * (int64_t)PN;
#pragma unroll
        for (int a = 0; a < SN; ++a)
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                st4(so + (pt * 16 + l16) * N + (w * SN + a) * 16 + 4 * q,
                    bf16x4{(bf16)acc[a][pt][0], (bf16)acc[a][pt][1], (bf16)acc[a][pt][2], (bf16)acc[a][pt][3]});
                acc[a][pt] *= dch;
            }

        // S^T += table^T-fragments x weighted rows, k over the chunk's tokens, half by half
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            if (e == 1) load_half(cn, 0);
#pragma unroll
            for (int kk = 0; kk < KH; ++kk) {
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    const bf16x8 xf = frag_xs_o(Xs, xo[pt], (e * KH + kk) * 32);
#pragma unroll
                    for (int a = 0; a < SN; ++a) acc[a][pt] = mma(acc[a][pt], bt[e][kk][a], xf);
                }
            }
        }
    }
    if (fin) {
#pragma unroll
        for (int a = 0; a < SN; ++a)
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                const int p = pt * 16 + l16, n = (w * SN + a) * 16 + 4 * q;
                st4(fin + (bh * P + p) * N + n, acc[a][pt]);
            }
    }
}

}  // namespace ssd
