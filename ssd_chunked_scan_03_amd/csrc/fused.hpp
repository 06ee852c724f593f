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
// Wave priorities: the work between a chunk's closing barrier and the next chunk's top
// barrier (the next x transfer and the next chunk's tables and H_c, which every wave of the
// work-group waits for) runs at priority 3, the C B^T fragment loops of the output passes
// at 2, the state update at 1 and the state terms at 0.  With two or three work-groups per
// CU, a SIMD then issues first for the wave that gates its work-group's next barrier, then
// for the one in its fragment loop, and the state terms fill the gaps: 302 -> 272 us at
// the 2.7B layer shape, bit-identical.
#pragma once

#include "kernels.hpp"

namespace ssd {

template <int Q, int N>
struct FusedCfg {
    static constexpr int P = 64;
    static constexpr int RPW = Q / 64;            // row tiles per wave
    static constexpr int TPP = RPW >= 2 ? 2 : 1;  // row tiles per output pass
    static constexpr int NPASS = RPW / TPP;       // output passes per chunk
    // C B^T fragments (16 rows x 32 columns) one pass needs: the two tiles of a pass
    // together always cover Q/32 + 1 of them; a single tile at most 2
    static constexpr int NU = TPP == 2 ? Q / 32 + 1 : 2;
    static constexpr int SN = N / 64;             // state n-tiles per wave
    static constexpr int KS = Q / 32;             // k-steps per chunk
    static constexpr int XR = Q / 32;             // 16-byte x vectors per thread and chunk
    static constexpr int NF = N / 32;             // C fragments per row tile
    static constexpr size_t lds_bytes = (size_t)Q * P * 2 + (size_t)P * N * 2 + 3 * Q * 4;
};

// Row tile t of output pass `pass` for wave w.  Tiles r and (Q/16 - 1 - r)-style partners
// are paired so that every pass of every wave holds the same number of causal fragments:
// Q = 256: (w, 15 - w) then (7 - w, 8 + w); Q = 128: (w, 7 - w); Q = 64: (w).
template <int Q>
__device__ __forceinline__ int fused_tile(int pass, int t, int w) {
    if (Q == 256) return pass == 0 ? (t == 0 ? w : 15 - w) : (t == 0 ? 7 - w : 8 + w);
    if (Q == 128) return t == 0 ? w : 7 - w;
    return w;
}

template <int Q, int N>
__global__ __launch_bounds__(kThreads, 3) void k_fused(const bf16* __restrict__ x, const bf16* __restrict__ Cf,
                                                    const bf16* __restrict__ cb, const bf16* __restrict__ Bt,
                                                    const float* __restrict__ A, const float* __restrict__ D,
                                                    const float* __restrict__ cdt, const float* __restrict__ h0,
                                                    bf16* __restrict__ y, float* __restrict__ hT, Rows rows,
                                                    int G) {
    typedef FusedCfg<Q, N> CF;
    constexpr int P = 64, TPP = CF::TPP, NPASS = CF::NPASS, NU = CF::NU, SN = CF::SN, KS = CF::KS,
                  XR = CF::XR, NF = CF::NF;
    constexpr int GW = NU < 4 ? NU : 4;  // C B^T fragments in flight ahead of the one in use
    constexpr float LOG2E = 1.4426950408889634f;
    __shared__ __attribute__((aligned(16))) bf16 Xs[Q * P];
    __shared__ __attribute__((aligned(16))) bf16 Hs[P * N];
    __shared__ float cds[Q], w2[Q], u2[Q];
    __shared__ __attribute__((aligned(16))) float cdq[Q];  // the next chunk's cdt row, by transfer

    // blocks k, k+8, k+16, ... run on one XCD: give each XCD a contiguous range of (row, h)
    const int H = rows.H, BH = rows.nrows * H;
    const int k = blockIdx.x;
    const int64_t bh = (BH % 8 == 0) ? (int64_t)(k % 8) * (BH / 8) + k / 8 : k;
    const int h = (int)(bh % H);
    const int ri = (int)(bh / H);
    const int g = h / (H / G);
    // this row's tokens [0, Tn) and chunks [0, nc) from its bases in each tensor
    const int64_t Tn = rows.len(ri), rt0 = rows.tok0(ri);
    const int nc = rows.nchunks(ri);
    const int64_t kb0 = rows.kbase(ri);
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), l16 = lane & 15, q = lane >> 4;
    const float ah2 = A[h] * LOG2E;
    const float Dh = D ? D[h] : 0.f;
    // one buffer resource per tensor, based at this batch row; rows t >= T fall outside
    // it, so they read as zero and their stores are dropped
    const uint32_t xbytes = (uint32_t)(Tn * H * P * 2);
    const brsrc rx = make_rsrc(x + rt0 * H * P, xbytes);
    const brsrc ry = make_rsrc(y + rt0 * H * P, xbytes);
    const brsrc rc = make_rsrc(Cf + kb0 * G * Q * N, (uint32_t)((int64_t)nc * G * Q * N * 2));
    const brsrc rcb = make_rsrc(cb + kb0 * G * Q * Q, (uint32_t)((int64_t)nc * G * Q * Q * 2));
    const brsrc rbt = make_rsrc(Bt + kb0 * G * N * Q, (uint32_t)((int64_t)nc * G * N * Q * 2));
    const int XS = H * P * 2;                                      // x / y row stride in bytes
    // per-lane byte offsets
    const int vf = lane * 16;                                      // a lane's 16 bytes of a table fragment

    // lane-constant LDS offsets: x fragments per p-tile, H rows per 32-wide n-step
    int xo[4], ho[NF];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) xo[pt] = xs_off(8 * q + ((lane & 15) >> 2), pt * 16 + 4 * (lane & 3));
#pragma unroll
    for (int n = 0; n < NF; ++n) ho[n] = hs_off<N>(l16, n * 32 + 8 * q);

    // state accumulators: lane holds H^T[n = (w SN + a) 16 + 4q + r][p = pt 16 + l16]
    f32x4 acc_h[SN][4];
#pragma unroll
    for (int a = 0; a < SN; ++a)
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
            const int p = pt * 16 + l16, n = (w * SN + a) * 16 + 4 * q;
            acc_h[a][pt] = h0 ? ld4(h0 + (bh * P + p) * N + n) : f32x4{0.f, 0.f, 0.f, 0.f};
        }

    // ---- what one output pass reads from global memory ----
    struct Front {                 // requested before the pass starts
        bf16x8 cf[NF];             //   C rows of the pass's first tile (state term)
        bf16x8 gf[GW];             //   the first C B^T fragments
    };
    auto pass_tiles = [&](int pass, int& tA, int& tB) {
        tA = fused_tile<Q>(pass, 0, w);
        tB = TPP == 2 ? fused_tile<Q>(pass, 1, w) : tA;
        // opaque per call: the offsets derived from the tile indices are recomputed each
        // chunk instead of being hoisted out of the chunk loop (and spilled)
        asm volatile("" : "+s"(tA), "+s"(tB));
    };
    // byte offset (in the C B^T resource) of fragment u of a pass with tiles tA, tB
    auto gf_off = [&](int c, int u, int tA, int tB) {
        const int KA = tA / 2 + 1;
        const bool inA = TPP == 1 || u < KA;
        const int tile = inA ? tA : tB;
        const int ks = TPP == 1 ? min(u, KA - 1) : (inA ? u : u - KA);
        return __builtin_amdgcn_readfirstlane(((c * G + g) * Q * Q + (tile * (Q / 32) + ks) * 512) * 2);
    };
    auto issue_front = [&](Front& f, int c, int pass) {
        int tA, tB;
        pass_tiles(pass, tA, tB);
        const int sb = __builtin_amdgcn_readfirstlane(((c * G + g) * Q * N + tA * (N / 32) * 512) * 2);
#pragma unroll
        for (int n = 0; n < NF; ++n) f.cf[n] = bload8(rc, vf, sb + n * 1024);
#pragma unroll
        for (int u = 0; u < GW; ++u) f.gf[u] = bload8(rcb, vf, gf_off(c, u, tA, tB));
    };
    // the chunk's cdt row straight into LDS (wave 0, one 16-byte slot per lane), so no
    // loaded value has to stay in registers across the chunk loop
    const brsrc rcd = make_rsrc(cdt + rows.cdt_row(ri, h, 0) * Q, (uint32_t)(nc * Q * 4));
    auto dma_cdt = [&](int c) {
        if (w == 0 && lane_now() * 4 < Q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rcd, (__attribute__((address_space(3))) void*)cdq, 16,
                                                     lane_now() * 16, __builtin_amdgcn_readfirstlane(c * Q * 4), 0, 0);
    };
    // chunk c's x rows straight into the (swizzled) x tile; rows past T arrive as zeros.
    // x is read once, so it is fetched non-temporal and leaves the L2 to the per-chunk
    // tables that every head of the batch row reads.
    auto dma_x = [&](int c) {
        int ln = lane;  // opaque: the two lane offsets are rebuilt per call, not kept live
        asm volatile("" : "+v"(ln));
        const int vd0 = xs_dma_lane(ln, 0, XS, h * P * 2), vd1 = xs_dma_lane(ln, 1, XS, h * P * 2);
#pragma unroll
        for (int r = 0; r < XR; ++r) {
            const int m = w * XR + r;
            const int s0 = __builtin_amdgcn_readfirstlane((c * Q + 8 * m) * XS);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void*)(Xs + m * 512), 16,
                                                     xs_dma_bit(m) ? vd1 : vd0, s0, 0, 2);
        }
    };

    Front fr;
    issue_front(fr, 0, 0);
    dma_cdt(0);
    __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): the cdt row is in place
    __syncthreads();

    // tables of a chunk from its cdt row (in cdq) and its entering state -> Hs; runs after
    // the previous chunk's closing barrier and before the chunk's x transfer is issued
    float dch = 1.f;
    int split_diag = 1;  // the chunk's diagonal blocks take the two-factor decay (see below)
    auto stage_tables = [&]() {
            const int ln = lane_now(), tl = w * 64 + ln, lr = ln & 15, lq = ln >> 4;
            const float cl = cdq[Q - 1];
            dch = exp2f_fast(ah2 * cl);  // decay over the whole chunk
            // widest decay across one 32-row block of this chunk (base 2): within 2^64 the
            // diagonal blocks split exp(A (cdt_i - cdt_j)) into u2_j * v_i like the blocks
            // below them (v_i >= 1 there, u2_j >= 2^-64: both far inside float32 range)
            float span = 0.f;
#pragma unroll
            for (int b = 0; b < Q / 32; ++b) span = fmaxf(span, cdq[32 * b + 31] - cdq[32 * b]);
            split_diag = __builtin_amdgcn_readfirstlane((int)(-ah2 * span <= 64.f));
            if (tl < Q) {
                const float cv = cdq[tl], cr = cdq[tl | 31];
                cds[tl] = cv;
                w2[tl] = exp2f_fast(ah2 * (cl - cv));  // decay from row j to the chunk end
                u2[tl] = exp2f_fast(ah2 * (cr - cv));  // decay from row j to its 32-row block end
            }
#pragma unroll
            for (int a = 0; a < SN; ++a)
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    const int p = pt * 16 + lr, n = (w * SN + a) * 16 + 4 * lq;
                    st4(Hs + hs_off<N>(p, n), bf16x4{(bf16)acc_h[a][pt][0], (bf16)acc_h[a][pt][1],
                                                     (bf16)acc_h[a][pt][2], (bf16)acc_h[a][pt][3]});
                }
    };
    stage_tables();
    // An empty row (packed sequences) reads zeros through its zero-size resources, skips
    // the loop and stores hT = h0; its first x transfer is not issued, so no transfer into
    // this work-group's LDS is still in flight when it ends.
    if (nc > 0) dma_x(0);
    for (int c = 0; c < nc; ++c) {
        const int64_t t0 = (int64_t)c * Q;
        __syncthreads();  // the chunk's tables and Hs are in place
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int a = 0; a < SN; ++a)
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) acc_h[a][pt] *= dch;

        // B^T fragments of the state update (the first two are requested during the last pass)
        const int sbt = __builtin_amdgcn_readfirstlane(((c * G + g) * N * Q + w * SN * (Q / 32) * 512) * 2);
        bf16x8 bt[3][SN];

        // ---- output passes ----
#pragma unroll
        for (int pass = 0; pass < NPASS; ++pass) {
            int tA, tB;
            pass_tiles(pass, tA, tB);
            const int KA = tA / 2 + 1, KB = tB / 2 + 1;  // k-steps of each tile (last = diagonal)
            __builtin_amdgcn_sched_barrier(0);

            // the second tile's C rows, requested now and consumed after the first tile's
            bf16x8 cfB[TPP == 2 ? NF : 1];
            if (TPP == 2) {
                const int sb = __builtin_amdgcn_readfirstlane(((c * G + g) * Q * N + tB * (N / 32) * 512) * 2);
#pragma unroll
                for (int n = 0; n < NF; ++n) cfB[n] = bload8(rc, vf, sb + n * 1024);
            }
            __builtin_amdgcn_sched_barrier(0);
            // state term, one tile at a time: y^T[p][i] = exp(A cdt_i) sum_n H_c[p][n] C_i[n]
            f32x4 acc[TPP][4];
#pragma unroll
            for (int t = 0; t < TPP; ++t) {
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) acc[t][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int n = 0; n < NF; ++n)
#pragma unroll
                    for (int pt = 0; pt < 4; ++pt)
                        acc[t][pt] = mma(acc[t][pt], ld8(Hs + ho[n] + pt * 16 * N), t == 0 ? fr.cf[n] : cfB[n]);
                const float sc = exp2f_fast(ah2 * cds[(t == 0 ? tA : tB) * 16 + l16]);
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) acc[t][pt] *= sc;
                __builtin_amdgcn_sched_barrier(0);
            }
            if (pass == 0) {
                // this wave's x transfers are done; after the barrier every wave's are
                __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
                __syncthreads();
            }
            __builtin_amdgcn_s_setprio(2);  // the fragment loop (see the header)
            bf16x8 gf[NU];
#pragma unroll
            for (int u = 0; u < GW; ++u) gf[u] = fr.gf[u];
            __builtin_amdgcn_sched_barrier(0);

            // y leaves in whole 128-byte rows (store_tile16)
            auto store_y = [&](const f32x4* a, int tile) {
                store_tile16(a, ry, __builtin_amdgcn_readfirstlane((int)((t0 + tile * 16) * XS)), XS, h * P * 2);
            };

            // C B^T fragments in order: tile A's k-steps, then tile B's.  The running tile's
            // accumulators are acc[0]; when tile A is done its y rows are stored and tile B's
            // accumulators move in.
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                // (no scheduling fences here or in the state update's k-step loop: letting
                // the compiler interleave neighbouring k-steps measured 2% faster)
                if (u + GW < NU) gf[u + GW] = bload8(rcb, vf, gf_off(c, u + GW, tA, tB));
                const bool inA = TPP == 1 || u < KA;
                if (TPP == 1 && u >= KA) break;
                if (TPP == 2 && u == KA) {
                    store_y(acc[0], tA);
#pragma unroll
                    for (int pt = 0; pt < 4; ++pt) acc[0][pt] = acc[TPP - 1][pt];
                }
                const int tile = inA ? tA : tB;
                const int ks = inA ? u : u - KA;
                const int kd = (inA ? KA : KB) - 1;  // the tile's diagonal k-step
                const int i = tile * 16 + l16, j0 = ks * 32 + 8 * q;
                const float ci = cds[i];
                bf16x8 m = gf[u];
                // Entries above the diagonal are exact zeros in the C B^T table, so no
                // causal cut is needed: any finite decay factor leaves them zero.
                if (ks < kd || split_diag) {
                    // exp(A (cdt_i - cdt_j)) = u2_j * v_i with r the 32-row block end:
                    // below the diagonal block both factors are <= 1; on it v_i >= 1, and
                    // the chunk was checked to keep it within 2^64
                    const float vi = exp2f_fast(ah2 * (ci - cds[ks * 32 + 31]));
                    if (ks < kd) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) m[e] = (bf16)((float)m[e] * (u2[j0 + e] * vi));
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            m[e] = (bf16)((float)m[e] * (u2[j0 + e] * vi) + ((j0 + e == i) ? Dh : 0.f));
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int j = j0 + e;
                        // exponent clamped to <= 0 so the unused (j > i) slots stay finite
                        const float v = (float)m[e] * exp2f_fast(fminf(ah2 * (ci - cds[j]), 0.f));
                        m[e] = (bf16)(v + ((j == i) ? Dh : 0.f));
                    }
                }
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) acc[0][pt] = mma(acc[0][pt], frag_xs_o(Xs, xo[pt], ks * 32), m);
            }
            // What the next phase reads first is requested before the pass's last y store:
            // the memory counter retires accesses in order, so a load issued after a store
            // cannot be waited for without waiting for the store too.
            __builtin_amdgcn_sched_barrier(0);
            if (pass + 1 < NPASS) {
                issue_front(fr, c, pass + 1);
            } else {
#pragma unroll
                for (int ks = 0; ks < 2 && ks < KS; ++ks)
#pragma unroll
                    for (int a = 0; a < SN; ++a) bt[ks][a] = bload8(rbt, vf, sbt + (a * (Q / 32) + ks) * 1024);
                // the next chunk's cdt row: every wave read this chunk's at the chunk top
                if (c + 1 < nc) dma_cdt(c + 1);
            }
            __builtin_amdgcn_sched_barrier(0);
            store_y(acc[0], TPP == 2 ? tB : tA);
            __builtin_amdgcn_s_setprio(0);
        }

        // ---- state update H_{c+1} = exp(A cdt_last) H_c + B^T diag(w) X_c, B^T fragments
        //      requested two k-steps ahead ----
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 2 < KS) {
#pragma unroll
                for (int a = 0; a < SN; ++a) bt[(ks + 2) % 3][a] = bload8(rbt, vf, sbt + (a * (Q / 32) + ks + 2) * 1024);
            }
            const int j0 = ks * 32 + 8 * q;
            bf16x8 bw[SN];
#pragma unroll
            for (int a = 0; a < SN; ++a)
#pragma unroll
                for (int e = 0; e < 8; ++e) bw[a][e] = (bf16)((float)bt[ks % 3][a][e] * w2[j0 + e]);
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                const bf16x8 xf = frag_xs_o(Xs, xo[pt], ks * 32);
#pragma unroll
                for (int a = 0; a < SN; ++a) acc_h[a][pt] = mma(acc_h[a][pt], bw[a], xf);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): the next cdt row has landed
        if (c + 1 < nc) issue_front(fr, c + 1, 0);
        __syncthreads();  // every wave is done with Xs, Hs and the tables of this chunk
        __builtin_amdgcn_s_setprio(3);  // the chunk boundary (see the header)
        if (c + 1 < nc) {
            dma_x(c + 1);
            stage_tables();
        }
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
