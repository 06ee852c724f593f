// kernels.hpp -- the SSD chunked-scan kernels for gfx950.
//
// The chunked algorithm ("Structured State Space Duality" concept page, section
// "The chunked algorithm takes both"): split the sequence into chunks of Q tokens;
// on every Q x Q diagonal block evaluate the quadratic (masked-attention) form; carry
// one state across chunks with one recurrence step per chunk; the off-diagonal blocks
// factor as (chunk output projection) x (accumulated decay) x (chunk input
// projection) and are never expanded.  Decay sums and states stay in float32
// (section "When it breaks").
//
// Kernels, in launch order (one launch each, all on the caller's stream):
//   k_cumsum  chunk-local inclusive cumulative sum of dt           -> cdt
//   k_cb      C_c B_c^T per (batch, chunk, group), scalar decay only -> cb
//   k_state   chunk state S_c = sum_j decay(last, j) x_j B_j^T      -> states
//   k_scan    H_0 = h0, H_{c+1} = decay(chunk c) H_c + S_c           -> hin, hT
//   k_out     y = (L o C B^T) x + decay(i) C_i H_c + D x  per chunk  -> y
// Shapes: x, y [b,T,H,P]; dt [b,T,H]; B, C [b,T,G,N]; cdt [b,H,nc,Q];
// cb [b,nc,G,Q,Q]; states [b,H,nc,P,N] f32; hin [b,H,nc,P,N] (x's dtype).
#pragma once

#include "device.hpp"

namespace ssd {

constexpr int kThreads = 256;  // 4 waves of 64

// ---------------------------------------------------------------------------
// The rows of a launch.  A row is one sequence with its own state; the state restarts at
// every row ("Structured State Space Duality" concept page, section "The chunked
// algorithm takes both": the chunks of one sequence pass the state along; separate
// sequences are separate maps).
//  * Dense: `nrows` rows of T tokens each; row r holds tokens [r T, (r + 1) T) and
//    chunks [r nc, (r + 1) nc).
//  * Packed (variable length): all rows share one token axis of T tokens; ts[r] is row
//    r's first token and kb[r] its first chunk (nrows + 1 entries each, built on the
//    device by k_rows from the caller's cu_seqlens).
// Per-chunk tables (C B^T, B^T) are indexed by the global chunk k = first chunk + c.
// cdt is [b][H][nc][Q] for dense rows and [H][kcap][Q] for packed rows.
// ---------------------------------------------------------------------------
struct Rows {
    const int* ts;  // nullptr: dense rows
    const int* kb;
    int64_t T;      // dense: tokens per row; packed: tokens of the shared axis
    int nc;         // dense: chunks per row
    int nrows, H;
    int kcap;       // packed: capacity of the global chunk axis (cdt row stride)
    __device__ bool packed() const { return ts != nullptr; }
    __device__ int64_t tok0(int r) const { return packed() ? (int64_t)ts[r] : (int64_t)r * T; }
    __device__ int64_t len(int r) const { return packed() ? (int64_t)(ts[r + 1] - ts[r]) : T; }
    __device__ int kbase(int r) const { return packed() ? kb[r] : r * nc; }
    __device__ int nchunks(int r) const { return packed() ? kb[r + 1] - kb[r] : nc; }
    __device__ int total_chunks() const { return packed() ? kb[nrows] : nrows * nc; }
    // the row holding global chunk k (0 <= k < total_chunks()): the last r with kb[r] <= k,
    // which skips empty rows
    __device__ int row_of(int k) const {
        if (!packed()) return k / nc;
        int lo = 0, hi = nrows;  // kb[lo] <= k < kb[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (kb[mid] <= k) lo = mid;
            else hi = mid;
        }
        return lo;
    }
    // first element of chunk c's cdt row of (row r, head h), in units of Q floats
    __device__ int64_t cdt_row(int r, int h, int c) const {
        return packed() ? (int64_t)h * kcap + kb[r] + c : ((int64_t)r * H + h) * nc + c;
    }
};

// The (batch row, head, chunk) item of a one-dimensional grid of b * H * nc work-groups:
// the heads of one (batch row, chunk) are adjacent, so the work-groups that read the same
// per-chunk rows of B / C and the group's tables run together, and each XCD (blocks k,
// k + 8, k + 16, ... are dispatched to one XCD) takes a contiguous range of items, so
// those readers share its L2.  Returns b * H + h; c is the chunk.
__device__ __forceinline__ int64_t chunk_item(int H, int nc, int& c) {
    const int64_t nb = gridDim.x;
    int64_t k = blockIdx.x;
    if (nb % 8 == 0) k = (k % 8) * (nb / 8) + k / 8;
    const int h = (int)(k % H);
    const int64_t bc = k / H;
    c = (int)(bc % nc);
    return (bc / nc) * H + h;
}

// ---------------------------------------------------------------------------
// k_rows: the packed-row map from the caller's cu_seqlens (nrows + 1 token offsets).
// ts[r] = cu[r] clamped to [ts[r-1], T] (so every row lies inside the token axis, in
// order, whatever the offsets hold), ts[0] = clamp(cu[0]); kb = prefix sums of
// ceil((ts[r+1] - ts[r]) / Q).  One work-group of 1024 threads, two block scans.
// ---------------------------------------------------------------------------
template <typename V, typename Op>
__device__ V block_inclusive_scan(V v, Op op, V* part) {  // part: >= 16 entries of LDS
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const V o = __shfl_up(v, off, 64);
        if (lane >= off) v = op(v, o);
    }
    if (lane == 63) part[w] = v;
    __syncthreads();
    if (w == 0) {
        V pv = lane < nw ? part[lane] : part[0];
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            const V o = __shfl_up(pv, off, 64);
            if (lane >= off) pv = op(pv, o);
        }
        if (lane < nw) part[lane] = pv;
    }
    __syncthreads();
    if (w > 0) v = op(v, part[w - 1]);
    __syncthreads();
    return v;
}

template <int BLOCK = 1024>  // a template so only the unit that launches it instantiates it
__global__ __launch_bounds__(BLOCK) void k_rows(const int* __restrict__ cu, int nrows, int64_t T, int Q,
                                               int* __restrict__ ts, int* __restrict__ kb) {
    __shared__ long long part[16];
    const int n = nrows + 1, per = (n + BLOCK - 1) / BLOCK, i0 = threadIdx.x * per;
    // 1. ts = running maximum of the clamped offsets (a nondecreasing sequence in [0, T])
    long long mx = 0;
    for (int i = i0; i < i0 + per && i < n; ++i) mx = max(mx, min((long long)max(cu[i], 0), (long long)T));
    const auto vmax = [](long long a, long long b) { return a > b ? a : b; };
    long long pre = block_inclusive_scan(mx, vmax, part);
    long long run = __shfl_up(pre, 1, 64);
    if ((threadIdx.x & 63) == 0) run = (threadIdx.x >> 6) > 0 ? part[(threadIdx.x >> 6) - 1] : 0;
    __syncthreads();
    for (int i = i0; i < i0 + per && i < n; ++i) {
        run = max(run, min((long long)max(cu[i], 0), (long long)T));
        ts[i] = (int)run;
    }
    __syncthreads();
    // 2. kb = exclusive prefix sums of the rows' chunk counts
    long long cnt = 0;
    for (int i = i0; i < i0 + per && i < nrows; ++i) cnt += (ts[i + 1] - ts[i] + Q - 1) / Q;
    const auto vadd = [](long long a, long long b) { return a + b; };
    const long long inc = block_inclusive_scan(cnt, vadd, part);
    long long acc = inc - cnt;
    for (int i = i0; i < i0 + per && i < nrows; ++i) {
        kb[i] = (int)acc;
        acc += (ts[i + 1] - ts[i] + Q - 1) / Q;
    }
    if (threadIdx.x == BLOCK - 1) kb[nrows] = (int)inc;
}

// ---------------------------------------------------------------------------
// k_cumsum: cdt[r,h,c,i] = sum_{k=0..i} dt[row r, cQ+k, h] (restarting every chunk;
// positions past the row's end repeat the last valid value exactly).  The log-decay of
// the chunk-local product of a_k is A * cdt.  Grid (chunks, 1, ceil(H/16)) over the
// global chunk axis; a [Q x 16] tile of dt is transposed through LDS, then each wave
// scans one head at a time: Q/64 consecutive tokens per lane, a lane-serial sum and a
// wave prefix sum.
// ---------------------------------------------------------------------------
constexpr int kCumsumHeads = 16;  // heads per cumsum work-group
template <int Q>
constexpr size_t cumsum_smem() { return (size_t)kCumsumHeads * (Q + 1) * sizeof(float); }

template <int Q>
__device__ __forceinline__ void cumsum_body(const float* __restrict__ dt, float* __restrict__ cdt, Rows rows,
                                            int k, int hz, float (*s)[Q + 1]) {
    constexpr int HS = kCumsumHeads, QPL = Q / 64;
    if (k >= rows.total_chunks()) return;
    const int r = rows.row_of(k);
    const int c = k - rows.kbase(r);
    const int64_t T = rows.len(r), rt0 = rows.tok0(r);
    const int H = rows.H;
    const int hbase = hz * HS;
    const int tid = threadIdx.x;
    for (int idx = tid; idx < Q * HS; idx += kThreads) {
        const int t = idx / HS, hh = idx - t * HS;
        const int64_t tok = (int64_t)c * Q + t;
        const int h = hbase + hh;
        s[hh][t] = (tok < T && h < H) ? dt[(rt0 + tok) * H + h] : 0.f;
    }
    __syncthreads();
    const int lane = tid & 63, w = tid >> 6;
    for (int hh = w; hh < HS && hbase + hh < H; hh += 4) {
        float v[QPL];
        float run = 0.f;
#pragma unroll
        for (int e = 0; e < QPL; ++e) {
            run += s[hh][lane * QPL + e];
            v[e] = run;
        }
        float incl = run;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float o = __shfl_up(incl, off, 64);
            if (lane >= off) incl += o;
        }
        float excl = __shfl_up(incl, 1, 64);
        if (lane == 0) excl = 0.f;
#pragma unroll
        for (int e = 0; e < QPL; ++e) v[e] += excl;
        // A ragged last chunk: positions past T take the last valid value bit for bit
        // (the prefix tree would otherwise round them differently), so that the decay
        // from any token to the chunk end is exactly 1 for the last token.
        const int64_t rem = T - (int64_t)c * Q;
        if (rem < Q) {
            const int pl = (int)rem - 1, ll = pl / QPL, el = pl - ll * QPL;
            float cand = v[0];
#pragma unroll
            for (int e = 1; e < QPL; ++e)
                if (e == el) cand = v[e];
            const float lastv = __shfl(cand, ll, 64);
#pragma unroll
            for (int e = 0; e < QPL; ++e)
                if (lane * QPL + e > pl) v[e] = lastv;
        }
        float* out = cdt + rows.cdt_row(r, hbase + hh, c) * Q + lane * QPL;
#pragma unroll
        for (int e = 0; e < QPL; ++e) out[e] = v[e];
    }
}

template <int Q>
__global__ __launch_bounds__(kThreads) void k_cumsum(const float* __restrict__ dt,
                                                     float* __restrict__ cdt, Rows rows) {
    __shared__ float s[kCumsumHeads][Q + 1];
    cumsum_body<Q>(dt, cdt, rows, blockIdx.x, blockIdx.z, s);
}

// ---------------------------------------------------------------------------
// k_cb: cb[b,c,g][i][j] = sum_n C[b,cQ+i,g,n] B[b,cQ+j,g,n] for the 64x64 blocks on
// and below the diagonal (block row >= block column); tokens past T read as 0.
// This is the query-key product of the diagonal block, shared by every head of the
// group.  In the blocks on the diagonal the entries above it (j > i, outside the causal
// form) are stored as exact zeros, so that a consumer's decay factor there needs no
// causal cut (0 times any finite factor is 0).  Grid (chunks, nb(nb+1)/2, G) over the global chunk axis, nb = Q/64.  Each wave computes the transposed
// tile cb^T[j][i] for 16 j x 64 i, so a lane ends up owning 4 consecutive j of one
// row i and stores them as one vector.
// TR = true writes the same blocks transposed, cbt[j][i] = B_j . C_i (i >= j blocks, i
// contiguous), the layout the backward pass reads its input-gradient operand from: the
// operands swap places in the matrix-core step, so a lane then owns 4 consecutive i.
// ---------------------------------------------------------------------------
// dstate from which the 64 C rows of a block are staged in LDS once (shared by its 4 waves)
// rather than loaded by every wave
constexpr int kCbStageN = 256;
template <typename T, int N>
constexpr size_t cb_smem() { return (sizeof(T) == 2 && N >= kCbStageN) ? (size_t)64 * (N + 8) * sizeof(T) : 0; }

template <typename T, int N, bool TR = false>
__device__ __forceinline__ void cb_body(const T* __restrict__ Bm, const T* __restrict__ Cm, T* __restrict__ cb,
                                        Rows rows, int G, int Q, int kg, int pidx, int g, T* __restrict__ cs) {
    typedef typename V8<T>::type v8;
    typedef typename V4<T>::type v4;
    if (kg >= rows.total_chunks()) return;
    const int rr = rows.row_of(kg);
    const int c = kg - rows.kbase(rr);
    const int64_t Tn = rows.len(rr);
    // this row's B / C start here; its tokens are [0, Tn) from this base
    Bm += rows.tok0(rr) * G * N;
    Cm += rows.tok0(rr) * G * N;
    const int64_t bi = 0;
    int I = 0;
    while ((I + 1) * (I + 2) / 2 <= pidx) ++I;
    const int J = pidx - I * (I + 1) / 2;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int l16 = lane & 15, q = lane >> 4;
    const int64_t tok0 = (int64_t)c * Q;
    const int jr = J * 64 + 16 * w + l16;
    // (32-bit buffer offsets: the batch row's B / C must span less than 2 GiB)
    if constexpr (sizeof(T) == 2 && N % 32 == 0) if (Tn * G * N * 2 < ((int64_t)1 << 31)) {
        // bfloat16: branch-free buffer loads (rows past T read as zero), requested four
        // k-steps ahead of the matrix-core step that consumes them
        constexpr int KS = N / 32, DEPTH = KS < 4 ? KS : 4;
        const uint32_t rowb = (uint32_t)(G * N * 2);
        const brsrc rb = make_rsrc(Bm + bi * Tn * G * N, (uint32_t)(Tn * G * N * 2));
        const brsrc rc = make_rsrc(Cm + bi * Tn * G * N, (uint32_t)(Tn * G * N * 2));
        const int s0 = __builtin_amdgcn_readfirstlane((int)(tok0 * rowb + g * N * 2));
        const int vb = jr * rowb + 16 * q;                     // B row jr, k-group q
        const int vc = (I * 64 + l16) * rowb + 16 * q;          // C row I*64 + l16 (+ 16 ct rows)
        constexpr bool STAGE = N >= kCbStageN;
        constexpr int LDC = N + 8;
        if constexpr (STAGE) {
            for (int v = threadIdx.x; v < 64 * N / 8; v += kThreads) {
                const int r = v / (N / 8), n0 = (v - r * (N / 8)) * 8;
                st8(cs + r * LDC + n0, bload8(rc, r * (int)rowb + n0 * 2, s0 + I * 64 * (int)rowb));
            }
            __syncthreads();
        }
        bf16x8 fb[KS], fc[KS][4];
        auto load = [&](int ks) {
            fb[ks] = bload8(rb, vb, s0 + ks * 64);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
                fc[ks][ct] = STAGE ? ld8(reinterpret_cast<const bf16*>(cs) + (16 * ct + l16) * LDC + ks * 32 + 8 * q)
                                   : bload8(rc, vc, s0 + ks * 64 + ct * 16 * (int)rowb);
        };
        f32x4 acc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < DEPTH; ++ks) load(ks);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            __builtin_amdgcn_sched_barrier(0);
            if (ks + DEPTH < KS) load(ks + DEPTH);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) acc[ct] = TR ? mma(acc[ct], fc[ks][ct], fb[ks]) : mma(acc[ct], fb[ks], fc[ks][ct]);
        }
        T* out = cb + ((int64_t)kg * G + g) * (int64_t)Q * Q;
        const int j0 = J * 64 + 16 * w + 4 * q;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            const int i = I * 64 + 16 * ct + l16;
            bf16x4 v = bf16x4{(bf16)acc[ct][0], (bf16)acc[ct][1], (bf16)acc[ct][2], (bf16)acc[ct][3]};
            if (!TR && I == J)
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = (j0 + r > i) ? (bf16)0.f : v[r];
            if (TR) st4(out + tfrag(J * 64 + 16 * w + l16, I * 64 + 16 * ct + 4 * q, Q), v);
            else st4(out + tfrag(i, j0, Q), v);
        }
        return;
    }
    const bool jv = tok0 + jr < Tn;
    const T* brow = Bm + ((bi * Tn + tok0 + (jv ? jr : 0)) * G + g) * N;
    f32x4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
    for (int k0 = 0; k0 < N; k0 += 32) {
        const bool kv = (N % 32 == 0) || (k0 + 8 * q < N);  // N = 16: half the k-step is padding
        const v8 a = (jv && kv) ? ld8(brow + k0 + 8 * q) : zero8<T>();
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            const int ir = I * 64 + 16 * ct + l16;
            const bool iv = kv && tok0 + ir < Tn;
            const v8 b = iv ? ld8(Cm + ((bi * Tn + tok0 + ir) * G + g) * N + k0 + 8 * q) : zero8<T>();
            acc[ct] = TR ? mma(acc[ct], b, a) : mma(acc[ct], a, b);
        }
    }
    T* out = cb + ((int64_t)kg * G + g) * (int64_t)Q * Q;
    const int j0 = J * 64 + 16 * w + 4 * q;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
        const int i = I * 64 + 16 * ct + l16;
        v4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = from_f<T>((!TR && I == J && j0 + r > i) ? 0.f : acc[ct][r]);
        if (TR) st4(out + tfrag(J * 64 + 16 * w + l16, I * 64 + 16 * ct + 4 * q, Q), v);
        else st4(out + tfrag(i, j0, Q), v);
    }
}

// dstate from which k_prep takes a whole 64-row block row of C B^T per work-group
constexpr int kPrepRowN = 128;

// One 64-row block row I of a chunk's C B^T (tiles J = 0 .. I, I < 4) for bfloat16 with
// dstate >= kPrepRowN: the block row's C rows are staged in LDS once and serve every
// tile; each tile's B rows are in flight while the previous tile computes.  Same
// output as cb_body on each tile (the same products in the same order).  (Taking the
// tiles in pairs, so that each C fragment read from LDS feeds two matrix-core steps,
// measured slower: 214 against 194 us at the long workload.)
template <int N>
__device__ __forceinline__ void cb_row_body(const bf16* __restrict__ Bm, const bf16* __restrict__ Cm,
                                            bf16* __restrict__ cb, Rows rows, int G, int Q, int kg, int I, int g,
                                            bf16* __restrict__ cs) {
    static_assert(N % 32 == 0 && N >= kPrepRowN, "staged block rows");
    if (kg >= rows.total_chunks()) return;
    const int rr = rows.row_of(kg);
    const int c = kg - rows.kbase(rr);
    const int64_t Tn = rows.len(rr);
    Bm += rows.tok0(rr) * G * N;
    Cm += rows.tok0(rr) * G * N;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int l16 = lane & 15, q = lane >> 4;
    const int64_t tok0 = (int64_t)c * Q;
    constexpr int KS = N / 32, LDC = N + 8;
    const uint32_t rowb = (uint32_t)(G * N * 2);
    const uint32_t span = (uint32_t)(Tn * G * N * 2);  // the caller checks it is under 2 GiB
    const brsrc rb = make_rsrc(Bm, span);
    const brsrc rc = make_rsrc(Cm, span);
    const int s0 = __builtin_amdgcn_readfirstlane((int)(tok0 * rowb + g * N * 2));
    for (int v = threadIdx.x; v < 64 * N / 8; v += kThreads) {
        const int r = v / (N / 8), n0 = (v - r * (N / 8)) * 8;
        st8(cs + r * LDC + n0, bload8(rc, r * (int)rowb + n0 * 2, s0 + I * 64 * (int)rowb));
    }
    __syncthreads();
    bf16* out = cb + ((int64_t)kg * G + g) * (int64_t)Q * Q;
    // B rows of tile J + 1 are requested while tile J computes (two register sets; the
    // tile loop is unrolled so both are indexed statically)
    bf16x8 fb[2][KS];
    auto load = [&](int J, int set) {
        const int vb = (J * 64 + 16 * w + l16) * rowb + 16 * q;  // B row of this wave's column, k-group q
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) fb[set][ks] = bload8(rb, vb, s0 + ks * 64);
    };
    load(0, 0);
#pragma unroll
    for (int J = 0; J < 4; ++J) {
        if (J > I) break;
        __builtin_amdgcn_sched_barrier(0);
        if (J + 1 <= I) load(J + 1, (J + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
        f32x4 acc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
                acc[ct] = mma(acc[ct], fb[J & 1][ks], ld8(cs + (16 * ct + l16) * LDC + ks * 32 + 8 * q));
        const int j0 = J * 64 + 16 * w + 4 * q;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            const int i = I * 64 + 16 * ct + l16;
            bf16x4 v = bf16x4{(bf16)acc[ct][0], (bf16)acc[ct][1], (bf16)acc[ct][2], (bf16)acc[ct][3]};
            if (J == I)  // above the diagonal: exact zeros
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = (j0 + r > i) ? (bf16)0.f : v[r];
            st4(out + tfrag(i, j0, Q), v);
        }
    }
}

// C B^T work items of one chunk and group in k_prep: a block row per work-group where
// the staged path applies (bfloat16, dstate >= kPrepRowN), else one 64 x 64 tile each
template <typename T, int N>
__host__ __device__ constexpr bool prep_cb_rows() { return sizeof(T) == 2 && N >= kPrepRowN && N % 32 == 0; }
template <typename T, int N>
__host__ __device__ constexpr int prep_cb_tasks(int nb) { return prep_cb_rows<T, N>() ? nb : nb * (nb + 1) / 2; }

template <typename T, int N, bool TR = false>
__global__ __launch_bounds__(kThreads) void k_cb(const T* __restrict__ Bm, const T* __restrict__ Cm,
                                                 T* __restrict__ cb, Rows rows, int G, int Q) {
    __shared__ __attribute__((aligned(16))) unsigned char cs[cb_smem<T, N>() > 0 ? cb_smem<T, N>() : 16];
    cb_body<T, N, TR>(Bm, Cm, cb, rows, G, Q, blockIdx.x, blockIdx.y, blockIdx.z, reinterpret_cast<T*>(cs));
}

// ---------------------------------------------------------------------------
// k_bt: Bt[b,c,g][n][j] = B[b, cQ+j, g, n] (0 past T): each chunk's B by token, the
// operand the fused kernel's state update (and the backward's walks) read; with Cf, also
// Cf[b,c,g][i][n] = C[b, cQ+i, g, n] (0 past T), the operand of the fused kernel's state
// term.  Both in fragment order (tfrag).  Grid (chunks * Q/64, G) over the global chunk
// axis: one 64-token slab per work-group, B transposed through LDS.
// ---------------------------------------------------------------------------
template <typename T, int N>
constexpr size_t bt_smem() { return (size_t)N * (64 + 8) * sizeof(T); }

template <typename T, int N>
__device__ __forceinline__ void bt_body(const T* __restrict__ Bm, T* __restrict__ Bt, const T* __restrict__ Cm,
                                        T* __restrict__ Cf, Rows rows, int G, int Q, int kg, int j0, int g,
                                        T* __restrict__ s) {
    typedef typename V8<T>::type v8;
    constexpr int JB = 64, LD = JB + 8;
    if (kg >= rows.total_chunks()) return;
    const int rr = rows.row_of(kg);
    const int c = kg - rows.kbase(rr);
    const int64_t Tn = rows.len(rr);
    Bm += rows.tok0(rr) * G * N;
    const int64_t bi = 0;
    const int64_t tok0 = (int64_t)c * Q + j0;
    if constexpr (N % 32 == 0) {
        if (Cf) {
            Cm += rows.tok0(rr) * G * N;
            T* cout = Cf + ((int64_t)kg * G + g) * (int64_t)Q * N;
            for (int v = threadIdx.x; v < JB * N / 8; v += kThreads) {
                const int jj = v / (N / 8), n0 = (v - jj * (N / 8)) * 8;
                const v8 val = (tok0 + jj < Tn) ? ld8(Cm + ((bi * Tn + tok0 + jj) * G + g) * N + n0) : zero8<T>();
                st8(cout + tfrag(j0 + jj, n0, N), val);
            }
        }
    }
    for (int v = threadIdx.x; v < JB * N / 8; v += kThreads) {
        const int jj = v / (N / 8), n0 = (v - jj * (N / 8)) * 8;
        const v8 val = (tok0 + jj < Tn) ? ld8(Bm + ((bi * Tn + tok0 + jj) * G + g) * N + n0) : zero8<T>();
#pragma unroll
        for (int e = 0; e < 8; ++e) s[(n0 + e) * LD + jj] = val[e];
    }
    __syncthreads();
    T* out = Bt + ((int64_t)kg * G + g) * (int64_t)N * Q;
    for (int v = threadIdx.x; v < N * JB / 8; v += kThreads) {
        const int n = v / (JB / 8), jv = (v - n * (JB / 8)) * 8;
        st8(out + tfrag(n, j0 + jv, Q), ld8(&s[n * LD + jv]));
    }
}

template <typename T, int N>
__global__ __launch_bounds__(kThreads) void k_bt(const T* __restrict__ Bm, T* __restrict__ Bt,
                                                 const T* __restrict__ Cm, T* __restrict__ Cf, Rows rows, int G,
                                                 int Q) {
    __shared__ __attribute__((aligned(16))) T s[N * (64 + 8)];
    const int slabs = Q / 64;
    const int kg = blockIdx.x / slabs;
    bt_body<T, N>(Bm, Bt, Cm, Cf, rows, G, Q, kg, (blockIdx.x - kg * slabs) * 64, blockIdx.y, s);
}

// ---------------------------------------------------------------------------
// k_prep: the per-chunk preparation of a forward in one launch.  The three tables do
// not depend on one another, so one grid (chunks, tasks) runs them side by side:
//   y in [0, nh)                       k_cumsum's work for heads 16 y .. 16 y + 15
//   y in [nh, nh + npair G)            k_cb's work for block pair (y - nh) % npair, group (y - nh) / npair
//   y in [nh + npair G, + nslab G)     k_bt's work for 64-token slab, group (when BT)
// (nh = ceil(H / 16), npair = nb (nb + 1) / 2 with nb = Q / 64, nslab = Q / 64.)
// ---------------------------------------------------------------------------
template <typename T, int N, int Q, bool BT>
__global__ __launch_bounds__(kThreads) void k_prep(const float* __restrict__ dt, float* __restrict__ cdt,
                                                   const T* __restrict__ Bm, const T* __restrict__ Cm,
                                                   T* __restrict__ cb, T* __restrict__ Bt, Rows rows, int G) {
    constexpr int nb = Q / 64, nslab = Q / 64;
    // one LDS buffer for whichever task the work-group runs
    constexpr size_t s1 = cumsum_smem<Q>(), s3 = BT ? bt_smem<T, N>() : 0;
    constexpr size_t s2 = prep_cb_rows<T, N>() ? (size_t)64 * (N + 8) * 2 : cb_smem<T, N>();
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
    constexpr int ncb = prep_cb_tasks<T, N>(nb);
    if (y < ncb * G) {
        if constexpr (prep_cb_rows<T, N>()) {
            // block rows need the batch row's B / C to span under 2 GiB (32-bit buffer offsets)
            const int64_t span = rows.len(rows.row_of(k < rows.total_chunks() ? k : 0)) * G * N * 2;
            if (span < ((int64_t)1 << 31)) {
                cb_row_body<N>(Bm, Cm, cb, rows, G, Q, k, y % ncb, y / ncb, reinterpret_cast<bf16*>(smem));
                return;
            }
            // otherwise each tile of the block row, as k_cb computes it
            const int I = y % ncb;
            for (int J = 0; J <= I; ++J) {
                cb_body<T, N, false>(Bm, Cm, cb, rows, G, Q, k, I * (I + 1) / 2 + J, y / ncb, reinterpret_cast<T*>(smem));
                __syncthreads();
            }
        } else {
            cb_body<T, N, false>(Bm, Cm, cb, rows, G, Q, k, y % ncb, y / ncb, reinterpret_cast<T*>(smem));
        }
        return;
    }
    y -= ncb * G;
    // (the C copy follows the B^T tables of every chunk in the same region)
    if (BT) bt_body<T, N>(Bm, Bt, Cm, Bt + (int64_t)rows.kcap * G * N * Q, rows, G, Q, k, (y % nslab) * 64,
                          y / nslab, reinterpret_cast<T*>(smem));
}

// ---------------------------------------------------------------------------
// The bfloat16 x tile of 64-element rows (headdim 64) in LDS, shared by the chunk kernels.
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

// Fragment with rows ra + e (e < 4) and rb + e - 4 (e >= 4) of column c0 + l % 16, as
// frag_rows_split, from the swizzled tile.
__device__ __forceinline__ bf16x8 frag_xs_split(const bf16* Xs, int ra, int rb, int c0, int lane) {
    const int s = lane & 15;
    const int col = c0 + 4 * (s & 3);
    const s16x4 a = ds_tr16(Xs + xs_off(ra + (s >> 2), col));
    const s16x4 b = ds_tr16(Xs + xs_off(rb + (s >> 2), col));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Direct-to-LDS transfer m (1 KB) of a chunk's x tile fills LDS bytes [1024 m, 1024 m + 1024)
// lane by lane: x-tile rows 8 m .. 8 m + 7, eight 16-byte slots each.  Lane l takes row
// 8 m + l/8 and slot l % 8; the row swizzle decides which column chunk that slot holds.
// Within the row the swizzle depends on (l/8) & 3 and on one bit of m (bit 0 ^ bit 1), so
// a lane needs two source offsets, one per value of that bit; the row offset is uniform.
__device__ __forceinline__ int xs_dma_lane(int lane, int bit, int XS, int hcol) {
    const int r = lane >> 3, slot = lane & 7;
    const int ch = ((((slot >> 1) ^ (r & 3) ^ bit)) << 1) | (slot & 1);
    return r * XS + hcol + ch * 16;
}
__device__ __forceinline__ int xs_dma_bit(int m) { return (m ^ (m >> 1)) & 1; }

// The 16 rows of an output tile leave as whole 128-byte bfloat16 rows (headdim 64).  The
// accumulators hold the tile transposed: lane (i, q) has p = 16 pt + 4 q + r of row i.
// v_permlane16_swap trades p-tiles between lanes q and q ^ 1, so every lane holds two
// 16-byte runs of consecutive p (its row's bytes [0, 64) and [64, 128) between the 4 lanes
// of the row).  A lane ^ 8 swizzle then hands the second run to the lane of row i ^ 8, and
// each 16-byte store writes 8 complete rows: whole lines, sent non-temporal.  (Four 32-byte
// pieces per row, even merged in L2, made every write a partial-line miss.)  sy: the byte
// offset of the tile's first row (uniform), XS: the row stride, hcol: the head's byte
// offset within a row.
__device__ __forceinline__ void store_tile16(const f32x4* a, brsrc ry, int sy, int XS, int hcol) {
    u32x2 yv[4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
        yv[pt] = __builtin_bit_cast(u32x2, bf16x4{(bf16)a[pt][0], (bf16)a[pt][1], (bf16)a[pt][2], (bf16)a[pt][3]});
    u32x4v lo, hi;  // 16-byte runs from p-tiles 0, 1 (row bytes 0..63) and 2, 3 (64..127)
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        const auto r01 = __builtin_amdgcn_permlane16_swap(yv[0][d], yv[1][d], false, false);
        const auto r23 = __builtin_amdgcn_permlane16_swap(yv[2][d], yv[3][d], false, false);
        lo[d] = r01[0]; lo[2 + d] = r01[1];
        hi[d] = r23[0]; hi[2 + d] = r23[1];
    }
    u32x4v hx;  // the other half-row of this lane's partner i ^ 8
#pragma unroll
    for (int d = 0; d < 4; ++d) hx[d] = (unsigned)__builtin_amdgcn_ds_swizzle((int)hi[d], 0x201F);
    const int ln = lane_now(), qq = ln >> 4, ii = ln & 15;
    const bool up = ii >= 8;
    // byte of the lane's run in its row: q = 0, 2 hold p 0..7, 8..15; q = 1, 3 hold 16..23, 24..31
    const int vrow = (ii & 7) * XS + hcol + (qq & 1) * 32 + (qq & 2) * 8;
    // The data registers of a 16-byte buffer store must not be rewritten by the next
    // instructions: the store then sends the new values (seen on gfx950 with an SGPR
    // offset, where no wait is inserted).  Each store is fenced off with s_nop.
    __builtin_amdgcn_raw_buffer_store_b128(up ? hx : lo, ry, vrow + (up ? 64 : 0), sy, 2);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 4");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_raw_buffer_store_b128(up ? lo : hx, ry, vrow + (up ? 0 : 64), sy + 8 * XS, 2);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 4");
    __builtin_amdgcn_sched_barrier(0);
}

// Element offset of state element (p, n) in a [P][N] bfloat16 LDS tile whose 16-byte chunks
// are XOR-swizzled by row, so that the 16 rows a matrix-core fragment reads hit distinct banks.
template <int N>
__device__ __forceinline__ int hs_off(int p, int n) {
    constexpr int HSW = (N / 8) < 16 ? (N / 8) : 16;
    return p * N + ((((n >> 3) ^ (p % HSW))) << 3) + (n & 7);
}

// A chunk's Q rows of a headdim-64 bfloat16 tensor (x, dy) and a [64][N] bfloat16 state tile
// (H_c, R_c) straight into LDS by direct transfers, wave w taking its quarter of each: the
// rows into Ts in xs_off's layout, the state into Hs in hs_off's.  srow0: byte offset of
// the chunk's first row in rrows (row stride XS, the head at byte hcol); sstate0: byte
// offset of the state tile in rstate.  The caller waits (vmcnt) and synchronises.
template <int Q, int N>
__device__ __forceinline__ void dma_rows_state(bf16* Ts, bf16* Hs, brsrc rrows, int srow0, int XS, int hcol,
                                               brsrc rstate, int sstate0, int w) {
    constexpr int XR = Q / 32, HR = N / 32, SRW = 512 / N, HSW = (N / 8) < 16 ? (N / 8) : 16;
    int ln = lane_now();  // rebuilt per call, not kept live
    const int vd0 = xs_dma_lane(ln, 0, XS, hcol), vd1 = xs_dma_lane(ln, 1, XS, hcol);
#pragma unroll
    for (int r = 0; r < XR; ++r) {
        const int m = w * XR + r;  // 1 KB transfer m: rows 8 m .. 8 m + 7
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rrows, (__attribute__((address_space(3))) void*)(Ts + m * 512), 16,
                                                 xs_dma_bit(m) ? vd1 : vd0,
                                                 __builtin_amdgcn_readfirstlane(srow0 + 8 * m * XS), 0, 0);
    }
    // state transfer m: rows p = m SRW + l / (N / 8); LDS slot l % (N / 8) holds n-chunk slot ^ (p % HSW)
#pragma unroll
    for (int r = 0; r < HR; ++r) {
        const int m = w * HR + r;
        const int pr = ln / (N / 8), slot = ln % (N / 8), p = m * SRW + pr;
        const int ch = slot ^ (p % HSW);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rstate, (__attribute__((address_space(3))) void*)(Hs + m * 512), 16,
                                                 (pr * N + ch * 8) * 2,
                                                 __builtin_amdgcn_readfirstlane(sstate0 + m * SRW * N * 2), 0, 0);
    }
}

// Element offsets of a chunk's x rows in LDS: the swizzled 64-element rows for bfloat16
// at headdim 64 (no bank conflicts in the transpose reads), else rows padded by 8.
template <typename T, int P, bool ALLOW = true>
struct XRows {
    static constexpr bool SWZ = ALLOW && sizeof(T) == 2 && P == 64;
    static constexpr int LD = SWZ ? 64 : P + 8;
    __device__ static int off(int j, int p) {
        if constexpr (SWZ) return xs_off(j, p);
        else return j * LD + p;
    }
};
template <typename T, int P, bool ALLOW = true>
__device__ __forceinline__ typename V8<T>::type frag_x(const T* Xs, int k0, int c0, int lane) {
    if constexpr (XRows<T, P, ALLOW>::SWZ) return frag_xs(Xs, k0, c0, lane);
    else return frag_rows(Xs, XRows<T, P, ALLOW>::LD, k0, c0, lane);
}
template <typename T, int P, bool ALLOW = true>
__device__ __forceinline__ typename V8<T>::type frag_x_split(const T* Xs, int ra, int rb, int c0, int lane) {
    if constexpr (XRows<T, P, ALLOW>::SWZ) return frag_xs_split(Xs, ra, rb, c0, lane);
    else return frag_rows_split(Xs, XRows<T, P, ALLOW>::LD, ra, rb, c0, lane);
}

// ---------------------------------------------------------------------------
// Wave tiling of a [N/16] x [P/16] grid of 16x16 output tiles over 4 waves: each
// wave owns WN x WP tiles starting at (n-tile n0, p-tile p0) (or none).
// ---------------------------------------------------------------------------
template <int P, int N>
struct StateTiling {
    static constexpr int NTN = N / 16, NTP = P / 16;
    static constexpr int WN = NTN >= 4 ? NTN / 4 : (NTP >= 4 ? NTN : 1);
    static constexpr int WP = NTN >= 4 ? NTP : (NTP >= 4 ? NTP / 4 : 1);
    __device__ static bool active(int w) { return NTN >= 4 || NTP >= 4 || w < NTN * NTP; }
    __device__ static int n0(int w) { return NTN >= 4 ? w * WN : (NTP >= 4 ? 0 : w / NTP); }
    __device__ static int p0(int w) { return NTN >= 4 ? 0 : (NTP >= 4 ? w * WP : w % NTP); }
};

// ---------------------------------------------------------------------------
// k_state: the chunk input projection decayed to the chunk end,
//   S_c[p][n] = sum_{j in chunk} x_j[p] * B_j[n] * exp(A (cdt_last - cdt_j))
// (A = A_h, or A_{h,n} for the diagonal decay).  One work-group per (b, h, c).
// The contraction runs over tokens j, the strided dimension of x and B in memory, so
// 64-token slabs of x and B are staged row-major in LDS (16-byte coalesced loads and
// stores) and read back as token-contiguous fragments with the LDS transpose read.
// The decay weight multiplies the smaller operand once per element while staging: x
// rows (one weight per token) for the scalar decay, B elements for the diagonal decay.
// The next slab's global loads are issued into registers before the current slab's
// matrix-core work.  Waves compute S^T tiles [n][p], so each lane stores 4
// consecutive n.
// ADJ = true weights token j by its decay from the chunk start instead,
// exp(A cdt_j): called with (dy, C) for (x, B) it gives the backward pass's adjoint
// chunk input sum_{i in chunk} exp(A cdt_i) dy_i C_i^T.
// ST is the type S_c is stored in: float32 for the backward; the forward stores it in the
// input type (each S_c is rounded once, and the scan that sums them accumulates in float32).
// ---------------------------------------------------------------------------
template <typename T, int P, int N, bool DIAG, bool ADJ = false, typename ST = float>
__global__ __launch_bounds__(kThreads) void k_state(const T* __restrict__ x, const T* __restrict__ Bm,
                                                    const float* __restrict__ A,
                                                    const float* __restrict__ cdt,
                                                    ST* __restrict__ S, int64_t Tn, int H, int G,
                                                    int Q, int nc) {
    typedef typename V8<T>::type v8;
    typedef StateTiling<P, N> TL;
    typedef XRows<T, P> XL;
    constexpr int JB = 64, LDX = XL::LD, LDB = N + 8;
    constexpr int XV = JB * P / 8, BV = JB * N / 8;                       // 8-element vectors per slab
    constexpr int XR = (XV + kThreads - 1) / kThreads, BR = (BV + kThreads - 1) / kThreads;
    __shared__ __attribute__((aligned(16))) T Xs[JB * LDX];
    __shared__ __attribute__((aligned(16))) T Bs[JB * LDB];
    __shared__ float cds[256];
    __shared__ float an2[DIAG ? N : 1];
    int c;
    const int64_t bh = chunk_item(H, nc, c);
    const int h = (int)(bh % H);
    const int64_t bi = bh / H;
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, q = lane >> 4;
    const int64_t tok0 = (int64_t)c * Q;
    const int len = (int)((Tn - tok0) < Q ? (Tn - tok0) : Q);
    const float* cd = cdt + (bh * nc + c) * (int64_t)Q;
    for (int i = tid; i < Q; i += kThreads) cds[i] = cd[i];
    if (DIAG)
        for (int n = tid; n < N; n += kThreads) an2[n] = A[h * N + n] * 1.4426950408889634f;
    const float ah2 = DIAG ? 0.f : A[h] * 1.4426950408889634f;
    const T* xb = x + ((bi * Tn + tok0) * H + h) * P;   // row j at xb + j * H * P
    const T* bb = Bm + ((bi * Tn + tok0) * G + g) * N;  // row j at bb + j * G * N

    v8 xv[XR], bv[BR];
    auto prefetch = [&](int j0) {
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
    };
    prefetch(0);
    __syncthreads();  // cds, an2
    const float last = cds[Q - 1];

    f32x4 acc[TL::WN][TL::WP];
#pragma unroll
    for (int a = 0; a < TL::WN; ++a)
#pragma unroll
        for (int b = 0; b < TL::WP; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bool wact = TL::active(w);
    const int wn0 = TL::n0(w), wp0 = TL::p0(w);

    for (int j0 = 0; j0 < len; j0 += JB) {
        // slab j0 -> LDS, decay weight applied once per element
#pragma unroll
        for (int r = 0; r < XR; ++r) {
            const int v = tid + r * kThreads;
            if (v < XV) {
                const int jj = v / (P / 8), p0 = (v - jj * (P / 8)) * 8;
                v8 o = xv[r];
                if (!DIAG) {
                    const float wj = exp2f_fast(ah2 * (ADJ ? cds[j0 + jj] : last - cds[j0 + jj]));
#pragma unroll
                    for (int e = 0; e < 8; ++e) o[e] = from_f<T>(to_f(o[e]) * wj);
                }
                st8(Xs + XL::off(jj, p0), o);
            }
        }
#pragma unroll
        for (int r = 0; r < BR; ++r) {
            const int v = tid + r * kThreads;
            if (v < BV) {
                const int jj = v / (N / 8), n0 = (v - jj * (N / 8)) * 8;
                v8 o = bv[r];
                if (DIAG) {
                    const float dc = ADJ ? cds[j0 + jj] : last - cds[j0 + jj];
#pragma unroll
                    for (int e = 0; e < 8; ++e) o[e] = from_f<T>(to_f(o[e]) * exp2f_fast(an2[n0 + e] * dc));
                }
                st8(&Bs[jj * LDB + n0], o);
            }
        }
        __syncthreads();
        if (j0 + JB < len) prefetch(j0 + JB);
        if (wact) {
#pragma unroll
            for (int kk = 0; kk < JB; kk += 32) {
                v8 bf[TL::WP];
#pragma unroll
                for (int b = 0; b < TL::WP; ++b) bf[b] = frag_x<T, P>(Xs, kk, (wp0 + b) * 16, lane);
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
    ST* out = S + (bh * nc + c) * (int64_t)(P * N);
    // Where the state tile fits the B slab's LDS (stored in 16-bit types, P <= 64), it is
    // staged there as rows and leaves in whole 16-byte row pieces; else each lane stores
    // its 4 consecutive n straight from the accumulators (16 rows per store).
    constexpr int LDS_ = N + 8;
    if constexpr (sizeof(ST) == 2 && (size_t)P * LDS_ * sizeof(ST) <= (size_t)JB * LDB * sizeof(T)) {
        ST* Ss = reinterpret_cast<ST*>(Bs);  // every wave is past its last read of Bs
        if (wact) {
#pragma unroll
            for (int a = 0; a < TL::WN; ++a)
#pragma unroll
                for (int b = 0; b < TL::WP; ++b) {
                    typename V4<ST>::type o;
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] = from_f<ST>(acc[a][b][r]);
                    st4(Ss + ((wp0 + b) * 16 + l16) * LDS_ + (wn0 + a) * 16 + 4 * q, o);
                }
        }
        __syncthreads();
        for (int v = tid; v < P * N / 8; v += kThreads) {
            const int p = v / (N / 8), n0 = (v - p * (N / 8)) * 8;
            st8(out + p * N + n0, ld8(Ss + p * LDS_ + n0));
        }
    } else if (wact) {
#pragma unroll
        for (int a = 0; a < TL::WN; ++a)
#pragma unroll
            for (int b = 0; b < TL::WP; ++b) {
                typename V4<ST>::type o;
#pragma unroll
                for (int r = 0; r < 4; ++r) o[r] = from_f<ST>(acc[a][b][r]);
                st4(out + ((wp0 + b) * 16 + l16) * N + (wn0 + a) * 16 + 4 * q, o);
            }
    }
}

// ---------------------------------------------------------------------------
// k_scan: the state carried across chunks, one recurrence step per chunk:
//   H_0 = h0;  hin[c] = H_c;  H_{c+1} = exp(A cdt_last(c)) H_c + S_c;  hT = H_nc
// (per n for the diagonal decay).  Sequential over chunks, parallel over
// b x H x P x N: each thread owns 4 consecutive (p, n) elements of one head and
// streams its chunk states with loads issued 8 chunks ahead.
// Grid (b*H*ceil(P*N/1024), segments).
//
// When b H P N is too small to fill the GPU, the chunks are cut into segments of L and
// the step, being linear (H -> a H + S composes associatively: (a2, S2) o (a1, S1) =
// (a2 a1, a2 S1 + S2)), runs as a parallel scan ("Semiseparable Matrix Transformations"
// keyword page, definition: parallel scans evaluate the same map) in three launches:
//   MODE 1  each segment from a zero state -> its end state E_s      (into `carry`),
//           and the sum of its chunks' cdt totals                     (into `segsum`)
//   k_scan_carry   in segment order: carry[s] <- H entering segment s
//   MODE 2  each segment again from carry[s]: hin, and hT from the last segment
// MODE 0 is the whole sequence in one segment (L = nc).  ST: the type the chunk states
// are stored in (k_state's); the carried state is float32 throughout.
// ---------------------------------------------------------------------------
template <typename T, bool DIAG, int MODE, typename ST = float>
__global__ __launch_bounds__(kThreads) void k_scan(const ST* __restrict__ S, T* __restrict__ hin,
                                                   float* __restrict__ hT, const float* __restrict__ h0,
                                                   const float* __restrict__ A,
                                                   const float* __restrict__ cdt, float* __restrict__ carry,
                                                   float* __restrict__ segsum, int H, int PN, int N, int Q,
                                                   int nc, int per_head, int L, int64_t BHPN) {
    typedef typename V4<T>::type v4;
    const int64_t bh = blockIdx.x / per_head;
    const int part = (int)(blockIdx.x - bh * per_head);
    const int h = (int)(bh % H);
    const int e0 = (part * kThreads + threadIdx.x) * 4;
    if (e0 >= PN) return;
    const int seg = blockIdx.y;
    const int cb = seg * L, ce = min(nc, cb + L);
    const int n0 = e0 % N;
    float a4[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) a4[k] = DIAG ? A[h * N + n0 + k] : A[h];
    f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
    if (MODE == 2) st = ld4(carry + seg * BHPN + bh * PN + e0);
    else if (MODE == 0 && h0) st = ld4(h0 + bh * PN + e0);
    const float* cl = cdt + bh * (int64_t)nc * Q + (Q - 1);
    const ST* sp = S + bh * (int64_t)nc * PN + e0;
    T* hp = hin + bh * (int64_t)nc * PN + e0;
    constexpr int DEPTH = 8;
    float lsum = 0.f;  // the segment's log-decay per unit A (MODE 1)
    for (int c0 = cb; c0 < ce; c0 += DEPTH) {
        typename V4<ST>::type s[DEPTH];
        float Lc[DEPTH];
#pragma unroll
        for (int k = 0; k < DEPTH; ++k) {
            if (c0 + k < ce) {
                s[k] = ld4(sp + (int64_t)(c0 + k) * PN);
                Lc[k] = cl[(int64_t)(c0 + k) * Q];
            }
        }
#pragma unroll
        for (int k = 0; k < DEPTH; ++k) {
            if (c0 + k < ce) {
                if (MODE != 1) {
                    v4 o;
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] = from_f<T>(st[r]);
                    st4(hp + (int64_t)(c0 + k) * PN, o);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) st[r] = exp_f(a4[r] * Lc[k]) * st[r] + to_f(s[k][r]);
                if (MODE == 1) lsum += Lc[k];
            }
        }
    }
    if (MODE == 1) {
        st4(carry + seg * BHPN + bh * PN + e0, st);
        if (e0 == 0) segsum[bh * gridDim.y + seg] = lsum;
    }
    else if (hT && ce == nc) st4(hT + bh * PN + e0, st);
}

// The segments in order: carry[s] holds segment s's end state from a zero start and is
// replaced by the state entering it; the segment's decay is exp(A * segsum[s]).
template <bool DIAG>
__global__ __launch_bounds__(kThreads) void k_scan_carry(const float* __restrict__ h0, const float* __restrict__ A,
                                                         const float* __restrict__ segsum, float* __restrict__ carry,
                                                         int H, int PN, int N, int per_head, int nseg, int64_t BHPN) {
    const int64_t bh = blockIdx.x / per_head;
    const int part = (int)(blockIdx.x - bh * per_head);
    const int h = (int)(bh % H);
    const int e0 = (part * kThreads + threadIdx.x) * 4;
    if (e0 >= PN) return;
    const int n0 = e0 % N;
    float a4[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) a4[k] = DIAG ? A[h * N + n0 + k] : A[h];
    f32x4 st = h0 ? ld4(h0 + bh * PN + e0) : f32x4{0.f, 0.f, 0.f, 0.f};
    for (int sg = 0; sg < nseg; ++sg) {
        float* cp = carry + sg * BHPN + bh * PN + e0;
        const f32x4 e = ld4(cp);
        const float ls = segsum[bh * nseg + sg];
        st4(cp, st);
#pragma unroll
        for (int r = 0; r < 4; ++r) st[r] = exp_f(a4[r] * ls) * st[r] + e[r];
    }
}

// ---------------------------------------------------------------------------
// k_out: output of one (b, h, c) chunk,
//   y_i = sum_{j<=i} cb[i][j] exp(A (cdt_i - cdt_j)) x_j        (diagonal block)
//       + exp(A cdt_i) * sum_n C_i[n] H_c[p][n]                   (off-diagonal blocks)
//       + D_h x_i
// Waves compute y^T tiles [p][i] (x^T from the LDS transpose read as A operand, the
// masked block row as B operand), so a lane ends up with 4 consecutive p of one row.
// Scalar decay:
//  * the state term uses raw C and H fragments; its per-row factor exp(A cdt_i)
//    scales the accumulator afterwards;
//  * on the block's 32-token k-steps strictly before the row tile, the mask factors
//    as exp(A (cdt_i - cdt_r)) exp(A (cdt_r - cdt_j)) with r the last token of the
//    k-step, both <= 1: one exp per lane and k-step, the second factor from LDS;
//  * the k-step holding the row tile takes direct exps, the causal cut and D_h on
//    the diagonal (D x_i rides along in the same product).
// Diagonal decay: the per-head block G_ij = sum_n C_in B_jn exp(A_n(cdt_i-cdt_j)) is
// formed on the matrix cores from rescaled operands for every 16 x 16 sub-block pair
// (I >= J): C~_i = C_i exp(A (cdt_i - cdt_sI)), B~_j = B_j exp(A (cdt_eJ - cdt_j)),
// times exp(A (cdt_sI - cdt_eJ)) per n (sI first row of I, eJ last row of J); the three
// factors are <= 1 off the diagonal.  A diagonal sub-block whose decay span is too
// wide for that split (|A| span > 80) is summed directly with per-term exps.
// Each wave owns Q/64 row tiles of 16 rows, paired (k, 7-k) within every 128 rows so
// the causal work is balanced.  y is staged through LDS (aliasing x) for row stores.
// ---------------------------------------------------------------------------
// SWZR (diagonal decay): the x rows and the rescaled C / B rows in swizzled unpadded
// layouts (a smaller tile, chosen where it fits one more work-group per CU) instead of
// rows padded by 8.
template <typename T, int P, int N, bool DIAG, bool TAB = false, bool SWZR = false>
struct OutSmem {
    static constexpr bool RESCALED = DIAG && !TAB;  // rescaled C / B rows in LDS
    static constexpr bool XSWZ = !RESCALED || SWZR;   // x rows swizzled where XRows allows
    static constexpr int LDX = XRows<T, P, XSWZ>::LD;  // x (then y) rows
    // rescaled C / B rows: with SWZR and a 16-bit type unpadded, their 16-byte chunks
    // XOR-swizzled by row (rc_off); else padded by 8
    static constexpr bool RSWZ = SWZR && sizeof(T) == 2;
    static constexpr int LDN = RSWZ ? N : N + 8;
    // element offset of (row r, column n) of a rescaled C / B tile, n a multiple of 8 plus
    // e < 8: the 16 rows a fragment reads land in distinct banks
    __device__ static int rc_off(int r, int n) {
        if constexpr (RSWZ) {
            constexpr int RPB = (128 / N) > 1 ? 128 / N : 1;       // rows per 64-bank cycle
            constexpr int NCH = (N / 8) < 16 ? N / 8 : 16;         // chunks the swizzle spans
            return r * N + ((((n >> 3) ^ ((r / RPB) & (NCH - 1)))) << 3) + (n & 7);
        } else {
            return r * LDN + n;
        }
    }
    __host__ __device__ static int xs(int Q) { return Q * LDX; }
    __host__ __device__ static int diag_elems(int Q) { return RESCALED ? 2 * Q * LDN : 0; }
    __host__ __device__ static int floats(int Q) { return 2 * Q + (RESCALED ? N : 0); }
    __host__ __device__ static size_t bytes(int Q) {
        return (size_t)(xs(Q) + diag_elems(Q)) * sizeof(T) + (size_t)floats(Q) * sizeof(float);
    }
};

// Work-groups per CU the output kernel is compiled for: three for bfloat16 up to headdim 64
// (its registers then fit 168 per lane without spills; two per CU left latency exposed:
// 371 -> 327 us at the 2.7B layer's split schedule), else what its tile needs.
template <typename T, int P>
constexpr int out_min_blocks() { return (sizeof(T) == 2 && P <= 64) ? 3 : 1; }

template <typename T, int P, int N, bool DIAG, bool TAB = false, bool SWZR = false>
__global__ __launch_bounds__(kThreads, (out_min_blocks<T, P>())) void k_out(const T* __restrict__ x, const T* __restrict__ Bm,
                                                  const T* __restrict__ Cm, const T* __restrict__ cb,
                                                  const T* __restrict__ hin, const float* __restrict__ A,
                                                  const float* __restrict__ D,
                                                  const float* __restrict__ cdt, T* __restrict__ y,
                                                  int64_t Tn, int H, int G, int Q, int nc) {
    typedef typename V8<T>::type v8;
    typedef typename V4<T>::type v4;
    typedef OutSmem<T, P, N, DIAG, TAB, SWZR> SM;
    typedef XRows<T, P, SM::XSWZ> XL;
    constexpr bool SCAL = !DIAG || TAB;  // diagonal block from a table of query-key products
    constexpr int LDN = SM::LDN;
    constexpr int PT = P / 16;
    constexpr float LOG2E = 1.4426950408889634f;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    T* Xs = reinterpret_cast<T*>(smem_raw);
    T* Ys = Xs;
    T* Ct = Xs + SM::xs(Q);
    T* Bt = Ct + (DIAG ? Q * LDN : 0);
    float* cds = reinterpret_cast<float*>(Xs + SM::xs(Q) + SM::diag_elems(Q));
    float* u2 = cds + Q;       // scalar: exp(A (cdt_r(j) - cdt_j)), r(j) = j | 31
    float* an2 = u2 + Q;       // diagonal: A_n log2(e)

    int c;
    const int64_t bh = chunk_item(H, nc, c);
    const int h = (int)(bh % H);
    const int64_t bi = bh / H;
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, q = lane >> 4;
    const int64_t tok0 = (int64_t)c * Q;
    const int len = (int)((Tn - tok0) < Q ? (Tn - tok0) : Q);
    const int rpw = Q / 64;  // row tiles per wave
    const T* xb = x + ((bi * Tn + tok0) * H + h) * P;   // row j at xb + j * H * P
    const T* cbase_rows = Cm + ((bi * Tn + tok0) * G + g) * N;  // row i at + i * G * N
    const T* hbase = hin + (bh * nc + c) * (int64_t)(P * N);
    const float* cd = cdt + (bh * nc + c) * (int64_t)Q;
    const float ah2 = DIAG ? 0.f : A[h] * LOG2E;
    const float Dh = D ? D[h] : 0.f;

    auto row_tile = [&](int k) { return (rpw == 1) ? w : ((k & 1) ? 8 * (k >> 1) + 7 - w : 8 * (k >> 1) + w); };

    // 1. x rows of the chunk, loaded and stored to LDS before the state term
    constexpr int XR = (256 * P / 8 + kThreads - 1) / kThreads;  // enough for Q = 256
    const int XV = Q * P / 8;
    v8 xv[XR];
#pragma unroll
    for (int r = 0; r < XR; ++r) {
        const int v = tid + r * kThreads;
        const int jj = v / (P / 8), p0 = (v - jj * (P / 8)) * 8;
        const int jr = jj < len ? jj : len - 1;
        xv[r] = sel8(v < XV && jj < len, ld8(xb + (int64_t)jr * H * P + p0));
    }
    float cdv = 0.f;
    if (tid < Q) cdv = cd[tid];
    // x rows to LDS now, so their registers are free during the state term
#pragma unroll
    for (int r = 0; r < XR; ++r) {
        const int v = tid + r * kThreads;
        if (v < XV) {
            const int jj = v / (P / 8), p0 = (v - jj * (P / 8)) * 8;
            st8(Xs + XL::off(jj, p0), xv[r]);
        }
    }

    f32x4 acc[4][PT];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[k][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // C B^T fragments of a row tile, requested just before its own k-steps (a second set
    // in flight ahead of use costs the registers of a third work-group per CU)
    // scalar decay: the group's C B^T table; diagonal decay (TAB): this head's table of
    // decay-weighted products, D on its diagonal
    const T* cbb_pf = cb + (TAB ? bh * nc + c : (bi * nc + c) * G + g) * (int64_t)Q * Q;
    auto load_gf = [&](int k, v8* gf) {
        const int rt = row_tile(k);
        const int nks = rt / 2 + 1;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) gf[ks] = ld8(cbb_pf + tfrag(rt * 16 + l16, (ks < nks ? ks : nks - 1) * 32 + 8 * q, Q));
    };
    v8 gfa[8];

    // 2. state term y^T[p][i] += sum_n H[p][n] C[i][n] from raw fragments (scalar decay:
    //    the row factor exp(A cdt_i) follows in step 4); diagonal decay with a table:
    //    each C element scaled by its own exp(A_n cdt_i) <= 1
    if (SCAL) {
        float crow[4];
        if (TAB)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = row_tile(k) * 16 + l16;
                crow[k] = cd[k < rpw && i < len ? i : 0];
            }
#pragma unroll
        for (int n0 = 0; n0 < N; n0 += 32) {
            const int nn = n0 + 8 * q;
            const bool nv = (N % 32 == 0) || (nn < N);  // N = 16: half the k-step is padding
            v8 hf[PT], cf[4];
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) hf[pt] = sel8(nv, ld8(hbase + (pt * 16 + l16) * N + (nv ? nn : 0)));
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = row_tile(k) * 16 + l16;
                const int ir = i < len ? i : len - 1;
                cf[k] = sel8(k < rpw && nv && i < len, ld8(cbase_rows + (int64_t)ir * G * N + (nv ? nn : 0)));
            }
            if (TAB) {
                const f32x8 an = ld8(A + (int64_t)h * N + (nv ? nn : 0));
#pragma unroll
                for (int k = 0; k < 4; ++k)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        cf[k][e] = from_f<T>(to_f(cf[k][e]) * exp2f_fast(an[e] * LOG2E * crow[k]));
            }
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (k < rpw)
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) acc[k][pt] = mma(acc[k][pt], hf[pt], cf[k]);
        }
    }

    // 3. chunk decay tables
    if (tid < Q) cds[tid] = cdv;
    if (SM::RESCALED)
        for (int n = tid; n < N; n += kThreads) an2[n] = A[h * N + n] * LOG2E;
    __syncthreads();
    if (!DIAG && tid < Q) u2[tid] = exp2f_fast(ah2 * (cds[tid | 31] - cds[tid]));
    if (SM::RESCALED) {
        // rescaled rows: Ct[i][n] = C_i[n] e^{A_n (cdt_i - cdt_sI)}, Bt[j][n] = B_j[n] e^{A_n (cdt_eJ - cdt_j)}
        const T* bbase_rows = Bm + ((bi * Tn + tok0) * G + g) * N;
        for (int v = tid; v < Q * N / 8; v += kThreads) {
            const int ii = v / (N / 8), n0 = (v - ii * (N / 8)) * 8;
            v8 cv = zero8<T>(), bv = zero8<T>();
            if (ii < len) {
                const v8 cr = ld8(cbase_rows + (int64_t)ii * G * N + n0);
                const v8 br = ld8(bbase_rows + (int64_t)ii * G * N + n0);
                const float dcs = cds[ii] - cds[ii & ~15];
                const float dce = cds[ii | 15] - cds[ii];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    cv[e] = from_f<T>(to_f(cr[e]) * exp2f_fast(an2[n0 + e] * dcs));
                    bv[e] = from_f<T>(to_f(br[e]) * exp2f_fast(an2[n0 + e] * dce));
                }
            }
            st8(&Ct[SM::rc_off(ii, n0)], cv);
            st8(&Bt[SM::rc_off(ii, n0)], bv);
        }
    }
    __syncthreads();

    if (SCAL) {
        // 4. per-row factor of the state term: this lane's column is row i
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (!TAB && k < rpw) {
                const float sc = exp2f_fast(ah2 * cds[row_tile(k) * 16 + l16]);
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) acc[k][pt] *= sc;
            }
        // 5. diagonal block
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (k < rpw) {
                const int rt = row_tile(k);
                const int i = rt * 16 + l16;
                const int nks = rt / 2 + 1;  // k-steps of 32 tokens up to this row tile
                v8* gf = gfa;
                load_gf(k, gfa);
                const float ci = cds[i];
#pragma unroll
                for (int ks = 0; ks < 8; ++ks) {
                    if (ks < nks) {
                        const int j0 = ks * 32 + 8 * q;
                        v8 mf;
                        if (TAB) {
                            mf = gf[ks];  // decay, causal zeros and D are in the table
                        } else if (ks < nks - 1) {
                            const float vi = exp2f_fast(ah2 * (ci - cds[ks * 32 + 31]));
#pragma unroll
                            for (int e = 0; e < 8; ++e) mf[e] = from_f<T>(to_f(gf[ks][e]) * (u2[j0 + e] * vi));
                        } else {
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                const int j = j0 + e;
                                // exponent clamped to <= 0 so the (j > i) slots stay finite: the
                                // table holds exact zeros there, so they need no causal cut
                                const float m = to_f(gf[ks][e]) * exp2f_fast(fminf(ah2 * (ci - cds[j]), 0.f));
                                mf[e] = from_f<T>(m + ((j == i) ? Dh : 0.f));
                            }
                        }
#pragma unroll
                        for (int pt = 0; pt < PT; ++pt) {
                            const v8 xf = frag_x<T, P, SM::XSWZ>(Xs, ks * 32, pt * 16, lane);
                            acc[k][pt] = mma(acc[k][pt], xf, mf);
                        }
                    }
                }
            }
        }
    } else {
        float amax = 0.f;  // widest per-n decay rate, for the diagonal sub-block split
        for (int n = 0; n < N; ++n) amax = fmaxf(amax, -an2[n]);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (k < rpw) {
                const int rt = row_tile(k);
                const int sI = rt * 16;
                const int i = sI + l16;
                for (int u = 0; 2 * u <= rt; ++u) {
                    f32x4 gt[2];
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
                        gt[s2] = f32x4{0.f, 0.f, 0.f, 0.f};
                        const int J = 2 * u + s2;
                        if (J > rt) continue;
                        const int eJ = J * 16 + 15;
                        const bool direct = (J == rt) && !(amax * (cds[eJ] - cds[sI]) <= 80.f * LOG2E);
                        if (!direct) {
                            // gt = B~_J diag(m) C~_I^T: lane holds G^T[j = 16J + 4q + r][i = sI + l16]
                            const float dm = cds[sI] - cds[eJ];
#pragma unroll
                            for (int n0 = 0; n0 < N; n0 += 32) {
                                const int nn = n0 + 8 * q;
                                const bool nv = (N % 32 == 0) || (nn < N);
                                v8 a = zero8<T>(), b = zero8<T>();
                                if (nv) {
                                    a = ld8(&Bt[SM::rc_off(J * 16 + l16, nn)]);
#pragma unroll
                                    for (int e = 0; e < 8; ++e)
                                        a[e] = from_f<T>(to_f(a[e]) * exp2f_fast(an2[nn + e] * dm));
                                    b = ld8(&Ct[SM::rc_off(sI + l16, nn)]);
                                }
                                gt[s2] = mma(gt[s2], a, b);
                            }
                        } else {
                            // direct sums for this lane's 4 entries (i, j = sI + 4q + r)
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const int jj = sI + 4 * q + r;
                                float sum = 0.f;
                                if (jj <= i && i < len) {
                                    const T* cr = cbase_rows + (int64_t)i * G * N;
                                    const T* br = Bm + ((bi * Tn + tok0 + jj) * G + g) * N;
                                    const float dd = cds[i] - cds[jj];
                                    for (int n = 0; n < N; ++n)
                                        sum += to_f(cr[n]) * to_f(br[n]) * exp2f_fast(an2[n] * dd);
                                }
                                gt[s2][r] = sum;
                            }
                        }
                        if (J == rt) {
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                if (4 * q + r > l16) gt[s2][r] = 0.f;       // causal: j <= i
                                else if (4 * q + r == l16) gt[s2][r] += Dh;  // skip term on the diagonal
                            }
                        }
                    }
                    // B operand: column i = l16, k = (s2, 4q + r) -> token j = 32u + 16 s2 + 4q + r
                    v8 mf;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        mf[r] = from_f<T>(gt[0][r]);
                        mf[4 + r] = from_f<T>(gt[1][r]);
                    }
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) {
                        const v8 xf = frag_x_split<T, P, SM::XSWZ>(Xs, 32 * u + 4 * q, 32 * u + 16 + 4 * q, pt * 16, lane);
                        acc[k][pt] = mma(acc[k][pt], xf, mf);
                    }
                }
                // state term: y^T[p][i] += sum_n H[p][n] C[i][n] e^{A_n cdt_i}, with
                // C[i][n] e^{A_n cdt_i} = C~[i][n] e^{A_n cdt_sI}
                const float csI = cds[sI];
#pragma unroll
                for (int n0 = 0; n0 < N; n0 += 32) {
                    const int nn = n0 + 8 * q;
                    const bool nv = (N % 32 == 0) || (nn < N);
                    v8 cf = zero8<T>();
                    if (nv) {
                        cf = ld8(&Ct[SM::rc_off(i, nn)]);
#pragma unroll
                        for (int e = 0; e < 8; ++e) cf[e] = from_f<T>(to_f(cf[e]) * exp2f_fast(an2[nn + e] * csI));
                    }
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) {
                        const v8 hf = nv ? ld8(hbase + (pt * 16 + l16) * N + nn) : zero8<T>();
                        acc[k][pt] = mma(acc[k][pt], hf, cf);
                    }
                }
            }
        }
    }

    // 6. y^T tiles -> LDS rows (4 consecutive p per lane), then 16-byte row stores
    __syncthreads();  // every wave is done reading Xs
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (k < rpw) {
            const int i = row_tile(k) * 16 + l16;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                v4 o;
#pragma unroll
                for (int r = 0; r < 4; ++r) o[r] = from_f<T>(acc[k][pt][r]);
                st4(Ys + XL::off(i, pt * 16 + 4 * q), o);
            }
        }
    }
    __syncthreads();
    for (int v = tid; v < len * (P / 8); v += kThreads) {
        const int ii = v / (P / 8), p0 = (v - ii * (P / 8)) * 8;
        st8(y + ((bi * Tn + tok0 + ii) * H + h) * P + p0, ld8(Ys + XL::off(ii, p0)));
    }
}

// ---------------------------------------------------------------------------
// k_outs: k_out for the scalar decay at bfloat16 and headdim 64 (dstate 64, 128 or 256),
// laid out like the fused kernel's output passes: the chunk's x rows and its entering state
// H_c go straight into swizzled LDS tiles by direct transfers (no register holds them in
// flight), each wave takes its row tiles one at a time -- state term from the LDS state
// tile and the tile's C rows, decay-masked C B^T fragments from the group's table times x
// fragments, D x_i riding in the diagonal k-step -- and y leaves in whole rows.  Three
// work-groups per CU up to dstate 128 (two at 256, whose state tile is 32 KB).
// ---------------------------------------------------------------------------
template <int Q, int N>
__global__ __launch_bounds__(kThreads, N <= 128 ? 3 : 2) void k_outs(const bf16* __restrict__ x,
                                                                 const bf16* __restrict__ Cm,
                                                                 const bf16* __restrict__ cb,
                                                                 const bf16* __restrict__ hin,
                                                                 const float* __restrict__ A,
                                                                 const float* __restrict__ D,
                                                                 const float* __restrict__ cdt,
                                                                 bf16* __restrict__ y, int64_t Tn, int H, int G,
                                                                 int nc) {
    constexpr int P = 64, RPW = Q / 64, KS = Q / 32, NF = N / 32, PN = P * N;
    constexpr float LOG2E = 1.4426950408889634f;
    __shared__ __attribute__((aligned(16))) bf16 Ts[Q * P];  // x rows (swizzled)
    __shared__ __attribute__((aligned(16))) bf16 Hs[P * N];  // H_c (chunks swizzled by row)
    __shared__ float cds[Q], u2[Q];

    int c;
    const int64_t bh = chunk_item(H, nc, c);
    const int h = (int)(bh % H);
    const int64_t bi = bh / H;
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), l16 = lane & 15, q = lane >> 4;
    const float ah2 = A[h] * LOG2E;
    const float Dh = D ? D[h] : 0.f;

    // buffer resources based at this batch row (rows past T read as zero, stores dropped),
    // the group's table and this chain's entering states
    const int XS = H * P * 2, CS = G * N * 2;
    const uint32_t xbytes = (uint32_t)(Tn * H * P * 2);
    const brsrc rx = make_rsrc(x + bi * Tn * H * P, xbytes);
    const brsrc ry = make_rsrc(y + bi * Tn * H * P, xbytes);
    const brsrc rc = make_rsrc(Cm + bi * Tn * G * N, (uint32_t)(Tn * G * N * 2));
    const brsrc rcb = make_rsrc(cb + bi * nc * G * Q * Q, (uint32_t)((int64_t)nc * G * Q * Q * 2));
    const brsrc rh = make_rsrc(hin + bh * nc * PN, (uint32_t)((int64_t)nc * PN * 2));
    const int hcol = h * P * 2;
    const int tab0 = (c * G + g) * Q * Q * 2;
    const int vc = l16 * CS + 8 * q * 2;

    dma_rows_state<Q, N>(Ts, Hs, rx, c * Q * XS, XS, hcol, rh, c * PN * 2, w);
    if (tid < Q) {
        const float* cd = cdt + (bh * nc + c) * (int64_t)Q;
        const float cv = cd[tid], cr = cd[tid | 31];
        cds[tid] = cv;
        u2[tid] = exp2f_fast(ah2 * (cr - cv));  // exp(A (cdt_{j|31} - cdt_j))
    }
    __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): this wave's transfers have landed
    __syncthreads();                    // ... every wave's, and the tables are in place

#pragma unroll
    for (int k = 0; k < RPW; ++k) {
        const int rt = (RPW == 1) ? w : ((k & 1) ? 8 * (k >> 1) + 7 - w : 8 * (k >> 1) + w);
        const int i = rt * 16 + l16, nks = rt / 2 + 1;
        bf16x8 gf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            if (ks < nks) gf[ks] = bload8(rcb, lane * 16, __builtin_amdgcn_readfirstlane(tab0 + (rt * (Q / 32) + ks) * 1024));
        // state term y^T[p][i] = exp(A cdt_i) sum_n H_c[p][n] C_i[n]
        bf16x8 cf[NF];
        const int sc0 = __builtin_amdgcn_readfirstlane((c * Q + rt * 16) * CS + g * N * 2);
#pragma unroll
        for (int n = 0; n < NF; ++n) cf[n] = bload8(rc, vc, sc0 + n * 64);
        f32x4 acc[4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int n = 0; n < NF; ++n)
#pragma unroll
            for (int pt = 0; pt < 4; ++pt)
                acc[pt] = mma(acc[pt], ld8(Hs + hs_off<N>(pt * 16 + l16, n * 32 + 8 * q)), cf[n]);
        const float ci = cds[i];
        const float sc = exp2f_fast(ah2 * ci);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc[pt] *= sc;
        // diagonal block: below the row tile's k-step the decay factors as u2_j v_i (both
        // <= 1); on it, direct exps with D on the diagonal (the table is zero above it)
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
                        mf[e] = (bf16)(m + ((j == i) ? Dh : 0.f));
                    }
                }
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) acc[pt] = mma(acc[pt], frag_xs(Ts, ks * 32, pt * 16, lane), mf);
                __builtin_amdgcn_sched_barrier(0);  // (hoisting every k-step's reads spills)
            }
        }
        store_tile16(acc, ry, __builtin_amdgcn_readfirstlane((c * Q + rt * 16) * XS), XS, hcol);
        __builtin_amdgcn_sched_barrier(0);  // one row tile's operands in flight at a time
    }
}

// ---------------------------------------------------------------------------
// k_gtab: the diagonal decay's query-key block of one (b, h, c), as a table for k_out
// when a chunk's rescaled C and B rows do not fit LDS next to its x rows:
//   tab[i][j] = sum_n C_i[n] B_j[n] exp(A_n (cdt_i - cdt_j)) for j < i,
//   tab[i][i] = the same + D_h,  tab[i][j] = 0 for j > i within the 64 x 64 blocks on the
//   diagonal (every entry of those blocks is written: the output kernel reads them)
// ("Structured State Space Duality" concept page, "What the duality gives up": each state
// dimension decays at its own rate, so the block is a sum of N scalar-decay masked
// products).  One work-group per (b, h, c) and 64 x 64 block pair (I >= J): the block
// pair's C rows and B rows are staged in LDS rescaled within their 16-row sub-blocks,
// C~_i = C_i exp(A (cdt_i - cdt_sI)), B~_j = B_j exp(A (cdt_eJ - cdt_j)) (sI first row of
// i's sub-block, eJ last row of j's), and each 16 x 16 sub-block pair is
// B~_J diag(exp(A (cdt_sI - cdt_eJ))) C~_I^T on the matrix cores (all three factors <= 1
// off the diagonal sub-blocks).  A diagonal sub-block whose decay span exceeds 2^115 is
// summed directly with per-term exponentials.  Wave w owns sub-block row w of the pair.
// Grid (b H nc, nb (nb + 1) / 2), nb = Q / 64; dynamic LDS gtab_smem<T, N>().
// ---------------------------------------------------------------------------
template <typename T, int N>
constexpr size_t gtab_smem() { return (size_t)2 * 64 * (N + 8) * sizeof(T) + (size_t)(128 + N) * sizeof(float); }

template <typename T, int N>
__global__ __launch_bounds__(kThreads) void k_gtab(const T* __restrict__ Bm, const T* __restrict__ Cm,
                                                   const float* __restrict__ A, const float* __restrict__ D,
                                                   const float* __restrict__ cdt, T* __restrict__ tab,
                                                   int64_t Tn, int H, int G, int Q, int nc) {
    typedef typename V8<T>::type v8;
    typedef typename V4<T>::type v4;
    constexpr int LDN = N + 8;
    constexpr float LOG2E = 1.4426950408889634f;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    T* Cs = reinterpret_cast<T*>(smem_raw);          // 64 rescaled C rows of block I
    T* Bs = Cs + 64 * LDN;                           // 64 rescaled B rows of block J
    float* ci = reinterpret_cast<float*>(Bs + 64 * LDN);  // cdt of block I's rows
    float* cj = ci + 64;                             // cdt of block J's rows
    float* an2 = cj + 64;                            // A_n log2(e)

    int c;
    const int64_t bh = chunk_item(H, nc, c);
    const int h = (int)(bh % H);
    const int64_t bi = bh / H;
    const int g = h / (H / G);
    int I = 0;
    while ((I + 1) * (I + 2) / 2 <= (int)blockIdx.y) ++I;
    const int J = (int)blockIdx.y - I * (I + 1) / 2;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, q = lane >> 4;
    const int64_t tok0 = (int64_t)c * Q;
    const int len = (int)((Tn - tok0) < Q ? (Tn - tok0) : Q);
    const float* cd = cdt + (bh * nc + c) * (int64_t)Q;
    const T* crows = Cm + ((bi * Tn + tok0) * G + g) * N;  // chunk row r at + r * G * N
    const T* brows = Bm + ((bi * Tn + tok0) * G + g) * N;
    for (int n = tid; n < N; n += kThreads) an2[n] = A[(int64_t)h * N + n] * LOG2E;
    if (tid < 64) ci[tid] = cd[I * 64 + tid];
    else if (tid < 128) cj[tid - 64] = cd[J * 64 + tid - 64];
    __syncthreads();
    for (int v = tid; v < 64 * N / 8; v += kThreads) {
        const int r = v / (N / 8), n0 = (v - r * (N / 8)) * 8;
        v8 cv = zero8<T>(), bv = zero8<T>();
        if (I * 64 + r < len) {
            const v8 cr = ld8(crows + (int64_t)(I * 64 + r) * G * N + n0);
            const float dc = ci[r] - ci[r & ~15];
#pragma unroll
            for (int e = 0; e < 8; ++e) cv[e] = from_f<T>(to_f(cr[e]) * exp2f_fast(an2[n0 + e] * dc));
        }
        if (J * 64 + r < len) {
            const v8 br = ld8(brows + (int64_t)(J * 64 + r) * G * N + n0);
            const float db = cj[r | 15] - cj[r];
#pragma unroll
            for (int e = 0; e < 8; ++e) bv[e] = from_f<T>(to_f(br[e]) * exp2f_fast(an2[n0 + e] * db));
        }
        st8(&Cs[r * LDN + n0], cv);
        st8(&Bs[r * LDN + n0], bv);
    }
    __syncthreads();
    float amax = 0.f;  // widest per-n decay rate, for the diagonal sub-block split
    for (int n = 0; n < N; ++n) amax = fmaxf(amax, -an2[n]);
    const float Dh = D ? D[h] : 0.f;
    T* out = tab + (bh * nc + c) * (int64_t)Q * Q;
    const int sI = 16 * w;  // this wave's sub-block row (local rows sI .. sI + 15 of block I)
    const int i = I * 64 + sI + l16;
    for (int J16 = 0; J16 < 4; ++J16) {
        const bool on_diag = I == J && J16 == w;
        if (I == J && J16 > w) {  // above the diagonal: zeros (the output kernel reads them)
            st4(out + tfrag(i, J * 64 + 16 * J16 + 4 * q, Q), v4{});
            continue;
        }
        const int eJ = 16 * J16 + 15;
        f32x4 gt = f32x4{0.f, 0.f, 0.f, 0.f};  // lane: G^T[j = 16 J16 + 4q + r][i = sI + l16]
        if (!on_diag || amax * (cj[eJ] - ci[sI]) <= 80.f * LOG2E) {
            const float dm = ci[sI] - cj[eJ];
#pragma unroll
            for (int n0 = 0; n0 < N; n0 += 32) {
                const int nn = n0 + 8 * q;
                const bool nv = (N % 32 == 0) || (nn < N);
                v8 a = zero8<T>(), b = zero8<T>();
                if (nv) {
                    a = ld8(&Bs[(16 * J16 + l16) * LDN + nn]);
#pragma unroll
                    for (int e = 0; e < 8; ++e) a[e] = from_f<T>(to_f(a[e]) * exp2f_fast(an2[nn + e] * dm));
                    b = ld8(&Cs[(sI + l16) * LDN + nn]);
                }
                gt = mma(gt, a, b);
            }
        } else {
            // direct sums for this lane's 4 entries (i, j = J 64 + 16 J16 + 4q + r)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int jl = 16 * J16 + 4 * q + r, j = J * 64 + jl;
                float sum = 0.f;
                if (j <= i && i < len) {
                    const T* cr = crows + (int64_t)i * G * N;
                    const T* br = brows + (int64_t)j * G * N;
                    const float dd = ci[sI + l16] - cj[jl];
                    for (int n = 0; n < N; ++n) sum += to_f(cr[n]) * to_f(br[n]) * exp2f_fast(an2[n] * dd);
                }
                gt[r] = sum;
            }
        }
        v4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = J * 64 + 16 * J16 + 4 * q + r;
            float m = gt[r];
            if (on_diag) m = (j > i) ? 0.f : (j == i ? m + Dh : m);
            v[r] = from_f<T>(m);
        }
        st4(out + tfrag(i, J * 64 + 16 * J16 + 4 * q, Q), v);
    }
}

}  // namespace ssd
