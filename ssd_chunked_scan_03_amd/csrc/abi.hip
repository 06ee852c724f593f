// abi.hip -- the C ABI of libssd.so (declared in include/ssd.h): host-side
// validation, workspace layout and launch sequencing.  No allocation; every check
// happens before the first HIP call.  The only global state is the per-device address
// of the no-allocation forward's scratch array, looked up once per device.
#include <string.h>

#include "bwd_launch.hpp"
#include "launch.hpp"
#include "step.hpp"
#include "ssd.h"

#include <mutex>

// Workspace of ssd_scan_fwd_noalloc: one copy of this array per GPU, in the library's
// device code, held until the process ends.  In host code its name is only a stand-in
// for the symbol; kernels receive the per-device address hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

namespace {

// hT = h0 (or 0) for an empty sequence: a fill kernel, not a memset, so that the
// call stays safe under stream capture.
__global__ void k_copy_state(const float* __restrict__ h0, float* __restrict__ hT, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) hT[i] = h0 ? h0[i] : 0.f;
}

// dst[0 .. n) = 0: the empty-problem values of the backward's parameter gradients
__global__ void k_zero(float* __restrict__ dst, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = 0.f;
}

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool pn_supported(int64_t P, int64_t N) {
    const bool p = P == 16 || P == 32 || P == 64 || P == 128;
    const bool n = N == 16 || N == 32 || N == 64 || N == 128 || N == 256;
    return p && n;
}

size_t esize(int32_t dtype) { return dtype == SSD_BF16 ? 2 : 4; }

// Shape checks shared by every entry point.
int check_problem(const ssd_problem* p) {
    if (!p) return SSD_ERR_NULL;
    if (p->batch < 0 || p->seqlen < 0 || p->nheads <= 0 || p->headdim <= 0 || p->dstate <= 0 ||
        p->ngroups <= 0 || p->chunk <= 0)
        return SSD_ERR_SHAPE;
    if (p->nheads % p->ngroups != 0) return SSD_ERR_SHAPE;
    if (p->dtype != SSD_F32 && p->dtype != SSD_BF16) return SSD_ERR_UNSUPPORTED;
    if (p->chunk != 64 && p->chunk != 128 && p->chunk != 256) return SSD_ERR_UNSUPPORTED;
    if (!pn_supported(p->headdim, p->dstate)) return SSD_ERR_UNSUPPORTED;
    if (p->flags & ~(SSD_STAGE_ALL | SSD_SCHEDULE_SPLIT | SSD_SCHEDULE_FUSED)) return SSD_ERR_UNSUPPORTED;
    if ((p->flags & SSD_SCHEDULE_SPLIT) && (p->flags & SSD_SCHEDULE_FUSED)) return SSD_ERR_UNSUPPORTED;
    // launch-grid limits: blocks per launch and the batch / group grid dimensions
    const int64_t nc = (p->seqlen + p->chunk - 1) / p->chunk;
    if (p->batch > 65535 || p->batch * p->ngroups > 65535) return SSD_ERR_UNSUPPORTED;
    // the preparation launches' second grid dimension: ceil(nheads / 16) cumsum tasks plus
    // at most 28 table tasks per group (the backward's, at chunk 256)
    if ((p->nheads + 15) / 16 + 28 * p->ngroups > 65535) return SSD_ERR_UNSUPPORTED;
    if (p->nheads > (int64_t)1 << 20 || nc > (int64_t)1 << 24) return SSD_ERR_UNSUPPORTED;
    if (p->batch * p->nheads * (nc > 0 ? nc : 1) > 0x7fffffffLL) return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

// Whether a forward of this problem runs the fused schedule (the launch code takes the
// same decision from the same fields).
bool runs_fused(const ssd_problem* p, int diag) {
    ssd::RunArgs a = {};
    a.b = p->batch; a.T = p->seqlen; a.H = p->nheads; a.P = p->headdim; a.N = p->dstate;
    a.G = p->ngroups; a.Q = p->chunk;
    a.nc = (p->seqlen + p->chunk - 1) / p->chunk;
    a.diag = diag;
    a.ts = nullptr;
    a.force_split = (p->flags & SSD_SCHEDULE_SPLIT) != 0;
    a.force_fused = (p->flags & SSD_SCHEDULE_FUSED) != 0;
    return ssd::fused_applies(a, p->dtype == SSD_BF16);
}

// The regions of the schedule that runs: cdt and (scalar decay) cb always; bt for the
// fused schedule; chunk states, entering states and the segmented scan's carry for the
// split one.  A region the schedule never touches takes no bytes.
ssd_workspace_layout layout_of(const ssd_problem* p, int diag) {
    ssd_workspace_layout L;
    memset(&L, 0, sizeof(L));
    const bool fused = runs_fused(p, diag);
    const int64_t nc = (p->seqlen + p->chunk - 1) / p->chunk;
    const size_t bhc = (size_t)(p->batch * p->nheads * nc);
    const size_t es = esize(p->dtype);
    size_t off = 0;
    L.cdt_off = off;
    L.cdt_bytes = bhc * (size_t)p->chunk * 4;
    off += align_up(L.cdt_bytes);
    L.cb_off = off;
    // scalar decay: the group's C B^T per chunk; diagonal decay: each head's table of
    // decay-weighted products, only where the output kernel's LDS tile does not fit
    const bool tab = diag && ssd::diag_uses_table(p->chunk, p->headdim, p->dstate, es);
    L.cb_bytes = tab    ? bhc * (size_t)(p->chunk * p->chunk) * es
                 : diag ? 0
                        : (size_t)(p->batch * nc * p->ngroups) * (size_t)(p->chunk * p->chunk) * es;
    off += align_up(L.cb_bytes);
    L.states_off = off;
    L.states_bytes = fused ? 0 : bhc * (size_t)(p->headdim * p->dstate) * es;
    off += align_up(L.states_bytes);
    L.hin_off = off;
    L.hin_bytes = fused ? 0 : bhc * (size_t)(p->headdim * p->dstate) * es;
    off += align_up(L.hin_bytes);
    L.bt_off = off;
    // B^T of every chunk, then C of every chunk (both in fragment order)
    L.bt_bytes = (diag || !fused) ? 0 : 2 * (size_t)(p->batch * nc * p->ngroups) * (size_t)(p->dstate * p->chunk) * es;
    off += align_up(L.bt_bytes);
    // the split schedule's state scan in segments (few state elements, many chunks)
    const int64_t sl = ssd::scan_segment_len(p->batch, p->nheads, p->headdim, p->dstate, nc);
    const int64_t nseg = nc > 0 ? (nc + sl - 1) / sl : 0;
    L.carry_off = off;
    L.carry_bytes = (!fused && nseg > 1)
                        ? (size_t)nseg * (size_t)(p->batch * p->nheads) * (size_t)(p->headdim * p->dstate + 1) * 4
                        : 0;
    off += align_up(L.carry_bytes);
    L.total_bytes = (p->batch == 0 || p->seqlen == 0) ? 0 : off;
    return L;
}

bool aligned(const void* ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

struct Range {
    const void* p;
    size_t n;
};
bool overlap(Range a, Range b) {
    if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
    const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
    return a0 < b0 + b.n && b0 < a0 + a.n;
}

// check_only: run every check except those of the workspace (which the caller supplies
// later) and return without any HIP call.
int scan(const ssd_problem* p, int diag, const void* x, const float* dt, const float* A,
         const void* B, const void* C, const float* D, const float* h0, void* y, float* hT,
         void* ws, size_t ws_bytes, void* stream, bool check_only = false) {
    int st = check_problem(p);
    if (st) return st;
    const int64_t b = p->batch, T = p->seqlen, H = p->nheads, P = p->headdim, N = p->dstate,
                  G = p->ngroups, Q = p->chunk;
    const size_t es = esize(p->dtype);
    const size_t state_bytes = (size_t)(b * H * P * N) * 4;
    if (b == 0) return SSD_OK;
    if (!A) return SSD_ERR_NULL;
    if (!aligned(A, 4) || (D && !aligned(D, 4)) || (h0 && !aligned(h0, 16)) || (hT && !aligned(hT, 16)))
        return SSD_ERR_ALIGN;
    if (T == 0) {
        // empty sequence: hT = h0 (or 0); y is empty
        if (!hT) return SSD_OK;
        if (overlap({hT, state_bytes}, {h0, state_bytes})) return SSD_ERR_ALIAS;
        if (check_only) return SSD_OK;
        const int64_t n = b * H * P * N;
        k_copy_state<<<(unsigned)((n + 255) / 256), 256, 0, (hipStream_t)stream>>>(h0, hT, n);
        return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_HIP;
    }
    if (!x || !dt || !B || !C || !y) return SSD_ERR_NULL;
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(y, 16) || !aligned(dt, 4))
        return SSD_ERR_ALIGN;
    const ssd_workspace_layout L = layout_of(p, diag);
    if (check_only) {
        ws = nullptr;  // the workspace is checked once it is known
    } else {
        if (!ws || ws_bytes < L.total_bytes) return SSD_ERR_WORKSPACE;
        if (!aligned(ws, kAlign)) return SSD_ERR_ALIGN;
    }

    const size_t xb = (size_t)(b * T * H * P) * es;
    const Range ins[] = {{x, xb},
                         {dt, (size_t)(b * T * H) * 4},
                         {A, (size_t)(diag ? H * N : H) * 4},
                         {B, (size_t)(b * T * G * N) * es},
                         {C, (size_t)(b * T * G * N) * es},
                         {D, D ? (size_t)H * 4 : 0},
                         {h0, h0 ? state_bytes : 0},
                         {ws, L.total_bytes}};
    const Range ry = {y, xb}, rh = {hT, hT ? state_bytes : 0};
    for (const Range& r : ins)
        if (overlap(ry, r) || overlap(rh, r)) return SSD_ERR_ALIAS;
    if (overlap(ry, rh)) return SSD_ERR_ALIAS;
    if (check_only) return SSD_OK;

    ssd::RunArgs a;
    a.b = b; a.T = T; a.H = H; a.P = P; a.N = N; a.G = G; a.Q = Q;
    a.nc = (T + Q - 1) / Q;
    a.diag = diag;
    a.x = x; a.dt = dt; a.A = A; a.B = B; a.C = C; a.D = D; a.h0 = h0;
    a.y = y; a.hT = hT;
    char* w = static_cast<char*>(ws);
    a.cdt = reinterpret_cast<float*>(w + L.cdt_off);
    a.cb = L.cb_bytes ? static_cast<void*>(w + L.cb_off) : nullptr;
    a.states = L.states_bytes ? static_cast<void*>(w + L.states_off) : nullptr;
    a.hin = L.hin_bytes ? static_cast<void*>(w + L.hin_off) : nullptr;
    a.bt = L.bt_bytes ? static_cast<void*>(w + L.bt_off) : nullptr;
    a.carry = L.carry_bytes ? reinterpret_cast<float*>(w + L.carry_off) : nullptr;
    a.ts = nullptr; a.kb = nullptr; a.kcap = 0;
    a.stream = (hipStream_t)stream;
    a.stages = p->flags & SSD_STAGE_ALL;
    a.force_split = (p->flags & SSD_SCHEDULE_SPLIT) != 0;
    a.force_fused = (p->flags & SSD_SCHEDULE_FUSED) != 0;
    return p->dtype == SSD_BF16 ? ssd::run_bf16(a) : ssd::run_f32(a);
}

// ---- the forward without caller workspace (ssd_scan_fwd_noalloc) ----
// The scratch array's device address on each GPU, looked up once per device (with that
// device current) and kept; later calls reuse it.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

int scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return SSD_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return SSD_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SSD_ERR_HIP;
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return SSD_OK;
}

int scan_noalloc(const ssd_problem* p, const void* x, const float* dt, const float* A, const void* B,
                 const void* C, const float* D, const float* h0, void* y, float* hT, void* stream) {
    // every argument check first, then the size limit, before any HIP call
    int st = scan(p, 0, x, dt, A, B, C, D, h0, y, hT, nullptr, 0, stream, true);
    if (st) return st;
    const ssd_workspace_layout L = layout_of(p, 0);
    if (L.total_bytes > (size_t)SSD_NOALLOC_SCRATCH_BYTES) return SSD_ERR_WORKSPACE;
    void* ws = nullptr;
    if (L.total_bytes > 0) {
        st = scratch_of_current_device(&ws);
        if (st) return st;
    }
    return scan(p, 0, x, dt, A, B, C, D, h0, y, hT, ws, SSD_NOALLOC_SCRATCH_BYTES, stream);
}

// ---- packed variable-length sequences (ssd_scan_fwd_varlen) ----
// batch = number of sequences, seqlen = tokens of the packed axis.  Workspace: cdt
// [H][kcap][Q] f32, C B^T [kcap][G][Q][Q], B^T [kcap][G][N][Q] and C [kcap][G][Q][N] in the
// problem dtype,
// then the row maps ts and kb (batch + 1 int32 each).  kcap = ceil(T/Q) + batch bounds
// the chunks of all sequences together (each adds at most one partial chunk).
struct VarlenLayout {
    size_t cdt_off, cb_off, bt_off, ts_off, kb_off, total;
    int64_t kcap;
};

VarlenLayout varlen_layout_of(const ssd_problem* p) {
    VarlenLayout L;
    memset(&L, 0, sizeof(L));
    const int64_t Q = p->chunk, nseq = p->batch;
    L.kcap = (p->seqlen + Q - 1) / Q + nseq;
    const size_t es = esize(p->dtype), kc = (size_t)L.kcap;
    size_t off = 0;
    L.cdt_off = off;
    off += align_up((size_t)p->nheads * kc * (size_t)Q * 4);
    L.cb_off = off;
    off += align_up(kc * (size_t)p->ngroups * (size_t)(Q * Q) * es);
    L.bt_off = off;
    off += align_up(2 * kc * (size_t)p->ngroups * (size_t)(p->dstate * Q) * es);  // B^T, then C
    L.ts_off = off;
    off += align_up((size_t)(nseq + 1) * 4);
    L.kb_off = off;
    off += align_up((size_t)(nseq + 1) * 4);
    L.total = (nseq == 0 || p->seqlen == 0) ? 0 : off;
    return L;
}

// Packed sequences run on the fused schedule only: bf16, scalar decay, P = 64, N in
// {64, 128}, and every buffer-resource span under 2 GiB.
int check_varlen(const ssd_problem* p) {
    const int st = check_problem(p);
    if (st) return st;
    if (p->flags & SSD_SCHEDULE_SPLIT) return SSD_ERR_UNSUPPORTED;
    if (p->dtype != SSD_BF16 || p->headdim != 64 || (p->dstate != 64 && p->dstate != 128))
        return SSD_ERR_UNSUPPORTED;
    const int64_t T = p->seqlen, H = p->nheads, G = p->ngroups, N = p->dstate, Q = p->chunk;
    const int64_t lim = (int64_t)1 << 31, kcap = (T + Q - 1) / Q + p->batch;
    if (T * H * 64 * 2 >= lim || T * G * N * 2 >= lim || kcap * H * Q >= lim) return SSD_ERR_UNSUPPORTED;
    if (kcap * G * Q * Q * 2 >= lim || kcap * G * N * Q * 2 >= lim) return SSD_ERR_UNSUPPORTED;
    if (p->batch * H >= lim) return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

int scan_varlen(const ssd_problem* p, const int* cu, const void* x, const float* dt, const float* A,
                const void* B, const void* C, const float* D, const float* h0, void* y, float* hT,
                void* ws, size_t ws_bytes, void* stream) {
    int st = check_varlen(p);
    if (st) return st;
    const int64_t nseq = p->batch, T = p->seqlen, H = p->nheads, P = p->headdim, N = p->dstate,
                  G = p->ngroups, Q = p->chunk;
    const size_t es = esize(p->dtype);
    const size_t state_bytes = (size_t)(nseq * H * P * N) * 4;
    if (nseq == 0) return SSD_OK;
    if (!A) return SSD_ERR_NULL;
    if (!aligned(A, 4) || (D && !aligned(D, 4)) || (h0 && !aligned(h0, 16)) || (hT && !aligned(hT, 16)))
        return SSD_ERR_ALIGN;
    if (T == 0) {
        // every sequence is empty: hT = h0 (or 0)
        if (!hT) return SSD_OK;
        if (overlap({hT, state_bytes}, {h0, state_bytes})) return SSD_ERR_ALIAS;
        const int64_t n = nseq * H * P * N;
        k_copy_state<<<(unsigned)((n + 255) / 256), 256, 0, (hipStream_t)stream>>>(h0, hT, n);
        return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_HIP;
    }
    if (!cu || !x || !dt || !B || !C || !y) return SSD_ERR_NULL;
    if (!aligned(cu, 4) || !aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(y, 16) ||
        !aligned(dt, 4))
        return SSD_ERR_ALIGN;
    const VarlenLayout L = varlen_layout_of(p);
    if (!ws || ws_bytes < L.total) return SSD_ERR_WORKSPACE;
    if (!aligned(ws, kAlign)) return SSD_ERR_ALIGN;
    const size_t xb = (size_t)(T * H * P) * es;
    const Range ins[] = {{x, xb},
                         {dt, (size_t)(T * H) * 4},
                         {A, (size_t)H * 4},
                         {B, (size_t)(T * G * N) * es},
                         {C, (size_t)(T * G * N) * es},
                         {D, D ? (size_t)H * 4 : 0},
                         {h0, h0 ? state_bytes : 0},
                         {cu, (size_t)(nseq + 1) * 4},
                         {ws, L.total}};
    const Range ry = {y, xb}, rh = {hT, hT ? state_bytes : 0};
    for (const Range& r : ins)
        if (overlap(ry, r) || overlap(rh, r)) return SSD_ERR_ALIAS;
    if (overlap(ry, rh)) return SSD_ERR_ALIAS;
    if (overlap({cu, (size_t)(nseq + 1) * 4}, {ws, L.total})) return SSD_ERR_ALIAS;

    char* w = static_cast<char*>(ws);
    int* ts = reinterpret_cast<int*>(w + L.ts_off);
    int* kb = reinterpret_cast<int*>(w + L.kb_off);
    if (!(p->flags & SSD_STAGE_ALL) || (p->flags & 1)) {  // the row map goes with the cumsum stage
        ssd::k_rows<1024><<<1, 1024, 0, (hipStream_t)stream>>>(cu, (int)nseq, T, (int)Q, ts, kb);
        if (hipGetLastError() != hipSuccess) return SSD_ERR_HIP;
    }
    ssd::RunArgs a;
    a.b = nseq; a.T = T; a.H = H; a.P = P; a.N = N; a.G = G; a.Q = Q;
    a.nc = (T + Q - 1) / Q;
    a.diag = 0;
    a.x = x; a.dt = dt; a.A = A; a.B = B; a.C = C; a.D = D; a.h0 = h0;
    a.y = y; a.hT = hT;
    a.cdt = reinterpret_cast<float*>(w + L.cdt_off);
    a.cb = static_cast<void*>(w + L.cb_off);
    a.states = nullptr;
    a.hin = nullptr;
    a.bt = static_cast<void*>(w + L.bt_off);
    a.ts = ts; a.kb = kb; a.kcap = L.kcap;
    a.carry = nullptr;
    a.stream = (hipStream_t)stream;
    a.stages = p->flags & SSD_STAGE_ALL;
    a.force_split = false;
    a.force_fused = true;
    return ssd::run_bf16(a);
}

// The token-by-token recurrence on a caller-held state (ssd_step / ssd_diag_step).
int step(const ssd_problem* p, int diag, const void* x, const float* dt, const float* A, const void* B,
         const void* C, const float* D, float* h, void* y, void* stream) {
    if (!p) return SSD_ERR_NULL;
    if (p->batch < 0 || p->seqlen < 0 || p->nheads <= 0 || p->headdim <= 0 || p->dstate <= 0 ||
        p->ngroups <= 0 || p->nheads % p->ngroups != 0)
        return SSD_ERR_SHAPE;
    if (p->dtype != SSD_F32 && p->dtype != SSD_BF16) return SSD_ERR_UNSUPPORTED;
    if (!pn_supported(p->headdim, p->dstate) || p->flags != 0) return SSD_ERR_UNSUPPORTED;
    const int64_t b = p->batch, T = p->seqlen, H = p->nheads, P = p->headdim, N = p->dstate, G = p->ngroups;
    if (b * H > 0x7fffffffLL || b * T * H * P > ((int64_t)1 << 40)) return SSD_ERR_UNSUPPORTED;
    if (b == 0 || T == 0) return SSD_OK;  // nothing to do: h is left as it is
    if (!x || !dt || !A || !B || !C || !h || !y) return SSD_ERR_NULL;
    const size_t es = esize(p->dtype);
    if (!aligned(h, 16) || !aligned(dt, 4) || !aligned(A, 4) || (D && !aligned(D, 4)) || !aligned(x, es) ||
        !aligned(y, es) || !aligned(B, 4 * es) || !aligned(C, 4 * es))
        return SSD_ERR_ALIGN;
    const Range ins[] = {{x, (size_t)(b * T * H * P) * es},
                         {dt, (size_t)(b * T * H) * 4},
                         {A, (size_t)(diag ? H * N : H) * 4},
                         {B, (size_t)(b * T * G * N) * es},
                         {C, (size_t)(b * T * G * N) * es},
                         {D, D ? (size_t)H * 4 : 0}};
    const Range rh = {h, (size_t)(b * H * P * N) * 4}, ry = {y, (size_t)(b * T * H * P) * es};
    for (const Range& r : ins)
        if (overlap(ry, r) || overlap(rh, r)) return SSD_ERR_ALIAS;
    if (overlap(ry, rh)) return SSD_ERR_ALIAS;
    ssd::StepArgs a;
    a.b = b; a.T = T; a.H = H; a.P = P; a.N = N; a.G = G;
    a.diag = diag;
    a.x = x; a.dt = dt; a.A = A; a.B = B; a.C = C; a.D = D; a.h = h; a.y = y;
    a.stream = (hipStream_t)stream;
    return p->dtype == SSD_BF16 ? ssd::run_step<ssd::bf16>(a) : ssd::run_step<float>(a);
}


// ---- backward pass (ssd_scan_bwd) ----
struct BwdLayout {
    size_t cdt, cb, cbt, bt, ct, bcp, ccp, states, hin, rin, hTf, ds, dDp, dAp, kpart, zh, yh, dxp, ddtp, total;
    bool has_states;
    bool has_copies;  // B and C per chunk by token (k_bwd_xs)  // (the chunk walks need no chunk-state region)
};

// Scalar decay: C B^T tables, per-token decay terms and boundary partials, and the chunk
// states unless the chunk walks run.  Diagonal decay: per-token Zh / Yh of every head and,
// when dstate is split over several waves, per-slice partials of dx and ddt, and the chunk
// states.  Both: cumulative dt, H_c, R_c, hT and the per-chunk partial sums of dA and dD.
BwdLayout bwd_layout_of(const ssd_problem* p, int diag) {
    BwdLayout L;
    memset(&L, 0, sizeof(L));
    const int64_t b = p->batch, T = p->seqlen, H = p->nheads, P = p->headdim, N = p->dstate, G = p->ngroups,
                  Q = p->chunk;
    const int64_t nc = (p->seqlen + Q - 1) / Q;
    const size_t es = esize(p->dtype), bhc = (size_t)(b * H * nc), bgc = (size_t)(b * nc * G);
    size_t off = 0;
    auto take = [&](size_t& at, size_t bytes) {
        at = off;
        off += align_up(bytes);
    };
    if (diag) {
        const int nsl = ssd::diag_bwd_slices(P, N);
        take(L.cdt, bhc * (size_t)Q * 4);
        take(L.states, bhc * (size_t)(P * N) * 4);
        L.has_states = true;
        take(L.hin, bhc * (size_t)(P * N) * es);
        take(L.rin, bhc * (size_t)(P * N) * es);
        take(L.hTf, (size_t)(b * H * P * N) * 4);
        take(L.zh, bhc * (size_t)(Q * N) * 4);
        take(L.yh, bhc * (size_t)(Q * N) * 4);
        if (nsl > 1) {
            take(L.dxp, (size_t)nsl * (size_t)(b * T * H * P) * 4);
            take(L.ddtp, (size_t)nsl * (size_t)(b * T * H) * 4);
        }
        take(L.dDp, bhc * 4);
        take(L.dAp, bhc * (size_t)N * 4);
        L.total = (b == 0 || T == 0) ? 0 : off;
        return L;
    }
    take(L.cdt, bhc * (size_t)Q * 4);
    take(L.cb, bgc * (size_t)(Q * Q) * es);
    take(L.cbt, bgc * (size_t)(Q * Q) * es);
    take(L.bt, bgc * (size_t)(N * Q) * es);
    take(L.ct, bgc * (size_t)(N * Q) * es);
    L.has_copies = ssd::xs_applies(p->dtype == SSD_BF16, T, H, P, N, G, Q);
    if (L.has_copies) {
        take(L.bcp, bgc * (size_t)(N * Q) * es);
        take(L.ccp, bgc * (size_t)(N * Q) * es);
    }
    // chunk states (and the adjoint's chunk inputs) only where the chunk walks do not run
    L.has_states = !ssd::walks_apply(p->dtype == SSD_BF16, b, T, H, P, N, G, Q);
    if (L.has_states) take(L.states, bhc * (size_t)(P * N) * 4);
    take(L.hin, bhc * (size_t)(P * N) * es);
    take(L.rin, bhc * (size_t)(P * N) * es);
    take(L.hTf, (size_t)(b * H * P * N) * 4);
    take(L.ds, bhc * (size_t)Q * 4);
    take(L.dDp, bhc * 4);
    take(L.dAp, bhc * 4);
    take(L.kpart, bhc * (size_t)(4 * ((P * N / 4 + 255) / 256)) * 4);
    L.total = (b == 0 || p->seqlen == 0) ? 0 : off;
    return L;
}

int check_bwd(const ssd_problem* p, int diag) {
    const int st = check_problem(p);
    if (st) return st;
    if (p->flags != 0) return SSD_ERR_UNSUPPORTED;
    const int64_t nc = (p->seqlen + p->chunk - 1) / p->chunk;
    if (diag) {
        // one-dimensional grids: the walks (4 waves per work-group) and the element-wise
        // reductions (4 elements per thread)
        const int64_t walks = p->batch * p->nheads * nc * ssd::diag_bwd_slices(p->headdim, p->dstate);
        const int64_t elems = p->batch * p->seqlen * p->nheads * (p->headdim > p->dstate ? p->headdim : p->dstate);
        if ((walks + 3) / 4 > 0x7fffffffLL || elems / 4 / 256 + 1 > 0x7fffffffLL) return SSD_ERR_UNSUPPORTED;
        return SSD_OK;
    }
    // k_bwd_bc's grid: (batch, chunk, group, 64-token slab, n range)
    if (p->batch * (nc > 0 ? nc : 1) * p->ngroups * (p->chunk / 64) * 2 > 0x7fffffffLL) return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

int scan_bwd(const ssd_problem* p, int diag, const void* x, const float* dt, const float* A, const void* B,
             const void* C, const float* D, const float* h0, const void* dy, const float* dhT, void* dx,
             float* ddt, float* dA, void* dB, void* dC, float* dD, float* dh0, void* ws, size_t ws_bytes,
             void* stream) {
    int st = check_bwd(p, diag);
    if (st) return st;
    const int64_t b = p->batch, T = p->seqlen, H = p->nheads, P = p->headdim, N = p->dstate, G = p->ngroups,
                  Q = p->chunk;
    const size_t es = esize(p->dtype);
    const size_t state_bytes = (size_t)(b * H * P * N) * 4;
    const size_t a_bytes = (size_t)(diag ? H * N : H) * 4;  // A and dA
    if (!A || !dA) return SSD_ERR_NULL;
    if (!aligned(A, 4) || !aligned(dA, 4) || (D && !aligned(D, 4)) || (dD && !aligned(dD, 4)) ||
        (h0 && !aligned(h0, 16)) || (dhT && !aligned(dhT, 16)) || (dh0 && !aligned(dh0, 16)))
        return SSD_ERR_ALIGN;
    const Range rdA = {dA, a_bytes}, rdD = {dD, dD ? (size_t)H * 4 : 0}, rdh0 = {dh0, dh0 ? state_bytes : 0};
    hipStream_t s = (hipStream_t)stream;
    if (b == 0 || T == 0) {
        // no tokens: dA = dD = 0 and dh0 = dhT (hT is h0 itself); nothing else to write
        const Range small_in[] = {{A, a_bytes}, {D, D ? (size_t)H * 4 : 0}, {h0, h0 ? state_bytes : 0},
                                  {dhT, dhT ? state_bytes : 0}};
        const Range small_out[] = {rdA, rdD, rdh0};
        for (const Range& o : small_out) {
            for (const Range& r : small_in)
                if (overlap(o, r)) return SSD_ERR_ALIAS;
            for (const Range& o2 : small_out)
                if (&o != &o2 && overlap(o, o2)) return SSD_ERR_ALIAS;
        }
        k_zero<<<(unsigned)((a_bytes / 4 + 255) / 256), 256, 0, s>>>(dA, (int64_t)(a_bytes / 4));
        if (dD) k_zero<<<(unsigned)((H + 255) / 256), 256, 0, s>>>(dD, H);
        if (dh0 && b > 0) {
            const int64_t n = b * H * P * N;
            k_copy_state<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(dhT, dh0, n);
        }
        return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_HIP;
    }
    if (!x || !dt || !B || !C || !dy || !dx || !ddt || !dB || !dC) return SSD_ERR_NULL;
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(dy, 16) || !aligned(dx, 16) ||
        !aligned(dB, 16) || !aligned(dC, 16) || !aligned(dt, 4) || !aligned(ddt, 4))
        return SSD_ERR_ALIGN;
    const BwdLayout L = bwd_layout_of(p, diag);
    if (!ws || ws_bytes < L.total) return SSD_ERR_WORKSPACE;
    if (!aligned(ws, kAlign)) return SSD_ERR_ALIGN;
    const size_t xb = (size_t)(b * T * H * P) * es, bcb = (size_t)(b * T * G * N) * es;
    const Range ins[] = {{x, xb},
                         {dt, (size_t)(b * T * H) * 4},
                         {A, a_bytes},
                         {B, bcb},
                         {C, bcb},
                         {D, D ? (size_t)H * 4 : 0},
                         {h0, h0 ? state_bytes : 0},
                         {dy, xb},
                         {dhT, dhT ? state_bytes : 0},
                         {ws, L.total}};
    const Range outs[] = {{dx, xb}, {ddt, (size_t)(b * T * H) * 4}, rdA, {dB, bcb}, {dC, bcb}, rdD, rdh0};
    for (const Range& o : outs) {
        for (const Range& r : ins)
            if (overlap(o, r)) return SSD_ERR_ALIAS;
        for (const Range& o2 : outs)
            if (&o != &o2 && overlap(o, o2)) return SSD_ERR_ALIAS;
    }

    ssd::BwdArgs a;
    a.b = b; a.T = T; a.H = H; a.P = P; a.N = N; a.G = G; a.Q = Q;
    a.nc = (T + Q - 1) / Q;
    a.x = x; a.dt = dt; a.A = A; a.B = B; a.C = C; a.D = D; a.h0 = h0; a.dy = dy; a.dhT = dhT;
    a.dx = dx; a.ddt = ddt; a.dA = dA; a.dB = dB; a.dC = dC; a.dD = dD; a.dh0 = dh0;
    char* w = static_cast<char*>(ws);
    a.cdt = reinterpret_cast<float*>(w + L.cdt);
    a.cb = w + L.cb;
    a.cbt = w + L.cbt;
    a.bt = w + L.bt;
    a.ct = w + L.ct;
    a.bcp = L.has_copies ? static_cast<void*>(w + L.bcp) : nullptr;
    a.ccp = L.has_copies ? static_cast<void*>(w + L.ccp) : nullptr;
    a.states = L.has_states ? reinterpret_cast<float*>(w + L.states) : nullptr;
    a.hin = w + L.hin;
    a.rin = w + L.rin;
    a.hTf = reinterpret_cast<float*>(w + L.hTf);
    a.ds = reinterpret_cast<float*>(w + L.ds);
    a.dDp = reinterpret_cast<float*>(w + L.dDp);
    a.dAp = reinterpret_cast<float*>(w + L.dAp);
    a.kpart = reinterpret_cast<float*>(w + L.kpart);
    a.zh = reinterpret_cast<float*>(w + L.zh);
    a.yh = reinterpret_cast<float*>(w + L.yh);
    a.dxp = reinterpret_cast<float*>(w + L.dxp);
    a.ddtp = reinterpret_cast<float*>(w + L.ddtp);
    a.stream = s;
    if (diag) return p->dtype == SSD_BF16 ? ssd::run_bwd_diag_bf16(a) : ssd::run_bwd_diag_f32(a);
    return p->dtype == SSD_BF16 ? ssd::run_bwd_bf16(a) : ssd::run_bwd_f32(a);
}

}  // namespace

extern "C" {

int ssd_step(const ssd_problem* p, const void* x, const float* dt, const float* A, const void* B,
             const void* C, const float* D, float* h, void* y, void* stream) {
    return step(p, 0, x, dt, A, B, C, D, h, y, stream);
}

int ssd_diag_step(const ssd_problem* p, const void* x, const float* dt, const float* A, const void* B,
                  const void* C, const float* D, float* h, void* y, void* stream) {
    return step(p, 1, x, dt, A, B, C, D, h, y, stream);
}

size_t ssd_workspace_bytes(const ssd_problem* p, int diag) {
    if (check_problem(p)) return 0;
    return layout_of(p, diag ? 1 : 0).total_bytes;
}

int ssd_get_workspace_layout(const ssd_problem* p, int diag, ssd_workspace_layout* out) {
    if (!out) return SSD_ERR_NULL;
    const int st = check_problem(p);
    if (st) return st;
    *out = layout_of(p, diag ? 1 : 0);
    return SSD_OK;
}

int ssd_scan_fwd(const ssd_problem* p, const void* x, const float* dt, const float* A,
                 const void* B, const void* C, const float* D, const float* h0, void* y,
                 float* hT, void* ws, size_t ws_bytes, void* stream) {
    return scan(p, 0, x, dt, A, B, C, D, h0, y, hT, ws, ws_bytes, stream);
}

int ssd_scan_fwd_noalloc(const ssd_problem* p, const void* x, const float* dt, const float* A,
                         const void* B, const void* C, const float* D, const float* h0, void* y,
                         float* hT, void* stream) {
    return scan_noalloc(p, x, dt, A, B, C, D, h0, y, hT, stream);
}

int ssd_diag_scan_fwd(const ssd_problem* p, const void* x, const float* dt, const float* A,
                      const void* B, const void* C, const float* D, const float* h0, void* y,
                      float* hT, void* ws, size_t ws_bytes, void* stream) {
    return scan(p, 1, x, dt, A, B, C, D, h0, y, hT, ws, ws_bytes, stream);
}

size_t ssd_varlen_workspace_bytes(const ssd_problem* p) {
    if (check_varlen(p)) return 0;
    return varlen_layout_of(p).total;
}

int ssd_scan_fwd_varlen(const ssd_problem* p, const int32_t* cu_seqlens, const void* x, const float* dt,
                        const float* A, const void* B, const void* C, const float* D, const float* h0,
                        void* y, float* hT, void* ws, size_t ws_bytes, void* stream) {
    return scan_varlen(p, cu_seqlens, x, dt, A, B, C, D, h0, y, hT, ws, ws_bytes, stream);
}

size_t ssd_bwd_workspace_bytes(const ssd_problem* p) {
    if (check_bwd(p, 0)) return 0;
    return bwd_layout_of(p, 0).total;
}

int ssd_scan_bwd(const ssd_problem* p, const void* x, const float* dt, const float* A, const void* B,
                 const void* C, const float* D, const float* h0, const void* dy, const float* dhT, void* dx,
                 float* ddt, float* dA, void* dB, void* dC, float* dD, float* dh0, void* ws, size_t ws_bytes,
                 void* stream) {
    return scan_bwd(p, 0, x, dt, A, B, C, D, h0, dy, dhT, dx, ddt, dA, dB, dC, dD, dh0, ws, ws_bytes, stream);
}

size_t ssd_diag_bwd_workspace_bytes(const ssd_problem* p) {
    if (check_bwd(p, 1)) return 0;
    return bwd_layout_of(p, 1).total;
}

int ssd_diag_scan_bwd(const ssd_problem* p, const void* x, const float* dt, const float* A, const void* B,
                      const void* C, const float* D, const float* h0, const void* dy, const float* dhT, void* dx,
                      float* ddt, float* dA, void* dB, void* dC, float* dD, float* dh0, void* ws, size_t ws_bytes,
                      void* stream) {
    return scan_bwd(p, 1, x, dt, A, B, C, D, h0, dy, dhT, dx, ddt, dA, dB, dC, dD, dh0, ws, ws_bytes, stream);
}

const char* ssd_status_string(int status) {
    switch (status) {
        case SSD_OK: return "ok";
        case SSD_ERR_NULL: return "a required pointer is NULL";
        case SSD_ERR_SHAPE: return "invalid shape (negative/zero dimension or nheads % ngroups != 0)";
        case SSD_ERR_UNSUPPORTED: return "unsupported chunk, headdim, dstate, dtype, flags or size";
        case SSD_ERR_WORKSPACE: return "workspace missing or too small";
        case SSD_ERR_ALIGN: return "pointer misaligned (16 B for tensors, 4 B for dt/A/D, 256 B for workspace)";
        case SSD_ERR_ALIAS: return "an output overlaps an input, the workspace or the other output";
        case SSD_ERR_HIP: return "HIP kernel launch failed";
        default: return "unknown status";
    }
}

int ssd_version(void) { return SSD_VERSION; }

}  // extern "C"
