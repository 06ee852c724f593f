// step.hpp -- the recurrence itself, token by token, on a caller-held state (the linear
// form of the map: "Structured State Space Duality" concept page, section "The recurrence
// as one matrix"; the section "When it breaks" notes that serving runs this form):
//
//   for t = 0 .. T-1:   h <- a_t h + x_t B_t^T        a_t = exp(dt_t A_h)  (or A_{h,n})
//                       y_t = h C_t + D_h x_t
//
// h is read once, kept in registers across the tokens and written back in place, so a
// decode step (T = 1) moves the state twice and nothing else of size: the kernel is
// bound by HBM bandwidth on the state.  One thread owns 8 consecutive elements
// (p, n .. n+7) of a head's row-major P x N state, two 16-byte loads in flight per
// thread; the N/8 threads of one row p are consecutive lanes of one wave and reduce
// y_t[p] with butterfly shuffles.  Grid (b H, ceil(P N / 2048)), 256 threads.
#pragma once

#include "device.hpp"

namespace ssd {

template <typename T>
__device__ __forceinline__ void ld8f(const T* p, float* v) {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = to_f(p[k]);
}

template <typename T, bool DIAG>
__global__ __launch_bounds__(256) void k_step(const T* __restrict__ x, const float* __restrict__ dt,
                                              const float* __restrict__ A, const T* __restrict__ Bm,
                                              const T* __restrict__ Cm, const float* __restrict__ D,
                                              float* __restrict__ h, T* __restrict__ y, int64_t Tn, int H, int P,
                                              int N, int G) {
    constexpr float LOG2E = 1.4426950408889634f;
    constexpr int E = 8;  // state elements per thread
    const int64_t bh = blockIdx.x;
    const int hh = (int)(bh % H);
    const int64_t bi = bh / H;
    const int g = hh / (H / G);
    const int e0 = (blockIdx.y * 256 + threadIdx.x) * E;  // first owned element of the flattened state
    const bool active = e0 < P * N;
    const int ec = active ? e0 : 0;                        // in-bounds index for idle lanes
    const int p = ec / N, n0 = ec % N;
    const int R = N / E;                                   // lanes per state row (power of 2, <= 32)
    const int lane = threadIdx.x & 63;

    float* hp = h + bh * (int64_t)P * N + ec;
    f32x4 h0v = f32x4{0.f, 0.f, 0.f, 0.f}, h1v = h0v;
    if (active) {
        h0v = *reinterpret_cast<const f32x4*>(hp);
        h1v = *reinterpret_cast<const f32x4*>(hp + 4);
    }
    float hv[E];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        hv[k] = h0v[k];
        hv[4 + k] = h1v[k];
    }
    float a2[E];  // A * log2(e): one per owned element (diagonal decay) or the head's (scalar)
#pragma unroll
    for (int k = 0; k < E; ++k) a2[k] = (DIAG ? A[(int64_t)hh * N + n0 + k] : A[hh]) * LOG2E;
    const float Dh = D ? D[hh] : 0.f;

    for (int64_t t = 0; t < Tn; ++t) {
        const int64_t row = bi * Tn + t;  // token row of x / dt / B / C / y
        const float d = dt[row * H + hh];
        const float xp = to_f(x[(row * H + hh) * P + p]);
        float bv[E], cv[E];
        ld8f(Bm + (row * G + g) * N + n0, bv);
        ld8f(Cm + (row * G + g) * N + n0, cv);
        float part = 0.f;
#pragma unroll
        for (int k = 0; k < E; ++k) {
            const float a = exp2f_fast(d * a2[k]);
            hv[k] = a * hv[k] + xp * bv[k];
            part += hv[k] * cv[k];
        }
        // sum over the R lanes of this row (aligned groups of R lanes)
        for (int off = R >> 1; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
        if (active && (lane & (R - 1)) == 0) y[(row * H + hh) * P + p] = from_f<T>(part + Dh * xp);
    }
    if (active) {
        *reinterpret_cast<f32x4*>(hp) = f32x4{hv[0], hv[1], hv[2], hv[3]};
        *reinterpret_cast<f32x4*>(hp + 4) = f32x4{hv[4], hv[5], hv[6], hv[7]};
    }
}

struct StepArgs {
    int64_t b, T, H, P, N, G;
    int diag;
    const void* x;
    const float* dt;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    float* h;
    void* y;
    hipStream_t stream;
};

template <typename T>
int run_step(const StepArgs& a) {
    const dim3 grid((unsigned)(a.b * a.H), (unsigned)((a.P * a.N + 2047) / 2048));
    const T* x = static_cast<const T*>(a.x);
    const T* B = static_cast<const T*>(a.B);
    const T* C = static_cast<const T*>(a.C);
    T* y = static_cast<T*>(a.y);
    if (a.diag)
        k_step<T, true><<<grid, 256, 0, a.stream>>>(x, a.dt, a.A, B, C, a.D, a.h, y, a.T, (int)a.H, (int)a.P,
                                                    (int)a.N, (int)a.G);
    else
        k_step<T, false><<<grid, 256, 0, a.stream>>>(x, a.dt, a.A, B, C, a.D, a.h, y, a.T, (int)a.H, (int)a.P,
                                                     (int)a.N, (int)a.G);
    return hipGetLastError() == hipSuccess ? 0 : 7;
}

}  // namespace ssd
