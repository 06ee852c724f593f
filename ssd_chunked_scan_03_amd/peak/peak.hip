// peak.hip -- measured denominators for the roofline: a streaming copy (HBM bandwidth the
// chip delivers to a plain read-once / write-once kernel) and a dense loop of bf16
// matrix-core steps (the matrix-core rate the chip sustains).  Measurement only: built
// into its own library, which the benchmark loads; the SSD library does not use it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// dst[i] = src[i] for n 16-byte elements, grid-stride; each thread has four 16-byte
// loads in flight before its stores.  NT: non-temporal loads and stores (streamed once).
template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4* p) { return NT ? __builtin_nontemporal_load(p) : *p; }
template <bool NT>
__device__ __forceinline__ void st(u32x4* p, u32x4 v) {
    if (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}
template <bool NT>
__global__ __launch_bounds__(256) void k_copy16(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const u32x4 a = ld<NT>(src + i), b = ld<NT>(src + i + stride), c = ld<NT>(src + i + 2 * stride),
                    d = ld<NT>(src + i + 3 * stride);
        st<NT>(dst + i, a);
        st<NT>(dst + i + stride, b);
        st<NT>(dst + i + 2 * stride, c);
        st<NT>(dst + i + 3 * stride, d);
    }
    for (; i < n; i += stride) st<NT>(dst + i, ld<NT>(src + i));
}

// `iters` rounds of 8 independent 16x16x32 bf16 matrix-core steps per wave (8 chains hide
// the step latency); the accumulators are summed and written so nothing is dropped.
__global__ __launch_bounds__(256) void k_mfma(float* __restrict__ out, int iters, float seed) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(seed * (float)(lane + e));
        b[e] = (__bf16)(seed * (float)(lane - e));
    }
    f32x4 acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the steps are written as instructions so that the compiler keeps each chain in its
    // own accumulator registers (as builtins, it rotated them through copies every round)
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 8; ++k)
            asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[k]) : "v"(a), "v"(b));
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Enqueue one copy of `bytes` (a multiple of 16) from src to dst on `stream` with
// `blocks` work-groups of 256 threads; nt != 0: non-temporal accesses.
int peak_copy(const void* src, void* dst, int64_t bytes, int blocks, int nt, void* stream) {
    if (!src || !dst || bytes <= 0 || bytes % 16 || blocks <= 0) return 1;
    const int64_t n = bytes / 16;
    if (nt)
        k_copy16<true><<<blocks, 256, 0, (hipStream_t)stream>>>(static_cast<const u32x4*>(src),
                                                                static_cast<u32x4*>(dst), n);
    else
        k_copy16<false><<<blocks, 256, 0, (hipStream_t)stream>>>(static_cast<const u32x4*>(src),
                                                                 static_cast<u32x4*>(dst), n);
    return hipGetLastError() == hipSuccess ? 0 : 7;
}

// Enqueue `blocks` work-groups of 4 waves, each wave `iters` x 8 bf16 16x16x32 steps;
// `out` holds blocks * 256 floats.  Returns the matrix-core flops enqueued in *flops.
int peak_mfma(float* out, int blocks, int iters, double* flops, void* stream) {
    if (!out || blocks <= 0 || iters <= 0 || !flops) return 1;
    k_mfma<<<blocks, 256, 0, (hipStream_t)stream>>>(out, iters, 1e-3f);
    *flops = (double)blocks * 4 * iters * 8 * (2.0 * 16 * 16 * 32);
    return hipGetLastError() == hipSuccess ? 0 : 7;
}

}  // extern "C"
