// device.hpp -- gfx950 building blocks for the SSD kernels: element types,
// 8-element operand fragments, the 16x16x32 matrix-core step and a base-2 exp.
//
// Matrix-core tiles.  One 64-lane wave computes a 16x16 fp32 tile D += A * B
// with K = 32:
//   A fragment: lane l holds A[row = l % 16][k = 8 * (l / 16) + e], e = 0..7
//   B fragment: lane l holds B[k = 8 * (l / 16) + e][col = l % 16]
//   D tile    : lane l holds D[row = 4 * (l / 16) + r][col = l % 16], r = 0..3
// A and B share one lane/element -> k map, so any consistent permutation of k
// between the two operands gives the same contraction.  bfloat16 operands use
// one v_mfma_f32_16x16x32_bf16; float32 operands use eight v_mfma_f32_16x16x4f32,
// the e-th taking element e of every lane (k = 8 * (l / 16) + e again).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

template <typename T> struct V8;
template <> struct V8<bf16> { typedef bf16x8 type; };
template <> struct V8<float> { typedef f32x8 type; };
template <typename T> struct V4;
template <> struct V4<bf16> { typedef bf16x4 type; };
template <> struct V4<float> { typedef f32x4 type; };

// e^x through the hardware 2^x (v_exp_f32): e^x = 2^(x * log2(e)).
__device__ __forceinline__ float exp_f(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

__device__ __forceinline__ float to_f(bf16 v) { return (float)v; }
__device__ __forceinline__ float to_f(float v) { return v; }
template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ bf16 from_f<bf16>(float v) { return (bf16)v; }
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }

// 8 consecutive elements, 16-byte aligned address (global or LDS).
__device__ __forceinline__ bf16x8 ld8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ f32x8 ld8(const float* p) {
    const f32x4 a = reinterpret_cast<const f32x4*>(p)[0];
    const f32x4 b = reinterpret_cast<const f32x4*>(p)[1];
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ void st8(bf16* p, bf16x8 v) { *reinterpret_cast<bf16x8*>(p) = v; }
__device__ __forceinline__ void st8(float* p, f32x8 v) {
    reinterpret_cast<f32x4*>(p)[0] = __builtin_shufflevector(v, v, 0, 1, 2, 3);
    reinterpret_cast<f32x4*>(p)[1] = __builtin_shufflevector(v, v, 4, 5, 6, 7);
}
// 4 consecutive elements (8-byte aligned for bf16, 16-byte for float).
__device__ __forceinline__ bf16x4 ld4(const bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }
__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st4(bf16* p, bf16x4 v) { *reinterpret_cast<bf16x4*>(p) = v; }
__device__ __forceinline__ void st4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }

template <typename T> __device__ __forceinline__ typename V8<T>::type zero8() {
    typename V8<T>::type z;
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = from_f<T>(0.f);
    return z;
}

__device__ __forceinline__ f32x4 mma(f32x4 c, bf16x8 a, bf16x8 b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(f32x4 c, f32x8 a, f32x8 b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
    return c;
}

}  // namespace ssd
