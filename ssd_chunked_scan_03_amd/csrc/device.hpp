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
// 2^x (v_exp_f32); callers fold log2(e) into their decay constants.
__device__ __forceinline__ float exp2f_fast(float x) { return __builtin_amdgcn_exp2f(x); }

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

// Select without branching: loads are always issued (from an address the caller keeps
// valid, e.g. a clamped row) and masked afterwards, so no load sits in a divergent
// branch that would force a wait at the join.
__device__ __forceinline__ bf16x8 sel8(bool keep, bf16x8 v) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 b = __builtin_bit_cast(u32x4, v);
    const unsigned m = keep ? 0xffffffffu : 0u;
    return __builtin_bit_cast(bf16x8, u32x4{b[0] & m, b[1] & m, b[2] & m, b[3] & m});
}
__device__ __forceinline__ f32x8 sel8(bool keep, f32x8 v) {
    f32x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = keep ? v[e] : 0.f;
    return r;
}

// ---------------------------------------------------------------------------
// Buffer loads/stores: a 128-bit resource (base, byte size) in SGPRs, a per-lane 32-bit
// byte offset and a uniform 32-bit byte offset.  Accesses past the resource's size read
// as zero and drop stores, which the fused kernel uses for rows past the sequence end.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t brsrc;
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));

// The base and size are made wave-uniform explicitly (readfirstlane), so the resource
// lives in SGPRs and no buffer access needs a loop over distinct resources.
__device__ __forceinline__ brsrc make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void* p = (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
// Element offset of entry (r, col) of a per-chunk table whose rows hold Q columns (C B^T
// and its transpose, B^T and C^T per chunk), stored in matrix-core fragment order: the
// 16-row x 32-column fragment (r / 16, col / 32) is 512 consecutive elements, in which lane
// l = 16 ((col % 32) / 8) + r % 16 of a fragment load finds its 8 consecutive columns.  A
// wave's fragment load is then one contiguous 1 KB run (bfloat16) rather than a piece of
// each of 16 rows.
__host__ __device__ __forceinline__ int64_t tfrag(int64_t r, int col, int Q) {
    return ((r >> 4) * (Q >> 5) + (col >> 5)) * 512 + (((col & 31) >> 3) << 7) + ((r & 15) << 3) + (col & 7);
}

// Lane index recomputed from the execution mask (two VALU ops) instead of kept live:
// values needed only at chunk boundaries are rebuilt there rather than spilled.
__device__ __forceinline__ int lane_now() {
    int l;
    // volatile: recomputed where it is used, never hoisted and kept live
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// wave index within the work-group, known uniform to the compiler
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }
__device__ __forceinline__ bf16x8 bload8(brsrc r, int voff, int soff) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ void bstore4(brsrc r, bf16x4 v, int voff, int soff) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, voff, soff, 0);
}

template <typename T> __device__ __forceinline__ typename V8<T>::type zero8() {
    typename V8<T>::type z;
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = from_f<T>(0.f);
    return z;
}

// ---------------------------------------------------------------------------
// Operand fragments whose k index runs down the rows of a row-major LDS tile.
// gfx950's ds_read_b64_tr_b16 works on 16-lane groups: source lane s supplies the
// address of 4 consecutive 16-bit elements, destination lane i receives element i % 4
// of source lanes i/4, i/4 + 4, i/4 + 8, i/4 + 12.  If source lane s points at
// row (base + s/4), column (c0 + 4 (s % 4)), destination lane i therefore gets rows
// base..base+3 of column c0 + i: four k-consecutive values of one MFMA column.
// Two such reads make the 8-element fragment.  float32 tiles read element by element.
// ---------------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ s16x4 ds_tr16(const void* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

// Lane l (group q = l / 16) receives M[ra + e][c0 + l % 16] for e = 0..3 and
// M[rb + e - 4][c0 + l % 16] for e = 4..7, where ra, rb are this lane's group row bases.
__device__ __forceinline__ bf16x8 frag_rows_split(const bf16* M, int ld, int ra, int rb, int c0, int lane) {
    const int s = lane & 15;
    const s16x4 a = ds_tr16(M + (ra + (s >> 2)) * ld + c0 + 4 * (s & 3));
    const s16x4 b = ds_tr16(M + (rb + (s >> 2)) * ld + c0 + 4 * (s & 3));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}
__device__ __forceinline__ f32x8 frag_rows_split(const float* M, int ld, int ra, int rb, int c0, int lane) {
    const int col = c0 + (lane & 15);
    f32x8 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[e] = M[(ra + e) * ld + col];
        v[4 + e] = M[(rb + e) * ld + col];
    }
    return v;
}
// The standard layout: lane l holds M[k0 + 8 (l/16) + e][c0 + l % 16], e = 0..7.
template <typename T>
__device__ __forceinline__ typename V8<T>::type frag_rows(const T* M, int ld, int k0, int c0, int lane) {
    const int r = k0 + 8 * (lane >> 4);
    return frag_rows_split(M, ld, r, r + 4, c0, lane);
}

__device__ __forceinline__ bf16x4 pack4(bf16 a, bf16 b, bf16 c, bf16 d) { return bf16x4{a, b, c, d}; }

__device__ __forceinline__ f32x4 mma(f32x4 c, bf16x8 a, bf16x8 b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(f32x4 c, f32x8 a, f32x8 b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
    return c;
}

}  // namespace ssd
