// Device-side building blocks shared by the gfx950 kernels of libgqe.
//
// Matrix products run on the CDNA4 matrix cores through one 16x16 output
// block abstraction, `mma16`, whose contraction step is 32 elements:
//   * bf16: one v_mfma_f32_16x16x32_bf16;
//   * fp32: eight v_mfma_f32_16x16x4_f32 (used only by fp32 layers).
// Operand fragments hold, for lane l, 8 consecutive contraction elements
// (offset 8*(l/16)) of row (or column) l%16. Both operands use the same
// contraction mapping, so the product is exact whatever order the hardware
// walks the 32 elements in. The 16x16 fp32 result block puts column l%16,
// rows 4*(l/16)+v (v = 0..3) in lane l.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqe {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

// Eight contraction elements of one lane.
template <typename T> struct Frag;
template <> struct Frag<bf16> {
    bf16x8 v;
};
template <> struct Frag<float> {
    f32x4 lo, hi;
};

__device__ __forceinline__ f32x4 mma16(const Frag<bf16>& a, const Frag<bf16>& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(const Frag<float>& a, const Frag<float>& b, f32x4 c) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[j], b.lo[j], c, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[j], b.hi[j], c, 0, 0, 0);
    return c;
}

// 16-byte loads and stores (all pointers are 16-byte aligned by contract).
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

template <typename T> __device__ __forceinline__ Frag<T> ld_frag(const void* p);
template <> __device__ __forceinline__ Frag<bf16> ld_frag<bf16>(const void* p) {
    Frag<bf16> f;
    f.v = *reinterpret_cast<const bf16x8*>(p);
    return f;
}
template <> __device__ __forceinline__ Frag<float> ld_frag<float>(const void* p) {
    Frag<float> f;
    f.lo = reinterpret_cast<const f32x4*>(p)[0];
    f.hi = reinterpret_cast<const f32x4*>(p)[1];
    return f;
}

__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(float v) { return v; }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }   // RNE
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }

// Elements of T in one 16-byte vector.
template <typename T> struct Vec16 { static constexpr int N = 16 / sizeof(T); };

// Eight fp32 values -> 8 elements of T at p (16 bytes for bf16, 32 for fp32).
template <typename T> __device__ __forceinline__ void store8(T* p, const float* v);
template <> __device__ __forceinline__ void store8<bf16>(bf16* p, const float* v) {
    bf16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (bf16)v[i];
    *reinterpret_cast<bf16x8*>(p) = o;
}
template <> __device__ __forceinline__ void store8<float>(float* p, const float* v) {
    f32x4 a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
    reinterpret_cast<f32x4*>(p)[0] = a;
    reinterpret_cast<f32x4*>(p)[1] = b;
}

// Eight elements of T at p -> fp32.
template <typename T> __device__ __forceinline__ void load8(const T* p, float* v);
template <> __device__ __forceinline__ void load8<bf16>(const bf16* p, float* v) {
    bf16x8 a = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)a[i];
}
template <> __device__ __forceinline__ void load8<float>(const float* p, float* v) {
    f32x4 a = reinterpret_cast<const f32x4*>(p)[0], b = reinterpret_cast<const f32x4*>(p)[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
}

// Workgroups of one launch are dealt to the 8 XCDs of the chip round-robin
// (id i runs on XCD i % 8). Remap so that ids [x*n/8, (x+1)*n/8) all run on
// XCD x: neighbours in the logical order then share that XCD's L2.
__device__ __forceinline__ int64_t xcd_logical_id(int64_t hw, int64_t n) {
    if (n % 8 != 0) return hw;
    return (hw % 8) * (n / 8) + hw / 8;
}

}  // namespace gqe
