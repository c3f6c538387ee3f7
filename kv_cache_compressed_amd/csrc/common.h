// Device primitives shared by the MTLA kernels (gfx950 / CDNA4, wave64).
//
// MFMA operand layouts used throughout (checked on the hardware):
//   v_mfma_f32_16x16x32_bf16: A (16 x 32): lane l holds row l%16, k = 8*(l/16)+e
//                             B (32 x 16): lane l holds col l%16, k = 8*(l/16)+e
//                             D (16 x 16): lane l holds col l%16, rows 4*(l/16)+i
//   v_mfma_f32_16x16x4_f32:   A lane l: row l%16, k = l/16 (one element).
// A K=32 step on fp32 data is eight 16x16x4 MFMAs where instruction e takes
// element e of each lane; together they cover k = 8*(l/16)+e for all e, i.e.
// the same lane-to-k assignment as the bf16 instruction, so fragments of both
// types have identical layouts (8 elements per lane) and every kernel is
// written once over the storage type T.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtla {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;

template <typename T> struct Frag;
template <> struct Frag<bf16> { typedef bf16x8 type; };
template <> struct Frag<float> { typedef f32x8 type; };

__device__ __forceinline__ f32x4 mma_k32(const bf16x8 &a, const bf16x8 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mma_k32(const f32x8 &a, const f32x8 &b, f32x4 c) {
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

// 8 consecutive elements from a 16-byte aligned address (global or LDS).
__device__ __forceinline__ void load8(bf16x8 &v, const bf16 *p) { v = *(const bf16x8 *)p; }
__device__ __forceinline__ void load8(f32x8 &v, const float *p) {
  f32x4 a = *(const f32x4 *)p, b = *(const f32x4 *)(p + 4);
  v = (f32x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

template <typename T> __device__ __forceinline__ typename Frag<T>::type zero_frag() {
  typename Frag<T>::type v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (T)0.0f;
  return v;
}

// 16-byte chunk copy helpers used by the staging loops.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ldg16(const void *p) { return *(const u32x4 *)p; }
__device__ __forceinline__ void sts16(void *p, u32x4 v) { *(u32x4 *)p = v; }

__device__ __forceinline__ float sigmoidf(float g) { return 1.0f / (1.0f + expf(-g)); }

__device__ __forceinline__ float wave_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

}  // namespace mtla
