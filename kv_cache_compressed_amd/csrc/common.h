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

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtla {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
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

// K=16 step: O (16x16) += A (16 x 16) B (16 x 16); lane l holds row/col l%16
// and k = 4*(l/16)+e, e < 4 (the layout of a ds_read_tr16_b64 result).
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mma_k16(const bf16x4 &a, const bf16x4 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                    __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_k16(const f32x4 &a, const f32x4 &b, f32x4 c) {
#pragma unroll
  for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
  return c;
}

template <typename T> struct Frag4;
template <> struct Frag4<bf16> { typedef bf16x4 type; };
template <> struct Frag4<float> { typedef f32x4 type; };

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

// 4 consecutive elements (8- or 16-byte aligned) <-> fp32.
__device__ __forceinline__ f32x4 load4f(const bf16 *p) {
  const bf16x4 v = *(const bf16x4 *)p;
  return (f32x4){(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ f32x4 load4f(const float *p) { return *(const f32x4 *)p; }
__device__ __forceinline__ void store4f(bf16 *p, f32x4 v) {
  *(bf16x4 *)p = (bf16x4){(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}
__device__ __forceinline__ void store4f(float *p, f32x4 v) { *(f32x4 *)p = v; }

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

// Max / sum over the four lanes c, c+16, c+32, c+48 (the lane groups that
// share an MFMA output column), with gfx950's cross-row swaps
// v_permlane16_swap / v_permlane32_swap: VALU operations, no LDS round trip
// (a shuffle through ds_bpermute waits on the LDS pipe every time).  Written
// in asm to obtain both registers the swap writes; s_nop pads the VALU
// hazards around them.
__device__ __forceinline__ void perm_swap16(float &a, float &b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void perm_swap32(float &a, float &b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float max_g(float v) {
  float a = v, b = v;
  perm_swap16(a, b);
  float c = fmaxf(a, b), d = c;
  perm_swap32(c, d);
  return fmaxf(c, d);
}
__device__ __forceinline__ float sum_g(float v) {
  float a = v, b = v;
  perm_swap16(a, b);
  float c = a + b, d = c;
  perm_swap32(c, d);
  return c + d;
}

// ---- 16-row LDS tiles filled by direct global->LDS loads ------------------
//
// A tile holds 16 rows of RB bytes (RB a multiple of 64) as RB/64 blocks of
// 1 KB: block q holds bytes [64q, 64q + 64) of the 16 rows, row i at offset
// 64 i, with the row's four 16-byte chunks permuted by XOR with swz(i).  One
// global_load_lds_dwordx4 (64 lanes x 16 B, lane l landing at 16 l) fills one
// block when lane l fetches chunk (l%4) ^ swz(l/4) of row l/4.  The
// permutation makes both read patterns conflict free whether the LDS serves
// 128 or 256 bytes per clock: the 16-byte reads that feed an MFMA operand (16
// rows, same columns) and the 8-byte transposing reads (4 rows x 32
// contiguous bytes per 16 lanes).
__device__ __forceinline__ int swz(int row) {
  return ((((row >> 1) ^ (row >> 2) ^ (row >> 3)) & 1) << 1) | ((row >> 2) & 1);
}

__device__ __forceinline__ int tile_off(int row, int byte) {
  return ((byte >> 6) << 10) + (row << 6) + ((((byte >> 4) & 3) ^ swz(row)) << 4) + (byte & 15);
}

typedef __attribute__((address_space(3))) void lds_void;

// Issue one block load.  `row_ptr` is the global address of the row this
// lane copies (row lane/4 of the block), `q` the block's 64-byte column
// segment, `dst` the block's LDS address (wave-uniform).
__device__ __forceinline__ void dma_block(const char *row_ptr, int q, char *dst) {
  const int lane = threadIdx.x & 63;
  const int u = (lane & 3) ^ swz(lane >> 2);
  __builtin_amdgcn_global_load_lds((const void *)(row_ptr + q * 64 + u * 16), (lds_void *)dst, 16,
                                   0, 0);
}

// 32-bit LDS address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// Eight ds_read_b64_tr_b16 (see the decode kernel) issued together, in one
// asm statement that also waits for them: the compiler cannot tell that these
// reads do not alias direct-to-LDS loads still in flight and would otherwise
// wait for all of those (vmcnt(0)) before the builtin's read.  Outputs are
// early-clobber, so no address register is reused while a read is pending.
__device__ __forceinline__ void ds_read_tr8(bf16x4 (&v)[8], const uint32_t (&a)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %12\n\t"
      "ds_read_b64_tr_b16 %5, %13\n\t"
      "ds_read_b64_tr_b16 %6, %14\n\t"
      "ds_read_b64_tr_b16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
        "=&v"(v[6]), "=&v"(v[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// wait for every outstanding direct-to-LDS load); the empty asm statements
// keep the compiler from moving memory accesses across it.  Callers order
// their own loads with wait_vm / wait_lgkm0 first.
__device__ __forceinline__ void bar() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(N): at most N vector-memory operations of this wave still
// outstanding (they complete in issue order).  Other counters untouched.
template <int N> __device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

// s_waitcnt lgkmcnt(0): this wave's LDS accesses have completed.
__device__ __forceinline__ void wait_lgkm0() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);
  asm volatile("" ::: "memory");
}

// ---- reading MFMA operands from 16-row tiles --------------------------------

// S operand: the 8 values of row `row`, k-step ks (32 values) that lane
// group g feeds to the K=32 MFMA.
template <typename T>
__device__ __forceinline__ typename Frag<T>::type s_frag(const char *tile, int row, int ks, int g) {
  if constexpr (sizeof(T) == 2) {
    return *(const bf16x8 *)(tile + tile_off(row, ks * 64 + g * 16));
  } else {
    const f32x4 x = *(const f32x4 *)(tile + tile_off(row, ks * 128 + g * 32));
    const f32x4 y = *(const f32x4 *)(tile + tile_off(row, ks * 128 + g * 32 + 16));
    return (f32x8){x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  }
}

// fp32 transposed operand C^T for channels ch0..ch0+15 of the tile's keys
// 4g..4g+3: lane (g, j) receives channel ch0 + j of those four keys.
__device__ __forceinline__ f32x4 v_frag_f32(const char *tile, int ch0, int g, int j) {
  f32x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = *(const float *)(tile + tile_off(4 * g + e, (ch0 + j) * 4));
  return v;
}

// Wait until at most `after` stages issued after the current one are still
// in flight (each wave issues LPW loads per stage; loads complete in order).
template <int N> constexpr int capped() { return N < 63 ? N : 63; }
template <int LPW> __device__ __forceinline__ void wait_stages(int after) {
  switch (after) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<capped<LPW>()>(); break;
    case 2: wait_vm<capped<2 * LPW>()>(); break;
    case 3: wait_vm<capped<3 * LPW>()>(); break;
    case 4: wait_vm<capped<4 * LPW>()>(); break;
    case 5: wait_vm<capped<5 * LPW>()>(); break;
    case 6: wait_vm<capped<6 * LPW>()>(); break;
    default: wait_vm<capped<7 * LPW>()>(); break;
  }
}

// ---- handing partial results between workgroups of one kernel -------------
//
// The L2 of each XCD is not coherent with the others', so a workgroup's plain
// stores are not visible to a workgroup on another XCD until the L2 is
// written back (what a release fence does, for the whole L2 at once: far too
// costly per workgroup).  Partial results are therefore stored and loaded
// with the sc1 cache policy -- the accesses the memory model uses for
// agent-scope atomics, coherent across XCDs -- as 16-byte buffer accesses
// (coalesced, unlike per-lane atomics).  Protocol: the writer stores with
// st_coh, waits for its stores (__syncthreads waits for them), then bumps a
// counter with ctr_add; the workgroup that brings the counter to its final
// value loads the partials with ld_coh.
constexpr int kCoherent = 16;   // cache policy bits: sc1

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, bytes, 0x00020000);
}
__device__ __forceinline__ void st_coh4(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kCoherent);
}
__device__ __forceinline__ f32x4 ld_coh4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherent));
}
__device__ __forceinline__ void st_coh1(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, kCoherent);
}
__device__ __forceinline__ float ld_coh1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kCoherent));
}
__device__ __forceinline__ int ctr_add(int *p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Raise a kernel's dynamic-LDS limit to everything its static LDS leaves of
// the CU's 160 KB, once per instantiation (thread-safe static
// initialisation), so that launches made later -- possibly under graph
// capture -- issue nothing but the launch.  A failure here is cleared so it
// cannot be mistaken for a launch error; the launch itself then reports it.
template <auto Kernel> void allow_lds() {
  static const bool once = [] {
    hipFuncAttributes attr;
    size_t stat = 0;
    if (hipFuncGetAttributes(&attr, (const void *)Kernel) == hipSuccess) stat = attr.sharedSizeBytes;
    if (hipFuncSetAttribute((const void *)Kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)(160 * 1024 - stat)) != hipSuccess)
      (void)hipGetLastError();
    return true;
  }();
  (void)once;
}

// Launch a kernel taking one argument struct; when ev0/ev1 are given, the
// runtime stamps them with the kernel's own start and end (hipExtLaunchKernel:
// no separate marker packets, so nothing is added between kernels).
template <class Args>
hipError_t launch_timed(const void *kernel, dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                        Args *args, hipEvent_t ev0, hipEvent_t ev1) {
  void *argv[] = {(void *)args};
  if (ev0 || ev1) {
    const hipError_t e = hipExtLaunchKernel(kernel, grid, block, argv, lds, stream, ev0, ev1, 0);
    if (e != hipSuccess) return e;
    return hipGetLastError();
  }
  const hipError_t e = hipLaunchKernel(kernel, grid, block, argv, lds, stream);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace mtla
