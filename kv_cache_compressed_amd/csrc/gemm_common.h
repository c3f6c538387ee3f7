// Shared by the dense-product sources: B as up to three row segments, the
// fused epilogues, and the large-tile bf16 product of gemm_big.hip.
#pragma once

#include "common.h"

namespace mtla {

struct BSeg {
  const void *B1, *B2, *B3;
  int N1, N2;
  int ldb;
  template <typename T> __device__ __forceinline__ const T *row(int n) const {
    if (n < N1) return (const T *)B1 + (size_t)n * ldb;
    if (n < N2) return (const T *)B2 + (size_t)(n - N1) * ldb;
    return (const T *)B3 + (size_t)(n - N2) * ldb;
  }
};

// ---- epilogues: called per output element (m, n) with its fp32 value ----

template <typename T> struct EpiStore {
  T *out;
  int ldc;
  __device__ void operator()(int m, int n, float v) const { out[(size_t)m * ldc + n] = from_f32<T>(v); }
  // Columns n .. n+3 of row m (n + 3 < N, n a multiple of 4).
  __device__ void four(int m, int n, f32x4 v) const { store4f(out + (size_t)m * ldc + n, v); }
  bool four_aligned() const { return ldc % 4 == 0; }
};

// fp32 output, stored or added to what is there.
struct EpiAccF32 {
  float *out;
  int ldc;
  int add;
  __device__ void operator()(int m, int n, float v) const {
    float *p = out + (size_t)m * ldc + n;
    *p = add ? *p + v : v;
  }
  // Columns n .. n+3 of row m (n + 3 < N, n a multiple of 4).
  __device__ void four(int m, int n, f32x4 v) const {
    f32x4 *p = (f32x4 *)(out + (size_t)m * ldc + n);
    *p = add ? *p + v : v;
  }
  // The 256 x 256 tile takes stored outputs only: its epilogue, one
  // workgroup per CU, would wait out every read of an accumulation in turn.
  bool four_aligned() const { return !add && ldc % 4 == 0 && ((uintptr_t)out & 15) == 0; }
};

// bf16 output = an fp32 term already computed + the product (the last of a
// sum of products, rounded once).
struct EpiAddBf16 {
  const float *acc;
  int lda;
  bf16 *out;
  int ldc;
  __device__ void operator()(int m, int n, float v) const {
    out[(size_t)m * ldc + n] = (bf16)(acc[(size_t)m * lda + n] + v);
  }
};

struct EpiBiasF32 {
  float *out;
  const void *bias;
  int is_bf16;
  int ldc;
  __device__ void operator()(int m, int n, float v) const {
    float b = is_bf16 ? to_f32(((const bf16 *)bias)[n]) : ((const float *)bias)[n];
    out[(size_t)m * ldc + n] = v + b;
  }
};

// Columns [0, 2r): latent c and gate pre-activation, fp32 into cg [M, 2r];
// columns [2r, 2r + HR): absorbed queries into qt [M, HR] (storage type).
template <typename T> struct EpiProj {
  float *cg;
  T *qt;
  int r2, HR;
  __device__ void operator()(int m, int n, float v) const {
    if (n < r2) cg[(size_t)m * r2 + n] = v;
    else qt[(size_t)m * HR + (n - r2)] = from_f32<T>(v);
  }
  // Columns n .. n+3 of row m (n + 3 < N; r2 is a multiple of 4, so the four
  // lie on one side of it).
  __device__ void four(int m, int n, f32x4 v) const {
    if (n < r2) *(f32x4 *)(cg + (size_t)m * r2 + n) = v;
    else store4f(qt + (size_t)m * HR + (n - r2), v);
  }
  bool four_aligned() const { return r2 % 4 == 0 && HR % 4 == 0; }
};

// Large bf16 products (gemm_big.hip): C = A B^T with M, N large and K a
// multiple of 64; one workgroup of 4 waves per compute unit owns a 256 x 256
// tile, stored four columns at a time (epi.four, rows aligned to 4 values:
// epi.four_aligned()).  Instantiated for EpiStore<bf16> and EpiProj<bf16>.
bool gemm_big_supported(int M, int N, int K);

// Weight-streaming bf16 product for 65..128 rows (gemm_stream.hip): C = X W^T
// with K a multiple of 64.  The plan fixes the work split: `tiles` column
// tiles of `ng` 16-column groups (at most), each split `splits` ways over K
// (`kst` 64-wide k-stages per split) with an LDS ring of `nst` stages.  With
// splits > 1, `part` holds stream_gemm_part_bytes of fp32 partials and
// `counters` `tiles` ints that are zero on entry (and again on exit).
// `zero`: ints cleared by the kernel before anything else (may be null).
struct StreamPlan {
  int ng, tiles, gbase, grem, splits, kst, nst;
};
bool stream_gemm_plan(int esz, int M, int N, int K, StreamPlan *p);
size_t stream_gemm_part_bytes(const StreamPlan &p);
template <class Epi>
hipError_t launch_stream_gemm(const bf16 *X, int ldx, const BSeg &bs, int M, int N, int K,
                              const StreamPlan &p, float *part, int *counters, int *zero,
                              int nzero, Epi epi, hipStream_t stream);
template <class Epi>
hipError_t launch_gemm_big(const bf16 *A, int lda, const BSeg &bs, int M, int N, int K, Epi epi,
                           hipStream_t stream);

}  // namespace mtla
