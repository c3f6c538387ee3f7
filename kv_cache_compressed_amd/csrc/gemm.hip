// Dense NT products C = A B^T on gfx950 MFMA, with fused epilogues for the
// MTLA projections and the hyper-network gate.
//
// Tiling: a workgroup of 4 waves owns a BM x BN output tile; the waves are
// arranged WGM x WGN and each computes (BM/WGM) x (BN/WGN) with 16x16 MFMA
// tiles.  K advances 32 elements at a time through two LDS buffers: while a
// step is multiplied out of one buffer, the next step's A and B chunks are
// already in flight from global memory into registers, then stored to the
// other buffer (one barrier per step).  LDS rows are padded by 16 bytes so
// that the 16 rows a fragment read touches fall in distinct banks.
//
// B may be split in two row segments (rows < N1 from B1, the rest from B2) so
// one launch can produce the latent c = X W_dkv^T and the absorbed queries
// q~ = X A^T from a single pass over X.

#include "common.h"
#include "kernels.h"

namespace mtla {

namespace {

constexpr int BK = 32;

template <typename T, int BM, int BN, int WGM, int WGN, class Epi>
__global__ __launch_bounds__(256) void gemm_nt_kernel(const T *__restrict__ A, int lda,
                                                      const T *__restrict__ B1,
                                                      const T *__restrict__ B2, int N1, int ldb,
                                                      int M, int N, int K, Epi epi) {
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int EPC = 16 / sizeof(T);          // elements per 16-byte chunk
  constexpr int CPR = BK / EPC;                // chunks per tile row
  constexpr int ROWB = BK * sizeof(T) + 16;    // padded LDS row bytes
  constexpr int ACH = BM * CPR, BCH = BN * CPR;
  constexpr int ALD = (ACH + 255) / 256, BLD = (BCH + 255) / 256;
  static_assert(WGM * WGN == 4, "four waves");
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile");

  __shared__ __attribute__((aligned(16))) char smem[2][(BM + BN) * ROWB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int wm0 = (wave / WGN) * WM, wn0 = (wave % WGN) * WN;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const T *Bseg = n0 < N1 ? B1 + (size_t)n0 * ldb : B2 + (size_t)(n0 - N1) * ldb;

  u32x4 ra[ALD], rb[BLD];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < ALD; ++i) {
      int idx = tid + 256 * i;
      ra[i] = (u32x4){0u, 0u, 0u, 0u};
      if (idx < ACH) {
        int row = idx / CPR, ch = idx % CPR;
        if (m0 + row < M) ra[i] = ldg16(A + (size_t)(m0 + row) * lda + k0 + ch * EPC);
      }
    }
#pragma unroll
    for (int i = 0; i < BLD; ++i) {
      int idx = tid + 256 * i;
      rb[i] = (u32x4){0u, 0u, 0u, 0u};
      if (idx < BCH) {
        int row = idx / CPR, ch = idx % CPR;
        if (n0 + row < N) rb[i] = ldg16(Bseg + (size_t)row * ldb + k0 + ch * EPC);
      }
    }
  };
  auto stash = [&](int buf) {
    char *base = smem[buf];
#pragma unroll
    for (int i = 0; i < ALD; ++i) {
      int idx = tid + 256 * i;
      if (idx < ACH) sts16(base + (idx / CPR) * ROWB + (idx % CPR) * 16, ra[i]);
    }
#pragma unroll
    for (int i = 0; i < BLD; ++i) {
      int idx = tid + 256 * i;
      if (idx < BCH) sts16(base + (BM + idx / CPR) * ROWB + (idx % CPR) * 16, rb[i]);
    }
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  fetch(0);
  stash(0);
  __syncthreads();
  int buf = 0;
  for (int k0 = 0; k0 < K; k0 += BK) {
    const bool more = k0 + BK < K;
    if (more) fetch(k0 + BK);
    const char *base = smem[buf];
    typename Frag<T>::type fa[TM], fb[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
      load8(fa[i], (const T *)(base + (wm0 + 16 * i + c) * ROWB + g * 8 * sizeof(T)));
#pragma unroll
    for (int j = 0; j < TN; ++j)
      load8(fb[j], (const T *)(base + (BM + wn0 + 16 * j + c) * ROWB + g * 8 * sizeof(T)));
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mma_k32(fa[i], fb[j], acc[i][j]);
    if (more) stash(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = n0 + wn0 + 16 * j + c;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + wm0 + 16 * i + 4 * g + e;
        if (m < M && n < N) epi(m, n, acc[i][j][e]);
      }
    }
}

// ---- epilogues ---------------------------------------------------------------

template <typename T> struct EpiStore {
  T *out;
  int ldc;
  __device__ void operator()(int m, int n, float v) const { out[(size_t)m * ldc + n] = from_f32<T>(v); }
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

template <typename T> struct EpiLatentQuery {
  float *c_f32;
  T *c_T;
  T *qt;
  int r, HR;
  __device__ void operator()(int m, int n, float v) const {
    if (n < r) {
      c_f32[(size_t)m * r + n] = v;
      c_T[(size_t)m * r + n] = from_f32<T>(v);
    } else {
      qt[(size_t)m * HR + (n - r)] = from_f32<T>(v);
    }
  }
};

template <typename T> struct EpiGatePrefill {
  const float *c_f32;
  const T *b_hc;
  const float *table;
  float *U;
  int r, T_len, s;
  __device__ void operator()(int m, int n, float v) const {
    const int i = m % T_len, j = i / s;
    const float g = (v + to_f32(b_hc[n])) * table[(size_t)j * r + n];
    U[(size_t)m * r + n] = sigmoidf(g) * c_f32[(size_t)m * r + n];
  }
};

template <typename T> struct EpiGateMerge {
  const float *c_f32;
  const T *b_hc;
  const float *table;
  const int32_t *pos;
  T *cache;
  const T *KR;
  int64_t bstride;
  int r, dR, s;
  __device__ void operator()(int b, int n, float v) const {
    const int t = pos[b], j = t / s;
    const float g = (v + to_f32(b_hc[n])) * table[(size_t)j * r + n];
    const float u = sigmoidf(g) * c_f32[(size_t)b * r + n];
    T *slot = cache + (size_t)b * bstride + (size_t)j * (r + dR);
    const float prev = (t % s == 0) ? 0.0f : to_f32(slot[n]);
    slot[n] = from_f32<T>(prev + u);
    if (n < dR) slot[r + n] = KR[(size_t)b * dR + n];
  }
};

// ---- dispatch ------------------------------------------------------------------

template <typename T, class Epi>
hipError_t run_gemm(const T *A, int lda, const T *B1, const T *B2, int N1, int ldb, int M, int N,
                    int K, Epi epi, hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (M <= 32) {
    dim3 grid((N + 63) / 64, (M + 31) / 32);
    hipLaunchKernelGGL((gemm_nt_kernel<T, 32, 64, 1, 4, Epi>), grid, dim3(256), 0, stream, A, lda,
                       B1, B2, N1, ldb, M, N, K, epi);
  } else if (M <= 128) {
    dim3 grid((N + 63) / 64, (M + 127) / 128);
    hipLaunchKernelGGL((gemm_nt_kernel<T, 128, 64, 4, 1, Epi>), grid, dim3(256), 0, stream, A, lda,
                       B1, B2, N1, ldb, M, N, K, epi);
  } else if (sizeof(T) == 4) {
    // fp32 tiles of 128 x 128 would need more than 64 KB of static LDS.
    dim3 grid((N + 63) / 64, (M + 127) / 128);
    hipLaunchKernelGGL((gemm_nt_kernel<T, 128, 64, 4, 1, Epi>), grid, dim3(256), 0, stream, A, lda,
                       B1, B2, N1, ldb, M, N, K, epi);
  } else {
    dim3 grid((N + 127) / 128, (M + 127) / 128);
    hipLaunchKernelGGL((gemm_nt_kernel<T, 128, 128, 2, 2, Epi>), grid, dim3(256), 0, stream, A,
                       lda, B1, B2, N1, ldb, M, N, K, epi);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t latent_query_t(const void *X, int M, int d, const void *W_dkv, int r, const void *A,
                          int HR, float *c_f32, void *c_T, void *qt, hipStream_t stream) {
  EpiLatentQuery<T> epi{c_f32, (T *)c_T, (T *)qt, r, HR};
  return run_gemm<T>((const T *)X, d, (const T *)W_dkv, (const T *)A, r, d, M, r + HR, d, epi,
                     stream);
}

}  // namespace

hipError_t launch_gemm_store(int dtype, const void *A, int lda, const void *Bm, int ldb, int M,
                             int N, int K, void *out, int ldc, hipStream_t stream) {
  if (dtype == 1)
    return run_gemm<bf16>((const bf16 *)A, lda, (const bf16 *)Bm, (const bf16 *)Bm, N, ldb, M, N,
                          K, EpiStore<bf16>{(bf16 *)out, ldc}, stream);
  return run_gemm<float>((const float *)A, lda, (const float *)Bm, (const float *)Bm, N, ldb, M, N,
                         K, EpiStore<float>{(float *)out, ldc}, stream);
}

hipError_t launch_pos_table(int dtype, const void *pe, int rows, int d_pe, const void *W_hp,
                            const void *b_hp, int r, float *table, hipStream_t stream) {
  EpiBiasF32 epi{table, b_hp, dtype == 1, r};
  if (dtype == 1)
    return run_gemm<bf16>((const bf16 *)pe, d_pe, (const bf16 *)W_hp, (const bf16 *)W_hp, r, d_pe,
                          rows, r, d_pe, epi, stream);
  return run_gemm<float>((const float *)pe, d_pe, (const float *)W_hp, (const float *)W_hp, r, d_pe,
                         rows, r, d_pe, epi, stream);
}

hipError_t launch_latent_query(int dtype, const void *X, int M, int d, const void *W_dkv, int r,
                               const void *A, int HR, float *c_f32, void *c_T, void *qt,
                               hipStream_t stream) {
  if (dtype == 1) return latent_query_t<bf16>(X, M, d, W_dkv, r, A, HR, c_f32, c_T, qt, stream);
  return latent_query_t<float>(X, M, d, W_dkv, r, A, HR, c_f32, c_T, qt, stream);
}

hipError_t launch_gate_prefill(int dtype, const void *c_T, const float *c_f32, int M, int r,
                               const void *W_hc, const void *b_hc, const float *table, int T,
                               int s, float *U, hipStream_t stream) {
  if (dtype == 1) {
    EpiGatePrefill<bf16> epi{c_f32, (const bf16 *)b_hc, table, U, r, T, s};
    return run_gemm<bf16>((const bf16 *)c_T, r, (const bf16 *)W_hc, (const bf16 *)W_hc, r, r, M, r,
                          r, epi, stream);
  }
  EpiGatePrefill<float> epi{c_f32, (const float *)b_hc, table, U, r, T, s};
  return run_gemm<float>((const float *)c_T, r, (const float *)W_hc, (const float *)W_hc, r, r, M,
                         r, r, epi, stream);
}

hipError_t launch_gate_merge(int dtype, const void *c_T, const float *c_f32, int B, int r, int dR,
                             const void *W_hc, const void *b_hc, const float *table,
                             const int32_t *pos, int s, void *cache, int64_t batch_stride,
                             const void *KR_t, hipStream_t stream) {
  if (dtype == 1) {
    EpiGateMerge<bf16> epi{c_f32, (const bf16 *)b_hc, table, pos, (bf16 *)cache,
                           (const bf16 *)KR_t, batch_stride, r, dR, s};
    return run_gemm<bf16>((const bf16 *)c_T, r, (const bf16 *)W_hc, (const bf16 *)W_hc, r, r, B, r,
                          r, epi, stream);
  }
  EpiGateMerge<float> epi{c_f32, (const float *)b_hc, table, pos, (float *)cache,
                          (const float *)KR_t, batch_stride, r, dR, s};
  return run_gemm<float>((const float *)c_T, r, (const float *)W_hc, (const float *)W_hc, r, r, B,
                         r, r, epi, stream);
}

}  // namespace mtla
