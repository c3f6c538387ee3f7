// Weight-streaming product C = X W^T for 65..128 rows of X in bf16: the
// projections of one decoding step of a large layer ([Notes] = "Multi-head
// Temporal Latent Attention" paper notes, method section: the latent,
// gate and absorbed-query maps of the current frame, and the output map).
//
// Every byte of W is read exactly once and W dwarfs X (at d = 4096 with 32
// heads of r = 512: 134 MB of weights against 1-4 MB of X), so the product is
// bound by streaming W from HBM; the 128 rows give each weight byte 128
// multiply-adds, about 40% of what the matrix cores could do in that time.
//
// One workgroup per compute unit, 8 waves in two roles:
//  * four producer waves stream the stage operands through a ring of LDS
//    stages with direct global->LDS loads of whole 128-byte lines: the
//    workgroup's 16 * NG columns of W (non-temporal: each weight line is used
//    once) and all 128 rows of X (cached: every workgroup reads them).  A
//    stage is 64 values of k; the ring holds up to 8 stages.
//  * four consumer waves each own 32 rows of the output tile and run the
//    MFMAs of the current stage from LDS.
// One barrier per stage: producers pass it once stage k has landed (their
// own loads waited for in issue order), consumers once they have finished
// reading stage k-1, whose slot the producers then refill.  Loading X by the
// consumers instead (straight into registers) was measured slower: their
// loads then wait behind the memory pipe and hold up the MFMAs.
//
// Work split: W's rows (the output columns) form G = ceil(N/16) groups of 16.
// With at least four groups per compute unit, every workgroup takes floor or
// ceil(G / #workgroups) consecutive groups over the whole of K (no partial
// sums); otherwise tiles of four groups are split over K as well, and the
// last workgroup of a tile to finish adds the fp32 partials in split order
// (deterministic; its eight waves share the tile's fragments, all loads of a
// round in flight together) before the epilogue.

#include <atomic>

#include "common.h"
#include "gemm_common.h"

namespace mtla {

namespace {

constexpr int kWeightPolicy = 2;   // non-temporal: each weight line is used once
constexpr int kMaxRing = 16;
constexpr int kMaxSplits = 8;

struct StreamArgs {
  const bf16 *X;
  int ldx;
  BSeg bs;
  int M, N, K64;        // K64 = K / 64
  int tiles, gbase, grem;   // tile t: gbase + (t < grem) groups from t gbase + min(t, grem)
  int splits, kst, nst;     // k-stages per split, LDS ring slots
  float *part;              // [splits][tiles][4][2][NG] x 64 lanes x f32x4 when splits > 1
  int *counters;            // [tiles], zero on entry when splits > 1 (zero again on exit)
  int *zero;                // ints cleared by workgroup 0 before anything else
  int nzero;
};

// LDS byte of value byte b (0..127) of row R (0..15) in a 16-row group of
// 128-byte rows: two 1 KB blocks of 8 rows, each row's eight 16-byte chunks
// permuted by XOR with the row index (R & 7).  One direct load fills a block
// when lane l copies chunk (l & 7) ^ (l >> 3) of row l >> 3 of the block.
// The MFMA operand reads (16 rows, one chunk column) then hit distinct banks.
__device__ __forceinline__ int grp_off(int R, int chunk) {
  return ((R >> 3) << 10) + ((R & 7) << 7) + ((chunk ^ (R & 7)) << 4);
}

template <int LPW> __device__ __forceinline__ void wait_ring(int after) {
  switch (after) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<capped<LPW>()>(); break;
    case 2: wait_vm<capped<2 * LPW>()>(); break;
    case 3: wait_vm<capped<3 * LPW>()>(); break;
    case 4: wait_vm<capped<4 * LPW>()>(); break;
    case 5: wait_vm<capped<5 * LPW>()>(); break;
    case 6: wait_vm<capped<6 * LPW>()>(); break;
    case 7: wait_vm<capped<7 * LPW>()>(); break;
    case 8: wait_vm<capped<8 * LPW>()>(); break;
    case 9: wait_vm<capped<9 * LPW>()>(); break;
    case 10: wait_vm<capped<10 * LPW>()>(); break;
    case 11: wait_vm<capped<11 * LPW>()>(); break;
    case 12: wait_vm<capped<12 * LPW>()>(); break;
    case 13: wait_vm<capped<13 * LPW>()>(); break;
    default: wait_vm<capped<14 * LPW>()>(); break;
  }
}

template <int NG, class Epi>
__global__ __launch_bounds__(512) void stream_gemm_kernel(StreamArgs a, Epi epi) {
  constexpr int STAGE = (8 + NG) * 2048;       // X: groups 0..7, W: groups 8..8+NG-1
  constexpr int LPW = (16 + 2 * NG + 3) / 4;   // 1 KB blocks per producer wave per stage
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;

  // Consecutive workgroups (dispatched round-robin over the XCDs) take
  // consecutive tiles of one split.  Placing each split on fixed XCDs instead
  // (so that an XCD's L2 holds only its k-range of X) was measured slower: the
  // splits then draw on the memory channels unevenly.
  const int tile = blockIdx.x % a.tiles, split = blockIdx.x / a.tiles;
  const int ng = a.gbase + (tile < a.grem);
  const int g0 = tile * a.gbase + min(tile, a.grem);
  const int st0 = split * a.kst, nstage = min(a.K64, st0 + a.kst) - st0;
  char *dummy = smem + a.nst * STAGE;

  if (a.nzero && blockIdx.x == 0)
    for (int i = tid; i < a.nzero; i += 512) a.zero[i] = 0;

  f32x4 acc[2][NG];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NG; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  if (wave >= 4) {
    // ---- producers: block q = p + 4u of every stage; blocks 0..15 are X
    // (group q/2, rows 8 (q&1) ..), the rest W (group (q-16)/2) ----
    const int p = wave - 4, i8 = lane >> 3, v = lane & 7;
    const char *src[LPW];
    int dst[LPW];
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
      const int q = p + 4 * u;
      if (u < 4) {   // q < 16
        const int m = min(16 * (q >> 1) + 8 * (q & 1) + i8, a.M - 1);
        src[u] = (const char *)(a.X + (size_t)m * a.ldx) + (size_t)st0 * 128 + ((v ^ i8) << 4);
        dst[u] = q * 1024;
        continue;
      }
      const int qq = q - 16, j = qq >> 1, h = qq & 1;
      if (qq < 2 * ng) {
        const int n = min(16 * (g0 + j) + 8 * h + i8, a.N - 1);
        src[u] = (const char *)a.bs.row<bf16>(n) + (size_t)st0 * 128 + ((v ^ i8) << 4);
        dst[u] = (8 + j) * 2048 + h * 1024;
      } else {
        src[u] = nullptr;   // no block: a load of one hot line keeps the count uniform
        dst[u] = -1;
      }
    }
    auto issue = [&](int s) {
      char *sb = smem + (s % a.nst) * STAGE;
#pragma unroll
      for (int u = 0; u < LPW; ++u) {
        if (u < 4)
          __builtin_amdgcn_global_load_lds((const void *)(src[u] + (size_t)s * 128),
                                           (lds_void *)(sb + dst[u]), 16, 0, 0);
        else if (dst[u] >= 0)
          __builtin_amdgcn_global_load_lds((const void *)(src[u] + (size_t)s * 128),
                                           (lds_void *)(sb + dst[u]), 16, 0, kWeightPolicy);
        else
          __builtin_amdgcn_global_load_lds((const void *)a.X, (lds_void *)dummy, 16, 0, 0);
      }
    };
    const int pro = min(a.nst - 1, nstage);
    for (int s = 0; s < pro; ++s) issue(s);
    for (int k = 0; k < nstage; ++k) {
      wait_ring<LPW>(min(a.nst - 2, nstage - 1 - k));
      bar();   // B(k): stage k is in LDS; every consumer is done with stage k-1
      if (k + a.nst - 1 < nstage) issue(k + a.nst - 1);
    }
  } else {
    // ---- consumers: rows 32 wave .. 32 wave + 31 against all NG groups ----
    const bool full = ng == NG;
    for (int k = 0; k < nstage; ++k) {
      wait_lgkm0();
      bar();   // B(k)
      const char *sb = smem + (k % a.nst) * STAGE;
      bf16x8 xr[2][2], fb[2][NG];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
          xr[kk][i] = *(const bf16x8 *)(sb + (2 * wave + i) * 2048 + grp_off(c, 4 * kk + g));
#pragma unroll
        for (int j = 0; j < NG; ++j)
          if (j < NG - 1 || full)
            fb[kk][j] = *(const bf16x8 *)(sb + (8 + j) * 2048 + grp_off(c, 4 * kk + g));
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int j = 0; j < NG; ++j)
          if (j < NG - 1 || full) {
            acc[0][j] = mma_k32(xr[kk][0], fb[kk][j], acc[0][j]);
            acc[1][j] = mma_k32(xr[kk][1], fb[kk][j], acc[1][j]);
          }
    }
  }

  // Fragment (w, i, j) of consumer wave w: rows 32 w + 16 i + 4 g + e, column
  // 16 (g0 + j) + c.
  auto apply = [&](int w, int i, int j, f32x4 v) {
    const int n = 16 * (g0 + j) + c;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 32 * w + 16 * i + 4 * g + e;
      if (m < a.M && n < a.N) epi(m, n, v[e]);
    }
  };
  if (a.splits == 1) {
    if (wave < 4) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NG; ++j)
          if (j < ng) apply(wave, i, j, acc[i][j]);
    }
    return;
  }
  // K split: fp32 partials in fragment order (XCD-coherent stores); the last
  // workgroup of the tile to finish adds them in split order, its eight waves
  // sharing the fragments with all loads of a round in flight together.
  constexpr int NF = 8 * NG;                    // fragments (w, i, j) per tile
  const __amdgpu_buffer_rsrc_t rp =
      make_rsrc(a.part, (uint32_t)((size_t)a.splits * a.tiles * NF * 1024));
  auto poff = [&](int sp, int f) {
    return (uint32_t)((((size_t)sp * a.tiles + tile) * NF + f) * 64 + lane) * 16;
  };
  if (wave < 4) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < NG; ++j)
        if (j < ng) st_coh4(rp, poff(split, (wave * 2 + i) * NG + j), acc[i][j]);
  }
  int *last = (int *)(dummy + 1024);
  __syncthreads();   // this workgroup's partial stores have completed
  if (tid == 0) *last = ctr_add(&a.counters[tile], 1) == a.splits - 1;
  __syncthreads();
  if (!*last) return;
  constexpr int FPW = NF / 8;                   // fragments per wave
  constexpr int RF = FPW < 2 ? FPW : 2;         // fragments per round (16 loads in flight)
  for (int f0 = 0; f0 < FPW; f0 += RF) {
    f32x4 pv[RF][kMaxSplits];
#pragma unroll
    for (int r = 0; r < RF; ++r)
#pragma unroll
      for (int u = 0; u < kMaxSplits; ++u)
        pv[r][u] = ld_coh4(rp, poff(min(u, a.splits - 1), wave * FPW + min(f0 + r, FPW - 1)));
#pragma unroll
    for (int r = 0; r < RF; ++r) {
      if (f0 + r >= FPW) break;
      const int f = wave * FPW + f0 + r, w = f / (2 * NG), i = (f / NG) & 1, j = f % NG;
      if (j >= ng) continue;
      f32x4 sum = pv[r][0];
#pragma unroll
      for (int u = 1; u < kMaxSplits; ++u)
        if (u < a.splits) sum += pv[r][u];
      apply(w, i, j, sum);
    }
  }
  if (tid == 0) __hip_atomic_store(&a.counters[tile], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Compute units of the current device, looked up once per device (the plan
// is made on every call; races only ever store the same value).
int device_cus() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cus[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
    (void)hipGetLastError();
    return 256;
  }
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    n = 256;
  }
  cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <int NG, class Epi>
hipError_t stream_t(const StreamArgs &a, int grid, Epi epi, hipStream_t stream) {
  const size_t lds = (size_t)a.nst * (8 + NG) * 2048 + 1024 + 16;
  allow_lds<stream_gemm_kernel<NG, Epi>>();
  hipLaunchKernelGGL((stream_gemm_kernel<NG, Epi>), dim3(grid), dim3(512), lds, stream, a, epi);
  return hipGetLastError();
}

}  // namespace

bool stream_gemm_plan(int esz, int M, int N, int K, StreamPlan *p) {
  if (esz != 2 || M <= 64 || M > 128 || N <= 0 || K <= 0 || K % 64 != 0) return false;
  const int ncu = device_cus();
  const int G = (N + 15) / 16, K64 = K / 64;
  StreamPlan q;
  if (G >= 4 * ncu) {
    q.tiles = ncu > (G + 7) / 8 ? ncu : (G + 7) / 8;
    q.splits = 1;
  } else {
    q.tiles = (G + 3) / 4;
    int s = ncu / q.tiles;
    if (s > 8) s = 8;
    if (s > K64 / 4) s = K64 / 4;   // at least four stages per split
    q.splits = s < 1 ? 1 : s;
  }
  q.gbase = G / q.tiles;
  q.grem = G % q.tiles;
  q.ng = q.gbase + (q.grem > 0);
  if (q.ng < 1 || q.ng > 8) return false;
  q.kst = (K64 + q.splits - 1) / q.splits;
  q.splits = (K64 + q.kst - 1) / q.kst;
  const size_t stage = (size_t)(8 + q.ng) * 2048;
  int nst = (int)((158 * 1024 - 1040) / stage);
  if (nst > kMaxRing) nst = kMaxRing;
  if (nst > q.kst + 1) nst = q.kst + 1;
  if (nst < 2) nst = 2;
  q.nst = nst;
  *p = q;
  return true;
}

size_t stream_gemm_part_bytes(const StreamPlan &p) {
  return p.splits > 1 ? (size_t)p.splits * p.tiles * 8 * p.ng * 1024 : 0;
}

template <class Epi>
hipError_t launch_stream_gemm(const bf16 *X, int ldx, const BSeg &bs, int M, int N, int K,
                              const StreamPlan &p, float *part, int *counters, int *zero,
                              int nzero, Epi epi, hipStream_t stream) {
  if (p.splits > 1 && (!part || !counters)) return hipErrorInvalidValue;
  StreamArgs a;
  a.X = X;
  a.ldx = ldx;
  a.bs = bs;
  a.M = M;
  a.N = N;
  a.K64 = K / 64;
  a.tiles = p.tiles;
  a.gbase = p.gbase;
  a.grem = p.grem;
  a.splits = p.splits;
  a.kst = p.kst;
  a.nst = p.nst;
  a.part = part;
  a.counters = counters;
  a.zero = zero;
  a.nzero = zero ? nzero : 0;
  const int grid = p.tiles * p.splits;
  switch (p.ng) {
    case 1: return stream_t<1>(a, grid, epi, stream);
    case 2: return stream_t<2>(a, grid, epi, stream);
    case 3: return stream_t<3>(a, grid, epi, stream);
    case 4: return stream_t<4>(a, grid, epi, stream);
    case 5: return stream_t<5>(a, grid, epi, stream);
    case 6: return stream_t<6>(a, grid, epi, stream);
    case 7: return stream_t<7>(a, grid, epi, stream);
    case 8: return stream_t<8>(a, grid, epi, stream);
  }
  return hipErrorInvalidValue;
}

template hipError_t launch_stream_gemm<EpiProj<bf16>>(const bf16 *, int, const BSeg &, int, int,
                                                      int, const StreamPlan &, float *, int *,
                                                      int *, int, EpiProj<bf16>, hipStream_t);
template hipError_t launch_stream_gemm<EpiStore<bf16>>(const bf16 *, int, const BSeg &, int, int,
                                                       int, const StreamPlan &, float *, int *,
                                                       int *, int, EpiStore<bf16>, hipStream_t);

}  // namespace mtla
