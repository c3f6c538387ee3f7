// Dense NT products C = A B^T on gfx950 MFMA, with fused epilogues for the
// MTLA projections ([Notes] = "Multi-head Temporal Latent Attention" paper
// notes, method section: overall framework, hyper-network temporal merging,
// the Y formula of decoupled RoPE).
//
// Two kernels here, and gemm_big_kernel (gemm_big.hip) for large bf16
// products:
//  * gemm_nt_kernel, for many rows (the parallel form): a workgroup of 4
//    waves owns a BM x BN output tile; K advances 32 at a time through two
//    LDS buffers with register prefetch (one barrier per step); LDS rows are
//    padded by 16 bytes so the 16 rows of a fragment read hit distinct banks.
//  * skinny_gemm_kernel, for at most 128 rows (one decoding step): the
//    product is bound by reading B once, so each workgroup owns a narrow
//    column strip (16 or 32 columns) over all rows, and streams its A and B
//    tiles through a ring of LDS stages by direct global->LDS loads, several
//    stages in flight.  K may be split over workgroups; the fp32 partial
//    tiles (XCD-coherent stores) are then summed, in split order, by the
//    last workgroup of the strip to finish (atomic counter).
//
// B may consist of three row segments (rows < N1 from B1, < N2 from B2, the
// rest from B3), so that one pass over X yields the latent c = X W_dkv^T, the
// gate pre-activation X W_gate^T and the absorbed queries q~ = X A^T.

#include <type_traits>

#include "common.h"
#include "gemm_common.h"
#include "kernels.h"

namespace mtla {

namespace {

constexpr int BK = 32;


// K split over blockIdx.z: split z covers k in [z kchunk, (z+1) kchunk).
// With more than one split the fp32 partial tiles go to `part` (coherent
// stores) and the last split of a tile to finish (counter per tile, zero on
// entry and again on exit) adds them in split order and applies the epilogue.
struct KSplit {
  int kchunk;
  float *part;
  int *counters;
};

template <typename T, int BM, int BN, int WGM, int WGN, class Epi>
__global__ __launch_bounds__(256) void gemm_nt_kernel(const T *__restrict__ A, int lda, BSeg bs,
                                                      int M, int N, int K, Epi epi, KSplit ksp) {
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
  // Workgroups are dispatched round-robin over the 8 XCDs, each with its own
  // L2.  When the tile count allows, XCD x takes a contiguous run of tiles in
  // row-major order, so the column tiles that share one A row block run at
  // about the same time on one L2 instead of fetching it once per XCD.
  int tm = blockIdx.y, tn = blockIdx.x;
  {
    const int nT = gridDim.x * gridDim.y;
    if (nT % 8 == 0) {
      const int id = blockIdx.y * gridDim.x + blockIdx.x;
      const int t = (id % 8) * (nT / 8) + id / 8;
      tm = t / gridDim.x;
      tn = t % gridDim.x;
    }
  }
  const int m0 = tm * BM, n0 = tn * BN;

  const T *brow[BLD];
#pragma unroll
  for (int i = 0; i < BLD; ++i) {
    const int idx = tid + 256 * i, row = idx / CPR;
    brow[i] = (idx < BCH && n0 + row < N) ? bs.row<T>(n0 + row) : nullptr;
  }

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
      if (brow[i]) rb[i] = ldg16(brow[i] + k0 + (idx % CPR) * EPC);
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

  const int nsplit = gridDim.z;
  const int kb = blockIdx.z * ksp.kchunk, ke = min(K, kb + ksp.kchunk);
  fetch(kb);
  stash(0);
  __syncthreads();
  int buf = 0;
  for (int k0 = kb; k0 < ke; k0 += BK) {
    const bool more = k0 + BK < ke;
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

  auto apply = [&](int i, int j, f32x4 v) {
    const int n = n0 + wn0 + 16 * j + c;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = m0 + wm0 + 16 * i + 4 * g + e;
      if (m < M && n < N) epi(m, n, v[e]);
    }
  };
  if (nsplit == 1) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) apply(i, j, acc[i][j]);
    return;
  }
  // Partials in fragment order: [split][tile][wave][i][j][lane] x 16 bytes.
  const int ntile = gridDim.x * gridDim.y, tile = tm * gridDim.x + tn;
  const __amdgpu_buffer_rsrc_t rp =
      make_rsrc(ksp.part, (uint32_t)((size_t)nsplit * ntile * BM * BN * 4));
  auto poff = [&](int sp, int i, int j) {
    return (uint32_t)((((((size_t)sp * ntile + tile) * 4 + wave) * TM + i) * TN + j) * 64 + lane) * 16;
  };
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) st_coh4(rp, poff(blockIdx.z, i, j), acc[i][j]);
  __shared__ int last;
  __syncthreads();   // this workgroup's partial stores have completed
  if (tid == 0) last = ctr_add(&ksp.counters[tile], 1) == nsplit - 1;
  __syncthreads();
  if (!last) return;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      for (int s0 = 0; s0 < nsplit; s0 += 8) {
        f32x4 pv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) pv[u] = ld_coh4(rp, poff(min(s0 + u, nsplit - 1), i, j));
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (s0 + u < nsplit) v += pv[u];
      }
      apply(i, j, v);
    }
  if (tid == 0) __hip_atomic_store(&ksp.counters[tile], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- skinny products (rows <= 128) -------------------------------------------

template <typename T> struct SkinnyCfg {
  static constexpr int ES = (int)sizeof(T);
  static constexpr int SK = 128 / ES / 32 * 2;   // 32-wide k-steps per stage (256-byte rows)
  static constexpr int RB = SK * 32 * ES, NSEG = RB / 64, TILE_B = 16 * RB;
};

struct SkinnyArgs {
  const void *X;
  int ldx;
  BSeg bs;
  int M, N, KS;         // KS = K / 32
  int kps, ksplit, nst; // k-steps per split, splits, ring stages
  float *part;          // split partials when ksplit > 1: [ksplit][strip][tile][lane] f32x4
  int *counters;        // [strips], zero on entry when ksplit > 1 (zero again on exit)
  int *zero;            // ints cleared by workgroup (0, 0) before anything else
  int nzero;
};

template <typename T, int BM, int NT, class Epi>
__global__ __launch_bounds__(256) void skinny_gemm_kernel(SkinnyArgs a, Epi epi) {
  using C = SkinnyCfg<T>;
  constexpr int XG = BM / 16, NG = NT / 16, OT = XG * NG;
  constexpr int WPT = OT >= 4 ? 1 : 4 / OT, OTW = OT >= 4 ? OT / 4 : 1;
  constexpr int STAGE_B = (XG + NG) * C::TILE_B;
  constexpr int NBLK = (XG + NG) * C::NSEG, LPW = (NBLK + 3) / 4;
  static_assert(OT >= 4 ? OT % 4 == 0 : 4 % OT == 0, "tile split");
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int strip = blockIdx.x, split = blockIdx.y;
  const int n0 = strip * NT;
  if (a.nzero && strip == 0 && split == 0)
    for (int i = tid; i < a.nzero; i += 256) a.zero[i] = 0;
  const int ks0 = split * a.kps, ks1 = min(a.KS, ks0 + a.kps);
  const int nstage = (ks1 - ks0 + C::SK - 1) / C::SK;
  char *dummy = smem + a.nst * STAGE_B;

  // Row pointers of the rows this lane copies, one per 16-row group.
  const char *xrow[XG], *wrow[NG];
#pragma unroll
  for (int i = 0; i < XG; ++i)
    xrow[i] = (const char *)((const T *)a.X + (size_t)min(16 * i + (lane >> 2), a.M - 1) * a.ldx);
#pragma unroll
  for (int i = 0; i < NG; ++i)
    wrow[i] = (const char *)a.bs.row<T>(min(n0 + 16 * i + (lane >> 2), a.N - 1));

  auto issue = [&](int sidx) {
    char *sb = smem + (sidx % a.nst) * STAGE_B;
    const int kst = ks0 + sidx * C::SK;      // first k-step of the stage
    const size_t koff = (size_t)kst * 32 * C::ES;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int blk = wave + 4 * i;
      const int grp = blk / C::NSEG, q = blk % C::NSEG;
      // a block is real if it exists and its k-step lies inside the split
      const bool real = blk < NBLK && kst + (q * 64) / (32 * C::ES) < ks1;
      const char *rp = grp < XG ? xrow[grp < XG ? grp : 0] : wrow[grp - XG < NG ? grp - XG : 0];
      dma_block(rp + (real ? koff : 0), real ? q : 0, real ? sb + grp * C::TILE_B + q * 1024 : dummy);
    }
  };

  f32x4 acc[OTW];
#pragma unroll
  for (int i = 0; i < OTW; ++i) acc[i] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int pro = min(a.nst, nstage);
  for (int k = 0; k < pro; ++k) issue(k);
  const int ot0 = OT >= 4 ? wave : wave % OT;   // first output tile of this wave
  const int kpar = OT >= 4 ? 0 : wave / OT;     // k-step parity class when sharing a tile
  for (int k = 0; k < nstage; ++k) {
    const int after = min(a.nst - 1, nstage - 1 - k);
    constexpr int A1 = LPW, A2 = 2 * LPW < 63 ? 2 * LPW : 63, A3 = 3 * LPW < 63 ? 3 * LPW : 63;
    if (after >= 3) wait_vm<A3>();
    else if (after == 2) wait_vm<A2>();
    else if (after == 1) wait_vm<A1>();
    else wait_vm<0>();
    bar();
    const char *sb = smem + (k % a.nst) * STAGE_B;
    const int kst = ks0 + k * C::SK;
#pragma unroll
    for (int kk = 0; kk < C::SK; ++kk) {
      if (kk % WPT != kpar || kst + kk >= ks1) continue;
#pragma unroll
      for (int i = 0; i < OTW; ++i) {
        const int ot = ot0 + 4 * i, xi = ot / NG, ni = ot % NG;
        typename Frag<T>::type fa, fb;
        if constexpr (sizeof(T) == 2) {
          fa = *(const bf16x8 *)(sb + xi * C::TILE_B + tile_off(c, kk * 64 + g * 16));
          fb = *(const bf16x8 *)(sb + (XG + ni) * C::TILE_B + tile_off(c, kk * 64 + g * 16));
        } else {
          const char *pa = sb + xi * C::TILE_B, *pb = sb + (XG + ni) * C::TILE_B;
          const f32x4 a0 = *(const f32x4 *)(pa + tile_off(c, kk * 128 + g * 32));
          const f32x4 a1 = *(const f32x4 *)(pa + tile_off(c, kk * 128 + g * 32 + 16));
          const f32x4 b0 = *(const f32x4 *)(pb + tile_off(c, kk * 128 + g * 32));
          const f32x4 b1 = *(const f32x4 *)(pb + tile_off(c, kk * 128 + g * 32 + 16));
          fa = (f32x8){a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          fb = (f32x8){b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        }
        acc[i] = mma_k32(fa, fb, acc[i]);
      }
    }
    if (k + a.nst < nstage) {
      wait_lgkm0();
      bar();
      issue(k + a.nst);
    }
  }

  // Waves that shared an output tile add their k-step classes, in order.
  if constexpr (WPT > 1) {
    wait_lgkm0();
    bar();
    f32x4 *red = (f32x4 *)smem;   // [4 waves][64 lanes]
    red[wave * 64 + lane] = acc[0];
    __syncthreads();
    if (wave < OT) {
#pragma unroll
      for (int k = 1; k < WPT; ++k) acc[0] += red[(wave + k * OT) * 64 + lane];
    }
  }
  const bool writer = OT >= 4 || wave < OT;
  if (a.ksplit == 1) {
    if (writer) {
#pragma unroll
      for (int i = 0; i < OTW; ++i) {
        const int ot = ot0 + 4 * i, xi = ot / NG, ni = ot % NG;
        const int n = n0 + 16 * ni + c;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = 16 * xi + 4 * g + e;
          if (m < a.M && n < a.N) epi(m, n, acc[i][e]);
        }
      }
    }
    return;
  }
  // K split: partials in fragment order, XCD-coherent; the last workgroup of
  // the strip to finish adds them in split order and applies the epilogue.
  const int strips = gridDim.x;
  const __amdgpu_buffer_rsrc_t rp =
      make_rsrc(a.part, (uint32_t)((size_t)a.ksplit * strips * OT * 64 * 16));
  if (writer) {
#pragma unroll
    for (int i = 0; i < OTW; ++i) {
      const int ot = ot0 + 4 * i;
      st_coh4(rp, (uint32_t)(((((size_t)split * strips + strip) * OT + ot) * 64 + lane) * 16),
              acc[i]);
    }
  }
  int *last = (int *)smem;
  __syncthreads();   // this workgroup's partial stores have completed
  if (tid == 0) *last = ctr_add(&a.counters[strip], 1) == a.ksplit - 1;
  __syncthreads();
  if (!*last) return;
  for (int it = tid; it < OT * 64; it += 256) {
    const int ot = it / 64, ln = it % 64, xi = ot / NG, ni = ot % NG;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < a.ksplit; k0 += 8) {
      f32x4 pv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int kk = min(k0 + j, a.ksplit - 1);
        pv[j] = ld_coh4(rp, (uint32_t)(((((size_t)kk * strips + strip) * OT + ot) * 64 + ln) * 16));
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (k0 + j < a.ksplit) v += pv[j];
    }
    const int n = n0 + 16 * ni + (ln & 15);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 16 * xi + 4 * (ln >> 4) + e;
      if (m < a.M && n < a.N) epi(m, n, v[e]);
    }
  }
  if (tid == 0) __hip_atomic_store(&a.counters[strip], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// W_gate[i, k] = sum_j W_hc[i, j] W_dkv[j, k], accumulated in fp32.
template <typename T>
__global__ __launch_bounds__(256) void gate_map_kernel(const T *W_hc, const T *W_dkv, int r, int d,
                                                       T *W_gate) {
  const int k = blockIdx.x * 256 + threadIdx.x, i = blockIdx.y;
  if (k >= d) return;
  float acc = 0.0f;
  for (int j = 0; j < r; ++j) acc += to_f32(W_hc[(size_t)i * r + j]) * to_f32(W_dkv[(size_t)j * d + k]);
  W_gate[(size_t)i * d + k] = from_f32<T>(acc);
}

// ---- dispatch ------------------------------------------------------------------

template <typename T, class Epi>
hipError_t run_gemm(const T *A, int lda, const BSeg &bs, int M, int N, int K, Epi epi,
                    hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  // Stored outputs of large bf16 products take the 256 x 256 tile; fp32
  // read-modify-write epilogues stay here (they outweigh its gain).
  if constexpr (sizeof(T) == 2 && (std::is_same_v<Epi, EpiStore<bf16>> || std::is_same_v<Epi, EpiProj<bf16>> ||
                                   std::is_same_v<Epi, EpiAccF32>))
    if (gemm_big_supported(M, N, K) && epi.four_aligned())
      return launch_gemm_big(A, lda, bs, M, N, K, epi, stream);
  if (M <= 128 || sizeof(T) == 4) {
    // fp32 tiles of 128 x 128 would need more than 64 KB of static LDS.
    dim3 grid((N + 63) / 64, (M + 127) / 128);
    hipLaunchKernelGGL((gemm_nt_kernel<T, 128, 64, 4, 1, Epi>), grid, dim3(256), 0, stream, A, lda,
                       bs, M, N, K, epi, KSplit{K, nullptr, nullptr});
  } else {
    dim3 grid((N + 127) / 128, (M + 127) / 128);
    hipLaunchKernelGGL((gemm_nt_kernel<T, 128, 128, 2, 2, Epi>), grid, dim3(256), 0, stream, A,
                       lda, bs, M, N, K, epi, KSplit{K, nullptr, nullptr});
  }
  return hipGetLastError();
}


// Tiled product of at most 128 rows with K split over about 256 workgroups
// (BN = 128 for bf16, 64 for fp32); `part` holds tiled_splitk_part_bytes.
struct TiledSplit {
  int bn, tiles, splits, kchunk;
};
TiledSplit tiled_splitk_plan(int esz, int N, int K) {
  TiledSplit t;
  t.bn = esz == 2 ? 128 : 64;
  t.tiles = (N + t.bn - 1) / t.bn;
  int sp = 256 / t.tiles;
  if (sp > 8) sp = 8;
  if (sp > K / 256) sp = K / 256;   // at least 8 k-steps per split
  if (sp < 1) sp = 1;
  t.kchunk = ((K + sp - 1) / sp + BK - 1) / BK * BK;
  t.splits = (K + t.kchunk - 1) / t.kchunk;
  return t;
}

template <typename T, class Epi>
hipError_t run_gemm_splitk(const T *A, int lda, const BSeg &bs, int M, int N, int K, float *part,
                           int *counters, Epi epi, hipStream_t stream) {
  const TiledSplit t = tiled_splitk_plan((int)sizeof(T), N, K);
  const KSplit ksp{t.kchunk, part, counters};
  dim3 grid(t.tiles, 1, t.splits);
  if constexpr (sizeof(T) == 2)
    hipLaunchKernelGGL((gemm_nt_kernel<T, 128, 128, 2, 2, Epi>), grid, dim3(256), 0, stream, A,
                       lda, bs, M, N, K, epi, ksp);
  else
    hipLaunchKernelGGL((gemm_nt_kernel<T, 128, 64, 4, 1, Epi>), grid, dim3(256), 0, stream, A, lda,
                       bs, M, N, K, epi, ksp);
  return hipGetLastError();
}

template <typename T, int BM, int NT, class Epi>
hipError_t skinny_t(SkinnyArgs a, int strips, Epi epi, hipStream_t stream) {
  using C = SkinnyCfg<T>;
  constexpr size_t stage = (size_t)(BM / 16 + NT / 16) * C::TILE_B;
  const int nstage_max = (a.kps + C::SK - 1) / C::SK;
  int nst = nstage_max < 8 ? nstage_max : 8;
  while (nst > 1 && nst * stage + 1024 > 150 * 1024) --nst;
  a.nst = nst;
  size_t lds = nst * stage + 1024;
  if (lds < 4096) lds = 4096;   // room for the cross-wave reduction
  allow_lds<skinny_gemm_kernel<T, BM, NT, Epi>>();
  hipLaunchKernelGGL((skinny_gemm_kernel<T, BM, NT, Epi>), dim3(strips, a.ksplit), dim3(256), lds,
                     stream, a, epi);
  return hipGetLastError();
}

// Skinny product of M <= 128 rows: picks the row tile and column strip and,
// when `ksplit` > 1 and `part`/`counters` are given, splits K over
// workgroups.  `zero`: ints cleared at the start (may be null).
template <typename T, class Epi>
hipError_t run_skinny(const T *X, int ldx, const BSeg &bs, int M, int N, int K, int ksplit,
                      float *part, int *counters, int *zero, int nzero, Epi epi,
                      hipStream_t stream) {
  SkinnyArgs a;
  a.X = X;
  a.ldx = ldx;
  a.bs = bs;
  a.M = M;
  a.N = N;
  a.KS = K / 32;
  if (ksplit < 1 || !part || !counters) ksplit = 1;
  if (ksplit > a.KS) ksplit = a.KS;
  a.kps = (a.KS + ksplit - 1) / ksplit;
  a.ksplit = (a.KS + a.kps - 1) / a.kps;
  a.nst = 1;
  a.part = part;
  a.counters = counters;
  a.zero = zero;
  a.nzero = zero ? nzero : 0;
  if (M <= 16) return skinny_t<T, 16, 16>(a, (N + 15) / 16, epi, stream);
  if (M <= 32) return skinny_t<T, 32, 16>(a, (N + 15) / 16, epi, stream);
  if (M <= 64) return skinny_t<T, 64, 16>(a, (N + 15) / 16, epi, stream);
  return skinny_t<T, 128, 32>(a, (N + 31) / 32, epi, stream);
}

__global__ __launch_bounds__(256) void zero_kernel(int *p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

template <typename T>
hipError_t proj_t(const void *X, int M, int d, const void *W_dkv, const void *W_gate, int r,
                  const void *A, int HR, float *cg, void *qt, int *zero, int nzero,
                  hipStream_t stream) {
  EpiProj<T> epi{cg, (T *)qt, 2 * r, HR};
  BSeg bs{W_dkv, W_gate, A, r, 2 * r, d};
  const int N = 2 * r + (A ? HR : 0);
  // Up to 64 rows the strip-per-workgroup product streams the weights with
  // little else; beyond that, re-reading all of X for every narrow strip and
  // the per-tile fragment reads dominate (at 128 rows, d = 4096: 0.4 TB/s of
  // weights against 2.0 TB/s for the tiled product), so the tiled kernel
  // takes over.
  if (M <= 64)
    return run_skinny<T>((const T *)X, d, bs, M, N, d, 1, nullptr, nullptr, zero, nzero, epi,
                         stream);
  if constexpr (sizeof(T) == 2) {
    // 65..128 rows: the weight-streaming product (no K split for this shape
    // when the columns fill the compute units; it clears `zero` itself).
    StreamPlan sp;
    if (stream_gemm_plan(2, M, N, d, &sp) && sp.splits == 1)
      return launch_stream_gemm((const bf16 *)X, d, bs, M, N, d, sp, nullptr, nullptr, zero, nzero,
                                epi, stream);
  }
  if (zero && nzero > 0) {
    hipLaunchKernelGGL(zero_kernel, dim3((nzero + 255) / 256), dim3(256), 0, stream, zero, nzero);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return run_gemm<T>((const T *)X, d, bs, M, N, d, epi, stream);
}

}  // namespace

int out_proj_strips(int M, int N) {
  if (M > 128) return 0;
  return M <= 64 ? (N + 15) / 16 : (N + 31) / 32;
}

int out_proj_counters(int esz, int M, int N, int K) {
  StreamPlan sp;
  int n = out_proj_strips(M, N);
  if (stream_gemm_plan(esz, M, N, K, &sp) && sp.tiles > n) n = sp.tiles;
  return n;
}

size_t out_proj_part_bytes(int esz, int M, int N, int K) {
  if (M > 128) return 0;
  StreamPlan sp;
  if (stream_gemm_plan(esz, M, N, K, &sp)) return stream_gemm_part_bytes(sp);
  const int mpad = M <= 16 ? 16 : M <= 32 ? 32 : M <= 64 ? 64 : 128;
  if (M > 64) {
    const TiledSplit t = tiled_splitk_plan(esz, N, K);
    return t.splits > 1 ? (size_t)t.splits * t.tiles * 128 * t.bn * 4 : 0;
  }
  return (size_t)out_proj_splits(M, N, K) * mpad * (N + 32) * 4;
}

int out_proj_splits(int M, int N, int K) {
  if (M > 128) return 1;
  const int strips = out_proj_strips(M, N);
  int ks = (256 + strips - 1) / strips;   // aim at about 256 workgroups
  const int KS = K / 32;
  if (ks > KS / 8) ks = KS / 8 > 0 ? KS / 8 : 1;   // at least 8 k-steps per split
  if (ks < 1) ks = 1;
  return ks;
}

hipError_t launch_gemm_store(int dtype, const void *A, int lda, const void *Bm, int ldb, int M,
                             int N, int K, void *out, int ldc, hipStream_t stream) {
  BSeg bs{Bm, Bm, Bm, N, N, ldb};
  if (dtype == 1)
    return run_gemm<bf16>((const bf16 *)A, lda, bs, M, N, K, EpiStore<bf16>{(bf16 *)out, ldc},
                          stream);
  return run_gemm<float>((const float *)A, lda, bs, M, N, K, EpiStore<float>{(float *)out, ldc},
                         stream);
}

hipError_t launch_gemm_store2(int dtype, const void *A, int lda, const void *B1, const void *B2,
                              int N1, int ldb, int M, int N, int K, void *out, int ldc,
                              hipStream_t stream) {
  BSeg bs{B1, B2, B2, N1, N, ldb};
  if (dtype == 1)
    return run_gemm<bf16>((const bf16 *)A, lda, bs, M, N, K, EpiStore<bf16>{(bf16 *)out, ldc},
                          stream);
  return run_gemm<float>((const float *)A, lda, bs, M, N, K, EpiStore<float>{(float *)out, ldc},
                         stream);
}

hipError_t launch_gemm_f32(int dtype, const void *A, int lda, const void *Bm, int ldb, int M, int N,
                           int K, float *out, int ldc, bool add, hipStream_t stream) {
  BSeg bs{Bm, Bm, Bm, N, N, ldb};
  const EpiAccF32 epi{out, ldc, add ? 1 : 0};
  if (dtype == 1) return run_gemm<bf16>((const bf16 *)A, lda, bs, M, N, K, epi, stream);
  return run_gemm<float>((const float *)A, lda, bs, M, N, K, epi, stream);
}

hipError_t launch_gemm_add_bf16(const void *A, int lda, const void *Bm, int ldb, int M, int N, int K,
                                const float *acc, int ldacc, void *out, int ldc,
                                hipStream_t stream) {
  BSeg bs{Bm, Bm, Bm, N, N, ldb};
  return run_gemm<bf16>((const bf16 *)A, lda, bs, M, N, K,
                        EpiAddBf16{acc, ldacc, (bf16 *)out, ldc}, stream);
}

hipError_t launch_gemm_f32_2(int dtype, const void *A, int lda, const void *B1, const void *B2,
                             int N1, int ldb, int M, int N, int K, float *out, int ldc,
                             hipStream_t stream) {
  BSeg bs{B1, B2, B2, N1, N, ldb};
  const EpiAccF32 epi{out, ldc, 0};
  if (dtype == 1) return run_gemm<bf16>((const bf16 *)A, lda, bs, M, N, K, epi, stream);
  return run_gemm<float>((const float *)A, lda, bs, M, N, K, epi, stream);
}

hipError_t launch_out_proj(int dtype, const void *O, int M, int K, const void *Bvo, int N, void *Y,
                           float *part, int *counters, hipStream_t stream) {
  if (M > 128) return launch_gemm_store(dtype, O, K, Bvo, K, M, N, K, Y, N, stream);
  BSeg bs{Bvo, Bvo, Bvo, N, N, K};
  StreamPlan sp;
  if (dtype == 1 && stream_gemm_plan(2, M, N, K, &sp) && (sp.splits == 1 || (part && counters)))
    return launch_stream_gemm((const bf16 *)O, K, bs, M, N, K, sp, part, counters, nullptr, 0,
                              EpiStore<bf16>{(bf16 *)Y, N}, stream);
  if (M > 64 && part && counters) {
    // 65..128 rows: the tiled product (fragments reused across each wave's
    // block of tiles) with K split, instead of narrow strips that each read
    // all of O.
    if (dtype == 1)
      return run_gemm_splitk<bf16>((const bf16 *)O, K, bs, M, N, K, part, counters,
                                   EpiStore<bf16>{(bf16 *)Y, N}, stream);
    return run_gemm_splitk<float>((const float *)O, K, bs, M, N, K, part, counters,
                                  EpiStore<float>{(float *)Y, N}, stream);
  }
  const int ks = (part && counters) ? out_proj_splits(M, N, K) : 1;
  if (dtype == 1)
    return run_skinny<bf16>((const bf16 *)O, K, bs, M, N, K, ks, part, counters, nullptr, 0,
                            EpiStore<bf16>{(bf16 *)Y, N}, stream);
  return run_skinny<float>((const float *)O, K, bs, M, N, K, ks, part, counters, nullptr, 0,
                           EpiStore<float>{(float *)Y, N}, stream);
}

hipError_t launch_pos_table(int dtype, const void *pe, int rows, int d_pe, const void *W_hp,
                            const void *b_hp, int r, float *table, hipStream_t stream) {
  EpiBiasF32 epi{table, b_hp, dtype == 1, r};
  BSeg bs{W_hp, W_hp, W_hp, r, r, d_pe};
  if (dtype == 1) return run_gemm<bf16>((const bf16 *)pe, d_pe, bs, rows, r, d_pe, epi, stream);
  return run_gemm<float>((const float *)pe, d_pe, bs, rows, r, d_pe, epi, stream);
}

hipError_t launch_gate_map(int dtype, const void *W_hc, const void *W_dkv, int r, int d,
                           void *W_gate, hipStream_t stream) {
  dim3 grid((d + 255) / 256, r);
  if (dtype == 1)
    hipLaunchKernelGGL(gate_map_kernel<bf16>, grid, dim3(256), 0, stream, (const bf16 *)W_hc,
                       (const bf16 *)W_dkv, r, d, (bf16 *)W_gate);
  else
    hipLaunchKernelGGL(gate_map_kernel<float>, grid, dim3(256), 0, stream, (const float *)W_hc,
                       (const float *)W_dkv, r, d, (float *)W_gate);
  return hipGetLastError();
}

hipError_t launch_proj(int dtype, const void *X, int M, int d, const void *W_dkv,
                       const void *W_gate, int r, const void *A, int HR, float *cg, void *qt,
                       int *zero, int nzero, hipStream_t stream) {
  if (dtype == 1) return proj_t<bf16>(X, M, d, W_dkv, W_gate, r, A, HR, cg, qt, zero, nzero, stream);
  return proj_t<float>(X, M, d, W_dkv, W_gate, r, A, HR, cg, qt, zero, nzero, stream);
}

}  // namespace mtla
