// Large bf16 NT products C = A B^T on gfx950 MFMA (the projections of the
// parallel form: many thousands of rows), with the fused epilogues of
// gemm_common.h.
//
// A workgroup of 4 waves owns a 256 x 256 output tile, one workgroup per
// compute unit, and each wave a 128 x 128 quarter: 64 accumulator tiles of
// 16 x 16 (256 registers, held in AGPRs -- this file is built without the
// flag that keeps accumulators in ordinary VGPRs).  Each 16-byte operand
// fragment read from LDS then feeds 8 products (32 flops per LDS byte per
// operand), against 4 in a 64 x 64 wave tile, which left the older kernel
// bound by LDS bandwidth.
//
// K advances 32 at a time through a ring of 4 LDS stages (32 KB each: the
// 256 A rows and 256 B rows of the step, as 16-row tiles in the swizzled
// layout of common.h) filled by direct global->LDS loads.  Stage k+1's
// fragments are read into the second register set while the products of
// stage k run, so the products never wait on LDS; one barrier per stage.

#include "common.h"
#include "gemm_common.h"

#ifndef MTLA_GEMM_BIG_MIN_K
#define MTLA_GEMM_BIG_MIN_K 512
#endif

namespace mtla {

namespace {

constexpr int GB_TILE = 1024;                    // 16 rows x 64 bytes
constexpr int GB_ROWT = 256 / 16;                // 16-row tiles of A (and of B) per stage
constexpr int GB_STAGE = 2 * GB_ROWT * GB_TILE;  // 32 KB
constexpr int GB_NST = 4;
constexpr int GB_LPW = 2 * GB_ROWT / 4;          // loads per wave per stage
constexpr int GB_LDS = GB_NST * GB_STAGE;

typedef bf16x8 GbFrag[8];
typedef __attribute__((address_space(3))) bf16x4 gb_lds_b4;

template <class Epi>
__global__ __launch_bounds__(256, 1) void gemm_big_kernel(const bf16 *__restrict__ A, int lda,
                                                          BSeg bs, int M, int N, int K, Epi epi) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int wm = wave >> 1, wn = wave & 1;

  // Workgroups go round-robin to the 8 XCDs; when the tile count allows,
  // XCD x takes a contiguous run of tiles in row-major order, so the column
  // tiles sharing an A row block run together on one L2.
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
  const int m0 = tm * 256, n0 = tn * 256;

  // This wave's loads of a stage: block blk = wave + 4 i is A row tile blk
  // (blk < 16) or B row tile blk - 16; lane l copies row l/4 of the tile.
  // Rows past M or N read the last row (valid memory; never stored).
  const char *rp[GB_LPW];
#pragma unroll
  for (int i = 0; i < GB_LPW; ++i) {
    const int blk = wave + 4 * i;
    if (blk < GB_ROWT) {
      const int row = min(m0 + 16 * blk + (lane >> 2), M - 1);
      rp[i] = (const char *)(A + (size_t)row * lda);
    } else {
      const int row = min(n0 + 16 * (blk - GB_ROWT) + (lane >> 2), N - 1);
      rp[i] = (const char *)bs.row<bf16>(row);
    }
  }
  auto issue = [&](int kt) {
    char *sb = smem + (kt % GB_NST) * GB_STAGE;
#pragma unroll
    for (int i = 0; i < GB_LPW; ++i) dma_block(rp[i] + kt * 64, 0, sb + (wave + 4 * i) * GB_TILE);
  };
  // Fragments of stage kt: A row tiles 8 wm + i, B row tiles 8 wn + j; lane
  // (g, c) holds row c, k 8 g .. 8 g + 7 of the stage.
  auto frags = [&](int kt, GbFrag &fa, GbFrag &fb) {
    const char *sb = smem + (kt % GB_NST) * GB_STAGE + tile_off(c, g * 16);
#pragma unroll
    for (int i = 0; i < 8; ++i) fa[i] = *(const bf16x8 *)(sb + (8 * wm + i) * GB_TILE);
#pragma unroll
    for (int j = 0; j < 8; ++j) fb[j] = *(const bf16x8 *)(sb + (GB_ROWT + 8 * wn + j) * GB_TILE);
  };

  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int KT = K / 32;
  const int pro = min(GB_NST, KT);
  for (int kt = 0; kt < pro; ++kt) issue(kt);
  int last = pro - 1;
  // Stages 0 and 1 resident before the first barrier.
  wait_stages<GB_LPW>(last - min(1, KT - 1));
  bar();
  GbFrag fa0, fb0, fa1, fb1;
  frags(0, fa0, fb0);
  // Nothing from LDS may be in flight at the loop head: the compiler merges
  // the loop entry with the back edge there, and reads still pending from
  // the entry made it wait for every LDS read, including the next stage's,
  // before the products of each even stage.
  wait_lgkm0();
  // Every wave has read stage 0 before iteration 0 refills its slot.
  bar();

  // Iteration kt: refill the slot of stage kt (its fragments were read in
  // iteration kt-1, before the last barrier) with stage kt + NST; read stage
  // kt+1's fragments (resident and visible since that barrier); the 64
  // products of stage kt; stage kt+2 resident, then the barrier.
  auto iter = [&](int kt, GbFrag &fa, GbFrag &fb, GbFrag &na, GbFrag &nb) {
    const bool refill = kt + GB_NST < KT;
    if (refill) last = kt + GB_NST;
    if (kt + 1 < KT) frags(kt + 1, na, nb);
    // The refill's 8 loads go one per row of 8 products, so that a wave (the
    // only one on its SIMD) never holds the matrix core idle behind a burst
    // of load issues.
    char *rs = smem + (kt % GB_NST) * GB_STAGE;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (refill) dma_block(rp[i] + (kt + GB_NST) * 64, 0, rs + (wave + 4 * i) * GB_TILE);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = mma_k32(fb[j], fa[i], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (kt + 2 < KT) wait_stages<GB_LPW>(last - (kt + 2));
    // Stage kt+1's fragments are in registers before its slot can be refilled.
    wait_lgkm0();
    bar();
  };
  // KT is even (K is a multiple of 64): the two register sets alternate.
  for (int kt = 0; kt < KT; kt += 2) {
    iter(kt, fa0, fb0, fa1, fb1);
    iter(kt + 1, fa1, fb1, fa0, fb0);
  }

  // The products are C^T tiles (B rows as the A operand): lane (g, c) holds
  // row 16 i + c and the four consecutive columns 16 j + 4 g .. + 3 of the
  // wave's quarter.  Stored like that, each store instruction would write
  // 32-byte pieces of 16 rows.  Instead each wave passes its rows through
  // its own LDS block (the ring is free after the last barrier), 16 at a
  // time: written in the product layout, read back so that 32 lanes cover
  // one row's 128 columns, and stored as whole row runs.  Rows are padded to
  // 528 bytes so that the 16 rows of a write fall in distinct banks.  A
  // wave's LDS accesses complete in order, so no barrier is needed.
  constexpr int SROW = 528;
  char *stg = smem + wave * 16 * SROW;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) *(f32x4 *)(stg + c * SROW + (16 * j + 4 * g) * 4) = acc[i][j];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int rr = 2 * k + (lane >> 5), cc = 4 * (lane & 31);
      const f32x4 v = *(const f32x4 *)(stg + rr * SROW + cc * 4);
      const int m = m0 + 128 * wm + 16 * i + rr;
      const int n = n0 + 128 * wn + cc;
      if (m >= M) continue;
      if (n + 3 < N) {
        epi.four(m, n, v);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < N) epi(m, n + e, v[e]);
      }
    }
  }
}

// out[N1, N2] (fp32) = A[M, N1]^T B[M, N2] (bf16, rows of both operands
// indexed by the frame m, the contraction index), for the weight gradients of
// the backward.  The same tile as gemm_big_kernel -- 256 x 256 per
// workgroup, 128 x 128 per wave in AGPRs, a ring of 4 LDS stages of 32
// frames filled by direct loads, stage kt+1's fragments read while stage kt's
// products run -- except that both operands are column slices of row-major
// [M, N] arrays, so each fragment is two transposing reads (lane (g, c):
// column c of rows 4g..4g+3 of each 16-row tile; the same row order for A and
// B, so the products pair the right frames).  Frames are split over
// blockIdx.z (mchunk each); split z stores its partial product, in row order,
// into slab z of `part` (N1 x N2 floats), or into `out` when there is one
// split.  Needs N1, N2 multiples of 32 and 16-byte aligned rows.
constexpr int TB_TILE = 16 * 512;       // 16 frames x 256 columns of bf16
constexpr int TB_OP = 2 * TB_TILE;      // 32 frames of one operand
constexpr int TB_STAGE = 2 * TB_OP;     // A then B: 32 KB
constexpr int TB_NST = 4;
constexpr int TB_LPW = 2 * 2 * 8 / 4;   // 1 KB blocks per wave per stage
constexpr int TB_LDS = TB_NST * TB_STAGE;

__global__ __launch_bounds__(256, 1) void tn_big_kernel(const bf16 *__restrict__ A, int lda,
                                                        const bf16 *__restrict__ Bm, int ldb, int M,
                                                        int N1, int N2, int mchunk, float *out,
                                                        int ldo, float *part) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int wy = wave >> 1, wx = wave & 1;
  const int n1_0 = blockIdx.y * 256, n2_0 = blockIdx.x * 256;
  const int m_lo = blockIdx.z * mchunk, m_hi = min(M, m_lo + mchunk);
  // Steps of 32 frames, rounded up to even so that the two fragment sets
  // alternate in a fixed pattern; a step past the split is all masked.
  const int KT = ((m_hi - m_lo + 63) / 64) * 2;

  // This wave's 1 KB blocks of a stage: i < 4 are A's, i >= 4 B's, block
  // blk = wave + 4 (i mod 4) in [0, 16) of its operand being 16-frame tile
  // blk / 8 and 64-byte column segment blk mod 8.  Lane l copies frame l / 4
  // of the tile.  Frames past the split read its last frame and segments past
  // N the last whole one (valid memory; their products are masked or never
  // stored).
  const char *cp[TB_LPW];
  int q[TB_LPW], rt[TB_LPW], ld[TB_LPW], doff[TB_LPW];
#pragma unroll
  for (int i = 0; i < TB_LPW; ++i) {
    const int blk = wave + 4 * (i & 3);
    const bool isb = i >= 4;
    const int N = isb ? N2 : N1, n0 = isb ? n2_0 : n1_0;
    rt[i] = blk >> 3;
    q[i] = min(blk & 7, (N - n0) / 32 - 1);   // source segment (clamped)
    ld[i] = isb ? ldb : lda;
    cp[i] = (const char *)((isb ? Bm : A) + n0);
    doff[i] = (isb ? TB_OP : 0) + rt[i] * TB_TILE + (blk & 7) * 1024;   // the block's own slot
  }
  auto issue = [&](int kt) {
    char *sb = smem + (kt % TB_NST) * TB_STAGE;
#pragma unroll
    for (int i = 0; i < TB_LPW; ++i) {
      const int m = min(m_lo + 32 * kt + 16 * rt[i] + (lane >> 2), m_hi - 1);
      dma_block(cp[i] + (size_t)m * ld[i] * 2, q[i], sb + doff[i]);
    }
  };
  // Fragments of stage kt: A columns 128 wy + 16 i, B columns 128 wx + 16 j;
  // in the last step, frames past the split are zeroed in both.
  auto frags = [&](int kt, GbFrag &fa, GbFrag &fb) {
    const char *sb = smem + (kt % TB_NST) * TB_STAGE;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const char *pa = sb + tile_off(4 * g + (c >> 2), (128 * wy + 16 * i + 4 * (c & 3)) * 2);
      const char *pb = sb + TB_OP + tile_off(4 * g + (c >> 2), (128 * wx + 16 * i + 4 * (c & 3)) * 2);
      const bf16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((gb_lds_b4 *)pa);
      const bf16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((gb_lds_b4 *)(pa + TB_TILE));
      const bf16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((gb_lds_b4 *)pb);
      const bf16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((gb_lds_b4 *)(pb + TB_TILE));
      fa[i] = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
      fb[i] = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    const int valid = m_hi - (m_lo + 32 * kt);
    if (valid < 32) {
      // Element e of a fragment is frame (e < 4 ? 0 : 16) + 4 g + (e mod 4):
      // clear the 16-bit halves of the frames past the split.
      u32x4 mk;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int f0 = (w < 2 ? 0 : 16) + 4 * g + 2 * (w & 1);
        mk[w] = (f0 < valid ? 0xffffu : 0u) | (f0 + 1 < valid ? 0xffff0000u : 0u);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        fa[i] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, fa[i]) & mk);
        fb[i] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, fb[i]) & mk);
      }
    }
  };

  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int pro = min(TB_NST, KT);
  for (int kt = 0; kt < pro; ++kt) issue(kt);
  int last = pro - 1;
  wait_stages<TB_LPW>(last - min(1, KT - 1));
  bar();
  GbFrag fa0, fb0, fa1, fb1;
  frags(0, fa0, fb0);
  wait_lgkm0();
  bar();   // every wave has read stage 0 before iteration 0 refills its slot

  // Iteration kt: stage kt+1's fragments into the other set, refill stage
  // kt's slot with stage kt + NST (its fragments were read in iteration
  // kt-1, before the last barrier), the 64 products of stage kt, stage kt+2
  // resident, then the barrier.
  auto iter = [&](int kt, GbFrag &fa, GbFrag &fb, GbFrag &na, GbFrag &nb) {
    const bool refill = kt + TB_NST < KT;
    if (refill) last = kt + TB_NST;
    if (kt + 1 < KT) frags(kt + 1, na, nb);
    char *rs = smem + (kt % TB_NST) * TB_STAGE;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (refill) {
        const int m = min(m_lo + 32 * (kt + TB_NST) + 16 * rt[i] + (lane >> 2), m_hi - 1);
        dma_block(cp[i] + (size_t)m * ld[i] * 2, q[i], rs + doff[i]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = mma_k32(fb[j], fa[i], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (kt + 2 < KT) wait_stages<TB_LPW>(last - (kt + 2));
    wait_lgkm0();
    bar();
  };
  for (int kt = 0; kt < KT; kt += 2) {
    iter(kt, fa0, fb0, fa1, fb1);
    iter(kt + 1, fa1, fb1, fa0, fb0);
  }

  // acc[i][j]: lane (g, c) holds n1 = 128 wy + 16 i + c and the four
  // consecutive n2 = 128 wx + 16 j + 4 g .. + 3.  Rows pass through the wave's
  // own LDS block (the ring is idle after the last barrier), 16 at a time,
  // and are stored as whole row runs.
  float *dst = gridDim.z == 1 ? out : part + (size_t)blockIdx.z * N1 * N2;
  const int ldd = gridDim.z == 1 ? ldo : N2;
  constexpr int SROW = 528;
  char *stg = smem + wave * 16 * SROW;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) *(f32x4 *)(stg + c * SROW + (16 * j + 4 * g) * 4) = acc[i][j];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int rr = 2 * k + (lane >> 5), cc = 4 * (lane & 31);
      const f32x4 v = *(const f32x4 *)(stg + rr * SROW + cc * 4);
      const int n1 = n1_0 + 128 * wy + 16 * i + rr, n2 = n2_0 + 128 * wx + cc;
      if (n1 < N1 && n2 < N2) *(f32x4 *)(dst + (size_t)n1 * ldd + n2) = v;
    }
  }
}

}  // namespace

bool tn_big_supported(int N1, int N2) {
  return N1 % 32 == 0 && N2 % 32 == 0 && ((N1 + 255) / 256) * ((N2 + 255) / 256) >= 4;
}

hipError_t launch_tn_big(const void *A, int lda, const void *Bm, int ldb, int M, int N1, int N2,
                         int mchunk, int splits, float *out, int ldo, float *part,
                         hipStream_t stream) {
  allow_lds<tn_big_kernel>();
  dim3 grid((N2 + 255) / 256, (N1 + 255) / 256, splits);
  hipLaunchKernelGGL(tn_big_kernel, grid, dim3(256), TB_LDS, stream, (const bf16 *)A, lda,
                     (const bf16 *)Bm, ldb, M, N1, N2, mchunk, out, ldo, part);
  return hipGetLastError();
}

bool gemm_big_supported(int M, int N, int K) {
  // Enough 256 x 256 tiles to fill the compute units, and K long enough
  // (512: 16 stages) that a tile's loop outweighs its epilogue, which with
  // one workgroup per compute unit overlaps nothing.  At K = 512 the input
  // projection of the parallel form (65,536 rows, 2,560 columns) takes
  // 13-30 us less than in gemm_nt_kernel; at K = 2048 the output projection
  // 172 against 206 us.
  // The column tiles must also be at least three quarters used: the
  // rotary inputs' product (N = 288) took 82 us on two 256-wide tiles against
  // 43 us in gemm_nt_kernel.
  const int ntiles = (N + 255) / 256;
  return M >= 2048 && N >= 256 && K >= MTLA_GEMM_BIG_MIN_K && K % 64 == 0 &&
         4 * N >= 3 * 256 * ntiles && (size_t)((M + 255) / 256) * ntiles >= 256;
}

template <class Epi>
hipError_t launch_gemm_big(const bf16 *A, int lda, const BSeg &bs, int M, int N, int K, Epi epi,
                           hipStream_t stream) {
  allow_lds<gemm_big_kernel<Epi>>();
  dim3 grid((N + 255) / 256, (M + 255) / 256);
  hipLaunchKernelGGL(gemm_big_kernel<Epi>, grid, dim3(256), GB_LDS, stream, A, lda, bs, M, N, K,
                     epi);
  return hipGetLastError();
}

template hipError_t launch_gemm_big<EpiStore<bf16>>(const bf16 *, int, const BSeg &, int, int, int,
                                                    EpiStore<bf16>, hipStream_t);
template hipError_t launch_gemm_big<EpiProj<bf16>>(const bf16 *, int, const BSeg &, int, int, int,
                                                   EpiProj<bf16>, hipStream_t);
template hipError_t launch_gemm_big<EpiAccF32>(const bf16 *, int, const BSeg &, int, int, int,
                                               EpiAccF32, hipStream_t);

}  // namespace mtla
