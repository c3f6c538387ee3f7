// Parallel (prefill / training-forward) form of MTLA on gfx950: the gate and
// group scan that build the intermediate states C', and the stride-aware
// masked attention kernel.
//
// [Notes] = "Multi-head Temporal Latent Attention" paper notes (zhaoyang97
// Paper-Notes): key designs / hyper-network temporal merging, stride-aware
// causal mask and decoupled RoPE (the Y formula); [Fig2] = sciencestack.ai
// page, Figure 2 (c).
//
// Attention kernels.  Query rows are (frame m, head h) pairs, row = m*H + h.
// Row (m, h) sees the compact keys j < floor(m/s) -- the group-final states of
// the groups that ended before m, i.e. the stride-aware mask's columns
// n < m with n mod s = s-1 -- plus its own state C'_m, which seeds the online
// softmax.  The compact keys stream through a ring of LDS stages (32 keys
// each) by direct global->LDS loads, in the swizzled 16-row tile layout; the
// loop ends at the workgroup's causal frontier, so masked tiles are never
// visited.  Two kernels:
//   * prefill_attn_kernel (fp32 storage, and r = 512): a workgroup owns
//     4 * 16 * NQ consecutive rows, each wave 16 * NQ of them with their
//     queries and O^T (r x rows) accumulators in registers.  Per 16-key tile
//     a wave computes S^T = K . Q^T (K from LDS, K=32 MFMA), the online
//     softmax in log2 units (reference max moved lazily, by > 2^8), and
//     O^T += C^T . P^T (C^T by transposing LDS reads, K=16 MFMA).  Each K
//     fragment read from LDS feeds NQ products and each C^T fragment NQ more.
//   * prefill_ws_kernel (bf16, r = 256): the warp-specialised form described
//     above its definition.

#include <float.h>
#include <math.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace mtla {

namespace {

constexpr float kNegInf = -INFINITY;

// ---------------------------------------------------------------------------
// parallel form ([Notes] stride-aware causal mask; [Fig2] (c))
// ---------------------------------------------------------------------------

// One thread per (sequence b, slot j, channel): computes the gated latents
// of the s frames of group j ([Notes] hyper-network temporal merging) and
// their running sum ([Notes] stride-aware causal mask; [Fig2] (c)).
template <typename T>
__global__ __launch_bounds__(256) void group_scan_kernel(const float *cg, const T *b_hc,
                                                         const float *table, const T *KR,
                                                         int T_len, int R, int DR, int s, int nS,
                                                         T *Cp, T *keys, int64_t kstride, T *cache,
                                                         int64_t cstride) {
  // One thread per (slot j, four consecutive channels): 16-byte fp32 loads of
  // c and g, 4-value stores (R, DR and every row stride are multiples of 4).
  const int b = blockIdx.y;
  const int RK = R + DR, Q = RK / 4;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)nS * Q) return;
  const int j = (int)(idx / Q), ch = 4 * (int)(idx % Q);
  const int i0 = j * s, i1 = min(i0 + s, T_len) - 1;
  f32x4 v;
  if (ch < R) {
    const f32x4 bb = load4f(b_hc + ch), pj = *(const f32x4 *)(table + (size_t)j * R + ch);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int i = i0; i <= i1; ++i) {
      const size_t row = (size_t)b * T_len + i;
      const float *r = cg + row * 2 * R;
      const f32x4 c = *(const f32x4 *)(r + ch), g = *(const f32x4 *)(r + R + ch);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += sigmoidf((g[e] + bb[e]) * pj[e]) * c[e];
      store4f(Cp + row * R + ch, acc);
    }
    v = acc;
  } else {
    v = load4f(KR + ((size_t)b * T_len + i1) * DR + (ch - R));
  }
  store4f(keys + (size_t)b * kstride + (size_t)j * RK + ch, v);
  if (cache) store4f(cache + (size_t)b * cstride + (size_t)j * RK + ch, v);
}

struct PrefillArgs {
  const void *qt;        // [B, T, H, R]
  const void *QR;        // [B, T, H, DR]
  const char *keys;      // [B] x keys_stride: ceil(T/s) compact rows of R + DR values
  int64_t kstride_bytes;
  const void *Cp;        // [B, T, R]
  const void *KR;        // [B, T, DR]
  void *O;               // [B, T, H, R]
  int B, T, H, s, tiles, nst;
  float sl2;
};

template <typename T, int R, int DR, int NQ> struct PreCfg {
  static constexpr int RK = R + DR, ES = (int)sizeof(T), RB = RK * ES, NSEG = RB / 64;
  static constexpr int KS = RK / 32, MT = R / 16;
  static constexpr int ROWS_W = 16 * NQ, ROWS = 4 * ROWS_W;
  static constexpr int TPS = 2, SROWS = 16 * TPS;          // 32 keys per stage
  static constexpr int TILE_B = 16 * RB, STAGE_B = TPS * TILE_B;
  static constexpr int NBLK = TPS * NSEG, LPW = (NBLK + 3) / 4;
  static_assert(MT % 8 == 0, "channel blocks come in groups of 8");
};

template <typename T, int R, int DR, int NQ>
__global__ __launch_bounds__(256) void prefill_attn_kernel(PrefillArgs a) {
  using C = PreCfg<T, R, DR, NQ>;
  typedef typename Frag4<T>::type P4;
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int H = a.H, Tn = a.T, s = a.s;

  // Heavy tiles (late queries) first; when the batch splits evenly over the
  // 8 XCDs, each XCD serves whole sequences so their keys stay in its L2.
  int b, qtile;
  {
    const int bid = blockIdx.x;
    if (a.B % 8 == 0) {
      const int per = a.B / 8, xcd = bid % 8, k = bid / 8;
      qtile = a.tiles - 1 - k / per;
      b = xcd + 8 * (k % per);
    } else {
      qtile = a.tiles - 1 - bid / a.B;
      b = bid % a.B;
    }
  }
  const int nrows = Tn * H;
  const int rw = qtile * C::ROWS + wave * C::ROWS_W;   // first row of this wave

  // Queries, the self term and the initial state of every row of the wave.
  typename Frag<T>::type q[NQ][C::KS];
  f32x4 o[NQ][C::MT];
  float m[NQ], l[NQ];
  int lim[NQ];
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    // Rows past the end read row 0 (valid memory) and are never written back.
    const int row = rw + 16 * qi + c;
    const bool ok = row < nrows;
    const int rr = ok ? row : 0;
    const int mf = rr / H, h = rr % H;
    lim[qi] = ok ? mf / s : 0;
    const size_t qoff = ((size_t)b * Tn + mf) * H + h;
    const size_t coff = (size_t)b * Tn + mf;
    float dot = 0.0f;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const int k = 32 * ks + 8 * g;
      typename Frag<T>::type d;
      if (k < R) {
        load8(q[qi][ks], (const T *)a.qt + qoff * R + k);
        load8(d, (const T *)a.Cp + coff * R + k);
      } else {
        load8(q[qi][ks], (const T *)a.QR + qoff * DR + (k - R));
        load8(d, (const T *)a.KR + coff * DR + (k - R));
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) dot += to_f32(q[qi][ks][e]) * to_f32(d[e]);
    }
    m[qi] = sum_g(dot) * a.sl2;
    l[qi] = (g == 0) ? 1.0f : 0.0f;
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) o[qi][mt] = load4f((const T *)a.Cp + coff * R + 16 * mt + 4 * g);
  }
  asm volatile("" ::: "memory");

  // Keys this wave / workgroup can see at most (row limits grow with the row).
  const int wlast = min(rw + C::ROWS_W, nrows) - 1;
  const int wlim = wlast >= rw ? (wlast / H) / s : 0;
  const int glast = min(qtile * C::ROWS + C::ROWS, nrows) - 1;
  const int kmax = (glast / H) / s;
  const int nstage = (kmax + C::SROWS - 1) / C::SROWS;
  const char *src = a.keys + (size_t)b * a.kstride_bytes;
  char *dummy = smem + a.nst * C::STAGE_B;

  auto issue = [&](int sidx) {
    char *sb = smem + (sidx % a.nst) * C::STAGE_B;
    const int row0 = sidx * C::SROWS;
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) {
      const int blk = wave + 4 * i;
      const bool real = (C::NBLK % 4 == 0) || blk < C::NBLK;
      const int tl = real ? blk / C::NSEG : 0, qq = real ? blk % C::NSEG : 0;
      const int key = min(row0 + tl * 16 + (lane >> 2), kmax - 1);
      dma_block(src + (size_t)key * C::RB, qq, real ? sb + tl * C::TILE_B + qq * 1024 : dummy);
    }
  };
  const int pro = min(a.nst, nstage);
  for (int k = 0; k < pro; ++k) issue(k);
  int last = pro - 1;   // newest stage issued so far

  for (int k = 0; k < nstage; ++k) {
    // Stage k has landed once at most last - k stages issued after it are
    // still in flight (this wave's loads complete in issue order).
    wait_stages<C::LPW>(last - k);
    bar();
    // Every wave is past stage k-1 here: its ring slot can be refilled.
    if (k >= 1 && k - 1 + a.nst < nstage) {
      issue(k - 1 + a.nst);
      last = k - 1 + a.nst;
    }
    const char *sb = smem + (k % a.nst) * C::STAGE_B;
#pragma unroll
    for (int tl = 0; tl < C::TPS; ++tl) {
      const int kb = k * C::SROWS + tl * 16;
      if (kb >= wlim) continue;
      const char *tile = sb + tl * C::TILE_B;
      // S^T for the NQ row tiles; each K fragment feeds NQ products.
      f32x4 sc[NQ];
#pragma unroll
      for (int qi = 0; qi < NQ; ++qi) sc[qi] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const typename Frag<T>::type af = s_frag<T>(tile, c, ks, g);
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) sc[qi] = mma_k32(af, q[qi][ks], sc[qi]);
      }
      // Online softmax per row; the reference max moves only by steps > 2^8.
      float z[NQ][4];
      bool up_any = false;
      float mnew[NQ];
#pragma unroll
      for (int qi = 0; qi < NQ; ++qi) {
        float mx = kNegInf;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          z[qi][e] = (kb + 4 * g + e < lim[qi]) ? sc[qi][e] * a.sl2 : kNegInf;
          mx = fmaxf(mx, z[qi][e]);
        }
        mx = max_g(mx);
        const bool up = mx > m[qi] + 8.0f;
        mnew[qi] = up ? mx : m[qi];
        up_any |= up;
      }
      if (__builtin_amdgcn_ballot_w64(up_any)) {
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
          const float alpha = __builtin_amdgcn_exp2f(m[qi] - mnew[qi]);
          l[qi] *= alpha;
#pragma unroll
          for (int mt = 0; mt < C::MT; ++mt) o[qi][mt] *= alpha;
          m[qi] = mnew[qi];
        }
      }
      P4 pf[NQ];
#pragma unroll
      for (int qi = 0; qi < NQ; ++qi) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = __builtin_amdgcn_exp2f(z[qi][e] - m[qi]);
          l[qi] += p;
          pf[qi][e] = from_f32<T>(p);
        }
      }
      // O^T += C^T P^T; each C^T fragment feeds NQ products.
#pragma unroll
      for (int m0 = 0; m0 < C::MT; m0 += 8) {
        typename Frag4<T>::type vv[8];
        if constexpr (sizeof(T) == 2) {
          uint32_t ad[8];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            ad[j] = lds_addr(tile + tile_off(4 * g + (c >> 2), (16 * (m0 + j) + 4 * (c & 3)) * 2));
          ds_read_tr8(vv, ad);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) vv[j] = v_frag_f32(tile, 16 * (m0 + j), g, c);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int qi = 0; qi < NQ; ++qi) o[qi][m0 + j] = mma_k16(vv[j], pf[qi], o[qi][m0 + j]);
      }
    }
  }

  // O = O^T / l, written back row-major [B, T, H, R].
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    const float lt = sum_g(l[qi]);
    const int row = rw + 16 * qi + c;
    if (row < nrows) {
      const float inv = 1.0f / lt;
      T *dst = (T *)a.O + ((size_t)b * nrows + row) * R + 4 * g;
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) store4f(dst + 16 * mt, o[qi][mt] * inv);
    }
  }
}

template <typename T, int R, int DR, int NQ>
hipError_t prefill_attn_t(int B, int T_len, int H, int s, float sl2, const void *qt,
                          const void *QR, const void *keys, int64_t kstride, const void *Cp,
                          const void *KR, void *O, hipStream_t stream, hipEvent_t ev0,
                          hipEvent_t ev1) {
  using C = PreCfg<T, R, DR, NQ>;
  const int tiles = (T_len * H + C::ROWS - 1) / C::ROWS;
  int nst = (int)(144 * 1024 / C::STAGE_B);
  if (nst > 4) nst = 4;
  if (nst < 1) nst = 1;
  const size_t lds = (size_t)nst * C::STAGE_B + 1024;
  auto kern = prefill_attn_kernel<T, R, DR, NQ>;
  allow_lds<prefill_attn_kernel<T, R, DR, NQ>>();
  PrefillArgs args{qt, QR, (const char *)keys, kstride * C::ES, Cp, KR, O, B, T_len, H, s, tiles,
                   nst, sl2};
  return launch_timed((const void *)kern, dim3(tiles * B), dim3(256), lds, stream, &args, ev0, ev1);
}

// ---------------------------------------------------------------------------
// Warp-specialised attention for bf16 latents with r = 256, d_hR = 32: eight
// waves, two per SIMD, over the same LDS ring of compact keys.
//   Score waves 0-3 own 48 rows each (three 16-row tiles): they hold the
//   queries, compute S^T for the 32 keys of a stage (K=32 MFMAs, each K^T
//   fragment feeding three products), run the online softmax and pass the
//   bf16 probabilities P^T, the per-row rescale factors and a per-wave
//   rescale flag to the value waves through LDS.
//   Value wave v holds O^T for all 192 rows of the workgroup and the channel
//   quarter [64 v, 64 v + 64): each C^T fragment, fetched with gfx950's
//   transposing LDS read (half the bandwidth of a 16-byte read), feeds twelve
//   products, and the P^T fragments come with full-rate 16-byte reads.
// Splitting the roles splits the register state (queries vs accumulators),
// so each wave fits in half the SIMD's register file and a score wave and a
// value wave share each SIMD: one's VALU work overlaps the other's matrix
// products and each covers the other's LDS latency.  Two workgroup barriers
// per stage order the handoff and split the stage into two phases: in phase
// A the score waves run the products S^T of stage k (and tile 0's
// exponentials, threaded between tile 1's products), in phase B the rest of
// the softmax of stage k, while tile 0's K^T fragments of stage k+1 are
// fetched; the value waves spread their products for stage k-1 over both
// phases (half the row tiles each).  The 16x16x32 bf16 MFMA is used
// throughout: gfx950 runs the 16x16x16 form at half its rate.
// ---------------------------------------------------------------------------
#ifndef MTLA_WS_SPLIT
#define MTLA_WS_SPLIT 6
#endif
struct WsCfg {
  static constexpr int R = 256, DR = 32, RK = R + DR, RB = RK * 2, NSEG = RB / 64;
  static constexpr int NQ = 3, KS = RK / 32, MT = R / 16;
  static constexpr int ROWS_W = 16 * NQ, ROWS = 4 * ROWS_W;
  static constexpr int SROWS = 32, TILE_B = 16 * RB, STAGE_B = 2 * TILE_B;
  static constexpr int NBLK = 2 * NSEG, LPW = (NBLK + 3) / 4;
  static constexpr int NRT = 4 * NQ;            // 16-row tiles per workgroup
  static constexpr int NB = MT / 4;              // channel blocks per value wave
  static constexpr int P_B = NRT * 64 * 16;      // P slot: row tiles x 64 lanes x 16 B
  static constexpr int A_B = 16 * NRT * 4;       // per-row floats [lane row c][row tile]
  static constexpr int F_B = 16;                 // rescale flags of the 4 score waves
  // The rows [C'_f | K^R_f] of the workgroup's frames (RB bytes each) stay in
  // LDS for the whole workgroup when they fit SELF_B: at most SELF_FR frames
  // (every H >= 5); with fewer heads they are read per lane instead.
  static constexpr int SELF_B = 24 * 1024;
  static constexpr int SELF_FR = (SELF_B / 16) / (RB / 16);
  static constexpr int EXTRA = 2 * P_B + 3 * A_B + 2 * F_B + 1024 + SELF_B;
  // Ring depth, fixed at compile time so that slot indices need no runtime
  // division: six 18 KB stages plus the P, rescale and flag buffers fill
  // 135 KB of the 160 KB LDS.
  static constexpr int NST = 6;
  static_assert(KS == NSEG, "a K^T fragment row spans one 1 KB block per k-step");
  static_assert(NST * STAGE_B + EXTRA <= 160 * 1024, "the ring and buffers fit the LDS");
};

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// acc + sum of the 8 products x[e] y[e], in fp32 (four v_dot2_f32_bf16).
__device__ __forceinline__ float dot8(const bf16x8 &x, const bf16x8 &y, float acc) {
#pragma unroll
  for (int e = 0; e < 8; e += 2)
    acc = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){x[e], x[e + 1]}, (bf16x2){y[e], y[e + 1]}, acc,
                                          false);
  return acc;
}

__global__ __launch_bounds__(512) void prefill_ws_kernel(PrefillArgs a) {
  using C = WsCfg;
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int H = a.H, Tn = a.T, s = a.s;
  constexpr int nst = C::NST;

  int b, qtile;
  {
    const int bid = blockIdx.x;
    if (a.B % 8 == 0) {
      const int per = a.B / 8, xcd = bid % 8, k = bid / 8;
      qtile = a.tiles - 1 - k / per;
      b = xcd + 8 * (k % per);
    } else {
      qtile = a.tiles - 1 - bid / a.B;
      b = bid % a.B;
    }
  }
  const int nrows = Tn * H;
  const int w = wave & 3;
  const int rw = qtile * C::ROWS + w * C::ROWS_W;   // first row of this wave pair
  const int wlast = min(rw + C::ROWS_W, nrows) - 1;
  const int wlim = wlast >= rw ? (wlast / H) / s : 0;
  const int glast = min(qtile * C::ROWS + C::ROWS, nrows) - 1;
  const int kmax = (glast / H) / s;
  const int nstage = (kmax + C::SROWS - 1) / C::SROWS;

  char *pbase = smem + nst * C::STAGE_B;
  float *abase = (float *)(pbase + 2 * C::P_B);   // rescale factors, two slots
  float *lbuf = abase + 2 * (C::A_B / 4);          // row sums
  float *fbase = lbuf + C::A_B / 4;                // rescale flags, two slots
  char *dummy = (char *)(fbase + 2 * (C::F_B / 4));
  char *selfb = dummy + 1024;                      // the frames' rows
  float *sbuf = abase;   // after the loop: each row's self-term factor
  // Frames of the workgroup's rows: each row's own term (its score seeds the
  // softmax, its value C'_m joins the output at the end) comes from the
  // frame's row, copied once into LDS when the frames fit.
  const int f0 = (qtile * C::ROWS) / H, nfr = glast / H - f0 + 1;
  const bool self_lds = nfr <= C::SELF_FR;

  if (wave < 4) {
    // ---------------- score wave ----------------
    const char *src = a.keys + (size_t)b * a.kstride_bytes;
    auto issue = [&](int sidx) {
      char *sb = smem + (sidx % nst) * C::STAGE_B;
      const int row0 = sidx * C::SROWS;
#pragma unroll
      for (int i = 0; i < C::LPW; ++i) {
        const int blk = w + 4 * i;
        const bool real = blk < C::NBLK;
        const int tl = real ? blk / C::NSEG : 0, qq = real ? blk % C::NSEG : 0;
        const int key = min(row0 + tl * 16 + (lane >> 2), kmax - 1);
        dma_block(src + (size_t)key * C::RB, qq, real ? sb + tl * C::TILE_B + qq * 1024 : dummy);
      }
    };

    // The key stream goes out first, so that its round trip overlaps that of
    // the queries (waiting for the queries then waits for the first stages
    // too -- loads complete in order -- which the loop needs next anyway).
    const int pro = min(nst, nstage);
    for (int k = 0; k < pro; ++k) issue(k);

    bf16x8 q[C::NQ][C::KS];
    float m[C::NQ], l[C::NQ], dot[C::NQ], m0[C::NQ];
    int lim[C::NQ], fl[C::NQ];
    size_t qoff[C::NQ], coff[C::NQ];
#pragma unroll
    for (int qi = 0; qi < C::NQ; ++qi) {
      // Rows past the end read row 0 (valid memory; its frame's LDS row is
      // the workgroup's first) and are never written back.
      const int row = rw + 16 * qi + c;
      const bool ok = row < nrows;
      const int rr = ok ? row : 0;
      const int mf = rr / H, h = rr % H;
      lim[qi] = ok ? mf / s : 0;
      fl[qi] = ok ? mf - f0 : 0;
      qoff[qi] = ((size_t)b * Tn + mf) * H + h;
      coff[qi] = (size_t)b * Tn + mf;
      dot[qi] = 0.0f;
    }
    // Queries (lane group g: values 32 ks + 8 g .. + 7 of k-step ks); with
    // few heads, the rows' own states too, read per lane.
    auto load_q = [&](int qi, int ks) {
      const int k = 32 * ks + 8 * g;
      if (k < C::R)
        load8(q[qi][ks], (const bf16 *)a.qt + qoff[qi] * C::R + k);
      else
        load8(q[qi][ks], (const bf16 *)a.QR + qoff[qi] * C::DR + (k - C::R));
    };
    if (self_lds) {
#pragma unroll
      for (int qi = 0; qi < C::NQ; ++qi)
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) load_q(qi, ks);
    } else {
#pragma unroll
      for (int qi = 0; qi < C::NQ; ++qi)
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          load_q(qi, ks);
          const int k = 32 * ks + 8 * g;
          bf16x8 d;
          if (k < C::R)
            load8(d, (const bf16 *)a.Cp + coff[qi] * C::R + k);
          else
            load8(d, (const bf16 *)a.KR + coff[qi] * C::DR + (k - C::R));
          dot[qi] = dot8(q[qi][ks], d, dot[qi]);
        }
    }
    // The value waves' copy of the frames' rows has landed.
    bar();
#pragma unroll
    for (int qi = 0; qi < C::NQ; ++qi) {
      if (self_lds) {
        // Row (frame f) at (f - f0) * RB; k-step ks, lane group g: bytes
        // 64 ks + 16 g, the same offset in C' (k < R) and K^R (k >= R).
        const char *dr = selfb + fl[qi] * C::RB + 16 * g;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
          dot[qi] = dot8(q[qi][ks], *(const bf16x8 *)(dr + 64 * ks), dot[qi]);
      }
      // The row's own state seeds the softmax: weight 1 at reference max m0.
      // The value waves start from O^T = 0 and add C'_m with the factor
      // 2^(m0 - m) that the later moves of m leave on that weight.
      m[qi] = sum_g(dot[qi]) * a.sl2;
      m0[qi] = m[qi];
      l[qi] = (g == 0) ? 1.0f : 0.0f;
    }

    // Keys below wmin are visible to every row of the wave: no mask needed.
    const int wmin = rw < nrows ? ((rw / H) / s) : 0;
    int last = pro - 1;
    if (nstage > 0) wait_stages<C::LPW>(last);

    // K^T fragments of the stage about to be processed: row c of each tile,
    // this lane group's 16-byte chunk of every k-step.  Tile 0's are read one
    // phase ahead (during the previous stage's softmax) and tile 1's at the
    // start of phase A, behind tile 0's products, so that phase A issues
    // matrix products without waiting on LDS.
    bf16x8 kf0[C::KS];
    auto krow = [&](int k) { return smem + (k % nst) * C::STAGE_B + tile_off(c, g * 16); };
    auto read_k0 = [&](int k) {
      const char *row = krow(k);
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) kf0[ks] = *(const bf16x8 *)(row + ks * 1024);
    };
    for (int k = 0; k <= nstage; ++k) {
      bar();
      // Stage k-2 has been consumed by both roles: refill its slot.
      if (k >= 2 && k - 2 + nst < nstage) {
        issue(k - 2 + nst);
        last = k - 2 + nst;
      }
      const bool act = k < nstage && k * C::SROWS < wlim;
      const int kb = k * C::SROWS;
      f32x4 sc[2][C::NQ];
      // Online softmax in log2 units with a lazily moved reference max m
      // per row: p = 2^(s sl2 - m) against the current m, and only when some
      // p of the wave exceeds 2^8 (a row's maximum rose by more than 8) are
      // the exact row maxima taken and m moved to those that did.  pr holds
      // tile 0's p in [0, 4) and tile 1's in [4, 8).
      float pr[C::NQ][8];
      float pmax = 0.0f;
      bool moved = false;
      // Phase A: the products S^T of stage k, and tile 0's p while tile 1's
      // products run (needing no row maximum, they only wait for tile 0's).
      if (act) {
        if (k == 0) read_k0(0);
        bf16x8 kf1[C::KS];
        const char *row1 = krow(k) + C::TILE_B;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) kf1[ks] = *(const bf16x8 *)(row1 + ks * 1024);
        // Keep the nine reads ahead of tile 0's products (the compiler would
        // otherwise spread them out, each behind a full wait).
        asm volatile("" ::: "memory");
#pragma unroll
        for (int qi = 0; qi < C::NQ; ++qi) {
          sc[0][qi] = (f32x4){0.f, 0.f, 0.f, 0.f};
          sc[1][qi] = (f32x4){0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
          for (int qi = 0; qi < C::NQ; ++qi) sc[0][qi] = mma_k32(kf0[ks], q[qi][ks], sc[0][qi]);
        // Tile 0's products first: nothing is scheduled across this point.
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
          for (int qi = 0; qi < C::NQ; ++qi) sc[1][qi] = mma_k32(kf1[ks], q[qi][ks], sc[1][qi]);
#pragma unroll
        for (int qi = 0; qi < C::NQ; ++qi)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pr[qi][e] = __builtin_amdgcn_exp2f(fmaf(sc[0][qi][e], a.sl2, -m[qi]));
            pmax = fmaxf(pmax, pr[qi][e]);
          }
        // Tile 1's products with tile 0's exponentials threaded between them.
#pragma unroll
        for (int i = 0; i < 12; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
      }
      // Stage k+1 resident before the next barrier, so that it can be read
      // during phase B.
      if (k + 1 < nstage) wait_stages<C::LPW>(last - (k + 1));
      bar();
      // Phase B: softmax of stage k on the VALU while the value waves'
      // products of stage k-1 occupy the matrix cores; tile 0's K^T
      // fragments of stage k+1 are read meanwhile.
      if (k + 1 < nstage && (k + 1) * C::SROWS < wlim) read_k0(k + 1);
      if (act) {
        if (kb + C::SROWS > wmin) {
          // Diagonal stage: mask the keys a row cannot see and redo tile 0.
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int qi = 0; qi < C::NQ; ++qi)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (kb + 16 * t + 4 * g + e >= lim[qi]) sc[t][qi][e] = kNegInf;
          pmax = 0.0f;
#pragma unroll
          for (int qi = 0; qi < C::NQ; ++qi)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              pr[qi][e] = __builtin_amdgcn_exp2f(fmaf(sc[0][qi][e], a.sl2, -m[qi]));
              pmax = fmaxf(pmax, pr[qi][e]);
            }
        }
#pragma unroll
        for (int qi = 0; qi < C::NQ; ++qi)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pr[qi][4 + e] = __builtin_amdgcn_exp2f(fmaf(sc[1][qi][e], a.sl2, -m[qi]));
            pmax = fmaxf(pmax, pr[qi][4 + e]);
          }
        float alpha[C::NQ];
#pragma unroll
        for (int qi = 0; qi < C::NQ; ++qi) alpha[qi] = 1.0f;
        moved = __builtin_amdgcn_ballot_w64(!(pmax <= 256.0f)) != 0;
        if (moved) {
#pragma unroll
          for (int qi = 0; qi < C::NQ; ++qi) {
            float v = kNegInf;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
              for (int e = 0; e < 4; ++e) v = fmaxf(v, sc[t][qi][e]);
            // sl2 > 0, so the maximum commutes with the scaling.
            const float mx = max_g(v) * a.sl2;
            if (mx > m[qi] + 8.0f) {
              alpha[qi] = __builtin_amdgcn_exp2f(m[qi] - mx);
              l[qi] *= alpha[qi];
              m[qi] = mx;
#pragma unroll
              for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  pr[qi][4 * t + e] = __builtin_amdgcn_exp2f(fmaf(sc[t][qi][e], a.sl2, -m[qi]));
            }
          }
        }
        char *pb = pbase + (k & 1) * C::P_B + w * (C::NQ * 1024);
        float *ab = abase + (k & 1) * (C::A_B / 4) + c * C::NRT + C::NQ * w;
        const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
        for (int qi = 0; qi < C::NQ; ++qi) {
          // P^T fragment: k index 8g+e holds key 4g+e of tile 0 (e < 4) and
          // key 4g+e-4 of tile 1 (e >= 4) -- the same order in which the
          // value wave assembles C^T from its two transposing reads.  The
          // row sum accumulates the bf16 values the products use.
          bf16x8 pf;
#pragma unroll
          for (int e = 0; e < 8; ++e) pf[e] = (bf16)pr[qi][e];
#pragma unroll
          for (int e = 0; e < 8; e += 2)
            l[qi] = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){pf[e], pf[e + 1]}, ones, l[qi], false);
          *(bf16x8 *)(pb + qi * 1024 + lane * 16) = pf;
          if (g == 0) ab[qi] = alpha[qi];
        }
      }
      // Whether this wave moved its reference maxima (the value waves then
      // rescale its rows); a wave with no keys left in this stage writes 0.
      if (k < nstage && lane == 0) fbase[(k & 1) * 4 + w] = moved ? 1.0f : 0.0f;
      // This wave's P / alpha written before the next barrier.
      wait_lgkm0();
    }
#pragma unroll
    for (int qi = 0; qi < C::NQ; ++qi) {
      const float lt = sum_g(l[qi]);
      if (g == 0) {
        lbuf[c * C::NRT + C::NQ * w + qi] = lt;
        sbuf[c * C::NRT + C::NQ * w + qi] = __builtin_amdgcn_exp2f(m0[qi] - m[qi]);
      }
    }
    wait_lgkm0();
    bar();
    bar();   // the value waves' staged output is complete (they store it)
  } else {
    // ---------------- value wave ----------------
    // Value wave v holds O^T for all NRT row tiles of the workgroup and the
    // channel quarter [64 v, 64 v + 64) (NB blocks of 16): each C^T fragment
    // it reads with the half-rate transposing reads then feeds NRT products,
    // while the P^T fragments come with full-rate 16-byte reads.
    const int v = w;
    f32x4 o[C::NRT][C::NB];
    int wl[4];   // key limit of each score wave's rows
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r0 = qtile * C::ROWS + u * C::ROWS_W, r1 = min(r0 + C::ROWS_W, nrows) - 1;
      wl[u] = r1 >= r0 ? (r1 / H) / s : 0;
    }
#pragma unroll
    for (int rt = 0; rt < C::NRT; ++rt)
#pragma unroll
      for (int mb = 0; mb < C::NB; ++mb) o[rt][mb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    if (self_lds) {
      // Copy the frames' rows into LDS: 16-byte chunk i of the region is
      // chunk i mod (RB/16) of frame f0 + i / (RB/16); the last load's lanes
      // past the end repeat the last frame (inside the region).
      constexpr int CPR = C::RB / 16, RCH = C::R / 8;
      const int nld = (nfr * CPR + 63) / 64;
      for (int i = v; i < nld; i += 4) {
        const int ch = i * 64 + lane;
        const int fr = min(ch / CPR, nfr - 1), part = ch - (ch / CPR) * CPR;
        const size_t f = (size_t)b * Tn + f0 + fr;
        const bf16 *src = part < RCH ? (const bf16 *)a.Cp + f * C::R + 8 * part
                                     : (const bf16 *)a.KR + f * C::DR + 8 * (part - RCH);
        __builtin_amdgcn_global_load_lds((const void *)src, (lds_void *)(selfb + i * 1024), 16, 0,
                                         0);
      }
      wait_vm<0>();
    }
    bar();
    // O^T += C^T P^T for row tiles [r0, r1) of stage kk.
    auto pv = [&](int kk, const bf16x8 (&vf)[C::NB], auto r0c, auto r1c) {
      constexpr int r0 = decltype(r0c)::value, r1 = decltype(r1c)::value;
      const char *pb = pbase + (kk & 1) * C::P_B;
#pragma unroll
      for (int rt = r0; rt < r1; ++rt) {
        if (kk * C::SROWS >= wl[rt / C::NQ]) continue;   // that score wave had no keys
        const bf16x8 pf = *(const bf16x8 *)(pb + rt * 1024 + lane * 16);
#pragma unroll
        for (int mb = 0; mb < C::NB; ++mb) o[rt][mb] = mma_k32(vf[mb], pf, o[rt][mb]);
      }
    };
    using Half = std::integral_constant<int, MTLA_WS_SPLIT>;
    using Zero = std::integral_constant<int, 0>;
    using Full = std::integral_constant<int, C::NRT>;
    for (int k = 0; k <= nstage; ++k) {
      bar();
      const int kk = k - 1;
      const bool act = kk >= 0;
      bf16x8 vf[C::NB];
      // Phase A: rescale if a score wave moved its maxima, read this
      // quarter's C^T fragments of stage k-1 and do the first half of the
      // row tiles (alongside the score waves' products).
      if (act) {
        const f32x4 fl = *(const f32x4 *)(fbase + (kk & 1) * 4);
        if (fl[0] + fl[1] + fl[2] + fl[3] != 0.0f) {
          const float *ab = abase + (kk & 1) * (C::A_B / 4) + c * C::NRT;
          float al[C::NRT];
#pragma unroll
          for (int i = 0; i < C::NRT; i += 4) {
            const f32x4 x = *(const f32x4 *)(ab + i);
            al[i] = x[0]; al[i + 1] = x[1]; al[i + 2] = x[2]; al[i + 3] = x[3];
          }
#pragma unroll
          for (int rt = 0; rt < C::NRT; ++rt) {
            // Rows of a wave without a flag keep their factor of 1.
            const float f = fl[rt / C::NQ] != 0.0f ? al[rt] : 1.0f;
#pragma unroll
            for (int mb = 0; mb < C::NB; ++mb) o[rt][mb] *= f;
          }
        }
        const char *sb = smem + (kk % nst) * C::STAGE_B;
#pragma unroll
        for (int mb = 0; mb < C::NB; ++mb) {
          // Lane (g, c) addresses row 4g + c/4, channels 16m + 4(c%4)..+3 of
          // block m; the transposing read hands it channel 16m + c of keys
          // 4g..4g+3 (tile 0, low half) and of tile 1 (high half).
          const int m = 4 * v + mb;
          const char *p0 = sb + tile_off(4 * g + (c >> 2), (16 * m + 4 * (c & 3)) * 2);
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p0);
          const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p0 + C::TILE_B));
          vf[mb] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
        pv(kk, vf, Zero(), Half());
      }
      bar();
      // Phase B: the second half (alongside the score waves' softmax).
      if (act) pv(kk, vf, Half(), Full());
    }
    bar();
    // Output: normalised O rows staged through the (now idle) key ring in
    // row-major order, OST bytes apart, then stored whole: each 16-byte lane
    // store then covers an eighth of a 128-byte line, instead of the
    // accumulator layout's 32 bytes of each of 16 rows.
    constexpr int OST = C::R * 2 + 16;
    static_assert(C::ROWS * OST <= C::NST * C::STAGE_B, "the output fits the ring");
    const float *lb = lbuf + c * C::NRT, *sf = sbuf + c * C::NRT;
    // Each row's own value C'_m (from the LDS copy, else from global memory:
    // two separate loops, so that each read's address space is known).
    auto stage_out = [&](auto cmrow) {
      // Frame of row 16 rt + c, relative to f0: q0 + floor((r0 + 16 rt + 1/2) / H)
      // with (q0, r0) = divmod(first row of the lane, H).  The numerator stays
      // below 240, so the fp32 reciprocal cannot move it across an integer.
      const int rl = qtile * C::ROWS + c, q0 = rl / H - f0, r0 = rl - (rl / H) * H;
      const float invH = 1.0f / (float)H;
      // Row tile rt+1's operands are read before row tile rt's results are
      // written: the compiler cannot tell that the LDS copy and the staging
      // area do not overlap, and would otherwise wait out each read behind
      // the previous write.
      bf16x4 cvn[C::NB];
      float ln, sn;
      auto fetch = [&](int rt) {
        const int row = qtile * C::ROWS + 16 * rt + c;
        const int fq = q0 + (int)(((float)(r0 + 16 * rt) + 0.5f) * invH);
        const bf16 *cm = cmrow(row < nrows ? fq : 0) + 64 * v + 4 * g;   // rows past the end are not stored
#pragma unroll
        for (int mb = 0; mb < C::NB; ++mb) cvn[mb] = *(const bf16x4 *)(cm + 16 * mb);
        ln = lb[rt];
        sn = sf[rt];
      };
      fetch(0);
#pragma unroll
      for (int rt = 0; rt < C::NRT; ++rt) {
        bf16x4 cv[C::NB];
#pragma unroll
        for (int mb = 0; mb < C::NB; ++mb) cv[mb] = cvn[mb];
        const float inv = __builtin_amdgcn_rcpf(ln), fs = sn * inv;
        if (rt + 1 < C::NRT) fetch(rt + 1);
        char *srow = smem + (16 * rt + c) * OST + 2 * (64 * v + 4 * g);
#pragma unroll
        for (int mb = 0; mb < C::NB; ++mb) {
          const f32x4 x = o[rt][mb] * inv + fs * (f32x4){to_f32(cv[mb][0]), to_f32(cv[mb][1]),
                                                         to_f32(cv[mb][2]), to_f32(cv[mb][3])};
          *(bf16x4 *)(srow + 32 * mb) = (bf16x4){(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
        }
      }
    };
    if (self_lds)
      stage_out([&](int frl) { return (const bf16 *)(selfb + frl * C::RB); });
    else
      stage_out([&](int frl) { return (const bf16 *)a.Cp + ((size_t)b * Tn + f0 + frl) * C::R; });
    wait_lgkm0();
    bar();
    // Value wave v stores rows [48 v, 48 v + 48): two 512-byte rows per
    // instruction, lane i covering bytes 16 (i mod 32) of row 2 j + i / 32.
    const int row0 = qtile * C::ROWS;
#pragma unroll 4
    for (int j = 0; j < C::ROWS / 8; ++j) {
      const int r = (C::ROWS / 4) * v + 2 * j + (lane >> 5);
      const u32x4 x = *(const u32x4 *)(smem + r * OST + 16 * (lane & 31));
      if (row0 + r < nrows)
        *(u32x4 *)((char *)a.O + ((size_t)b * nrows + row0 + r) * (C::R * 2) + 16 * (lane & 31)) = x;
    }
  }
}

hipError_t prefill_ws(int B, int T_len, int H, int s, float sl2, const void *qt, const void *QR,
                      const void *keys, int64_t kstride, const void *Cp, const void *KR, void *O,
                      hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  using C = WsCfg;
  const int tiles = (T_len * H + C::ROWS - 1) / C::ROWS;
  const int nst = C::NST;
  const size_t lds = (size_t)nst * C::STAGE_B + C::EXTRA;
  allow_lds<prefill_ws_kernel>();
  // Masked scores are -inf before the fused scale-and-subtract, which needs
  // a positive scale (0 * -inf is NaN); a scale that underflows to zero is
  // raised to the smallest normal value, a change below fp32 resolution of
  // every finite scaled score.
  if (!(sl2 >= FLT_MIN)) sl2 = FLT_MIN;
  PrefillArgs args{qt, QR, (const char *)keys, kstride * 2, Cp, KR, O, B, T_len, H, s, tiles,
                   nst, sl2};
  return launch_timed((const void *)prefill_ws_kernel, dim3(tiles * B), dim3(512), lds, stream,
                      &args, ev0, ev1);
}

}  // namespace

hipError_t launch_group_scan(int dtype, const float *cg, const void *b_hc, const float *table,
                             const void *KR, int B, int T, int r, int dR, int s, void *Cp,
                             void *keys, int64_t keys_stride, void *cache, int64_t cache_stride,
                             hipStream_t stream) {
  const int nS = (T + s - 1) / s;
  const int64_t work = (int64_t)nS * ((r + dR) / 4);
  dim3 grid((unsigned)((work + 255) / 256), B);
  if (dtype == 1)
    hipLaunchKernelGGL(group_scan_kernel<bf16>, grid, dim3(256), 0, stream, cg, (const bf16 *)b_hc,
                       table, (const bf16 *)KR, T, r, dR, s, nS, (bf16 *)Cp, (bf16 *)keys,
                       keys_stride, (bf16 *)cache, cache_stride);
  else
    hipLaunchKernelGGL(group_scan_kernel<float>, grid, dim3(256), 0, stream, cg,
                       (const float *)b_hc, table, (const float *)KR, T, r, dR, s, nS, (float *)Cp,
                       (float *)keys, keys_stride, (float *)cache, cache_stride);
  return hipGetLastError();
}

bool prefill_attention_supported(int dtype, int H, int r, int dR) {
  (void)dtype;
  if (!((r == 256 && dR == 32) || (r == 512 && dR == 64))) return false;
  return H >= 1 && H <= 64;
}

hipError_t launch_prefill_attention(int dtype, int B, int T, int H, int r, int dR, int s,
                                    float scale, const void *qt, const void *QR, const void *keys,
                                    int64_t keys_stride, const void *Cp, const void *KR, void *O,
                                    hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  const float sl2 = scale * kLog2e;
  if (dtype == 1) {
    if (r == 256)
      return prefill_ws(B, T, H, s, sl2, qt, QR, keys, keys_stride, Cp, KR, O, stream, ev0, ev1);
    return prefill_attn_t<bf16, 512, 64, 1>(B, T, H, s, sl2, qt, QR, keys, keys_stride, Cp, KR, O,
                                            stream, ev0, ev1);
  }
  if (r == 256)
    return prefill_attn_t<float, 256, 32, 2>(B, T, H, s, sl2, qt, QR, keys, keys_stride, Cp, KR, O,
                                             stream, ev0, ev1);
  return prefill_attn_t<float, 512, 64, 1>(B, T, H, s, sl2, qt, QR, keys, keys_stride, Cp, KR, O,
                                           stream, ev0, ev1);
}

}  // namespace mtla
