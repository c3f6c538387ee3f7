// Parallel (prefill / training-forward) form of MTLA on gfx950: the gate and
// group scan that build the intermediate states C', and the stride-aware
// masked attention kernel.
//
// [Notes] = "Multi-head Temporal Latent Attention" paper notes (zhaoyang97
// Paper-Notes): key designs / hyper-network temporal merging, stride-aware
// causal mask and decoupled RoPE (the Y formula); [Fig2] = sciencestack.ai
// page, Figure 2 (c).
//
// Attention kernel.  Query rows are (frame m, head h) pairs, row = m*H + h.
// Row (m, h) sees the compact keys j < floor(m/s) -- the group-final states of
// the groups that ended before m, i.e. the stride-aware mask's columns
// n < m with n mod s = s-1 -- plus its own state C'_m, which seeds the online
// softmax.  A workgroup owns 4 * 16 * NQ consecutive rows; each wave holds
// 16 * NQ of them (NQ 16-row tiles) with their queries in registers and
// their O^T (r x rows) accumulators in AGPRs.  The compact keys stream
// through a ring of LDS stages (32 keys each) by direct global->LDS loads,
// in the swizzled 16-row tile layout; the loop ends at the workgroup's causal
// frontier, so masked tiles are never visited.  Per 16-key tile a wave:
//   S^T (16 keys x 16 rows) = K . Q^T        K from LDS, A operand, K=32 MFMA
//   online softmax in log2 units, reference max moved lazily (by > 2^8)
//   O^T (r x 16 rows)     += C^T . P^T      C^T by ds_read_tr16_b64, K=16 MFMA
// Each K fragment read from LDS feeds NQ MFMAs and each C^T fragment NQ more,
// which keeps LDS traffic below what the matrix cores consume.

#include <float.h>
#include <math.h>

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
  const int b = blockIdx.y;
  const int RK = R + DR;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)nS * RK) return;
  const int j = (int)(idx / RK), ch = (int)(idx % RK);
  const int i0 = j * s, i1 = min(i0 + s, T_len) - 1;
  T v;
  if (ch < R) {
    const float bb = to_f32(b_hc[ch]), pj = table[(size_t)j * R + ch];
    float acc = 0.0f;
    for (int i = i0; i <= i1; ++i) {
      const size_t row = (size_t)b * T_len + i;
      const float *r = cg + row * 2 * R;
      acc += sigmoidf((r[R + ch] + bb) * pj) * r[ch];
      Cp[row * R + ch] = from_f32<T>(acc);
    }
    v = from_f32<T>(acc);
  } else {
    v = KR[((size_t)b * T_len + i1) * DR + (ch - R)];
  }
  keys[(size_t)b * kstride + (size_t)j * RK + ch] = v;
  if (cache) cache[(size_t)b * cstride + (size_t)j * RK + ch] = v;
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

  for (int k = 0; k < nstage; ++k) {
    wait_stages<C::LPW>(min(a.nst - 1, nstage - 1 - k));
    bar();
    // Every wave is past stage k-1 here: its ring slot can be refilled.
    if (k >= 1 && k - 1 + a.nst < nstage) issue(k - 1 + a.nst);
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
// waves, two per SIMD.  Waves 0-3 ("score waves") own 48 rows each: they
// hold the queries, compute S^T for the 32 keys of a stage, run the online
// softmax and pass the bf16 probabilities P^T and the per-row rescale
// factors to their partner through LDS.  Waves 4-7 ("value waves") hold the
// O^T accumulators of the same rows and add C^T P^T over the stage's 32 keys
// with K=32 products (gfx950's 16x16x32 bf16 MFMA runs at twice the rate of
// the 16x16x16 form).  A score wave and its partner share a SIMD, so the
// softmax arithmetic of one overlaps the matrix products of the other and
// each hides the other's LDS latency; splitting the roles also splits the
// register state (queries vs accumulators) so each wave fits in half the
// SIMD's register file.  One workgroup barrier per stage orders the
// handoff: at iteration k the score waves process stage k while the value
// waves consume stage k-1.
// ---------------------------------------------------------------------------
struct WsCfg {
  static constexpr int R = 256, DR = 32, RK = R + DR, RB = RK * 2, NSEG = RB / 64;
  static constexpr int NQ = 3, KS = RK / 32, MT = R / 16;
  static constexpr int ROWS_W = 16 * NQ, ROWS = 4 * ROWS_W;
  static constexpr int SROWS = 32, TILE_B = 16 * RB, STAGE_B = 2 * TILE_B;
  static constexpr int NBLK = 2 * NSEG, LPW = (NBLK + 3) / 4;
  static constexpr int P_B = 4 * NQ * 64 * 16;   // P slot: 4 waves x NQ fragments x 64 lanes x 16 B
  static constexpr int A_B = 4 * ROWS_W * 4;     // rescale-factor slot (also the row sums)
  static constexpr int EXTRA = 2 * P_B + 3 * A_B + 1024;
  static constexpr int MAX_NST = 6;
};

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__global__ __launch_bounds__(512) void prefill_ws_kernel(PrefillArgs a) {
  using C = WsCfg;
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int H = a.H, Tn = a.T, s = a.s, nst = a.nst;

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
  float *abase = (float *)(pbase + 2 * C::P_B);
  float *lbuf = abase + 2 * (C::A_B / 4);
  char *dummy = (char *)(lbuf + C::A_B / 4);

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

    bf16x8 q[C::NQ][C::KS];
    float m[C::NQ], l[C::NQ];
    int lim[C::NQ];
#pragma unroll
    for (int qi = 0; qi < C::NQ; ++qi) {
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
        bf16x8 d;
        if (k < C::R) {
          load8(q[qi][ks], (const bf16 *)a.qt + qoff * C::R + k);
          load8(d, (const bf16 *)a.Cp + coff * C::R + k);
        } else {
          load8(q[qi][ks], (const bf16 *)a.QR + qoff * C::DR + (k - C::R));
          load8(d, (const bf16 *)a.KR + coff * C::DR + (k - C::R));
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) dot += to_f32(q[qi][ks][e]) * to_f32(d[e]);
      }
      // The row's own state seeds the softmax: weight 1 at reference max m.
      m[qi] = sum_g(dot) * a.sl2;
      l[qi] = (g == 0) ? 1.0f : 0.0f;
    }
    asm volatile("" ::: "memory");

    // Keys below wmin are visible to every row of the wave: no mask needed.
    const int wmin = rw < nrows ? ((rw / H) / s) : 0;
    const int pro = min(nst, nstage);
    for (int k = 0; k < pro; ++k) issue(k);
    int last = pro - 1;
    if (nstage > 0) wait_stages<C::LPW>(last);

    for (int k = 0; k <= nstage; ++k) {
      bar();
      // Stage k-2 has been consumed by both roles: refill its slot.
      if (k >= 2 && k - 2 + nst < nstage) {
        issue(k - 2 + nst);
        last = k - 2 + nst;
      }
      if (k < nstage && k * C::SROWS < wlim) {
        const char *sb = smem + (k % nst) * C::STAGE_B;
        const int kb = k * C::SROWS;
        f32x4 sc[2][C::NQ];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const char *tile = sb + t * C::TILE_B;
          bf16x8 kf[C::KS];
#pragma unroll
          for (int ks = 0; ks < C::KS; ++ks)
            kf[ks] = *(const bf16x8 *)(tile + tile_off(c, ks * 64 + g * 16));
#pragma unroll
          for (int qi = 0; qi < C::NQ; ++qi) sc[t][qi] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
            for (int qi = 0; qi < C::NQ; ++qi) sc[t][qi] = mma_k32(kf[ks], q[qi][ks], sc[t][qi]);
        }
        if (kb + C::SROWS > wmin) {
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int qi = 0; qi < C::NQ; ++qi)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (kb + 16 * t + 4 * g + e >= lim[qi]) sc[t][qi][e] = kNegInf;
        }
        // Online softmax in log2 units (sl2 > 0, so the max commutes with
        // the scaling); the reference max moves only by steps > 2^8.
        float mnew[C::NQ];
        bool up_any = false;
#pragma unroll
        for (int qi = 0; qi < C::NQ; ++qi) {
          float v = kNegInf;
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) v = fmaxf(v, sc[t][qi][e]);
          const float mx = max_g(v) * a.sl2;
          const bool up = mx > m[qi] + 8.0f;
          mnew[qi] = up ? mx : m[qi];
          up_any |= up;
        }
        float alpha[C::NQ];
#pragma unroll
        for (int qi = 0; qi < C::NQ; ++qi) alpha[qi] = 1.0f;
        if (__builtin_amdgcn_ballot_w64(up_any)) {
#pragma unroll
          for (int qi = 0; qi < C::NQ; ++qi) {
            alpha[qi] = __builtin_amdgcn_exp2f(m[qi] - mnew[qi]);
            l[qi] *= alpha[qi];
            m[qi] = mnew[qi];
          }
        }
        char *pb = pbase + (k & 1) * C::P_B + w * (C::NQ * 1024);
        float *ab = abase + (k & 1) * (C::A_B / 4) + w * C::ROWS_W;
#pragma unroll
        for (int qi = 0; qi < C::NQ; ++qi) {
          // P^T fragment: k index 8g+e holds key 4g+e of tile 0 (e < 4) and
          // key 4g+e-4 of tile 1 (e >= 4) -- the same order in which the
          // value wave assembles C^T from its two transposing reads.
          bf16x8 pf;
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float p = __builtin_amdgcn_exp2f(fmaf(sc[t][qi][e], a.sl2, -m[qi]));
              l[qi] += p;
              pf[4 * t + e] = (bf16)p;
            }
          *(bf16x8 *)(pb + qi * 1024 + lane * 16) = pf;
          if (g == 0) ab[qi * 16 + c] = alpha[qi];
        }
      }
      // Stage k+1 resident and this wave's P / alpha written before the
      // next barrier.
      if (k + 1 < nstage) wait_stages<C::LPW>(last - (k + 1));
      wait_lgkm0();
    }
#pragma unroll
    for (int qi = 0; qi < C::NQ; ++qi) {
      const float lt = sum_g(l[qi]);
      if (g == 0) lbuf[w * C::ROWS_W + qi * 16 + c] = lt;
    }
    wait_lgkm0();
    bar();
  } else {
    // ---------------- value wave ----------------
    f32x4 o[C::NQ][C::MT];
#pragma unroll
    for (int qi = 0; qi < C::NQ; ++qi) {
      const int row = rw + 16 * qi + c;
      const int rr = row < nrows ? row : 0;
      const size_t coff = (size_t)b * Tn + rr / H;
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
        o[qi][mt] = load4f((const bf16 *)a.Cp + coff * C::R + 16 * mt + 4 * g);
    }
    for (int k = 0; k <= nstage; ++k) {
      bar();
      const int kk = k - 1;
      if (kk >= 0 && kk * C::SROWS < wlim) {
        const char *sb = smem + (kk % nst) * C::STAGE_B;
        const char *pb = pbase + (kk & 1) * C::P_B + w * (C::NQ * 1024);
        const float *ab = abase + (kk & 1) * (C::A_B / 4) + w * C::ROWS_W;
        float al[C::NQ];
        bool resc = false;
#pragma unroll
        for (int qi = 0; qi < C::NQ; ++qi) {
          al[qi] = ab[qi * 16 + c];
          resc |= al[qi] != 1.0f;
        }
        if (__builtin_amdgcn_ballot_w64(resc)) {
#pragma unroll
          for (int qi = 0; qi < C::NQ; ++qi)
#pragma unroll
            for (int mt = 0; mt < C::MT; ++mt) o[qi][mt] *= al[qi];
        }
        bf16x8 pf[C::NQ];
#pragma unroll
        for (int qi = 0; qi < C::NQ; ++qi) pf[qi] = *(const bf16x8 *)(pb + qi * 1024 + lane * 16);
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt) {
          // Lane (g, c) addresses row 4g + c/4, channels 16mt + 4(c%4)..+3;
          // the transposing read hands it channel 16mt + c of keys 4g..4g+3.
          const char *p0 = sb + tile_off(4 * g + (c >> 2), (16 * mt + 4 * (c & 3)) * 2);
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p0);
          const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p0 + C::TILE_B));
          const bf16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int qi = 0; qi < C::NQ; ++qi) o[qi][mt] = mma_k32(v, pf[qi], o[qi][mt]);
        }
      }
    }
    bar();
#pragma unroll
    for (int qi = 0; qi < C::NQ; ++qi) {
      const int row = rw + 16 * qi + c;
      if (row < nrows) {
        const float inv = 1.0f / lbuf[w * C::ROWS_W + qi * 16 + c];
        bf16 *dst = (bf16 *)a.O + ((size_t)b * nrows + row) * C::R + 4 * g;
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt) store4f(dst + 16 * mt, o[qi][mt] * inv);
      }
    }
  }
}

hipError_t prefill_ws(int B, int T_len, int H, int s, float sl2, const void *qt, const void *QR,
                      const void *keys, int64_t kstride, const void *Cp, const void *KR, void *O,
                      hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  using C = WsCfg;
  const int tiles = (T_len * H + C::ROWS - 1) / C::ROWS;
  int nst = (int)((159 * 1024 - C::EXTRA) / C::STAGE_B);
  if (nst > C::MAX_NST) nst = C::MAX_NST;
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
  const int64_t work = (int64_t)nS * (r + dR);
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
