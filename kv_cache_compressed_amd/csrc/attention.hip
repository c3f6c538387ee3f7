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
      return prefill_attn_t<bf16, 256, 32, 3>(B, T, H, s, sl2, qt, QR, keys, keys_stride, Cp, KR, O,
                                              stream, ev0, ev1);
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
