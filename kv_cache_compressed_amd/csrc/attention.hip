// Parallel (prefill / training-forward) form of MTLA on gfx950: the gate and
// group scan that build the intermediate states C', and the stride-aware
// masked attention kernel.
//
// The attention kernel's wave-level step (attend32): a tile of 32
// compressed rows (latent r values followed by the RoPE key) sits in LDS, and
// a wave scores it against 16*NQ query columns held in registers:
//
//   S^T (32 keys x 16 cols) = K_tile (32 x (r+d_hR)) . Q^T     A = keys from LDS
//   O^T (r x 16 cols)     += C_tile^T (r x 32) . P^T          A = keys, read transposed
//
// Keys are the MFMA A operand in both products.  For the second one each lane
// needs 8 keys of one latent channel; gfx950's ds_read_tr16_b64 delivers them
// from the row-major tile (two reads per 16x16x32 MFMA).  The k index of the
// P.V product runs over the keys in the order {4g..4g+3, 16+4g..16+4g+3},
// which is exactly the order in which each lane already holds its
// probabilities after the score MFMA, so P needs no cross-lane movement.
// Softmax runs online in log2 units; a column's running max is shared by the
// four lane groups, the running sum stays per lane and is reduced at the end.
//
// [Notes] = "Multi-head Temporal Latent Attention" paper notes (zhaoyang97
// Paper-Notes): key designs / stride-aware causal mask and decoupled RoPE
// (the Y formula); [Fig2] = sciencestack.ai page, Figure 2.

#include <math.h>

#include "common.h"
#include "kernels.h"

namespace mtla {

namespace {

constexpr float kNegInf = -INFINITY;

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

template <typename T, int R, int DR, int NQ> struct AttnState {
  static constexpr int RK = R + DR, KS = RK / 32, MT = R / 16;
  typename Frag<T>::type q[NQ][KS];
  f32x4 o[NQ][MT];
  float m[NQ];
  float l[NQ];
};

// A operand of O^T += C^T P^T for latent channels ch0..ch0+15: lane (g, j)
// receives channel ch0 + j of keys {4g+e} (e < 4) and {16+4g+e-4} (e >= 4).
template <typename T>
__device__ __forceinline__ typename Frag<T>::type pv_frag(const char *kt, int stride, int ch0,
                                                          int g, int j) {
  if constexpr (sizeof(T) == 2) {
    // ds_read_tr16_b64: within a 16-lane group, lane i returns element
    // [4e + i/4][i%4] of the 16 x 4 block whose row k lane k addressed.
    const char *p0 = kt + (4 * g + (j >> 2)) * stride + (ch0 + 4 * (j & 3)) * 2;
    const char *p1 = p0 + 16 * stride;
    bf16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p0);
    bf16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p1);
    return (bf16x8){x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  } else {
    f32x8 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = *(const float *)(kt + (4 * g + e) * stride + (ch0 + j) * 4);
      v[4 + e] = *(const float *)(kt + (16 + 4 * g + e) * stride + (ch0 + j) * 4);
    }
    return v;
  }
}

// One 32-key tile: key kbase + k is visible to column q iff kbase + k < lim[q].
template <typename T, int R, int DR, int NQ>
__device__ __forceinline__ void attend32(AttnState<T, R, DR, NQ> &st, const char *kt, int stride,
                                         int kbase, const int (&lim)[NQ], float sl2) {
  constexpr int KS = AttnState<T, R, DR, NQ>::KS, MT = AttnState<T, R, DR, NQ>::MT;
  const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  f32x4 s0[NQ], s1[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) s0[q] = s1[q] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    typename Frag<T>::type a0, a1;
    load8(a0, (const T *)(kt + c * stride + (32 * ks + 8 * g) * (int)sizeof(T)));
    load8(a1, (const T *)(kt + (16 + c) * stride + (32 * ks + 8 * g) * (int)sizeof(T)));
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      s0[q] = mma_k32(a0, st.q[q][ks], s0[q]);
      s1[q] = mma_k32(a1, st.q[q][ks], s1[q]);
    }
  }
  typename Frag<T>::type pf[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    float mx = kNegInf;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k0 = kbase + 4 * g + e;
      const float v0 = k0 < lim[q] ? s0[q][e] * sl2 : kNegInf;
      const float v1 = k0 + 16 < lim[q] ? s1[q][e] * sl2 : kNegInf;
      s0[q][e] = v0;
      s1[q][e] = v1;
      mx = fmaxf(mx, fmaxf(v0, v1));
    }
    mx = fmaxf(mx, wave_xor(mx, 16));
    mx = fmaxf(mx, wave_xor(mx, 32));
    const float mn = fmaxf(st.m[q], mx);
    const bool none = (mn == kNegInf);
    const float alpha = none ? 1.0f : exp2f(st.m[q] - mn);
    float ps = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = none ? 0.0f : exp2f(s0[q][e] - mn);
      const float p1 = none ? 0.0f : exp2f(s1[q][e] - mn);
      ps += p0 + p1;
      pf[q][e] = (T)p0;
      pf[q][4 + e] = (T)p1;
    }
    st.l[q] = st.l[q] * alpha + ps;
    st.m[q] = mn;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) st.o[q][mt] *= alpha;
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const typename Frag<T>::type a = pv_frag<T>(kt, stride, 16 * mt, g, c);
#pragma unroll
    for (int q = 0; q < NQ; ++q) st.o[q][mt] = mma_k32(a, pf[q], st.o[q][mt]);
  }
}

template <typename T> constexpr int row_stride(int rk) { return rk * (int)sizeof(T) + 16; }

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
  const void *qt;
  const void *QR;
  const void *keys;
  int64_t kstride;
  const void *Cp;
  const void *KR;
  void *O;
  int B, T, H, s, tiles;
  float sl2;
};

// Rows of the query side are (frame m, head h) pairs, row = m*H + h; a
// workgroup owns 128 consecutive rows, each wave 32*NQ/2 of them (NQ tiles of
// 16).  Row (m, h) sees the compressed rows j < floor(m/s) -- the group-final
// states of the groups that ended before m -- plus its own state C'_m, which
// seeds the online softmax (score, weight 1, value C'_m) before the key loop.
template <typename T, int R, int DR, int NQ, bool PREFETCH>
__global__ __launch_bounds__(256) void prefill_attn_kernel(PrefillArgs a) {
  constexpr int RK = R + DR, STRIDE = row_stride<T>(RK);
  constexpr int CH = RK * (int)sizeof(T) / 16, EPC = 16 / (int)sizeof(T);
  constexpr int KBLK = 64, NCH = KBLK * CH, NLD = (NCH + 255) / 256;
  constexpr int KS = RK / 32, MT = R / 16;
  constexpr int ROWS = 64 * NQ;                // rows per workgroup
  extern __shared__ __attribute__((aligned(16))) char smem[];

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
  const int rw = qtile * ROWS + wave * 16 * NQ;

  AttnState<T, R, DR, NQ> st;
  int lim[NQ];
  int wlim = 0;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int row = rw + 16 * q + c;
    const bool ok = row < nrows;
    const int m = ok ? row / H : 0, h = ok ? row % H : 0;
    lim[q] = ok ? m / s : 0;
    const size_t qoff = ((size_t)b * Tn + m) * H + h;
    float dot = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int k = 32 * ks + 8 * g;
      typename Frag<T>::type d;
      if (ok) {
        if (k < R) {
          load8(st.q[q][ks], (const T *)a.qt + qoff * R + k);
          load8(d, (const T *)a.Cp + ((size_t)b * Tn + m) * R + k);
        } else {
          load8(st.q[q][ks], (const T *)a.QR + qoff * DR + (k - R));
          load8(d, (const T *)a.KR + ((size_t)b * Tn + m) * DR + (k - R));
        }
      } else {
        st.q[q][ks] = zero_frag<T>();
        d = zero_frag<T>();
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) dot += to_f32(st.q[q][ks][e]) * to_f32(d[e]);
    }
    dot += wave_xor(dot, 16);
    dot += wave_xor(dot, 32);
    st.m[q] = dot * a.sl2;
    st.l[q] = (g == 0) ? 1.0f : 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        st.o[q][mt][e] = ok ? to_f32(((const T *)a.Cp)[((size_t)b * Tn + m) * R + 16 * mt + 4 * g + e]) : 0.0f;
    }
  }
  // Largest key count any row of this wave / workgroup can see.
  {
    const int last = min(rw + 16 * NQ, nrows) - 1;
    wlim = last >= 0 ? (last / H) / s : 0;
  }
  const int last_wg = min(qtile * ROWS + ROWS, nrows) - 1;
  const int kmax = (last_wg / H) / s;

  const T *src = (const T *)a.keys + (size_t)b * a.kstride;
  u32x4 pre[NLD];
  auto fetch = [&](int kb0) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int idx = tid + 256 * i;
      const int row = idx / CH, ch = idx % CH;
      pre[i] = (u32x4){0u, 0u, 0u, 0u};
      if (idx < NCH && kb0 + row < kmax) pre[i] = ldg16(src + (size_t)(kb0 + row) * RK + ch * EPC);
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int idx = tid + 256 * i;
      if (idx < NCH) sts16(smem + (idx / CH) * STRIDE + (idx % CH) * 16, pre[i]);
    }
  };

  if (PREFETCH && kmax > 0) fetch(0);
  for (int kb0 = 0; kb0 < kmax; kb0 += KBLK) {
    if (!PREFETCH) fetch(kb0);
    __syncthreads();
    stash();
    __syncthreads();
    if (PREFETCH && kb0 + KBLK < kmax) fetch(kb0 + KBLK);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int kt = kb0 + 32 * half;
      if (kt < wlim) attend32<T, R, DR, NQ>(st, smem + 32 * half * STRIDE, STRIDE, kt, lim, a.sl2);
    }
  }

  // O = O^T / l, written back row-major [B, T, H, R].
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    float lt = st.l[q] + wave_xor(st.l[q], 16);
    lt += wave_xor(lt, 32);
    const int row = rw + 16 * q + c;
    if (row < nrows) {
      const float inv = 1.0f / lt;
      T *dst = (T *)a.O + ((size_t)b * nrows + row) * R;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[16 * mt + 4 * g + e] = from_f32<T>(st.o[q][mt][e] * inv);
    }
  }
}

// Raise the dynamic-LDS limit of a kernel to the full 160 KB once per
// instantiation (thread-safe static initialisation), so that launches made
// later -- possibly under graph capture -- issue nothing but the launch.

template <typename T, int R, int DR>
hipError_t prefill_attn_t(int B, int T_len, int H, int s, float sl2, const void *qt,
                          const void *QR, const void *keys, int64_t kstride, const void *Cp,
                          const void *KR, void *O, hipStream_t stream, hipEvent_t ev0,
                          hipEvent_t ev1) {
  constexpr int NQ = R <= 256 ? 2 : 1;
  constexpr bool PF = sizeof(T) == 2;
  constexpr int ROWS = 64 * NQ;
  const int tiles = (T_len * H + ROWS - 1) / ROWS;
  const size_t lds = (size_t)64 * row_stride<T>(R + DR);
  auto kern = prefill_attn_kernel<T, R, DR, NQ, PF>;
  allow_lds<prefill_attn_kernel<T, R, DR, NQ, PF>>();
  PrefillArgs args{qt, QR, keys, kstride, Cp, KR, O, B, T_len, H, s, tiles, sl2};
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
    if (r == 256) return prefill_attn_t<bf16, 256, 32>(B, T, H, s, sl2, qt, QR, keys, keys_stride, Cp, KR, O, stream, ev0, ev1);
    return prefill_attn_t<bf16, 512, 64>(B, T, H, s, sl2, qt, QR, keys, keys_stride, Cp, KR, O, stream, ev0, ev1);
  }
  if (r == 256) return prefill_attn_t<float, 256, 32>(B, T, H, s, sl2, qt, QR, keys, keys_stride, Cp, KR, O, stream, ev0, ev1);
  return prefill_attn_t<float, 512, 64>(B, T, H, s, sl2, qt, QR, keys, keys_stride, Cp, KR, O, stream, ev0, ev1);
}

}  // namespace mtla
