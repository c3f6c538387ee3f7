// Absorbed MTLA attention on gfx950: the split-K incremental-decoding kernel,
// its log-sum-exp combine, the group scan that builds the intermediate states
// of the parallel form, and the stride-aware masked prefill kernel.
//
// Both attention kernels run the same wave-level step (attend32): a tile of 32
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
// incremental decoding ([Notes] Y formula over the compressed cache; [Fig2] (a))
// ---------------------------------------------------------------------------

struct DecodeArgs {
  const int32_t *pos;
  const void *cache;
  int64_t bstride;
  const void *qt;
  const void *QR;
  float *part_o;
  float *part_ml;
  int H, s, chunk, splits;
  float sl2;
};

// grid (splits, B), 4 waves.  Wave w serves heads 16*(w % NHB) .. +15 and the
// slot tiles sl = w / NHB of every staged block of NSL*32 slots.
template <typename T, int R, int DR, int NHB, bool PREFETCH>
__global__ __launch_bounds__(256) void decode_attn_kernel(DecodeArgs a) {
  constexpr int RK = R + DR, NSL = 4 / NHB, BLOCK = NSL * 32;
  constexpr int STRIDE = row_stride<T>(RK);
  constexpr int CH = RK * (int)sizeof(T) / 16, EPC = 16 / (int)sizeof(T);
  constexpr int NCH = BLOCK * CH, NLD = (NCH + 255) / 256;
  constexpr int KS = RK / 32;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int b = blockIdx.y, split = blockIdx.x;
  const int n = a.pos[b] / a.s + 1;                  // slots 0..floor(pos/s)
  const int start = split * a.chunk;
  if (start >= n) return;
  const int end = min(n, start + a.chunk);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int hb = wave % NHB, sl = wave / NHB;
  const int H = a.H;
  const int head = hb * 16 + c;

  AttnState<T, R, DR, 1> st;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int k = 32 * ks + 8 * g;
    if (head < H) {
      if (k < R)
        load8(st.q[0][ks], (const T *)a.qt + ((size_t)b * H + head) * R + k);
      else
        load8(st.q[0][ks], (const T *)a.QR + ((size_t)b * H + head) * DR + (k - R));
    } else {
      st.q[0][ks] = zero_frag<T>();
    }
  }
  st.m[0] = kNegInf;
  st.l[0] = 0.0f;
#pragma unroll
  for (int mt = 0; mt < R / 16; ++mt) st.o[0][mt] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const T *src = (const T *)a.cache + (size_t)b * a.bstride;
  u32x4 pre[NLD];
  auto fetch = [&](int blk) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int idx = tid + 256 * i;
      const int row = idx / CH, ch = idx % CH;
      pre[i] = (u32x4){0u, 0u, 0u, 0u};
      if (idx < NCH && blk + row < end) pre[i] = ldg16(src + (size_t)(blk + row) * RK + ch * EPC);
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int idx = tid + 256 * i;
      if (idx < NCH) sts16(smem + (idx / CH) * STRIDE + (idx % CH) * 16, pre[i]);
    }
  };

  const int lim[1] = {end};
  if (PREFETCH) fetch(start);
  for (int blk = start; blk < end; blk += BLOCK) {
    if (!PREFETCH) fetch(blk);
    __syncthreads();
    stash();
    __syncthreads();
    if (PREFETCH && blk + BLOCK < end) fetch(blk + BLOCK);
    const int kb = blk + sl * 32;
    if (kb < end) attend32<T, R, DR, 1>(st, smem + sl * 32 * STRIDE, STRIDE, kb, lim, a.sl2);
  }

  // Merge the NSL slot-parallel waves of each head block through LDS.
  __syncthreads();
  float *red = (float *)smem;                 // [NSL][H][R]
  float *redm = red + (size_t)NSL * H * R;    // [NSL][H]
  float *redl = redm + NSL * H;               // [NSL][H]
  float lt = st.l[0] + wave_xor(st.l[0], 16);
  lt += wave_xor(lt, 32);
  if (head < H) {
#pragma unroll
    for (int mt = 0; mt < R / 16; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[((size_t)sl * H + head) * R + 16 * mt + 4 * g + e] = st.o[0][mt][e];
    if (g == 0) {
      redm[sl * H + head] = st.m[0];
      redl[sl * H + head] = lt;
    }
  }
  __syncthreads();
  const size_t pbase = ((size_t)b * a.splits + split) * H;
  for (int idx = tid; idx < H * R; idx += 256) {
    const int h = idx / R, ch = idx % R;
    float M = kNegInf;
#pragma unroll
    for (int k = 0; k < NSL; ++k) M = fmaxf(M, redm[k * H + h]);
    float acc = 0.0f, L = 0.0f;
#pragma unroll
    for (int k = 0; k < NSL; ++k) {
      const float mk = redm[k * H + h];
      const float w = (mk == kNegInf) ? 0.0f : exp2f(mk - M);
      acc += w * red[((size_t)k * H + h) * R + ch];
      L += w * redl[k * H + h];
    }
    a.part_o[(pbase + h) * R + ch] = acc;
    if (ch == 0) {
      a.part_ml[(pbase + h) * 2] = M;
      a.part_ml[(pbase + h) * 2 + 1] = L;
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void decode_combine_kernel(const int32_t *pos, int s, int chunk,
                                                             int splits, int H, int R,
                                                             const float *part_o,
                                                             const float *part_ml, T *o) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int n = pos[b] / s + 1;
  const int ns = (n + chunk - 1) / chunk;
  const size_t base = (size_t)b * splits * H;
  float M = kNegInf;
  for (int k = 0; k < ns; ++k) M = fmaxf(M, part_ml[((base + (size_t)k * H) + h) * 2]);
  float L = 0.0f;
  for (int k = 0; k < ns; ++k) {
    const size_t i = (base + (size_t)k * H) + h;
    L += exp2f(part_ml[i * 2] - M) * part_ml[i * 2 + 1];
  }
  const float inv = 1.0f / L;
  for (int ch = threadIdx.x; ch < R; ch += blockDim.x) {
    float acc = 0.0f;
    for (int k = 0; k < ns; ++k) {
      const size_t i = (base + (size_t)k * H) + h;
      acc += exp2f(part_ml[i * 2] - M) * part_o[i * R + ch];
    }
    o[((size_t)b * H + h) * R + ch] = from_f32<T>(acc * inv);
  }
}

// ---------------------------------------------------------------------------
// parallel form ([Notes] stride-aware causal mask; [Fig2] (c))
// ---------------------------------------------------------------------------

// One thread per (sequence b, slot j, channel): walks the s frames of group j.
template <typename T>
__global__ __launch_bounds__(256) void group_scan_kernel(const float *U, const T *KR, int T_len,
                                                         int R, int DR, int s, int nS, T *Cp,
                                                         T *keys, int64_t kstride, T *cache,
                                                         int64_t cstride) {
  const int b = blockIdx.y;
  const int RK = R + DR;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)nS * RK) return;
  const int j = (int)(idx / RK), ch = (int)(idx % RK);
  const int i0 = j * s, i1 = min(i0 + s, T_len) - 1;
  T v;
  if (ch < R) {
    float acc = 0.0f;
    for (int i = i0; i <= i1; ++i) {
      const size_t row = (size_t)b * T_len + i;
      acc += U[row * R + ch];
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
template <auto Kernel> void allow_lds() {
  static const bool once = [] {
    (void)hipFuncSetAttribute((const void *)Kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                              160 * 1024);
    return true;
  }();
  (void)once;
}

template <typename T, int R, int DR, int NHB>
hipError_t decode_attn_t(const DecodePlan &p, int B, int H, int s, float sl2, const int32_t *pos,
                         const void *cache, int64_t bstride, const void *qt, const void *QR,
                         float *part_o, float *part_ml, hipStream_t stream) {
  constexpr bool PF = sizeof(T) == 2;
  auto kern = decode_attn_kernel<T, R, DR, NHB, PF>;
  allow_lds<decode_attn_kernel<T, R, DR, NHB, PF>>();
  DecodeArgs args{pos, cache, bstride, qt, QR, part_o, part_ml, H, s, p.chunk, p.splits, sl2};
  hipLaunchKernelGGL(kern, dim3(p.splits, B), dim3(256), p.lds, stream, args);
  return hipGetLastError();
}

template <typename T, int R, int DR>
hipError_t decode_attn_h(const DecodePlan &p, int B, int H, int s, float sl2, const int32_t *pos,
                         const void *cache, int64_t bstride, const void *qt, const void *QR,
                         float *part_o, float *part_ml, hipStream_t stream) {
  switch (p.nhb) {
    case 1: return decode_attn_t<T, R, DR, 1>(p, B, H, s, sl2, pos, cache, bstride, qt, QR, part_o, part_ml, stream);
    case 2: return decode_attn_t<T, R, DR, 2>(p, B, H, s, sl2, pos, cache, bstride, qt, QR, part_o, part_ml, stream);
    default: return decode_attn_t<T, R, DR, 4>(p, B, H, s, sl2, pos, cache, bstride, qt, QR, part_o, part_ml, stream);
  }
}

template <typename T, int R, int DR>
hipError_t prefill_attn_t(int B, int T_len, int H, int s, float sl2, const void *qt,
                          const void *QR, const void *keys, int64_t kstride, const void *Cp,
                          const void *KR, void *O, hipStream_t stream) {
  constexpr int NQ = R <= 256 ? 2 : 1;
  constexpr bool PF = sizeof(T) == 2;
  constexpr int ROWS = 64 * NQ;
  const int tiles = (T_len * H + ROWS - 1) / ROWS;
  const size_t lds = (size_t)64 * row_stride<T>(R + DR);
  auto kern = prefill_attn_kernel<T, R, DR, NQ, PF>;
  allow_lds<prefill_attn_kernel<T, R, DR, NQ, PF>>();
  PrefillArgs args{qt, QR, keys, kstride, Cp, KR, O, B, T_len, H, s, tiles, sl2};
  hipLaunchKernelGGL(kern, dim3(tiles * B), dim3(256), lds, stream, args);
  return hipGetLastError();
}

}  // namespace

bool decode_plan(int dtype, int H, int r, int dR, int s, int B, int max_pos, DecodePlan *plan) {
  if (!((r == 256 && dR == 32) || (r == 512 && dR == 64))) return false;
  if (H < 1 || H > 64 || s < 1 || B < 1 || max_pos < 0) return false;
  const int esz = dtype == 1 ? 2 : 4;
  DecodePlan p;
  p.nhb = H <= 16 ? 1 : (H <= 32 ? 2 : 4);
  // Fewer slot-parallel waves (smaller staged blocks) when wide fp32 rows
  // would not fit the 160 KB of LDS.
  while (p.nhb < 4 && (size_t)(4 / p.nhb) * 32 * ((r + dR) * esz + 16) > 160 * 1024) p.nhb *= 2;
  const int nsl = 4 / p.nhb;
  p.block = nsl * 32;
  const int nmax = max_pos / s + 1;
  const int64_t total = (int64_t)B * nmax;
  int64_t chunk = (total + 1023) / 1024;
  chunk = ((chunk + p.block - 1) / p.block) * p.block;
  if (chunk < p.block) chunk = p.block;
  const int64_t cap = ((nmax + p.block - 1) / p.block) * (int64_t)p.block;
  if (chunk > cap) chunk = cap;
  p.chunk = (int)chunk;
  p.splits = (int)((nmax + chunk - 1) / chunk);
  const size_t stage = (size_t)p.block * ((r + dR) * esz + 16);
  const size_t reduce = (size_t)nsl * H * r * 4 + (size_t)2 * nsl * H * 4;
  p.lds = stage > reduce ? stage : reduce;
  if (p.lds > 160 * 1024) return false;
  *plan = p;
  return true;
}

hipError_t launch_decode_attention(int dtype, const DecodePlan &plan, int B, int H, int r, int dR,
                                   int s, float scale, const int32_t *pos, const void *cache,
                                   int64_t batch_stride, const void *qt, const void *QR,
                                   float *part_o, float *part_ml, hipStream_t stream) {
  const float sl2 = scale * kLog2e;
  if (dtype == 1) {
    if (r == 256) return decode_attn_h<bf16, 256, 32>(plan, B, H, s, sl2, pos, cache, batch_stride, qt, QR, part_o, part_ml, stream);
    return decode_attn_h<bf16, 512, 64>(plan, B, H, s, sl2, pos, cache, batch_stride, qt, QR, part_o, part_ml, stream);
  }
  if (r == 256) return decode_attn_h<float, 256, 32>(plan, B, H, s, sl2, pos, cache, batch_stride, qt, QR, part_o, part_ml, stream);
  return decode_attn_h<float, 512, 64>(plan, B, H, s, sl2, pos, cache, batch_stride, qt, QR, part_o, part_ml, stream);
}

hipError_t launch_decode_combine(int dtype, const DecodePlan &plan, int B, int H, int r, int s,
                                 const int32_t *pos, const float *part_o, const float *part_ml,
                                 void *o, hipStream_t stream) {
  if (dtype == 1)
    hipLaunchKernelGGL(decode_combine_kernel<bf16>, dim3(H, B), dim3(256), 0, stream, pos, s,
                       plan.chunk, plan.splits, H, r, part_o, part_ml, (bf16 *)o);
  else
    hipLaunchKernelGGL(decode_combine_kernel<float>, dim3(H, B), dim3(256), 0, stream, pos, s,
                       plan.chunk, plan.splits, H, r, part_o, part_ml, (float *)o);
  return hipGetLastError();
}

hipError_t launch_group_scan(int dtype, const float *U, const void *KR, int B, int T, int r, int dR,
                             int s, void *Cp, void *keys, int64_t keys_stride, void *cache,
                             int64_t cache_stride, hipStream_t stream) {
  const int nS = (T + s - 1) / s;
  const int64_t work = (int64_t)nS * (r + dR);
  dim3 grid((unsigned)((work + 255) / 256), B);
  if (dtype == 1)
    hipLaunchKernelGGL(group_scan_kernel<bf16>, grid, dim3(256), 0, stream, U, (const bf16 *)KR, T,
                       r, dR, s, nS, (bf16 *)Cp, (bf16 *)keys, keys_stride, (bf16 *)cache,
                       cache_stride);
  else
    hipLaunchKernelGGL(group_scan_kernel<float>, grid, dim3(256), 0, stream, U, (const float *)KR,
                       T, r, dR, s, nS, (float *)Cp, (float *)keys, keys_stride, (float *)cache,
                       cache_stride);
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
                                    hipStream_t stream) {
  const float sl2 = scale * kLog2e;
  if (dtype == 1) {
    if (r == 256) return prefill_attn_t<bf16, 256, 32>(B, T, H, s, sl2, qt, QR, keys, keys_stride, Cp, KR, O, stream);
    return prefill_attn_t<bf16, 512, 64>(B, T, H, s, sl2, qt, QR, keys, keys_stride, Cp, KR, O, stream);
  }
  if (r == 256) return prefill_attn_t<float, 256, 32>(B, T, H, s, sl2, qt, QR, keys, keys_stride, Cp, KR, O, stream);
  return prefill_attn_t<float, 512, 64>(B, T, H, s, sl2, qt, QR, keys, keys_stride, Cp, KR, O, stream);
}

}  // namespace mtla
