// Backward of the per-head parallel form with fp32 storage: the
// correctness-oriented counterpart of backward.hip for fp32 layers.  The
// chain rule is the same (output map, masked softmax with the scores
// recomputed, key / value / query maps; the group scan and gate backward are
// shared with the bf16 path); the kernels here are plain fp32 ones:
//
//   attention, query-stationary   four lanes per query frame m of one head,
//       each holding a quarter of Q_h, Q^R_h, dO_h and of the accumulators
//       dQ_h, dQ^R_h; the keys of the visible columns (the frame's own and
//       the group-final frames s j + s - 1, j < floor(m/s)) stream through
//       LDS.  The frame's own column also gives the frame's key-role
//       gradients as a key of itself, which initialise dK | dV and dK^R.
//   attention, key-stationary     four lanes per compact key j (frame
//       n = s j + s - 1), holding quarters of K_h, K^R, V_h and of dK_h, dV_h,
//       dK^R_h; the query frames that see it (floor(m/s) > j) stream through
//       LDS; the sums are added to the frame's row written by the first pass.
//   products                      one strided fp32 product C = C0 + A B for
//       every map and weight gradient (operands addressed through row and
//       column strides, so no transposed copies), each output summed over k
//       in order by one thread.
//
// P = exp2(z - lse) with z the score in log2 units and lse the forward's
// log2-sum-exp; dS = P (dO . V - D) scale with D = rowsum(dO * O).
//
// [Notes] = "Multi-head Temporal Latent Attention" paper notes (zhaoyang97
// Paper-Notes): key designs / stride-aware causal mask (the parallel form is
// what training runs); [Fig2] = sciencestack.ai page, Figure 2 (c).
// Everything repeats bit for bit: no atomics, every sum in a fixed order.

#include <math.h>

#include "common.h"
#include "kernels.h"

namespace mtla {

namespace {

template <int DH_, int DR_> struct BwF32 {
  static constexpr int DH = DH_, DR = DR_;
  static constexpr int LN = 4;                       // lanes per frame or key
  static constexpr int ROWS = 64, THREADS = LN * ROWS;
  static constexpr int QH = DH / LN, QR = DR / LN;   // a lane's quarter
  static constexpr int STAGE = 32;                   // rows per LDS stage
  static constexpr int KROW = 2 * DH + DR;           // K_h | K^R | V_h
  static constexpr int QROW = 2 * DH + DR + 4;       // Q_h | Q^R_h | dO_h | lse, D, pad
  static_assert(QH % 4 == 0 && QR % 4 == 0, "quarters of whole 16-byte pieces");
};

__device__ __forceinline__ float quad_sum(float v) {
  v += __shfl_xor(v, 1);
  return v + __shfl_xor(v, 2);
}

// Copies row pieces [0, DH) of a, [0, DR) of b and [0, DH) of c into an LDS
// row of 2 DH + DR floats, 16 bytes per step, for rows [0, n) of a stage.
template <int DH, int DR, int THREADS, class RowFn>
__device__ __forceinline__ void stage_rows(float *dst, int stride, int n, int tid, RowFn src) {
  constexpr int R4 = (2 * DH + DR) / 4;
  for (int e = tid; e < n * R4; e += THREADS) {
    const int k = e / R4, c = 4 * (e - k * R4);
    *(float4 *)(dst + k * stride + c) = *(const float4 *)src(k, c);
  }
}

struct BwF32Args {
  const float *q;    // [B*T, H*DH]
  const float *QR;   // [B*T, H, DR]
  const float *KV;   // [B*T, 2*H*DH]: K_h at column h*DH, V_h at (H + h)*DH
  const float *KR;   // [B*T, DR]
  const float *dO;   // [B*T, H*DH]
  const float *lse;  // [B*T, H] (log2 units)
  const float *Dr;   // [B*T, H]
  float *dKV;        // [B*T, 2*H*DH]
  float *dKRh;       // [B*T, H, DR]
  float *dQ;         // [B*T, H*DH] at row stride ldq
  float *dQR;        // [B*T, H, DR]
  int T, H, s, ldq;
  float sl2, scale;
};

template <int DH, int DR>
__global__ __launch_bounds__(256) void attn_bwd_f32_q_kernel(BwF32Args a) {
  using C = BwF32<DH, DR>;
  __shared__ float kt[C::STAGE * C::KROW];
  const int tid = threadIdx.x, ql = tid & 3, r = tid >> 2;
  const int h = blockIdx.y, b = blockIdx.z, T = a.T, H = a.H, s = a.s;
  const int m = blockIdx.x * C::ROWS + r;
  const bool ok = m < T;
  const int mf = ok ? m : T - 1;
  const size_t HD = (size_t)H * DH, KVW = 2 * HD, row = (size_t)b * T + mf;

  float qh[C::QH], qr[C::QR], dh[C::QH], dq[C::QH], dqr[C::QR];
  {
    const float *qp = a.q + row * HD + (size_t)h * DH + ql * C::QH;
    const float *rp = a.QR + (row * H + h) * DR + ql * C::QR;
    const float *op = a.dO + row * HD + (size_t)h * DH + ql * C::QH;
#pragma unroll
    for (int i = 0; i < C::QH; ++i) qh[i] = qp[i], dh[i] = op[i];
#pragma unroll
    for (int i = 0; i < C::QR; ++i) qr[i] = rp[i];
  }
  const float L = a.lse[row * H + h], Dv = a.Dr[row * H + h];

  // The frame's own column: as a key of itself it gives this frame's
  // key-role gradients, which start its rows of dK | dV and dK^R.
  {
    const float *kp = a.KV + row * KVW + (size_t)h * DH + ql * C::QH;
    const float *vp = kp + HD;
    const float *krp = a.KR + row * DR + ql * C::QR;
    float p1 = 0.0f, p2 = 0.0f;
#pragma unroll
    for (int i = 0; i < C::QH; ++i) p1 = fmaf(qh[i], kp[i], p1), p2 = fmaf(dh[i], vp[i], p2);
#pragma unroll
    for (int i = 0; i < C::QR; ++i) p1 = fmaf(qr[i], krp[i], p1);
    const float z = quad_sum(p1) * a.sl2, dp = quad_sum(p2);
    const float p = exp2f(z - L), ds = p * (dp - Dv) * a.scale;
#pragma unroll
    for (int i = 0; i < C::QH; ++i) dq[i] = ds * kp[i];
#pragma unroll
    for (int i = 0; i < C::QR; ++i) dqr[i] = ds * krp[i];
    if (ok) {
      float *dk = a.dKV + row * KVW + (size_t)h * DH + ql * C::QH;
      float *dv = dk + HD;
      float *dkr = a.dKRh + (row * H + h) * DR + ql * C::QR;
#pragma unroll
      for (int i = 0; i < C::QH; ++i) dk[i] = ds * qh[i], dv[i] = p * dh[i];
#pragma unroll
      for (int i = 0; i < C::QR; ++i) dkr[i] = ds * qr[i];
    }
  }

  // Compact keys j < floor(m/s); the workgroup walks to its last frame's.
  const int lim = ok ? m / s : 0;
  const int mlast = min((int)(blockIdx.x + 1) * C::ROWS, T) - 1;
  const int jmax = mlast / s;
  for (int j0 = 0; j0 < jmax; j0 += C::STAGE) {
    const int nk = min(C::STAGE, jmax - j0);
    __syncthreads();   // the previous stage has been read
    stage_rows<DH, DR, C::THREADS>(kt, C::KROW, nk, tid, [&](int k, int c) {
      const size_t n = (size_t)b * T + (size_t)(s * (j0 + k) + s - 1);
      return c < DH        ? a.KV + n * KVW + (size_t)h * DH + c
             : c < DH + DR ? a.KR + n * DR + (c - DH)
                           : a.KV + n * KVW + HD + (size_t)h * DH + (c - DH - DR);
    });
    __syncthreads();
    for (int k = 0; k < nk; ++k) {
      const float *kr = kt + k * C::KROW;
      const float *kk = kr + ql * C::QH, *rr = kr + DH + ql * C::QR, *vv = kr + DH + DR + ql * C::QH;
      float p1 = 0.0f, p2 = 0.0f;
#pragma unroll
      for (int i = 0; i < C::QH; ++i) p1 = fmaf(qh[i], kk[i], p1), p2 = fmaf(dh[i], vv[i], p2);
#pragma unroll
      for (int i = 0; i < C::QR; ++i) p1 = fmaf(qr[i], rr[i], p1);
      const float z = quad_sum(p1) * a.sl2, dp = quad_sum(p2);
      if (j0 + k >= lim) continue;   // not visible to this frame (all four lanes agree)
      const float ds = exp2f(z - L) * (dp - Dv) * a.scale;
#pragma unroll
      for (int i = 0; i < C::QH; ++i) dq[i] = fmaf(ds, kk[i], dq[i]);
#pragma unroll
      for (int i = 0; i < C::QR; ++i) dqr[i] = fmaf(ds, rr[i], dqr[i]);
    }
  }
  if (!ok) return;
  float *dqp = a.dQ + row * a.ldq + (size_t)h * DH + ql * C::QH;
  float *dqrp = a.dQR + (row * H + h) * DR + ql * C::QR;
#pragma unroll
  for (int i = 0; i < C::QH; ++i) dqp[i] = dq[i];
#pragma unroll
  for (int i = 0; i < C::QR; ++i) dqrp[i] = dqr[i];
}

template <int DH, int DR>
__global__ __launch_bounds__(256) void attn_bwd_f32_k_kernel(BwF32Args a, int nK) {
  using C = BwF32<DH, DR>;
  __shared__ float qt[C::STAGE * C::QROW];
  const int tid = threadIdx.x, ql = tid & 3, r = tid >> 2;
  const int h = blockIdx.y, b = blockIdx.z, T = a.T, H = a.H, s = a.s;
  const int j = blockIdx.x * C::ROWS + r;   // compact key
  const bool ok = j < nK;
  const int jf = ok ? j : nK - 1;
  const size_t HD = (size_t)H * DH, KVW = 2 * HD;
  const size_t n = (size_t)b * T + (size_t)(s * jf + s - 1);

  float kh[C::QH], kr[C::QR], vh[C::QH], dk[C::QH], dv[C::QH], dkr[C::QR];
  {
    const float *kp = a.KV + n * KVW + (size_t)h * DH + ql * C::QH;
    const float *vp = kp + HD;
    const float *rp = a.KR + n * DR + ql * C::QR;
#pragma unroll
    for (int i = 0; i < C::QH; ++i) kh[i] = kp[i], vh[i] = vp[i], dk[i] = 0.0f, dv[i] = 0.0f;
#pragma unroll
    for (int i = 0; i < C::QR; ++i) kr[i] = rp[i], dkr[i] = 0.0f;
  }

  // Query frames m >= s (j0 + 1) see some key of the workgroup; frame m sees
  // key j iff j < floor(m/s).
  const int j0 = blockIdx.x * C::ROWS;
  for (int m0 = s * (j0 + 1); m0 < T; m0 += C::STAGE) {
    const int nq = min(C::STAGE, T - m0);
    __syncthreads();
    stage_rows<DH, DR, C::THREADS>(qt, C::QROW, nq, tid, [&](int k, int c) {
      const size_t m = (size_t)b * T + m0 + k;
      return c < DH        ? a.q + m * HD + (size_t)h * DH + c
             : c < DH + DR ? a.QR + (m * H + h) * DR + (c - DH)
                           : a.dO + m * HD + (size_t)h * DH + (c - DH - DR);
    });
    for (int k = tid; k < nq; k += C::THREADS) {
      const size_t m = (size_t)b * T + m0 + k;
      qt[k * C::QROW + 2 * DH + DR] = a.lse[m * H + h];
      qt[k * C::QROW + 2 * DH + DR + 1] = a.Dr[m * H + h];
    }
    __syncthreads();
    for (int k = 0; k < nq; ++k) {
      const float *qrow = qt + k * C::QROW;
      const float *qq = qrow + ql * C::QH, *rr = qrow + DH + ql * C::QR,
                  *oo = qrow + DH + DR + ql * C::QH;
      float p1 = 0.0f, p2 = 0.0f;
#pragma unroll
      for (int i = 0; i < C::QH; ++i) p1 = fmaf(qq[i], kh[i], p1), p2 = fmaf(oo[i], vh[i], p2);
#pragma unroll
      for (int i = 0; i < C::QR; ++i) p1 = fmaf(rr[i], kr[i], p1);
      const float z = quad_sum(p1) * a.sl2, dp = quad_sum(p2);
      if (!ok || j >= (m0 + k) / s) continue;   // not visible (all four lanes agree)
      const float p = exp2f(z - qrow[2 * DH + DR]);
      const float ds = p * (dp - qrow[2 * DH + DR + 1]) * a.scale;
#pragma unroll
      for (int i = 0; i < C::QH; ++i) dk[i] = fmaf(ds, qq[i], dk[i]), dv[i] = fmaf(p, oo[i], dv[i]);
#pragma unroll
      for (int i = 0; i < C::QR; ++i) dkr[i] = fmaf(ds, rr[i], dkr[i]);
    }
  }
  if (!ok) return;
  // Added to the frame's own-column terms written by the query pass.
  float *dkp = a.dKV + n * KVW + (size_t)h * DH + ql * C::QH;
  float *dvp = dkp + HD;
  float *dkrp = a.dKRh + (n * H + h) * DR + ql * C::QR;
#pragma unroll
  for (int i = 0; i < C::QH; ++i) dkp[i] += dk[i], dvp[i] += dv[i];
#pragma unroll
  for (int i = 0; i < C::QR; ++i) dkrp[i] += dkr[i];
}

// D[i] = sum over the DH channels of dO[i, :] * O[i, :] (fp32), one thread
// per row, in channel order.
__global__ __launch_bounds__(256) void rowdot_f32_kernel(const float *dO, const float *O, int MH,
                                                         int DH, float *D) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= MH) return;
  const float *u = dO + (size_t)i * DH, *v = O + (size_t)i * DH;
  float acc = 0.0f;
  for (int k = 0; k < DH; ++k) acc = fmaf(u[k], v[k], acc);
  D[i] = acc;
}

// C[m, n] = C0[m, n] + sum over k < K, in order, of A(m, k) B(k, n), with
// A(m, k) = A[m sam + k sak], B(k, n) = B[k sbk + n sbn], C at row stride
// ldc and C0 at ldc0 (C0 may be C with ldc0 = ldc, or null for zero).  64 x 64 output tiles, K in
// steps of 16 through LDS; each thread owns a 4 x 4 block of outputs
// (rows ty + 16 i, columns tx + 16 j).
__global__ __launch_bounds__(256) void gemm_f32s_kernel(const float *A, size_t sam, size_t sak,
                                                        const float *Bm, size_t sbk, size_t sbn,
                                                        int M, int N, int K, const float *C0,
                                                        size_t ldc0, float *Cm, size_t ldc) {
  __shared__ float As[16][65], Bs[16][65];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int e = tid; e < 1024; e += 256) {
      // A: along m when its m stride is 1, else along k; B likewise along n or k.
      const int am = sam == 1 ? e & 63 : e >> 4, ak = sam == 1 ? e >> 6 : e & 15;
      const int bn = sbn == 1 ? e & 63 : e >> 4, bk = sbn == 1 ? e >> 6 : e & 15;
      const int gm = m0 + am, gk = k0 + ak, gn = n0 + bn, gk2 = k0 + bk;
      As[ak][am] = (gm < M && gk < K) ? A[gm * sam + gk * sak] : 0.0f;
      Bs[bk][bn] = (gk2 < K && gn < N) ? Bm[gk2 * sbk + gn * sbn] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[k][ty + 16 * i], bv[i] = Bs[k][tx + 16 * i];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[i][jj] = fmaf(av[i], bv[jj], acc[i][jj]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int gm = m0 + ty + 16 * i, gn = n0 + tx + 16 * jj;
      if (gm < M && gn < N)
        Cm[(size_t)gm * ldc + gn] = (C0 ? C0[(size_t)gm * ldc0 + gn] : 0.0f) + acc[i][jj];
    }
}

}  // namespace

hipError_t launch_attn_bwd_f32(int B, int T, int H, int d_h, int s, float scale, const float *q,
                               const float *QR, const float *KV, const float *KR, const float *dO,
                               const float *lse, const float *D, float *dKV, float *dKRh,
                               float *dQ, int ldq, float *dQR, hipStream_t stream) {
  BwF32Args a;
  a.q = q, a.QR = QR, a.KV = KV, a.KR = KR, a.dO = dO, a.lse = lse, a.Dr = D;
  a.dKV = dKV, a.dKRh = dKRh, a.dQ = dQ, a.dQR = dQR;
  a.T = T, a.H = H, a.s = s, a.ldq = ldq;
  a.sl2 = scale * kLog2e, a.scale = scale;
  const int nK = (T - 1) / s;   // compact keys some frame sees
  const dim3 gq((T + 63) / 64, H, B), gk((nK + 63) / 64, H, B);
  if (d_h == 128) {
    hipLaunchKernelGGL((attn_bwd_f32_q_kernel<128, 64>), gq, dim3(256), 0, stream, a);
    if (nK > 0) hipLaunchKernelGGL((attn_bwd_f32_k_kernel<128, 64>), gk, dim3(256), 0, stream, a, nK);
  } else {
    hipLaunchKernelGGL((attn_bwd_f32_q_kernel<64, 32>), gq, dim3(256), 0, stream, a);
    if (nK > 0) hipLaunchKernelGGL((attn_bwd_f32_k_kernel<64, 32>), gk, dim3(256), 0, stream, a, nK);
  }
  return hipGetLastError();
}

hipError_t launch_rowdot_f32(const float *dO, const float *O, int MH, int d_h, float *D,
                             hipStream_t stream) {
  hipLaunchKernelGGL(rowdot_f32_kernel, dim3((MH + 255) / 256), dim3(256), 0, stream, dO, O, MH,
                     d_h, D);
  return hipGetLastError();
}

hipError_t launch_gemm_f32s(const float *A, size_t sam, size_t sak, const float *Bm, size_t sbk,
                            size_t sbn, int M, int N, int K, const float *C0, size_t ldc0,
                            float *C, size_t ldc, hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const dim3 grid((N + 63) / 64, (M + 63) / 64);
  hipLaunchKernelGGL(gemm_f32s_kernel, grid, dim3(256), 0, stream, A, sam, sak, Bm, sbk, sbn, M, N,
                     K, C0, ldc0, C, ldc);
  return hipGetLastError();
}

}  // namespace mtla
