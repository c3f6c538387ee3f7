// Per-head (unabsorbed) strided attention with fp32 storage: the
// correctness-oriented form of heads_attn_kernel (heads.hip), for fp32
// layers.  Same operands and layouts: queries Q_h [B*T, H*DH] (head h at
// column h*DH), Q^R [B*T, H, DR], per-head keys and values KV [B*T, 2*H*DH]
// (K_h at column h*DH, V_h at (H + h)*DH), the shared rotary keys K^R
// [B*T, DR], output O [B*T, H*DH].
//
// [Notes] = "Multi-head Temporal Latent Attention" paper notes (zhaoyang97
// Paper-Notes): key designs / stride-aware causal mask and decoupled RoPE;
// [Fig1] = sciencestack.ai page, Figure 1 (the per-head maps before
// absorption).  Query frame m of head h sees its own column and the
// group-final frames n = s j + s - 1 with j < floor(m/s); the score is
// (Q_h[m] . K_h[n] + Q^R_h[m] . K^R[n]) * scale and the output the softmax-
// weighted sum of V_h[n].
//
// Kernel layout.  A workgroup of 128 threads owns 64 query frames of one
// (sequence, head); each frame is handled by a pair of adjacent lanes, each
// holding half of the frame's score channels (DH/2 of Q_h and DR/2 of Q^R)
// and half of its output channels (DH/2).  The compact keys stream through
// LDS 32 at a time (each key's K_h | K^R | V_h row, fp32).  Per key a lane
// takes its half of the dot product, the pair adds the halves with one lane
// exchange, and both lanes run the same online softmax in log2 units (the
// running maximum moved whenever a score exceeds it) and update their half
// of the output.  Each frame's own column seeds the softmax with weight 1.
// For the backward the kernel can also write each row's log2-sum-exp of the
// scores in log2 units, lse [B*T, H].

#include <math.h>

#include "common.h"
#include "kernels.h"

namespace mtla {

namespace {

template <int DH, int DR> struct F32Heads {
  static constexpr int ROWS = 64, THREADS = 2 * ROWS;
  static constexpr int KEYS = 32;                    // keys per LDS stage
  static constexpr int RW = DH + DR + DH;            // K_h | K^R | V_h floats per key
  static constexpr int HQ = DH / 2, HR = DR / 2;     // a lane's halves
  static_assert(DH % 8 == 0 && DR % 8 == 0, "halves of whole 16-byte chunks");
};

template <int DH, int DR>
__global__ __launch_bounds__(128) void heads_attn_f32_kernel(const float *__restrict__ q,
                                                             const float *__restrict__ QR,
                                                             const float *__restrict__ KV,
                                                             const float *__restrict__ KR,
                                                             float *__restrict__ O,
                                                             float *__restrict__ lse, int T, int H,
                                                             int s, float sl2) {
  using C = F32Heads<DH, DR>;
  __shared__ float kt[C::KEYS * C::RW];

  const int tid = threadIdx.x, half = tid & 1, r = tid >> 1;
  const int h = blockIdx.y, b = blockIdx.z;
  const int m = blockIdx.x * C::ROWS + r;           // this pair's query frame
  const bool ok = m < T;
  const int mf = ok ? m : T - 1;                    // frames past the end repeat the last
  const size_t HD = (size_t)H * DH, KVW = 2 * HD;
  const size_t row = (size_t)b * T + mf;

  // This lane's halves of the query and of the frame's own key and value.
  float qh[C::HQ], qr[C::HR], o[C::HQ];
  const float *qp = q + row * HD + (size_t)h * DH + half * C::HQ;
  const float *qrp = QR + (row * H + h) * DR + half * C::HR;
#pragma unroll
  for (int i = 0; i < C::HQ; ++i) qh[i] = qp[i];
#pragma unroll
  for (int i = 0; i < C::HR; ++i) qr[i] = qrp[i];
  float part = 0.0f;
  {
    const float *kp = KV + row * KVW + (size_t)h * DH + half * C::HQ;
    const float *krp = KR + row * DR + half * C::HR;
#pragma unroll
    for (int i = 0; i < C::HQ; ++i) part = fmaf(qh[i], kp[i], part);
#pragma unroll
    for (int i = 0; i < C::HR; ++i) part = fmaf(qr[i], krp[i], part);
    const float *vp = KV + row * KVW + HD + (size_t)h * DH + half * C::HQ;
#pragma unroll
    for (int i = 0; i < C::HQ; ++i) o[i] = vp[i];
  }
  // The frame's own column: weight 1 at the running maximum it sets.
  float mx = (part + __shfl_xor(part, 1)) * sl2, l = 1.0f;

  // Keys visible to this frame: j < lim; the workgroup walks to the largest.
  const int lim = ok ? m / s : 0;
  const int mlast = min((int)(blockIdx.x + 1) * C::ROWS, T) - 1;
  const int jmax = mlast / s;
  for (int j0 = 0; j0 < jmax; j0 += C::KEYS) {
    const int nk = min(C::KEYS, jmax - j0);
    __syncthreads();   // the previous stage has been read
    // 16-byte pieces; DH and DR are multiples of 4, so none straddles two
    // of the row's three parts.
    constexpr int R4 = C::RW / 4;
    for (int e = tid; e < nk * R4; e += C::THREADS) {
      const int kk = e / R4, c = 4 * (e - kk * R4);
      const size_t nrow = (size_t)b * T + (size_t)(s * (j0 + kk) + s - 1);
      const float *src = c < DH        ? KV + nrow * KVW + (size_t)h * DH + c
                         : c < DH + DR ? KR + nrow * DR + (c - DH)
                                       : KV + nrow * KVW + HD + (size_t)h * DH + (c - DH - DR);
      *(float4 *)(kt + kk * C::RW + c) = *(const float4 *)src;
    }
    __syncthreads();
    for (int kk = 0; kk < nk; ++kk) {
      const float *kr = kt + kk * C::RW;
      float p = 0.0f;
#pragma unroll
      for (int i = 0; i < C::HQ; ++i) p = fmaf(qh[i], kr[half * C::HQ + i], p);
#pragma unroll
      for (int i = 0; i < C::HR; ++i) p = fmaf(qr[i], kr[DH + half * C::HR + i], p);
      const float z = (p + __shfl_xor(p, 1)) * sl2;
      if (j0 + kk >= lim) continue;   // not visible to this frame (both lanes agree)
      if (z > mx) {
        const float a = exp2f(mx - z);
        l *= a;
#pragma unroll
        for (int i = 0; i < C::HQ; ++i) o[i] *= a;
        mx = z;
      }
      const float w = exp2f(z - mx);
      l += w;
      const float *vr = kr + DH + DR + half * C::HQ;
#pragma unroll
      for (int i = 0; i < C::HQ; ++i) o[i] = fmaf(w, vr[i], o[i]);
    }
  }
  if (!ok) return;
  if (lse && half == 0) lse[row * H + h] = mx + log2f(l);   // log2 units
  const float inv = 1.0f / l;
  float *op = O + row * HD + (size_t)h * DH + half * C::HQ;
#pragma unroll
  for (int i = 0; i < C::HQ; ++i) op[i] = o[i] * inv;
}

template <int DH, int DR>
hipError_t heads_f32_t(int B, int T, int H, int s, float sl2, const void *q, const void *QR,
                       const void *KV, const void *KR, void *O, float *lse, hipStream_t stream,
                       hipEvent_t ev0, hipEvent_t ev1) {
  using C = F32Heads<DH, DR>;
  const dim3 grid((T + C::ROWS - 1) / C::ROWS, H, B);
  auto kern = heads_attn_f32_kernel<DH, DR>;
  const float *qf = (const float *)q, *qrf = (const float *)QR, *kvf = (const float *)KV,
              *krf = (const float *)KR;
  float *of = (float *)O;
  void *args[] = {(void *)&qf, (void *)&qrf, (void *)&kvf, (void *)&krf, (void *)&of,
                  (void *)&lse, (void *)&T,  (void *)&H,   (void *)&s,   (void *)&sl2};
  if (ev0) (void)hipEventRecord(ev0, stream);
  const hipError_t e =
      hipLaunchKernel((const void *)kern, grid, dim3(C::THREADS), args, 0, stream);
  if (ev1) (void)hipEventRecord(ev1, stream);
  return e != hipSuccess ? e : hipGetLastError();
}

}  // namespace

hipError_t launch_heads_attention_f32(int B, int T, int H, int d_h, int s, float scale,
                                      const void *q, const void *QR, const void *KV,
                                      const void *KR, void *O, float *lse, hipStream_t stream,
                                      hipEvent_t ev0, hipEvent_t ev1) {
  const float sl2 = scale * kLog2e;
  if (d_h == 128)
    return heads_f32_t<128, 64>(B, T, H, s, sl2, q, QR, KV, KR, O, lse, stream, ev0, ev1);
  return heads_f32_t<64, 32>(B, T, H, s, sl2, q, QR, KV, KR, O, lse, stream, ev0, ev1);
}

}  // namespace mtla
