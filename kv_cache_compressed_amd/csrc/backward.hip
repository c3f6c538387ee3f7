// Backward of the per-head parallel form of MTLA on gfx950: the gradients
// that training under the stride-aware mask needs ([Notes] stride-aware
// causal mask: the mask is what lets MTLA train in parallel; [Fig2] (c)), by
// the chain rule through the forward steps, last step first:
//
//   output map      dO = dY W_O,                    dW_O = dY^T O
//   attention       P = exp2(z sl2 - lse) (scores recomputed), D = rowsum(dO * O)
//                   dS = P (dO . V - D) scale
//                   dQ = dS K,  dQ^R = dS K^R,  dK = dS^T Q,  dK^R = sum_h dS^T Q^R_h,
//                   dV = P^T dO                     (over the visible columns)
//   key/value maps  dC' = dK W_K + dV W_V,          dW_K = dK^T C', dW_V = dV^T C'
//   query map       dX += dQ W_Q,                   dW_Q = dQ^T X
//   group sums      dU_i = sum of dC' over the frames of i's group from i on
//   gate            a = W_hc c + b_hc, w = Sigmoid(a * P_j), u = w * c:
//                   dg = dU c w (1 - w),  da = dg P_j,  dP_j += dg a,  db_hc += da,
//                   dW_hc += da c^T,  dc = dU w + W_hc^T da
//   latent map      dX += dc W_dkv,                 dW_dkv = dc^T X
//
// [Notes] = "Multi-head Temporal Latent Attention" paper notes (zhaoyang97
// Paper-Notes): key designs / hyper-network temporal merging, stride-aware
// causal mask; [Fig2] = sciencestack.ai page, Figure 2 (c).
//
// Kernels here: the attention backward as two kernels over the same tiles as
// the forward -- one stationary in the queries (dQ, dQ^R, and every frame's
// own column), one stationary in the compact keys (dK, dV, dK^R of the
// group-final frames) -- the reverse group scan with the gate backward, a
// split-M product A^T B for the weight gradients (the 256 x 256 form is in
// gemm_big.hip), and small helpers.  Every reduction across workgroups adds
// its partials in a fixed order (a separate pass over the weight-gradient
// slabs; the last workgroup to finish for the bias column sums), so the
// gradients repeat bit for bit.

#include <float.h>
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace mtla {

namespace {

// Head widths and tiling of the attention backward: (DH, DR) = (64, 32) with
// two 16-row tiles (32 keys, or 32 query frames) per wave, or (128, 64) with
// one (the accumulators of twice the width then fit the 256 registers of two
// waves per SIMD, with four spilled in the key pass: two workgroups per CU
// measured 3.86 ms per backward call against 4.59 ms for one without spills).
// Streamed rows hold, in the 16-row swizzled tile layout, K_h | K^R | V_h
// (key rows) or Q_h | Q^R_h | dO_h (query rows): 2 DH + DR bf16.
template <int DH_, int DR_, int NT_, int NST_, int OCC_> struct BwCfg {
  static constexpr int DH = DH_, DR = DR_, QK = DH + DR;
  static constexpr int RB = (2 * DH + DR) * 2, NSEG = RB / 64;
  static constexpr int KSEG = DH * 2 / 64, RSEG = DR * 2 / 64;   // 64-byte blocks of K, of K^R
  static constexpr int OFF_C = QK * 2;                           // byte offset of V_h / dO_h
  static constexpr int KS = QK / 32, VS = DH / 32;               // k-steps of the scores, of dP
  static constexpr int MB = DH / 16, RBK = DR / 16;              // 16-channel blocks
  static constexpr int NT = NT_, WROWS = 16 * NT, GROWS = 4 * WROWS;
  static constexpr int TILE_B = 16 * RB, STAGE_B = 2 * TILE_B, SROWS = 32;
  static constexpr int NBLK = 2 * NSEG, LPW = (NBLK + 3) / 4;
  static constexpr int NST = NST_, OCC = OCC_;
  static_assert(QK % 32 == 0 && DH % 32 == 0 && DR % 32 == 0, "whole 64-byte blocks");
  static_assert(MB % 4 == 0 && (RBK % 4 == 0 || RBK == 2), "transposing reads eight at a time");
  static_assert(OCC * (NST * STAGE_B + 1024) <= 160 * 1024, "LDS per CU");
};
using Bw64 = BwCfg<64, 32, 2, 4, 2>;
using Bw128 = BwCfg<128, 64, 1, 3, 2>;

typedef __attribute__((address_space(3))) bf16x4 lds_b4;

// Transposing reads of a 32-row stage (two 16-row tiles): lane (g, c) gets
// channel ch0 + c of rows 4g..4g+3 of tile 0 (low half) and of tile 1 (high
// half), where the channel is a bf16 column of the row.
__device__ __forceinline__ uint32_t tr_addr(const char *sb, int ch0, int g, int c) {
  return lds_addr(sb + tile_off(4 * g + (c >> 2), (ch0 + 4 * (c & 3)) * 2));
}

__device__ __forceinline__ bf16x8 join(const bf16x4 &lo, const bf16x4 &hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// fr[i] = the transposed fragment of channels ch0 + 16 i .. + 15 (i < N), in
// batches of eight transposing reads.
template <class C, int N>
__device__ __forceinline__ void read_tr(const char *sb, int ch0, int g, int c, bf16x8 (&fr)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i0 = 0; i0 < N; i0 += 4) {
      uint32_t ad[8];
      bf16x4 v[8];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        ad[2 * mb] = tr_addr(sb, ch0 + 16 * (i0 + mb), g, c);
        ad[2 * mb + 1] = ad[2 * mb] + C::TILE_B;
      }
      ds_read_tr8(v, ad);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) fr[i0 + mb] = join(v[2 * mb], v[2 * mb + 1]);
    }
  } else {
    static_assert(N == 2, "two blocks, each read twice to fill the batch");
    uint32_t ad[8];
    bf16x4 v[8];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      ad[2 * mb] = tr_addr(sb, ch0 + 16 * (mb & 1), g, c);
      ad[2 * mb + 1] = ad[2 * mb] + C::TILE_B;
    }
    ds_read_tr8(v, ad);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) fr[mb] = join(v[2 * mb], v[2 * mb + 1]);
  }
}

// One direct global->LDS load of 16 bytes per lane into block dst (lane l
// fetches chunk (l%4)^swz(l/4) of row l/4 from `seg`, the row's 64-byte
// segment in global memory).
__device__ __forceinline__ void dma_seg(const char *seg, char *dst, int u) {
  __builtin_amdgcn_global_load_lds((const void *)(seg + u * 16), (lds_void *)dst, 16, 0, 0);
}

struct AttnBwdArgs {
  const bf16 *q;     // [B*T, H*DH]
  const bf16 *QR;    // [B*T, H, DR]
  const bf16 *KV;    // [B*T, 2*H*DH]: K_h at column h*DH, V_h at (H + h)*DH
  const bf16 *KR;    // [B*T, DR]
  const bf16 *dO;    // [B*T, H*DH]
  const float *lse;  // [B*T, H]
  const float *Dr;   // [B*T, H]: rowsum(dO * O)
  float *dKVc;       // [B*nS, 2*H*DH]: key-role dK | dV of compact key (b, j)
  float *dKRc;       // [B*nS, H, DR]:   key-role dK^R per head
  bf16 *dKV;         // [B*T, 2*H*DH]: total dK | dV of every frame
  float *dKRh;       // [B*T, H, DR]:   total dK^R per head of every frame
  bf16 *dQ;          // [B*T, H*DH] at row stride ldq
  bf16 *dQR;         // [B*T, H, DR]
  int B, T, H, s, nS, nK, tiles;
  float sl2, scale;
  int ldq;
};

// ---------------------------------------------------------------------------
// Key-stationary pass: a workgroup owns 4 * 16 NT compact keys of one
// (sequence, head) -- 16 NT per wave, with K^T and V^T fragments in
// registers -- and streams the query frames that can see them (frame m sees
// key j iff j < floor(m/s)) through an LDS ring of 32-frame stages
// (Q | Q^R | dO).  Per stage a wave computes S and dP for its keys (the
// query tile from LDS as the A operand), P and dS on the VALU, and
// accumulates dV^T += dO^T P, dK^T += Q^T dS, dK^R^T += Q^R^T dS with the
// transposed query-side tiles from transposing reads.  Results are the
// key-role gradients of each compact key, written to dKVc / dKRc.
// ---------------------------------------------------------------------------
template <class C>
__global__ __launch_bounds__(256, C::OCC) void attn_bwd_dkdv_kernel(AttnBwdArgs a) {
  constexpr int DH = C::DH, DR = C::DR, NT = C::NT, SROWS = C::SROWS, NST = C::NST;
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int H = a.H, Tn = a.T, s = a.s;
  const int BH = a.B * H;
  // Heavy key blocks (early keys: the most queries) first; XCD-aware as in
  // the forward.
  int bh, kblk;
  {
    const int bid = blockIdx.x;
    if (BH % 8 == 0) {
      const int per = BH / 8, xcd = bid % 8, k = bid / 8;
      kblk = k / per;
      bh = xcd + 8 * (k % per);
    } else {
      kblk = bid / BH;
      bh = bid % BH;
    }
  }
  const int b = bh / H, h = bh % H;
  const size_t kvw = (size_t)2 * H * DH;
  const int kb0 = kblk * C::GROWS;            // first key of the workgroup
  const int kw0 = kb0 + C::WROWS * wave;      // first key of this wave
  if (kb0 >= a.nK) return;                    // whole workgroup: uniform

  // K^T / V^T fragments (B operands): lane (g, c) holds key kw0 + 16 nk + c,
  // channels 32 ks + 8 g .. + 7.
  bf16x8 kf[NT][C::KS], vf[NT][C::VS];
#pragma unroll
  for (int nk = 0; nk < NT; ++nk) {
    const int j = min(kw0 + 16 * nk + c, a.nK - 1);
    const size_t fr = (size_t)b * Tn + (size_t)s * j + (s - 1);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const int k = 32 * ks + 8 * g;
      if (k < DH) load8(kf[nk][ks], a.KV + fr * kvw + h * DH + k);
      else load8(kf[nk][ks], a.KR + fr * DR + (k - DH));
    }
#pragma unroll
    for (int ks = 0; ks < C::VS; ++ks)
      load8(vf[nk][ks], a.KV + fr * kvw + (size_t)(H + h) * DH + 32 * ks + 8 * g);
  }
  f32x4 dv[NT][C::MB], dk[NT][C::MB], dkr[NT][C::RBK];
#pragma unroll
  for (int nk = 0; nk < NT; ++nk) {
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) dv[nk][mb] = dk[nk][mb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mb = 0; mb < C::RBK; ++mb) dkr[nk][mb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  asm volatile("" ::: "memory");

  // Query frames that see key kb0 start at s (kb0 + 1); stages of 32 frames.
  const int q0 = (s * (kb0 + 1)) / SROWS * SROWS;
  const int nstage = q0 < Tn ? (Tn - q0 + SROWS - 1) / SROWS : 0;
  const int wfirst = s * (kw0 + 1);           // first frame that sees a key of this wave
  char *dummy = smem + NST * C::STAGE_B;
  const int u = (lane & 3) ^ swz(lane >> 2);
  auto issue = [&](int sidx) {
    char *sb = smem + (sidx % NST) * C::STAGE_B;
    const int f0 = q0 + sidx * SROWS;
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) {
      const int blk = wave + 4 * i;
      const bool real = blk < C::NBLK;
      const int tl = real ? blk / C::NSEG : 0, qq = real ? blk % C::NSEG : 0;
      const int f = min(f0 + tl * 16 + (lane >> 2), Tn - 1);
      const size_t row = (size_t)b * Tn + f;
      const char *seg;
      if (qq < C::KSEG) seg = (const char *)(a.q + row * H * DH + h * DH) + qq * 64;
      else if (qq < C::KSEG + C::RSEG) seg = (const char *)(a.QR + (row * H + h) * DR) + (qq - C::KSEG) * 64;
      else seg = (const char *)(a.dO + row * H * DH + h * DH) + (qq - C::KSEG - C::RSEG) * 64;
      dma_seg(seg, real ? sb + tl * C::TILE_B + qq * 1024 : dummy, u);
    }
  };
  const int pro = min(NST, nstage);
  for (int k = 0; k < pro; ++k) issue(k);
  int last = pro - 1;

  for (int k = 0; k < nstage; ++k) {
    wait_stages<C::LPW>(last - k);
    bar();
    if (k >= 1 && k - 1 + NST < nstage) {
      issue(k - 1 + NST);
      last = k - 1 + NST;
    }
    const int fs = q0 + k * SROWS;            // first frame of the stage
    if (fs + SROWS <= wfirst) continue;       // no frame here sees this wave's keys
    const char *sb = smem + (k % NST) * C::STAGE_B;

    // S[q, key] and dP[q, key] for both 16-frame tiles: lane (g, c) holds key
    // column c, frames 4g..4g+3 of the tile.
    f32x4 sc[2][NT], dp[2][NT];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const char *tile = sb + t * C::TILE_B;
#pragma unroll
      for (int nk = 0; nk < NT; ++nk) sc[t][nk] = dp[t][nk] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const bf16x8 af = *(const bf16x8 *)(tile + tile_off(c, ks * 64 + g * 16));
#pragma unroll
        for (int nk = 0; nk < NT; ++nk) sc[t][nk] = mma_k32(af, kf[nk][ks], sc[t][nk]);
      }
#pragma unroll
      for (int ks = 0; ks < C::VS; ++ks) {
        const bf16x8 af = *(const bf16x8 *)(tile + tile_off(c, C::OFF_C + ks * 64 + g * 16));
#pragma unroll
        for (int nk = 0; nk < NT; ++nk) dp[t][nk] = mma_k32(af, vf[nk][ks], dp[t][nk]);
      }
    }
    // P and dS; frame f sees key j iff j < floor(f/s) (and f < T).
    bf16x8 pp[NT], ds[NT];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int f = fs + 16 * t + 4 * g + e;
        const int fc = min(f, Tn - 1);
        const size_t ri = ((size_t)b * Tn + fc) * H + h;
        const float L = a.lse[ri], Dv = a.Dr[ri];
        const int lim = f < Tn ? f / s : 0;
#pragma unroll
        for (int nk = 0; nk < NT; ++nk) {
          const int j = kw0 + 16 * nk + c;
          const float p = j < lim ? __builtin_amdgcn_exp2f(sc[t][nk][e] * a.sl2 - L) : 0.0f;
          pp[nk][4 * t + e] = (bf16)p;
          ds[nk][4 * t + e] = (bf16)(p * (dp[t][nk][e] - Dv) * a.scale);
        }
      }
    }
    // Transposed query-side tiles (frames of tile 0 in the low half, tile 1
    // in the high half), one part at a time: dO^T (channels QK ..), then
    // Q^T (0 ..), then Q^R^T (DH ..).
    {
      bf16x8 doT[C::MB];
      read_tr<C>(sb, C::QK, g, c, doT);
#pragma unroll
      for (int nk = 0; nk < NT; ++nk)
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) dv[nk][mb] = mma_k32(doT[mb], pp[nk], dv[nk][mb]);
    }
    {
      bf16x8 qT[C::MB];
      read_tr<C>(sb, 0, g, c, qT);
#pragma unroll
      for (int nk = 0; nk < NT; ++nk)
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) dk[nk][mb] = mma_k32(qT[mb], ds[nk], dk[nk][mb]);
    }
    {
      bf16x8 qrT[C::RBK];
      read_tr<C>(sb, DH, g, c, qrT);
#pragma unroll
      for (int nk = 0; nk < NT; ++nk)
#pragma unroll
        for (int mb = 0; mb < C::RBK; ++mb) dkr[nk][mb] = mma_k32(qrT[mb], ds[nk], dkr[nk][mb]);
    }
  }

  // Key-role gradients of compact key (b, j): lane holds key column c,
  // channels 16 mb + 4g .. + 3.
#pragma unroll
  for (int nk = 0; nk < NT; ++nk) {
    const int j = kw0 + 16 * nk + c;
    if (j < a.nK) {
      float *row = a.dKVc + ((size_t)b * a.nS + j) * kvw;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        *(f32x4 *)(row + h * DH + 16 * mb + 4 * g) = dk[nk][mb];
        *(f32x4 *)(row + (size_t)(H + h) * DH + 16 * mb + 4 * g) = dv[nk][mb];
      }
      float *rr = a.dKRc + (((size_t)b * a.nS + j) * H + h) * DR;
#pragma unroll
      for (int mb = 0; mb < C::RBK; ++mb) *(f32x4 *)(rr + 16 * mb + 4 * g) = dkr[nk][mb];
    }
  }
}

// ---------------------------------------------------------------------------
// Query-stationary pass: a workgroup owns 4 * 16 NT query frames of one
// (sequence, head), 16 NT per wave with Q, Q^R and dO fragments in
// registers; the compact keys stream through the forward's LDS ring
// (K | K^R | V).  Per stage: S^T and dP^T (key tile from LDS as the A
// operand), P and dS, then dQ^T += K^T dS^T and dQ^R^T += K^R^T dS^T with the
// transposed key tiles.  Each frame's own column is done in the prologue:
// it seeds dQ and dQ^R, and its key-side terms (dS_mm Q_m, P_mm dO_m,
// dS_mm Q^R_m) are added to the key-role gradients of the frame (if it is a
// compact key) and written out as the frame's total dK, dV and dK^R.
// ---------------------------------------------------------------------------
template <class C>
__global__ __launch_bounds__(256, C::OCC) void attn_bwd_dq_kernel(AttnBwdArgs a) {
  constexpr int DH = C::DH, DR = C::DR, NT = C::NT, SROWS = C::SROWS, NST = C::NST;
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int H = a.H, Tn = a.T, s = a.s;
  const int BH = a.B * H;
  int bh, qtile;
  {
    const int bid = blockIdx.x;
    if (BH % 8 == 0) {
      const int per = BH / 8, xcd = bid % 8, k = bid / 8;
      qtile = a.tiles - 1 - k / per;
      bh = xcd + 8 * (k % per);
    } else {
      qtile = a.tiles - 1 - bid / BH;
      bh = bid % BH;
    }
  }
  const int b = bh / H, h = bh % H;
  const size_t kvw = (size_t)2 * H * DH;
  const int rw = qtile * C::GROWS + wave * C::WROWS;   // first frame of this wave

  bf16x8 qf[NT][C::KS], dof[NT][C::VS];
  f32x4 dq[NT][C::MB], dqr[NT][C::RBK];
  float L[NT], Dv[NT];
  int lim[NT];
#pragma unroll
  for (int qi = 0; qi < NT; ++qi) {
    const int fr = rw + 16 * qi + c;
    const bool ok = fr < Tn;
    const int mf = ok ? fr : 0;
    lim[qi] = ok ? mf / s : 0;
    const size_t row = (size_t)b * Tn + mf;
    const size_t ri = row * H + h;
    L[qi] = a.lse[ri];
    Dv[qi] = a.Dr[ri];
    float sdot = 0.0f, pdot = 0.0f;
    bf16x8 kd[C::KS], vd[C::VS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const int k = 32 * ks + 8 * g;
      if (k < DH) {
        load8(qf[qi][ks], a.q + row * H * DH + h * DH + k);
        load8(kd[ks], a.KV + row * kvw + h * DH + k);
      } else {
        load8(qf[qi][ks], a.QR + ri * DR + (k - DH));
        load8(kd[ks], a.KR + row * DR + (k - DH));
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) sdot += (float)qf[qi][ks][e] * (float)kd[ks][e];
    }
#pragma unroll
    for (int ks = 0; ks < C::VS; ++ks) {
      load8(dof[qi][ks], a.dO + row * H * DH + h * DH + 32 * ks + 8 * g);
      load8(vd[ks], a.KV + row * kvw + (size_t)(H + h) * DH + 32 * ks + 8 * g);
#pragma unroll
      for (int e = 0; e < 8; ++e) pdot += (float)dof[qi][ks][e] * (float)vd[ks][e];
    }
    // Own column: score, weight, and dS.
    const float p = __builtin_amdgcn_exp2f(sum_g(sdot) * a.sl2 - L[qi]);
    const float dss = p * (sum_g(pdot) - Dv[qi]) * a.scale;
    // dQ and dQ^R start from the own column's dS K_m and dS K^R_m (O^T
    // layout: lane holds frame c, channels 16 mb + 4 g .. + 3).
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
      dq[qi][mb] = load4f(a.KV + row * kvw + h * DH + 16 * mb + 4 * g) * dss;
#pragma unroll
    for (int mb = 0; mb < C::RBK; ++mb)
      dqr[qi][mb] = load4f(a.KR + row * DR + 16 * mb + 4 * g) * dss;
    if (ok) {
      // Total dK, dV, dK^R of frame fr: the own column's terms plus the
      // key-role gradients when fr is a compact key (group-final with a
      // later frame in the sequence).
      const int j = fr / s;
      const bool key = (fr % s == s - 1) && j < a.nK;
      const float *kc = a.dKVc + ((size_t)b * a.nS + j) * kvw;
      const float *krc = a.dKRc + (((size_t)b * a.nS + j) * H + h) * DR;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const int k = 32 * ks + 8 * g;
        float v8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v8[e] = dss * (float)qf[qi][ks][e];
        if (k < DH) {
          if (key) {
            const f32x4 x0 = *(const f32x4 *)(kc + h * DH + k), x1 = *(const f32x4 *)(kc + h * DH + k + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) { v8[e] += x0[e]; v8[4 + e] += x1[e]; }
          }
          bf16x8 o;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = (bf16)v8[e];
          *(bf16x8 *)(a.dKV + row * kvw + h * DH + k) = o;
        } else {
          if (key) {
            const f32x4 x0 = *(const f32x4 *)(krc + (k - DH)), x1 = *(const f32x4 *)(krc + (k - DH) + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) { v8[e] += x0[e]; v8[4 + e] += x1[e]; }
          }
          float *dst = a.dKRh + ri * DR + (k - DH);
          *(f32x4 *)dst = (f32x4){v8[0], v8[1], v8[2], v8[3]};
          *(f32x4 *)(dst + 4) = (f32x4){v8[4], v8[5], v8[6], v8[7]};
        }
      }
#pragma unroll
      for (int ks = 0; ks < C::VS; ++ks) {
        const int k = 32 * ks + 8 * g;
        float v8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v8[e] = p * (float)dof[qi][ks][e];
        if (key) {
          const float *src = kc + (size_t)(H + h) * DH + k;
          const f32x4 x0 = *(const f32x4 *)src, x1 = *(const f32x4 *)(src + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) { v8[e] += x0[e]; v8[4 + e] += x1[e]; }
        }
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (bf16)v8[e];
        *(bf16x8 *)(a.dKV + row * kvw + (size_t)(H + h) * DH + k) = o;
      }
    }
  }
  asm volatile("" ::: "memory");

  const int wlast = min(rw + C::WROWS, Tn) - 1;
  const int wlim = wlast >= rw ? wlast / s : 0;
  const int glast = min(qtile * C::GROWS + C::GROWS, Tn) - 1;
  const int kmax = glast / s;
  const int nstage = (kmax + SROWS - 1) / SROWS;
  const int wst = (wlim + SROWS - 1) / SROWS;
  const int wmin = rw < Tn ? rw / s : 0;
  char *dummy = smem + NST * C::STAGE_B;
  const int u = (lane & 3) ^ swz(lane >> 2);
  auto issue = [&](int sidx) {
    char *sb = smem + (sidx % NST) * C::STAGE_B;
    const int row0 = sidx * SROWS;
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) {
      const int blk = wave + 4 * i;
      const bool real = blk < C::NBLK;
      const int tl = real ? blk / C::NSEG : 0, qq = real ? blk % C::NSEG : 0;
      const int key = min(row0 + tl * 16 + (lane >> 2), kmax - 1);
      const size_t fr = (size_t)b * Tn + (size_t)s * key + (s - 1);
      const char *seg;
      if (qq < C::KSEG) seg = (const char *)(a.KV + fr * kvw + h * DH) + qq * 64;
      else if (qq < C::KSEG + C::RSEG) seg = (const char *)(a.KR + fr * DR) + (qq - C::KSEG) * 64;
      else seg = (const char *)(a.KV + fr * kvw + (size_t)(H + h) * DH) + (qq - C::KSEG - C::RSEG) * 64;
      dma_seg(seg, real ? sb + tl * C::TILE_B + qq * 1024 : dummy, u);
    }
  };
  const int pro = min(NST, nstage);
  for (int k = 0; k < pro; ++k) issue(k);
  int last = pro - 1;

  for (int k = 0; k < nstage; ++k) {
    wait_stages<C::LPW>(last - k);
    bar();
    if (k >= 1 && k - 1 + NST < nstage) {
      issue(k - 1 + NST);
      last = k - 1 + NST;
    }
    if (k >= wst) continue;
    const char *sb = smem + (k % NST) * C::STAGE_B;
    const int kb = k * SROWS;
    // Transposed key tiles: K^T (channels 0 ..) and K^R^T (DH ..).
    bf16x8 kT[C::MB], krT[C::RBK];
    read_tr<C>(sb, 0, g, c, kT);
    read_tr<C>(sb, DH, g, c, krT);
    // S^T[key, q] and dP^T[key, q]: lane (g, c) holds frame column c, keys
    // 4g..4g+3 of the tile.
    f32x4 sc[2][NT], dp[2][NT];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const char *tile = sb + t * C::TILE_B;
#pragma unroll
      for (int qi = 0; qi < NT; ++qi) sc[t][qi] = dp[t][qi] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const bf16x8 af = *(const bf16x8 *)(tile + tile_off(c, ks * 64 + g * 16));
#pragma unroll
        for (int qi = 0; qi < NT; ++qi) sc[t][qi] = mma_k32(af, qf[qi][ks], sc[t][qi]);
      }
#pragma unroll
      for (int ks = 0; ks < C::VS; ++ks) {
        const bf16x8 af = *(const bf16x8 *)(tile + tile_off(c, C::OFF_C + ks * 64 + g * 16));
#pragma unroll
        for (int qi = 0; qi < NT; ++qi) dp[t][qi] = mma_k32(af, dof[qi][ks], dp[t][qi]);
      }
    }
    const bool full = kb + SROWS <= wmin;
    bf16x8 ds[NT];
#pragma unroll
    for (int qi = 0; qi < NT; ++qi)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool vis = full || (kb + 16 * t + 4 * g + e < lim[qi]);
          const float p = vis ? __builtin_amdgcn_exp2f(sc[t][qi][e] * a.sl2 - L[qi]) : 0.0f;
          ds[qi][4 * t + e] = (bf16)(p * (dp[t][qi][e] - Dv[qi]) * a.scale);
        }
#pragma unroll
    for (int qi = 0; qi < NT; ++qi) {
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) dq[qi][mb] = mma_k32(kT[mb], ds[qi], dq[qi][mb]);
#pragma unroll
      for (int mb = 0; mb < C::RBK; ++mb) dqr[qi][mb] = mma_k32(krT[mb], ds[qi], dqr[qi][mb]);
    }
  }

#pragma unroll
  for (int qi = 0; qi < NT; ++qi) {
    const int fr = rw + 16 * qi + c;
    if (fr < Tn) {
      const size_t row = (size_t)b * Tn + fr;
      bf16 *dst = a.dQ + row * a.ldq + h * DH + 4 * g;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) store4f(dst + 16 * mb, dq[qi][mb]);
      bf16 *dr = a.dQR + (row * H + h) * DR + 4 * g;
#pragma unroll
      for (int mb = 0; mb < C::RBK; ++mb) store4f(dr + 16 * mb, dqr[qi][mb]);
    }
  }
}

// D[row, h] = sum over the head's DH channels of dO * O: DH / 8 consecutive
// lanes (8 or 16) share a row, 16 bytes each (coalesced), and add their
// partial sums across those lanes.
__global__ __launch_bounds__(256) void rowdot_kernel(const bf16 *dO, const bf16 *O, int MH,
                                                     int DH, float *D) {
  const int lpr = DH / 8;   // lanes per row: a power of two dividing the wave
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t i = t / lpr;
  const int part = (int)(t % lpr);
  float acc = 0.0f;
  if (i < (size_t)MH) {
    const bf16x8 u = *(const bf16x8 *)(dO + i * DH + 8 * part);
    const bf16x8 v = *(const bf16x8 *)(O + i * DH + 8 * part);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)u[e] * (float)v[e];
  }
  for (int m = 1; m < lpr; m <<= 1) acc += __shfl_xor(acc, m);
  if (i < (size_t)MH && part == 0) D[i] = acc;
}

// dKR[row, ch] = sum_h dKRh[row, h, ch] (the RoPE key is shared by the heads).
template <class OutT>
__global__ __launch_bounds__(256) void head_sum_kernel(const float *dKRh, int M, int H, int DR,
                                                       OutT *dKR) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= M * DR) return;
  const int row = i / DR, ch = i % DR;
  float acc = 0.0f;
  for (int hh = 0; hh < H; ++hh) acc += dKRh[((size_t)row * H + hh) * DR + ch];
  dKR[i] = (OutT)acc;
}

// Reverse group scan and gate backward, one thread per (sequence b, slot j,
// latent channel).  dU runs over the frames of the group from the last one
// down: dU_i = dC'_i + dU_{i+1}.  Writes da (fp32 and bf16), dc's direct term
// dU w (fp32), c (bf16, for dW_hc), and adds dP_j.  BiasT: the storage type
// of b_hc.
template <class BiasT>
__global__ __launch_bounds__(256) void scan_gate_bwd_kernel(const float *dCp, const float *cg,
                                                            const BiasT *b_hc, const float *table,
                                                            int T, int R, int s, int nS,
                                                            float *da32, bf16 *dab, float *dc32,
                                                            bf16 *cb, float *dPpart) {
  const int b = blockIdx.y;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= nS * R) return;
  const int j = idx / R, ch = idx % R;
  const int i0 = j * s, i1 = min(i0 + s, T) - 1;
  const float bb = (float)b_hc[ch], pj = table[(size_t)j * R + ch];
  float dU = 0.0f, dPacc = 0.0f;
  for (int i = i1; i >= i0; --i) {
    const size_t row = (size_t)b * T + i;
    dU += dCp[row * R + ch];
    const float cv = cg[row * 2 * R + ch];
    const float av = cg[row * 2 * R + R + ch] + bb;
    const float w = sigmoidf(av * pj);
    const float dgate = dU * cv * w * (1.0f - w);
    const float da = dgate * pj;
    dPacc += dgate * av;
    da32[row * R + ch] = da;
    dab[row * R + ch] = (bf16)da;
    dc32[row * R + ch] = dU * w;
    cb[row * R + ch] = (bf16)cv;
  }
  dPpart[((size_t)b * nS + j) * R + ch] = dPacc;   // summed over b in order by sum_b_kernel
}

// out[j, ch] = sum over b = 0..B-1, in that order, of part[b, j, ch] for
// j < nS; rows nS..rows-1 of out are zero.
__global__ __launch_bounds__(256) void sum_b_kernel(const float *part, int B, int nS, int R,
                                                    int rows, float *out) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)rows * R) return;
  const size_t j = i / R;
  float acc = 0.0f;
  if (j < (size_t)nS)
    for (int b = 0; b < B; ++b) acc += part[(size_t)b * nS * R + i];
  out[i] = acc;
}

// out[N] = column sums of x [M, N] (fp32), in a fixed order.  Workgroup =
// 64 columns x 4 row lanes, one chunk of rows (blockIdx.y): row lane q adds
// rows q, q + 4, ... of the chunk into eight interleaved sums, and the four
// lanes' totals meet in LDS, so each chunk's partial does not depend on
// timing.  The last chunk of a column block to finish adds the partials in
// chunk order, again spread over the four row lanes (lane q: chunks q,
// q + 4, ...) and combined the same way.
__global__ __launch_bounds__(256) void colsum_kernel(const float *x, int M, int N, int rows,
                                                     float *part, int *ctr, float *out) {
  const int lane = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int ch = blockIdx.x * 64 + lane;
  const int chunks = gridDim.y;
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(part, (uint32_t)((size_t)chunks * N * 4));
  __shared__ float red[4][64];
  __shared__ int last;
  auto combine = [&](float v) {   // ((q0 + q1) + (q2 + q3)), in thread q == 0
    red[q][lane] = v;
    __syncthreads();
    return (red[0][lane] + red[1][lane]) + (red[2][lane] + red[3][lane]);
  };
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (ch < N) {
    const int r0 = blockIdx.y * rows, r1 = min(M, r0 + rows);
    int r = r0 + q;
    for (; r + 28 < r1; r += 32)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += x[(size_t)(r + 4 * e) * N + ch];
    for (int e = 0; r < r1; r += 4, ++e) acc[e & 7] += x[(size_t)r * N + ch];
  }
  const float mine = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  const float tot = combine(mine);
  if (q == 0 && ch < N) st_coh1(rp, (uint32_t)(((size_t)blockIdx.y * N + ch) * 4), tot);
  __syncthreads();   // this workgroup's partial stores have completed
  if (threadIdx.x == 0) last = ctr_add(&ctr[blockIdx.x], 1) == chunks - 1;
  __syncthreads();
  if (!last) return;
  float v = 0.0f;
  if (ch < N) {
    for (int c0 = q; c0 < chunks; c0 += 4 * 16) {
      float pv[16];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        pv[u] = ld_coh1(rp, (uint32_t)(((size_t)min(c0 + 4 * u, chunks - 1) * N + ch) * 4));
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (c0 + 4 * u < chunks) v += pv[u];
    }
  }
  __syncthreads();   // every lane has read red[] above before it is reused
  const float res = combine(v);
  if (q == 0 && ch < N) out[ch] = res;
  if (threadIdx.x == 0) __hip_atomic_store(&ctr[blockIdx.x], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float *p, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// out[C, R] = in[R, C]^T (bf16), 64x64 tiles through LDS.
__global__ __launch_bounds__(256) void transpose_kernel(const bf16 *in, int R, int C, int ldi,
                                                        bf16 *out, int ldo) {
  __shared__ bf16 t[64][66];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int rr = i / 64, cc = i % 64, r = r0 + rr, col = c0 + cc;
    t[rr][cc] = (r < R && col < C) ? in[(size_t)r * ldi + col] : (bf16)0.0f;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int cc = i / 64, rr = i % 64, r = r0 + rr, col = c0 + cc;
    if (r < R && col < C) out[(size_t)col * ldo + r] = t[rr][cc];
  }
}

// out[N1, N2] = A[M, N1]^T B[M, N2] (fp32).  M may be split over
// workgroups (blockIdx.z): each split then stores its partial tile, in row
// order, into its own slab of `part` (split z at z * N1 * N2 floats), and
// tn_sum_kernel adds the slabs in split order.  Workgroup tile 128 x 128,
// each wave 64 x 64 (4 x 4 MFMA tiles); per step 32 rows of A and B are
// staged in LDS as two 16-row tiles each (rows of 256 bytes), and both
// operands come from transposing reads (lane (g, c): column c of rows
// 4g..4g+3 of each tile -- the same row order for A and B, so the products
// pair the right rows).
constexpr int TN_T = 128;
__global__ __launch_bounds__(256) void tn_gemm_kernel(const bf16 *A, int lda, const bf16 *Bm,
                                                      int ldb, int M, int N1, int N2, int mchunk,
                                                      float *out, int ldo, float *part) {
  constexpr int RT = 16 * TN_T * 2;   // one 16-row tile: 16 rows x 256 bytes
  __shared__ __attribute__((aligned(1024))) char lds[2][2 * RT];   // [A|B][2 row tiles]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int n2_0 = blockIdx.x * TN_T, n1_0 = blockIdx.y * TN_T;
  const int m_lo = blockIdx.z * mchunk, m_hi = min(M, m_lo + mchunk);
  const int wy = wave >> 1, wx = wave & 1;
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // Staging: thread t moves 32 bytes of A and of B: row t/8 of the step,
  // 16-column chunk t%8 (two 8-column halves).  Rows past the split and
  // columns past N are zero.
  const int sr = tid >> 3, sc16 = (tid & 7) * 16;
  auto fetch = [&](const bf16 *X, int ld, int n0, int N, int m0, u32x4 (&v)[2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v[h] = (u32x4){0u, 0u, 0u, 0u};
      const int m = m0 + sr, n = n0 + sc16 + 8 * h;
      if (m < m_hi && n < N) {
        if (n + 8 <= N && ((((size_t)m * ld + n) & 7) == 0)) {
          v[h] = ldg16(X + (size_t)m * ld + n);
        } else {
          bf16x8 t8;
#pragma unroll
          for (int e = 0; e < 8; ++e) t8[e] = n + e < N ? X[(size_t)m * ld + n + e] : (bf16)0.0f;
          v[h] = __builtin_bit_cast(u32x4, t8);
        }
      }
    }
  };
  u32x4 va[2], vb[2];
  fetch(A, lda, n1_0, N1, m_lo, va);
  fetch(Bm, ldb, n2_0, N2, m_lo, vb);
  for (int m0 = m_lo; m0 < m_hi; m0 += 32) {
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int to = (sr >> 4) * RT + tile_off(sr & 15, (sc16 + 8 * h) * 2);
      *(u32x4 *)(lds[0] + to) = va[h];
      *(u32x4 *)(lds[1] + to) = vb[h];
    }
    __syncthreads();
    if (m0 + 32 < m_hi) {
      fetch(A, lda, n1_0, N1, m0 + 32, va);
      fetch(Bm, ldb, n2_0, N2, m0 + 32, vb);
    }
    bf16x8 fa[4], fb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const char *pa = lds[0] + tile_off(4 * g + (c >> 2), (64 * wy + 16 * i + 4 * (c & 3)) * 2);
      fa[i] = join(__builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_b4 *)pa),
                   __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_b4 *)(pa + RT)));
      const char *pb = lds[1] + tile_off(4 * g + (c >> 2), (64 * wx + 16 * i + 4 * (c & 3)) * 2);
      fb[i] = join(__builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_b4 *)pb),
                   __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_b4 *)(pb + RT)));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) acc[i][jj] = mma_k32(fa[i], fb[jj], acc[i][jj]);
  }
  // acc[i][jj]: lane (g, c) holds column n2 = .. + c, rows n1 = .. + 4g + e.
  float *dst = gridDim.z == 1 ? out : part + (size_t)blockIdx.z * N1 * N2;
  const int ld = gridDim.z == 1 ? ldo : N2;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int n2 = n2_0 + 64 * wx + 16 * jj + c;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n1 = n1_0 + 64 * wy + 16 * i + 4 * g + e;
        if (n1 < N1 && n2 < N2) dst[(size_t)n1 * ld + n2] = acc[i][jj][e];
      }
    }
}

// out[n1, n2] = sum over the splits, in split order, of the slabs of
// tn_gemm_kernel (one thread per output element).
__global__ __launch_bounds__(256) void tn_sum_kernel(const float *part, int splits, int N1, int N2,
                                                     float *out, int ldo) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x, n = (size_t)N1 * N2;
  if (i >= n) return;
  float v = 0.0f;
  int s = 0;
  for (; s + 8 <= splits; s += 8) {
    float pv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) pv[u] = part[(size_t)(s + u) * n + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) v += pv[u];
  }
  for (; s < splits; ++s) v += part[(size_t)s * n + i];
  out[(i / N2) * ldo + i % N2] = v;
}

}  // namespace

bool attn_bwd_supported(int dtype, int H, int d_h, int dR) {
  return dtype == 1 && ((d_h == 64 && dR == 32) || (d_h == 128 && dR == 64)) && H >= 1 && H <= 64;
}

namespace {
template <class C>
hipError_t attn_bwd_t(int B, int T, int H, int s, float scale, const void *q, const void *QR,
                      const void *KV, const void *KR, const void *dO, const float *lse,
                      const float *D, float *dKVc, float *dKRc, void *dKV, float *dKRh, void *dQ,
                      void *dQR, int ldq, hipStream_t stream) {
  const int nS = (T + s - 1) / s, nK = (T - 1) / s;
  float sl2 = scale * kLog2e;
  if (!(sl2 >= FLT_MIN)) sl2 = FLT_MIN;
  AttnBwdArgs a{(const bf16 *)q, (const bf16 *)QR, (const bf16 *)KV, (const bf16 *)KR,
                (const bf16 *)dO, lse, D, dKVc, dKRc, (bf16 *)dKV, dKRh, (bf16 *)dQ,
                (bf16 *)dQR, B, T, H, s, nS, nK, (T + C::GROWS - 1) / C::GROWS, sl2, scale, ldq};
  const size_t lds = (size_t)C::NST * C::STAGE_B + 1024;
  allow_lds<attn_bwd_dkdv_kernel<C>>();
  allow_lds<attn_bwd_dq_kernel<C>>();
  const int kblocks = (nK + C::GROWS - 1) / C::GROWS;
  if (kblocks > 0) {
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<C>, dim3(kblocks * B * H), dim3(256), lds, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(attn_bwd_dq_kernel<C>, dim3(a.tiles * B * H), dim3(256), lds, stream, a);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_attn_bwd(int B, int T, int H, int d_h, int s, float scale, const void *q,
                           const void *QR, const void *KV, const void *KR, const void *dO,
                           const float *lse, const float *D, float *dKVc, float *dKRc, void *dKV,
                           float *dKRh, void *dQ, void *dQR, int ldq, hipStream_t stream) {
  if (d_h == 128)
    return attn_bwd_t<Bw128>(B, T, H, s, scale, q, QR, KV, KR, dO, lse, D, dKVc, dKRc, dKV, dKRh,
                             dQ, dQR, ldq, stream);
  return attn_bwd_t<Bw64>(B, T, H, s, scale, q, QR, KV, KR, dO, lse, D, dKVc, dKRc, dKV, dKRh, dQ,
                          dQR, ldq, stream);
}

hipError_t launch_rowdot(const void *dO, const void *O, int MH, int d_h, float *D,
                         hipStream_t stream) {
  const size_t lanes = (size_t)MH * (d_h / 8);
  hipLaunchKernelGGL(rowdot_kernel, dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, stream,
                     (const bf16 *)dO, (const bf16 *)O, MH, d_h, D);
  return hipGetLastError();
}

hipError_t launch_head_sum(int dtype, const float *dKRh, int M, int H, int dR, void *dKR,
                           hipStream_t stream) {
  const dim3 grid((M * dR + 255) / 256);
  if (dtype == 0)
    hipLaunchKernelGGL(head_sum_kernel<float>, grid, dim3(256), 0, stream, dKRh, M, H, dR,
                       (float *)dKR);
  else
    hipLaunchKernelGGL(head_sum_kernel<bf16>, grid, dim3(256), 0, stream, dKRh, M, H, dR,
                       (bf16 *)dKR);
  return hipGetLastError();
}

hipError_t launch_scan_gate_bwd(int dtype, const float *dCp, const float *cg, const void *b_hc,
                                const float *table, int B, int T, int R, int s, float *da32,
                                void *dab, float *dc32, void *cb, float *dPpart, int rows,
                                float *dPtab, hipStream_t stream) {
  const int nS = (T + s - 1) / s;
  dim3 grid((unsigned)(((int64_t)nS * R + 255) / 256), B);
  if (dtype == 0)
    hipLaunchKernelGGL(scan_gate_bwd_kernel<float>, grid, dim3(256), 0, stream, dCp, cg,
                       (const float *)b_hc, table, T, R, s, nS, da32, (bf16 *)dab, dc32,
                       (bf16 *)cb, dPpart);
  else
    hipLaunchKernelGGL(scan_gate_bwd_kernel<bf16>, grid, dim3(256), 0, stream, dCp, cg,
                       (const bf16 *)b_hc, table, T, R, s, nS, da32, (bf16 *)dab, dc32,
                       (bf16 *)cb, dPpart);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sum_b_kernel, dim3((unsigned)(((size_t)rows * R + 255) / 256)), dim3(256), 0,
                     stream, dPpart, B, nS, R, rows, dPtab);
  return hipGetLastError();
}

namespace {
int colsum_chunks(int M) { return M < 256 ? (M > 0 ? M : 1) : 256; }
}  // namespace

size_t colsum_part_bytes(int M, int N) { return (size_t)colsum_chunks(M) * N * 4; }
int colsum_counters(int N) { return (N + 63) / 64; }

hipError_t launch_colsum(const float *x, int M, int N, float *part, int *ctr, float *out,
                         hipStream_t stream) {
  const int chunks = colsum_chunks(M), rows = (M + chunks - 1) / chunks;
  dim3 grid((N + 63) / 64, (M + rows - 1) / rows);
  hipLaunchKernelGGL(colsum_kernel, grid, dim3(256), 0, stream, x, M, N, rows, part, ctr, out);
  return hipGetLastError();
}

hipError_t launch_zero_i32(int *p, size_t n, hipStream_t stream) {
  return launch_zero_f32((float *)p, n, stream);   // all-zero bits either way
}

hipError_t launch_zero_f32(float *p, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p,
                     n);
  return hipGetLastError();
}

hipError_t launch_transpose(const void *in, int R, int C, int ldi, void *out, int ldo,
                            hipStream_t stream) {
  dim3 grid((C + 63) / 64, (R + 63) / 64);
  hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, stream, (const bf16 *)in, R, C, ldi,
                     (bf16 *)out, ldo);
  return hipGetLastError();
}

namespace {
struct TnPlan {
  int tiles, splits, mchunk;
};
TnPlan tn_plan(int M, int N1, int N2) {
  TnPlan p;
  p.tiles = ((N1 + TN_T - 1) / TN_T) * ((N2 + TN_T - 1) / TN_T);
  int splits = (768 + p.tiles - 1) / p.tiles;   // about three workgroups per CU
  const int maxs = (M + 255) / 256;             // at least 8 steps each
  if (splits > maxs) splits = maxs;
  if (splits > 64) splits = 64;
  if (splits < 1) splits = 1;
  p.mchunk = ((M + splits - 1) / splits + 31) / 32 * 32;
  p.splits = (M + p.mchunk - 1) / p.mchunk;
  return p;
}
// The 256 x 256 tile: about one workgroup per CU, at least 64 frames each.
TnPlan tn_big_plan(int M, int N1, int N2) {
  TnPlan p;
  p.tiles = ((N1 + 255) / 256) * ((N2 + 255) / 256);
  int splits = (256 + p.tiles - 1) / p.tiles;
  const int maxs = (M + 63) / 64;
  if (splits > maxs) splits = maxs;
  if (splits > 64) splits = 64;
  if (splits < 1) splits = 1;
  p.mchunk = ((M + splits - 1) / splits + 63) / 64 * 64;
  p.splits = (M + p.mchunk - 1) / p.mchunk;
  return p;
}
}  // namespace

size_t tn_gemm_part_bytes(int M, int N1, int N2) {
  const TnPlan p = tn_plan(M, N1, N2);
  size_t b = p.splits > 1 ? (size_t)p.splits * N1 * N2 * 4 : 0;
  if (tn_big_supported(N1, N2)) {
    const TnPlan q = tn_big_plan(M, N1, N2);
    if (q.splits > 1 && (size_t)q.splits * N1 * N2 * 4 > b) b = (size_t)q.splits * N1 * N2 * 4;
  }
  return b;
}
hipError_t launch_tn_gemm(const void *A, int lda, const void *Bm, int ldb, int M, int N1, int N2,
                          float *out, int ldo, float *part, hipStream_t stream) {
  // The large tile reads 16-byte row pieces with direct loads: it needs
  // 16-byte aligned rows.
  const bool big = tn_big_supported(N1, N2) && lda % 8 == 0 && ldb % 8 == 0 &&
                   ((uintptr_t)A & 15) == 0 && ((uintptr_t)Bm & 15) == 0;
  const TnPlan p = big ? tn_big_plan(M, N1, N2) : tn_plan(M, N1, N2);
  if (big) {
    const hipError_t e =
        launch_tn_big(A, lda, Bm, ldb, M, N1, N2, p.mchunk, p.splits, out, ldo, part, stream);
    if (e != hipSuccess) return e;
  } else {
    dim3 grid((N2 + TN_T - 1) / TN_T, (N1 + TN_T - 1) / TN_T, p.splits);
    hipLaunchKernelGGL(tn_gemm_kernel, grid, dim3(256), 0, stream, (const bf16 *)A, lda,
                       (const bf16 *)Bm, ldb, M, N1, N2, p.mchunk, out, ldo, part);
  }
  if (p.splits > 1) {
    const size_t n = (size_t)N1 * N2;
    hipLaunchKernelGGL(tn_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       (const float *)part, p.splits, N1, N2, out, ldo);
  }
  return hipGetLastError();
}

}  // namespace mtla
