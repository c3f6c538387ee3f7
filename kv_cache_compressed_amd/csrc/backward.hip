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
// split-M product A^T B for the weight gradients, and small helpers.

#include <float.h>
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace mtla {

namespace {

constexpr float kNegInfB = -INFINITY;
constexpr int DH = 64, DR = 32, QK = DH + DR;
// LDS row of a streamed frame, in the 16-row swizzled tile layout: 160 bf16
// (320 B, five 64-byte blocks).  Key rows: K_h | K^R | V_h.  Query rows:
// Q_h | Q^R_h | dO_h.  Byte offsets of the parts:
constexpr int RB = 320, NSEG = 5, OFF_B = 128, OFF_C = 192;
constexpr int TILE_B = 16 * RB, STAGE_B = 2 * TILE_B, SROWS = 32;
constexpr int NBLK = 2 * NSEG, LPW = (NBLK + 3) / 4;
constexpr int NST = 4;

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
  bf16 *dQ;          // [B*T, H*DH]
  bf16 *dQR;         // [B*T, H, DR]
  int B, T, H, s, nS, nK, tiles;
  float sl2, scale;
};

// ---------------------------------------------------------------------------
// Key-stationary pass: a workgroup owns 128 compact keys of one (sequence,
// head) -- 32 per wave, with K^T and V^T fragments in registers -- and
// streams the query frames that can see them (frame m sees key j iff
// j < floor(m/s)) through an LDS ring of 32-frame stages (Q | Q^R | dO).
// Per stage a wave computes S and dP for its 32 keys (the query tile from
// LDS as the A operand), P and dS on the VALU, and accumulates
// dV^T += dO^T P, dK^T += Q^T dS, dK^R^T += Q^R^T dS with the transposed
// query-side tiles from transposing reads.  Results are the key-role
// gradients of each compact key, written to dKVc / dKRc.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256, 2) void attn_bwd_dkdv_kernel(AttnBwdArgs a) {
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
  const int kb0 = kblk * 128;                 // first key of the workgroup
  const int kw0 = kb0 + 32 * wave;            // first key of this wave
  if (kb0 >= a.nK) return;                    // whole workgroup: uniform

  // K^T / V^T fragments (B operands): lane (g, c) holds key kw0 + 16 nk + c,
  // channels 32 ks + 8 g .. + 7.
  bf16x8 kf[2][3], vf[2][2];
#pragma unroll
  for (int nk = 0; nk < 2; ++nk) {
    const int j = min(kw0 + 16 * nk + c, a.nK - 1);
    const size_t fr = (size_t)b * Tn + (size_t)s * j + (s - 1);
#pragma unroll
    for (int ks = 0; ks < 3; ++ks) {
      const int k = 32 * ks + 8 * g;
      if (k < DH) load8(kf[nk][ks], a.KV + fr * kvw + h * DH + k);
      else load8(kf[nk][ks], a.KR + fr * DR + (k - DH));
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) load8(vf[nk][ks], a.KV + fr * kvw + (size_t)(H + h) * DH + 32 * ks + 8 * g);
  }
  f32x4 dv[2][4], dk[2][4], dkr[2][2];
#pragma unroll
  for (int nk = 0; nk < 2; ++nk) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) dv[nk][mb] = dk[nk][mb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    dkr[nk][0] = dkr[nk][1] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  asm volatile("" ::: "memory");

  // Query frames that see key kb0 start at s (kb0 + 1); stages of 32 frames.
  const int q0 = (s * (kb0 + 1)) / SROWS * SROWS;
  const int nstage = q0 < Tn ? (Tn - q0 + SROWS - 1) / SROWS : 0;
  const int wfirst = s * (kw0 + 1);           // first frame that sees a key of this wave
  char *dummy = smem + NST * STAGE_B;
  const int u = (lane & 3) ^ swz(lane >> 2);
  auto issue = [&](int sidx) {
    char *sb = smem + (sidx % NST) * STAGE_B;
    const int f0 = q0 + sidx * SROWS;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int blk = wave + 4 * i;
      const bool real = blk < NBLK;
      const int tl = real ? blk / NSEG : 0, qq = real ? blk % NSEG : 0;
      const int f = min(f0 + tl * 16 + (lane >> 2), Tn - 1);
      const size_t row = (size_t)b * Tn + f;
      const char *seg;
      if (qq < 2) seg = (const char *)(a.q + row * H * DH + h * DH) + qq * 64;
      else if (qq == 2) seg = (const char *)(a.QR + (row * H + h) * DR);
      else seg = (const char *)(a.dO + row * H * DH + h * DH) + (qq - 3) * 64;
      dma_seg(seg, real ? sb + tl * TILE_B + qq * 1024 : dummy, u);
    }
  };
  const int pro = min(NST, nstage);
  for (int k = 0; k < pro; ++k) issue(k);
  int last = pro - 1;

  for (int k = 0; k < nstage; ++k) {
    wait_stages<LPW>(last - k);
    bar();
    if (k >= 1 && k - 1 + NST < nstage) {
      issue(k - 1 + NST);
      last = k - 1 + NST;
    }
    const int fs = q0 + k * SROWS;            // first frame of the stage
    if (fs + SROWS <= wfirst) continue;       // no frame here sees this wave's keys
    const char *sb = smem + (k % NST) * STAGE_B;

    // S[q, key] and dP[q, key] for both 16-frame tiles: lane (g, c) holds key
    // column c, frames 4g..4g+3 of the tile.
    f32x4 sc[2][2], dp[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const char *tile = sb + t * TILE_B;
#pragma unroll
      for (int nk = 0; nk < 2; ++nk) sc[t][nk] = dp[t][nk] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 3; ++ks) {
        const bf16x8 af = *(const bf16x8 *)(tile + tile_off(c, ks * 64 + g * 16));
#pragma unroll
        for (int nk = 0; nk < 2; ++nk) sc[t][nk] = mma_k32(af, kf[nk][ks], sc[t][nk]);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 af = *(const bf16x8 *)(tile + tile_off(c, OFF_C + ks * 64 + g * 16));
#pragma unroll
        for (int nk = 0; nk < 2; ++nk) dp[t][nk] = mma_k32(af, vf[nk][ks], dp[t][nk]);
      }
    }
    // P and dS; frame f sees key j iff j < floor(f/s) (and f < T).
    bf16x8 pp[2], ds[2];
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
        for (int nk = 0; nk < 2; ++nk) {
          const int j = kw0 + 16 * nk + c;
          const float p = j < lim ? __builtin_amdgcn_exp2f(sc[t][nk][e] * a.sl2 - L) : 0.0f;
          pp[nk][4 * t + e] = (bf16)p;
          ds[nk][4 * t + e] = (bf16)(p * (dp[t][nk][e] - Dv) * a.scale);
        }
      }
    }
    // Transposed query-side tiles: Q^T (channels 0..63), Q^R^T (64..95),
    // dO^T (96..159), low half frames of tile 0, high half of tile 1.
    bf16x8 qT[4], qrT[2], doT[4];
    {
      uint32_t ad[8];
      bf16x4 v[8];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        ad[2 * mb] = tr_addr(sb, 16 * mb, g, c);
        ad[2 * mb + 1] = ad[2 * mb] + TILE_B;
      }
      ds_read_tr8(v, ad);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) qT[mb] = join(v[2 * mb], v[2 * mb + 1]);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        ad[2 * mb] = tr_addr(sb, 96 + 16 * mb, g, c);
        ad[2 * mb + 1] = ad[2 * mb] + TILE_B;
      }
      ds_read_tr8(v, ad);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) doT[mb] = join(v[2 * mb], v[2 * mb + 1]);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        ad[2 * mb] = tr_addr(sb, 64 + 16 * (mb & 1), g, c);
        ad[2 * mb + 1] = ad[2 * mb] + TILE_B;
      }
      ds_read_tr8(v, ad);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) qrT[mb] = join(v[2 * mb], v[2 * mb + 1]);
    }
    // dV^T += dO^T P,  dK^T += Q^T dS,  dK^R^T += Q^R^T dS.
#pragma unroll
    for (int nk = 0; nk < 2; ++nk) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) dv[nk][mb] = mma_k32(doT[mb], pp[nk], dv[nk][mb]);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) dk[nk][mb] = mma_k32(qT[mb], ds[nk], dk[nk][mb]);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) dkr[nk][mb] = mma_k32(qrT[mb], ds[nk], dkr[nk][mb]);
    }
  }

  // Key-role gradients of compact key (b, j): lane holds key column c,
  // channels 16 mb + 4g .. + 3.
#pragma unroll
  for (int nk = 0; nk < 2; ++nk) {
    const int j = kw0 + 16 * nk + c;
    if (j < a.nK) {
      float *row = a.dKVc + ((size_t)b * a.nS + j) * kvw;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        *(f32x4 *)(row + h * DH + 16 * mb + 4 * g) = dk[nk][mb];
        *(f32x4 *)(row + (size_t)(H + h) * DH + 16 * mb + 4 * g) = dv[nk][mb];
      }
      float *rr = a.dKRc + (((size_t)b * a.nS + j) * H + h) * DR;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) *(f32x4 *)(rr + 16 * mb + 4 * g) = dkr[nk][mb];
    }
  }
}

// ---------------------------------------------------------------------------
// Query-stationary pass: a workgroup owns 128 query frames of one (sequence,
// head), 32 per wave (two 16-row tiles) with Q, Q^R and dO fragments in
// registers; the compact keys stream through the forward's LDS ring
// (K | K^R | V).  Per stage: S^T and dP^T (key tile from LDS as the A
// operand), P and dS, then dQ^T += K^T dS^T and dQ^R^T += K^R^T dS^T with the
// transposed key tiles.  Each frame's own column is done in the prologue:
// it seeds dQ and dQ^R, and its key-side terms (dS_mm Q_m, P_mm dO_m,
// dS_mm Q^R_m) are added to the key-role gradients of the frame (if it is a
// compact key) and written out as the frame's total dK, dV and dK^R.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(AttnBwdArgs a) {
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
  const int rw = qtile * 128 + wave * 32;     // first frame of this wave

  bf16x8 qf[2][3], dof[2][2];
  f32x4 dq[2][4], dqr[2][2];
  float L[2], Dv[2];
  int lim[2];
#pragma unroll
  for (int qi = 0; qi < 2; ++qi) {
    const int fr = rw + 16 * qi + c;
    const bool ok = fr < Tn;
    const int mf = ok ? fr : 0;
    lim[qi] = ok ? mf / s : 0;
    const size_t row = (size_t)b * Tn + mf;
    const size_t ri = row * H + h;
    L[qi] = a.lse[ri];
    Dv[qi] = a.Dr[ri];
    float sdot = 0.0f, pdot = 0.0f;
    bf16x8 kd[3], vd[2];
#pragma unroll
    for (int ks = 0; ks < 3; ++ks) {
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
    for (int ks = 0; ks < 2; ++ks) {
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
    for (int mb = 0; mb < 4; ++mb)
      dq[qi][mb] = load4f(a.KV + row * kvw + h * DH + 16 * mb + 4 * g) * dss;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) dqr[qi][mb] = load4f(a.KR + row * DR + 16 * mb + 4 * g) * dss;
    if (ok) {
      // Total dK, dV, dK^R of frame fr: the own column's terms plus the
      // key-role gradients when fr is a compact key (group-final with a
      // later frame in the sequence).
      const int j = fr / s;
      const bool key = (fr % s == s - 1) && j < a.nK;
      const float *kc = a.dKVc + ((size_t)b * a.nS + j) * kvw;
      const float *krc = a.dKRc + (((size_t)b * a.nS + j) * H + h) * DR;
#pragma unroll
      for (int ks = 0; ks < 3; ++ks) {
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
      for (int ks = 0; ks < 2; ++ks) {
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

  const int wlast = min(rw + 32, Tn) - 1;
  const int wlim = wlast >= rw ? wlast / s : 0;
  const int glast = min(qtile * 128 + 128, Tn) - 1;
  const int kmax = glast / s;
  const int nstage = (kmax + SROWS - 1) / SROWS;
  const int wst = (wlim + SROWS - 1) / SROWS;
  const int wmin = rw < Tn ? rw / s : 0;
  char *dummy = smem + NST * STAGE_B;
  const int u = (lane & 3) ^ swz(lane >> 2);
  auto issue = [&](int sidx) {
    char *sb = smem + (sidx % NST) * STAGE_B;
    const int row0 = sidx * SROWS;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int blk = wave + 4 * i;
      const bool real = blk < NBLK;
      const int tl = real ? blk / NSEG : 0, qq = real ? blk % NSEG : 0;
      const int key = min(row0 + tl * 16 + (lane >> 2), kmax - 1);
      const size_t fr = (size_t)b * Tn + (size_t)s * key + (s - 1);
      const char *seg;
      if (qq < 2) seg = (const char *)(a.KV + fr * kvw + h * DH) + qq * 64;
      else if (qq == 2) seg = (const char *)(a.KR + fr * DR);
      else seg = (const char *)(a.KV + fr * kvw + (size_t)(H + h) * DH) + (qq - 3) * 64;
      dma_seg(seg, real ? sb + tl * TILE_B + qq * 1024 : dummy, u);
    }
  };
  const int pro = min(NST, nstage);
  for (int k = 0; k < pro; ++k) issue(k);
  int last = pro - 1;

  for (int k = 0; k < nstage; ++k) {
    wait_stages<LPW>(last - k);
    bar();
    if (k >= 1 && k - 1 + NST < nstage) {
      issue(k - 1 + NST);
      last = k - 1 + NST;
    }
    if (k >= wst) continue;
    const char *sb = smem + (k % NST) * STAGE_B;
    const int kb = k * SROWS;
    // Transposed key tiles: K^T (channels 0..63) and K^R^T (64..95).
    bf16x8 kT[4], krT[2];
    {
      uint32_t ad[8];
      bf16x4 v[8];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        ad[2 * mb] = tr_addr(sb, 16 * mb, g, c);
        ad[2 * mb + 1] = ad[2 * mb] + TILE_B;
      }
      ds_read_tr8(v, ad);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) kT[mb] = join(v[2 * mb], v[2 * mb + 1]);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        ad[2 * mb] = tr_addr(sb, 64 + 16 * (mb & 1), g, c);
        ad[2 * mb + 1] = ad[2 * mb] + TILE_B;
      }
      ds_read_tr8(v, ad);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) krT[mb] = join(v[2 * mb], v[2 * mb + 1]);
    }
    // S^T[key, q] and dP^T[key, q]: lane (g, c) holds frame column c, keys
    // 4g..4g+3 of the tile.
    f32x4 sc[2][2], dp[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const char *tile = sb + t * TILE_B;
#pragma unroll
      for (int qi = 0; qi < 2; ++qi) sc[t][qi] = dp[t][qi] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 3; ++ks) {
        const bf16x8 af = *(const bf16x8 *)(tile + tile_off(c, ks * 64 + g * 16));
#pragma unroll
        for (int qi = 0; qi < 2; ++qi) sc[t][qi] = mma_k32(af, qf[qi][ks], sc[t][qi]);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 af = *(const bf16x8 *)(tile + tile_off(c, OFF_C + ks * 64 + g * 16));
#pragma unroll
        for (int qi = 0; qi < 2; ++qi) dp[t][qi] = mma_k32(af, dof[qi][ks], dp[t][qi]);
      }
    }
    const bool full = kb + SROWS <= wmin;
    bf16x8 ds[2];
#pragma unroll
    for (int qi = 0; qi < 2; ++qi)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool vis = full || (kb + 16 * t + 4 * g + e < lim[qi]);
          const float p = vis ? __builtin_amdgcn_exp2f(sc[t][qi][e] * a.sl2 - L[qi]) : 0.0f;
          ds[qi][4 * t + e] = (bf16)(p * (dp[t][qi][e] - Dv[qi]) * a.scale);
        }
#pragma unroll
    for (int qi = 0; qi < 2; ++qi) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) dq[qi][mb] = mma_k32(kT[mb], ds[qi], dq[qi][mb]);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) dqr[qi][mb] = mma_k32(krT[mb], ds[qi], dqr[qi][mb]);
    }
  }

#pragma unroll
  for (int qi = 0; qi < 2; ++qi) {
    const int fr = rw + 16 * qi + c;
    if (fr < Tn) {
      const size_t row = (size_t)b * Tn + fr;
      bf16 *dst = a.dQ + row * H * DH + h * DH + 4 * g;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) store4f(dst + 16 * mb, dq[qi][mb]);
      bf16 *dr = a.dQR + (row * H + h) * DR + 4 * g;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) store4f(dr + 16 * mb, dqr[qi][mb]);
    }
  }
}

// D[row, h] = sum over the head's channels of dO * O: eight consecutive
// lanes share a 64-channel row, 16 bytes each (coalesced), and add their
// partial sums across the eight lanes.
__global__ __launch_bounds__(256) void rowdot_kernel(const bf16 *dO, const bf16 *O, int MH,
                                                     float *D) {
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t i = t >> 3;
  const int part = (int)(t & 7);
  float acc = 0.0f;
  if (i < (size_t)MH) {
    const bf16x8 u = *(const bf16x8 *)(dO + i * DH + 8 * part);
    const bf16x8 v = *(const bf16x8 *)(O + i * DH + 8 * part);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)u[e] * (float)v[e];
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  if (i < (size_t)MH && part == 0) D[i] = acc;
}

// dKR[row, ch] = sum_h dKRh[row, h, ch] (the RoPE key is shared by the heads).
__global__ __launch_bounds__(256) void head_sum_kernel(const float *dKRh, int M, int H,
                                                       bf16 *dKR) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= M * DR) return;
  const int row = i / DR, ch = i % DR;
  float acc = 0.0f;
  for (int hh = 0; hh < H; ++hh) acc += dKRh[((size_t)row * H + hh) * DR + ch];
  dKR[i] = (bf16)acc;
}

// Reverse group scan and gate backward, one thread per (sequence b, slot j,
// latent channel).  dU runs over the frames of the group from the last one
// down: dU_i = dC'_i + dU_{i+1}.  Writes da (fp32 and bf16), dc's direct term
// dU w (fp32), c (bf16, for dW_hc), and adds dP_j.
__global__ __launch_bounds__(256) void scan_gate_bwd_kernel(const float *dCp, const float *cg,
                                                            const bf16 *b_hc, const float *table,
                                                            int T, int R, int s, int nS,
                                                            float *da32, bf16 *dab, float *dc32,
                                                            bf16 *cb, float *dPtab) {
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
  atomicAdd(dPtab + (size_t)j * R + ch, dPacc);
}

// out[ch] += column sums of x [M, N] (fp32), each workgroup a block of rows
// (eight independent partial sums per thread keep eight loads in flight).
__global__ __launch_bounds__(256) void colsum_kernel(const float *x, int M, int N, int rows,
                                                     float *out) {
  const int ch = blockIdx.x * 256 + threadIdx.x;
  if (ch >= N) return;
  const int r0 = blockIdx.y * rows, r1 = min(M, r0 + rows);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int r = r0;
  for (; r + 8 <= r1; r += 8)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += x[(size_t)(r + e) * N + ch];
  for (; r < r1; ++r) acc[0] += x[(size_t)r * N + ch];
  atomicAdd(out + ch, ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7])));
}

__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const float *x, size_t n, bf16 *y) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  if (i + 4 <= n) {
    store4f(y + i, *(const f32x4 *)(x + i));
  } else {
    for (size_t k = i; k < n; ++k) y[k] = (bf16)x[k];
  }
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

// out[N1, N2] += A[M, N1]^T B[M, N2] over the rows of this split (fp32,
// added atomically: the caller zeroes `out`).  Workgroup tile 64 x 64, each
// wave 32 x 32 (2 x 2 MFMA tiles); per step 32 rows of A and B are staged in
// LDS as two 16-row tiles each, and both operands come from transposing
// reads (lane (g, c): column c of rows 4g..4g+3 of each tile -- the same
// row order for A and B, so the products pair the right rows).
__global__ __launch_bounds__(256) void tn_gemm_kernel(const bf16 *A, int lda, const bf16 *Bm,
                                                      int ldb, int M, int N1, int N2, int mchunk,
                                                      float *out, int ldo) {
  __shared__ __attribute__((aligned(1024))) char lds[2][2 * 2048];   // [A|B][2 tiles x 2 blocks]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int n2_0 = blockIdx.x * 64, n1_0 = blockIdx.y * 64;
  const int m_lo = blockIdx.z * mchunk, m_hi = min(M, m_lo + mchunk);
  const int wy = wave >> 1, wx = wave & 1;
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) acc[i][0] = acc[i][1] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // Staging: thread t moves 16 bytes of A and of B: row t/8 of the step,
  // 8-column chunk t%8.
  const int sr = tid >> 3, sc8 = (tid & 7) * 8;
  auto fetch = [&](const bf16 *X, int ld, int n0, int N, int m0) {
    u32x4 v = (u32x4){0u, 0u, 0u, 0u};
    const int m = m0 + sr, n = n0 + sc8;
    if (m < m_hi && n < N) {
      if (n + 8 <= N && ((((size_t)m * ld + n) & 7) == 0)) {
        v = ldg16(X + (size_t)m * ld + n);
      } else {
        bf16x8 t8;
#pragma unroll
        for (int e = 0; e < 8; ++e) t8[e] = n + e < N ? X[(size_t)m * ld + n + e] : (bf16)0.0f;
        v = __builtin_bit_cast(u32x4, t8);
      }
    }
    return v;
  };
  u32x4 va = fetch(A, lda, n1_0, N1, m_lo), vb = fetch(Bm, ldb, n2_0, N2, m_lo);
  for (int m0 = m_lo; m0 < m_hi; m0 += 32) {
    __syncthreads();
    const int to = (sr >> 4) * 2048 + tile_off(sr & 15, sc8 * 2);
    *(u32x4 *)(lds[0] + to) = va;
    *(u32x4 *)(lds[1] + to) = vb;
    __syncthreads();
    if (m0 + 32 < m_hi) {
      va = fetch(A, lda, n1_0, N1, m0 + 32);
      vb = fetch(Bm, ldb, n2_0, N2, m0 + 32);
    }
    bf16x8 fa[2], fb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const char *pa = lds[0] + tile_off(4 * g + (c >> 2), (32 * wy + 16 * i + 4 * (c & 3)) * 2);
      fa[i] = join(__builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_b4 *)pa),
                   __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_b4 *)(pa + 2048)));
      const char *pb = lds[1] + tile_off(4 * g + (c >> 2), (32 * wx + 16 * i + 4 * (c & 3)) * 2);
      fb[i] = join(__builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_b4 *)pb),
                   __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_b4 *)(pb + 2048)));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) acc[i][jj] = mma_k32(fa[i], fb[jj], acc[i][jj]);
  }
  // acc[i][jj]: lane (g, c) holds column n2 = .. + c, rows n1 = .. + 4g + e.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int n2 = n2_0 + 32 * wx + 16 * jj + c;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n1 = n1_0 + 32 * wy + 16 * i + 4 * g + e;
        if (n1 < N1 && n2 < N2) atomicAdd(out + (size_t)n1 * ldo + n2, acc[i][jj][e]);
      }
    }
}

}  // namespace

bool attn_bwd_supported(int dtype, int H, int d_h, int dR) {
  return dtype == 1 && d_h == DH && dR == DR && H >= 1 && H <= 64;
}

hipError_t launch_attn_bwd(int B, int T, int H, int s, float scale, const void *q, const void *QR,
                           const void *KV, const void *KR, const void *dO, const float *lse,
                           const float *D, float *dKVc, float *dKRc, void *dKV, float *dKRh,
                           void *dQ, void *dQR, hipStream_t stream) {
  const int nS = (T + s - 1) / s, nK = (T - 1) / s;
  float sl2 = scale * kLog2e;
  if (!(sl2 >= FLT_MIN)) sl2 = FLT_MIN;
  AttnBwdArgs a{(const bf16 *)q, (const bf16 *)QR, (const bf16 *)KV, (const bf16 *)KR,
                (const bf16 *)dO, lse, D, dKVc, dKRc, (bf16 *)dKV, dKRh, (bf16 *)dQ,
                (bf16 *)dQR, B, T, H, s, nS, nK, (T + 127) / 128, sl2, scale};
  const size_t lds = (size_t)NST * STAGE_B + 1024;
  allow_lds<attn_bwd_dkdv_kernel>();
  allow_lds<attn_bwd_dq_kernel>();
  const int kblocks = (nK + 127) / 128;
  if (kblocks > 0) {
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel, dim3(kblocks * B * H), dim3(256), lds, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(attn_bwd_dq_kernel, dim3(a.tiles * B * H), dim3(256), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_rowdot(const void *dO, const void *O, int MH, float *D, hipStream_t stream) {
  hipLaunchKernelGGL(rowdot_kernel, dim3((unsigned)(((size_t)MH * 8 + 255) / 256)), dim3(256), 0,
                     stream,
                     (const bf16 *)dO, (const bf16 *)O, MH, D);
  return hipGetLastError();
}

hipError_t launch_head_sum(const float *dKRh, int M, int H, void *dKR, hipStream_t stream) {
  hipLaunchKernelGGL(head_sum_kernel, dim3((M * DR + 255) / 256), dim3(256), 0, stream, dKRh, M, H,
                     (bf16 *)dKR);
  return hipGetLastError();
}

hipError_t launch_scan_gate_bwd(const float *dCp, const float *cg, const void *b_hc,
                                const float *table, int B, int T, int R, int s, float *da32,
                                void *dab, float *dc32, void *cb, float *dPtab,
                                hipStream_t stream) {
  const int nS = (T + s - 1) / s;
  dim3 grid((unsigned)(((int64_t)nS * R + 255) / 256), B);
  hipLaunchKernelGGL(scan_gate_bwd_kernel, grid, dim3(256), 0, stream, dCp, cg, (const bf16 *)b_hc,
                     table, T, R, s, nS, da32, (bf16 *)dab, dc32, (bf16 *)cb, dPtab);
  return hipGetLastError();
}

hipError_t launch_colsum(const float *x, int M, int N, float *out, hipStream_t stream) {
  const int rows = 64;
  dim3 grid((N + 255) / 256, (M + rows - 1) / rows);
  hipLaunchKernelGGL(colsum_kernel, grid, dim3(256), 0, stream, x, M, N, rows, out);
  return hipGetLastError();
}

hipError_t launch_f32_to_bf16(const float *x, size_t n, void *y, hipStream_t stream) {
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3((unsigned)((n + 1023) / 1024)), dim3(256), 0, stream,
                     x, n, (bf16 *)y);
  return hipGetLastError();
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

hipError_t launch_tn_gemm(const void *A, int lda, const void *Bm, int ldb, int M, int N1, int N2,
                          float *out, int ldo, hipStream_t stream) {
  const int tiles = ((N1 + 63) / 64) * ((N2 + 63) / 64);
  int splits = (1024 + tiles - 1) / tiles;                 // about 1024 workgroups
  const int maxs = (M + 255) / 256;                         // at least 8 steps each
  if (splits > maxs) splits = maxs;
  if (splits < 1) splits = 1;
  const int mchunk = ((M + splits - 1) / splits + 31) / 32 * 32;
  splits = (M + mchunk - 1) / mchunk;
  dim3 grid((N2 + 63) / 64, (N1 + 63) / 64, splits);
  hipLaunchKernelGGL(tn_gemm_kernel, grid, dim3(256), 0, stream, (const bf16 *)A, lda,
                     (const bf16 *)Bm, ldb, M, N1, N2, mchunk, out, ldo);
  return hipGetLastError();
}

}  // namespace mtla
