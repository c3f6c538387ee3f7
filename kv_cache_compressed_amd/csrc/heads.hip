// Unabsorbed (per-head) form of the MTLA parallel forward on gfx950: the
// stride-aware masked attention at head width, with explicit per-head keys
// and values computed from the intermediate states.
//
// [Notes] = "Multi-head Temporal Latent Attention" paper notes (zhaoyang97
// Paper-Notes): key designs / stride-aware causal mask and decoupled RoPE
// (training may use the uncompressed RoPE keys); [Fig1] = sciencestack.ai
// page, Figure 1 (the per-head maps W_Q, W_K, W_V, W_O before they are
// absorbed into the query and output maps).
//
// For head h the keys are K_h = C' W_K^(h) and the values V_h = C' W_V^(h)
// (d_h = 64 wide each), the queries Q_h = X W_Q^(h), and the score of query m
// and column n is (Q_h[m] . K_h[n] + Q^R_h[m] . K^R[n]) * scale over the
// columns the mask lets m see: the group-final frames before m and m itself.
// Absorption trades these explicit per-head products for attention at the
// latent width r = 4 d_h; in the parallel form, where every intermediate state
// is a key, the explicit form needs 2 (d_h + d_hR) + 2 d_h = 320 flops per
// visible pair and head against 2 (r + d_hR) + 2 r = 1088.
//
// Kernel layout.  A workgroup owns 256 consecutive query frames of one
// (sequence, head); each of its four waves owns 64 of them (four 16-row
// tiles) with their queries and O^T accumulators in registers.  The compact
// keys of the head -- group-final frames e_j = s j + s - 1, j < floor(m/s) --
// stream through a ring of LDS stages of 32 keys, each key row assembled by
// direct global->LDS loads from three places: K_h[e_j] (128 B), K^R[e_j]
// (64 B) and V_h[e_j] (128 B), in the swizzled 16-row tile layout of the
// other attention kernels.  Per stage a wave computes S^T = K Q^T for both
// 16-key tiles (K=32 MFMAs over the 96 score channels, each K fragment
// feeding four products), runs the online softmax in log2 units with the
// reference maximum moved lazily (by steps > 2^8), and accumulates
// O^T += V^T P^T with one K=32 MFMA per (channel block, row tile): V^T comes
// from gfx950's transposing LDS reads, P^T straight from the score registers
// (the two tiles' keys 4g..4g+3 are the MFMA's k = 8g..8g+7).  Each query's
// own column seeds its online softmax (score, weight 1, value V_h[m]).

#include <float.h>
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace mtla {

namespace {

constexpr float kNegInfH = -INFINITY;

struct HeadsArgs {
  const bf16 *q;    // [B*T, H*DH]: Q_h at column h*DH
  const bf16 *QR;   // [B*T, H, DR]
  const bf16 *KV;   // [B*T, 2*H*DH]: K_h at column h*DH, V_h at (H + h)*DH
  const bf16 *KR;   // [B*T, DR]
  bf16 *O;          // [B*T, H*DH]
  float *lse;       // [B*T, H] or null: log2 of each row's softmax sum, in scaled log2 units
  int B, T, H, s, tiles, nst;
  float sl2;        // scale * log2(e)
};

#ifndef MTLA_HEADS_WAVES
#define MTLA_HEADS_WAVES 4
#endif
#ifndef MTLA_HEADS_NST
#define MTLA_HEADS_NST 5
#endif

// Head widths (DH, DR): (64, 32) and, at the LLM-scale model dims
// (r = 4 d_h = 512), (128, 64).  NQ 16-row query tiles per wave, NST ring
// stages, OCC workgroups per CU (the register and LDS budget: at d_h = 128 a
// wave holds two row tiles so that queries, accumulators and both tiles'
// K^T fragments stay within the 256 registers of two waves per SIMD).
template <int DH_, int DR_, int NQ_, int NST_, int OCC_> struct HdCfg {
  static constexpr int DH = DH_, DR = DR_, QK = DH + DR;  // score channels
  static constexpr int RB = (QK + DH) * 2;                // LDS key row K | K^R | V
  static constexpr int NSEG = RB / 64;                    // 64-byte blocks per row
  static constexpr int KSEG = DH * 2 / 64, RSEG = DR * 2 / 64;   // blocks of K, of K^R
  static constexpr int VOFF = QK * 2;                     // byte offset of V in a key row
  static constexpr int KS = QK / 32, MB = DH / 16;        // k-steps, channel blocks
  static constexpr int NW = MTLA_HEADS_WAVES;            // waves per workgroup
  static constexpr int NQ = NQ_, ROWS_W = 16 * NQ, ROWS = NW * ROWS_W;
  static constexpr int SROWS = 32, TILE_B = 16 * RB, STAGE_B = 2 * TILE_B;
  static constexpr int NBLK = 2 * NSEG, LPW = (NBLK + NW - 1) / NW;
  static constexpr int NST = NST_;   // ring stages (>= 3: slots k, k+1 and the refill)
  static constexpr int OCC = OCC_;
  static_assert(NST >= 3, "the pipeline reads two stages while a third is refilled");
  static_assert(QK % 32 == 0 && DH % 32 == 0 && DR % 32 == 0, "whole 64-byte blocks");
  static_assert(MB % 4 == 0, "transposing reads issued eight at a time");
  static_assert(OCC * (NST * STAGE_B + 1024) <= 160 * 1024, "LDS per CU");
};
using HdCfg64 = HdCfg<64, 32, 4, MTLA_HEADS_NST, 2>;
using HdCfg128 = HdCfg<128, 64, 2, 3, 2>;

template <class C>
__global__ __launch_bounds__(64 * C::NW, C::OCC) void heads_attn_kernel(HeadsArgs a) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int H = a.H, Tn = a.T, s = a.s, nst = a.nst;
  const int BH = a.B * H;

  // Heavy tiles (late queries) first; when the (sequence, head) pairs split
  // evenly over the 8 XCDs, each XCD serves whole pairs so their keys stay in
  // its L2.
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
  const size_t kvw = (size_t)2 * H * C::DH;     // KV row width (elements)
  const int rw = qtile * C::ROWS + wave * C::ROWS_W;   // first query frame of this wave

  // Queries, the self term and the initial state of every row of the wave.
  bf16x8 q[C::NQ][C::KS];
  f32x4 o[C::NQ][C::MB];
  float m[C::NQ], l[C::NQ];
  int lim[C::NQ];
#pragma unroll
  for (int qi = 0; qi < C::NQ; ++qi) {
    // Frames past the end read frame 0 (valid memory) and are never written.
    const int fr = rw + 16 * qi + c;
    const bool ok = fr < Tn;
    const int mf = ok ? fr : 0;
    lim[qi] = ok ? mf / s : 0;
    const size_t row = (size_t)b * Tn + mf;
    float dot = 0.0f;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const int k = 32 * ks + 8 * g;
      bf16x8 d;
      if (k < C::DH) {
        load8(q[qi][ks], a.q + row * H * C::DH + h * C::DH + k);
        load8(d, a.KV + row * kvw + h * C::DH + k);
      } else {
        load8(q[qi][ks], a.QR + (row * H + h) * C::DR + (k - C::DH));
        load8(d, a.KR + row * C::DR + (k - C::DH));
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) dot += (float)q[qi][ks][e] * (float)d[e];
    }
    m[qi] = sum_g(dot) * a.sl2;
    l[qi] = (g == 0) ? 1.0f : 0.0f;
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
      o[qi][mb] = load4f(a.KV + row * kvw + (size_t)(H + h) * C::DH + 16 * mb + 4 * g);
  }
  asm volatile("" ::: "memory");

  // Keys this wave / workgroup can see at most (limits grow with the frame).
  const int wlast = min(rw + C::ROWS_W, Tn) - 1;
  const int wlim = wlast >= rw ? wlast / s : 0;
  const int glast = min(qtile * C::ROWS + C::ROWS, Tn) - 1;
  const int kmax = glast / s;
  const int nstage = (kmax + C::SROWS - 1) / C::SROWS;
  char *dummy = smem + nst * C::STAGE_B;
  const int u = (lane & 3) ^ swz(lane >> 2);   // 16-byte chunk this lane moves

  // Stage sidx: keys 32 sidx .. 32 sidx + 31 (clamped to kmax - 1; the
  // clamped rows are masked by every query's limit).  Block (tl, qq) holds
  // the 64-byte segment qq of the 16 rows of tile tl.
  auto issue = [&](int sidx) {
    char *sb = smem + (sidx % nst) * C::STAGE_B;
    const int row0 = sidx * C::SROWS;
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) {
      const int blk = wave + C::NW * i;
      const bool real = blk < C::NBLK;
      const int tl = real ? blk / C::NSEG : 0, qq = real ? blk % C::NSEG : 0;
      const int key = min(row0 + tl * 16 + (lane >> 2), kmax - 1);
      const size_t fr = (size_t)b * Tn + (size_t)s * key + (s - 1);
      const char *seg;
      if (qq < C::KSEG) seg = (const char *)(a.KV + fr * kvw + h * C::DH) + qq * 64;
      else if (qq < C::KSEG + C::RSEG) seg = (const char *)(a.KR + fr * C::DR) + (qq - C::KSEG) * 64;
      else seg = (const char *)(a.KV + fr * kvw + (size_t)(H + h) * C::DH) + (qq - C::KSEG - C::RSEG) * 64;
      __builtin_amdgcn_global_load_lds((const void *)(seg + u * 16),
                                       (lds_void *)(real ? sb + tl * C::TILE_B + qq * 1024 : dummy),
                                       16, 0, 0);
    }
  };
  const int pro = min(nst, nstage);
  for (int k = 0; k < pro; ++k) issue(k);
  int last = pro - 1;   // newest stage issued so far

  // Stages holding a key some row of this wave can see, and the keys every
  // valid row of the wave can see (no mask needed below them).
  const int wst = (wlim + C::SROWS - 1) / C::SROWS;
  const int wmin = rw < Tn ? rw / s : 0;

  // K^T fragments of stage kk (row c of each tile, this lane group's chunk
  // of every k-step), and S^T of one tile from them: each fragment feeds NQ
  // products.
  auto read_k = [&](int kk, bf16x8 (&kf)[2][C::KS]) {
    const char *sb = smem + (kk % nst) * C::STAGE_B;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
        kf[t][ks] = *(const bf16x8 *)(sb + t * C::TILE_B + tile_off(c, ks * 64 + g * 16));
  };
  auto mma_tile = [&](const bf16x8 (&kf)[C::KS], f32x4 (&sc)[C::NQ]) {
#pragma unroll
    for (int qi = 0; qi < C::NQ; ++qi) sc[qi] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
      for (int qi = 0; qi < C::NQ; ++qi) sc[qi] = mma_k32(kf[ks], q[qi][ks], sc[qi]);
  };

  // Software pipeline: the scores of stage k+1 are computed while the
  // softmax of stage k runs -- tile 0's products beside the row maxima,
  // tile 1's beside the exponentials -- so that each wave has matrix
  // products to issue between its dependent vector operations.
  f32x4 scur[2][C::NQ];
  if (nstage > 0) {
    wait_stages<C::LPW>(last);           // stage 0
    bar();
    if (wst > 0) {
      bf16x8 kf[2][C::KS];
      read_k(0, kf);
      mma_tile(kf[0], scur[0]);
      mma_tile(kf[1], scur[1]);
    }
  }
  const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
  for (int k = 0; k < nstage; ++k) {
    // Stage k+1 has landed once at most last - (k+1) stages issued after it
    // are still in flight (this wave's loads complete in issue order).
    if (k + 1 < nstage) wait_stages<C::LPW>(last - (k + 1));
    bar();
    // Every wave is past stage k-1 here (its last reads of that slot were
    // the V^T reads of iteration k-1): refill the slot.
    if (k >= 1 && k - 1 + nst < nstage) {
      issue(k - 1 + nst);
      last = k - 1 + nst;
    }
    if (k >= wst) continue;               // nothing this wave can see from here on
    const char *sb = smem + (k % nst) * C::STAGE_B;
    const int kb = k * C::SROWS;

    // K^T of stage k+1 (past the last stage the slot holds stale data whose
    // products go unused), then V^T of stage k: lane (g, c) addresses row
    // 4g + c/4, channels 16 mb + 4 (c%4)..+3; the transposing read hands it
    // channel 16 mb + c of keys 4g..4g+3 (tile 0: low half, tile 1: high
    // half).  The eight transposing reads go out in one asm statement that
    // waits for all of this wave's LDS reads (ds_read_tr8): the builtin form
    // would make the compiler wait for every direct-to-LDS load in flight.
    bf16x8 kf[2][C::KS];
    read_k(k + 1, kf);
    bf16x8 vf[C::MB];
#pragma unroll
    for (int m0 = 0; m0 < C::MB; m0 += 4) {
      uint32_t ad[8];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const char *p0 = sb + tile_off(4 * g + (c >> 2), C::VOFF + (16 * (m0 + mb) + 4 * (c & 3)) * 2);
        ad[2 * mb] = lds_addr(p0);
        ad[2 * mb + 1] = lds_addr(p0 + C::TILE_B);
      }
      bf16x4 vv[8];
      ds_read_tr8(vv, ad);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        vf[m0 + mb] = __builtin_shufflevector(vv[2 * mb], vv[2 * mb + 1], 0, 1, 2, 3, 4, 5, 6, 7);
    }

    // Online softmax of stage k per row (lane holds keys 4g..4g+3 of each
    // tile), in log2 units; the reference maximum moves only by steps > 2^8.
    // Keys a row cannot see become -inf (only on stages that reach past the
    // keys every row of the wave sees).
    if (kb + C::SROWS > wmin) {
#pragma unroll
      for (int qi = 0; qi < C::NQ; ++qi)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (!(kb + 16 * t + 4 * g + e < lim[qi])) scur[t][qi][e] = kNegInfH;
    }
    f32x4 snext[2][C::NQ];
    mma_tile(kf[0], snext[0]);
    bool up_any = false;
    float mnew[C::NQ];
#pragma unroll
    for (int qi = 0; qi < C::NQ; ++qi) {
      float mx = fmaxf(fmaxf(fmaxf(scur[0][qi][0], scur[0][qi][1]), fmaxf(scur[0][qi][2], scur[0][qi][3])),
                       fmaxf(fmaxf(scur[1][qi][0], scur[1][qi][1]), fmaxf(scur[1][qi][2], scur[1][qi][3])));
      mx = max_g(mx) * a.sl2;
      const bool up = mx > m[qi] + 8.0f;
      mnew[qi] = up ? mx : m[qi];
      up_any |= up;
    }
#pragma unroll
    for (int i = 0; i < C::KS * C::NQ; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // VALU
    }
    if (__builtin_amdgcn_ballot_w64(up_any)) {
#pragma unroll
      for (int qi = 0; qi < C::NQ; ++qi) {
        const float alpha = __builtin_amdgcn_exp2f(m[qi] - mnew[qi]);
        l[qi] *= alpha;
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) o[qi][mb] *= alpha;
        m[qi] = mnew[qi];
      }
    }
    mma_tile(kf[1], snext[1]);
    bf16x8 pf[C::NQ];
#pragma unroll
    for (int qi = 0; qi < C::NQ; ++qi) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          pf[qi][4 * t + e] = (bf16)__builtin_amdgcn_exp2f(fmaf(scur[t][qi][e], a.sl2, -m[qi]));
      // The row sum adds the rounded weights the products use.
#pragma unroll
      for (int e = 0; e < 8; e += 2)
        l[qi] = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){pf[qi][e], pf[qi][e + 1]}, ones, l[qi],
                                                false);
    }
#pragma unroll
    for (int i = 0; i < C::KS * C::NQ; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // VALU
    }

    // O^T += V^T P^T; each V^T fragment feeds NQ products.
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int qi = 0; qi < C::NQ; ++qi) o[qi][mb] = mma_k32(vf[mb], pf[qi], o[qi][mb]);

#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int qi = 0; qi < C::NQ; ++qi) scur[t][qi] = snext[t][qi];
  }

  // O = O^T / l, row (b, m), columns h*DH + channel.
#pragma unroll
  for (int qi = 0; qi < C::NQ; ++qi) {
    const float lt = sum_g(l[qi]);
    // p = exp2(z * sl2 - lse) recovers a row's softmax weights from its scores.
    if (a.lse && g == 0 && rw + 16 * qi + c < Tn)
      a.lse[((size_t)b * Tn + rw + 16 * qi + c) * H + h] = m[qi] + __log2f(lt);
    const int fr = rw + 16 * qi + c;
    if (fr < Tn) {
      const float inv = 1.0f / lt;
      bf16 *dst = a.O + ((size_t)b * Tn + fr) * H * C::DH + h * C::DH + 4 * g;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) store4f(dst + 16 * mb, o[qi][mb] * inv);
    }
  }
}

}  // namespace

bool heads_attention_supported(int dtype, int H, int d_h, int dR) {
  return (dtype == 0 || dtype == 1) && ((d_h == 64 && dR == 32) || (d_h == 128 && dR == 64)) &&
         H >= 1 && H <= 64;
}

namespace {
template <class C>
hipError_t heads_t(int B, int T, int H, int s, float sl2, const void *q, const void *QR,
                   const void *KV, const void *KR, void *O, float *lse, hipStream_t stream,
                   hipEvent_t ev0, hipEvent_t ev1) {
  const int tiles = (T + C::ROWS - 1) / C::ROWS;
  const size_t lds = (size_t)C::NST * C::STAGE_B + 1024;
  allow_lds<heads_attn_kernel<C>>();
  HeadsArgs args{(const bf16 *)q, (const bf16 *)QR, (const bf16 *)KV, (const bf16 *)KR,
                 (bf16 *)O, lse, B, T, H, s, tiles, C::NST, sl2};
  return launch_timed((const void *)heads_attn_kernel<C>, dim3(tiles * B * H), dim3(64 * C::NW),
                      lds, stream, &args, ev0, ev1);
}
}  // namespace

hipError_t launch_heads_attention(int B, int T, int H, int d_h, int s, float scale, const void *q,
                                  const void *QR, const void *KV, const void *KR, void *O,
                                  float *lse, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  // Masked scores are -inf before the fused scale-and-subtract, which needs
  // a positive scale (0 * -inf is NaN): a scale that underflows to zero is
  // raised to the smallest normal value.
  float sl2 = scale * kLog2e;
  if (!(sl2 >= FLT_MIN)) sl2 = FLT_MIN;
  if (d_h == 128)
    return heads_t<HdCfg128>(B, T, H, s, sl2, q, QR, KV, KR, O, lse, stream, ev0, ev1);
  return heads_t<HdCfg64>(B, T, H, s, sl2, q, QR, KV, KR, O, lse, stream, ev0, ev1);
}

}  // namespace mtla
