// Incremental decoding over the compressed cache on gfx950: the hyper-network
// merge of the new frame into its slot, and the split-K absorbed attention
// over slots 0..floor(t/s) with the temporary (partially merged) newest slot.
//
// [Notes] = "Multi-head Temporal Latent Attention" paper notes (zhaoyang97
// Paper-Notes), method section, key designs: hyper-network temporal merging,
// stride-aware causal mask (why inference attends a temporary slot), and
// decoupled RoPE with temporal compression (the Y formula).
// [Fig2] = "Multi-head Temporal Latent Attention" (sciencestack.ai), Fig. 2 (a).
//
// Attention kernel, one workgroup (4 waves) per (sequence b, split of `chunk`
// slots).  All heads of a sequence read the same compressed rows (one latent
// cache shared by every head), so each row is fetched from HBM once:
//  * The split's rows stream into a ring of LDS stages by direct
//    global->LDS loads (global_load_lds_dwordx4, no register staging), up to
//    `nst` stages in flight.  A stage is TPS 16-row tiles, TPS = 4 / NHB for
//    NHB blocks of 16 heads.
//  * Scores: wave w takes one (tile, head block) pair of the stage and
//    computes S^T (16 keys x 16 heads) = K . Q^T on the K=32 MFMA, K (latent
//    ++ RoPE key, r + d_hR wide) from LDS as the A operand, Q^T from
//    registers.
//  * Softmax: the column maxima of all pairs meet in LDS, so every wave
//    derives the same per-head reference max; it moves lazily (only when a
//    score exceeds it by more than 2^8), which skips the rescale of O on
//    almost every stage.  P = 2^(z - m) goes to LDS in bf16 (fp32 storage:
//    fp32).
//  * Values: wave w accumulates O^T for its quarter of the r latent channels,
//    all heads, all tiles of the stage: O^T += C^T . P^T on the K=16 MFMA,
//    C^T read from the row-major tile with ds_read_tr16_b64 (its A layout)
//    and P^T from LDS (the score layout is the B layout).  O needs no
//    cross-wave reduction at the end.
//  * The split that owns the newest slot j = floor(t/s) first merges the new
//    frame: u = Sigmoid((g + b_hc) * Linear(pe_j)) * c, slot j = u (t mod s
//    == 0) or slot j + u, RoPE key j = K^R_t, written to the cache and into
//    its LDS copy before that row is attended.
//  * Splits store (max, sum, O) partials with XCD-coherent accesses; the
//    last split of a sequence to finish (atomic counter) merges them by
//    log-sum-exp in split order (deterministic results).  A sequence that
//    fits one split is normalised and written directly.

#include <math.h>

#include "common.h"
#include "kernels.h"

namespace mtla {

namespace {

constexpr float kNegInf = -INFINITY;

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

template <typename T, int R, int DR, int NHB> struct DecCfg {
  static constexpr int RK = R + DR, ES = (int)sizeof(T), RB = RK * ES, NSEG = RB / 64;
  static constexpr int TPS = 4 / NHB;                    // 16-row tiles per stage
  static constexpr int SROWS = 16 * TPS;
  static constexpr int TILE_B = 16 * RB, STAGE_B = TPS * TILE_B;
  static constexpr int NBLK = TPS * NSEG, LPW = (NBLK + 3) / 4;
  static constexpr int KS = RK / 32;                     // k-steps of the scores
  static constexpr int MQ = R / 64;                      // 16-channel blocks per wave
  static constexpr int NU = (R + 255) / 256;
  static constexpr int HW = 16 * NHB;                    // heads covered (padded)
  // LDS after the ring: dummy block, per-pair column maxima, P tiles
  static constexpr int SMAX_B = TPS * HW * 4;
  static constexpr int P_B = TPS * NHB * 64 * 4 * ES;   // then one int (last-split flag)
  static_assert(RB % 64 == 0, "row bytes must be a multiple of 64");
  static_assert(NHB * TPS == 4, "one (tile, head block) pair per wave");
};

struct DecodeArgs {
  const int32_t *pos;
  char *cache;
  int64_t bstride_bytes;
  const void *qt;      // [B, H, R]
  const void *QR;      // [B, H, DR]
  const void *KR;      // [B, DR]
  const float *cg;     // [B, 2R]: latent c then gate pre-activation g
  const void *b_hc;    // [R]
  const float *gate_pos;
  float *part_o;       // [B, splits, H, R]
  float *part_ml;      // [B, splits, H, 2]
  int *counters;       // [B], zero on entry (zero again on exit)
  void *o;             // [B, H, R]
  int H, s, chunk, splits, nst;
  float sl2;
};

template <typename T, int R, int DR, int NHB>
__global__ __launch_bounds__(256) void decode_attn_kernel(DecodeArgs a) {
  using C = DecCfg<T, R, DR, NHB>;
  typedef typename Frag4<T>::type P4;
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int b = blockIdx.y, split = blockIdx.x;
  const int t = a.pos[b], s = a.s, jn = t / s, n = jn + 1;
  const int start = split * a.chunk;
  if (start >= n) return;
  const int end = min(n, start + a.chunk);
  const int ns = (n + a.chunk - 1) / a.chunk;
  const bool owner = end == n;
  const int nstage = (end - start + C::SROWS - 1) / C::SROWS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int st_tile = wave % C::TPS, st_hb = wave / C::TPS;   // score pair of this wave
  const int H = a.H, shead = st_hb * 16 + c;
  char *seq = a.cache + (size_t)b * a.bstride_bytes;
  char *dummy = smem + a.nst * C::STAGE_B;
  float *smax = (float *)(dummy + 1024);                       // [TPS][HW]
  char *pbuf = (char *)smax + C::SMAX_B;                       // [TPS][NHB][64][4]

  // Everything read from global memory besides the stream is fetched first,
  // so that later waits for it never wait for the cache loads behind it.
  typename Frag<T>::type q[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    const int k = 32 * ks + 8 * g;
    if (shead < H) {
      if (k < R) load8(q[ks], (const T *)a.qt + ((size_t)b * H + shead) * R + k);
      else load8(q[ks], (const T *)a.QR + ((size_t)b * H + shead) * DR + (k - R));
    } else {
      q[ks] = zero_frag<T>();
    }
  }
  // b_hc and K^R stay in the storage type until used, so that no wait for
  // these loads (and for every load issued before them) precedes the stream.
  float mc[C::NU], mg[C::NU], mp[C::NU];
  T mb[C::NU], mkr = from_f32<T>(0.0f);
#pragma unroll
  for (int i = 0; i < C::NU; ++i) {
    mc[i] = mg[i] = mp[i] = 0.0f;
    mb[i] = from_f32<T>(0.0f);
  }
  if (owner) {
#pragma unroll
    for (int i = 0; i < C::NU; ++i) {
      const int ch = tid + 256 * i;
      if (ch < R) {
        mc[i] = a.cg[(size_t)b * 2 * R + ch];
        mg[i] = a.cg[(size_t)b * 2 * R + R + ch];
        mb[i] = ((const T *)a.b_hc)[ch];
        mp[i] = a.gate_pos[(size_t)jn * R + ch];
      }
    }
    if (tid < DR) mkr = ((const T *)a.KR)[(size_t)b * DR + tid];
  }
  asm volatile("" ::: "memory");

  auto issue = [&](int sidx) {
    char *sb = smem + (sidx % a.nst) * C::STAGE_B;
    const int row0 = start + sidx * C::SROWS;
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) {
      const int blk = wave + 4 * i;
      const bool real = (C::NBLK % 4 == 0) || blk < C::NBLK;
      const int tl = real ? blk / C::NSEG : 0, qq = real ? blk % C::NSEG : 0;
      const int slot = min(row0 + tl * 16 + (lane >> 2), end - 1);
      dma_block(seq + (size_t)slot * C::RB, qq, real ? sb + tl * C::TILE_B + qq * 1024 : dummy);
    }
  };
  const int pro = min(a.nst, nstage);
  for (int k = 0; k < pro; ++k) issue(k);
  int lastst = pro - 1;   // newest stage issued so far

  // o[hb][qb]: O^T block of channels 16 (wave * MQ + qb) + 4g + e, head
  // hb * 16 + c.  m[hb]: reference max of head hb * 16 + c (same in every
  // wave).  lp: partial sum of P over this wave's score pairs.
  f32x4 o[NHB][C::MQ];
  float m[NHB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    m[hb] = kNegInf;
#pragma unroll
    for (int qb = 0; qb < C::MQ; ++qb) o[hb][qb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  float lp = 0.0f;

  for (int k = 0; k < nstage; ++k) {
    // Stage k has landed once at most lastst - k stages issued after it are
    // still in flight (this wave's loads complete in issue order).
    wait_stages<C::LPW>(lastst - k);
    bar();
    // Every wave is past stage k-1 here: its ring slot can be refilled.
    if (k >= 1 && k - 1 + a.nst < nstage) {
      issue(k - 1 + a.nst);
      lastst = k - 1 + a.nst;
    }
    char *sb = smem + (k % a.nst) * C::STAGE_B;
    const int row0 = start + k * C::SROWS;
    if (k == nstage - 1) {
      // Rows past the split read as zeros (their weight is exactly 0, but
      // the P.V product must not meet stale non-finite LDS contents).
      const int nz = row0 + C::SROWS - end;
      for (int idx = tid; idx < nz * (C::RB / 16); idx += 256) {
        const int r = end - row0 + idx / (C::RB / 16), ch = idx % (C::RB / 16);
        *(u32x4 *)(sb + (r >> 4) * C::TILE_B + tile_off(r & 15, ch * 16)) = (u32x4){0u, 0u, 0u, 0u};
      }
      if (owner) {
        // Merge the new frame into the newest slot ([Notes] hyper-network
        // temporal merging; [Fig2] (a)), in the cache and in its LDS copy.
        const int rr = jn - row0;
        char *trow = sb + (rr >> 4) * C::TILE_B;
        T *grow = (T *)(seq + (size_t)jn * C::RB);
        const bool open = (t % s) == 0;
#pragma unroll
        for (int i = 0; i < C::NU; ++i) {
          const int ch = tid + 256 * i;
          if (ch < R) {
            T *lpnt = (T *)(trow + tile_off(rr & 15, ch * C::ES));
            const float u = sigmoidf((mg[i] + to_f32(mb[i])) * mp[i]) * mc[i];
            const T v = from_f32<T>(open ? u : to_f32(*lpnt) + u);
            *lpnt = v;
            grow[ch] = v;
          }
        }
        if (tid < DR) {
          const T v = mkr;
          *(T *)(trow + tile_off(rr & 15, (R + tid) * C::ES)) = v;
          grow[R + tid] = v;
        }
      }
      wait_lgkm0();
      bar();
    }

    // Scores of this wave's (tile, head block) pair.
    const char *stile = sb + st_tile * C::TILE_B;
    const int kb = row0 + st_tile * 16;
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks + 1 < C::KS; ks += 2) {
      s0 = mma_k32(s_frag<T>(stile, c, ks, g), q[ks], s0);
      s1 = mma_k32(s_frag<T>(stile, c, ks + 1, g), q[ks + 1], s1);
    }
    if constexpr (C::KS % 2) s0 = mma_k32(s_frag<T>(stile, c, C::KS - 1, g), q[C::KS - 1], s0);
    float z[4], mx = kNegInf;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      z[e] = (kb + 4 * g + e < end) ? (s0[e] + s1[e]) * a.sl2 : kNegInf;
      mx = fmaxf(mx, z[e]);
    }
    mx = max_g(mx);   // -inf only for a tile wholly past the split
    if (g == 0) smax[st_tile * C::HW + shead] = mx;
    wait_lgkm0();
    bar();

    // Reference max per head, identical in every wave; rescale when it moves.
    float mnew[NHB];
    bool up_any = false;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      float sm = kNegInf;
#pragma unroll
      for (int tl = 0; tl < C::TPS; ++tl) sm = fmaxf(sm, smax[tl * C::HW + hb * 16 + c]);
      const bool up = sm > m[hb] + 8.0f;
      mnew[hb] = up ? sm : m[hb];
      up_any |= up;
    }
    if (__builtin_amdgcn_ballot_w64(up_any)) {
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        const float alpha = __builtin_amdgcn_exp2f(m[hb] - mnew[hb]);
#pragma unroll
        for (int qb = 0; qb < C::MQ; ++qb) o[hb][qb] *= alpha;
        if (hb == st_hb) lp *= alpha;
        m[hb] = mnew[hb];
      }
    }
    float mref = m[0];
#pragma unroll
    for (int hb = 1; hb < NHB; ++hb)
      if (hb == st_hb) mref = m[hb];
    P4 pf;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p = __builtin_amdgcn_exp2f(z[e] - mref);
      lp += p;
      pf[e] = from_f32<T>(p);
    }
    *(P4 *)(pbuf + ((st_tile * NHB + st_hb) * 64 + lane) * 4 * C::ES) = pf;
    wait_lgkm0();
    bar();

    // O^T += C^T P^T for this wave's channel quarter, every pair of the stage.
    if constexpr (sizeof(T) == 2 && C::TPS % 2 == 0) {
      // bf16: two 16-slot tiles form one 32-deep contraction (the full-rate
      // 16x16x32 product).  k index 8g+e stands for slot 4g+e of the first
      // tile (e < 4) and of the second (e >= 4), in both operands: C^T from
      // one transposing read of each tile, P^T from the two tiles' P blocks.
#pragma unroll
      for (int tl = 0; tl < C::TPS; tl += 2) {
        // A pair wholly past the split contributes nothing (a partly past
        // second tile has P = 0 and zeroed rows).
        if (row0 + tl * 16 >= end) continue;
        const char *t0 = sb + tl * C::TILE_B;
        bf16x8 pp[NHB];
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
          const bf16x4 p0 = *(const bf16x4 *)(pbuf + ((tl * NHB + hb) * 64 + lane) * 8);
          const bf16x4 p1 = *(const bf16x4 *)(pbuf + (((tl + 1) * NHB + hb) * 64 + lane) * 8);
          pp[hb] = __builtin_shufflevector(p0, p1, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int q0 = 0; q0 < C::MQ; q0 += 4) {
          uint32_t ad[8];
          bf16x4 v[8];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int ch0 = 16 * (wave * C::MQ + q0 + j);
            ad[2 * j] = lds_addr(t0 + tile_off(4 * g + (c >> 2), (ch0 + 4 * (c & 3)) * 2));
            ad[2 * j + 1] = ad[2 * j] + C::TILE_B;
          }
          ds_read_tr8(v, ad);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bf16x8 vv = __builtin_shufflevector(v[2 * j], v[2 * j + 1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
            for (int hb = 0; hb < NHB; ++hb) o[hb][q0 + j] = mma_k32(vv, pp[hb], o[hb][q0 + j]);
          }
        }
      }
    } else {
#pragma unroll
    for (int tl = 0; tl < C::TPS; ++tl) {
      if (row0 + tl * 16 >= end) continue;
      const char *tile = sb + tl * C::TILE_B;
      P4 pp[NHB];
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb)
        pp[hb] = *(const P4 *)(pbuf + ((tl * NHB + hb) * 64 + lane) * 4 * C::ES);
#pragma unroll
      for (int q0 = 0; q0 < C::MQ; q0 += 8) {
        constexpr int QN = C::MQ < 8 ? C::MQ : 8;
        typename Frag4<T>::type vv[8];
        if constexpr (sizeof(T) == 2) {
          uint32_t ad[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int ch0 = 16 * (wave * C::MQ + q0 + (j < QN ? j : 0));
            ad[j] = lds_addr(tile + tile_off(4 * g + (c >> 2), (ch0 + 4 * (c & 3)) * 2));
          }
          ds_read_tr8(vv, ad);
        } else {
#pragma unroll
          for (int j = 0; j < QN; ++j) vv[j] = v_frag_f32(tile, 16 * (wave * C::MQ + q0 + j), g, c);
        }
#pragma unroll
        for (int j = 0; j < QN; ++j)
#pragma unroll
          for (int hb = 0; hb < NHB; ++hb) o[hb][q0 + j] = mma_k16(vv[j], pp[hb], o[hb][q0 + j]);
      }
    }
    }
  }

  // Row sums: lane partials -> per head, over the waves of each head block.
  const float lt = sum_g(lp);
  wait_lgkm0();
  bar();
  if (g == 0) smax[st_tile * C::HW + shead] = lt;
  wait_lgkm0();
  bar();
  const size_t pbase = ((size_t)b * a.splits + split) * H;
  const __amdgpu_buffer_rsrc_t ro =
      make_rsrc(a.part_o, (uint32_t)((size_t)gridDim.y * a.splits * H * R * 4));
  const __amdgpu_buffer_rsrc_t rml =
      make_rsrc(a.part_ml, (uint32_t)((size_t)gridDim.y * a.splits * H * 8));
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const int head = hb * 16 + c;
    if (head >= H) continue;
    float L = 0.0f;
#pragma unroll
    for (int tl = 0; tl < C::TPS; ++tl) L += smax[tl * C::HW + head];
#pragma unroll
    for (int qb = 0; qb < C::MQ; ++qb) {
      const int ch = 16 * (wave * C::MQ + qb) + 4 * g;
      if (ns == 1) {
        T *dst = (T *)a.o + ((size_t)b * H + head) * R + ch;
        const float inv = 1.0f / L;
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[e] = from_f32<T>(o[hb][qb][e] * inv);
      } else {
        st_coh4(ro, (uint32_t)(((pbase + head) * R + ch) * 4), o[hb][qb]);
      }
    }
    if (ns > 1 && wave == 0 && g == 0) {
      st_coh1(rml, (uint32_t)((pbase + head) * 8), m[hb]);
      st_coh1(rml, (uint32_t)((pbase + head) * 8 + 4), L);
    }
  }
  if (ns == 1) return;

  // The last split of this sequence to finish merges all of them (log-sum-
  // exp in split order: deterministic).  A thread takes two 4-channel chunks
  // at a time and loads up to eight splits' partials of both in one batch,
  // so a merge of up to eight splits waits for one round trip.
  int *last = (int *)(pbuf + C::P_B);
  __syncthreads();   // this workgroup's partial stores have completed
  if (tid == 0) *last = ctr_add(&a.counters[b], 1) == ns - 1;
  __syncthreads();
  if (!*last) return;
  constexpr int QC = R / 4;   // 4-channel chunks per head
  constexpr int UB = 2, SB = 8;
  const int nch = H * QC;
  const size_t base = (size_t)b * a.splits * H;
  for (int c0 = tid; c0 < nch; c0 += UB * 256) {
    float M[UB], L[UB];
    f32x4 acc[UB];
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      M[u] = kNegInf;
      L[u] = 0.0f;
      acc[u] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    for (int k0 = 0; k0 < ns; k0 += SB) {
      float pm[UB][SB], pl[UB][SB];
      f32x4 po[UB][SB];
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int ci = min(c0 + 256 * u, nch - 1), h = ci / QC, ch = (ci % QC) * 4;
#pragma unroll
        for (int j = 0; j < SB; ++j) {
          pm[u][j] = kNegInf;
          pl[u][j] = 0.0f;
          po[u][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
          if (k0 + j < ns) {
            const size_t i = base + (size_t)(k0 + j) * H + h;
            pm[u][j] = ld_coh1(rml, (uint32_t)(i * 8));
            pl[u][j] = ld_coh1(rml, (uint32_t)(i * 8 + 4));
            po[u][j] = ld_coh4(ro, (uint32_t)((i * R + ch) * 4));
          }
        }
      }
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        float Mn = M[u];
#pragma unroll
        for (int j = 0; j < SB; ++j) Mn = fmaxf(Mn, pm[u][j]);
        const float sc = __builtin_amdgcn_exp2f(M[u] - Mn);
        L[u] *= sc;
        acc[u] *= sc;
#pragma unroll
        for (int j = 0; j < SB; ++j) {
          const float w = (k0 + j < ns) ? __builtin_amdgcn_exp2f(pm[u][j] - Mn) : 0.0f;
          L[u] += w * pl[u][j];
          acc[u] += w * po[u][j];
        }
        M[u] = Mn;
      }
    }
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int ci = c0 + 256 * u;
      if (ci >= nch) continue;
      const int h = ci / QC, ch = (ci % QC) * 4;
      T *dst = (T *)a.o + ((size_t)b * H + h) * R + ch;
      const float inv = 1.0f / L[u];
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e] = from_f32<T>(acc[u][e] * inv);
    }
  }
  if (tid == 0) __hip_atomic_store(&a.counters[b], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Stand-alone merge-append: one workgroup per sequence.
template <typename T>
__global__ __launch_bounds__(256) void merge_kernel(const int32_t *pos, int s, int R, int DR,
                                                    const float *cg, const T *b_hc,
                                                    const float *gate_pos, const T *KR,
                                                    char *cache, int64_t bstride_bytes) {
  const int b = blockIdx.x, t = pos[b], j = t / s;
  const bool open = (t % s) == 0;
  T *row = (T *)(cache + (size_t)b * bstride_bytes) + (size_t)j * (R + DR);
  for (int ch = threadIdx.x; ch < R; ch += blockDim.x) {
    const float u = sigmoidf((cg[(size_t)b * 2 * R + R + ch] + to_f32(b_hc[ch])) *
                             gate_pos[(size_t)j * R + ch]) *
                    cg[(size_t)b * 2 * R + ch];
    row[ch] = from_f32<T>(open ? u : to_f32(row[ch]) + u);
  }
  for (int ch = threadIdx.x; ch < DR; ch += blockDim.x) row[R + ch] = KR[(size_t)b * DR + ch];
}


template <typename T, int R, int DR, int NHB>
hipError_t decode_attn_t(const DecodePlan &p, int B, DecodeArgs args, hipStream_t stream,
                         hipEvent_t ev0, hipEvent_t ev1) {
  auto kern = decode_attn_kernel<T, R, DR, NHB>;
  allow_lds<decode_attn_kernel<T, R, DR, NHB>>();
  return launch_timed((const void *)kern, dim3(p.splits, B), dim3(256), p.lds, stream, &args,
                      ev0, ev1);
}

template <typename T, int R, int DR>
hipError_t decode_attn_h(const DecodePlan &p, int B, const DecodeArgs &args, hipStream_t stream,
                         hipEvent_t ev0, hipEvent_t ev1) {
  if (p.nhb == 1) return decode_attn_t<T, R, DR, 1>(p, B, args, stream, ev0, ev1);
  if (p.nhb == 2) return decode_attn_t<T, R, DR, 2>(p, B, args, stream, ev0, ev1);
  return decode_attn_t<T, R, DR, 4>(p, B, args, stream, ev0, ev1);
}

}  // namespace

#ifndef MTLA_DECODE_TARGET_WGS
#define MTLA_DECODE_TARGET_WGS 256
#endif

bool decode_plan(int dtype, int H, int r, int dR, int s, int B, int max_pos, DecodePlan *plan) {
  if (!((r == 256 && dR == 32) || (r == 512 && dR == 64))) return false;
  if (H < 1 || H > 64 || s < 1 || B < 1 || max_pos < 0) return false;
  const int esz = dtype == 1 ? 2 : 4;
  DecodePlan p;
  p.nhb = H <= 16 ? 1 : (H <= 32 ? 2 : 4);
  const int tps = 4 / p.nhb, srows = 16 * tps;
  const size_t stage = (size_t)srows * (r + dR) * esz;
  const size_t extra =
      1024 + (size_t)tps * 16 * p.nhb * 4 + (size_t)tps * p.nhb * 64 * 4 * esz + 16;
  const int64_t nmax = max_pos / s + 1;
  const int64_t total = (int64_t)B * nmax;
  int64_t chunk = (total + MTLA_DECODE_TARGET_WGS - 1) / MTLA_DECODE_TARGET_WGS;
  chunk = ((chunk + srows - 1) / srows) * srows;
  const int64_t cap = ((nmax + srows - 1) / srows) * srows;
  if (chunk > cap) chunk = cap;
  p.block = srows;
  p.chunk = (int)chunk;
  p.splits = (int)((nmax + chunk - 1) / chunk);
  // Ring: about 4 stages of 36 KB, or more of smaller stages (at most 8).
  int nst = (int)(144 * 1024 / stage);
  if (nst > 8) nst = 8;
  if (nst < 2) {
    // A one-slot ring cannot refill a slot that the same stage still reads:
    // give each split a single stage instead (more splits, same bytes).
    nst = 1;
    chunk = srows;
    p.chunk = (int)chunk;
    p.splits = (int)((nmax + chunk - 1) / chunk);
  }
  if (nst > chunk / srows) nst = (int)(chunk / srows);
  if (nst < 1) nst = 1;
  p.nst = nst;
  p.lds = nst * stage + extra;
  if (p.lds > 159 * 1024) return false;
  *plan = p;
  return true;
}

hipError_t launch_decode_attention(int dtype, const DecodePlan &plan, int B, int H, int r, int dR,
                                   int s, float scale, const int32_t *pos, void *cache,
                                   int64_t batch_stride, const void *qt, const void *QR,
                                   const void *KR_t, const float *cg, const void *b_hc,
                                   const float *gate_pos, float *part_o, float *part_ml,
                                   int *counters, void *o, hipStream_t stream, hipEvent_t ev0,
                                   hipEvent_t ev1) {
  const int esz = dtype == 1 ? 2 : 4;
  DecodeArgs args{pos,      (char *)cache, batch_stride * esz, qt,         QR,
                  KR_t,     cg,            b_hc,               gate_pos,   part_o,
                  part_ml,  counters,      o,                  H,          s,
                  plan.chunk, plan.splits, plan.nst,           scale * kLog2e};
  if (dtype == 1) {
    if (r == 256) return decode_attn_h<bf16, 256, 32>(plan, B, args, stream, ev0, ev1);
    return decode_attn_h<bf16, 512, 64>(plan, B, args, stream, ev0, ev1);
  }
  if (r == 256) return decode_attn_h<float, 256, 32>(plan, B, args, stream, ev0, ev1);
  return decode_attn_h<float, 512, 64>(plan, B, args, stream, ev0, ev1);
}

hipError_t launch_merge(int dtype, int B, int r, int dR, int s, const int32_t *pos, const float *cg,
                        const void *b_hc, const float *gate_pos, const void *KR_t, void *cache,
                        int64_t batch_stride, hipStream_t stream) {
  const int esz = dtype == 1 ? 2 : 4;
  if (dtype == 1)
    hipLaunchKernelGGL(merge_kernel<bf16>, dim3(B), dim3(256), 0, stream, pos, s, r, dR, cg,
                       (const bf16 *)b_hc, gate_pos, (const bf16 *)KR_t, (char *)cache,
                       batch_stride * esz);
  else
    hipLaunchKernelGGL(merge_kernel<float>, dim3(B), dim3(256), 0, stream, pos, s, r, dR, cg,
                       (const float *)b_hc, gate_pos, (const float *)KR_t, (char *)cache,
                       batch_stride * esz);
  return hipGetLastError();
}

}  // namespace mtla
