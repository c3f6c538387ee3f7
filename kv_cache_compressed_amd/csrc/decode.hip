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
// Attention kernel: one workgroup (4 waves) per (sequence b, split of its
// slots).  All heads of a sequence read the same compressed rows (one latent
// cache shared by every head), so each row is fetched from HBM once:
//  * Work list.  Every workgroup derives the same balanced assignment from
//    the positions: a sequence of m_b stages (SROWS slots each) gets
//    ceil(m_b / c) splits of at most c stages, c the smallest value (from
//    ceil(sum m_b / G) up) for which all splits fit the G workgroups of the
//    grid, so ragged batches stream equal slot counts per workgroup.  Above
//    256 sequences the splits are uniform, sized from max_pos.
//  * Streaming.  The split's rows stream HBM -> LDS by direct loads
//    (global_load_lds_dwordx4, non-temporal) into a ring of up to `nst`
//    stages.  Each 1 KB load covers 8 rows x one whole 128-byte line (rows of
//    576 bytes are paired into 1152-byte super-rows), with a per-row XOR
//    permutation of the 16-byte chunks that keeps the MFMA operand reads
//    below conflict free.  A stage is TPS 16-row tiles, TPS = 4 / NHB for NHB
//    blocks of 16 heads.
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
//    all heads, all tiles of the stage: O^T += C^T . P^T, C^T read from the
//    tile with ds_read_b64_tr_b16 (its A layout) and P^T from LDS (the score
//    layout is the B layout).  O needs no cross-wave reduction at the end.
//  * The split that owns the newest slot j = floor(t/s) first merges the new
//    frame: u = Sigmoid((g + b_hc) * Linear(pe_j)) * c, slot j = u (t mod s
//    == 0) or slot j + u, RoPE key j = K^R_t, written to the cache and into
//    its LDS copy before that row is attended.
//  * Splits store (max, sum, O) partials with XCD-coherent accesses; the
//    last split of a sequence to finish (atomic counter) merges them by
//    log-sum-exp in split order (deterministic results).  A sequence that
//    fits one split is normalised and written directly.
//  * Positions.  A sequence whose pos[b] lies outside [0, max_pos] (the
//    caller's bound, which the host checked against the cache and the gate
//    table) is dropped: nothing is merged or read, its output row is zero,
//    and the status word counts it.

#include <math.h>

#include "common.h"
#include "kernels.h"

namespace mtla {

namespace {

constexpr float kNegInf = -INFINITY;

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// LDS layout of one 16-row tile of streamed cache rows (RB bytes each): RB/64
// blocks of 1 KB, each filled by one direct load of 8 rows x one 128-byte
// line.  Rows whose length is a multiple of 128 bytes: block 2q + h holds
// line q of rows 8h..8h+7 (row i of the block at 128 i).  576-byte rows: rows
// 2k and 2k+1 form a 1152-byte super-row k, and block q holds line q of the
// 8 super-rows.  The 16-byte chunks of the 128-byte run of block row i are
// permuted by XOR with i, which keeps both the score operand reads (16 rows x
// 16 bytes per k-step) and the transposing reads (4 rows x 32 bytes per 16
// lanes) free of bank conflicts; the choice was measured with the LDS
// bank-conflict counter against other permutations, several of which
// conflict two-way.
template <int RB> struct DecLayout {
  static constexpr bool PAIRED = (RB % 128) != 0;
  static_assert(!PAIRED || RB == 576, "rows must be 576 bytes or a multiple of 128");
  // Byte offset within the tile of byte b of row R (0 <= R < 16).
  __device__ static int off(int R, int b) {
    if constexpr (!PAIRED) {
      return ((b >> 7) << 11) + ((R >> 3) << 10) + ((R & 7) << 7) +
             ((((b >> 4) & 7) ^ (R & 7)) << 4) + (b & 15);
    } else {
      const int sb = (R & 1) * 576 + b, k = R >> 1;
      return ((sb >> 7) << 10) + (k << 7) + ((((sb >> 4) & 7) ^ k) << 4) + (sb & 15);
    }
  }
  // The row and byte that lane `lane` copies for block `blk` of a tile (its
  // 16 bytes land at byte 16 lane of the block).
  __device__ static void src(int blk, int lane, int &R, int &b) {
    const int i = lane >> 3, v = lane & 7;
    if constexpr (!PAIRED) {
      R = ((blk & 1) << 3) + i;
      b = ((blk >> 1) << 7) + ((v ^ i) << 4);
    } else {
      const int sb = (blk << 7) + ((v ^ i) << 4);
      const int hi = sb >= 576;
      R = 2 * i + hi;
      b = sb - (hi ? 576 : 0);
    }
  }
};

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

// Score operand (row `row`, k-step ks, lane group g) and fp32 value operand
// from a tile in the decode layout; the same lane mapping as s_frag and
// v_frag_f32.
template <typename T, class Lay>
__device__ __forceinline__ typename Frag<T>::type dec_frag(const char *tile, int row, int ks, int g) {
  if constexpr (sizeof(T) == 2) {
    return *(const bf16x8 *)(tile + Lay::off(row, ks * 64 + g * 16));
  } else {
    const f32x4 x = *(const f32x4 *)(tile + Lay::off(row, ks * 128 + g * 32));
    const f32x4 y = *(const f32x4 *)(tile + Lay::off(row, ks * 128 + g * 32 + 16));
    return (f32x8){x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  }
}
template <class Lay>
__device__ __forceinline__ f32x4 dec_vfrag_f32(const char *tile, int ch0, int g, int j) {
  f32x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = *(const float *)(tile + Lay::off(4 * g + e, (ch0 + j) * 4));
  return v;
}

// Cache policy of the stream's loads: non-temporal (each row is read once).
constexpr int kStreamPolicy = 2;

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
  float *part_o;       // [nparts, H, R]
  float *part_ml;      // [nparts, H, 2]
  int *counters;       // [B], zero on entry (zero again on exit)
  int *status;         // count of dropped sequences (cleared before the kernel)
  void *o;             // [B, H, R]
  int B, H, s, chunk, splits, nst, nparts, max_pos, flat;
  float sl2;
};

// Wave-wide integer scans and reductions on DPP row shifts and lane reads
// (VALU only: no LDS round trips in the kernel's prologue).
__device__ __forceinline__ int dpp_shr(int v, int n) {
  switch (n) {
    case 1: return __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);
    case 2: return __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);
    case 4: return __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);
    default: return __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);
  }
}
// Inclusive scan over the 64 lanes; *total receives the sum of all lanes.
__device__ __forceinline__ int wave_incl_scan(int v, int *total) {
  v += dpp_shr(v, 1);
  v += dpp_shr(v, 2);
  v += dpp_shr(v, 4);
  v += dpp_shr(v, 8);   // inclusive within each row of 16 lanes
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47), r3 = __builtin_amdgcn_readlane(v, 63);
  const int row = (threadIdx.x & 63) >> 4;
  v += (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
  *total = r0 + r1 + r2 + r3;
  return v;
}
__device__ __forceinline__ int wave_max_nonneg(int v) {
  v = max(v, dpp_shr(v, 1));
  v = max(v, dpp_shr(v, 2));
  v = max(v, dpp_shr(v, 4));
  v = max(v, dpp_shr(v, 8));
  return max(max(__builtin_amdgcn_readlane(v, 15), __builtin_amdgcn_readlane(v, 31)),
             max(__builtin_amdgcn_readlane(v, 47), __builtin_amdgcn_readlane(v, 63)));
}

// Balanced work list (every wave of every workgroup computes the same one):
// sequence b has m_b = ceil(n_b / SROWS) stages (n_b slots; 0 when dropped)
// and takes max(1, ceil(m_b / c)) splits of at most c stages.  c is the
// smallest value from ceil(sum m_b / G) up (eight tries, then max m_b, which
// always fits because G >= B) for which the splits fit the G workgroups.
// Lane l owns sequences [l P, l P + P).  Returns the sequence of workgroup w
// (-1 when w has no work) with its split index, split count, first partial
// index and c.
template <int SROWS>
__device__ void flat_assign(const DecodeArgs &a, int w, int &b, int &split, int &ns, int &pbase,
                            int &cst) {
  constexpr int PMAX = 4;
  const int lane = threadIdx.x & 63;
  const int P = (a.B + 63) / 64;
  int m[PMAX];
  int msum = 0, mmax = 0;
#pragma unroll
  for (int i = 0; i < PMAX; ++i) {
    m[i] = 0;
    const int bb = lane * P + i;
    if (i < P && bb < a.B) {
      const int t = a.pos[bb];
      const bool valid = t >= 0 && t <= a.max_pos;
      m[i] = valid ? (t / a.s + SROWS) / SROWS : 0;   // ceil((floor(t/s) + 1) / SROWS)
    }
    msum += m[i];
    mmax = max(mmax, m[i]);
  }
  int M;
  (void)wave_incl_scan(msum, &M);
  mmax = wave_max_nonneg(mmax);
  const int G = (int)gridDim.x;
  auto splits_of = [&](int c) {
    int v = 0;
#pragma unroll
    for (int i = 0; i < PMAX; ++i)
      if (i < P && lane * P + i < a.B) v += m[i] > 0 ? (m[i] + c - 1) / c : 1;
    return v;
  };
  int c = max(1, (M + G - 1) / G);
  int tries = 0, mine, total;
  for (;;) {
    mine = splits_of(c);
    (void)wave_incl_scan(mine, &total);
    if (total <= G) break;
    if (++tries >= 8) {
      c = max(1, mmax);
      mine = splits_of(c);
      break;
    }
    ++c;
  }
  // Exclusive prefix of the split counts over the lanes, then the owner.
  int pre = wave_incl_scan(mine, &total) - mine;
  int fb = -1, fs = 0, fn = 0, fp = 0;
#pragma unroll
  for (int i = 0; i < PMAX; ++i) {
    const int bb = lane * P + i;
    if (i < P && bb < a.B) {
      const int k = m[i] > 0 ? (m[i] + c - 1) / c : 1;
      if (w >= pre && w < pre + k) {
        fb = bb;
        fs = w - pre;
        fn = k;
        fp = pre;
      }
      pre += k;
    }
  }
  // At most one lane found w: its values reach every lane.
  const unsigned long long hit = __ballot(fb >= 0);
  if (hit == 0ull) {
    b = -1;
    split = ns = pbase = 0;
  } else {
    const int src = __ffsll((long long)hit) - 1;
    b = __builtin_amdgcn_readlane(fb, src);
    split = __builtin_amdgcn_readlane(fs, src);
    ns = __builtin_amdgcn_readlane(fn, src);
    pbase = __builtin_amdgcn_readlane(fp, src);
  }
  cst = c;
}

// The slot range [start, end) of sequence b that this workgroup attends,
// from the balanced work list or the uniform splits, with the sequence's
// split count ns and first partial index pbase; t = pos[b].  Returns false
// when the workgroup has nothing to attend -- no split of its own, or a
// dropped frame (a position outside [0, max_pos]), whose output row the
// sequence's first split then writes as zeros and counts.
template <typename T, int R, int SROWS>
__device__ bool decode_work(const DecodeArgs &a, int &b, int &split, int &ns, int &pbase,
                            int &start, int &end, int &t) {
  if (a.flat) {
    int cst;
    flat_assign<SROWS>(a, (int)blockIdx.x, b, split, ns, pbase, cst);
    if (b < 0) return false;
    start = split * cst * SROWS;
    end = start + cst * SROWS;   // clipped to n below
  } else {
    b = blockIdx.y;
    split = blockIdx.x;
    pbase = b * a.splits;
    start = split * a.chunk;
    end = start + a.chunk;
    ns = -1;   // from n below
  }
  t = a.pos[b];
  if (t < 0 || t > a.max_pos) {
    if (split != 0) return false;
    if (threadIdx.x == 0) atomicAdd(a.status, 1);
    for (int i = threadIdx.x; i < a.H * R; i += blockDim.x)
      ((T *)a.o)[(size_t)b * a.H * R + i] = from_f32<T>(0.0f);
    return false;
  }
  const int n = t / a.s + 1;
  if (ns < 0) ns = (n + a.chunk - 1) / a.chunk;
  if (start >= n) return false;
  end = min(n, end);
  return true;
}

// The last split of a sequence to finish merges all of its partials (log-sum-
// exp in split order: deterministic).  A thread takes two 4-channel chunks at
// a time and loads up to eight splits' partials of both in one batch, so a
// merge of up to eight splits waits for one round trip.
template <typename T, int R>
__device__ void merge_partials(const DecodeArgs &a, int b, int ns, int pbase,
                               __amdgpu_buffer_rsrc_t ro, __amdgpu_buffer_rsrc_t rml) {
  constexpr int QC = R / 4;   // 4-channel chunks per head
  constexpr int UB = 2, SB = 8;
  const int H = a.H, nthr = blockDim.x;
  const int nch = H * QC;
  const size_t base = (size_t)pbase * H;
  for (int c0 = threadIdx.x; c0 < nch; c0 += UB * nthr) {
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
        const int ci = min(c0 + nthr * u, nch - 1), h = ci / QC, ch = (ci % QC) * 4;
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
      const int ci = c0 + nthr * u;
      if (ci >= nch) continue;
      const int h = ci / QC, ch = (ci % QC) * 4;
      T *dst = (T *)a.o + ((size_t)b * H + h) * R + ch;
      const float inv = 1.0f / L[u];
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e] = from_f32<T>(acc[u][e] * inv);
    }
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(&a.counters[b], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T, int R, int DR, int NHB>
__global__ __launch_bounds__(256) void decode_attn_kernel(DecodeArgs a) {
  using C = DecCfg<T, R, DR, NHB>;
  using Lay = DecLayout<C::RB>;
  typedef typename Frag4<T>::type P4;
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int b, split, ns, pbase, start, end, t;
  if (!decode_work<T, R, C::SROWS>(a, b, split, ns, pbase, start, end, t)) return;
  const int s = a.s, H = a.H;
  const int jn = t / s, n = jn + 1;
  const bool owner = end == n;
  const int nstage = (end - start + C::SROWS - 1) / C::SROWS;
  const int g = lane >> 4, c = lane & 15;
  const int st_tile = wave % C::TPS, st_hb = wave / C::TPS;   // score pair of this wave
  const int shead = st_hb * 16 + c;
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
      const int tl = real ? blk / C::NSEG : 0, bq = real ? blk % C::NSEG : 0;
      int rr, bb;
      Lay::src(bq, lane, rr, bb);
      const int slot = min(row0 + tl * 16 + rr, end - 1);
      __builtin_amdgcn_global_load_lds((const void *)(seq + (size_t)slot * C::RB + bb),
                                       (lds_void *)(real ? sb + tl * C::TILE_B + bq * 1024 : dummy),
                                       16, 0, kStreamPolicy);
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

  // Software pipeline over the stages: an iteration computes the scores of
  // stage k+1 beside the P.V of stage k (independent work), then the max
  // exchange and softmax of stage k+1 (after P.V(k), so a moved reference max
  // rescales O with stage k already in it).  Stage k's ring slot stays in use
  // until P.V(k), so the slot refilled after stage k+1 lands is stage k-1's.
  auto land = [&](int k) {
    // Stage k has landed once at most lastst - k stages issued after it are
    // still in flight (this wave's loads complete in issue order).
    wait_stages<C::LPW>(lastst - k);
    bar();
    // Every wave is past the P.V of stage k-2 here: its slot can be refilled.
    if (k >= 2 && k - 2 + a.nst < nstage) {
      issue(k - 2 + a.nst);
      lastst = k - 2 + a.nst;
    }
    char *sb = smem + (k % a.nst) * C::STAGE_B;
    const int row0 = start + k * C::SROWS;
    if (k == nstage - 1) {
      // Rows past the split read as zeros (their weight is exactly 0, but
      // the P.V product must not meet stale non-finite LDS contents).
      const int nz = row0 + C::SROWS - end;
      for (int idx = tid; idx < nz * (C::RB / 16); idx += 256) {
        const int r = end - row0 + idx / (C::RB / 16), ch = idx % (C::RB / 16);
        *(u32x4 *)(sb + (r >> 4) * C::TILE_B + Lay::off(r & 15, ch * 16)) = (u32x4){0u, 0u, 0u, 0u};
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
            T *lpnt = (T *)(trow + Lay::off(rr & 15, ch * C::ES));
            const float u = sigmoidf((mg[i] + to_f32(mb[i])) * mp[i]) * mc[i];
            const T v = from_f32<T>(open ? u : to_f32(*lpnt) + u);
            *lpnt = v;
            grow[ch] = v;
          }
        }
        if (tid < DR) {
          const T v = mkr;
          *(T *)(trow + Lay::off(rr & 15, (R + tid) * C::ES)) = v;
          grow[R + tid] = v;
        }
      }
      wait_lgkm0();
      bar();
    }

  };
  auto stage_scores = [&](int k, float (&z)[4]) {
    char *sb = smem + (k % a.nst) * C::STAGE_B;
    const int row0 = start + k * C::SROWS;
    // Scores of this wave's (tile, head block) pair.
    const char *stile = sb + st_tile * C::TILE_B;
    const int kb = row0 + st_tile * 16;
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks + 1 < C::KS; ks += 2) {
      s0 = mma_k32(dec_frag<T, Lay>(stile, c, ks, g), q[ks], s0);
      s1 = mma_k32(dec_frag<T, Lay>(stile, c, ks + 1, g), q[ks + 1], s1);
    }
    if constexpr (C::KS % 2) s0 = mma_k32(dec_frag<T, Lay>(stile, c, C::KS - 1, g), q[C::KS - 1], s0);
    float mx = kNegInf;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      z[e] = (kb + 4 * g + e < end) ? (s0[e] + s1[e]) * a.sl2 : kNegInf;
      mx = fmaxf(mx, z[e]);
    }
  };
  // Max exchange and softmax of a stage's scores: rescales O when a head's
  // reference max moves, writes P to LDS.
  auto stage_softmax = [&](float (&z)[4]) {
    float mx = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
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
  };
  auto stage_pv = [&](int k) {
    char *sb = smem + (k % a.nst) * C::STAGE_B;
    const int row0 = start + k * C::SROWS;
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
            ad[2 * j] = lds_addr(t0 + Lay::off(4 * g + (c >> 2), (ch0 + 4 * (c & 3)) * 2));
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
            ad[j] = lds_addr(tile + Lay::off(4 * g + (c >> 2), (ch0 + 4 * (c & 3)) * 2));
          }
          ds_read_tr8(vv, ad);
        } else {
#pragma unroll
          for (int j = 0; j < QN; ++j) vv[j] = dec_vfrag_f32<Lay>(tile, 16 * (wave * C::MQ + q0 + j), g, c);
        }
#pragma unroll
        for (int j = 0; j < QN; ++j)
#pragma unroll
          for (int hb = 0; hb < NHB; ++hb) o[hb][q0 + j] = mma_k16(vv[j], pp[hb], o[hb][q0 + j]);
      }
    }
    }
  };

  float zc[4];
  land(0);
  stage_scores(0, zc);
  stage_softmax(zc);
  for (int k = 0; k < nstage; ++k) {
    if (k + 1 < nstage) {
      land(k + 1);
      float zn[4];
      stage_scores(k + 1, zn);
      stage_pv(k);
      stage_softmax(zn);
    } else {
      stage_pv(k);
    }
  }

  // Row sums: lane partials -> per head, over the waves of each head block.
  const float lt = sum_g(lp);
  wait_lgkm0();
  bar();
  if (g == 0) smax[st_tile * C::HW + shead] = lt;
  wait_lgkm0();
  bar();
  const size_t pidx = ((size_t)pbase + split) * H;
  const __amdgpu_buffer_rsrc_t ro =
      make_rsrc(a.part_o, (uint32_t)((size_t)a.nparts * H * R * 4));
  const __amdgpu_buffer_rsrc_t rml =
      make_rsrc(a.part_ml, (uint32_t)((size_t)a.nparts * H * 8));
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
        st_coh4(ro, (uint32_t)(((pidx + head) * R + ch) * 4), o[hb][qb]);
      }
    }
    if (ns > 1 && wave == 0 && g == 0) {
      st_coh1(rml, (uint32_t)((pidx + head) * 8), m[hb]);
      st_coh1(rml, (uint32_t)((pidx + head) * 8 + 4), L);
    }
  }
  if (ns == 1) return;

  // The last split of this sequence to finish merges all of them.
  int *last = (int *)(pbuf + C::P_B);
  __syncthreads();   // this workgroup's partial stores have completed
  if (tid == 0) *last = ctr_add(&a.counters[b], 1) == ns - 1;
  __syncthreads();
  if (!*last) return;
  merge_partials<T, R>(a, b, ns, pbase, ro, rml);
}

// Nine score operand fragments of a tile (row lane % 16, k-steps ks0 ..
// ks0 + 8), read in one batch: k-step ks sits at (ks odd ? o : e) +
// (ks >> 1) * stride bytes in the decode tile layout (stride 2048 for rows of
// a multiple of 128 bytes, 1024 for paired 576-byte rows).  Each asm block
// waits for its own reads.
__device__ __forceinline__ void read_frags_l1_lo(bf16x8 (&f)[9], uint32_t e, uint32_t o) {
  asm volatile(
      "ds_read_b128 %0, %9 offset:0\n\t"
      "ds_read_b128 %1, %10 offset:0\n\t"
      "ds_read_b128 %2, %9 offset:2048\n\t"
      "ds_read_b128 %3, %10 offset:2048\n\t"
      "ds_read_b128 %4, %9 offset:4096\n\t"
      "ds_read_b128 %5, %10 offset:4096\n\t"
      "ds_read_b128 %6, %9 offset:6144\n\t"
      "ds_read_b128 %7, %10 offset:6144\n\t"
      "ds_read_b128 %8, %9 offset:8192\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3]), "=&v"(f[4]), "=&v"(f[5]), "=&v"(f[6]), "=&v"(f[7]), "=&v"(f[8])
      : "v"(e), "v"(o)
      : "memory");
}
__device__ __forceinline__ void read_frags_l1_hi(bf16x8 (&f)[9], uint32_t e, uint32_t o) {
  asm volatile(
      "ds_read_b128 %0, %10 offset:8192\n\t"
      "ds_read_b128 %1, %9 offset:10240\n\t"
      "ds_read_b128 %2, %10 offset:10240\n\t"
      "ds_read_b128 %3, %9 offset:12288\n\t"
      "ds_read_b128 %4, %10 offset:12288\n\t"
      "ds_read_b128 %5, %9 offset:14336\n\t"
      "ds_read_b128 %6, %10 offset:14336\n\t"
      "ds_read_b128 %7, %9 offset:16384\n\t"
      "ds_read_b128 %8, %10 offset:16384\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3]), "=&v"(f[4]), "=&v"(f[5]), "=&v"(f[6]), "=&v"(f[7]), "=&v"(f[8])
      : "v"(e), "v"(o)
      : "memory");
}
__device__ __forceinline__ void read_frags_l2(bf16x8 (&f)[9], uint32_t e, uint32_t o) {
  asm volatile(
      "ds_read_b128 %0, %9 offset:0\n\t"
      "ds_read_b128 %1, %10 offset:0\n\t"
      "ds_read_b128 %2, %9 offset:1024\n\t"
      "ds_read_b128 %3, %10 offset:1024\n\t"
      "ds_read_b128 %4, %9 offset:2048\n\t"
      "ds_read_b128 %5, %10 offset:2048\n\t"
      "ds_read_b128 %6, %9 offset:3072\n\t"
      "ds_read_b128 %7, %10 offset:3072\n\t"
      "ds_read_b128 %8, %9 offset:4096\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3]), "=&v"(f[4]), "=&v"(f[5]), "=&v"(f[6]), "=&v"(f[7]), "=&v"(f[8])
      : "v"(e), "v"(o)
      : "memory");
}

// Warp-specialised form of the attention kernel (bf16, an even number of
// 16-row tiles per stage: up to 32 heads).  Eight waves, two per SIMD:
//  * score waves 0-3 stream the stages and compute the scores of stage k
//    (wave w: one (tile, head block) pair), writing the scaled scores and the
//    pair's per-head maxima to LDS;
//  * value waves 4-7 run the softmax of stage k (reference max per head,
//    lazily moved; O rescaled when it moves; P kept in registers in the
//    layout of the P.V operand, which is the layout of the score products)
//    and accumulate O^T += C^T P^T of stage k for their quarter of the latent
//    channels, while the score waves compute stage k+1.
// A score wave and a value wave share each SIMD, so one's products and
// waits overlap the other's.  One barrier per stage: once it is passed,
// stage k has landed, the scores of stage k-1 are written (scores and maxima
// are double-buffered by stage parity), and the P.V of stage k-2 is done, so
// its ring slot can be refilled.
template <int R, int DR, int NHB>
__global__ __launch_bounds__(512) void decode_ws_kernel(DecodeArgs a) {
  using T = bf16;
  using C = DecCfg<T, R, DR, NHB>;
  using Lay = DecLayout<C::RB>;
  static_assert(C::TPS % 2 == 0, "pairs of 16-row tiles per stage");
  static_assert(C::KS == 18 || C::KS == 9, "batched score reads for r + d_hR = 576 or 288");
  constexpr int HW = C::HW;
  constexpr int NPAIR = C::TPS / 2;
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int b, split, ns, pbase, start, end, t;
  if (!decode_work<T, R, C::SROWS>(a, b, split, ns, pbase, start, end, t)) return;
  const int s = a.s, H = a.H;
  const int jn = t / s, n = jn + 1;
  const bool owner = end == n;
  const int nstage = (end - start + C::SROWS - 1) / C::SROWS;
  const bool scorer = wave < 4;
  const int w4 = wave & 3, stid = tid & 255;
  const int g = lane >> 4, c = lane & 15;
  char *seq = a.cache + (size_t)b * a.bstride_bytes;
  char *dummy = smem + a.nst * C::STAGE_B;
  float *smax = (float *)(dummy + 1024);                  // [2][TPS][HW] maxima of the pairs
  f32x4 *zbuf = (f32x4 *)((char *)smax + 2 * C::SMAX_B);  // [2][TPS][NHB][64] scaled scores
  int *last = (int *)(zbuf + 2 * C::TPS * NHB * 64);      // last-split flag
  constexpr int ZB = C::TPS * NHB * 64;                   // scores per buffer

  auto issue = [&](int sidx) {
    char *sb = smem + (sidx % a.nst) * C::STAGE_B;
    const int row0 = start + sidx * C::SROWS;
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) {
      const int blk = w4 + 4 * i;
      const bool real = (C::NBLK % 4 == 0) || blk < C::NBLK;
      const int tl = real ? blk / C::NSEG : 0, bq = real ? blk % C::NSEG : 0;
      int rr, bb;
      Lay::src(bq, lane, rr, bb);
      const int slot = min(row0 + tl * 16 + rr, end - 1);
      __builtin_amdgcn_global_load_lds((const void *)(seq + (size_t)slot * C::RB + bb),
                                       (lds_void *)(real ? sb + tl * C::TILE_B + bq * 1024 : dummy),
                                       16, 0, kStreamPolicy);
    }
  };

  const size_t pidx = ((size_t)pbase + split) * H;
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.part_o, (uint32_t)((size_t)a.nparts * H * R * 4));
  const __amdgpu_buffer_rsrc_t rml = make_rsrc(a.part_ml, (uint32_t)((size_t)a.nparts * H * 8));

  // The two roles run separate loops with the same barriers in the same
  // order (so each role's registers are live only in its own loop).
  if (scorer) {
    const int st_tile = w4 % C::TPS, st_hb = w4 / C::TPS;   // this wave's score pair
    const int shead = st_hb * 16 + c;
    // Queries, and (owner) the merge inputs, fetched before the stream so
    // that later waits for them never wait for the stream.
    bf16x8 q[C::KS];
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
        const int ch = stid + 256 * i;
        if (ch < R) {
          mc[i] = a.cg[(size_t)b * 2 * R + ch];
          mg[i] = a.cg[(size_t)b * 2 * R + R + ch];
          mb[i] = ((const T *)a.b_hc)[ch];
          mp[i] = a.gate_pos[(size_t)jn * R + ch];
        }
      }
      if (stid < DR) mkr = ((const T *)a.KR)[(size_t)b * DR + stid];
    }
    asm volatile("" ::: "memory");
    const int pro = min(a.nst, nstage);
    for (int k = 0; k < pro; ++k) issue(k);
    int lastst = pro - 1;   // newest stage issued so far

    for (int k = 0; k <= nstage; ++k) {
      if (k < nstage) wait_stages<C::LPW>(lastst - k);
      wait_lgkm0();
      bar();   // stage k landed; scores k-1 written; P.V(k-2) done, its slot free
      if (k >= 2 && k - 2 + a.nst < nstage) {
        issue(k - 2 + a.nst);
        lastst = k - 2 + a.nst;
      }
      if (k == nstage - 1) {
        // Last stage: rows past the split read as zeros (their weight is
        // exactly 0, but the P.V product must not meet stale non-finite LDS
        // contents), and the owner merges the new frame into the newest slot
        // ([Notes] hyper-network temporal merging; [Fig2] (a)), in the cache
        // and in its LDS copy.
        char *sb = smem + (k % a.nst) * C::STAGE_B;
        const int row0 = start + k * C::SROWS;
        const int nz = row0 + C::SROWS - end;
        for (int idx = stid; idx < nz * (C::RB / 16); idx += 256) {
          const int r = end - row0 + idx / (C::RB / 16), ch = idx % (C::RB / 16);
          *(u32x4 *)(sb + (r >> 4) * C::TILE_B + Lay::off(r & 15, ch * 16)) = (u32x4){0u, 0u, 0u, 0u};
        }
        if (owner) {
          const int rr = jn - row0;
          char *trow = sb + (rr >> 4) * C::TILE_B;
          T *grow = (T *)(seq + (size_t)jn * C::RB);
          const bool open = (t % s) == 0;
#pragma unroll
          for (int i = 0; i < C::NU; ++i) {
            const int ch = stid + 256 * i;
            if (ch < R) {
              T *lpnt = (T *)(trow + Lay::off(rr & 15, ch * 2));
              const float u = sigmoidf((mg[i] + to_f32(mb[i])) * mp[i]) * mc[i];
              const T v = from_f32<T>(open ? u : to_f32(*lpnt) + u);
              *lpnt = v;
              grow[ch] = v;
            }
          }
          if (stid < DR) {
            *(T *)(trow + Lay::off(rr & 15, (R + stid) * 2)) = mkr;
            grow[R + stid] = mkr;
          }
        }
        wait_lgkm0();
        bar();
      }
      if (k < nstage) {
        // Scores of this wave's (tile, head block) pair.
        const char *stile = smem + (k % a.nst) * C::STAGE_B + st_tile * C::TILE_B;
        const int kb = start + k * C::SROWS + st_tile * 16;
        const uint32_t fe = lds_addr(stile + Lay::off(c, 16 * g));
        const uint32_t fo = lds_addr(stile + Lay::off(c, 64 + 16 * g));
        f32x4 sa[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sa[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
        {
          bf16x8 kf[9];
          if constexpr (C::KS == 18) read_frags_l1_lo(kf, fe, fo);
          else read_frags_l2(kf, fe, fo);
#pragma unroll
          for (int i = 0; i < 9; ++i) sa[i & 3] = mma_k32(kf[i], q[i], sa[i & 3]);
        }
        if constexpr (C::KS == 18) {
          bf16x8 kf[9];
          read_frags_l1_hi(kf, fe, fo);
#pragma unroll
          for (int i = 0; i < 9; ++i) sa[(9 + i) & 3] = mma_k32(kf[i], q[9 + i], sa[(9 + i) & 3]);
        }
        f32x4 z;
        float mx = kNegInf;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          z[e] = (kb + 4 * g + e < end) ? ((sa[0][e] + sa[1][e]) + (sa[2][e] + sa[3][e])) * a.sl2
                                        : kNegInf;
          mx = fmaxf(mx, z[e]);
        }
        mx = max_g(mx);   // -inf only for a tile wholly past the split
        if (g == 0) smax[(k & 1) * (C::TPS * HW) + st_tile * HW + shead] = mx;
        zbuf[(k & 1) * ZB + (st_tile * NHB + st_hb) * 64 + lane] = z;
      }
    }
  } else {
    // o[hb][qb]: O^T of channels 16 (w4 * MQ + qb) + 4g + e, head hb * 16 +
    // c.  m[hb]: reference max of that head (the same in every value wave);
    // lp[hb]: this lane's partial sum of its P.  pp: P of the stage awaiting
    // its P.V, per head block and tile pair, in the operand layout (k index
    // 8g + e: slot 4g + e of the pair's first tile for e < 4, of its second
    // for e >= 4).
    f32x4 o[NHB][C::MQ];
    float m[NHB], lp[NHB];
    bf16x8 pp[NHB][NPAIR];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      m[hb] = kNegInf;
      lp[hb] = 0.0f;
#pragma unroll
      for (int qb = 0; qb < C::MQ; ++qb) o[hb][qb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    for (int k = 0; k <= nstage; ++k) {
      wait_lgkm0();
      bar();   // stage k landed; scores k-1 written
      if (k == nstage - 1) bar();   // the score waves' last-stage fix-ups
      if (k == 0) continue;
      const int kk = k - 1;   // the stage this iteration finishes
      {
        // Softmax of stage kk: move the reference max of a head when a score
        // exceeds it by more than 2^8 (rescaling O, which holds the stages
        // before kk), then P = 2^(z - m) in the operand layout.
        const float *sm_k = smax + (kk & 1) * (C::TPS * HW);
        const f32x4 *zb = zbuf + (kk & 1) * ZB;
        float mnew[NHB];
        bool up_any = false;
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
          float sm = kNegInf;
#pragma unroll
          for (int tl = 0; tl < C::TPS; ++tl) sm = fmaxf(sm, sm_k[tl * HW + hb * 16 + c]);
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
            lp[hb] *= alpha;
            m[hb] = mnew[hb];
          }
        }
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
#pragma unroll
          for (int pair = 0; pair < NPAIR; ++pair) {
            const f32x4 z0 = zb[((2 * pair) * NHB + hb) * 64 + lane];
            const f32x4 z1 = zb[((2 * pair + 1) * NHB + hb) * 64 + lane];
            bf16x8 pv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float p0 = __builtin_amdgcn_exp2f(z0[e] - m[hb]);
              const float p1 = __builtin_amdgcn_exp2f(z1[e] - m[hb]);
              lp[hb] += p0 + p1;
              pv[e] = from_f32<T>(p0);
              pv[4 + e] = from_f32<T>(p1);
            }
            pp[hb][pair] = pv;
          }
        }
      }
      // O^T += C^T P^T of stage kk, this wave's channel quarter.
      const char *sb = smem + (kk % a.nst) * C::STAGE_B;
      const int row0 = start + kk * C::SROWS;
#pragma unroll
      for (int pair = 0; pair < NPAIR; ++pair) {
        const int tl = 2 * pair;
        if (row0 + tl * 16 >= end) continue;   // a pair wholly past the split
        const char *t0 = sb + tl * C::TILE_B;
#pragma unroll
        for (int q0 = 0; q0 < C::MQ; q0 += 4) {
          uint32_t ad[8];
          bf16x4 v[8];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int ch0 = 16 * (w4 * C::MQ + q0 + j);
            ad[2 * j] = lds_addr(t0 + Lay::off(4 * g + (c >> 2), (ch0 + 4 * (c & 3)) * 2));
            ad[2 * j + 1] = ad[2 * j] + C::TILE_B;
          }
          ds_read_tr8(v, ad);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bf16x8 vv = __builtin_shufflevector(v[2 * j], v[2 * j + 1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
            for (int hb = 0; hb < NHB; ++hb) o[hb][q0 + j] = mma_k32(vv, pp[hb][pair], o[hb][q0 + j]);
          }
        }
      }
    }
    // Row sums over the lane groups, then this split's result.
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      const int head = hb * 16 + c;
      const float L = sum_g(lp[hb]);
      if (head >= H) continue;
#pragma unroll
      for (int qb = 0; qb < C::MQ; ++qb) {
        const int ch = 16 * (w4 * C::MQ + qb) + 4 * g;
        if (ns == 1) {
          T *dst = (T *)a.o + ((size_t)b * H + head) * R + ch;
          const float inv = 1.0f / L;
#pragma unroll
          for (int e = 0; e < 4; ++e) dst[e] = from_f32<T>(o[hb][qb][e] * inv);
        } else {
          st_coh4(ro, (uint32_t)(((pidx + head) * R + ch) * 4), o[hb][qb]);
        }
      }
      if (ns > 1 && w4 == 0 && g == 0) {
        st_coh1(rml, (uint32_t)((pidx + head) * 8), m[hb]);
        st_coh1(rml, (uint32_t)((pidx + head) * 8 + 4), L);
      }
    }
  }
  if (ns == 1) return;
  __syncthreads();   // this workgroup's partial stores have completed
  if (tid == 0) *last = ctr_add(&a.counters[b], 1) == ns - 1;
  __syncthreads();
  if (!*last) return;
  merge_partials<T, R>(a, b, ns, pbase, ro, rml);
}

// Stand-alone merge-append: one workgroup per sequence.  A position outside
// [0, max_pos] drops the frame (counted in *status).
template <typename T>
__global__ __launch_bounds__(256) void merge_kernel(const int32_t *pos, int max_pos, int s, int R,
                                                    int DR, const float *cg, const T *b_hc,
                                                    const float *gate_pos, const T *KR,
                                                    char *cache, int64_t bstride_bytes,
                                                    int *status) {
  const int b = blockIdx.x, t = pos[b];
  if (t < 0 || t > max_pos) {
    if (threadIdx.x == 0) atomicAdd(status, 1);
    return;
  }
  const int j = t / s;
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
  const dim3 grid = p.flat ? dim3(p.grid) : dim3(p.splits, B);
  if constexpr (sizeof(T) == 2 && NHB <= 2) {
    if (p.ws) {
      auto kern = decode_ws_kernel<R, DR, NHB>;
      allow_lds<decode_ws_kernel<R, DR, NHB>>();
      return launch_timed((const void *)kern, grid, dim3(512), p.lds, stream, &args, ev0, ev1);
    }
  }
  auto kern = decode_attn_kernel<T, R, DR, NHB>;
  allow_lds<decode_attn_kernel<T, R, DR, NHB>>();
  return launch_timed((const void *)kern, grid, dim3(256), p.lds, stream, &args, ev0, ev1);
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
  // Warp-specialised kernel: bf16 with pairs of 16-row tiles per stage.
  p.ws = (dtype == 1 && p.nhb <= 2) ? 1 : 0;
  const size_t hw = (size_t)16 * p.nhb;
  const size_t extra = p.ws ? 1024 + 2 * (size_t)tps * hw * 4 + 2 * (size_t)tps * p.nhb * 64 * 16 + 16
                            : 1024 + (size_t)tps * hw * 4 + (size_t)tps * p.nhb * 64 * 4 * esz + 16;
  const int64_t nmax = max_pos / s + 1;
  const int64_t mstages = (nmax + srows - 1) / srows;   // stages of the longest sequence
  p.block = srows;
  // Ring: about 4 stages of 36 KB, or more of smaller stages (at most 8).
  int nst = (int)(144 * 1024 / stage);
  if (nst > 8) nst = 8;
  // The kernels refill a stage's slot two stages after its scores (once its
  // P.V is done), so a split of several stages needs a ring of at least three.
  // Balanced work list on the device for up to 256 sequences (four per lane
  // of the kernel's tables), when a split may hold more than one stage.
  p.flat = (B <= 256 && nst >= 3) ? 1 : 0;
  if (p.flat) {
    int64_t G = B <= MTLA_DECODE_TARGET_WGS / 2
                    ? MTLA_DECODE_TARGET_WGS
                    : ((2 * (int64_t)B + MTLA_DECODE_TARGET_WGS - 1) / MTLA_DECODE_TARGET_WGS) *
                          MTLA_DECODE_TARGET_WGS;
    if (G > (int64_t)B * mstages) G = (int64_t)B * mstages;   // never more splits than stages
    if (G < B) G = B;
    p.grid = (int)G;
    p.nparts = (int)G;
    p.chunk = 0;
    p.splits = 0;
    if (nst > mstages) nst = (int)mstages;
  } else {
    const int64_t total = (int64_t)B * nmax;
    int64_t chunk = (total + MTLA_DECODE_TARGET_WGS - 1) / MTLA_DECODE_TARGET_WGS;
    chunk = ((chunk + srows - 1) / srows) * srows;
    const int64_t cap = mstages * srows;
    if (chunk > cap) chunk = cap;
    if (nst < 3) {
      // A ring of fewer than three slots cannot refill the slot two stages
      // back while the newest one is read: give each split a single stage
      // instead (more splits, same bytes).
      nst = 1;
      chunk = srows;
    }
    if (nst > chunk / srows) nst = (int)(chunk / srows);
    p.chunk = (int)chunk;
    p.splits = (int)((nmax + chunk - 1) / chunk);
    p.grid = 0;
    if ((int64_t)B * p.splits > 0x7fffffffLL) return false;
    p.nparts = B * p.splits;
  }
  if (nst < 1) nst = 1;
  p.nst = nst;
  p.lds = nst * stage + extra;
  if (p.lds > 159 * 1024) return false;
  *plan = p;
  return true;
}

hipError_t launch_decode_attention(int dtype, const DecodePlan &plan, int B, int H, int r, int dR,
                                   int s, float scale, const int32_t *pos, int max_pos, void *cache,
                                   int64_t batch_stride, const void *qt, const void *QR,
                                   const void *KR_t, const float *cg, const void *b_hc,
                                   const float *gate_pos, float *part_o, float *part_ml,
                                   int *counters, int *status, void *o, hipStream_t stream,
                                   hipEvent_t ev0, hipEvent_t ev1) {
  const int esz = dtype == 1 ? 2 : 4;
  DecodeArgs args;
  args.pos = pos;
  args.cache = (char *)cache;
  args.bstride_bytes = batch_stride * esz;
  args.qt = qt;
  args.QR = QR;
  args.KR = KR_t;
  args.cg = cg;
  args.b_hc = b_hc;
  args.gate_pos = gate_pos;
  args.part_o = part_o;
  args.part_ml = part_ml;
  args.counters = counters;
  args.status = status;
  args.o = o;
  args.B = B;
  args.H = H;
  args.s = s;
  args.chunk = plan.chunk;
  args.splits = plan.splits;
  args.nst = plan.nst;
  args.nparts = plan.nparts;
  args.max_pos = max_pos;
  args.flat = plan.flat;
  args.sl2 = scale * kLog2e;
  if (dtype == 1) {
    if (r == 256) return decode_attn_h<bf16, 256, 32>(plan, B, args, stream, ev0, ev1);
    return decode_attn_h<bf16, 512, 64>(plan, B, args, stream, ev0, ev1);
  }
  if (r == 256) return decode_attn_h<float, 256, 32>(plan, B, args, stream, ev0, ev1);
  return decode_attn_h<float, 512, 64>(plan, B, args, stream, ev0, ev1);
}

hipError_t launch_merge(int dtype, int B, int r, int dR, int s, const int32_t *pos, int max_pos,
                        const float *cg, const void *b_hc, const float *gate_pos, const void *KR_t,
                        void *cache, int64_t batch_stride, int *status, hipStream_t stream) {
  const int esz = dtype == 1 ? 2 : 4;
  if (dtype == 1)
    hipLaunchKernelGGL(merge_kernel<bf16>, dim3(B), dim3(256), 0, stream, pos, max_pos, s, r, dR,
                       cg, (const bf16 *)b_hc, gate_pos, (const bf16 *)KR_t, (char *)cache,
                       batch_stride * esz, status);
  else
    hipLaunchKernelGGL(merge_kernel<float>, dim3(B), dim3(256), 0, stream, pos, max_pos, s, r, dR,
                       cg, (const float *)b_hc, gate_pos, (const float *)KR_t, (char *)cache,
                       batch_stride * esz, status);
  return hipGetLastError();
}

}  // namespace mtla
