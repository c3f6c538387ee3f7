// Launchers of the MTLA kernels; every launcher enqueues on `stream` and
// returns hipGetLastError() of its launch.  Attention launchers take an
// optional pair of events that the runtime stamps with the kernel's own
// start and end.  Pointers are device pointers in
// the storage type selected by `dtype` (0 fp32, 1 bf16) unless typed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtla {

// ---- dense NT products (C = A B^T) on MFMA --------------------------------

// out[M, N] = A[M, K] B[N, K]^T, written in the storage type with row stride ldc.
hipError_t launch_gemm_store(int dtype, const void *A, int lda, const void *Bm, int ldb, int M,
                             int N, int K, void *out, int ldc, hipStream_t stream);

// out[M, N] = A[M, K] [B1; B2]^T: output columns < N1 from the rows of B1,
// the others from the rows of B2 (both with row stride ldb).
hipError_t launch_gemm_store2(int dtype, const void *A, int lda, const void *B1, const void *B2,
                              int N1, int ldb, int M, int N, int K, void *out, int ldc,
                              hipStream_t stream);

// out[M, N] (fp32, row stride ldc) = A[M, K] B[N, K]^T, or += when add.
hipError_t launch_gemm_f32(int dtype, const void *A, int lda, const void *Bm, int ldb, int M, int N,
                           int K, float *out, int ldc, bool add, hipStream_t stream);

// out[M, N] (bf16, row stride ldc) = acc[M, N] (fp32, row stride ldacc) + A[M, K] B[N, K]^T
// (bf16 operands).
hipError_t launch_gemm_add_bf16(const void *A, int lda, const void *Bm, int ldb, int M, int N, int K,
                                const float *acc, int ldacc, void *out, int ldc,
                                hipStream_t stream);

// out[M, N] (fp32) = A[M, K] [B1; B2]^T (columns < N1 from B1's rows).
hipError_t launch_gemm_f32_2(int dtype, const void *A, int lda, const void *B1, const void *B2,
                             int N1, int ldb, int M, int N, int K, float *out, int ldc,
                             hipStream_t stream);

// Decoupled-RoPE inputs: G [M, HR + DR] (fp32 scratch) = X [M, d] [W_QR; W_KR]^T,
// then QR [M, HR] and KR [M, DR] (storage type) = G's adjacent pairs turned
// by pos[m] * base^(-2k/DR) (k: the pair's index within its DR-wide vector).
hipError_t launch_rope_inputs(int dtype, const void *X, int M, int d, const void *W_QR, int HR,
                              const void *W_KR, int DR, const int32_t *pos, float base, float *G,
                              void *QR, void *KR, hipStream_t stream);

// table[rows, r] (fp32) = pe[rows, d_pe] W_hp[r, d_pe]^T + b_hp.
hipError_t launch_pos_table(int dtype, const void *pe, int rows, int d_pe, const void *W_hp,
                            const void *b_hp, int r, float *table, hipStream_t stream);

// W_gate[r, d] = W_hc[r, r] W_dkv[r, d] (fp32 accumulation, storage type).
hipError_t launch_gate_map(int dtype, const void *W_hc, const void *W_dkv, int r, int d,
                           void *W_gate, hipStream_t stream);

// One pass over X [M, d]: cg [M, 2r] (fp32) = (X W_dkv^T, X W_gate^T), and,
// when A != nullptr, qt [M, HR] (storage type) = X A^T with A [HR, d].  When
// `zero` is given its first `nzero` ints are cleared first (the counters of
// the kernels that follow in a decoding step).
hipError_t launch_proj(int dtype, const void *X, int M, int d, const void *W_dkv,
                       const void *W_gate, int r, const void *A, int HR, float *cg, void *qt,
                       int *zero, int nzero, hipStream_t stream);

// Y [M, N] = O [M, K] Bvo [N, K]^T.  For M <= 128 with `part` and `counters`
// given, K is split over workgroups with fp32 partials in `part`
// (out_proj_part_bytes) and counters (at most out_proj_counters of them),
// zero on entry and zero again on exit: up to 64 rows as narrow column strips
// (out_proj_splits splits); 65..128 rows in bf16 with K a multiple of 64 by
// the weight-streaming product (stream_gemm_plan), otherwise as 128-row
// tiles.
hipError_t launch_out_proj(int dtype, const void *O, int M, int K, const void *Bvo, int N, void *Y,
                           float *part, int *counters, hipStream_t stream);
int out_proj_splits(int M, int N, int K);
// Bytes of fp32 partials launch_out_proj needs in `part` (esz: storage bytes).
size_t out_proj_part_bytes(int esz, int M, int N, int K);
int out_proj_strips(int M, int N);
// Counters launch_out_proj may use (esz: storage bytes).
int out_proj_counters(int esz, int M, int N, int K);

// ---- incremental decoding ---------------------------------------------------

struct DecodePlan {
  int nhb;      // head blocks of 16
  int block;    // slots per LDS stage
  int flat;     // 1: balanced work list derived on the device from the positions
  int ws;       // 1: warp-specialised kernel (512 threads)
  int grid;     // workgroups (flat)
  int chunk;    // slots per split (uniform splits, flat == 0)
  int splits;   // splits per sequence (uniform: grid x, with grid y = B)
  int nparts;   // split partials the workspace holds
  int nst;      // LDS ring stages
  size_t lds;   // dynamic LDS bytes
};

// Work decomposition of the split-K decode attention for B sequences whose
// positions are all <= max_pos.  Returns false for unsupported shapes.
bool decode_plan(int dtype, int H, int r, int dR, int s, int B, int max_pos, DecodePlan *plan);

// Merge of frame pos[b] into slot floor(pos[b]/s) of every sequence (from
// cg = (c, gate pre-activation) and the tables), then attention over slots
// 0..floor(pos[b]/s) into o [B, H, r] (storage type).  qt [B, H, r], QR
// [B, H, dR], KR_t [B, dR]; split partials part_o [plan.nparts, H, r] and
// part_ml [plan.nparts, H, 2] fp32; counters [B], zero on entry (zero again
// on exit).  A sequence with pos[b] outside [0, max_pos] is dropped (no
// merge, o row zero) and counted in *status (cleared by the caller).
hipError_t launch_decode_attention(int dtype, const DecodePlan &plan, int B, int H, int r, int dR,
                                   int s, float scale, const int32_t *pos, int max_pos, void *cache,
                                   int64_t batch_stride, const void *qt, const void *QR,
                                   const void *KR_t, const float *cg, const void *b_hc,
                                   const float *gate_pos, float *part_o, float *part_ml,
                                   int *counters, int *status, void *o, hipStream_t stream,
                                   hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);

// Merge alone (no attention), one workgroup per sequence; positions outside
// [0, max_pos] are dropped and counted in *status.
hipError_t launch_merge(int dtype, int B, int r, int dR, int s, const int32_t *pos, int max_pos,
                        const float *cg, const void *b_hc, const float *gate_pos, const void *KR_t,
                        void *cache, int64_t batch_stride, int *status, hipStream_t stream);

// Chunked merge-append: sequence b folds frames pos0[b] .. pos0[b] + n_b - 1
// (n_b = lens[b] clamped to [0, L], or L when lens is null) into its cache in
// frame order, continuing a live partial slot, from cg [B, L, 2r]; KR
// [B, L, dR].  Cp [B, L, r] (nullable) receives each frame's running slot
// state.  Slots >= jlim are skipped.  chunk_slots(L, s) bounds the slots one
// chunk of L frames can touch.
hipError_t launch_chunk_merge(int dtype, int B, int L, int r, int dR, int s, const int32_t *pos0,
                              const int32_t *lens, const float *cg, const void *b_hc,
                              const float *table, int jlim, const void *KR, void *Cp, void *cache,
                              int64_t batch_stride, hipStream_t stream);
int chunk_slots(int L, int s);

// ---- parallel form ----------------------------------------------------------

// Hyper-network gate and segmented (per group of s frames) inclusive sum:
// U[b, i] = Sigmoid((g + b_hc) * table[floor(i/s)]) * c from cg [B*T, 2r],
// then the intermediate states C' [B, T, r], plus the compressed rows
// keys[b, j] = (C'_e(j), KR_e(j)) with e(j) = min(s*j + s - 1, T - 1), into
// `keys` [B, keys_stride] and, when cache != nullptr, into the caller's cache.
hipError_t launch_group_scan(int dtype, const float *cg, const void *b_hc, const float *table,
                             const void *KR, int B, int T, int r, int dR, int s, void *Cp,
                             void *keys, int64_t keys_stride, void *cache, int64_t cache_stride,
                             hipStream_t stream);

// Stride-aware masked attention: O [B, T, H, r] from queries qt [B, T, H, r],
// QR [B, T, H, dR], the compressed keys [B, keys_stride] (ceil(T/s) rows of
// r + dR), and the diagonal terms C' [B, T, r], KR [B, T, dR].
hipError_t launch_prefill_attention(int dtype, int B, int T, int H, int r, int dR, int s,
                                    float scale, const void *qt, const void *QR, const void *keys,
                                    int64_t keys_stride, const void *Cp, const void *KR, void *O,
                                    hipStream_t stream,
                                    hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);

bool prefill_attention_supported(int dtype, int H, int r, int dR);

// Per-head (unabsorbed) stride-aware masked attention, bf16, (d_h, dR) =
// (64, 32) or (128, 64): O [B*T, H*d_h] from q [B*T, H*d_h], QR [B*T, H, dR],
// KV [B*T, 2*H*d_h] (K_h at column d_h h, V_h at d_h (H + h)) and KR
// [B*T, dR].  lse (nullable) [B*T, H] fp32 receives each row's log2 softmax
// sum in the kernel's scaled log2 units (weights p = exp2(z * scale *
// log2(e) - lse)).
hipError_t launch_heads_attention(int B, int T, int H, int d_h, int s, float scale, const void *q,
                                  const void *QR, const void *KV, const void *KR, void *O,
                                  float *lse, hipStream_t stream, hipEvent_t ev0 = nullptr,
                                  hipEvent_t ev1 = nullptr);
// The same attention with fp32 storage (heads_f32.hip): a correctness-
// oriented kernel with the same operand layouts; lse (optional, [B*T, H])
// receives each row's log2-sum-exp of the scores in log2 units.
hipError_t launch_heads_attention_f32(int B, int T, int H, int d_h, int s, float scale,
                                      const void *q, const void *QR, const void *KV,
                                      const void *KR, void *O, float *lse, hipStream_t stream,
                                      hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
bool heads_attention_supported(int dtype, int H, int d_h, int dR);

// ---- backward of the per-head parallel form (bf16 MFMA kernels, (d_h, dR) = (64, 32) or (128, 64)) ----

bool attn_bwd_supported(int dtype, int H, int d_h, int dR);
// Attention backward over the forward's q, QR, KV, KR, its lse and
// D = rowsum(dO * O): key-role gradients of the compact keys into dKVc
// [B*nS, 2*H*d_h] and dKRc [B*nS, H, dR] (fp32 scratch), then every frame's
// total dK | dV into dKV [B*T, 2*H*d_h] (bf16) and per-head dK^R into dKRh
// [B*T, H, dR] (fp32), and dQ [B*T, H*d_h] (row stride ldq), dQR [B*T, H, dR] (bf16).
hipError_t launch_attn_bwd(int B, int T, int H, int d_h, int s, float scale, const void *q,
                           const void *QR, const void *KV, const void *KR, const void *dO,
                           const float *lse, const float *D, float *dKVc, float *dKRc, void *dKV,
                           float *dKRh, void *dQ, void *dQR, int ldq, hipStream_t stream);
// D[i] = sum over d_h channels of dO[i, :] * O[i, :], i < MH (rows of d_h).
hipError_t launch_rowdot(const void *dO, const void *O, int MH, int d_h, float *D,
                         hipStream_t stream);
// dKR [M, dR] (storage dtype) = sum over heads of dKRh [M, H, dR].
hipError_t launch_head_sum(int dtype, const float *dKRh, int M, int H, int dR, void *dKR,
                           hipStream_t stream);
// Reverse group scan and gate backward from dC' [B*T, R] (fp32) and the
// forward's cg: da (fp32 and bf16), dc's direct term (fp32), c (bf16).
// dPpart [B, ceil(T/s), R] receives each sequence's position-branch
// gradient, and dPtab [rows, R] = their sum over the sequences in order
// (rows past ceil(T/s) are zero).
hipError_t launch_scan_gate_bwd(int dtype, const float *dCp, const float *cg, const void *b_hc,
                                const float *table, int B, int T, int R, int s, float *da32,
                                void *dab, float *dc32, void *cb, float *dPpart, int rows,
                                float *dPtab, hipStream_t stream);
// out[N] = column sums of x [M, N] (fp32), partial sums over row chunks
// added in a fixed order: part holds colsum_part_bytes, ctr colsum_counters
// ints (zero on entry, zero again on exit).
hipError_t launch_colsum(const float *x, int M, int N, float *part, int *ctr, float *out,
                         hipStream_t stream);
size_t colsum_part_bytes(int M, int N);
int colsum_counters(int N);
hipError_t launch_zero_f32(float *p, size_t n, hipStream_t stream);
hipError_t launch_zero_i32(int *p, size_t n, hipStream_t stream);
// out[C, R] (row stride ldo) = in[R, C]^T (bf16, row stride ldi).
hipError_t launch_transpose(const void *in, int R, int C, int ldi, void *out, int ldo,
                            hipStream_t stream);
// out[N1, N2] (fp32, row stride ldo) = A[M, N1]^T B[M, N2] (bf16), split
// over M; the splits' partials (in part) are added in split order.
hipError_t launch_tn_gemm(const void *A, int lda, const void *Bm, int ldb, int M, int N1, int N2,
                          float *out, int ldo, float *part, hipStream_t stream);
// Partials (bytes) launch_tn_gemm needs for this shape.
size_t tn_gemm_part_bytes(int M, int N1, int N2);
// The 256 x 256 tile of A^T B (csrc/gemm_big.hip): shapes it takes, and the
// launch of its product over `splits` frame chunks of mchunk (slab z of part
// at z * N1 * N2 floats, or out when splits == 1).
bool tn_big_supported(int N1, int N2);
hipError_t launch_tn_big(const void *A, int lda, const void *Bm, int ldb, int M, int N1, int N2,
                         int mchunk, int splits, float *out, int ldo, float *part,
                         hipStream_t stream);

// ---- backward of the per-head parallel form with fp32 storage (backward_f32.hip) ----

// Attention backward from the fp32 forward's q, QR, KV, KR, lse (log2
// units) and D = rowsum(dO * O): every frame's dK | dV into dKV [B*T,
// 2*H*d_h], per-head dK^R into dKRh [B*T, H, dR], dQ [B*T, H*d_h] (row
// stride ldq) and dQR [B*T, H, dR], all fp32.  d_h = 64 (dR = 32) or 128 (64).
hipError_t launch_attn_bwd_f32(int B, int T, int H, int d_h, int s, float scale, const float *q,
                               const float *QR, const float *KV, const float *KR, const float *dO,
                               const float *lse, const float *D, float *dKV, float *dKRh,
                               float *dQ, int ldq, float *dQR, hipStream_t stream);
// D[i] = sum over d_h channels of dO[i, :] * O[i, :] (fp32), i < MH.
hipError_t launch_rowdot_f32(const float *dO, const float *O, int MH, int d_h, float *D,
                             hipStream_t stream);
// C[m, n] (row stride ldc) = C0[m, n] (row stride ldc0; C0 may be C, or
// null for zero) + sum over k < K in order of A[m sam + k sak] B[k sbk + n sbn], fp32.
hipError_t launch_gemm_f32s(const float *A, size_t sam, size_t sak, const float *Bm, size_t sbk,
                            size_t sbn, int M, int N, int K, const float *C0, size_t ldc0,
                            float *C, size_t ldc, hipStream_t stream);

}  // namespace mtla
