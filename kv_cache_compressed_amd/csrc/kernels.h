// Launchers of the MTLA kernels; every launcher enqueues on `stream` and
// returns hipGetLastError() of its launch.  Pointers are device pointers in
// the storage type selected by `dtype` (0 fp32, 1 bf16) unless typed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtla {

// ---- dense NT products (C = A B^T) on MFMA --------------------------------

// out[M, N] = A[M, K] B[N, K]^T, written in the storage type with row stride ldc.
hipError_t launch_gemm_store(int dtype, const void *A, int lda, const void *Bm, int ldb, int M,
                             int N, int K, void *out, int ldc, hipStream_t stream);

// table[rows, r] (fp32) = pe[rows, d_pe] W_hp[r, d_pe]^T + b_hp.
hipError_t launch_pos_table(int dtype, const void *pe, int rows, int d_pe, const void *W_hp,
                            const void *b_hp, int r, float *table, hipStream_t stream);

// Latent projection c = X W_dkv^T for M frames, written both as fp32
// (c_f32 [M, r]) and in the storage type (c_T [M, r]).  When HR > 0 the same
// launch also produces the absorbed queries q~ = X A^T into qt [M, HR]
// (storage type), A being [HR, d].
hipError_t launch_latent_query(int dtype, const void *X, int M, int d, const void *W_dkv, int r,
                               const void *A, int HR, float *c_f32, void *c_T, void *qt,
                               hipStream_t stream);

// Hyper-network gate of the parallel form: for row m = b*T + i,
//   U[m, :] = Sigmoid((c_T[m] W_hc^T + b_hc) * table[floor(i/s)]) * c_f32[m].
hipError_t launch_gate_prefill(int dtype, const void *c_T, const float *c_f32, int M, int r,
                               const void *W_hc, const void *b_hc, const float *table, int T,
                               int s, float *U, hipStream_t stream);

// Hyper-network gate of the incremental form, merged into the cache in
// place: for sequence b with t = pos[b], j = floor(t/s),
//   u = Sigmoid((c_T[b] W_hc^T + b_hc) * table[j]) * c_f32[b]
//   slot j latent = (t mod s == 0 ? 0 : slot j latent) + u;  slot j key = KR_t[b].
hipError_t launch_gate_merge(int dtype, const void *c_T, const float *c_f32, int B, int r, int dR,
                             const void *W_hc, const void *b_hc, const float *table,
                             const int32_t *pos, int s, void *cache, int64_t batch_stride,
                             const void *KR_t, hipStream_t stream);

// ---- incremental-decoding attention ---------------------------------------

struct DecodePlan {
  int nhb;      // head blocks of 16 per wave
  int block;    // slots staged per workgroup iteration
  int chunk;    // slots per split (workgroup)
  int splits;   // splits per sequence (grid x)
  size_t lds;   // dynamic LDS bytes
};

// Work decomposition of the split-K decode attention for B sequences whose
// positions are all <= max_pos.  Returns false for unsupported shapes.
bool decode_plan(int dtype, int H, int r, int dR, int s, int B, int max_pos, DecodePlan *plan);

// Split-K attention over slots 0..floor(pos[b]/s) of every sequence.
// qt [B, H, r] and QR [B, H, dR] in the storage type; partials fp32:
// part_o [B, splits, H, r] (un-normalised, relative to part_ml's max) and
// part_ml [B, splits, H, 2] = (running max in log2 units, sum of exponentials).
hipError_t launch_decode_attention(int dtype, const DecodePlan &plan, int B, int H, int r, int dR,
                                   int s, float scale, const int32_t *pos, const void *cache,
                                   int64_t batch_stride, const void *qt, const void *QR,
                                   float *part_o, float *part_ml, hipStream_t stream);

// Log-sum-exp combine of the splits into o [B, H, r] (storage type).
hipError_t launch_decode_combine(int dtype, const DecodePlan &plan, int B, int H, int r, int s,
                                 const int32_t *pos, const float *part_o, const float *part_ml,
                                 void *o, hipStream_t stream);

// ---- parallel form ----------------------------------------------------------

// Segmented (per group of s frames) inclusive sum of U into the intermediate
// states C' [B, T, r], plus the compressed rows keys[b, j] = (C'_e(j), KR_e(j))
// with e(j) = min(s*j + s - 1, T - 1), into `keys` [B, keys_stride] and, when
// cache != nullptr, into the caller's cache.
hipError_t launch_group_scan(int dtype, const float *U, const void *KR, int B, int T, int r, int dR,
                             int s, void *Cp, void *keys, int64_t keys_stride, void *cache,
                             int64_t cache_stride, hipStream_t stream);

// Stride-aware masked attention: O [B, T, H, r] from queries qt [B, T, H, r],
// QR [B, T, H, dR], the compressed keys [B, keys_stride] (ceil(T/s) rows of
// r + dR), and the diagonal terms C' [B, T, r], KR [B, T, dR].
hipError_t launch_prefill_attention(int dtype, int B, int T, int H, int r, int dR, int s,
                                    float scale, const void *qt, const void *QR, const void *keys,
                                    int64_t keys_stride, const void *Cp, const void *KR, void *O,
                                    hipStream_t stream);

bool prefill_attention_supported(int dtype, int H, int r, int dR);

}  // namespace mtla
