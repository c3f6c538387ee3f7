// Chunked merge-append on gfx950: L consecutive frames per sequence folded
// into the compressed cache in one launch.
//
// [Notes] = "Multi-head Temporal Latent Attention" paper notes (zhaoyang97
// Paper-Notes): key designs / hyper-network temporal merging; [Fig2] =
// sciencestack.ai page, Figure 2 (a) incremental inference.
//
// The incremental merge of [Fig2] (a) folds one frame into slot floor(t/s):
// the slot is opened by the first frame of its group and accumulated by the
// others.  Applied to frames t0 .. t0+n-1 in order, every slot the chunk
// touches ends as (its stored partial state, if the chunk enters the group
// after the group's first frame, else 0) plus the gated latents of its frames
// in the chunk, added in frame order -- which is what one thread per
// (slot, channel) computes here, with the running sums of the intermediate
// frames as a by-product.

#include "common.h"
#include "kernels.h"

namespace mtla {

namespace {

struct ChunkArgs {
  const float *cg;        // [B, L, 2R] fp32: c = W_dkv x, then W_gate x
  const void *b_hc;       // [R]
  const float *table;     // [rows, R] fp32: Linear(pe_j)
  const void *KR;         // [B, L, DR]
  const int32_t *pos0;    // [B] first frame of each sequence's chunk
  const int32_t *lens;    // [B] frames per sequence, clamped to [0, L]; null: L
  void *Cp;               // [B, L, R] or null
  char *cache;            // [B] x bstride_bytes: rows of R + DR values
  int64_t bstride_bytes;
  int L, R, DR, s, nJ, jlim;
};

// One thread per (sequence b = blockIdx.y, slot jj of the chunk, channel of
// a cache row).  Channels < R carry the latent sum, the others copy the
// rotary key of the slot's newest frame.
template <typename T>
__global__ __launch_bounds__(256) void chunk_merge_kernel(ChunkArgs a) {
  const int b = blockIdx.y, RK = a.R + a.DR;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= a.nJ * RK) return;
  const int jj = idx / RK, ch = idx - jj * RK;
  const int t0 = a.pos0[b];
  const int n = a.lens ? min(max(a.lens[b], 0), a.L) : a.L;
  if (t0 < 0 || n == 0) return;
  const int j = t0 / a.s + jj;
  if (j > (t0 + n - 1) / a.s || j >= a.jlim) return;
  const int f0 = max(t0, a.s * j), f1 = min(t0 + n - 1, a.s * j + a.s - 1);
  T *row = (T *)(a.cache + (size_t)b * a.bstride_bytes) + (size_t)j * RK;
  const int64_t base = (int64_t)b * a.L - t0;   // row of frame f in [B, L]: base + f
  if (ch < a.R) {
    float acc = f0 > a.s * j ? to_f32(row[ch]) : 0.0f;   // enters a live partial slot
    const float bb = to_f32(((const T *)a.b_hc)[ch]), pj = a.table[(size_t)j * a.R + ch];
    for (int f = f0; f <= f1; ++f) {
      const float *r = a.cg + (base + f) * 2 * a.R;
      acc += sigmoidf((r[a.R + ch] + bb) * pj) * r[ch];
      if (a.Cp) ((T *)a.Cp)[(base + f) * a.R + ch] = from_f32<T>(acc);
    }
    row[ch] = from_f32<T>(acc);
  } else {
    row[ch] = ((const T *)a.KR)[(base + f1) * a.DR + (ch - a.R)];
  }
}

}  // namespace

int chunk_slots(int L, int s) { return L < 1 ? 0 : (L - 1) / s + 2; }

hipError_t launch_chunk_merge(int dtype, int B, int L, int r, int dR, int s, const int32_t *pos0,
                              const int32_t *lens, const float *cg, const void *b_hc,
                              const float *table, int jlim, const void *KR, void *Cp, void *cache,
                              int64_t batch_stride, hipStream_t stream) {
  const int esz = dtype == 1 ? 2 : 4, nJ = chunk_slots(L, s);
  ChunkArgs a{cg, b_hc, table, KR, pos0, lens, Cp, (char *)cache, batch_stride * esz,
              L, r, dR, s, nJ, jlim};
  const int64_t work = (int64_t)nJ * (r + dR);
  dim3 grid((unsigned)((work + 255) / 256), B);
  if (dtype == 1)
    hipLaunchKernelGGL(chunk_merge_kernel<bf16>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(chunk_merge_kernel<float>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mtla
