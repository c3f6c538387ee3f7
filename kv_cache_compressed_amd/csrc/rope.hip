// Decoupled-RoPE inputs on gfx950: Q^R and K^R of every frame from its
// input x and absolute position ([Notes] decoupled RoPE with temporal
// compression: the RoPE-carrying query and key parts).
//
// [Notes] = "Multi-head Temporal Latent Attention" paper notes (zhaoyang97
// Paper-Notes), key designs / decoupled RoPE.  The rotary form is the
// standard one (the pages do not spell it out): adjacent pairs (2k, 2k+1) of
// a width-w vector turn by pos * base^(-2k/w).
//
// One product pass gives [W_QR x | W_KR x] in fp32, then the rotation: one
// thread per row and four columns of the head width, across all heads.  The angle pos * theta_k reaches tens of thousands of
// radians at long contexts, so it is formed and reduced to [-pi, pi] in
// fp64 before the fp32 sine and cosine.

#include <math.h>

#include "common.h"
#include "kernels.h"

namespace mtla {

namespace {

template <typename T>
__global__ __launch_bounds__(256) void rope_rotate_kernel(const float *G, const int32_t *pos,
                                                          int M, int H, int DR, double lbase,
                                                          T *QR, T *KR) {
  // Every head of a row turns by the same DR/2 angles, so a thread owns
  // columns 4 q .. 4 q + 3 of one row in every head (the H query heads, then
  // the key head, which follows them in G): two angles, then H + 1 16-byte
  // loads and 4-value stores.
  const int QD = DR / 4, HR = H * DR, N = HR + DR;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)M * QD) return;
  const int m = (int)(i / QD), q = (int)(i % QD);
  float sn[2], cs[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int k = 2 * q + h;
    const double theta = exp2(-2.0 * k / DR * lbase);
    double ang = (double)pos[m] * theta;
    ang -= 6.283185307179586 * rint(ang * 0.15915494309189535);
    sincosf((float)ang, &sn[h], &cs[h]);
  }
  const float *g = G + (size_t)m * N + 4 * q;
#pragma unroll 3
  for (int hd = 0; hd <= H; ++hd) {
    const f32x4 a = *(const f32x4 *)(g + hd * DR);
    f32x4 out;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      out[2 * h] = a[2 * h] * cs[h] - a[2 * h + 1] * sn[h];
      out[2 * h + 1] = a[2 * h] * sn[h] + a[2 * h + 1] * cs[h];
    }
    store4f(hd < H ? QR + (size_t)m * HR + hd * DR + 4 * q : KR + (size_t)m * DR + 4 * q, out);
  }
}

}  // namespace

hipError_t launch_rope_inputs(int dtype, const void *X, int M, int d, const void *W_QR, int HR,
                              const void *W_KR, int DR, const int32_t *pos, float base, float *G,
                              void *QR, void *KR, hipStream_t stream) {
  const int N = HR + DR;
  if (DR % 4 != 0 || HR % DR != 0) return hipErrorInvalidValue;
  hipError_t e = launch_gemm_f32_2(dtype, X, d, W_QR, W_KR, HR, d, M, N, d, G, N, stream);
  if (e != hipSuccess) return e;
  const int64_t threads = (int64_t)M * (DR / 4);
  const double lbase = log2((double)base);
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (dtype == 1)
    hipLaunchKernelGGL(rope_rotate_kernel<bf16>, grid, dim3(256), 0, stream, G, pos, M, HR / DR,
                       DR, lbase, (bf16 *)QR, (bf16 *)KR);
  else
    hipLaunchKernelGGL(rope_rotate_kernel<float>, grid, dim3(256), 0, stream, G, pos, M, HR / DR,
                       DR, lbase, (float *)QR, (float *)KR);
  return hipGetLastError();
}

}  // namespace mtla
