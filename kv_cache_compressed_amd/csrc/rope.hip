// Decoupled-RoPE inputs on gfx950: Q^R and K^R of every frame from its
// input x and absolute position ([Notes] decoupled RoPE with temporal
// compression: the RoPE-carrying query and key parts).
//
// [Notes] = "Multi-head Temporal Latent Attention" paper notes (zhaoyang97
// Paper-Notes), key designs / decoupled RoPE.  The rotary form is the
// standard one (the pages do not spell it out): adjacent pairs (2k, 2k+1) of
// a width-w vector turn by pos * base^(-2k/w).
//
// One product pass gives [W_QR x | W_KR x] in fp32, then one thread per
// pair rotates it.  The angle pos * theta_k reaches tens of thousands of
// radians at long contexts, so it is formed and reduced to [-pi, pi] in
// fp64 before the fp32 sine and cosine.

#include <math.h>

#include "common.h"
#include "kernels.h"

namespace mtla {

namespace {

template <typename T>
__global__ __launch_bounds__(256) void rope_rotate_kernel(const float *G, const int32_t *pos,
                                                          int M, int HR, int DR, double lbase,
                                                          T *QR, T *KR) {
  const int N = HR + DR, NP = N / 2;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)M * NP) return;
  const int m = (int)(i / NP), n = 2 * (int)(i % NP);
  const bool q = n < HR;
  const int k = (q ? n % DR : n - HR) / 2;
  const double theta = exp2(-2.0 * k / DR * lbase);
  double ang = (double)pos[m] * theta;
  ang -= 6.283185307179586 * rint(ang * 0.15915494309189535);
  float sn, cs;
  sincosf((float)ang, &sn, &cs);
  const float a = G[(size_t)m * N + n], b = G[(size_t)m * N + n + 1];
  T *dst = q ? QR + (size_t)m * HR + n : KR + (size_t)m * DR + (n - HR);
  dst[0] = from_f32<T>(a * cs - b * sn);
  dst[1] = from_f32<T>(a * sn + b * cs);
}

}  // namespace

hipError_t launch_rope_inputs(int dtype, const void *X, int M, int d, const void *W_QR, int HR,
                              const void *W_KR, int DR, const int32_t *pos, float base, float *G,
                              void *QR, void *KR, hipStream_t stream) {
  const int N = HR + DR;
  hipError_t e = launch_gemm_f32_2(dtype, X, d, W_QR, W_KR, HR, d, M, N, d, G, N, stream);
  if (e != hipSuccess) return e;
  const int64_t pairs = (int64_t)M * (N / 2);
  const double lbase = log2((double)base);
  const dim3 grid((unsigned)((pairs + 255) / 256));
  if (dtype == 1)
    hipLaunchKernelGGL(rope_rotate_kernel<bf16>, grid, dim3(256), 0, stream, G, pos, M, HR, DR,
                       lbase, (bf16 *)QR, (bf16 *)KR);
  else
    hipLaunchKernelGGL(rope_rotate_kernel<float>, grid, dim3(256), 0, stream, G, pos, M, HR, DR,
                       lbase, (float *)QR, (float *)KR);
  return hipGetLastError();
}

}  // namespace mtla
