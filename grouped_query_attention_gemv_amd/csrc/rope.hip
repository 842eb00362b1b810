// RoPE table: rope[p][i] = (cos, sin)(p * f_i) for the 64 pairs of a head
// (the table R [positions, 64 pairs] on page "Llama 3.1 8B . Grouped-query
// attention"; pairs rotated as in its evidence "rope").
#include "kernels.h"

namespace gqa {

// Per-pair frequency, fp64.  Unscaled: theta^(-2i/128).  Scaled (Llama 3.1
// long-context rule): wavelengths below 8192/4 keep f, above 8192 take f/8,
// and in between f is blended linearly in 8192/wavelength.
__device__ double rope_freq(int i, double theta, int scaled) {
  double f = pow(theta, -2.0 * (double)i / (double)HD);
  if (!scaled) return f;
  const double kOldContext = 8192.0, kScale = 8.0, kLow = 1.0, kHigh = 4.0;
  double wavelen = 2.0 * M_PI / f;
  if (wavelen < kOldContext / kHigh) return f;
  if (wavelen > kOldContext / kLow) return f / kScale;
  double t = (kOldContext / wavelen - kLow) / (kHigh - kLow);
  return (1.0 - t) * f / kScale + t * f;
}

__global__ void __launch_bounds__(256) rope_table_kernel(float2* __restrict__ rope, int T_max,
                                                         double theta, int scaled) {
  long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)T_max * PAIRS) return;
  int p = (int)(idx / PAIRS);
  int i = (int)(idx % PAIRS);
  double ang = (double)p * rope_freq(i, theta, scaled);
  double s, c;
  sincos(ang, &s, &c);
  rope[idx] = make_float2((float)c, (float)s);
}

hipError_t launch_rope_table(float* rope, int T_max, double theta, int scaled, hipStream_t s) {
  long n = (long)T_max * PAIRS;
  int blocks = (int)((n + 255) / 256);
  hipLaunchKernelGGL(rope_table_kernel, dim3(blocks), dim3(256), 0, s,
                     reinterpret_cast<float2*>(rope), T_max, theta, scaled);
  return hipGetLastError();
}

}  // namespace gqa
