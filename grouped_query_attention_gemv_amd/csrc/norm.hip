// Pre-norm of the block's residual stream (page "Llama 3.1 8B .
// Grouped-query attention", code section: the layer feeds attention_norm(x)
// to the attention and adds its update to x; the norm is RMSNorm over the
// model dimension with eps = norm_eps, 1e-5 in the catalogue entry).  The
// pages construct the norm but do not print its body; this is the standard
// root-mean-square normalisation with a per-feature gain:
//   xn[k] = x[k] / sqrt(mean_k x[k]^2 + eps) * g[k]
// computed in fp32 and rounded once to bf16, the dtype the projections read.
#include <math.h>

#include "kernels.h"

namespace gqa {

// One workgroup per row of 4096: 16 elements per thread.
__global__ void __launch_bounds__(256) rmsnorm_kernel(const uint16_t* __restrict__ x,
                                                       const uint16_t* __restrict__ g, float eps,
                                                       uint16_t* __restrict__ xn,
                                                       float* __restrict__ h) {
  __shared__ float part[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const size_t row = (size_t)blockIdx.x * D;
  float v[16];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const u32x4 u = ld_u32x4(x + row + half * (D / 2) + tid * 8);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[half * 8 + 2 * q] = bf16_bits_to_f32(u[q] & 0xffffu);
      v[half * 8 + 2 * q + 1] = bf16_bits_to_f32(u[q] >> 16);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) ss += v[i] * v[i];
  ss = wave_sum(ss);
  if (lane == 0) part[w] = ss;
  __syncthreads();
  ss = (part[0] + part[1]) + (part[2] + part[3]);
  const float r = 1.f / sqrtf(ss * (1.f / D) + eps);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const size_t off = half * (D / 2) + tid * 8;
    const u32x4 gu = ld_u32x4(g + off);
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float a = v[half * 8 + 2 * q] * r * bf16_bits_to_f32(gu[q] & 0xffffu);
      const float b = v[half * 8 + 2 * q + 1] * r * bf16_bits_to_f32(gu[q] >> 16);
      o[q] = pack_bf16x2(a, b);
    }
    *reinterpret_cast<u32x4*>(xn + row + off) = o;
    if (h) {
      float* hr = h + row + off;
      *reinterpret_cast<f32x4*>(hr) =
          f32x4{v[half * 8], v[half * 8 + 1], v[half * 8 + 2], v[half * 8 + 3]};
      *reinterpret_cast<f32x4*>(hr + 4) =
          f32x4{v[half * 8 + 4], v[half * 8 + 5], v[half * 8 + 6], v[half * 8 + 7]};
    }
  }
}

hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* g, float eps, int M, uint16_t* xn,
                          float* h, hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(M), dim3(256), 0, s, x, g, eps, xn, h);
  return hipGetLastError();
}

}  // namespace gqa
