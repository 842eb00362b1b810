// Vocabulary projection (page "Llama 3.1 8B . Vocabulary projection"):
// L = z W_out with the weight stored [out, in] = [V][4096] and z the final
// norm of the last hidden state, "cast to float32 before it is returned":
// the projection's output is taken in the model's bf16 and handed back as
// fp32, so each logit is the bf16 rounding (nearest even) of its fp32 dot
// product.  The norm in front (the page's code: self.norm, an RMSNorm with
// norm_eps) is optional here and read as in the layer pre-norm.
//
// A bandwidth GEMV over 1.05 GB of weights at V = 128,256: each wave takes
// pairs of weight rows in a grid-strided loop, with the next pair's 16 loads
// issued before the current pair's products (two pairs in flight per wave);
// the B <= 8 token vectors are staged (and normalised) once per workgroup.
#include <algorithm>

#include "gemv.h"
#include "kernels.h"

namespace gqa {

template <int NB>
__global__ void __launch_bounds__(256) vocab_gemv_kernel(VocabParams p, int b0) {
  __shared__ uint32_t xs[NB * (D / 2)];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int pairs = (p.V + 1) / 2;
  const int stride = gridDim.x * 4;
  int pr = blockIdx.x * 4 + wave;
  auto rows = [&](int q, const uint16_t** w0, const uint16_t** w1) {
    const int r0 = 2 * q, r1 = min(2 * q + 1, p.V - 1);   // odd V: the last pair repeats a row
    *w0 = p.w + (size_t)r0 * D;
    *w1 = p.w + (size_t)r1 * D;
  };
  // z (and the norm gain) go out ahead of the first weight pair, so that
  // waiting for them leaves that pair's 16 loads in flight
  stage_rows_async<NB, 4>(xs, p.z + (size_t)b0 * D);
  uint32_t gp[(D / 2) / 256];
  if (p.norm_w) load_norm_gain<4>(p.norm_w, gp);
  u32x4 wa[2][8], wb[2][8];
  const uint16_t *w0, *w1;
  if (pr < pairs) {
    rows(pr, &w0, &w1);
    load_rows2(w0, w1, lane, wa[0], wb[0]);
    wait_loads_except<16>();
  } else {
    wait_loads_except<0>();
  }
  lds_barrier();
  if (p.norm_w) norm_rows<NB>(xs, gp, p.norm_eps);

  auto finish = [&](int q, const float (&acc)[2][NB]) {
    float v0 = 0.f, v1 = 0.f;
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const float s0 = wave_sum(acc[0][t]);
      const float s1 = wave_sum(acc[1][t]);
      if (lane == t) { v0 = s0; v1 = s1; }
    }
    if (lane < NB) {
      float* o = p.logits + (size_t)(b0 + lane) * p.V + 2 * q;
      o[0] = bf16_bits_to_f32(f32_to_bf16_bits(v0));
      if (2 * q + 1 < p.V) o[1] = bf16_bits_to_f32(f32_to_bf16_bits(v1));
    }
  };
  // two pairs in flight: issue pair pr + stride, then compute pair pr
  for (; pr < pairs; pr += 2 * stride) {
    const int q1 = pr + stride;
    if (q1 < pairs) {
      rows(q1, &w0, &w1);
      load_rows2(w0, w1, lane, wa[1], wb[1]);
    }
    float acc[2][NB];
    gemv_rows2<NB, 1>(wa[0], wb[0], xs, lane, acc);
    finish(pr, acc);
    if (q1 >= pairs) break;
    const int q2 = q1 + stride;
    if (q2 < pairs) {
      rows(q2, &w0, &w1);
      load_rows2(w0, w1, lane, wa[0], wb[0]);
    }
    gemv_rows2<NB, 1>(wa[1], wb[1], xs, lane, acc);
    finish(q1, acc);
  }
}

hipError_t launch_vocab_gemv(const VocabParams& p, hipStream_t s) {
  const int pairs = (p.V + 1) / 2;
  const int grid = std::min(2048, (pairs + 3) / 4);
  for (int b0 = 0; b0 < p.B; b0 += kGemvMaxNB) {
    const int nb = std::min(kGemvMaxNB, p.B - b0);
    switch (nb) {
      case 1: hipLaunchKernelGGL(vocab_gemv_kernel<1>, dim3(grid), dim3(256), 0, s, p, b0); break;
      case 2: hipLaunchKernelGGL(vocab_gemv_kernel<2>, dim3(grid), dim3(256), 0, s, p, b0); break;
      case 3: hipLaunchKernelGGL(vocab_gemv_kernel<3>, dim3(grid), dim3(256), 0, s, p, b0); break;
      case 4: hipLaunchKernelGGL(vocab_gemv_kernel<4>, dim3(grid), dim3(256), 0, s, p, b0); break;
      case 5: hipLaunchKernelGGL(vocab_gemv_kernel<5>, dim3(grid), dim3(256), 0, s, p, b0); break;
      case 6: hipLaunchKernelGGL(vocab_gemv_kernel<6>, dim3(grid), dim3(256), 0, s, p, b0); break;
      case 7: hipLaunchKernelGGL(vocab_gemv_kernel<7>, dim3(grid), dim3(256), 0, s, p, b0); break;
      default: hipLaunchKernelGGL(vocab_gemv_kernel<8>, dim3(grid), dim3(256), 0, s, p, b0); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gqa
