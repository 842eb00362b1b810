// Device building blocks of the bandwidth-bound GEMVs: the decode
// projections and the vocabulary projection.
#pragma once

#include "common.h"

namespace gqa {

// ---------------------------------------------------------------------------
// Bandwidth GEMV core
// ---------------------------------------------------------------------------
//
// One wave computes two adjacent weight rows for NB token vectors.  Lane l
// reads 16-byte pieces (c*64 + l)*8 .. +8 of each 4096-element row, c < 8, so
// a wave streams 16 KiB with every load coalesced and all 16 loads in flight
// before the first product.  The token vectors sit in LDS as NPARTS bf16 parts
// (the vector is the sum of its parts); products use the packed bf16 dot
// instruction with fp32 accumulation.
template <int NB, int NPARTS>
__device__ __forceinline__ void gemv_rows2(const u32x4 (&a)[8], const u32x4 (&b)[8],
                                           const uint32_t* xs, int lane, float (&acc)[2][NB]) {
#pragma unroll
  for (int t = 0; t < NB; ++t) acc[0][t] = acc[1][t] = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int e2 = (c * 64 + lane) * 4;
#pragma unroll
    for (int part = 0; part < NPARTS; ++part) {
#pragma unroll
      for (int t = 0; t < NB; ++t) {
        const u32x4 xv = *reinterpret_cast<const u32x4*>(xs + (part * NB + t) * (D / 2) + e2);
        float s0 = acc[0][t], s1 = acc[1][t];
        s0 = dot2_bf16(a[c].x, xv.x, s0);
        s1 = dot2_bf16(b[c].x, xv.x, s1);
        s0 = dot2_bf16(a[c].y, xv.y, s0);
        s1 = dot2_bf16(b[c].y, xv.y, s1);
        s0 = dot2_bf16(a[c].z, xv.z, s0);
        s1 = dot2_bf16(b[c].z, xv.z, s1);
        s0 = dot2_bf16(a[c].w, xv.w, s0);
        s1 = dot2_bf16(b[c].w, xv.w, s1);
        acc[0][t] = s0;
        acc[1][t] = s1;
      }
    }
  }
}

// Issue the 16 loads of two weight rows (lane l: pieces (c*64 + l)*8, c < 8).
__device__ __forceinline__ void load_rows2(const uint16_t* __restrict__ w0,
                                           const uint16_t* __restrict__ w1, int lane,
                                           u32x4 (&a)[8], u32x4 (&b)[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int e = (c * 64 + lane) * 8;
    a[c] = ld_nt_u32x4(w0 + e);
    b[c] = ld_nt_u32x4(w1 + e);
  }
}

// Copy NB rows of 4096 bf16 (one part) from global into LDS.
template <int NB>
__device__ __forceinline__ void stage_rows(uint32_t* xs, const uint16_t* __restrict__ src) {
  for (int i = threadIdx.x; i < NB * (D / 8); i += blockDim.x) {
    const int t = i / (D / 8), u = i % (D / 8);
    *reinterpret_cast<u32x4*>(xs + t * (D / 2) + u * 4) = ld_u32x4(src + (size_t)t * D + u * 8);
  }
}

// Layer pre-norm of the NB staged rows, in place: x -> bf16(x * r * g) with
// r = 1 / sqrt(mean(x^2) + eps) per row (page "Llama 3.1 8B . Grouped-query
// attention", code section: the block receives attention_norm(x); the norm
// is read as the standard RMSNorm with a per-feature gain).  Thread i owns
// bf16 pairs i + 256*j, j < 8, of every row; the row sums combine the four
// waves in a fixed order.
template <int NB>
__device__ __forceinline__ void norm_rows(uint32_t* xs, const uint16_t* __restrict__ g, float eps) {
  __shared__ float red[4 * NB];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  float ss[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    ss[t] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t u = xs[t * (D / 2) + tid + 256 * j];
      const float a = bf16_bits_to_f32(u & 0xffffu), b = bf16_bits_to_f32(u >> 16);
      ss[t] += a * a + b * b;
    }
    ss[t] = wave_sum(ss[t]);
    if (lane == 0) red[w * NB + t] = ss[t];
  }
  uint32_t gp[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) gp[j] = reinterpret_cast<const uint32_t*>(g)[tid + 256 * j];
  __syncthreads();
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    const float tot = (red[t] + red[NB + t]) + (red[2 * NB + t] + red[3 * NB + t]);
    const float r = 1.f / sqrtf(tot * (1.f / D) + eps);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t* q = xs + t * (D / 2) + tid + 256 * j;
      const uint32_t u = *q;
      *q = pack_bf16x2(bf16_bits_to_f32(u & 0xffffu) * r * bf16_bits_to_f32(gp[j] & 0xffffu),
                       bf16_bits_to_f32(u >> 16) * r * bf16_bits_to_f32(gp[j] >> 16));
    }
  }
  __syncthreads();
}

}  // namespace gqa
