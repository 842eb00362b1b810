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

// Start copying NB rows of 4096 bf16 (one part) from global memory into LDS
// with direct-to-LDS loads (16 bytes a lane, 1 KiB a wave instruction),
// spread over the W waves of the workgroup; row t starts at word t * PITCH.
// Issued before a wave's weight loads, the copy is complete once no more
// than those weight loads remain in flight (wait_loads_except), instead of
// queueing behind them.
template <int NB, int W, int PITCH = D / 2>
__device__ __forceinline__ void stage_rows_async(uint32_t* xs, const uint16_t* __restrict__ src) {
  constexpr int kPieces = NB * (D * 2 / 1024);      // 8 KiB a row
  static_assert(kPieces % W == 0, "every wave copies the same number of pieces");
  static_assert(PITCH % 4 == 0, "rows start on 16-byte boundaries");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < kPieces / W; ++j) {
    const int i = wave + W * j;
    const int t = i >> 3, piece = i & 7;
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(src + (size_t)i * 512 + lane * 8),
                                     (lds_void*)(reinterpret_cast<char*>(xs + t * PITCH) + piece * 1024),
                                     16, 0, 0);
  }
  asm volatile("" ::: "memory");
}

// Workgroup barrier for LDS data only: this wave's LDS accesses complete,
// then s_barrier.  Unlike __syncthreads() it does not wait for the wave's
// outstanding global loads (the weight stream keeps flowing); data that
// direct-to-LDS loads wrote must be waited for first (wait_loads_except).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until at most N memory loads of this wave are still in flight.  The
// builtin (not inline asm) lets the compiler's own counter bookkeeping see
// the wait, so it inserts no coarser one where earlier loads are used.
// Encoding of the gfx9 s_waitcnt immediate: vmcnt bits [3:0] and [15:14],
// expcnt [6:4] and lgkmcnt [11:8] left at their "no wait" maxima.
template <int N>
__device__ __forceinline__ void wait_loads_except() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit count");
  __builtin_amdgcn_s_waitcnt(((N >> 4) << 14) | (N & 15) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}


// Layer pre-norm of the NB staged rows, in place: x -> bf16(x * r * g) with
// r = 1 / sqrt(mean(x^2) + eps) per row (page "Llama 3.1 8B . Grouped-query
// attention", code section: the block receives attention_norm(x); the norm
// is read as the standard RMSNorm with a per-feature gain).  With W waves,
// thread i owns bf16 pairs i + 64W*j of every row; the row sums combine the
// waves pairwise in a fixed order.  The gain pairs gp come from
// load_norm_gain, issued before the weight stream so that waiting for them
// does not wait for the weights.
template <int W>
__device__ __forceinline__ void load_norm_gain(const uint16_t* __restrict__ g, uint32_t (&gp)[(D / 2) / (64 * W)]) {
  constexpr int NT = 64 * W, J = (D / 2) / NT;
#pragma unroll
  for (int j = 0; j < J; ++j) gp[j] = reinterpret_cast<const uint32_t*>(g)[threadIdx.x + NT * j];
}

template <int NB, int W = 4>
__device__ __forceinline__ void norm_rows(uint32_t* xs, const uint32_t (&gp)[(D / 2) / (64 * W)], float eps) {
  constexpr int NT = 64 * W, J = (D / 2) / NT;
  __shared__ float red[W * NB];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  float ss[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    ss[t] = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const uint32_t u = xs[t * (D / 2) + tid + NT * j];
      const float a = bf16_bits_to_f32(u & 0xffffu), b = bf16_bits_to_f32(u >> 16);
      ss[t] += a * a + b * b;
    }
    ss[t] = wave_sum(ss[t]);
    if (lane == 0) red[w * NB + t] = ss[t];
  }
  lds_barrier();
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    float v[W];
#pragma unroll
    for (int ww = 0; ww < W; ++ww) v[ww] = red[ww * NB + t];
#pragma unroll
    for (int step = 1; step < W; step *= 2)
#pragma unroll
      for (int ww = 0; ww + step < W; ww += 2 * step) v[ww] += v[ww + step];
    const float r = 1.f / sqrtf(v[0] * (1.f / D) + eps);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      uint32_t* q = xs + t * (D / 2) + tid + NT * j;
      const uint32_t u = *q;
      *q = pack_bf16x2(bf16_bits_to_f32(u & 0xffffu) * r * bf16_bits_to_f32(gp[j] & 0xffffu),
                       bf16_bits_to_f32(u >> 16) * r * bf16_bits_to_f32(gp[j] >> 16));
    }
  }
  lds_barrier();
}

}  // namespace gqa
