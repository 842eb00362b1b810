// Vocabulary projection (page "Llama 3.1 8B . Vocabulary projection"):
// L = z W_out with the weight stored [out, in] = [V][4096] and z the final
// norm of the last hidden state.  The page computes the projection in the
// model's bf16 and converts its result to fp32 on return, so each logit is
// the bf16 rounding (nearest even) of its fp32 dot product.  The norm in
// front (the page's code: self.norm, an RMSNorm with norm_eps) is optional
// here and read as in the layer pre-norm.
//
// Up to 5 sequences: a bandwidth GEMV over 1.05 GB of weights at V =
// 128,256: each wave takes pairs of weight rows in a grid-strided loop, with
// the next pair's 16 loads issued before the current pair's products (two
// pairs in flight per wave); the token vectors are staged (and normalised)
// once per workgroup.  From 6: the matrix-core kernel further down, one
// weight pass per 64 sequences (at V = 128,256: the GEMV takes 157, 185 and
// 205 us at 1, 4 and 5 sequences and 224 us at 6, the matrix-core kernel
// 219 us at 6 to 9 and 250 us at 64).
#include <algorithm>
#include <type_traits>

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

// ---------------------------------------------------------------------------
// From 6 tokens: the matrix-core projection
// ---------------------------------------------------------------------------
//
// C^T[rows x tokens] = W[rows x 4096] . Z^T[4096 x tokens] on
// v_mfma_f32_16x16x32_bf16, streaming the weights once per 64 tokens (the
// GEMV above streams them once per 8, and its vector work grows with the
// token count).  The vocabulary is long enough to fill the chip without
// splitting K:
//  - workgroup fb owns 128 vocabulary rows (its 4 waves two 16-row A tiles
//    each) and the whole K; the last block's rows past V are clamped loads
//    whose results are not stored;
//  - a launch covers NT column tiles of 16 tokens (1 to 4), the fewest that
//    hold its tokens, so that few tokens stage and multiply no more than
//    they need;
//  - K advances in chunks of 128.  The tokens' chunk is copied into LDS
//    (global_load_lds, 4 KiB per column tile, XOR-swizzled rows) and read by
//    all 4 waves as the B operand; each wave's weight rows come from HBM
//    straight into registers (its A operand; plain loads, which streamed
//    this 16-row pattern about 10% faster than non-temporal ones).  Both
//    run three chunks ahead of the matrix work through a 4-slot ring;
//  - the epilogue rounds each logit to bf16 as the GEMV does.
// Z is the caller's h, or its norm written beforehand by the norm kernel.
constexpr int kVcCols = 64;        // tokens per launch
constexpr int kVcFeat = 128;       // vocabulary rows per workgroup
constexpr int kVcKc = 128;         // K per chunk
constexpr int kVcRing = 4;         // chunk slots: loaded three ahead
constexpr int kVcChunks = D / kVcKc;

template <int NT>
__global__ void __launch_bounds__(256) vocab_mfma_kernel(VocabParams p, const uint16_t* __restrict__ z,
                                                         int c_base) {
  static_assert(NT >= 1 && NT <= kVcCols / 16, "1 to 4 column tiles");
  __shared__ __attribute__((aligned(16))) uint16_t sx[kVcRing][16 * NT * kVcKc];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int fb = blockIdx.x;
  const int ncols = min(16 * NT, p.B - c_base);

  // A operand: weight row of tile ft, k offset (lane >> 4) * 8 in each step
  const uint16_t* wrow[2];
#pragma unroll
  for (int ft = 0; ft < 2; ++ft) {
    const int f = fb * kVcFeat + 32 * w + 16 * ft + (lane & 15);
    wrow[ft] = p.w + (size_t)min(f, p.V - 1) * D + (lane >> 4) * 8;
  }
  // token copies: instruction j of this wave fills rows (NT w + j) * 4 .. + 3
  // of the chunk (256 bytes each); lane i writes row +i/16, 16-byte slot
  // i % 16, which holds logical slot (i % 16) ^ (row & 7).  Rows past the
  // last token copy the last token (their results are not stored).
  const uint16_t* xsrc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int row = (NT * w + j) * 4 + (lane >> 4);
    const int lchunk = (lane & 15) ^ (row & 7);
    xsrc[j] = z + (size_t)(c_base + min(row, ncols - 1)) * D + lchunk * 8;
  }

  u32x4 wb[kVcRing][2][4];                      // [slot][tile][k-step]
  auto load_chunk = [&](int chunk, int slot) {
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
      for (int s = 0; s < 4; ++s) wb[slot][ft][s] = ld_u32x4(wrow[ft] + chunk * kVcKc + s * 32);
#pragma unroll
    for (int j = 0; j < NT; ++j)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(xsrc[j] + chunk * kVcKc),
                                       (lds_void*)(&sx[slot][(NT * w + j) * 4 * kVcKc]), 16, 0, 0);
    asm volatile("" ::: "memory");              // chunks leave in order
  };

  f32x4 acc[2][NT];
#pragma unroll
  for (int ft = 0; ft < 2; ++ft)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[ft][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Chunk c has landed once no more than the loads of the chunks issued
  // after it (8 weight loads and NT copies a chunk) remain in flight.
  constexpr int kPerChunk = 8 + NT;
  static_assert(kVcChunks % kVcRing == 0, "the ring slot of a chunk is known at compile time");
  // one chunk: slot u, LATER chunks already issued after it
  auto step = [&](auto u_tag, auto later_tag, int c) {
    constexpr int u = decltype(u_tag)::value;
    constexpr int LATER = decltype(later_tag)::value;
    wait_loads_except<LATER * kPerChunk>();
    // every wave's copies of chunk c have landed, and every wave is done
    // with the slot refilled below (read in the previous chunk)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (LATER == kVcRing - 2) load_chunk(c + kVcRing - 1, (u + kVcRing - 1) % kVcRing);
    u32x4 xb[4][NT];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int row = 16 * t + (lane & 15);
        const int off = row * kVcKc + (((4 * s + (lane >> 4)) ^ (row & 7)) << 3);
        xb[s][t] = *reinterpret_cast<const u32x4*>(&sx[u][off]);
      }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int ft = 0; ft < 2; ++ft) acc[ft][t] = mfma_bf16(wb[u][ft][s], xb[s][t], acc[ft][t]);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
#pragma unroll
  for (int c = 0; c < kVcRing - 1; ++c) load_chunk(c, c);
  // all but the last four chunks load the chunk three ahead
  for (int c0 = 0; c0 < kVcChunks - kVcRing; c0 += kVcRing) {
    step(I0{}, I2{}, c0);
    step(I1{}, I2{}, c0 + 1);
    step(I2{}, I2{}, c0 + 2);
    step(I3{}, I2{}, c0 + 3);
  }
  constexpr int cl = kVcChunks - kVcRing;
  step(I0{}, I2{}, cl);                          // loads the last chunk
  step(I1{}, I2{}, cl + 1);                      // (kVcRing - 1 ahead: none left after)
  step(I2{}, I1{}, cl + 2);
  step(I3{}, I0{}, cl + 3);

  // lane holds rows 32w + 16ft + 4(lane >> 4) + e of the block for token
  // 16t + (lane & 15)
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int col = 16 * t + (lane & 15);
    if (col >= ncols) continue;
    float* lrow = p.logits + (size_t)(c_base + col) * p.V;
#pragma unroll
    for (int ft = 0; ft < 2; ++ft) {
      const int f0 = fb * kVcFeat + 32 * w + 16 * ft + 4 * (lane >> 4);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (f0 + e < p.V) lrow[f0 + e] = bf16_bits_to_f32(f32_to_bf16_bits(acc[ft][t][e]));
    }
  }
}

hipError_t launch_vocab_mfma(const VocabParams& p, const uint16_t* z, hipStream_t s) {
  const int nfb = (p.V + kVcFeat - 1) / kVcFeat;
  for (int c = 0; c < p.B; c += kVcCols) {
    switch ((std::min(kVcCols, p.B - c) + 15) / 16) {
      case 1: hipLaunchKernelGGL(vocab_mfma_kernel<1>, dim3(nfb), dim3(256), 0, s, p, z, c); break;
      case 2: hipLaunchKernelGGL(vocab_mfma_kernel<2>, dim3(nfb), dim3(256), 0, s, p, z, c); break;
      case 3: hipLaunchKernelGGL(vocab_mfma_kernel<3>, dim3(nfb), dim3(256), 0, s, p, z, c); break;
      default: hipLaunchKernelGGL(vocab_mfma_kernel<4>, dim3(nfb), dim3(256), 0, s, p, z, c); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
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
