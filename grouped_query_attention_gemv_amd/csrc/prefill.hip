// Prefill path of the attention block: T new tokens per sequence at
// positions start_pos .. start_pos+T-1, after start_pos cached rows, with the
// causal mask of the page "Llama 3.1 8B . Grouped-query attention" (evidence
// "scores" and the mask listing of its code section: new token i sits at
// position start_pos + i and sees every key j <= start_pos + i).
// start_pos = 0 is the plain prefill; start_pos > 0 continues a prefix
// (chunked prefill).
//
//   prefill_prep_kernel  wo bf16 -> fp16 copy in the workspace; cached K/V
//                        rows 0 .. start_pos-1 -> the fp16 attention copies
//   gemm_kernel<QKV>     [Q|K|V] = x [Wq;Wk;Wv]^T on bf16 matrix cores; the
//                        epilogue rotates Q/K pairs (RoPE), appends K/V to
//                        the bf16 cache and writes fp16 copies of Q (scaled
//                        by log2(e)/sqrt(128)), K and V^T for attention
//   prefill_attn_kernel  causal flash attention on fp16 matrix cores, one
//                        workgroup per (sequence, kv head, query tile) with
//                        the kv head's n_rep query heads sharing every K/V
//                        tile (64 queries for Llama 3.1 8B's n_rep = 4)
//   gemm_kernel<OUT>     Delta = O Wo^T on fp16 matrix cores, fp32 out
//
// Precision: the GEMM inputs x and W are bf16 already, products are exact and
// sums are fp32.  Attention and wo use fp16 operands: the cached K/V values
// and Wo are bf16 and convert to fp16 exactly inside fp16's normal range
// (2^-14 <= |v| <= 65504; smaller magnitudes lose low bits as fp16
// subnormals), while Q, P and O gain 3 significant bits over bf16.  A value
// beyond 65504, which bf16 can hold, is saturated to +-65504 and flagged in
// the workspace's error word (GQA_WS_ERR_FP16_RANGE) instead of becoming
// infinite.
#include <math.h>

#include <type_traits>

#include "kernels.h"

namespace gqa {


static size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

constexpr float kLazyRescale = 8.f;   // log2 headroom before the softmax reference moves
constexpr int AK = kPrefillTile;      // keys per attention tile (and per fp16 V^T block)

// ---------------------------------------------------------------------------
// Workspace
// ---------------------------------------------------------------------------

static size_t prefill_key_rows(int start_pos, int T) {
  return (size_t)(start_pos + T + kPrefillTile - 1) / kPrefillTile * kPrefillTile;
}

size_t prefill_ws_bytes(int B, int start_pos, int T, int kv) {
  const size_t M = (size_t)B * T;
  const size_t Tp = prefill_key_rows(start_pos, T);
  size_t n = kSyncBytes;                            // error word; decode's synchronisation words
  n += align256((size_t)D * D * 2);                 // wo16
  n += align256(M * D * 2);                         // q16
  n += align256((size_t)B * kv * Tp * HD * 2);      // k16
  n += align256((size_t)B * kv * HD * Tp * 2);      // v16t
  n += align256(M * D * 2);                         // o16
  return n;
}

void prefill_ws_carve(void* ws, PrefillParams* p) {
  const size_t M = (size_t)p->B * p->T;
  const size_t Tp = (size_t)p->Tp;
  p->err = static_cast<int*>(ws);   // the error word heads the workspace
  char* c = static_cast<char*>(ws) + kSyncBytes;
  p->wo16 = reinterpret_cast<uint16_t*>(c);
  c += align256((size_t)D * D * 2);
  p->q16 = reinterpret_cast<uint16_t*>(c);
  c += align256(M * D * 2);
  p->k16 = reinterpret_cast<uint16_t*>(c);
  c += align256((size_t)p->B * p->kv * Tp * HD * 2);
  p->v16t = reinterpret_cast<uint16_t*>(c);
  c += align256((size_t)p->B * p->kv * HD * Tp * 2);
  p->o16 = reinterpret_cast<uint16_t*>(c);
}

// ---------------------------------------------------------------------------
// Operand preparation: wo -> fp16, cached rows -> fp16 copies
// ---------------------------------------------------------------------------

// wo16 = fp16(wo) over threads tid0, tid0 + stride, ... (8 values each);
// returns whether any value saturated.
__device__ __forceinline__ bool convert_wo_part(const uint16_t* __restrict__ wo,
                                                uint16_t* __restrict__ wo16, long tid0,
                                                long stride) {
  bool sat = false;
  const long n8 = (long)D * D / 8;
  for (long i = tid0; i < n8; i += stride) {
    const u32x4 v = ld_nt_u32x4(wo + (size_t)i * 8);
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = bf16x2_to_f16x2_sat(v[q], sat);
    *reinterpret_cast<u32x4*>(wo16 + (size_t)i * 8) = o;
  }
  return sat;
}

__global__ void __launch_bounds__(256) wo_to_fp16_kernel(const uint16_t* wo, uint16_t* wo16) {
  (void)convert_wo_part(wo, wo16, (long)blockIdx.x * 256 + threadIdx.x, (long)gridDim.x * 256);
}

// Converts wo to fp16 (unless the caller passed its own copy), copies the
// cached rows 0 .. start_pos-1 of K and V into the fp16 attention copies
// (bf16 -> fp16 is exact inside fp16's normal range and saturates beyond
// it), and clears the positions [start_pos+T, Tp) of both copies (the
// attention tiles read them; they must be finite).
__global__ void __launch_bounds__(256) prefill_prep_kernel(PrefillParams p) {
  const long stride = (long)gridDim.x * 256;
  const long tid0 = (long)blockIdx.x * 256 + threadIdx.x;
  bool sat = false;
  if (p.convert_wo) sat = convert_wo_part(p.wo, p.wo16, tid0, stride);
  const int kv = p.kv;
  const int pairs = p.B * kv;
  const int nblk = p.Tp / AK;
  // cached prefix: 8 elements per item (a K row segment, or 8 positions of
  // one V dimension; the V items of an unaligned tail are element-wise)
  const int sp = p.start_pos;
  if (sp > 0) {
    const long nk = (long)pairs * sp * (HD / 8);
    for (long i = tid0; i < nk; i += stride) {
      const int pair = (int)(i / ((long)sp * (HD / 8)));
      const int r = (int)(i % ((long)sp * (HD / 8)));
      const int t = r / (HD / 8), d = (r % (HD / 8)) * 8;
      const u32x4 v = *reinterpret_cast<const u32x4*>(p.kcache + ((size_t)pair * p.T_max + t) * HD + d);
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = bf16x2_to_f16x2_sat(v[q], sat);
      *reinterpret_cast<u32x4*>(p.k16 + ((size_t)pair * p.Tp + t) * HD + d) = o;
    }
    const int groups = (sp + 7) / 8;
    const long nv = (long)pairs * HD * groups;
    for (long i = tid0; i < nv; i += stride) {
      const int pair = (int)(i / ((long)HD * groups));
      const int r = (int)(i % ((long)HD * groups));
      const int d = r / groups, t0 = (r % groups) * 8;
      const int b = pair / kv, g = pair % kv;
      uint16_t* dst = p.v16t + (((size_t)pair * nblk + t0 / AK) * HD + d) * AK + t0 % AK;
      if (t0 + 8 <= sp) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(p.vcache + vcache_index(b, g, t0, d, p.T_max, kv));
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = bf16x2_to_f16x2_sat(v[q], sat);
        *reinterpret_cast<u32x4*>(dst) = o;
      } else {
        for (int t = t0; t < sp; ++t) {
          const float f = sat_f16(bf16_bits_to_f32(p.vcache[vcache_index(b, g, t, d, p.T_max, kv)]), sat);
          dst[t - t0] = __builtin_bit_cast(uint16_t, (_Float16)f);
        }
      }
    }
  }
  if (sat) __hip_atomic_fetch_or(p.err, GQA_WS_ERR_FP16_RANGE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int lo = sp + p.T;
  const int pad = p.Tp - lo;
  if (pad == 0) return;
  // K rows: pairs * pad rows of 128; V^T: pairs * 128 dims of pad positions
  const long nk = (long)pairs * pad * HD;
  const long total = 2 * nk;
  for (long i = tid0; i < total; i += stride) {
    const long e = i < nk ? i : i - nk;
    const int pair = (int)(e / ((long)pad * HD));
    const int r = (int)(e % ((long)pad * HD));
    if (i < nk) {
      const int t = lo + r / HD, d = r % HD;
      p.k16[((size_t)pair * p.Tp + t) * HD + d] = 0;
    } else {
      const int d = r / pad, t = lo + r % pad;
      p.v16t[(((size_t)pair * nblk + t / AK) * HD + d) * AK + t % AK] = 0;
    }
  }
}

hipError_t launch_prefill_prep(const PrefillParams& p, hipStream_t s) {
  hipLaunchKernelGGL(prefill_prep_kernel, dim3(2048), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_wo_to_fp16(const uint16_t* wo, uint16_t* wo16, hipStream_t s) {
  hipLaunchKernelGGL(wo_to_fp16_kernel, dim3(2048), dim3(256), 0, s, wo, wo16);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 256 x 256 x 64 GEMM on the matrix cores, C = A B^T with A [M][4096] and
// B [N][4096] both K-contiguous.
// ---------------------------------------------------------------------------
//
// 8 waves in a 2 (M) x 4 (N) grid, each owning a 128 x 64 block of C as
// 8 x 4 16x16 tiles (128 accumulators, so two waves fit on a SIMD without the
// accumulators spilling into copies).  A and B tiles stream from global memory straight into LDS
// (global_load_lds, 16 bytes a lane), double-buffered.  In LDS a tile row of
// 64 elements is 8 chunks of 16 bytes stored at chunk ^ (row & 7), so the 16
// rows one matrix-core operand read touches fall in distinct banks.

constexpr int GBM = 256, GBN = 256, GBK = 64;
constexpr int kGemmLds = 2 * (GBM + GBN) * GBK * 2;   // 128 KiB
constexpr int kGroupM = 4;                             // m-tiles per tile-order group

enum GemmKind { GEMM_QKV = 0, GEMM_OUT = 1 };

// Row of B feeding tile column j of an n-tile starting at n0.  Each
// 32-column block holds the even features of 16 consecutive pairs in its
// first 16 columns and the odd ones in the next 16, so features (f, f+1) land
// in the same lane of neighbouring accumulators: the QKV epilogue rotates
// RoPE pairs in place, and both epilogues stage feature pairs as one 8-byte
// LDS write.
__device__ __forceinline__ int b_row_of(int n0, int j) {
  return n0 + (j & ~31) + 2 * (j & 15) + ((j >> 4) & 1);
}

// kvf: K (and V) features of the QKV GEMM, kv heads * 128
template <int KIND>
__device__ __forceinline__ const uint16_t* b_row_ptr(const uint16_t* b0, const uint16_t* b1,
                                                     const uint16_t* b2, int row, int kvf) {
  if (KIND == GEMM_QKV) {
    if (row < D) return b0 + (size_t)row * D;
    if (row < D + kvf) return b1 + (size_t)(row - D) * D;
    return b2 + (size_t)(row - D - kvf) * D;
  }
  return b0 + (size_t)row * D;
}

struct GemmArgs {
  const uint16_t* a;     // [M][4096]
  const uint16_t* b0;    // rows 0..   (Wq or wo16)
  const uint16_t* b1;    // Wk (QKV only)
  const uint16_t* b2;    // Wv (QKV only)
  int M, N;
  PrefillParams p;
};

template <int REGION, int HALF>
__device__ __forceinline__ void qkv_epilogue(const GemmArgs& g, const f32x4 (&acc)[8][4], char* st,
                                             int mw, int fw, int lane);
template <int HALF>
__device__ __forceinline__ void out_epilogue(const GemmArgs& g, const f32x4 (&acc)[8][4], char* st,
                                             int mw, int fw, int lane);

template <int KIND>
__global__ void __launch_bounds__(512, 1) gemm_kernel(GemmArgs g) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int wm = w >> 2, wn = w & 3;

  // XCD-aware tile order: the dispatcher's round-robin puts workgroup i on
  // XCD i % 8 on an idle chip; give each XCD a contiguous range of the
  // grouped tile order so its L2 serves 4 m-tiles against a sweep of n-tiles
  // (a locality heuristic: later workgroups go where slots free up).
  const int num_m = (g.M + GBM - 1) / GBM, num_n = g.N / GBN;
  const int total = num_m * num_n;
  int tl = blockIdx.x;
  if ((total & 7) == 0) tl = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int group = tl / (kGroupM * num_n);
  const int first_m = group * kGroupM;
  const int gm = min(kGroupM, num_m - first_m);
  const int within = tl - group * kGroupM * num_n;
  const int mt0 = first_m + within % gm;
  const int nt0 = within / gm;
  const int m0 = mt0 * GBM, n0 = nt0 * GBN;

  // per-lane global sources of the 4 A and 4 B load instructions of this
  // wave (wave w fills tile rows w*32 .. w*32+31, 8 rows per instruction;
  // lane l writes LDS chunk l & 7 of row l >> 3, holding logical chunk
  // (l & 7) ^ (l >> 3))
  const int lrow = lane >> 3;
  const int lchunk = (lane & 7) ^ lrow;
  // The tile's first A row and first B row are uniform bases (a B tile lies
  // in one of Wq / Wk / Wv); lanes keep 32-bit byte offsets from them.
  const char* a_base = reinterpret_cast<const char*>(g.a + (size_t)m0 * D);
  const char* b_base = reinterpret_cast<const char*>(b_row_ptr<KIND>(g.b0, g.b1, g.b2, n0, g.p.kv * HD));
  uint32_t a_off[4], b_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = w * 32 + i * 8 + lrow;
    const int am = min(m0 + r, g.M - 1) - m0;
    a_off[i] = (uint32_t)(am * D + lchunk * 8) * 2u;
    b_off[i] = (uint32_t)((b_row_of(n0, r) - n0) * D + lchunk * 8) * 2u;
  }

  auto load_stage = [&](int stage, int k0) {
    char* sa = smem + stage * (GBM + GBN) * GBK * 2;
    char* sb = sa + GBM * GBK * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_global_load_lds(a_base + a_off[i] + k0 * 2, (lds_void*)(sa + (w * 32 + i * 8) * 128), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(b_base + b_off[i] + k0 * 2, (lds_void*)(sb + (w * 32 + i * 8) * 128), 16, 0, 0);
    }
  };

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Two-phase ping-pong.  The waves of rows 0..127 of the tile (waves 0-3,
  // one per SIMD) and of rows 128..255 (waves 4-7) alternate between a memory
  // phase (read this stage's operand fragments from LDS, issue tile loads)
  // and a compute phase (the stage's 64 matrix-core ops), half a stage apart,
  // so each SIMD's two waves take turns on the matrix core and on LDS.
  // Workgroup barriers separate the phases; the second group starts one
  // barrier late and the first ends with one extra.
  //   group 0 loads its half (A and B rows 0..127) of stage k+1 in its
  //   memory phase of stage k, and waits for it at the end of compute k;
  //   group 1 loads its half (rows 128..255) of stage k+2 in its memory
  //   phase of stage k, into the buffer it has just read (group 0 read it
  //   one phase earlier), and waits for stage k+1's half at the same point.
  // Either way a half is complete before the barrier that precedes the first
  // read of its stage, and no buffer is overwritten before both groups have
  // read it.
  const int grp = w >> 2;
  constexpr int nk = D / GBK;
  load_stage(0, 0);
  if (grp == 1) {
    load_stage(1, GBK);
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __builtin_amdgcn_s_barrier();
  if (grp == 1) __builtin_amdgcn_s_barrier();
  for (int kb = 0; kb < nk; ++kb) {
    const char* sa = smem + (kb & 1) * (GBM + GBN) * GBK * 2;
    const char* sb = sa + GBM * GBK * 2;
    u32x4 af[2][8], bf[2][4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int chunk = ks * 4 + (lane >> 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rb = wn * 64 + j * 16 + (lane & 15);
        bf[ks][j] = *reinterpret_cast<const u32x4*>(sb + rb * 128 + ((chunk ^ (rb & 7)) << 4));
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ra = wm * 128 + i * 16 + (lane & 15);
        af[ks][i] = *reinterpret_cast<const u32x4*>(sa + ra * 128 + ((chunk ^ (ra & 7)) << 4));
      }
    }
    // group 0 loads stage kb+1, group 1 stage kb+2 (into the buffer just read)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int kl = kb + 1 + grp;
    if (kl < nk) {
      load_stage(kl & 1, kl * GBK);
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (KIND == GEMM_QKV)
            acc[i][j] = mfma_bf16(af[ks][i], bf[ks][j], acc[i][j]);
          else
            acc[i][j] = mfma_f16(af[ks][i], bf[ks][j], acc[i][j]);
        }
    __builtin_amdgcn_s_setprio(0);
    if (grp == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  }
  if (grp == 0) __builtin_amdgcn_s_barrier();

  // epilogue: acc[i][2u+s][e] is C[row m0 + wm*128 + i*16 + (lane>>4)*4 + e]
  //                               [feature n0 + wn*64 + 32u + 2*(lane&15) + s].
  // Once every wave is done with the last stage, wave w stages its 128 x 64
  // block through its own 16 KiB of LDS, 64 rows at a time, and writes it
  // with 16-byte stores.  The region (Q, K or V features) is uniform over
  // the workgroup's n-tile.
  __syncthreads();
  char* st = smem + w * 16384;
  const int mw = m0 + wm * 128, fw = n0 + 64 * wn;
  if (KIND == GEMM_QKV) {
    if (n0 < D) {
      qkv_epilogue<0, 0>(g, acc, st, mw, fw, lane);
      qkv_epilogue<0, 1>(g, acc, st, mw, fw, lane);
    } else if (n0 < D + g.p.kv * HD) {
      qkv_epilogue<1, 0>(g, acc, st, mw, fw, lane);
      qkv_epilogue<1, 1>(g, acc, st, mw, fw, lane);
    } else {
      qkv_epilogue<2, 0>(g, acc, st, mw, fw, lane);
      qkv_epilogue<2, 1>(g, acc, st, mw, fw, lane);
    }
  } else {
    out_epilogue<0>(g, acc, st, mw, fw, lane);
    out_epilogue<1>(g, acc, st, mw, fw, lane);
  }
}

// Epilogue staging.  Rows [64*HALF, 64*HALF + 64) of a wave's block go to
// its 16 KiB of LDS as fp32, either row-major (row r: 64 features in 16
// units of 16 bytes, unit u at u ^ (r & 15)) or, for V, feature-major
// (feature c: 64 rows in 16 units, unit u at u ^ (c & 15)).
__device__ __forceinline__ int stage_off(int line, int unit) {
  return line * 256 + ((unit ^ (line & 15)) << 4);
}

template <int HALF>
__device__ __forceinline__ void stage_rows(char* st, const f32x4 (&acc)[8][4], int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int r = i * 16 + (lane >> 4) * 4 + e;
        const int c = 32 * u + 2 * (lane & 15);
        *reinterpret_cast<float2*>(st + stage_off(r, c >> 2) + (c & 3) * 4) =
            make_float2(acc[4 * HALF + i][2 * u][e], acc[4 * HALF + i][2 * u + 1][e]);
      }
}

template <int HALF>
__device__ __forceinline__ void stage_cols(char* st, const f32x4 (&acc)[8][4], int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = 32 * (j >> 1) + 2 * (lane & 15) + (j & 1);
      *reinterpret_cast<f32x4*>(st + stage_off(c, i * 4 + (lane >> 4))) = acc[4 * HALF + i][j];
    }
}

__device__ __forceinline__ void lds_drain() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// QKV epilogue over rows [mw + 64*HALF, +64) and features [fw, fw + 64).
// Row m is token t = m mod T of sequence m / T, at position start_pos + t.
// REGION 0: Q (rotate, scale by log2(e)/sqrt(128), fp16 to the workspace);
// REGION 1: K (rotate, bf16 to the cache, fp16 copy); REGION 2: V (bf16 to the
// blocked dimension-major cache, fp16 copy).  For Q and K a lane owns 8
// consecutive features of one row (4 rotation pairs, one 32-byte RoPE load);
// for V it owns 8 consecutive positions of one feature, which are 16
// contiguous bytes of both value layouts when T and start_pos are multiples
// of 8.
template <int REGION, int HALF>
__device__ __forceinline__ void qkv_epilogue(const GemmArgs& g, const f32x4 (&acc)[8][4], char* st,
                                             int mw, int fw, int lane) {
  const PrefillParams& p = g.p;
  const int T = p.T;
  const int mh = mw + 64 * HALF;
  bool sat = false;                 // an fp16 copy saturated
  if (HALF) lds_drain();            // the previous half's reads have returned
  if (REGION < 2) {
    const int k = lane & 7;         // 8-feature chunk of the row
    stage_rows<HALF>(st, acc, lane);
    f32x4 cs[8][2];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int m = mh + it * 8 + (lane >> 3);
      const int pos = p.start_pos + m - (m / T) * T;  // in range for padding rows too
      const float* rr = p.rope + (size_t)pos * HD + (fw & (HD - 1)) + 8 * k;
      cs[it][0] = *reinterpret_cast<const f32x4*>(rr);
      cs[it][1] = *reinterpret_cast<const f32x4*>(rr + 4);
    }
    lds_drain();
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int r = it * 8 + (lane >> 3);
      const int m = mh + r;
      const f32x4 lo = *reinterpret_cast<const f32x4*>(st + stage_off(r, 2 * k));
      const f32x4 hi = *reinterpret_cast<const f32x4*>(st + stage_off(r, 2 * k + 1));
      if (m >= g.M) continue;
      float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const float c8[8] = {cs[it][0][0], cs[it][0][1], cs[it][0][2], cs[it][0][3],
                           cs[it][1][0], cs[it][1][1], cs[it][1][2], cs[it][1][3]};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = v[2 * j], c = v[2 * j + 1];
        const float co = c8[2 * j], si = c8[2 * j + 1];
        v[2 * j] = a * co - c * si;
        v[2 * j + 1] = a * si + c * co;
      }
      const int f = fw + 8 * k;
      if (p.probe) {
        float* pr = p.probe + (size_t)m * g.N + f;
        *reinterpret_cast<f32x4*>(pr) = f32x4{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4*>(pr + 4) = f32x4{v[4], v[5], v[6], v[7]};
      }
      if (REGION == 0) {
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          o[j] = pack_f16x2_sat(v[2 * j] * kScoreLog2, v[2 * j + 1] * kScoreLog2, sat);
        *reinterpret_cast<u32x4*>(p.q16 + (size_t)m * D + f) = o;
      } else {
        const int b = m / T, t = p.start_pos + m - b * T;
        const int ff = f - D, gg = ff / HD, d = ff % HD;
        u32x4 kb, kh;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          kb[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
          kh[j] = bf16x2_to_f16x2_sat(kb[j], sat);
        }
        *reinterpret_cast<u32x4*>(p.kcache + ((size_t)(b * p.kv + gg) * p.T_max + t) * HD + d) = kb;
        *reinterpret_cast<u32x4*>(p.k16 + ((size_t)(b * p.kv + gg) * p.Tp + t) * HD + d) = kh;
      }
    }
  } else {
    stage_cols<HALF>(st, acc, lane);
    lds_drain();
    const int q = lane & 7;         // 8-row group of the half
    // then a group is 8 aligned positions of one sequence
    const bool vec = ((T | p.start_pos) & 7) == 0;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int c = (lane >> 3) + 8 * it;
      const f32x4 lo = *reinterpret_cast<const f32x4*>(st + stage_off(c, 2 * q));
      const f32x4 hi = *reinterpret_cast<const f32x4*>(st + stage_off(c, 2 * q + 1));
      const float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const int f = fw + c;
      const int ff = f - D - p.kv * HD, gg = ff / HD, d = ff % HD;
      const int m0 = mh + 8 * q;
      if (p.probe) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (m0 + e < g.M) p.probe[(size_t)(m0 + e) * g.N + f] = v[e];
      }
      if (vec) {
        if (m0 >= g.M) continue;
        const int b = m0 / T, t = p.start_pos + m0 - b * T;
        u32x4 vb, vh;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          vb[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
          vh[j] = bf16x2_to_f16x2_sat(vb[j], sat);
        }
        *reinterpret_cast<u32x4*>(p.vcache + vcache_index(b, gg, t, d, p.T_max, p.kv)) = vb;
        *reinterpret_cast<u32x4*>(
            p.v16t + (((size_t)(b * p.kv + gg) * (p.Tp / AK) + t / AK) * HD + d) * AK + t % AK) = vh;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int m = m0 + e;
          if (m >= g.M) break;
          const int b = m / T, t = p.start_pos + m - b * T;
          const uint32_t vb = f32_to_bf16_bits(v[e]);
          p.vcache[vcache_index(b, gg, t, d, p.T_max, p.kv)] = (uint16_t)vb;
          const _Float16 h = (_Float16)sat_f16(bf16_bits_to_f32(vb), sat);
          p.v16t[(((size_t)(b * p.kv + gg) * (p.Tp / AK) + t / AK) * HD + d) * AK + t % AK] =
              __builtin_bit_cast(uint16_t, h);
        }
      }
    }
  }
  if (sat) __hip_atomic_fetch_or(p.err, GQA_WS_ERR_FP16_RANGE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// wo epilogue: fp32 rows of Delta (added to out when accumulating), one
// 16-byte unit per lane, 4 rows of 256 bytes per store instruction.
template <int HALF>
__device__ __forceinline__ void out_epilogue(const GemmArgs& g, const f32x4 (&acc)[8][4], char* st,
                                             int mw, int fw, int lane) {
  if (HALF) lds_drain();
  stage_rows<HALF>(st, acc, lane);
  lds_drain();
  const int mh = mw + 64 * HALF;
  const int u = lane & 15;
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    const int r = it * 4 + (lane >> 4);
    const f32x4 v = *reinterpret_cast<const f32x4*>(st + stage_off(r, u));
    const int m = mh + r;
    if (m >= g.M) continue;
    f32x4* dst = reinterpret_cast<f32x4*>(g.p.out + (size_t)m * D + fw + 4 * u);
    *dst = g.p.accumulate ? *dst + v : v;
  }
}

template <int KIND>
static hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_kernel<KIND>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds);
  if (e != hipSuccess) return e;
  const int tiles = ((g.M + GBM - 1) / GBM) * (g.N / GBN);
  hipLaunchKernelGGL(gemm_kernel<KIND>, dim3(tiles), dim3(512), kGemmLds, s, g);
  return hipGetLastError();
}

hipError_t launch_prefill_qkv(const PrefillParams& p, hipStream_t s) {
  GemmArgs g;
  g.a = p.x;
  g.b0 = p.wq;
  g.b1 = p.wk;
  g.b2 = p.wv;
  g.M = p.B * p.T;
  g.N = D + 2 * p.kv * HD;
  g.p = p;
  return launch_gemm<GEMM_QKV>(g, s);
}

hipError_t launch_prefill_wo(const PrefillParams& p, hipStream_t s) {
  GemmArgs g;
  g.a = p.o16;
  g.b0 = p.wo16;
  g.b1 = nullptr;
  g.b2 = nullptr;
  g.M = p.B * p.T;
  g.N = D;
  g.p = p;
  return launch_gemm<GEMM_OUT>(g, s);
}

// ---------------------------------------------------------------------------
// Causal flash attention (prefill)
// ---------------------------------------------------------------------------
//
// Workgroup = (sequence b, kv head g, query tile), 8 waves: wave w handles
// query head NR*g + (w % NR) for the 32 queries 32*(w / NR) .. of the tile,
// NR = 32 / KV query heads per kv head, so the tile spans 256 / NR queries
// (64 for Llama 3.1 8B's NR = 4; 128 for NR = 2; 256 for multi-head
// attention).  All 8 waves share every K/V tile in LDS and two waves run
// on each SIMD (one's softmax overlaps the other's matrix-core work).  Per
// 64-key tile, in fp16 on the matrix cores:
//   S^T[64 keys x 32 q] = K . Q^T      (A = K tile from LDS, B = Q in VGPRs)
//   O^T[128 dims x 32 q] += V^T . P^T  (A = V^T tile from LDS, B = P in VGPRs)
// Within each 32-key half, A-operand row r of score tile "sub" holds key
// (r >> 2)*8 + sub*4 + (r & 3); each lane then owns 8 consecutive keys of
// its query column, which is exactly its B operand for the P.V step.

constexpr int kAttnStage = 2 * AK * HD * 2;      // K and V^T tiles, fp16: 32 KiB

// LDS swizzles of the K and V^T tiles.  One fragment read touches 16 K rows
// (keys whose bits 0, 1, 3, 4 vary) or 16 consecutive V^T rows (128 bytes
// each, two to a 256-byte bank window), each lane a 16-byte slot.  K rows
// hold chunk c at c ^ kswz(key), V^T rows chunk c at c ^ (dim & 7).  Both
// were chosen by the LDS bank-conflict counter: with these maps the
// fragment reads register no conflicts on gfx950, while folding bit 3 of
// the dimension into the V^T map as well (a map that also spreads any 8
// consecutive rows over a 128-byte window) made the V^T reads take twice
// the LDS cycles.
__device__ __forceinline__ int attn_kswz(int key) { return (key & 3) | ((key >> 1) & 12); }
__device__ __forceinline__ int attn_vswz(int dim) { return dim & 7; }
constexpr int kAttnLds = 2 * kAttnStage;         // double-buffered: 64 KiB

// queries per workgroup of the attention kernel for kv heads KV
constexpr int attn_queries(int kv) { return 32 * (8 / (H / kv)); }

template <int KV>
__global__ void __launch_bounds__(512, 1) prefill_attn_kernel(PrefillParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int NR = H / KV;
  constexpr int AQW = attn_queries(KV);
  static_assert(NR == 1 || NR == 2 || NR == 4, "8 waves split over NR heads");

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int col = lane & 15, rg = lane >> 4;
  const int T = p.T, Tp = p.Tp;
  const int nqt = (T + AQW - 1) / AQW;
  const int pairs = p.B * KV;
  const int bg = blockIdx.x % pairs;
  const int qt = nqt - 1 - blockIdx.x / pairs;      // longest rows first
  const int b = bg / KV, g = bg % KV;
  const int h = g * NR + (w % NR);
  const int q0 = qt * AQW + 32 * (w / NR);          // first new token of this wave
  // key tiles 0 .. klast hold the keys of the workgroup's queries (positions
  // start_pos + t); from tile kmask on, some key lies past one of this wave's
  const int klast = (p.start_pos + min(qt * AQW + AQW - 1, T - 1)) / AK;
  const int kmask = (p.start_pos + q0) / AK;

  const uint16_t* kg = p.k16 + (size_t)bg * Tp * HD;
  const uint16_t* vg = p.v16t + (size_t)bg * HD * Tp;

  // Tile loads go straight to LDS (16 bytes a lane, a wave writes 1 KiB of
  // consecutive LDS per instruction).  Each lane picks the global chunk that
  // belongs at its LDS slot under the XOR swizzle: K rows (256 B) hold chunk
  // c at c ^ attn_kswz(key), V^T rows (128 B) hold chunk c at
  // c ^ attn_vswz(dim).  Wave w fills K rows w*8 .. +8 and V^T rows
  // w*16 .. +16.  Positions in [T, Tp) of the workspace copies are zero, so
  // no masking is needed here.
  const uint16_t* k_src[2];
  const uint16_t* v_src[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int key = w * 8 + i * 4 + (lane >> 4);
    k_src[i] = kg + (size_t)key * HD + (((lane & 15) ^ attn_kswz(key)) * 8);
    const int dim = w * 16 + i * 8 + (lane >> 3);
    v_src[i] = vg + (size_t)dim * AK + (((lane & 7) ^ attn_vswz(dim)) * 8);
  }
  // K tile kt lives in K buffer kt & 1 and V^T tile kt in V buffer kt & 1.
  // Iteration kt reads K tile kt+1 (the next scores) and V tile kt, so at
  // its start K tile kt+2 and V tile kt+1 can be fetched into the buffers
  // iteration kt-1 has finished with.
  auto sK = [&](int buf) { return smem + buf * (AK * HD * 2); };
  auto sV = [&](int buf) { return smem + 2 * (AK * HD * 2) + buf * (AK * HD * 2); };
  auto issue_k = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(k_src[i] + (size_t)kt * AK * HD),
                                       (lds_void*)(sK(kt & 1) + (w * 8 + i * 4) * 256), 16, 0, 0);
  };
  auto issue_v = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(v_src[i] + (size_t)kt * (HD * AK)),
                                       (lds_void*)(sV(kt & 1) + (w * 16 + i * 8) * 128), 16, 0, 0);
  };
  issue_k(0);
  issue_v(0);
  if (klast > 0) issue_k(1);

  // Q^T fragments: query q0 + nt*16 + col, dims rg*8 + 32*ks
  u32x4 qf[2][4];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int t = q0 + nt * 16 + col;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qf[nt][ks] = (t < T) ? ld_u32x4(p.q16 + ((size_t)b * T + t) * D + h * HD + rg * 8 + 32 * ks)
                           : u32x4{0u, 0u, 0u, 0u};
  }

  f32x4 oacc[8][2];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) oacc[dt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // m_run: the softmax reference of each query column (exp2 units, Q is
  // pre-scaled), -inf before the first tile; l_run: the column sums of
  // exp2(s - m_run) so far.
  float m_run[2], l_run[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    m_run[nt] = -INFINITY;
    l_run[nt] = 0.f;
  }

  // S^T - r = K . Q^T - r for the K tile at k_lds, where r is the reference
  // the column's exponentials will use, folded into the accumulators'
  // initial value so that no subtraction is needed afterwards.
  // sacc[mt][nt][e]: key 32*(mt>>1) + rg*8 + (mt&1)*4 + e of the tile, query q0 + nt*16 + col
  auto scores = [&](const char* k_lds, const float (&r)[2], f32x4 (&sacc)[4][2]) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) sacc[mt][nt] = f32x4{-r[nt], -r[nt], -r[nt], -r[nt]};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int key = 32 * (mt >> 1) + (col >> 2) * 8 + (mt & 1) * 4 + (col & 3);
        const int c = ks * 4 + rg;
        const u32x4 kf = *reinterpret_cast<const u32x4*>(k_lds + key * 256 + ((c ^ attn_kswz(key)) << 4));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) sacc[mt][nt] = mfma_f16(kf, qf[nt][ks], sacc[mt][nt]);
      }
    }
  };
  // causal mask of tile kt: keys past the query get -inf
  auto mask = [&](int kt, f32x4 (&sc)[4][2]) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int q = p.start_pos + q0 + nt * 16 + col;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = kt * AK + 32 * (mt >> 1) + rg * 8 + (mt & 1) * 4 + e;
          if (key > q) sc[mt][nt][e] = -INFINITY;
        }
    }
  };
  // Lazy rescaling: the reference only moves (and O, l are only rescaled)
  // when a column's maximum exceeds it by more than 2^8, so that
  // p = exp2(s - m_run) <= 256 (in range for fp16).  The decision is
  // wave-uniform and most tiles skip the rescale.  prepare() takes the
  // decision for scores sc computed against reference r and returns the
  // columns' maxima in cand; rescale() then moves the reference, scales O
  // and l and re-references sc (it must follow every P.V product of the
  // earlier tiles).  The first tile always rescales (m_run = -inf; its
  // columns all hold key 0, so their maxima are finite).
  auto prepare = [&](const f32x4 (&sc)[4][2], const float (&r)[2], float (&cand)[2]) -> bool {
    bool grow = false;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      // the column's 16 scores of this lane as a tree of 3-input maxima
      // (v_max3_f32): 5 + 2 + 1 instructions
      float a[5];
#pragma unroll
      for (int i = 0; i < 5; ++i)
        a[i] = fmaxf(fmaxf(sc[(3 * i) >> 2][nt][(3 * i) & 3], sc[(3 * i + 1) >> 2][nt][(3 * i + 1) & 3]),
                     sc[(3 * i + 2) >> 2][nt][(3 * i + 2) & 3]);
      float t = fmaxf(fmaxf(fmaxf(a[0], a[1]), a[2]), fmaxf(fmaxf(a[3], a[4]), sc[3][nt][3]));
      t = max_xor32(max_xor16(t));
      cand[nt] = r[nt] + t;
      grow |= cand[nt] > m_run[nt] + kLazyRescale;
    }
    return __any(grow);
  };
  auto rescale = [&](f32x4 (&sc)[4][2], const float (&r)[2], const float (&cand)[2]) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const float m_new = fmaxf(m_run[nt], cand[nt]);
      const float alpha = __builtin_amdgcn_exp2f(m_run[nt] - m_new);
      l_run[nt] *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) oacc[dt][nt] *= alpha;
      const float shift = m_new - r[nt];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) sc[mt][nt] -= shift;
      m_run[nt] = m_new;
    }
  };

  // One key tile kt (its scores sc already against reference m_run, masked):
  // P = exp2(sc) and O += V P, with the next tile's scores (into sn), mask
  // and rescale decision computed in between, so that matrix-core and
  // vector work interleave.  BUF = kt & 1 is a constant, so every LDS
  // address is one too.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  f32x4 sa[4][2], sb[4][2];
  {
    const float r0[2] = {0.f, 0.f};
    float cand[2];
    scores(sK(0), r0, sa);
    if (0 >= kmask || klast == 0) mask(0, sa);
    if (prepare(sa, r0, cand)) rescale(sa, r0, cand);
  }
  auto step = [&](auto last_tag, auto buf_tag, int kt, f32x4 (&sc)[4][2], f32x4 (&sn)[4][2]) {
    constexpr bool LAST = decltype(last_tag)::value;
    constexpr int BUF = decltype(buf_tag)::value;
    // K tile kt+1 and V tile kt have landed for every wave, and every wave
    // is done with K tile kt and V tile kt-1
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (!LAST) {
      if (kt + 2 <= klast) issue_k(kt + 2);
      issue_v(kt + 1);
    }
    const float r[2] = {m_run[0], m_run[1]};
    if (!LAST) scores(sK(BUF ^ 1), r, sn);

    // P = exp2(sc) as fp16 pairs (the B operand of P.V); l gathers the same
    // fp16 values that O does
    u32x4 pf[2][2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      uint32_t pk[2][4];
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
          const int mt = half * 2 + sub;
          pk[half][sub * 2] = pack_f16x2(__builtin_amdgcn_exp2f(sc[mt][nt][0]),
                                         __builtin_amdgcn_exp2f(sc[mt][nt][1]));
          pk[half][sub * 2 + 1] = pack_f16x2(__builtin_amdgcn_exp2f(sc[mt][nt][2]),
                                             __builtin_amdgcn_exp2f(sc[mt][nt][3]));
        }
      float ps = l_run[nt];
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int j = 0; j < 4; ++j) ps = dot2_f16(pk[half][j], 0x3c003c00u, ps);
      l_run[nt] = ps;
      pf[nt][0] = u32x4{pk[0][0], pk[0][1], pk[0][2], pk[0][3]};
      pf[nt][1] = u32x4{pk[1][0], pk[1][1], pk[1][2], pk[1][3]};
    }

    bool rs = false;
    float cand[2];
    if (!LAST) {
      if (kt + 1 >= kmask || kt + 1 == klast) mask(kt + 1, sn);
      rs = prepare(sn, r, cand);
    }

    // ---- O^T += V^T P^T ----
    const char* v_lds = sV(BUF);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int dim = dt * 16 + col;
        const int c = half * 4 + rg;
        const u32x4 vf = *reinterpret_cast<const u32x4*>(v_lds + dim * 128 + ((c ^ attn_vswz(dim)) << 4));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) oacc[dt][nt] = mfma_f16(vf, pf[nt][half], oacc[dt][nt]);
      }
    }
    if (!LAST && rs) rescale(sn, r, cand);
  };
  using F = std::false_type;
  using Tr = std::true_type;
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  int kt = 0;
  for (; kt + 2 <= klast; kt += 2) {
    step(F{}, B0{}, kt, sa, sb);
    step(F{}, B1{}, kt + 1, sb, sa);
  }
  if (kt < klast) {
    step(F{}, B0{}, kt, sa, sb);
    step(Tr{}, B1{}, kt + 1, sb, sa);
  } else {
    step(Tr{}, B0{}, kt, sa, sb);
  }

  // ---- normalise, stage through LDS, store O (fp16) ----
  // Wave w's 32 x 128 block goes to its own 8 KiB of LDS, row = query, with
  // 16-byte chunk c of a row at c ^ (row & 15); each lane then stores 16
  // bytes, 4 rows of 256 contiguous bytes per instruction.
  __syncthreads();                                  // every wave is done with the K/V tiles
  char* so = smem + w * (32 * HD * 2);
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    float l = l_run[nt];
    l = sum_xor32(sum_xor16(l));
    const float inv = 1.f / l;
    const int row = nt * 16 + col;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const f32x4 o = oacc[dt][nt];
      const u32x2 v = {pack_f16x2(o[0] * inv, o[1] * inv), pack_f16x2(o[2] * inv, o[3] * inv)};
      const int c = dt * 2 + (rg >> 1);
      *reinterpret_cast<u32x2*>(so + row * 256 + ((c ^ (row & 15)) << 4) + (rg & 1) * 8) = v;
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int row = it * 4 + (lane >> 4), c = lane & 15;
    const u32x4 v = *reinterpret_cast<const u32x4*>(so + row * 256 + ((c ^ (row & 15)) << 4));
    const int t = q0 + row;
    if (t < T) *reinterpret_cast<u32x4*>(p.o16 + ((size_t)b * T + t) * D + h * HD + c * 8) = v;
  }
}

template <int KV>
static hipError_t launch_attn(const PrefillParams& p, hipStream_t s) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(prefill_attn_kernel<KV>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, kAttnLds);
  if (e != hipSuccess) return e;
  const int nqt = (p.T + attn_queries(KV) - 1) / attn_queries(KV);
  hipLaunchKernelGGL(prefill_attn_kernel<KV>, dim3(p.B * KV * nqt), dim3(512), kAttnLds, s, p);
  return hipGetLastError();
}

hipError_t launch_prefill_attn(const PrefillParams& p, hipStream_t s) {
  switch (p.kv) {
    case 16: return launch_attn<16>(p, s);
    case 32: return launch_attn<32>(p, s);
    default: return launch_attn<KVH>(p, s);
  }
}

}  // namespace gqa
