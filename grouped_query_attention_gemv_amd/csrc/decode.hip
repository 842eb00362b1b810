// Decode path of the attention block: one new token per sequence at position
// start_pos (page "Llama 3.1 8B . Grouped-query attention", decode mode:
// cache row start_pos written, rows 0..start_pos read).
//
//   decode_qkv_kernel   Q|K|V = x [Wq;Wk;Wv]^T as a bandwidth GEMV, RoPE on the
//                       Q and K pairs, K/V appended to the bf16 cache
//   decode_attn_kernel  flash-decode on the matrix cores: positions split over
//                       workgroups, online softmax, (m, l, o) merge by the
//                       last-arriving workgroup of each (sequence, kv head)
//   decode_wo_kernel    Delta = O Wo^T as a bandwidth GEMV (+ residual), up to
//                       4 tokens; decode_wo_mfma_kernel for 5 to 8
//   decode_step_kernel  the three as roles of one launch (B <= 2)
//   decode_proj_kernel  QKV or wo above 8 tokens: split-K on the matrix cores
#include <math.h>

#include <algorithm>

#include "gemv.h"
#include "kernels.h"

namespace gqa {

// ---------------------------------------------------------------------------
// QKV projection + RoPE + cache append
// ---------------------------------------------------------------------------

// Output features of QKV workgroup `blk` of W waves: 2W consecutive
// features, 2 per wave, in feature order (three-launch schedule).  The fused
// schedule (W = 4, RPW = fused_qkv_rpw(KV) row pairs a wave, 8 RPW features
// a workgroup) gives kv head g the workgroups blk = g (mod KV), like the
// head's attention workgroups: Q of its 32 / KV query heads, then K, then
// V.  No hand-off depends on the XCD a workgroup lands on.
template <bool FUSED, int W, int KV>
__device__ __forceinline__ int qkv_first_feature(int blk) {
  static_assert(!FUSED || W == 4, "the fused schedule's roles are laid out for 4-wave workgroups");
  if (!FUSED) return blk * 2 * W;
  constexpr int FPW = 8 * fused_qkv_rpw(KV);    // features per workgroup
  constexpr int NR = H / KV, QW = NR * HD / FPW, KW = HD / FPW;   // Q and K (= V) workgroups of a head
  const int g = blk % KV, r = blk / KV;
  if (r < QW) return g * (NR * HD) + r * FPW;
  if (r < QW + KW) return D + g * HD + (r - QW) * FPW;
  return D + KV * HD + g * HD + (r - QW - KW) * FPW;
}

// RoPE, probe and stores of the output features (f, f+1) of token b (f
// even): Q into the workspace, K and V rounded into the cache (fused: also
// into the hand-off row that the attention workgroups poll).  cs is the RoPE
// table entry of the pair at position start_pos (ignored for V).
template <bool FUSED, int KV>
__device__ __forceinline__ void qkv_emit_pair(const DecodeParams& p, int b, int f, float v0, float v1,
                                              float2 cs) {
  constexpr int kNqkv = D + 2 * KV * HD;
  const bool is_v = f >= D + KV * HD;
  const int pos = p.start_pos;
  if (!is_v) {
    // rotate the pair (2i, 2i+1) of this head by position * f_i
    const float a = v0 * cs.x - v1 * cs.y;
    const float c = v0 * cs.y + v1 * cs.x;
    v0 = a;
    v1 = c;
  }
  if (p.probe) {
    *reinterpret_cast<float2*>(p.probe + (size_t)b * kNqkv + f) = make_float2(v0, v1);
  }
  if (f < D) {
    float* qd = p.q + (size_t)b * D + f;
    if (FUSED) {
      // read by attention workgroups of this launch, which poll these
      // words until they no longer hold the "not yet" marker: written
      // through to the device-wide coherence point
      st_dev(qd, v0);
      st_dev(qd + 1, v1);
    } else {
      *reinterpret_cast<float2*>(qd) = make_float2(v0, v1);
    }
  } else {
    const int rr = is_v ? f - D - KV * HD : f - D;
    const int g = rr / HD, d = rr % HD;
    const uint32_t pair = pack_bf16x2(v0, v1);
    if (!is_v) {
      uint16_t* dst = p.kcache + ((size_t)(b * KV + g) * p.T_max + pos) * HD + d;
      *reinterpret_cast<uint32_t*>(dst) = pair;
    } else {
      uint16_t* dst = p.vcache + vcache_index(b, g, pos, d, p.T_max, KV);
      dst[0] = (uint16_t)(pair & 0xffffu);
      dst[VB] = (uint16_t)(pair >> 16);
    }
    // the attention workgroups of the same launch poll the new row here
    if (FUSED) st_dev(p.kv_new + ((size_t)(b * 2 + (is_v ? 1 : 0)) * KV + g) * (HD / 2) + d / 2, pair);
  }
}

// RoPE table entry of the output feature pair (f, f+1) at position start_pos
// ((1, 0), the identity, for V features).
template <int KV>
__device__ __forceinline__ float2 qkv_rope_entry(const DecodeParams& p, int f) {
  if (f >= D + KV * HD) return make_float2(1.f, 0.f);
  const int rr = f < D ? f : f - D;
  return reinterpret_cast<const float2*>(p.rope)[(size_t)p.start_pos * PAIRS + ((rr & (HD - 1)) >> 1)];
}

// KV: kv heads of the projection (8, 16 or 32, both schedules); W: waves of
// the workgroup; the fused schedule gives each wave fused_qkv_rpw(KV)
// consecutive row pairs (the three-launch schedule one).
template <int NB, bool FUSED, int KV = KVH, int W = 4>
__device__ __forceinline__ void qkv_body(const DecodeParams& p, int b0, int blk, uint32_t* xs) {
  constexpr int RPW = FUSED ? fused_qkv_rpw(KV) : 1;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // first (even) feature of the wave; its RPW pairs lie in one of Q, K, V
  const int r0 = qkv_first_feature<FUSED, W, KV>(blk) + wave * 2 * RPW;
  const uint16_t* wbase;
  int rr;
  if (r0 < D) {
    wbase = p.wq; rr = r0;
  } else if (r0 < D + KV * HD) {
    wbase = p.wk; rr = r0 - D;
  } else {
    wbase = p.wv; rr = r0 - D - KV * HD;
  }
  // x goes to LDS by direct loads issued first, with the RoPE entries of the
  // wave's feature pairs (one position for the whole batch) and the norm
  // gain; the 16 RPW weight loads follow at once, and the rest has landed
  // once only they remain in flight
  stage_rows_async<NB, W>(xs, p.x + (size_t)b0 * D);
  float2 cs[RPW];
#pragma unroll
  for (int j = 0; j < RPW; ++j) cs[j] = qkv_rope_entry<KV>(p, r0 + 2 * j);
  uint32_t gp[(D / 2) / (64 * W)];
  if (p.norm_w) load_norm_gain<W>(p.norm_w, gp);
  u32x4 wa[RPW][8], wb[RPW][8];
#pragma unroll
  for (int j = 0; j < RPW; ++j)
    load_rows2(wbase + (size_t)(rr + 2 * j) * D, wbase + (size_t)(rr + 2 * j + 1) * D, lane, wa[j], wb[j]);
  wait_loads_except<16 * RPW>();
  if (!FUSED && blk == 0 && b0 == 0) {
    // the attention kernel that follows counts split arrivals from zero
    for (int i = threadIdx.x; i < p.B * KV; i += blockDim.x) p.counters[i] = 0;
  }
  lds_barrier();
  if (p.norm_w) norm_rows<NB, W>(xs, gp, p.norm_eps);

#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    float acc[2][NB];
    gemv_rows2<NB, 1>(wa[j], wb[j], xs, lane, acc);
    float v0 = 0.f, v1 = 0.f;
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const float s0 = wave_sum(acc[0][t]);
      const float s1 = wave_sum(acc[1][t]);
      if (lane == t) { v0 = s0; v1 = s1; }
    }
    if (lane < NB) qkv_emit_pair<FUSED, KV>(p, b0 + lane, r0 + 2 * j, v0, v1, cs[j]);
  }
}

// W waves a workgroup: 4, or 8 for 7 and 8 tokens, whose 56-64 KiB of staged
// inputs would otherwise leave room for only 512 resident 4-wave workgroups
// (the weights would stream in two rounds).
template <int NB, int KV, int W>
__global__ void __launch_bounds__(64 * W) decode_qkv_kernel(DecodeParams p, int b0) {
  __shared__ uint32_t xs[NB * (D / 2)];
  qkv_body<NB, false, KV, W>(p, b0, blockIdx.x, xs);
}

// ---------------------------------------------------------------------------
// Flash-decode on the matrix cores
// ---------------------------------------------------------------------------

// Workgroup (split, g, b) owns positions [split*chunk, min(L, (split+1)*chunk))
// of kv head g of sequence b and serves its 4 query heads.  Each wave steps
// over 32-position tiles:
//   S^T[32 keys x 16 cols] = K[keys x 128] . Qext^T, where Qext's 16 columns
//     are the 4 heads' bf16 high parts (cols 0-3), their low parts q - hi
//     (cols 4-7) and zeros, so hi + lo restores Q to ~16 significant bits and
//     each K row is read from HBM once for all 4 heads;
//   O^T[128 dims x 16 cols] += V^T[dims x keys] . Pext^T with the same hi/lo
//     split of the probabilities, V^T read directly from the dimension-major
//     value cache.
// The A-operand rows of the score tiles are assigned to positions so that
// each lane's 8 score values are 8 consecutive positions: exactly the B
// operand of the following P.V instruction, with no data movement.
//
// In the fused schedule the workgroup loads its first tiles before Q exists,
// waits for its kv head's release, then replaces the row of position
// start_pos (which the same launch writes) with the copy in kv_new.
// Floats of split partials per (sequence, kv head): nsplit splits of nr
// heads, rounded up to whole 128-byte lines.
__host__ __device__ constexpr size_t part_region_floats(int nsplit, int nr) {
  return ((size_t)nsplit * nr * kPartStride + 31) / 32 * 32;
}

// LDS of the 4-wave merge for n_rep query heads per kv head
constexpr int attn_lds_words(int rep) { return kAttnWaves * rep * HD + 2 * kAttnWaves * rep + 1; }
constexpr int kAttnLdsWords = attn_lds_words(REP);

// FUSED: Q, K and V come from the same launch.  The workgroup polls, with
// device-scope loads, the words of Q and of the appended row themselves
// (they hold a "not yet" marker until their QKV workgroup stores them), so
// value and arrival come in one round trip.  Every split but the last
// publishes its partials into marked words and ends; the last split polls
// them and merges, and O goes to the wo workgroups of the launch (on every
// XCD) through device-scope stores and one flag per wo workgroup.
// KV kv heads serve NR = 32 / KV query heads each (NR = 4 for Llama 3.1 8B;
// 2 and 1, the last being multi-head attention).  The MFMA operand columns
// are the NR heads' hi parts, then their lo parts.
template <bool FUSED, int KV = KVH>
__device__ __forceinline__ void attn_body(const DecodeParams& p, int blk, float* lds) {
  constexpr int NR = H / KV;
  static_assert(NR == 1 || NR == 2 || NR == 4, "the wave merge maps one 64-thread slice per head");
  constexpr int kShlNr = 0x100 + NR;             // DPP row_shl:NR, lane i <- lane i + NR
  constexpr int kShrNr = 0x110 + NR;             // DPP row_shr:NR, lane i <- lane i - NR
  // fused: g = blk mod KV, as for the head's QKV workgroups
  const int split = FUSED ? (blk / KV) % p.nsplit : blk % p.nsplit;
  const int g = FUSED ? blk % KV : (blk / p.nsplit) % KV;
  const int b = FUSED ? (blk / KV) / p.nsplit : blk / (p.nsplit * KV);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int col = lane & 15, rg = lane >> 4;
  const int head = col % NR;
  const bool valid_col = col < 2 * NR;
  const bool is_lo = (col / NR) == 1;
  const int L = p.start_pos + 1;
  const int P = p.start_pos;
  const int j_begin = split * p.chunk;
  const int j_end = min(L, j_begin + p.chunk);
  const int T_max = p.T_max;

  float (*sm_o)[NR][HD] = reinterpret_cast<float (*)[NR][HD]>(lds);
  float (*sm_m)[NR] = reinterpret_cast<float (*)[NR]>(lds + kAttnWaves * NR * HD);
  float (*sm_l)[NR] = reinterpret_cast<float (*)[NR]>(lds + kAttnWaves * NR * HD + kAttnWaves * NR);
  int* sm_last = reinterpret_cast<int*>(lds + kAttnWaves * NR * HD + 2 * kAttnWaves * NR);
  // fused schedule: Q of the 4 heads, after the merge words
  float* sm_q = lds + kFusedAttnQWord;

  const uint16_t* kbase = p.kcache + (size_t)(b * KV + g) * T_max * HD;
  const uint16_t* vbase = p.vcache + (size_t)(b * KV + g) * (T_max / VB) * (HD * VB);

  // Loads of one 32-position tile (tiles start at multiples of 32, so a tile
  // is one value-cache block).  Key rows past the last visible position are
  // clamped onto it (their scores are masked); value positions past it are
  // cleared after the load, since the cache may hold anything there.
  // Buffer loads off the (b, g) bases with 32-bit offsets (a 64-bit address
  // per load would cost registers the fused kernel does not have).
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kbase), 0, 0x7fffffff, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vbase), 0, 0x7fffffff, 0x00020000);
  auto load_tile = [&](int tile, u32x4 (&kf)[2][4], u32x4 (&vf)[8]) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int j = min(tile + (col >> 2) * 8 + mt * 4 + (col & 3), j_end - 1);
      const uint32_t off = (uint32_t)(j * HD + rg * 8) * 2u;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        kf[mt][ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krsrc, off + 64 * ks, 0, kNtPolicy));
    }
    // V^T rows col + 16 dt of the tile's block: dt * 1 KiB apart
    const uint32_t voff = (uint32_t)((tile / VB) * (HD * VB) + rg * 8 + col * VB) * 2u;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      vf[dt] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrsrc, voff + 1024 * (dt & 3), 4096 * (dt >> 2), kNtPolicy));
  };

  // Fused schedule: Q, the appended row and the split partials are all
  // published with device-scope stores into words that hold the "not yet"
  // marker, and polled with device-scope loads, which always see the
  // latest store whichever XCD made it (an L2-cached poll of a line the L2
  // already holds would not).

  // Fused schedule: replace the appended row (position start_pos, written by
  // this launch) with its copy in kv_new, for the lanes that hold it.  The
  // wave polls those words with device-scope loads until none holds the
  // "not yet" marker; a poll that runs out leaves the marker (a NaN) in
  // place and records the error.
  auto patch_tile = [&](int tile, u32x4 (&kf)[2][4], u32x4 (&vf)[8]) {
    if (P < tile || P >= tile + kAttnTile) return;     // wave-uniform
    const uint32_t kn_off = (uint32_t)(((b * 2) * KV + g) * HD) * 2u;   // bytes into kv_new
    const uint32_t* vn = p.kv_new + ((size_t)(b * 2 + 1) * KV + g) * (HD / 2);
    const int e = P - tile - rg * 8;     // element of this lane's 8 positions
    for (int polls = 0;; ++polls) {
      bool ok = true;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int j = min(tile + (col >> 2) * 8 + mt * 4 + (col & 3), j_end - 1);
        if (j == P) {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            kf[mt][ks] = ld_dev_x4(p.kv_new, kn_off + (uint32_t)(rg * 8 + 32 * ks) * 2u);
#pragma unroll
            for (int i = 0; i < 4; ++i) ok &= kf[mt][ks][i] != kNotYetPair;
          }
        }
      }
      if (e >= 0 && e < 8) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const int d = col + 16 * dt;
          const uint32_t wv = ld_dev(vn + d / 2);
          ok &= wv != kNotYetPair;
          const uint32_t h = (d & 1) ? (wv >> 16) : (wv & 0xffffu);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (q == (e >> 1)) {
              vf[dt][q] = (e & 1) ? ((vf[dt][q] & 0x0000ffffu) | (h << 16))
                                  : ((vf[dt][q] & 0xffff0000u) | h);
            }
          }
        }
      }
      if (__all(ok)) break;
      if (polls >= kMaxPolls) {
        if (lane == 0) __hip_atomic_fetch_or(p.sync + kSyncErr, GQA_WS_ERR_WAIT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  };

  u32x4 kf[2][4], vf[8];                  // one 32-position tile of K and V
  const int tile0 = j_begin + w * kAttnTile;
  int* grp_cnt = p.sync + kSyncGroup + 32 * g;
  int grp_prev = 0;
  u32x4 qf[4];
  float m_run, l_run;
  f32x4 oacc[8];

  // Q fragments, pre-scaled by log2(e)/sqrt(128)
  auto build_q = [&]() {
    const float* qrow = p.q + (size_t)b * D + (g * NR + head) * HD;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int d0 = rg * 8 + 32 * ks;
      float qv[8];
      if (FUSED) {
        const float4 qa = *reinterpret_cast<const float4*>(sm_q + head * HD + d0);
        const float4 qb = *reinterpret_cast<const float4*>(sm_q + head * HD + d0 + 4);
        qv[0] = qa.x; qv[1] = qa.y; qv[2] = qa.z; qv[3] = qa.w;
        qv[4] = qb.x; qv[5] = qb.y; qv[6] = qb.z; qv[7] = qb.w;
      } else {
        const float4 qa = *reinterpret_cast<const float4*>(qrow + d0);
        const float4 qb = *reinterpret_cast<const float4*>(qrow + d0 + 4);
        qv[0] = qa.x; qv[1] = qa.y; qv[2] = qa.z; qv[3] = qa.w;
        qv[4] = qb.x; qv[5] = qb.y; qv[6] = qb.z; qv[7] = qb.w;
      }
      uint32_t pk[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = qv[2 * e] * kScoreLog2, x1 = qv[2 * e + 1] * kScoreLog2;
        uint32_t h0 = f32_to_bf16_bits(x0), h1 = f32_to_bf16_bits(x1);
        if (is_lo) {
          h0 = f32_to_bf16_bits(x0 - bf16_bits_to_f32(h0));
          h1 = f32_to_bf16_bits(x1 - bf16_bits_to_f32(h1));
        }
        pk[e] = valid_col ? (h0 | (h1 << 16)) : 0u;
      }
      qf[ks] = u32x4{pk[0], pk[1], pk[2], pk[3]};
    }
  };

  auto compute_tile = [&](int tile, u32x4 (&kf)[2][4], u32x4 (&vf)[8]) {
    const int jv = tile + rg * 8;
    if (jv + 8 > j_end) {
      const int nv = j_end - jv;    // may be <= 0: the whole group is cleared
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t keep = (2 * q + 1 < nv) ? 0xffffffffu : (2 * q < nv ? 0x0000ffffu : 0u);
          vf[dt][q] &= keep;
        }
      }
    }

    f32x4 s[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) s[mt] = mfma_bf16(kf[mt][ks], qf[ks], s[mt]);
    }

    // lane (col, rg) holds position tile + rg*8 + mt*4 + i in s[mt][i]
    float sv[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = s[mt][i];
        const float sum = v + dpp<kShlNr>(v);            // hi + lo, valid in cols 0 .. NR-1
        const float bc = dpp<kShrNr>(sum);               // copy to cols NR .. 2NR-1
        const float full = (col < NR) ? sum : bc;
        const int j = jv + mt * 4 + i;
        sv[mt * 4 + i] = (j < j_end) ? full : -INFINITY;
        tmax = fmaxf(tmax, sv[mt * 4 + i]);
      }
    }
    tmax = max_xor32(max_xor16(tmax));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = valid_col ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
    float psum = 0.f;
    uint32_t pk[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float p0 = __builtin_amdgcn_exp2f(sv[2 * q] - m_new);
      const float p1 = __builtin_amdgcn_exp2f(sv[2 * q + 1] - m_new);
      psum += p0 + p1;
      uint32_t h0 = f32_to_bf16_bits(p0), h1 = f32_to_bf16_bits(p1);
      if (is_lo) {
        h0 = f32_to_bf16_bits(p0 - bf16_bits_to_f32(h0));
        h1 = f32_to_bf16_bits(p1 - bf16_bits_to_f32(h1));
      }
      pk[q] = valid_col ? (h0 | (h1 << 16)) : 0u;
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    const u32x4 pf = {pk[0], pk[1], pk[2], pk[3]};
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      oacc[dt] *= alpha;
      oacc[dt] = mfma_bf16(vf[dt], pf, oacc[dt]);
    }
  };

  // Fused schedule: the workgroup polls Q of its 4 heads (4 x 128 floats,
  // written by the head's QKV workgroups of this launch) with device-scope
  // loads until no word holds the "not yet" marker: the poll that succeeds
  // is the read.  The head's nsplit*B attention workgroups count themselves once
  // they have read Q and the appended row; the last writes the markers back
  // and rearms the counter (release_inputs).  A workspace without
  // gqa_workspace_init's magic word holds no valid markers: the workgroup
  // records the error and stops (the wo workgroups see the same and write
  // NaN).  A poll that runs out records its error and poisons Q with NaN, so
  // that Delta turns NaN.
  auto poll_q = [&]() {
    // thread i polls floats 2i, 2i+1 of the NR heads' Q (NR x 128 floats),
    // then leaves them in LDS for every wave
    if (2 * tid < NR * HD) {
      const float* qsrc = p.q + (size_t)b * D + g * NR * HD + 2 * tid;
      float2 v = make_float2(0.f, 0.f);
      for (int polls = 0;; ++polls) {
        v = make_float2(ld_dev(qsrc), ld_dev(qsrc + 1));
        if (__float_as_uint(v.x) != kNotYet && __float_as_uint(v.y) != kNotYet) break;
        if (polls >= kMaxPolls) {
          __hip_atomic_fetch_or(p.sync + kSyncErr, GQA_WS_ERR_WAIT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          v = make_float2(__uint_as_float(0xffffffffu), __uint_as_float(0xffffffffu));
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      *reinterpret_cast<float2*>(sm_q + 2 * tid) = v;
    }
    __syncthreads();
  };

  // the first tile's loads go out before the Q polls, so both round trips overlap
  if (tile0 < j_end) load_tile(tile0, kf, vf);
  if (FUSED) {
    if (tid == 0) {
      int state = 0;
      if (p.sync[kSyncMagic] != kWsMagic) {
        __hip_atomic_fetch_or(p.sync + kSyncErr, GQA_WS_ERR_INIT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        state = 2;
      } else if (blk == 0 && xcc_id() != g) {
        // placement diagnostic, once per launch: the first attention
        // workgroup counts the launch if the dispatcher put it away from XCD
        // g (results are unaffected)
        __hip_atomic_fetch_add(p.sync + kSyncOffHome, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      *sm_last = state;
    }
    __syncthreads();
    if (*sm_last == 2) return;
    poll_q();
    if (tile0 < j_end) patch_tile(tile0, kf, vf);
  }
  build_q();
  m_run = -INFINITY;
  l_run = 0.f;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One tile in registers per wave; latency is hidden by the other waves
  // resident on the SIMD (the kernel is sized for 3 waves per SIMD).
  int tile = tile0;
  while (tile < j_end) {
    compute_tile(tile, kf, vf);
    tile += kAttnWaves * kAttnTile;
    if (tile < j_end) {
      load_tile(tile, kf, vf);
      if (FUSED) patch_tile(tile, kf, vf);
    }
  }

  // wave result: l summed over the 4 lane rows, O = hi column + lo column
  l_run = sum_xor32(sum_xor16(l_run));
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = oacc[dt][i];
      const float o = v + dpp<kShlNr>(v);
      if (col < NR) sm_o[w][col][rg * 4 + i + 16 * dt] = o;
    }
  }
  if (lane < NR) {
    sm_m[w][lane] = m_run;
    sm_l[w][lane] = l_run;
  }
  __syncthreads();
  // every wave of the workgroup is past its reads of Q and the appended row
  if (FUSED && tid == 0) grp_prev = __hip_atomic_fetch_add(grp_cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // merge the 4 waves: thread -> (head, two dims); wave w takes head w (the
  // waves past NR only join the barriers)
  const int mh = tid >> 6, d2 = (tid & 63) * 2;
  const bool merges = mh < NR;
  const int mhc = merges ? mh : 0;
  float M = -INFINITY;
#pragma unroll
  for (int ww = 0; ww < kAttnWaves; ++ww) M = fmaxf(M, sm_m[ww][mhc]);
  float lsum = 0.f, o0 = 0.f, o1 = 0.f;
#pragma unroll
  for (int ww = 0; ww < kAttnWaves; ++ww) {
    const float f = __builtin_amdgcn_exp2f(sm_m[ww][mhc] - M);
    lsum += sm_l[ww][mhc] * f;
    o0 += sm_o[ww][mhc][d2] * f;
    o1 += sm_o[ww][mhc][d2 + 1] * f;
  }

  const size_t out_off = (size_t)b * D + (g * NR + mhc) * HD + d2;
  // O of (b, g) leaves as bf16 hi/lo parts; in the fused schedule through
  // device-scope stores, after which every wo workgroup is told
  auto emit = [&](float r0, float r1) {
    const uint32_t h0 = f32_to_bf16_bits(r0), h1 = f32_to_bf16_bits(r1);
    const uint32_t lo0 = f32_to_bf16_bits(r0 - bf16_bits_to_f32(h0));
    const uint32_t lo1 = f32_to_bf16_bits(r1 - bf16_bits_to_f32(h1));
    uint32_t* ph = reinterpret_cast<uint32_t*>(p.o_hi + out_off);
    uint32_t* pl = reinterpret_cast<uint32_t*>(p.o_lo + out_off);
    if (FUSED) {
      // every thread of the workgroup reaches the barrier (the waves past
      // NR store nothing)
      if (merges) {
        st_dev(ph, h0 | (h1 << 16));
        st_dev(pl, lo0 | (lo1 << 16));
      }
      wait_vm();
      __syncthreads();
      for (int wg = tid; wg < kFusedWoWG; wg += blockDim.x)
        st_dev(p.wo_slots + kFusedSlotWords * wg + b * KV + g, 1);
    } else if (merges) {
      *ph = h0 | (h1 << 16);
      *pl = lo0 | (lo1 << 16);
    }
  };

  // The head's last attention workgroup to count itself (every other one has
  // read Q and the appended row, so every producer's store has landed) writes
  // the markers back into Q of the head's query heads and into the appended
  // rows of every sequence, then rearms the counter; wave 0 does it.
  auto release_inputs = [&]() {
    if (!FUSED || w != 0) return;
    if (__shfl(grp_prev, 0) != p.nsplit * p.B - 1) return;
    for (int bb = 0; bb < p.B; ++bb) {
      float* qg = p.q + (size_t)bb * D + g * NR * HD;
#pragma unroll
      for (int i = 0; i < NR * HD / 64; ++i) st_dev(qg + i * 64 + lane, __uint_as_float(kNotYet));
#pragma unroll
      for (int kvp = 0; kvp < 2; ++kvp)
        st_dev(p.kv_new + ((size_t)(bb * 2 + kvp) * KV + g) * (HD / 2) + lane, kNotYetPair);
    }
    if (lane == 0) st_dev(grp_cnt, 0);
  };

  if (p.nsplit == 1) {
    emit(o0 / lsum, o1 / lsum);
    release_inputs();
    return;
  }

  // Each (sequence, kv head) owns a whole number of 128-byte lines of
  // partials: per split and head m, l, two unused words, o[128].
  const size_t split_stride = (size_t)NR * kPartStride;
  float* part0 = p.part + (size_t)(b * KV + g) * part_region_floats(p.nsplit, NR) +
                 (size_t)mhc * kPartStride;
  float* mine = part0 + (size_t)split * split_stride;

  // merge every split in a fixed order, one round trip per 8 splits,
  // rescaling the running sums as the maximum grows; get(s, mv, lv, ov0, ov1)
  // supplies split s (false: not there yet, ask again)
  constexpr int U = 8;
  auto merge_splits = [&](auto get) {
    float GM = -INFINITY, gl = 0.f, g0 = 0.f, g1 = 0.f;
    for (int s0 = 0; s0 < p.nsplit; s0 += U) {
      float mv[U], lv[U], ov0[U], ov1[U];
      for (int polls = 0;; ++polls) {
        bool ok = true;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int s = s0 + u;
          if (s >= p.nsplit) {
            mv[u] = -INFINITY; lv[u] = 0.f; ov0[u] = 0.f; ov1[u] = 0.f;
          } else {
            ok &= get(s, mv[u], lv[u], ov0[u], ov1[u]);
          }
        }
        if (ok) break;
        if (polls >= kMaxPolls) {
          __hip_atomic_fetch_or(p.sync + kSyncErr, GQA_WS_ERR_WAIT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
          for (int u = 0; u < U; ++u) mv[u] = __uint_as_float(0x7fc00000u);
          break;
        }
        // no sleep between these polls: one workgroup per (sequence, kv
        // head) polls, and asking again at once measured faster
      }
      float cm = GM;
#pragma unroll
      for (int u = 0; u < U; ++u) cm = fmaxf(cm, mv[u]);
      const float r = __builtin_amdgcn_exp2f(GM - cm);
      gl *= r;
      g0 *= r;
      g1 *= r;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float f = __builtin_amdgcn_exp2f(mv[u] - cm);
        gl += lv[u] * f;
        g0 += ov0[u] * f;
        g1 += ov1[u] * f;
      }
      GM = cm;
    }
    emit(g0 / gl, g1 / gl);
  };

  if (FUSED) {
    // The last split merges.  The others publish their partial with
    // device-scope stores into words that hold the "not yet" marker (8 bytes
    // a store: m with l, and each thread's two values of o; the merger checks
    // every 4-byte half, so a load that sees one store half landed only asks
    // again) and are done; the merging workgroup polls those words itself
    // (arrival and value in one round trip), takes its own partial from
    // registers, and writes the markers back once every thread has read
    // them.  Every path releases the head's inputs last: release_inputs
    // waits for the head counter's atomic, which should not hold up the
    // partials or O.
    if (split != p.nsplit - 1) {
      if (merges) {
        if (d2 == 0)
          st_dev(reinterpret_cast<uint64_t*>(mine),
                 (uint64_t)__float_as_uint(M) | ((uint64_t)__float_as_uint(lsum) << 32));
        st_dev(reinterpret_cast<uint64_t*>(mine + 4 + d2),
               (uint64_t)__float_as_uint(o0) | ((uint64_t)__float_as_uint(o1) << 32));
      }
      release_inputs();
      return;
    }
    merge_splits([&](int s, float& mv, float& lv, float& ov0, float& ov1) {
      if (s == split) {
        mv = M; lv = lsum; ov0 = o0; ov1 = o1;
        return true;
      }
      const float* ps = part0 + (size_t)s * split_stride;
      const uint64_t ml = __hip_atomic_load(reinterpret_cast<const uint64_t*>(ps), __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
      const uint64_t oo = __hip_atomic_load(reinterpret_cast<const uint64_t*>(ps + 4 + d2),
                                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      mv = __uint_as_float((uint32_t)ml);
      lv = __uint_as_float((uint32_t)(ml >> 32));
      ov0 = __uint_as_float((uint32_t)oo);
      ov1 = __uint_as_float((uint32_t)(oo >> 32));
      return __float_as_uint(mv) != kNotYet && __float_as_uint(lv) != kNotYet &&
             __float_as_uint(ov0) != kNotYet && __float_as_uint(ov1) != kNotYet;
    });
    // emit's barrier: every thread has read every partial
    if (merges) {
      for (int s = 0; s < p.nsplit - 1; ++s) {
        float* ps = part0 + (size_t)s * split_stride;
        const uint64_t nn = (uint64_t)kNotYet | ((uint64_t)kNotYet << 32);
        if (d2 == 0) st_dev(reinterpret_cast<uint64_t*>(ps), nn);
        st_dev(reinterpret_cast<uint64_t*>(ps + 4 + d2), nn);
      }
    }
    release_inputs();
    return;
  }

  // Three-launch schedule: publish this split's partial with device-scope
  // stores (through to the coherence point shared by all XCDs, without an L2
  // write-back), wait for them to land, then count it; the last workgroup to
  // arrive merges every partial.  The counter lives at the device-wide
  // coherence point (atomics are performed there, and the partials are read
  // with device-scope loads).
  int* split_cnt = p.counters + b * KV + g;
  if (merges) {
    if (d2 == 0) {
      st_dev(mine, M);
      st_dev(mine + 1, lsum);
    }
    st_dev(mine + 4 + d2, o0);
    st_dev(mine + 5 + d2, o1);
  }
  wait_vm();
  __syncthreads();
  if (tid == 0) {
    const int prev = __hip_atomic_fetch_add(split_cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *sm_last = (prev == p.nsplit - 1);
  }
  __syncthreads();
  if (!*sm_last) return;
  if (tid == 0) st_dev(split_cnt, 0);
  merge_splits([&](int s, float& mv, float& lv, float& ov0, float& ov1) {
    const float* ps = part0 + (size_t)s * split_stride;
    mv = ld_dev(ps);
    lv = ld_dev(ps + 1);
    ov0 = ld_dev(ps + 4 + d2);
    ov1 = ld_dev(ps + 5 + d2);
    return true;
  });
}

template <int KV>
__global__ void __launch_bounds__(256, 3) decode_attn_kernel(DecodeParams p) {
  __shared__ float lds[attn_lds_words(H / KV)];
  attn_body<false, KV>(p, blockIdx.x, lds);
}

// ---------------------------------------------------------------------------
// wo projection (+ residual)
// ---------------------------------------------------------------------------

// Output features (f, f+1) of token b: out = Delta, out += Delta
// (accumulate) or out = resid + Delta (layer), and the bf16 copy; NaN when
// the producer's wait failed.
__device__ __forceinline__ void wo_emit_pair(const DecodeParams& p, int b, int f, float v0, float v1,
                                             bool failed) {
  float2* o = reinterpret_cast<float2*>(p.out + (size_t)b * D + f);
  float2 r = make_float2(v0, v1);
  if (p.accumulate) {
    const float2 prev = *o;
    r.x += prev.x;
    r.y += prev.y;
  } else if (p.resid) {
    const uint32_t xr = *reinterpret_cast<const uint32_t*>(p.resid + (size_t)b * D + f);
    r.x += bf16_bits_to_f32(xr & 0xffffu);
    r.y += bf16_bits_to_f32(xr >> 16);
  }
  if (failed) r = make_float2(__uint_as_float(0x7fc00000u), __uint_as_float(0x7fc00000u));
  *o = r;
  if (p.out_bf16)
    *reinterpret_cast<uint32_t*>(p.out_bf16 + (size_t)b * D + f) = pack_bf16x2(r.x, r.y);
}

// KV: kv heads of the fused schedule's attention (one O-ready word per
// (sequence, kv head) in the workgroup's slot).
template <int NB, bool FUSED, int W = 4, int KV = KVH>
__device__ __forceinline__ void wo_body(const DecodeParams& p, int b0, int blk, uint32_t* xs) {
  static_assert(!FUSED || W == 4, "the fused schedule's wo roles are 4-wave workgroups");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r0 = (blk * W + wave) * 2;
  u32x4 wa[8], wb[8];
  if (FUSED) {
    // hold the weight stream back while QKV finishes (fused_wo_hold_ticks)
    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    while (__builtin_amdgcn_s_memrealtime() - t0 < fused_wo_hold_ticks(KV)) __builtin_amdgcn_s_sleep(8);
  } else {
    // O (hi and lo parts) goes to LDS by direct loads ahead of the weights
    stage_rows_async<NB, W>(xs, p.o_hi + (size_t)b0 * D);
    stage_rows_async<NB, W>(xs + NB * (D / 2), p.o_lo + (size_t)b0 * D);
  }
  load_rows2(p.wo + (size_t)r0 * D, p.wo + (size_t)(r0 + 1) * D, lane, wa, wb);
  if (!FUSED) {
    wait_loads_except<16>();
    lds_barrier();
  }
  // fused: 0 normal, 1 the wait timed out, 2 the workspace is uninitialised;
  // in either error case this workgroup's outputs are NaN
  __shared__ int wo_state;
  if (FUSED) {
    // wave 0 waits until every (b, g) has published O, one word per lane
    if (wave == 0) {
      int state = 0;
      if (p.sync[kSyncMagic] != kWsMagic) {
        if (lane == 0) __hip_atomic_fetch_or(p.sync + kSyncErr, GQA_WS_ERR_INIT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        state = 2;
      } else {
        int* slot = p.wo_slots + kFusedSlotWords * blk;
        const int nwords = p.B * KV;
        static_assert(kFusedSlotWords <= 64, "one word per lane");
        int polls = 0;
        while (true) {
          const int v = lane < nwords ? ld_dev(slot + lane) : 1;
          if (__all(v == 1)) break;
          __builtin_amdgcn_s_sleep(1);
          if (++polls > kMaxPolls) {
            if (lane == 0) __hip_atomic_fetch_or(p.sync + kSyncErr, GQA_WS_ERR_WO_WAIT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            state = 1;
            break;
          }
        }
        if (lane < nwords) st_dev(slot + lane, 0);
      }
      if (lane == 0) wo_state = state;
    }
    __syncthreads();
    if (wo_state == 2) {
      // no O to read: NaN outputs, the error word says why
      if (lane < NB) {
        const float nan = __uint_as_float(0x7fc00000u);
        *reinterpret_cast<float2*>(p.out + (size_t)(b0 + lane) * D + r0) = make_float2(nan, nan);
        if (p.out_bf16) *reinterpret_cast<uint32_t*>(p.out_bf16 + (size_t)(b0 + lane) * D + r0) = 0x7fc07fc0u;
      }
      return;
    }
    // every load goes out before the first LDS write (one round trip); no
    // workgroup reads O before all of it is complete, so the first reader on
    // each XCD fetches a line into its L2 and the rest of the XCD's wo
    // workgroups hit it
    constexpr int kPer = NB * (D / 8) / 256;       // 16-byte pieces per thread and part
    u32x4 hv[kPer], lv[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const uint32_t off = (uint32_t)(((size_t)b0 * D) * 2 + (threadIdx.x + 256 * k) * 16);
      hv[k] = ld_xcd_x4(p.o_hi, off);
      lv[k] = ld_xcd_x4(p.o_lo, off);
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      reinterpret_cast<u32x4*>(xs)[threadIdx.x + 256 * k] = hv[k];
      reinterpret_cast<u32x4*>(xs + NB * (D / 2))[threadIdx.x + 256 * k] = lv[k];
    }
    __syncthreads();
  }

  float acc[2][NB];
  gemv_rows2<NB, 2>(wa, wb, xs, lane, acc);

  float v0 = 0.f, v1 = 0.f;
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    const float s0 = wave_sum(acc[0][t]);
    const float s1 = wave_sum(acc[1][t]);
    if (lane == t) { v0 = s0; v1 = s1; }
  }
  if (lane < NB) wo_emit_pair(p, b0 + lane, r0, v0, v1, FUSED && wo_state == 1);
}

// Up to 4 tokens (5 to 8 run on the matrix cores, decode_wo_mfma_kernel).
template <int NB, int W>
__global__ void __launch_bounds__(64 * W) decode_wo_kernel(DecodeParams p, int b0) {
  __shared__ uint32_t xs[2 * NB * (D / 2)];
  wo_body<NB, false, W>(p, b0, blockIdx.x, xs);
}

// ---------------------------------------------------------------------------
// wo of 5 to 8 tokens on the matrix cores
// ---------------------------------------------------------------------------
//
// At 8 tokens the wo GEMV spends 1024 packed dot instructions per lane (the
// hi and lo parts of O) on each pair of weight rows, with the LDS reads that
// feed them, and that vector work lands behind the weight stream instead of
// under it (15.5 us at 8 tokens against 10.5 us at 2).  Here the products
// run on v_mfma_f32_16x16x32_bf16, C^T[16 rows x 16 columns] = Wo . X^T:
//  - a workgroup owns 16 consecutive rows of Wo and its wave w the K range
//    [1024w, 1024w + 1024); the wave's 32 A fragments (lane l: row l % 16,
//    the 8 consecutive k at 8 (l / 16) of each 32-k step) all go out at
//    once, 32 KiB a wave, the whole weight in flight in one pass;
//  - the columns are the tokens' hi parts followed by their lo parts,
//    staged in LDS by direct loads issued before the weights, each row
//    padded by 16 bytes so that the B fragments (lane l: 8 consecutive k of
//    column l % 16) fall on distinct banks; columns past the staged rows
//    repeat row 0 and are dropped;
//  - the 4 waves' partial tiles are summed in LDS in a fixed order, and each
//    output adds its hi and lo columns.
// (The same layout for the QKV projection measured no faster than its GEMV:
// the A fragments read 64 bytes of 16 rows per instruction, and the stream
// ran at about 2.8 TB/s against the GEMV's whole-row kilobytes.)
constexpr int kWoMfmaMinNB = 5;                  // fewer tokens stay on the GEMV
constexpr int kSkPitch = D / 2 + 4;              // u32 words per staged row
template <int NB>
constexpr size_t wo_mfma_lds_bytes() {
  return ((size_t)2 * NB * kSkPitch + 4 * 16 * 16) * 4;
}

template <int NB>
__global__ void __launch_bounds__(256) decode_wo_mfma_kernel(DecodeParams p, int b0) {
  static_assert(NB >= 1 && NB <= 8, "16 columns hold 8 tokens' hi and lo parts");
  constexpr int NR = 2 * NB;                     // staged rows: hi parts, then lo parts
  extern __shared__ __attribute__((aligned(16))) uint32_t xs[];
  float* red = reinterpret_cast<float*>(xs + NR * kSkPitch);   // [wave][16 rows][16 columns]
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int f0 = blockIdx.x * 16;

  stage_rows_async<NB, 4, kSkPitch>(xs, p.o_hi + (size_t)b0 * D);
  stage_rows_async<NB, 4, kSkPitch>(xs + NB * kSkPitch, p.o_lo + (size_t)b0 * D);
  const uint16_t* wk = p.wo + (size_t)(f0 + (lane & 15)) * D + 1024 * wave + 8 * (lane >> 4);
  u32x4 a[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) a[k] = ld_u32x4(wk + 32 * k);
  wait_loads_except<32>();
  lds_barrier();

  const int col = lane & 15;
  const uint32_t* xb = xs + (col < NR ? col : 0) * kSkPitch + 512 * wave + 4 * (lane >> 4);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < 32; ++k) acc = mfma_bf16(a[k], *reinterpret_cast<const u32x4*>(xb + 16 * k), acc);
  // lane l holds rows 4 (l / 16) + i of column l % 16
#pragma unroll
  for (int i = 0; i < 4; ++i) red[(wave * 16 + 4 * (lane >> 4) + i) * 16 + col] = acc[i];
  lds_barrier();
  auto total = [&](int m, int c) {
    return ((red[m * 16 + c] + red[(16 + m) * 16 + c]) + red[(32 + m) * 16 + c]) + red[(48 + m) * 16 + c];
  };
  // rows (2j, 2j+1) of token t: hi column t plus lo column NB + t
  const int j = threadIdx.x & 7, t = threadIdx.x >> 3;
  if (t < NB) {
    const float v0 = total(2 * j, t) + total(2 * j, NB + t);
    const float v1 = total(2 * j + 1, t) + total(2 * j + 1, NB + t);
    wo_emit_pair(p, b0 + t, f0 + 2 * j, v0, v1, false);
  }
}

// ---------------------------------------------------------------------------
// Fused schedule: the whole block step in one launch
// ---------------------------------------------------------------------------
//
// Workgroups [0, fused_qkv_wg(KV)) run the QKV projection (768 at 8 kv
// heads), the next nsplit*KV*B the flash-decode, the last 512 wo.  Dispatch
// follows the workgroup index and the QKV workgroups fill the chip (3 per
// CU at 8 kv heads), so they stream their weights from the start; the
// attention and wo workgroups take the places of retiring QKV ones.
// (Attention first measured slower: the QKV workgroups it displaced started
// late and stretched the QKV stream.)  Kv head g takes the QKV and attention
// workgroups with i = g (mod KV).  Each consumer starts its own HBM reads
// (K/V tiles, wo rows) before it waits, so the three phases overlap instead
// of paying a launch boundary each:
//   QKV -> attention: Q and the new row are stored into words that hold a
//     "not yet" marker; the head's attention workgroups poll the words
//     themselves, so arrival and value come in one round trip, and the last
//     of them (a per-head count) writes the markers back;
//   split -> merge: the splits but the last store their partials into marked
//     words and end; the last split polls them, merges in a fixed order and
//     restores the markers;
//   attention -> wo: the merging workgroup stores O of (b, g) with
//     device-scope stores and sets word b*KV + g of every wo workgroup's
//     slot.
// Producers that signal through a separate word wait for their stores to
// complete first; slots and marked words are polled with
// device-scope loads.  Every wait is bounded (kMaxPolls) and only the
// consumers wait.  The host admits a shape only if
// all waiting workgroups together fit in less than the chip's resident
// capacity, so producers always find room to run whatever order the hardware
// dispatches in.
template <int NB, int KV>
__global__ void __launch_bounds__(256, 3) decode_step_kernel(DecodeParams p) {
  __shared__ uint32_t lds[2 * NB * (D / 2) > kAttnLdsWords ? 2 * NB * (D / 2) : kAttnLdsWords];
  static_assert(kFusedAttnQWord + REP * HD <= sizeof(lds) / 4, "no LDS for the attention role's Q");
  constexpr int nqkv = fused_qkv_wg(KV);
  const int na = p.nsplit * KV * p.B;
  const int blk = blockIdx.x;
  if (blk < nqkv) {
    qkv_body<NB, true, KV>(p, 0, blk, lds);
  } else if (blk < nqkv + na) {
    attn_body<true, KV>(p, blk - nqkv, reinterpret_cast<float*>(lds));
  } else {
    wo_body<NB, true, 4, KV>(p, 0, blk - nqkv - na, lds);
  }
}

// ---------------------------------------------------------------------------
// Batched decode projections on the matrix cores
// ---------------------------------------------------------------------------
//
// Above 8 tokens the weights are streamed once through
// v_mfma_f32_16x16x32_bf16 as a split-K GEMM, C^T[features x columns] +=
// W[features x k] . X^T[k x columns]:
//  - workgroup (fb, ks) owns 128 output features and one of KS equal K
//    ranges (KS = 4 for QKV, 8 for wo); its 4 waves own 32 features each
//    (two 16-row A tiles);
//  - the activation columns (up to 64 per launch) of the workgroup's whole K
//    range are copied into LDS first (global_load_lds, 128 KiB) and read by
//    all 4 waves as the B operand, so each activation byte leaves L2 once per
//    workgroup.  Each wave's weight rows come straight from HBM into
//    registers (its A operand) in chunks of 128 K, three chunks ahead; after
//    the one barrier for the activations the waves run unsynchronised;
//  - the KS K ranges of a feature block are summed by the last of its KS
//    workgroups to finish (device-scope partials and counter, fixed order),
//    which then runs the epilogue.
// The K ranges alternate with the workgroup index, so that workgroups the
// dispatcher's round-robin puts on one XCD (i % 8 on an idle chip) read the
// same activation range from its L2; a locality heuristic only.
// Columns are tokens.  For wo the input O is the sum of two bf16 parts: each
// weight fragment multiplies both parts into the same accumulator.
// QKV epilogue of one column (token b) and features f .. f+3 (one head):
// RoPE on Q/K pairs with the table entries cs0 (pair f/2) and cs1 (pair
// f/2 + 1), Q to the workspace, K/V rounded into the cache.
template <int KV>
__device__ __forceinline__ void proj_qkv_store(const DecodeParams& p, f32x4 v, int b, int f,
                                               float2 cs0, float2 cs1) {
  const int pos = p.start_pos;
  float y[4] = {v[0], v[1], v[2], v[3]};
  if (f < D + KV * HD) {
    const float2 cs[2] = {cs0, cs1};
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      const float a = y[e] * cs[e / 2].x - y[e + 1] * cs[e / 2].y;
      const float bb = y[e] * cs[e / 2].y + y[e + 1] * cs[e / 2].x;
      y[e] = a;
      y[e + 1] = bb;
    }
  }
  if (p.probe)
    *reinterpret_cast<float4*>(p.probe + (size_t)b * (D + 2 * KV * HD) + f) = make_float4(y[0], y[1], y[2], y[3]);
  if (f < D) {
    *reinterpret_cast<float4*>(p.q + (size_t)b * D + f) = make_float4(y[0], y[1], y[2], y[3]);
  } else if (f < D + KV * HD) {
    const int ff = f - D, g = ff / HD, d = ff % HD;
    uint16_t* dst = p.kcache + ((size_t)(b * KV + g) * p.T_max + pos) * HD + d;
    *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
  } else {
    const int ff = f - D - KV * HD, g = ff / HD, d = ff % HD;
    uint16_t* dst = p.vcache + vcache_index(b, g, pos, d, p.T_max, KV);
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[e * VB] = (uint16_t)f32_to_bf16_bits(y[e]);
  }
}
constexpr int kP2Kc = 128;                   // K per chunk
// 16-row matrix-core tiles per wave: 2, so a 4-wave workgroup owns 128
// features.  One tile per wave with twice the workgroups, or twice the K
// splits, measured no faster at B = 64 (the chunk chain and the split-K
// tail, not the workgroup count, set the time).
template <int MODE>
constexpr int p2_tiles() { return 2; }
// features per workgroup
template <int MODE>
constexpr int p2_feat() { return 64 * p2_tiles<MODE>(); }
// K splits: 4 for QKV (192 workgroups), 8 for wo (256 workgroups)
template <int MODE>
constexpr int p2_splits() { return MODE == 0 ? 4 : 8; }
constexpr int kP2CntStride = 16;             // ints between split-K counters
constexpr int kP2Cols = 64;                  // columns per launch
constexpr int kP2Ring = 4;                   // weight chunks in flight: loaded 3 ahead
// dynamic LDS of a projection workgroup: the activations' whole K range
template <int MODE>
constexpr size_t p2_lds_bytes() { return (size_t)(MODE == 0 ? 1 : 2) * kP2Cols * (D / p2_splits<MODE>()) * 2; }

// 16-byte device-scope store at base + byte_off (base wave-uniform).
__device__ __forceinline__ void st_dev_x4(void* base, uint32_t byte_off, u32x4 v) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7fffffff, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, 16);
}

// KV: key/value heads of the QKV projection (MODE 0): 4096 + 2*KV*128 features.
template <int MODE, int KV = KVH>   // MODE 0: QKV + RoPE + cache append, 1: wo (+ residual)
__global__ void __launch_bounds__(256) decode_proj_kernel(DecodeParams p, int c_base) {
  constexpr int NP = MODE == 0 ? 1 : 2;        // activation parts (wo: hi, lo)
  constexpr int FT = p2_tiles<MODE>();         // 16-row weight tiles per wave
  constexpr int kP2Feat = p2_feat<MODE>();
  constexpr int kP2KS = p2_splits<MODE>();
  constexpr int kP2Kr = D / kP2KS;             // K range of a workgroup
  constexpr int kP2Chunks = kP2Kr / kP2Kc;
  // [NP][64 rows][kP2Kr] bf16, dynamic
  extern __shared__ __attribute__((aligned(16))) uint16_t sx_dyn[];
  __shared__ int sm_last;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int ks = blockIdx.x % kP2KS, fb = blockIdx.x / kP2KS;
  const int ncols = min(kP2Cols, p.B - c_base);
  const int kbase = ks * kP2Kr;
  if (p.sync[kSyncMagic] != kWsMagic) {
    // uninitialised workspace: the split-K counters cannot be trusted; the
    // error word says so and the output projection writes NaN
    if (tid == 0) __hip_atomic_fetch_or(p.sync + kSyncErr, GQA_WS_ERR_INIT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (MODE == 1 && ks == 0) {
      for (int i = tid; i < ncols * kP2Feat; i += 256) {
        const size_t o = (size_t)(c_base + i / kP2Feat) * D + fb * kP2Feat + i % kP2Feat;
        p.out[o] = __uint_as_float(0x7fc00000u);
        if (p.out_bf16) p.out_bf16[o] = 0x7fc0u;
      }
    }
    return;
  }
  if (MODE == 0 && blockIdx.x == 0 && c_base == 0) {
    // the attention kernel that follows counts split arrivals from zero
    for (int i = tid; i < p.B * KV; i += blockDim.x) p.counters[i] = 0;
  }

  // A operand: weight row of tile ft, k offset (lane >> 4) * 8 in each step
  const uint16_t* wrow[FT];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    const int f = fb * kP2Feat + 16 * FT * w + 16 * ft + (lane & 15);
    if (MODE == 0)
      wrow[ft] = (f < D ? p.wq + (size_t)f * D
                        : (f < D + KV * HD ? p.wk + (size_t)(f - D) * D
                                           : p.wv + (size_t)(f - D - KV * HD) * D)) +
                 kbase + (lane >> 4) * 8;
    else
      wrow[ft] = p.wo + (size_t)f * D + kbase + (lane >> 4) * 8;
  }

  // The activation columns' whole K range goes to LDS once, first:
  // [NP][64 rows][kP2Kr] bf16, 16-byte unit u of row r at physical unit
  // u ^ (r & 7).  Copy instruction i of a part fills bytes [1 KiB i, 1 KiB
  // (i+1)); lane l writes the unit l of that KiB.
  constexpr int kRowUnits = kP2Kr / 8;                      // 16-byte units a row
  constexpr int kCopies = kP2Cols * kP2Kr * 2 / 1024;       // per part
  static_assert(kCopies % 4 == 0, "each wave issues the same number of copies");
#pragma unroll
  for (int part = 0; part < NP; ++part) {
    const uint16_t* base = MODE == 0 ? p.x : (part == 0 ? p.o_hi : p.o_lo);
#pragma unroll
    for (int j = 0; j < kCopies / 4; ++j) {
      const int i = 4 * j + w;
      const int unit = i * 64 + lane;                       // physical, over the part
      const int row = unit / kRowUnits;
      const int lu = (unit % kRowUnits) ^ (row & 7);
      const int col = c_base + min(row, ncols - 1);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(base + (size_t)col * D + kbase + lu * 8),
                                       (lds_void*)(sx_dyn + (part * kP2Cols * kP2Kr) + i * 512), 16, 0, 0);
    }
  }
  // the wait counts below assume every copy is issued before any weight load
  asm volatile("" ::: "memory");

  u32x4 wb[kP2Ring][FT][4];                     // [ring slot][tile][k-step]
  auto load_w = [&](int chunk, u32x4 (&dst)[FT][4]) {
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
#pragma unroll
      for (int s = 0; s < 4; ++s) dst[ft][s] = ld_u32x4(wrow[ft] + chunk * kP2Kc + s * 32);
  };

  f32x4 acc[FT][4];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[ft][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Each wave's weight chunks stream kP2Ring - 1 ahead (4 FT loads each).
  // Chunk c has landed once no more than the loads of the chunks issued after
  // it remain in flight; the activations, issued before all of them, have
  // landed once the first kP2Ring - 1 chunks alone remain.  One barrier (for
  // the activations) and no other: each wave then runs at its own pace.
  constexpr int kPerChunk = 4 * FT;
  constexpr int kAhead = kP2Ring - 1 < kP2Chunks ? kP2Ring - 1 : kP2Chunks;   // chunks loaded first
  static_assert(kAhead * kPerChunk < 64, "vmcnt counts to 63");
#pragma unroll
  for (int c = 0; c < kAhead; ++c) {
    load_w(c, wb[c]);
    asm volatile("" ::: "memory");            // chunks leave in order
  }
  wait_loads_except<kAhead * kPerChunk>();
  lds_barrier();
#pragma unroll
  for (int c = 0; c < kP2Chunks; ++c) {
    const int later = min(kP2Ring - 2, kP2Chunks - 1 - c);    // chunks issued after c
    if (later >= 4) wait_loads_except<4 * kPerChunk>();
    else if (later == 3) wait_loads_except<3 * kPerChunk>();
    else if (later == 2) wait_loads_except<2 * kPerChunk>();
    else if (later == 1) wait_loads_except<kPerChunk>();
    else wait_loads_except<0>();
    if (c + kP2Ring - 1 < kP2Chunks) {
      load_w(c + kP2Ring - 1, wb[(c + kP2Ring - 1) % kP2Ring]);
      asm volatile("" ::: "memory");          // issued before this chunk's matrix work
    }
    // all of the chunk's B fragments of a part are read before its matrix
    // work, so the LDS reads overlap one another (column tiles past ncols
    // read rows of the copy that clamped onto the last column; their
    // results are never stored)
#pragma unroll
    for (int part = 0; part < NP; ++part) {
      u32x4 xb[4][4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int row = 16 * t + (lane & 15);
          const int lu = c * (kP2Kc / 8) + 4 * s + (lane >> 4);
          const int off = part * kP2Cols * kP2Kr + row * kP2Kr + ((lu ^ (row & 7)) << 3);
          xb[s][t] = *reinterpret_cast<const u32x4*>(sx_dyn + off);
        }
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int ft = 0; ft < FT; ++ft) acc[ft][t] = mfma_bf16(wb[c % kP2Ring][ft][s], xb[s][t], acc[ft][t]);
    }
  }

  // partials [fb][ks][64 columns][kP2Feat features] fp32; lane holds features
  // 16 FT w + 16ft + 4(lane >> 4) + e (e < 4) of column 16t + (lane & 15)
  float* part_fb = p.part;
  const uint32_t pbase = (uint32_t)((fb * kP2KS + ks) * kP2Cols) * kP2Feat * 4u;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int col = 16 * t + (lane & 15);
    if (col >= ncols) continue;
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      const int fl = 16 * FT * w + 16 * ft + 4 * (lane >> 4);
      st_dev_x4(part_fb, pbase + (uint32_t)(col * kP2Feat + fl) * 4u,
                __builtin_bit_cast(u32x4, acc[ft][t]));
    }
  }
  wait_vm();
  __syncthreads();
  int* cnt = p.sync + kSyncProj + kP2CntStride * fb;
  if (tid == 0) {
    const int prev = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm_last = prev == kP2KS - 1;
  }
  __syncthreads();
  if (!sm_last) return;
  if (tid == 0) st_dev(cnt, 0);

  // last of the feature block: sum the K ranges in order, then the epilogue;
  // all of a thread's loads (partials, RoPE entries, the residual) go out
  // before the first is used
  constexpr int kItems = kP2Cols * (kP2Feat / 4) / 256;     // 4 FT per thread
  constexpr int kBatch = kP2KS <= 4 ? kItems : kItems / 2;  // items whose loads go out together
  const int nitems = ncols * (kP2Feat / 4);
  const float2* rrow = reinterpret_cast<const float2*>(p.rope) + (size_t)p.start_pos * PAIRS;
  for (int it0 = 0; it0 < kItems; it0 += kBatch) {
  u32x4 parts[kBatch][kP2KS];
  float4 aux[kBatch];                          // RoPE pair entries, or the residual
#pragma unroll
  for (int it = 0; it < kBatch; ++it) {
    const int i = tid + 256 * (it0 + it);
    if (i >= nitems) continue;
    const int col = i / (kP2Feat / 4), f4 = i % (kP2Feat / 4);
    const int f = fb * kP2Feat + 4 * f4;
#pragma unroll
    for (int k = 0; k < kP2KS; ++k)
      parts[it][k] = ld_dev_x4(part_fb, (uint32_t)((((fb * kP2KS + k) * kP2Cols + col) * kP2Feat) + 4 * f4) * 4u);
    if (MODE == 0) {
      // pairs (f, f+1) and (f+2, f+3): two consecutive table entries
      aux[it] = *reinterpret_cast<const float4*>(rrow + ((f & (HD - 1)) >> 1));
    } else if (p.accumulate) {
      aux[it] = *reinterpret_cast<const float4*>(p.out + (size_t)(c_base + col) * D + f);
    }
  }
#pragma unroll
  for (int it = 0; it < kBatch; ++it) {
    const int i = tid + 256 * (it0 + it);
    if (i >= nitems) continue;
    const int col = i / (kP2Feat / 4), f4 = i % (kP2Feat / 4);
    f32x4 v = __builtin_bit_cast(f32x4, parts[it][0]);
#pragma unroll
    for (int k = 1; k < kP2KS; ++k) v += __builtin_bit_cast(f32x4, parts[it][k]);
    const int b = c_base + col;
    const int f = fb * kP2Feat + 4 * f4;
    if (MODE == 0) {
      proj_qkv_store<KV>(p, v, b, f, make_float2(aux[it].x, aux[it].y), make_float2(aux[it].z, aux[it].w));
    } else {
      float4 y = make_float4(v[0], v[1], v[2], v[3]);
      if (p.accumulate) {
        y.x += aux[it].x; y.y += aux[it].y; y.z += aux[it].z; y.w += aux[it].w;
      }
      *reinterpret_cast<float4*>(p.out + (size_t)b * D + f) = y;
      if (p.out_bf16)
        *reinterpret_cast<u32x2*>(p.out_bf16 + (size_t)b * D + f) =
            u32x2{pack_bf16x2(y.x, y.y), pack_bf16x2(y.z, y.w)};
    }
  }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

int decode_max_split(int B, int kv) {
  const int pairs = B * kv;
  const int want = (1024 + pairs - 1) / pairs;
  return max(1, min(kMaxSplit, want));
}

void decode_split(int B, int L, int kv, int* nsplit, int* chunk) {
  const int per_wg = kAttnWaves * kAttnTile;
  const int by_len = (L + per_wg - 1) / per_wg;
  int n = max(1, min(by_len, decode_max_split(B, kv)));
  int c = (L + n - 1) / n;
  c = (c + kAttnTile - 1) / kAttnTile * kAttnTile;
  n = (L + c - 1) / c;
  *nsplit = n;
  *chunk = c;
}

static size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Partials: the attention splits' (m, l, o), and for B > 8 also the split-K
// partials of the projections (the two never live at the same time), sized
// for the most key/value heads.
static size_t decode_part_bytes(int B, int kv) {
  size_t n = (size_t)B * kv * part_region_floats(decode_max_split(B, kv), H / kv) * 4;
  if (B > kGemvMaxB) {
    const size_t qkv = (size_t)(D + 2 * kv * HD) * p2_splits<0>() * kP2Cols * 4;
    const size_t wo = (size_t)D * p2_splits<1>() * kP2Cols * 4;
    n = std::max(n, std::max(qkv, wo));
  }
  return n;
}

size_t decode_ws_bytes(int B, int kv) {
  size_t n = kSyncBytes;
  n += align256((size_t)B * D * 4);                       // q
  n += 2 * align256((size_t)B * D * 2);                   // o_hi, o_lo
  n += align256((size_t)B * kv * 4);                      // counters
  n += align256(decode_part_bytes(B, kv));               // partials
  return n;
}

void decode_ws_carve(void* ws, int B, int kv, DecodeParams* p) {
  char* c = static_cast<char*>(ws);
  p->sync = reinterpret_cast<int*>(c);
  c += kSyncBytes;
  p->q = reinterpret_cast<float*>(c);
  c += align256((size_t)B * D * 4);
  p->o_hi = reinterpret_cast<uint16_t*>(c);
  c += align256((size_t)B * D * 2);
  p->o_lo = reinterpret_cast<uint16_t*>(c);
  c += align256((size_t)B * D * 2);
  p->counters = reinterpret_cast<int*>(c);
  c += align256((size_t)B * kv * 4);
  p->part = reinterpret_cast<float*>(c);
}

#define GQA_NB_SWITCH(NB_VAR, CALL) \
  switch (NB_VAR) {                 \
    case 1: CALL(1); break;         \
    case 2: CALL(2); break;         \
    case 3: CALL(3); break;         \
    case 4: CALL(4); break;         \
    case 5: CALL(5); break;         \
    case 6: CALL(6); break;         \
    case 7: CALL(7); break;         \
    default: CALL(8); break;        \
  }

hipError_t launch_decode_qkv(const DecodeParams& p, hipStream_t s) {
  if (p.B > kGemvMaxB) {
    const dim3 grid((D + 2 * p.kv * HD) / p2_feat<0>() * p2_splits<0>());
    const size_t lds = p2_lds_bytes<0>();
    for (int c = 0; c < p.B; c += kP2Cols) {
      switch (p.kv) {
        case 16: hipLaunchKernelGGL((decode_proj_kernel<0, 16>), grid, dim3(256), lds, s, p, c); break;
        case 32: hipLaunchKernelGGL((decode_proj_kernel<0, 32>), grid, dim3(256), lds, s, p, c); break;
        default: hipLaunchKernelGGL((decode_proj_kernel<0, KVH>), grid, dim3(256), lds, s, p, c); break;
      }
    }
    return hipGetLastError();
  }
  for (int b0 = 0; b0 < p.B; b0 += kGemvMaxNB) {
    const int nb = min(kGemvMaxNB, p.B - b0);
    // one wave per row pair
#define GQA_LAUNCH_QKV_KV(N, KV)                                                          \
    {                                                                                     \
      constexpr int W = (N) >= 7 ? 8 : 4;                                                 \
      hipLaunchKernelGGL((decode_qkv_kernel<N, KV, W>), dim3((D + 2 * p.kv * HD) / 2 / W), \
                         dim3(64 * W), 0, s, p, b0);                                      \
    }
#define GQA_LAUNCH_QKV(N)                                     \
    switch (p.kv) {                                           \
      case 16: GQA_LAUNCH_QKV_KV(N, 16); break;               \
      case 32: GQA_LAUNCH_QKV_KV(N, 32); break;               \
      default: GQA_LAUNCH_QKV_KV(N, KVH); break;              \
    }
    GQA_NB_SWITCH(nb, GQA_LAUNCH_QKV)
#undef GQA_LAUNCH_QKV
#undef GQA_LAUNCH_QKV_KV
  }
  return hipGetLastError();
}

hipError_t launch_decode_attn(const DecodeParams& p, hipStream_t s) {
  const dim3 grid(p.nsplit * p.kv * p.B);
  switch (p.kv) {
    case 16: hipLaunchKernelGGL(decode_attn_kernel<16>, grid, dim3(256), 0, s, p); break;
    case 32: hipLaunchKernelGGL(decode_attn_kernel<32>, grid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL(decode_attn_kernel<KVH>, grid, dim3(256), 0, s, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_decode_wo(const DecodeParams& p, hipStream_t s) {
  if (p.B > kGemvMaxB) {
    for (int c = 0; c < p.B; c += kP2Cols)
      hipLaunchKernelGGL(decode_proj_kernel<1>, dim3(D / p2_feat<1>() * p2_splits<1>()), dim3(256),
                         p2_lds_bytes<1>(), s, p, c);
    return hipGetLastError();
  }
  for (int b0 = 0; b0 < p.B; b0 += kWoMaxNB) {
    const int nb = min(kWoMaxNB, p.B - b0);
#define GQA_LAUNCH_WO(N)                                                                     \
    if constexpr ((N) >= kWoMfmaMinNB) {                                                     \
      /* up to 131 KiB of dynamic LDS (gfx950 has 160 KiB; no attribute call, so */            \
      /* the launch can sit in a captured graph) */                                          \
      hipLaunchKernelGGL(decode_wo_mfma_kernel<N>, dim3(D / 16), dim3(256),                   \
                         (wo_mfma_lds_bytes<N>()), s, p, b0);                                \
    } else {                                                                                 \
      hipLaunchKernelGGL((decode_wo_kernel<N, 4>), dim3(D / 2 / 4), dim3(256), 0, s, p, b0);  \
    }
    GQA_NB_SWITCH(nb, GQA_LAUNCH_WO)
#undef GQA_LAUNCH_WO
  }
  return hipGetLastError();
}

// The fused schedule keeps every waiting workgroup (attention and wo) below
// the resident capacity of the chip: 256 CUs x 3 workgroups of 256 threads at
// the kernel's register budget, with room left for at least 128 producers.
// Its split is decode_split's, with fewer splits where that would exceed
// kFusedMaxAttnWG attention workgroups (n_rep 1 and 2 at longer contexts); a
// shape whose splits would then cover more than kFusedMaxChunk positions is
// not admitted.
bool decode_fused_split(int B, int L, int kv, int* nsplit, int* chunk) {
  if (B < 1 || B > kFusedMaxB || kv > kFusedMaxKv) return false;
  int n, c;
  decode_split(B, L, kv, &n, &c);
  const int cap = kFusedMaxAttnWG / (kv * B);
  if (n > cap) {
    n = cap;
    c = (L + n - 1) / n;
    c = (c + kAttnTile - 1) / kAttnTile * kAttnTile;
    n = (L + c - 1) / c;
  }
  if (c > kFusedMaxChunk) return false;
  *nsplit = n;
  *chunk = c;
  return true;
}

hipError_t launch_decode_fused(const DecodeParams& p0, hipStream_t s) {
  int nsplit = 0, chunk = 0;
  if (!decode_fused_split(p0.B, p0.start_pos + 1, p0.kv, &nsplit, &chunk) || nsplit != p0.nsplit ||
      chunk != p0.chunk)
    return hipErrorInvalidValue;
  DecodeParams p = p0;
  // hand-off buffers with "not yet" markers, and the wo slots, after the
  // synchronisation words
  char* region = reinterpret_cast<char*>(p.sync);
  p.q = reinterpret_cast<float*>(region + kFusedQOff);
  p.kv_new = reinterpret_cast<uint32_t*>(region + kFusedKvOff);
  p.part = reinterpret_cast<float*>(region + kFusedPartOff);
  p.wo_slots = reinterpret_cast<int*>(region + kFusedSlotOff);
  const int grid = fused_qkv_wg(p.kv) + p.nsplit * p.kv * p.B + kFusedWoWG;
#define GQA_LAUNCH_STEP(NB, KV) hipLaunchKernelGGL((decode_step_kernel<NB, KV>), dim3(grid), dim3(256), 0, s, p)
  switch (p.kv * 4 + p.B) {
    case 16 * 4 + 1: GQA_LAUNCH_STEP(1, 16); break;
    case 16 * 4 + 2: GQA_LAUNCH_STEP(2, 16); break;
    case 32 * 4 + 1: GQA_LAUNCH_STEP(1, 32); break;
    case 32 * 4 + 2: GQA_LAUNCH_STEP(2, 32); break;
    case KVH * 4 + 1: GQA_LAUNCH_STEP(1, KVH); break;
    default: GQA_LAUNCH_STEP(2, KVH); break;
  }
#undef GQA_LAUNCH_STEP
  return hipGetLastError();
}

}  // namespace gqa
