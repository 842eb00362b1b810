// Shared device helpers for the gfx950 kernels of the attention block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gqa.h"

namespace gqa {

constexpr int D = GQA_D_MODEL;          // 4096
constexpr int H = GQA_N_HEADS;          // 32
constexpr int KVH = GQA_N_KV_HEADS;     // 8
constexpr int HD = GQA_HEAD_DIM;        // 128
constexpr int NQKV = GQA_QKV_DIM;       // 6144
constexpr int REP = H / KVH;            // 4 query heads per KV head
constexpr int PAIRS = GQA_ROPE_PAIRS;   // 64
constexpr int VB = GQA_V_BLOCK;         // 32 positions per value-cache block

// Element offset of value (b, g, t, d) in the blocked value cache of kv
// kv heads (8 for Llama 3.1 8B).
__device__ __forceinline__ size_t vcache_index(int b, int g, int t, int d, int T_max, int kv = KVH) {
  return ((size_t)(b * kv + g) * (T_max / VB) + t / VB) * (HD * VB) + d * VB + (t % VB);
}

// log2(e) / sqrt(128): folds the 1/sqrt(head_dim) score scale into exp2.
constexpr float kScoreLog2 = 0.12751743074843916f;

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((address_space(3))) void lds_void;     // LDS destination of global_load_lds

// ---------------------------------------------------------------------------
// Number formats
// ---------------------------------------------------------------------------

// fp32 -> bf16 by gfx950's conversion instruction (v_cvt_pk_bf16_f32):
// round to nearest even, NaN stays a NaN and comes out quiet.  Checked on
// the device against the bit-level rounding (add 0x7fff plus the kept lsb,
// keep the top half) over all 2^32 fp32 patterns: equal for every non-NaN,
// and every NaN gives a quiet NaN (never a signalling one such as the
// hand-off marker's halves).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {   // low half = a
  const bf16x2 h = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  f16x2 h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}

// v clamped to fp16's finite range: values that would round to infinity
// (|v| >= 65520) become +-65504 and set *sat; NaN stays NaN.
__device__ __forceinline__ float sat_f16(float v, bool& sat) {
  const bool big = fabsf(v) >= 65520.f;
  sat |= big;
  return big ? copysignf(65504.f, v) : v;
}

__device__ __forceinline__ uint32_t pack_f16x2_sat(float a, float b, bool& sat) {
  return pack_f16x2(sat_f16(a, sat), sat_f16(b, sat));
}

// bf16 pair (packed) -> fp16 pair (packed), saturating.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2_sat(uint32_t u, bool& sat) {
  return pack_f16x2_sat(bf16_bits_to_f32(u & 0xffffu), bf16_bits_to_f32(u >> 16), sat);
}

// ---------------------------------------------------------------------------
// Cross-lane
// ---------------------------------------------------------------------------

// DPP control codes (GFX9 encoding).
constexpr int DPP_QUAD_XOR1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int DPP_ROW_SHL4 = 0x104;      // lane i <- lane i+4 within a row of 16
constexpr int DPP_ROW_SHR4 = 0x114;      // lane i <- lane i-4 within a row of 16
constexpr int DPP_ROW_MIRROR = 0x140;    // lane i <- lane 15-i within a row
constexpr int DPP_ROW_HALF_MIRROR = 0x141;  // lane i <- lane 7-i within 8

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over the 16 lanes of each row; every lane of the row gets the sum.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<DPP_QUAD_XOR1>(v);
  v += dpp<DPP_QUAD_XOR2>(v);
  v += dpp<DPP_ROW_HALF_MIRROR>(v);
  v += dpp<DPP_ROW_MIRROR>(v);
  return v;
}

// Sum over all 64 lanes, result uniform.
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}

// op(own value, value of lane l ^ 16) and op(own, lane l ^ 32), the same in
// both lanes of a pair.  The row-swap permutes of gfx950 exchange 16-lane
// rows (0 <-> 1 and 2 <-> 3) or wave halves between their two operands in
// the VALU, with no LDS round trip; with both operands holding v, the two
// results are v and its partner's v in every lane.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------------------
// Memory
// ---------------------------------------------------------------------------

// cache-policy operand of a buffer load that streams (non-temporal)
constexpr int kNtPolicy = 2;

__device__ __forceinline__ u32x4 ld_nt_u32x4(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Device-scope coherent scalar load (reads past other XCDs' L2 caches).
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int ld_dev(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Device-scope stores: written through to the coherence point that every XCD
// reads with ld_dev.
template <typename T>
__device__ __forceinline__ void st_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 16-byte device-scope load at base + byte_off (base wave-uniform, 16-byte
// aligned address): a buffer load with the sc1 cache policy, the policy of
// the device-scope loads above.
__device__ __forceinline__ u32x4 ld_dev_x4(const void* base, uint32_t byte_off) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 16));
}

// Loads through the XCD's L2 (sc0 policy, base wave-uniform).  A store of
// another XCD does not refresh a copy that this L2 already holds, so such a
// load sees another workgroup's completed device-scope store only if its XCD
// has not cached the line since the kernel started (the caches are
// invalidated at every kernel start).  The one-launch decode uses them for
// data that is first read after a device-scope wait on its producers; the
// other readers of the same XCD then hit the L2 line the first one brought in.
__device__ __forceinline__ uint32_t ld_xcd(const void* base, uint32_t byte_off) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
  return __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 1);
}
__device__ __forceinline__ float ld_xcd_f(const void* base, uint32_t byte_off) {
  return __uint_as_float(ld_xcd(base, byte_off));
}
__device__ __forceinline__ u32x4 ld_xcd_x4(const void* base, uint32_t byte_off) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 1));
}

// XCD (XCC) the calling wave runs on, read from the hardware register
// HW_REG_XCC_ID (bits 3:0).
__device__ __forceinline__ int xcc_id() {
  return (int)(__builtin_amdgcn_s_getreg((3 << 11) | 20) & 15u);
}

// Wait until every memory access this wave has issued has completed (stores
// acknowledged by the memory system).
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ u32x4 ld_u32x4(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// MFMA wrappers (gfx950, 16x16 output tile, K = 32 per instruction).
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// c + a.lo * b.lo + a.hi * b.hi over packed fp16 pairs, fp32 accumulation
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

}  // namespace gqa
