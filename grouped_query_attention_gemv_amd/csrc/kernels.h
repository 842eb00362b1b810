// Host-side launchers of the block's kernels and the workspace layout.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace gqa {

// ---------------------------------------------------------------------------
// Decode
// ---------------------------------------------------------------------------

constexpr int kAttnTile = 32;        // keys per wave step of the flash-decode kernel
constexpr int kAttnWaves = 4;        // waves per flash-decode workgroup
constexpr int kMaxSplit = 64;        // most position splits per (sequence, kv head)
constexpr int kPartStride = 132;     // floats per (split, head) partial: m, l, pad, pad, o[128]
constexpr int kGemvMaxNB = 8;        // tokens per pass of the QKV bandwidth GEMV
constexpr int kGemvMaxB = 8;         // larger batches use the matrix-core projections
constexpr int kWoMaxNB = 8;          // tokens per pass of the wo GEMV (hi + lo parts in LDS)

// Synchronisation region at the start of every workspace, used by the
// decode kernels; prefill never touches it (except for the error word).  It
// holds two parts:
//  - 64 KiB of synchronisation words (offsets in ints below): zero before
//    the first decode on a workspace, and every call leaves them zero;
//  - the hand-off buffers of the one-launch schedule (Q, the appended rows,
//    the split partials), whose every word holds a "not yet" marker until
//    its producer overwrites it.  A consumer polls the words themselves, so
//    the value and its arrival travel together; the last consumer writes the
//    marker back.  The marker is a signalling NaN (fp32, or a pair of bf16
//    ones), which no arithmetic result and no bf16 rounding of one can be.
// gqa_workspace_init writes both parts.
constexpr int kSyncWordsBytes = 64 * 1024;
constexpr uint32_t kNotYet = 0x7f800001u;       // fp32 signalling NaN
constexpr uint32_t kNotYetPair = 0x7f817f81u;   // two bf16 signalling NaNs
constexpr int kFusedMaxB = 2;        // largest batch of the fused schedule
constexpr int kFusedMaxAttnWG = 128; // most attention workgroups of the fused schedule
constexpr int kFusedMaxKv = 32;      // most key/value heads of the fused schedule
constexpr int kFusedWoWG = 512;      // wo workgroups of the fused schedule, 8 rows each
constexpr size_t kFusedQOff = kSyncWordsBytes;                                  // fp32 [kFusedMaxB][4096]
constexpr size_t kFusedKvOff = kFusedQOff + (size_t)kFusedMaxB * D * 4;        // bf16 pairs [B][K, V][kv][64]
constexpr size_t kFusedPartOff = kFusedKvOff + (size_t)kFusedMaxB * 2 * kFusedMaxKv * HD * 2;
// partials of at most kFusedMaxAttnWG splits (each serving 32 / kv <= 4
// query heads), each (b, g) region rounded up to whole 128-byte lines
constexpr size_t kFusedPartBytes =
    ((size_t)kFusedMaxAttnWG * REP * kPartStride + kFusedMaxB * kFusedMaxKv * 32) * 4;
// the one part that holds zeros, not markers, at rest: one word per (b, g)
// for each wo workgroup, set once O of (b, g) is complete
constexpr int kFusedSlotWords = kFusedMaxB * kFusedMaxKv;
constexpr size_t kFusedSlotOff = kFusedPartOff + kFusedPartBytes;
constexpr size_t kFusedSlotBytes = (size_t)kFusedWoWG * kFusedSlotWords * 4;
constexpr int kSyncBytes = (int)(((kFusedSlotOff + kFusedSlotBytes) + 4095) / 4096 * 4096);
constexpr int kSyncErr = 0;          // sticky error bits (GQA_WS_ERR_*)
constexpr int kSyncMagic = 1;        // kWsMagic once gqa_workspace_init has run
constexpr int kSyncOffHome = 2;      // fused launches whose first attention workgroup ran
                                     // away from its kv head's XCD (diagnostic)
constexpr int kWsMagic = 0x31415147; // "GQA1"
constexpr int kSyncGroup = 32;       // + 32*g: attention workgroups of kv head g done with Q
constexpr int kSyncProj = 10752;     // + 16*fb: K ranges of projection feature block fb summed
// LDS word where an attention workgroup of the fused schedule keeps Q of its
// 4 heads (after the words of the 4-wave merge, 16-byte aligned)
constexpr int kFusedAttnQWord = (kAttnWaves * REP * HD + 2 * kAttnWaves * REP + 1 + 3) / 4 * 4;
// Row pairs per wave of the fused schedule's QKV role: 2 at 16 and 32 kv
// heads, so that their 6144 + 4096 or 12288 features fit one dispatch round
// (at 1 the role took 1024 and 1536 workgroups against 768 resident)
constexpr int fused_qkv_rpw(int kv) { return kv >= 16 ? 2 : 1; }
// QKV workgroups of the fused schedule, 8 * rpw features each: 768 for 8 kv
// heads (Q 64, K 16, V 16 per head), 512 for 16, 768 for 32
constexpr int fused_qkv_wg(int kv) { return kv * ((H / kv) * HD + 2 * HD) / (8 * fused_qkv_rpw(kv)); }
static_assert(fused_qkv_wg(8) == 768 && fused_qkv_wg(16) == 512 && fused_qkv_wg(32) == 768,
              "QKV role sizes");
// most positions an attention workgroup of the fused schedule covers (two
// tiles per wave)
constexpr int kFusedMaxChunk = 2 * kAttnWaves * kAttnTile;
constexpr int kMaxPolls = 1 << 18;   // bound on every wait of the fused schedule
// The fused schedule's wo workgroups start streaming their weights this many
// real-time ticks (100 MHz: 3.5 us at 8 kv heads, 4 us at 16 and 32) after
// they start.  They are dispatched as
// the QKV workgroups retire and do not need the weights until O is complete;
// starting at once, their 32 MiB competed with the tail of the QKV stream
// that the attention chain waits on.  Swept at B = 1 with the marker
// hand-offs: 3, 3.5, 4, 4.5, 5 and 6 us gave 24.2, 22.5, 22.4-22.7, 22.8,
// 23.4 and 23.8 us at P = 1000; after the 8-byte partials, the release
// reordering and the hardware bf16 conversion, 3, 3.5, 4 and 4.5 us give
// 22.60, 21.47-21.61, 21.74-21.77 and 21.98-22.02 us at P = 1000 and 19.68,
// 19.70-19.76, 19.86-19.88 and 19.77-19.80 us at P = 128.  At 16 and 32 kv
// heads 4 us stays ahead (26.02-26.05 against 26.08-26.15 us and 34.04-34.12
// against 34.24-34.27 us).
constexpr unsigned fused_wo_hold_ticks(int kv) { return kv == 8 ? 350 : 400; }
static_assert(kSyncGroup + 32 * kFusedMaxKv <= kSyncProj, "head counters overlap");
static_assert(kSyncProj + 16 * ((4096 + 2 * 32 * 128) / 64) <= kSyncWordsBytes / 4,
              "sync region too small for the projection counters of 32 kv heads");

struct DecodeParams {
  const uint16_t* x;        // [B][4096] bf16
  const uint16_t* wq;       // [4096][4096]
  const uint16_t* wk;       // [1024][4096]
  const uint16_t* wv;       // [1024][4096]
  const uint16_t* wo;       // [4096][4096]
  uint16_t* kcache;         // [B][8][T_max][128]
  uint16_t* vcache;         // [B][8][T_max/32][128][32]
  const float* rope;        // [T_max][64][2]
  float* out;               // [B][4096]
  uint16_t* out_bf16;       // optional [B][4096]
  float* probe;             // optional [B][6144]
  int T_max, start_pos, B, accumulate;
  // workspace
  float* q;                 // [B][4096] post-RoPE Q, fp32 (fused: in the hand-off region)
  uint16_t* o_hi;           // [B][4096] attention output, bf16 high part
  uint16_t* o_lo;           // [B][4096] bf16 low part (o - hi)
  int* counters;            // [B][8] split arrival counters
  float* part;              // [B][8][nsplit][4][kPartStride]
  uint32_t* kv_new;         // fused: [B][2][8][64] appended K, V rows as packed bf16 pairs
  int* sync;                // the workspace's synchronisation words
  int* wo_slots;            // fused: [kFusedWoWG][kFusedSlotWords] O-ready words
  int kv;                   // kv heads: 8 (Llama 3.1 8B), or 16 / 32 (n_rep 2, 1) on the
                            // GEMV path (B <= kGemvMaxB) with the three-launch schedule
  int nsplit, chunk;        // positions split over nsplit workgroups of chunk keys
  // layer mode of the GEMV path (B <= kGemvMaxB): the QKV prologue replaces
  // x by RMSNorm(x) * norm_w (rounded to bf16), and the wo epilogue writes
  // out = resid + Delta
  const uint16_t* norm_w;   // optional [4096] bf16 gain
  float norm_eps;
  const uint16_t* resid;    // optional [B][4096] bf16 residual
};

// Split of the L = start_pos + 1 visible positions over workgroups.
constexpr int kMaxKv = 32;           // most kv heads (n_rep 1)
void decode_split(int B, int L, int kv, int* nsplit, int* chunk);
int decode_max_split(int B, int kv);
size_t decode_ws_bytes(int B, int kv);
void decode_ws_carve(void* ws, int B, int kv, DecodeParams* p);

hipError_t launch_rope_table(float* rope, int T_max, double theta, int scaled, hipStream_t s);
hipError_t launch_decode_qkv(const DecodeParams& p, hipStream_t s);
hipError_t launch_decode_attn(const DecodeParams& p, hipStream_t s);
hipError_t launch_decode_wo(const DecodeParams& p, hipStream_t s);
// Whether the fused one-launch schedule applies to this call's shape, and
// its split of the L visible positions.
bool decode_fused_split(int B, int L, int kv, int* nsplit, int* chunk);
hipError_t launch_decode_fused(const DecodeParams& p, hipStream_t s);


// ---------------------------------------------------------------------------
// Prefill
// ---------------------------------------------------------------------------

struct PrefillParams {
  const uint16_t* x;        // [M][4096] bf16, M = B*T
  const uint16_t* wq;
  const uint16_t* wk;
  const uint16_t* wv;
  const uint16_t* wo;
  uint16_t* kcache;
  uint16_t* vcache;
  const float* rope;
  float* out;               // [M][4096]
  float* probe;             // optional [M][4096 + 2*kv*128]
  int kv;                   // key/value heads (8 for Llama 3.1 8B; 16, 32)
  int T_max, B, T;          // T new tokens per sequence, at positions start_pos ..
  int start_pos;            // cached rows 0 .. start_pos-1 precede them
  int accumulate;           // out += Delta instead of out = Delta
  int Tp;                   // start_pos + T rounded up to the attention tile
  int convert_wo;           // the prep kernel converts wo into wo16 (no caller copy)
  int* err;                 // the workspace's error word (GQA_WS_ERR_FP16_RANGE)
  // workspace
  uint16_t* wo16;           // [4096][4096] fp16 copy of wo (the workspace's, or the caller's)
  uint16_t* q16;            // [M][4096] fp16 Q * log2(e)/sqrt(128)
  uint16_t* k16;            // [B][kv][Tp][128] fp16 copy of keys 0 .. start_pos+T-1
  uint16_t* v16t;           // [B][kv][Tp/64][128][64] fp16 copy of the values
  uint16_t* o16;            // [M][4096] fp16 attention output
};

constexpr int kPrefillTile = 64;     // query and key tile of the prefill attention

size_t prefill_ws_bytes(int B, int start_pos, int T, int kv = KVH);
void prefill_ws_carve(void* ws, PrefillParams* p);   // reads B, T, Tp, kv

hipError_t launch_prefill_prep(const PrefillParams& p, hipStream_t s);
hipError_t launch_wo_to_fp16(const uint16_t* wo, uint16_t* wo16, hipStream_t s);
hipError_t launch_prefill_qkv(const PrefillParams& p, hipStream_t s);
hipError_t launch_prefill_attn(const PrefillParams& p, hipStream_t s);
hipError_t launch_prefill_wo(const PrefillParams& p, hipStream_t s);

// ---------------------------------------------------------------------------
// Vocabulary projection
// ---------------------------------------------------------------------------

struct VocabParams {
  const uint16_t* z;        // [B][4096] bf16 (normalised here when norm_w is set)
  const uint16_t* norm_w;   // optional [4096] bf16 gain of the final norm
  float norm_eps;
  const uint16_t* w;        // [V][4096] bf16, [out, in]
  float* logits;            // [B][V] fp32 (bf16-rounded values)
  int V, B;
};

// Below kVocabMfmaMinB tokens the bandwidth GEMV (norm fused), from there
// the matrix-core path over z (h, or its norm written into the workspace).
constexpr int kVocabMfmaMinB = 6;
hipError_t launch_vocab_gemv(const VocabParams& p, hipStream_t s);
hipError_t launch_vocab_mfma(const VocabParams& p, const uint16_t* z, hipStream_t s);

// ---------------------------------------------------------------------------
// Pre-norm of a layer
// ---------------------------------------------------------------------------

// xn[m] = bf16(RMSNorm(x[m]) * g) for M rows of 4096; h[m] = x[m] in fp32
// when h is non-null (the residual the block's update is added to).
hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* g, float eps, int M, uint16_t* xn,
                          float* h, hipStream_t s);

}  // namespace gqa
