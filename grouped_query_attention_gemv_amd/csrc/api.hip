// C ABI of libgqa.so (declared in include/gqa.h): argument validation on the
// host, workspace layout and kernel dispatch.  Every check runs before the
// first HIP call, so a rejected call launches nothing and changes nothing.
// The library keeps no state between calls: every choice is an argument.  The
// one exception is gqa_block_decode_noalloc's per-device scratch array and
// the cached device address of it.
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "kernels.h"

using namespace gqa;

static_assert(kSyncBytes == GQA_SYNC_BYTES, "sync region size differs from the header");
static_assert(kVocabMfmaMinB == GQA_VOCAB_MFMA_MIN_B, "vocabulary path threshold differs from the header");

namespace {

// key/value head counts the kernels are instantiated for
bool kv_supported(int kv) { return kv == KVH || kv == 16 || kv == 32; }

bool schedule_valid(int s) {
  return s == GQA_DECODE_AUTO || s == GQA_DECODE_SPLIT || s == GQA_DECODE_FUSED;
}

// The schedule a decode call of this shape runs when it asks for `requested`;
// -1 when the request is unknown or demands the one-launch schedule for a
// shape it does not admit.
int pick_schedule(int kv, int B, int start_pos, int requested) {
  if (!schedule_valid(requested)) return -1;
  int nsplit = 0, chunk = 0;
  const bool ok = decode_fused_split(B, start_pos + 1, kv, &nsplit, &chunk);
  // AUTO takes the one-launch schedule where it measured faster: wherever it
  // is admitted at 8 kv heads, and at B = 1 for 16 and 32 (at B = 2, 16 kv
  // heads and P = 1000, 33.9 against 31.8 us)
  const bool preferred = ok && (kv == KVH || B == 1);
  switch (requested) {
    case GQA_DECODE_SPLIT: return GQA_DECODE_SPLIT;
    case GQA_DECODE_FUSED: return ok ? GQA_DECODE_FUSED : -1;
    default: return preferred ? GQA_DECODE_FUSED : GQA_DECODE_SPLIT;
  }
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range span(const void* p, size_t bytes) {
  uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + bytes};
}

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Outputs must not overlap each other or any input.
bool any_alias(const Range* outs, int n_out, const Range* ins, int n_in) {
  for (int i = 0; i < n_out; ++i) {
    if (outs[i].lo == outs[i].hi) continue;
    for (int j = i + 1; j < n_out; ++j)
      if (outs[j].lo != outs[j].hi && overlaps(outs[i], outs[j])) return true;
    for (int j = 0; j < n_in; ++j)
      if (ins[j].lo != ins[j].hi && overlaps(outs[i], ins[j])) return true;
  }
  return false;
}

// Checks shared by the block calls.  `wo` may be NULL when the prefill gets
// the caller's fp16 copy (wo16).
int check_common(const void* x, const void* wq, const void* wk, const void* wv, const void* wo,
                 const void* kc, const void* vc, int kv, int T_max, const void* rope, int B,
                 const void* out, const void* ws) {
  if (!x || !wq || !wk || !wv || !wo || !kc || !vc || !rope || !out || !ws) return GQA_ERR_NULL;
  if (!kv_supported(kv)) return GQA_ERR_ARG;
  if (B < 1 || B > GQA_MAX_BATCH || T_max < 1 || T_max > GQA_MAX_T_MAX) return GQA_ERR_SHAPE;
  if (T_max % GQA_V_BLOCK != 0) return GQA_ERR_ALIGN;
  const void* ptrs[] = {x, wq, wk, wv, wo, kc, vc, rope, out, ws};
  for (const void* q : ptrs)
    if (!aligned16(q)) return GQA_ERR_ALIGN;
  return GQA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? GQA_OK : GQA_ERR_HIP; }

size_t cache_bytes(int B, int T_max, int kv) { return (size_t)B * kv * T_max * HD * 2; }

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Record events[i] when events is non-NULL.
inline hipError_t mark(hipEvent_t* events, int i, hipStream_t s) {
  return events ? hipEventRecord(events[i], s) : hipSuccess;
}

// Scratch of one operation; 0 for arguments out of range.
// workspace of gqa_vocab_logits: the synchronisation region, then the
// normalised tokens of the matrix-core path
size_t vocab_ws_bytes(int B) { return kSyncBytes + align256((size_t)B * D * 2); }

size_t ws_bytes_for(int op, int kv, int B, int start_pos, int T, int T_max) {
  if (!kv_supported(kv)) return 0;
  if (B < 1 || B > GQA_MAX_BATCH || T < 1 || T_max < 1 || T_max > GQA_MAX_T_MAX) return 0;
  if ((long)B * T > (1L << 24) || start_pos < 0 || (long)start_pos + T > T_max) return 0;
  switch (op) {
    case GQA_OP_VOCAB: return vocab_ws_bytes(B);
    case GQA_OP_PREFILL: return prefill_ws_bytes(B, start_pos, T, kv);
    case GQA_OP_DECODE: return T == 1 ? decode_ws_bytes(B, kv) : 0;
    case GQA_OP_LAYER_PREFILL:
      return align256(prefill_ws_bytes(B, start_pos, T, kv)) + (size_t)B * T * D * 2;
    case GQA_OP_LAYER_DECODE:
      return T == 1 ? align256(decode_ws_bytes(B, kv)) + (size_t)B * D * 2 : 0;
    default: return 0;
  }
}

int prefill_impl(const gqa_bf16* x, const gqa_bf16* wq, const gqa_bf16* wk, const gqa_bf16* wv,
                 const gqa_bf16* wo, const uint16_t* wo16, gqa_bf16* kcache, gqa_bf16* vcache,
                 int kv, int T_max, const float* rope, int start_pos, int B, int T, float* out,
                 void* ws, size_t ws_bytes, float* probe, hipEvent_t* events, hipStream_t stream,
                 int accumulate = 0, bool dry = false) {
  const void* wo_in = wo16 ? static_cast<const void*>(wo16) : static_cast<const void*>(wo);
  int st = check_common(x, wq, wk, wv, wo_in, kcache, vcache, kv, T_max, rope, B, out, ws);
  if (st != GQA_OK) return st;
  if (wo && !aligned16(wo)) return GQA_ERR_ALIGN;
  if (T < 1 || (long)B * T > (1L << 24)) return GQA_ERR_SHAPE;
  if (start_pos < 0 || (long)start_pos + T > T_max) return GQA_ERR_RANGE;
  if (probe && !aligned16(probe)) return GQA_ERR_ALIGN;
  if (ws_bytes < prefill_ws_bytes(B, start_pos, T, kv)) return GQA_ERR_WORKSPACE;
  const size_t M = (size_t)B * T;
  const size_t nqkv = (size_t)D + 2 * kv * HD;
  const Range outs[] = {span(out, M * D * 4), span(kcache, cache_bytes(B, T_max, kv)),
                        span(vcache, cache_bytes(B, T_max, kv)), span(ws, ws_bytes),
                        span(probe, probe ? M * nqkv * 4 : 0)};
  const Range ins[] = {span(x, M * D * 2), span(wq, (size_t)D * D * 2),
                       span(wk, (size_t)kv * HD * D * 2), span(wv, (size_t)kv * HD * D * 2),
                       span(wo16 ? nullptr : wo, wo16 ? 0 : (size_t)D * D * 2),
                       span(wo16, wo16 ? (size_t)D * D * 2 : 0),
                       span(rope, (size_t)T_max * PAIRS * 8)};
  if (any_alias(outs, 5, ins, 7)) return GQA_ERR_ALIAS;

  PrefillParams p;
  memset(&p, 0, sizeof(p));
  p.x = x; p.wq = wq; p.wk = wk; p.wv = wv; p.wo = wo;
  p.kcache = kcache; p.vcache = vcache; p.rope = rope; p.out = out; p.probe = probe;
  p.T_max = T_max; p.B = B; p.T = T; p.start_pos = start_pos; p.accumulate = accumulate;
  p.kv = kv;
  p.Tp = (start_pos + T + kPrefillTile - 1) / kPrefillTile * kPrefillTile;
  prefill_ws_carve(ws, &p);
  p.convert_wo = wo16 == nullptr;
  if (wo16) p.wo16 = const_cast<uint16_t*>(wo16);
  if (dry) return GQA_OK;

  (void)hipGetLastError();
  hipError_t e;
  if ((e = mark(events, 0, stream)) != hipSuccess) return GQA_ERR_HIP;
  if ((e = launch_prefill_prep(p, stream)) != hipSuccess) return hip_status(e);
  if ((e = mark(events, 1, stream)) != hipSuccess) return GQA_ERR_HIP;
  if ((e = launch_prefill_qkv(p, stream)) != hipSuccess) return hip_status(e);
  if ((e = mark(events, 2, stream)) != hipSuccess) return GQA_ERR_HIP;
  if ((e = launch_prefill_attn(p, stream)) != hipSuccess) return hip_status(e);
  if ((e = mark(events, 3, stream)) != hipSuccess) return GQA_ERR_HIP;
  if ((e = launch_prefill_wo(p, stream)) != hipSuccess) return hip_status(e);
  if ((e = mark(events, 4, stream)) != hipSuccess) return GQA_ERR_HIP;
  return GQA_OK;
}

int decode_impl(const gqa_bf16* x, const gqa_bf16* wq, const gqa_bf16* wk, const gqa_bf16* wv,
                const gqa_bf16* wo, gqa_bf16* kcache, gqa_bf16* vcache, int kv, int T_max,
                const float* rope, int start_pos, int B, float* out, gqa_bf16* out_bf16,
                int accumulate, int schedule, void* ws, size_t ws_bytes, float* probe,
                hipEvent_t* events, hipStream_t stream, bool dry = false,
                const gqa_bf16* norm_w = nullptr, float norm_eps = 0.f,
                const gqa_bf16* resid = nullptr, bool ws_is_scratch = false) {
  int st = check_common(x, wq, wk, wv, wo, kcache, vcache, kv, T_max, rope, B, out, ws);
  if (st != GQA_OK) return st;
  if (start_pos < 0 || start_pos >= T_max) return GQA_ERR_RANGE;
  if ((probe && !aligned16(probe)) || (out_bf16 && !aligned16(out_bf16))) return GQA_ERR_ALIGN;
  if (accumulate != 0 && accumulate != 1) return GQA_ERR_ARG;
  const int sched = pick_schedule(kv, B, start_pos, schedule);
  if (sched < 0) return GQA_ERR_ARG;
  if (ws_bytes < decode_ws_bytes(B, kv)) return GQA_ERR_WORKSPACE;
  const size_t Bz = (size_t)B;
  const size_t nqkv = (size_t)D + 2 * kv * HD;
  const Range outs[] = {span(out, Bz * D * 4), span(out_bf16, out_bf16 ? Bz * D * 2 : 0),
                        span(kcache, cache_bytes(B, T_max, kv)),
                        span(vcache, cache_bytes(B, T_max, kv)),
                        // the library's own scratch array cannot overlap caller memory
                        span(ws, ws_is_scratch ? 0 : ws_bytes),
                        span(probe, probe ? Bz * nqkv * 4 : 0)};
  const Range ins[] = {span(x, Bz * D * 2), span(wq, (size_t)D * D * 2),
                       span(wk, (size_t)kv * HD * D * 2), span(wv, (size_t)kv * HD * D * 2),
                       span(wo, (size_t)D * D * 2), span(rope, (size_t)T_max * PAIRS * 8)};
  if (any_alias(outs, 6, ins, 6)) return GQA_ERR_ALIAS;

  DecodeParams p;
  memset(&p, 0, sizeof(p));
  p.x = x; p.wq = wq; p.wk = wk; p.wv = wv; p.wo = wo;
  p.kcache = kcache; p.vcache = vcache; p.rope = rope;
  p.out = out; p.out_bf16 = out_bf16; p.probe = probe;
  p.T_max = T_max; p.start_pos = start_pos; p.B = B; p.accumulate = accumulate;
  p.norm_w = norm_w; p.norm_eps = norm_eps; p.resid = resid; p.kv = kv;
  if ((norm_w || resid) && (B > kGemvMaxB || accumulate)) return GQA_ERR_ARG;
  decode_ws_carve(ws, B, kv, &p);
  if (sched == GQA_DECODE_FUSED)
    decode_fused_split(B, start_pos + 1, kv, &p.nsplit, &p.chunk);
  else
    decode_split(B, start_pos + 1, kv, &p.nsplit, &p.chunk);
  if (dry) return GQA_OK;

  (void)hipGetLastError();
  hipError_t e;
  if ((e = mark(events, 0, stream)) != hipSuccess) return GQA_ERR_HIP;
  if (sched == GQA_DECODE_FUSED) {
    if ((e = launch_decode_fused(p, stream)) != hipSuccess) return hip_status(e);
    for (int i = 1; i <= GQA_DECODE_STAGES; ++i)
      if ((e = mark(events, i, stream)) != hipSuccess) return GQA_ERR_HIP;
    return GQA_OK;
  }
  if ((e = launch_decode_qkv(p, stream)) != hipSuccess) return hip_status(e);
  if ((e = mark(events, 1, stream)) != hipSuccess) return GQA_ERR_HIP;
  if ((e = launch_decode_attn(p, stream)) != hipSuccess) return hip_status(e);
  if ((e = mark(events, 2, stream)) != hipSuccess) return GQA_ERR_HIP;
  if ((e = launch_decode_wo(p, stream)) != hipSuccess) return hip_status(e);
  if ((e = mark(events, 3, stream)) != hipSuccess) return GQA_ERR_HIP;
  return GQA_OK;
}

// Checks shared by the layer entry points; on success *xn points at the
// normalised input inside ws, after the block's own block_bytes.
int layer_prologue(const gqa_bf16* x, const gqa_bf16* norm_w, float eps, int M, const void* h,
                   void* ws, size_t ws_bytes, size_t block_bytes, gqa_bf16** xn) {
  if (!x || !norm_w || !h || !ws) return GQA_ERR_NULL;
  if (!aligned16(x) || !aligned16(norm_w) || !aligned16(h) || !aligned16(ws)) return GQA_ERR_ALIGN;
  if (!(eps > 0.f) || !(eps < 1.f)) return GQA_ERR_ARG;
  if (block_bytes == 0) return GQA_ERR_SHAPE;
  const size_t base = align256(block_bytes);
  if (ws_bytes < base + (size_t)M * D * 2) return GQA_ERR_WORKSPACE;
  // the residual h must not overlap the input, the gain or the workspace
  const Range ins[] = {span(x, (size_t)M * D * 2), span(norm_w, (size_t)D * 2),
                       span(ws, ws_bytes)};
  const Range outs[] = {span(h, (size_t)M * D * 4)};
  if (any_alias(outs, 1, ins, 3)) return GQA_ERR_ALIAS;
  *xn = reinterpret_cast<gqa_bf16*>(static_cast<char*>(ws) + base);
  return GQA_OK;
}

// Prepares the GQA_SYNC_BYTES synchronisation region, 16 bytes per thread:
// zeros, with the magic word after the error word, then the one-launch
// decode's hand-off buffers filled with their "not yet" markers (bf16 pairs
// for the appended rows, fp32 elsewhere), then its wo slots, zero.
__global__ void __launch_bounds__(256) init_sync_kernel(u32x4* sync) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t byte = i * 16;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (byte >= kSyncWordsBytes && byte < kFusedSlotOff) {
    const uint32_t m = (byte >= kFusedKvOff && byte < kFusedPartOff) ? kNotYetPair : kNotYet;
    v = u32x4{m, m, m, m};
  } else if (i == 0) {
    v = u32x4{0u, (uint32_t)kWsMagic, 0u, 0u};
  }
  sync[i] = v;
}
static_assert(GQA_SYNC_BYTES % (16 * 256) == 0, "sync region is a whole number of fill blocks");
static_assert(kSyncErr == 0 && kSyncMagic == 1, "the fill kernel writes the magic into int 1");

// Workspace of gqa_block_decode_noalloc: one array per GPU, alive until the
// process ends.  In host code `scratch` is only a stand-in symbol; its device
// address is looked up once per device with hipGetSymbolAddress and kept in
// g_scratch_ptr, which is what kernels and fills receive.
constexpr size_t kScratchBytes = GQA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array, looked up on its
// first use; nullptr (and *err set) when the HIP calls fail.
void* scratch_on_current_device(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (*err != hipSuccess || !p) return nullptr;
  g_scratch_ptr[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace

extern "C" {

const char* gqa_status_string(int status) {
  switch (status) {
    case GQA_OK: return "GQA_OK";
    case GQA_ERR_NULL: return "GQA_ERR_NULL: a required pointer is NULL";
    case GQA_ERR_SHAPE: return "GQA_ERR_SHAPE: B, T or T_max out of range";
    case GQA_ERR_RANGE: return "GQA_ERR_RANGE: start_pos/T outside [0, T_max)";
    case GQA_ERR_ALIGN: return "GQA_ERR_ALIGN: pointer not 16-byte aligned or T_max % 32 != 0";
    case GQA_ERR_WORKSPACE: return "GQA_ERR_WORKSPACE: workspace too small";
    case GQA_ERR_HIP: return "GQA_ERR_HIP: a HIP call or kernel launch failed";
    case GQA_ERR_ALIAS: return "GQA_ERR_ALIAS: an output overlaps another buffer";
    case GQA_ERR_ARG: return "GQA_ERR_ARG: invalid argument";
    default: return "unknown gqa status";
  }
}

int gqa_rope_table(int T_max, double theta, int scaled, float* rope, hipStream_t stream) {
  if (T_max < 1 || T_max > GQA_MAX_T_MAX) return GQA_ERR_SHAPE;
  if (!(theta > 0.0) || (scaled != 0 && scaled != 1)) return GQA_ERR_ARG;
  if (!rope) return GQA_ERR_NULL;
  if (!aligned16(rope)) return GQA_ERR_ALIGN;
  (void)hipGetLastError();
  return hip_status(launch_rope_table(rope, T_max, theta, scaled, stream));
}

size_t gqa_workspace_bytes(int op, int n_kv_heads, int B, int start_pos, int T, int T_max) {
  return ws_bytes_for(op, n_kv_heads, B, start_pos, T, T_max);
}

int gqa_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!ws) return GQA_ERR_NULL;
  if (!aligned16(ws)) return GQA_ERR_ALIGN;
  if (ws_bytes < (size_t)GQA_SYNC_BYTES) return GQA_ERR_WORKSPACE;
  (void)hipGetLastError();
  // a fill kernel rather than hipMemsetAsync, so the call can also sit in a
  // captured graph
  hipLaunchKernelGGL(init_sync_kernel, dim3(GQA_SYNC_BYTES / 16 / 256), dim3(256), 0, stream,
                     static_cast<u32x4*>(ws));
  return hip_status(hipGetLastError());
}

int gqa_decode_schedule(int n_kv_heads, int B, int start_pos, int T_max, int schedule) {
  if (!kv_supported(n_kv_heads)) return GQA_ERR_ARG;
  if (B < 1 || B > GQA_MAX_BATCH || T_max < 1 || T_max > GQA_MAX_T_MAX) return GQA_ERR_SHAPE;
  if (start_pos < 0 || start_pos >= T_max) return GQA_ERR_RANGE;
  const int sched = pick_schedule(n_kv_heads, B, start_pos, schedule);
  return sched < 0 ? GQA_ERR_ARG : sched;
}

int gqa_wo_to_fp16(const gqa_bf16* wo, uint16_t* wo16, hipStream_t stream) {
  if (!wo || !wo16) return GQA_ERR_NULL;
  if (!aligned16(wo) || !aligned16(wo16)) return GQA_ERR_ALIGN;
  if (overlaps(span(wo, (size_t)D * D * 2), span(wo16, (size_t)D * D * 2))) return GQA_ERR_ALIAS;
  (void)hipGetLastError();
  return hip_status(launch_wo_to_fp16(wo, wo16, stream));
}

int gqa_block_prefill(const gqa_bf16* x, const gqa_bf16* wq, const gqa_bf16* wk,
                      const gqa_bf16* wv, const gqa_bf16* wo, const uint16_t* wo16,
                      gqa_bf16* kcache, gqa_bf16* vcache, int n_kv_heads, int T_max,
                      const float* rope, int start_pos, int B, int T, float* out, void* ws,
                      size_t ws_bytes, float* probe, hipEvent_t* events, hipStream_t stream) {
  return prefill_impl(x, wq, wk, wv, wo, wo16, kcache, vcache, n_kv_heads, T_max, rope,
                      start_pos, B, T, out, ws, ws_bytes, probe, events, stream);
}

int gqa_block_decode(const gqa_bf16* x, const gqa_bf16* wq, const gqa_bf16* wk,
                     const gqa_bf16* wv, const gqa_bf16* wo, gqa_bf16* kcache, gqa_bf16* vcache,
                     int n_kv_heads, int T_max, const float* rope, int start_pos, int B,
                     float* out, gqa_bf16* out_bf16, int accumulate, int schedule, void* ws,
                     size_t ws_bytes, float* probe, hipEvent_t* events, hipStream_t stream) {
  return decode_impl(x, wq, wk, wv, wo, kcache, vcache, n_kv_heads, T_max, rope, start_pos, B,
                     out, out_bf16, accumulate, schedule, ws, ws_bytes, probe, events, stream);
}

int gqa_block_decode_noalloc(const gqa_bf16* x, const gqa_bf16* wq, const gqa_bf16* wk,
                             const gqa_bf16* wv, const gqa_bf16* wo, gqa_bf16* kcache,
                             gqa_bf16* vcache, int n_kv_heads, int T_max, const float* rope,
                             int start_pos, int B, float* out, gqa_bf16* out_bf16,
                             int accumulate, int schedule, float* probe, hipStream_t stream) {
  // the scratch holds what a decode workspace of this shape would
  const size_t need = ws_bytes_for(GQA_OP_DECODE, n_kv_heads, B, start_pos, 1, T_max);
  if (need > kScratchBytes) return GQA_ERR_WORKSPACE;
  // full validation first, with an aligned stand-in for the scratch address
  // (never dereferenced: the dry run launches nothing)
  alignas(256) static const unsigned char stand_in[16] = {};
  void* const fake_ws = const_cast<unsigned char*>(stand_in);
  int st = decode_impl(x, wq, wk, wv, wo, kcache, vcache, n_kv_heads, T_max, rope, start_pos, B,
                       out, out_bf16, accumulate, schedule, fake_ws, kScratchBytes, probe,
                       nullptr, stream, true, nullptr, 0.f, nullptr, true);
  if (st != GQA_OK) return st;
  hipError_t e;
  void* ws = scratch_on_current_device(&e);
  if (!ws) return GQA_ERR_HIP;
  // every call starts from cleared synchronisation words (a fill kernel, so
  // the call may sit in a captured graph)
  (void)hipGetLastError();
  hipLaunchKernelGGL(init_sync_kernel, dim3(GQA_SYNC_BYTES / 16 / 256), dim3(256), 0, stream,
                     static_cast<u32x4*>(ws));
  if ((e = hipGetLastError()) != hipSuccess) return GQA_ERR_HIP;
  return decode_impl(x, wq, wk, wv, wo, kcache, vcache, n_kv_heads, T_max, rope, start_pos, B,
                     out, out_bf16, accumulate, schedule, ws, kScratchBytes, probe, nullptr,
                     stream, false, nullptr, 0.f, nullptr, true);
}

int gqa_layer_prefill(const gqa_bf16* x, const gqa_bf16* norm_w, float eps, const gqa_bf16* wq,
                      const gqa_bf16* wk, const gqa_bf16* wv, const gqa_bf16* wo,
                      const uint16_t* wo16, gqa_bf16* kcache, gqa_bf16* vcache, int n_kv_heads,
                      int T_max, const float* rope, int start_pos, int B, int T, float* h,
                      void* ws, size_t ws_bytes, float* probe, hipStream_t stream) {
  if (!x || !norm_w || !h || !ws) return GQA_ERR_NULL;
  if (!kv_supported(n_kv_heads)) return GQA_ERR_ARG;
  if (B < 1 || B > GQA_MAX_BATCH || T < 1 || (long)B * T > (1L << 24) || T_max < 1 ||
      T_max > GQA_MAX_T_MAX)
    return GQA_ERR_SHAPE;
  if (start_pos < 0 || (long)start_pos + T > T_max) return GQA_ERR_RANGE;
  const size_t block = ws_bytes_for(GQA_OP_PREFILL, n_kv_heads, B, start_pos, T, T_max);
  gqa_bf16* xn = nullptr;
  int st = layer_prologue(x, norm_w, eps, B * T, h, ws, ws_bytes, block, &xn);
  if (st != GQA_OK) return st;
  st = prefill_impl(xn, wq, wk, wv, wo, wo16, kcache, vcache, n_kv_heads, T_max, rope, start_pos,
                    B, T, h, ws, block, probe, nullptr, stream, 1, true);
  if (st != GQA_OK) return st;
  (void)hipGetLastError();
  if (launch_rmsnorm(x, norm_w, eps, B * T, xn, h, stream) != hipSuccess) return GQA_ERR_HIP;
  return prefill_impl(xn, wq, wk, wv, wo, wo16, kcache, vcache, n_kv_heads, T_max, rope,
                      start_pos, B, T, h, ws, block, probe, nullptr, stream, 1, false);
}

int gqa_layer_decode(const gqa_bf16* x, const gqa_bf16* norm_w, float eps, const gqa_bf16* wq,
                     const gqa_bf16* wk, const gqa_bf16* wv, const gqa_bf16* wo,
                     gqa_bf16* kcache, gqa_bf16* vcache, int n_kv_heads, int T_max,
                     const float* rope, int start_pos, int B, float* h, gqa_bf16* h_bf16,
                     int schedule, void* ws, size_t ws_bytes, float* probe, hipStream_t stream) {
  if (!x || !norm_w || !h || !ws) return GQA_ERR_NULL;
  if (!kv_supported(n_kv_heads)) return GQA_ERR_ARG;
  if (B < 1 || B > GQA_MAX_BATCH || T_max < 1 || T_max > GQA_MAX_T_MAX) return GQA_ERR_SHAPE;
  if (start_pos < 0 || start_pos >= T_max) return GQA_ERR_RANGE;
  const size_t block = ws_bytes_for(GQA_OP_DECODE, n_kv_heads, B, start_pos, 1, T_max);
  gqa_bf16* xn = nullptr;
  int st = layer_prologue(x, norm_w, eps, B, h, ws, ws_bytes, block, &xn);
  if (st != GQA_OK) return st;
  if (B <= kGemvMaxB) {
    // GEMV path: the QKV prologue normalises the staged rows and the wo
    // epilogue adds the residual, no extra launch
    return decode_impl(x, wq, wk, wv, wo, kcache, vcache, n_kv_heads, T_max, rope, start_pos, B,
                       h, h_bf16, 0, schedule, ws, block, probe, nullptr, stream, false, norm_w,
                       eps, x);
  }
  st = decode_impl(xn, wq, wk, wv, wo, kcache, vcache, n_kv_heads, T_max, rope, start_pos, B, h,
                   h_bf16, 1, schedule, ws, block, probe, nullptr, stream, true);
  if (st != GQA_OK) return st;
  (void)hipGetLastError();
  if (launch_rmsnorm(x, norm_w, eps, B, xn, h, stream) != hipSuccess) return GQA_ERR_HIP;
  return decode_impl(xn, wq, wk, wv, wo, kcache, vcache, n_kv_heads, T_max, rope, start_pos, B, h,
                     h_bf16, 1, schedule, ws, block, probe, nullptr, stream, false);
}

int gqa_vocab_logits(const gqa_bf16* h, const gqa_bf16* norm_w, float eps, const gqa_bf16* w_out,
                     int V, int B, float* logits, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!h || !w_out || !logits) return GQA_ERR_NULL;
  if (B < 1 || B > GQA_MAX_BATCH || V < 1 || V > GQA_MAX_VOCAB) return GQA_ERR_SHAPE;
  if (!aligned16(h) || !aligned16(w_out) || !aligned16(logits) || (norm_w && !aligned16(norm_w)))
    return GQA_ERR_ALIGN;
  if (norm_w && !(eps > 0.f && eps < 1.f)) return GQA_ERR_ARG;
  // the matrix-core path normalises into the workspace first
  const bool mfma = B >= kVocabMfmaMinB;
  const bool uses_ws = mfma && norm_w;
  if (uses_ws) {
    if (!ws || ws_bytes < vocab_ws_bytes(B)) return GQA_ERR_WORKSPACE;
    if (!aligned16(ws)) return GQA_ERR_ALIGN;
  }
  uint16_t* zn = uses_ws ? reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + kSyncBytes) : nullptr;
  const Range outs[] = {span(logits, (size_t)B * V * 4), span(zn, zn ? (size_t)B * D * 2 : 0)};
  const Range ins[] = {span(h, (size_t)B * D * 2), span(w_out, (size_t)V * D * 2),
                       span(norm_w, norm_w ? (size_t)D * 2 : 0)};
  if (any_alias(outs, 2, ins, 3)) return GQA_ERR_ALIAS;
  VocabParams p;
  p.z = h; p.norm_w = norm_w; p.norm_eps = eps; p.w = w_out; p.logits = logits; p.V = V; p.B = B;
  (void)hipGetLastError();
  if (!mfma) return hip_status(launch_vocab_gemv(p, stream));
  if (zn && launch_rmsnorm(h, norm_w, eps, B, zn, nullptr, stream) != hipSuccess) return GQA_ERR_HIP;
  return hip_status(launch_vocab_mfma(p, zn ? zn : h, stream));
}

}  // extern "C"
