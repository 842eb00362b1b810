// C ABI of libgqa.so (declared in include/gqa.h): argument validation on the
// host, workspace layout and kernel dispatch.  Every check runs before the
// first HIP call, so a rejected call launches nothing and changes nothing.
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "kernels.h"

using namespace gqa;

static_assert(kSyncBytes == GQA_SYNC_BYTES, "sync region size differs from the header");

namespace {

std::atomic<int> g_decode_schedule{GQA_DECODE_AUTO};

// Schedule a decode call of this shape runs with under the current setting;
// -1 when the setting demands the fused schedule and the shape does not admit it.
int pick_schedule(int B, int start_pos, int kv = KVH) {
  int nsplit = 0, chunk = 0;
  decode_split(B, start_pos + 1, kv, &nsplit, &chunk);
  const bool ok = kv == KVH && decode_fused_eligible(B, nsplit);
  switch (g_decode_schedule.load()) {
    case GQA_DECODE_SPLIT: return GQA_DECODE_SPLIT;
    case GQA_DECODE_FUSED: return ok ? GQA_DECODE_FUSED : -1;
    default: return ok ? GQA_DECODE_FUSED : GQA_DECODE_SPLIT;
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

int check_common(const void* x, const void* wq, const void* wk, const void* wv, const void* wo,
                 const void* kc, const void* vc, int T_max, const void* rope, int B,
                 const void* out, const void* ws) {
  if (!x || !wq || !wk || !wv || !wo || !kc || !vc || !rope || !out || !ws) return GQA_ERR_NULL;
  if (B < 1 || B > GQA_MAX_BATCH || T_max < 1 || T_max > GQA_MAX_T_MAX) return GQA_ERR_SHAPE;
  if (T_max % GQA_V_BLOCK != 0) return GQA_ERR_ALIGN;
  const void* ptrs[] = {x, wq, wk, wv, wo, kc, vc, rope, out, ws};
  for (const void* q : ptrs)
    if (!aligned16(q)) return GQA_ERR_ALIGN;
  return GQA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? GQA_OK : GQA_ERR_HIP; }

size_t cache_bytes(int B, int T_max, int kv = KVH) { return (size_t)B * kv * T_max * HD * 2; }

// key/value head counts the kernels are instantiated for
bool kv_supported(int kv) { return kv == KVH || kv == 16 || kv == 32; }

// Record events[i] when events is non-NULL.
inline hipError_t mark(hipEvent_t* events, int i, hipStream_t s) {
  return events ? hipEventRecord(events[i], s) : hipSuccess;
}

int prefill_impl(const gqa_bf16* x, const gqa_bf16* wq, const gqa_bf16* wk, const gqa_bf16* wv,
                 const gqa_bf16* wo, gqa_bf16* kcache, gqa_bf16* vcache, int T_max,
                 const float* rope, int start_pos, int B, int T, float* out, void* ws,
                 size_t ws_bytes, float* probe, hipStream_t stream, hipEvent_t* events,
                 int accumulate = 0, bool dry = false, int kv = KVH) {
  int st = check_common(x, wq, wk, wv, wo, kcache, vcache, T_max, rope, B, out, ws);
  if (st != GQA_OK) return st;
  if (!kv_supported(kv)) return GQA_ERR_ARG;
  if (T < 1 || (long)B * T > (1L << 24)) return GQA_ERR_SHAPE;
  if (start_pos < 0 || (long)start_pos + T > T_max) return GQA_ERR_RANGE;
  if (probe && !aligned16(probe)) return GQA_ERR_ALIGN;
  if (ws_bytes < gqa_workspace_bytes_kv(B, start_pos, T, T_max, kv)) return GQA_ERR_WORKSPACE;
  const size_t M = (size_t)B * T;
  const size_t nqkv = (size_t)D + 2 * kv * HD;
  const Range outs[] = {span(out, M * D * 4), span(kcache, cache_bytes(B, T_max, kv)),
                        span(vcache, cache_bytes(B, T_max, kv)), span(ws, ws_bytes),
                        span(probe, probe ? M * nqkv * 4 : 0)};
  const Range ins[] = {span(x, M * D * 2), span(wq, (size_t)D * D * 2),
                       span(wk, (size_t)kv * HD * D * 2), span(wv, (size_t)kv * HD * D * 2),
                       span(wo, (size_t)D * D * 2), span(rope, (size_t)T_max * PAIRS * 8)};
  if (any_alias(outs, 5, ins, 6)) return GQA_ERR_ALIAS;

  PrefillParams p;
  memset(&p, 0, sizeof(p));
  p.x = x; p.wq = wq; p.wk = wk; p.wv = wv; p.wo = wo;
  p.kcache = kcache; p.vcache = vcache; p.rope = rope; p.out = out; p.probe = probe;
  p.T_max = T_max; p.B = B; p.T = T; p.start_pos = start_pos; p.accumulate = accumulate;
  p.kv = kv;
  p.Tp = (start_pos + T + kPrefillTile - 1) / kPrefillTile * kPrefillTile;
  prefill_ws_carve(ws, &p);
  if (dry) return GQA_OK;

  (void)hipGetLastError();
  hipError_t e;
  if ((e = mark(events, 0, stream)) != hipSuccess) return GQA_ERR_HIP;
  if ((e = launch_convert_wo(p, stream)) != hipSuccess) return hip_status(e);
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
                const gqa_bf16* wo, gqa_bf16* kcache, gqa_bf16* vcache, int T_max,
                const float* rope, int start_pos, int B, float* out, gqa_bf16* out_bf16,
                int accumulate, void* ws, size_t ws_bytes, float* probe, hipStream_t stream,
                hipEvent_t* events, bool dry = false, const gqa_bf16* norm_w = nullptr,
                float norm_eps = 0.f, const gqa_bf16* resid = nullptr, int kv = KVH) {
  int st = check_common(x, wq, wk, wv, wo, kcache, vcache, T_max, rope, B, out, ws);
  if (st != GQA_OK) return st;
  if (!kv_supported(kv)) return GQA_ERR_ARG;
  if (start_pos < 0 || start_pos >= T_max) return GQA_ERR_RANGE;
  if ((probe && !aligned16(probe)) || (out_bf16 && !aligned16(out_bf16))) return GQA_ERR_ALIGN;
  if (accumulate != 0 && accumulate != 1) return GQA_ERR_ARG;
  if (ws_bytes < gqa_workspace_bytes(B, 1, T_max)) return GQA_ERR_WORKSPACE;
  const size_t Bz = (size_t)B;
  const size_t nqkv = (size_t)D + 2 * kv * HD;
  const Range outs[] = {span(out, Bz * D * 4), span(out_bf16, out_bf16 ? Bz * D * 2 : 0),
                        span(kcache, cache_bytes(B, T_max, kv)),
                        span(vcache, cache_bytes(B, T_max, kv)),
                        span(ws, ws_bytes), span(probe, probe ? Bz * nqkv * 4 : 0)};
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
  decode_ws_carve(ws, B, &p);
  decode_split(B, start_pos + 1, kv, &p.nsplit, &p.chunk);
  const int sched = pick_schedule(B, start_pos, kv);
  if (sched < 0) return GQA_ERR_ARG;
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
  const size_t base = (block_bytes + 255) & ~(size_t)255;
  if (ws_bytes < base + (size_t)M * D * 2) return GQA_ERR_WORKSPACE;
  // the residual h must not overlap the input, the gain or the workspace
  const Range ins[] = {span(x, (size_t)M * D * 2), span(norm_w, (size_t)D * 2),
                       span(ws, ws_bytes)};
  const Range outs[] = {span(h, (size_t)M * D * 4)};
  if (any_alias(outs, 1, ins, 3)) return GQA_ERR_ALIAS;
  *xn = reinterpret_cast<gqa_bf16*>(static_cast<char*>(ws) + base);
  return GQA_OK;
}

// Zeroes the GQA_SYNC_BYTES synchronisation region, 16 bytes per thread.
__global__ void __launch_bounds__(256) zero_sync_kernel(u32x4* sync) {
  sync[(size_t)blockIdx.x * 256 + threadIdx.x] = u32x4{0u, 0u, 0u, 0u};
}
static_assert(GQA_SYNC_BYTES % (16 * 256) == 0, "sync region is a whole number of fill blocks");

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

int gqa_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!ws) return GQA_ERR_NULL;
  if (!aligned16(ws)) return GQA_ERR_ALIGN;
  if (ws_bytes < (size_t)GQA_SYNC_BYTES) return GQA_ERR_WORKSPACE;
  (void)hipGetLastError();
  // a fill kernel rather than hipMemsetAsync, so the call can also sit in a
  // captured graph
  hipLaunchKernelGGL(zero_sync_kernel, dim3(GQA_SYNC_BYTES / 16 / 256), dim3(256), 0, stream,
                     static_cast<u32x4*>(ws));
  return hip_status(hipGetLastError());
}

int gqa_set_decode_schedule(int schedule) {
  if (schedule != GQA_DECODE_AUTO && schedule != GQA_DECODE_SPLIT && schedule != GQA_DECODE_FUSED)
    return GQA_ERR_ARG;
  return g_decode_schedule.exchange(schedule);
}

int gqa_decode_schedule(int B, int start_pos, int T_max) {
  if (B < 1 || B > GQA_MAX_BATCH || T_max < 1 || T_max > GQA_MAX_T_MAX) return GQA_ERR_SHAPE;
  if (start_pos < 0 || start_pos >= T_max) return GQA_ERR_RANGE;
  const int sched = pick_schedule(B, start_pos);
  return sched < 0 ? GQA_ERR_ARG : sched;
}

size_t gqa_workspace_bytes_kv(int B, int start_pos, int T, int T_max, int n_kv_heads) {
  if (B < 1 || B > GQA_MAX_BATCH || T < 1 || T_max < 1 || T_max > GQA_MAX_T_MAX) return 0;
  if ((long)B * T > (1L << 24) || start_pos < 0 || (long)start_pos + T > T_max) return 0;
  if (!kv_supported(n_kv_heads)) return 0;
  const size_t a = prefill_ws_bytes(B, start_pos, T, n_kv_heads);
  const size_t b = decode_ws_bytes(B);
  return a > b ? a : b;
}

size_t gqa_workspace_bytes_from(int B, int start_pos, int T, int T_max) {
  return gqa_workspace_bytes_kv(B, start_pos, T, T_max, KVH);
}

size_t gqa_workspace_bytes(int B, int T, int T_max) {
  if (B < 1 || B > GQA_MAX_BATCH || T < 1 || T_max < 1 || T_max > GQA_MAX_T_MAX) return 0;
  if ((long)B * T > (1L << 24)) return 0;
  const size_t a = prefill_ws_bytes(B, 0, T);
  const size_t b = decode_ws_bytes(B);
  return a > b ? a : b;
}

int gqa_block_prefill(const gqa_bf16* x, const gqa_bf16* wq, const gqa_bf16* wk,
                      const gqa_bf16* wv, const gqa_bf16* wo, gqa_bf16* kcache,
                      gqa_bf16* vcache, int T_max, const float* rope, int B, int T, float* out,
                      void* ws, size_t ws_bytes, float* probe, hipStream_t stream) {
  return prefill_impl(x, wq, wk, wv, wo, kcache, vcache, T_max, rope, 0, B, T, out, ws, ws_bytes,
                      probe, stream, nullptr);
}

int gqa_vocab_logits(const gqa_bf16* h, const gqa_bf16* norm_w, float eps, const gqa_bf16* w_out,
                     int V, int B, float* logits, hipStream_t stream) {
  if (!h || !w_out || !logits) return GQA_ERR_NULL;
  if (B < 1 || B > GQA_MAX_BATCH || V < 1 || V > GQA_MAX_VOCAB) return GQA_ERR_SHAPE;
  if (!aligned16(h) || !aligned16(w_out) || !aligned16(logits) || (norm_w && !aligned16(norm_w)))
    return GQA_ERR_ALIGN;
  if (norm_w && !(eps > 0.f && eps < 1.f)) return GQA_ERR_ARG;
  const Range outs[] = {span(logits, (size_t)B * V * 4)};
  const Range ins[] = {span(h, (size_t)B * D * 2), span(w_out, (size_t)V * D * 2),
                       span(norm_w, norm_w ? (size_t)D * 2 : 0)};
  if (any_alias(outs, 1, ins, 3)) return GQA_ERR_ALIAS;
  VocabParams p;
  p.z = h; p.norm_w = norm_w; p.norm_eps = eps; p.w = w_out; p.logits = logits; p.V = V; p.B = B;
  (void)hipGetLastError();
  return hip_status(launch_vocab_gemv(p, stream));
}

size_t gqa_layer_workspace_bytes_kv(int B, int start_pos, int T, int T_max, int n_kv_heads) {
  const size_t n = gqa_workspace_bytes_kv(B, start_pos, T, T_max, n_kv_heads);
  if (n == 0) return 0;
  return ((n + 255) & ~(size_t)255) + (size_t)B * T * D * 2;
}

size_t gqa_layer_workspace_bytes(int B, int start_pos, int T, int T_max) {
  return gqa_layer_workspace_bytes_kv(B, start_pos, T, T_max, KVH);
}

int gqa_layer_prefill_kv(const gqa_bf16* x, const gqa_bf16* norm_w, float eps,
                         const gqa_bf16* wq, const gqa_bf16* wk, const gqa_bf16* wv,
                         const gqa_bf16* wo, gqa_bf16* kcache, gqa_bf16* vcache, int n_kv_heads,
                         int T_max, const float* rope, int start_pos, int B, int T, float* h,
                         void* ws, size_t ws_bytes, float* probe, hipStream_t stream) {
  if (!x || !norm_w || !h || !ws) return GQA_ERR_NULL;
  if (!kv_supported(n_kv_heads)) return GQA_ERR_ARG;
  if (B < 1 || B > GQA_MAX_BATCH || T < 1 || (long)B * T > (1L << 24) || T_max < 1 ||
      T_max > GQA_MAX_T_MAX)
    return GQA_ERR_SHAPE;
  if (start_pos < 0 || (long)start_pos + T > T_max) return GQA_ERR_RANGE;
  const size_t block = gqa_workspace_bytes_kv(B, start_pos, T, T_max, n_kv_heads);
  gqa_bf16* xn = nullptr;
  int st = layer_prologue(x, norm_w, eps, B * T, h, ws, ws_bytes, block, &xn);
  if (st != GQA_OK) return st;
  st = prefill_impl(xn, wq, wk, wv, wo, kcache, vcache, T_max, rope, start_pos, B, T, h, ws, block,
                    probe, stream, nullptr, 1, true, n_kv_heads);
  if (st != GQA_OK) return st;
  (void)hipGetLastError();
  if (launch_rmsnorm(x, norm_w, eps, B * T, xn, h, stream) != hipSuccess) return GQA_ERR_HIP;
  return prefill_impl(xn, wq, wk, wv, wo, kcache, vcache, T_max, rope, start_pos, B, T, h, ws,
                      block, probe, stream, nullptr, 1, false, n_kv_heads);
}

int gqa_layer_prefill_from(const gqa_bf16* x, const gqa_bf16* norm_w, float eps,
                           const gqa_bf16* wq, const gqa_bf16* wk, const gqa_bf16* wv,
                           const gqa_bf16* wo, gqa_bf16* kcache, gqa_bf16* vcache, int T_max,
                           const float* rope, int start_pos, int B, int T, float* h, void* ws,
                           size_t ws_bytes, float* probe, hipStream_t stream) {
  return gqa_layer_prefill_kv(x, norm_w, eps, wq, wk, wv, wo, kcache, vcache, KVH, T_max, rope,
                              start_pos, B, T, h, ws, ws_bytes, probe, stream);
}

int gqa_layer_decode_kv(const gqa_bf16* x, const gqa_bf16* norm_w, float eps,
                        const gqa_bf16* wq, const gqa_bf16* wk, const gqa_bf16* wv,
                        const gqa_bf16* wo, gqa_bf16* kcache, gqa_bf16* vcache, int n_kv_heads,
                        int T_max, const float* rope, int start_pos, int B, float* h,
                        gqa_bf16* h_bf16, void* ws, size_t ws_bytes, float* probe,
                        hipStream_t stream) {
  if (!x || !norm_w || !h || !ws) return GQA_ERR_NULL;
  if (!kv_supported(n_kv_heads)) return GQA_ERR_ARG;
  if (B < 1 || B > GQA_MAX_BATCH || T_max < 1 || T_max > GQA_MAX_T_MAX) return GQA_ERR_SHAPE;
  if (start_pos < 0 || start_pos >= T_max) return GQA_ERR_RANGE;
  const size_t block = gqa_workspace_bytes_kv(B, 0, 1, T_max, n_kv_heads);
  gqa_bf16* xn = nullptr;
  int st = layer_prologue(x, norm_w, eps, B, h, ws, ws_bytes, block, &xn);
  if (st != GQA_OK) return st;
  if (B <= kGemvMaxB) {
    // GEMV path: the QKV prologue normalises the staged rows and the wo
    // epilogue adds the residual, no extra launch
    return decode_impl(x, wq, wk, wv, wo, kcache, vcache, T_max, rope, start_pos, B, h, h_bf16, 0,
                       ws, block, probe, stream, nullptr, false, norm_w, eps, x, n_kv_heads);
  }
  st = decode_impl(xn, wq, wk, wv, wo, kcache, vcache, T_max, rope, start_pos, B, h, h_bf16, 1, ws,
                   block, probe, stream, nullptr, true, nullptr, 0.f, nullptr, n_kv_heads);
  if (st != GQA_OK) return st;
  (void)hipGetLastError();
  if (launch_rmsnorm(x, norm_w, eps, B, xn, h, stream) != hipSuccess) return GQA_ERR_HIP;
  return decode_impl(xn, wq, wk, wv, wo, kcache, vcache, T_max, rope, start_pos, B, h, h_bf16, 1,
                     ws, block, probe, stream, nullptr, false, nullptr, 0.f, nullptr, n_kv_heads);
}

int gqa_layer_decode(const gqa_bf16* x, const gqa_bf16* norm_w, float eps, const gqa_bf16* wq,
                     const gqa_bf16* wk, const gqa_bf16* wv, const gqa_bf16* wo,
                     gqa_bf16* kcache, gqa_bf16* vcache, int T_max, const float* rope,
                     int start_pos, int B, float* h, gqa_bf16* h_bf16, void* ws, size_t ws_bytes,
                     float* probe, hipStream_t stream) {
  return gqa_layer_decode_kv(x, norm_w, eps, wq, wk, wv, wo, kcache, vcache, KVH, T_max, rope,
                             start_pos, B, h, h_bf16, ws, ws_bytes, probe, stream);
}

int gqa_block_prefill_from(const gqa_bf16* x, const gqa_bf16* wq, const gqa_bf16* wk,
                           const gqa_bf16* wv, const gqa_bf16* wo, gqa_bf16* kcache,
                           gqa_bf16* vcache, int T_max, const float* rope, int start_pos, int B,
                           int T, float* out, void* ws, size_t ws_bytes, float* probe,
                           hipStream_t stream) {
  return prefill_impl(x, wq, wk, wv, wo, kcache, vcache, T_max, rope, start_pos, B, T, out, ws,
                      ws_bytes, probe, stream, nullptr);
}

int gqa_block_prefill_profiled(const gqa_bf16* x, const gqa_bf16* wq, const gqa_bf16* wk,
                               const gqa_bf16* wv, const gqa_bf16* wo, gqa_bf16* kcache,
                               gqa_bf16* vcache, int T_max, const float* rope, int B, int T,
                               float* out, void* ws, size_t ws_bytes, float* probe,
                               hipStream_t stream, hipEvent_t* events) {
  if (!events) return GQA_ERR_NULL;
  return prefill_impl(x, wq, wk, wv, wo, kcache, vcache, T_max, rope, 0, B, T, out, ws, ws_bytes,
                      probe, stream, events);
}

int gqa_block_prefill_kv(const gqa_bf16* x, const gqa_bf16* wq, const gqa_bf16* wk,
                         const gqa_bf16* wv, const gqa_bf16* wo, gqa_bf16* kcache,
                         gqa_bf16* vcache, int n_kv_heads, int T_max, const float* rope,
                         int start_pos, int B, int T, float* out, void* ws, size_t ws_bytes,
                         float* probe, hipStream_t stream, hipEvent_t* events) {
  return prefill_impl(x, wq, wk, wv, wo, kcache, vcache, T_max, rope, start_pos, B, T, out, ws,
                      ws_bytes, probe, stream, events, 0, false, n_kv_heads);
}

int gqa_block_decode_kv(const gqa_bf16* x, const gqa_bf16* wq, const gqa_bf16* wk,
                        const gqa_bf16* wv, const gqa_bf16* wo, gqa_bf16* kcache,
                        gqa_bf16* vcache, int n_kv_heads, int T_max, const float* rope,
                        int start_pos, int B, float* out, gqa_bf16* out_bf16, int accumulate,
                        void* ws, size_t ws_bytes, float* probe, hipStream_t stream,
                        hipEvent_t* events) {
  return decode_impl(x, wq, wk, wv, wo, kcache, vcache, T_max, rope, start_pos, B, out, out_bf16,
                     accumulate, ws, ws_bytes, probe, stream, events, false, nullptr, 0.f, nullptr,
                     n_kv_heads);
}

int gqa_block_decode(const gqa_bf16* x, const gqa_bf16* wq, const gqa_bf16* wk,
                     const gqa_bf16* wv, const gqa_bf16* wo, gqa_bf16* kcache, gqa_bf16* vcache,
                     int T_max, const float* rope, int start_pos, int B, float* out,
                     gqa_bf16* out_bf16, int accumulate, void* ws, size_t ws_bytes, float* probe,
                     hipStream_t stream) {
  return decode_impl(x, wq, wk, wv, wo, kcache, vcache, T_max, rope, start_pos, B, out, out_bf16,
                     accumulate, ws, ws_bytes, probe, stream, nullptr);
}

int gqa_block_decode_profiled(const gqa_bf16* x, const gqa_bf16* wq, const gqa_bf16* wk,
                              const gqa_bf16* wv, const gqa_bf16* wo, gqa_bf16* kcache,
                              gqa_bf16* vcache, int T_max, const float* rope, int start_pos,
                              int B, float* out, gqa_bf16* out_bf16, int accumulate, void* ws,
                              size_t ws_bytes, float* probe, hipStream_t stream,
                              hipEvent_t* events) {
  if (!events) return GQA_ERR_NULL;
  return decode_impl(x, wq, wk, wv, wo, kcache, vcache, T_max, rope, start_pos, B, out, out_bf16,
                     accumulate, ws, ws_bytes, probe, stream, events);
}

}  // extern "C"
