/*
 * gqa.h -- C ABI of libgqa.so: one Llama 3.1 8B grouped-query attention block
 * (d = 4096, 32 query heads, 8 KV heads of width 128, no biases, scaled RoPE)
 * on one MI355X (gfx950).
 *
 * The operation is the one stated on the model-atlas page "Llama 3.1 8B .
 * Grouped-query attention" (header: in x [B, T, 4096] and R [positions, 64
 * pairs], out Delta_attn [B, T, 4096]; mode decode at P cached positions; state
 * "KV cache: writes row P, reads rows 0..P"), with the pieces shown in its
 * evidence sections:
 *   qkv       Q = x Wq^T, K = x Wk^T, V = x Wv^T (weights stored [out, in], as on
 *             page "Llama 3.1 8B . Query projection"), viewed as heads of 128;
 *   rope      adjacent pairs (2i, 2i+1) of each Q and K head rotated by the
 *             angle position * f_i;
 *   gqa       KV head g serves query heads 4g .. 4g+3;
 *   scores    softmax over keys of Q K^T / sqrt(128), causal: query at
 *             position p sees keys 0..p;
 *   retrieval P V, heads merged to feature h*128 + d, Delta = O Wo^T.
 *
 * Conventions for every entry point:
 *   - All pointers are DEVICE pointers owned by the caller, contiguous, and
 *     16-byte aligned.  bf16 values are passed as their 16-bit patterns
 *     (gqa_bf16).
 *   - Work is enqueued on `stream` (NULL = the null stream); calls return
 *     without synchronising.  Calls on different streams are safe when their
 *     buffers are disjoint.  The library holds no mutable global state.
 *   - Every argument is validated on the host before any HIP call.  On an
 *     error nothing is launched and no buffer is modified.  No C++ exception
 *     crosses this interface.
 *   - Returns GQA_OK (0) or a negative gqa_status.
 *
 * KV cache layout (bf16, updated in place; T_max = rows per sequence, a
 * multiple of 32):
 *   kcache [B][8][T_max][128]        key of position t, kv head g, dim d at
 *                                    ((b*8 + g)*T_max + t)*128 + d
 *   vcache [B][8][T_max/32][128][32] value of position t, kv head g, dim d at
 *                                    ((b*8 + g)*(T_max/32) + t/32)*4096
 *                                      + d*32 + t%32
 * Keys are head-major so that a run of positions of one head is contiguous.
 * Values come in blocks of 32 positions stored dimension-major, so the
 * positions that one probability multiplies are contiguous for the matrix
 * cores while a 32-position block stays one contiguous 8 KiB piece.  A call writes exactly the
 * rows start_pos .. start_pos+T-1 of sequences 0..B-1 and leaves every other
 * element bit-for-bit unchanged.  The appended values are the post-RoPE keys
 * and the values rounded to bf16 (nearest, ties to even); attention reads the
 * appended rows back in that rounded form.
 *
 * RoPE table layout: rope[T_max][64][2] fp32, (cos, sin) of position * f_i.
 */
#ifndef GQA_H
#define GQA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Shapes fixed by the Llama 3.1 8B catalogue entry (dim 4096, n_heads 32,
 * n_kv_heads 8; head_dim = dim / n_heads). */
#define GQA_D_MODEL     4096
#define GQA_N_HEADS     32
#define GQA_N_KV_HEADS  8
#define GQA_HEAD_DIM    128
#define GQA_QKV_DIM     6144            /* 4096 (Q) + 1024 (K) + 1024 (V) */
#define GQA_ROPE_PAIRS  64
#define GQA_V_BLOCK     32              /* positions per value-cache block */
#define GQA_MAX_BATCH   1024
#define GQA_MAX_VOCAB  (1 << 20)   /* rows of the vocabulary projection */
#define GQA_MAX_T_MAX   (1 << 20)

/* Leading bytes of every workspace that hold the decode synchronisation words. */
#define GQA_SYNC_BYTES  65536

/* Decode schedules (gqa_set_decode_schedule). */
#define GQA_DECODE_AUTO   0             /* fused where the shape admits it, else split */
#define GQA_DECODE_SPLIT  1             /* three launches: QKV, attention, wo */
#define GQA_DECODE_FUSED  2             /* one launch; shapes it does not admit fail */

/* Number of stages whose boundaries the *_profiled entry points record. */
#define GQA_DECODE_STAGES   3           /* QKV+RoPE+append, attention, wo */
#define GQA_PREFILL_STAGES  4           /* wo to fp16, QKV+RoPE+append, attention, wo */

typedef uint16_t gqa_bf16;

typedef enum {
    GQA_OK            = 0,
    GQA_ERR_NULL      = -1,  /* a required pointer is NULL */
    GQA_ERR_SHAPE     = -2,  /* B, T or T_max outside the supported range */
    GQA_ERR_RANGE     = -3,  /* start_pos < 0 or start_pos + T > T_max */
    GQA_ERR_ALIGN     = -4,  /* a pointer is not 16-byte aligned, or T_max % 32 != 0 */
    GQA_ERR_WORKSPACE = -5,  /* ws_bytes < gqa_workspace_bytes(...) */
    GQA_ERR_HIP       = -6,  /* a HIP call or kernel launch failed */
    GQA_ERR_ALIAS     = -7,  /* an output overlaps an input or another output */
    GQA_ERR_ARG       = -8   /* any other invalid argument (theta <= 0, flags) */
} gqa_status;

/* Readable name of a status code; never NULL. */
const char* gqa_status_string(int status);

/*
 * gqa_rope_table -- fill rope[T_max][64][2] with (cos, sin)(p * f_i) for
 * positions p < T_max (the table R of the block's header).
 *
 * f_i = theta^(-2i/128).  With scaled != 0 the Llama 3.1 long-context rule is
 * applied (catalogue entry use_scaled_rope: True; the page "Llama 3 8B .
 * Attention update" shows the unscaled Llama 3 setting): wavelengths
 * 2*pi/f_i below 8192/4 keep f_i, above 8192 use f_i/8, and in between f_i is
 * blended linearly in 8192/wavelength.  Angles are formed and evaluated in
 * fp64 and rounded once to fp32.
 *   T_max  1 .. GQA_MAX_T_MAX
 *   theta  > 0 (500000.0 for Llama 3 and 3.1)
 *   rope   device, T_max*64*2 floats
 * Errors: GQA_ERR_SHAPE, GQA_ERR_ARG, GQA_ERR_NULL, GQA_ERR_ALIGN, GQA_ERR_HIP.
 */
int gqa_rope_table(int T_max, double theta, int scaled, float* rope, hipStream_t stream);

/*
 * gqa_workspace_bytes -- device scratch needed by gqa_block_prefill(B, T) and
 * by gqa_block_decode(B, start_pos < T_max) with these arguments; 0 when the
 * arguments are out of range.  Calls that share a workspace must be ordered
 * (one stream, or events): they reuse its contents.
 *
 * The first GQA_SYNC_BYTES bytes hold the synchronisation words of the fused
 * decode schedule.  They must be zero before the first call on a workspace
 * (gqa_workspace_init); every call leaves them zero and prefill never writes
 * them.  Their first int is a sticky error word: nonzero after a fused decode
 * whose bounded waits timed out (that call's outputs are invalid; initialise
 * the workspace again).  The rest holds nothing the caller reads.
 */
size_t gqa_workspace_bytes(int B, int T, int T_max);

/*
 * gqa_workspace_bytes_from -- the same for gqa_block_prefill_from(start_pos,
 * B, T) (and decode); its fp16 K/V copies hold all start_pos + T keys.  0 when
 * the arguments are out of range (start_pos < 0 or start_pos + T > T_max
 * included).  gqa_workspace_bytes(B, T, T_max) equals the start_pos = 0 value.
 */
size_t gqa_workspace_bytes_from(int B, int start_pos, int T, int T_max);

/*
 * gqa_workspace_bytes_kv -- gqa_workspace_bytes_from for a model with
 * n_kv_heads key/value heads (8, 16 or 32; the prefill's fp16 K/V copies grow
 * with it).  0 for another n_kv_heads or out-of-range arguments; n_kv_heads = 8
 * equals gqa_workspace_bytes_from.
 */
size_t gqa_workspace_bytes_kv(int B, int start_pos, int T, int T_max, int n_kv_heads);

/*
 * gqa_workspace_init -- zero the synchronisation words of a workspace of
 * ws_bytes bytes (one small fill kernel on stream; no host synchronisation).
 * Errors: GQA_ERR_NULL, GQA_ERR_ALIGN, GQA_ERR_WORKSPACE (< GQA_SYNC_BYTES),
 * GQA_ERR_HIP.
 */
int gqa_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Decode schedule.  GQA_DECODE_SPLIT runs the three stages as three kernels.
 * GQA_DECODE_FUSED runs the whole step as one kernel whose workgroups pass
 * results to each other through the workspace (Q/K/V -> attention -> wo), so
 * that each consumer's HBM reads overlap its producer's; it admits B <= 2 and
 * contexts short enough for at most 128 attention workgroups (start_pos + 1
 * <= 2048 at B = 1, <= 1024 at B = 2).  GQA_DECODE_AUTO (the default) takes
 * the fused schedule where it is admitted.  Results agree between schedules
 * to rounding; each schedule is deterministic.
 *
 * gqa_set_decode_schedule sets the process-wide choice and returns the
 * previous one (GQA_ERR_ARG for an unknown value); gqa_decode_schedule
 * returns the schedule a decode call of this shape would run
 * (GQA_DECODE_SPLIT or GQA_DECODE_FUSED), or GQA_ERR_ARG when the setting is
 * GQA_DECODE_FUSED and the shape is not admitted (the call would fail with
 * that code), GQA_ERR_SHAPE / GQA_ERR_RANGE for invalid arguments.
 */
int gqa_set_decode_schedule(int schedule);
int gqa_decode_schedule(int B, int start_pos, int T_max);

/*
 * gqa_block_prefill -- the block over T new tokens of B sequences starting
 * at position 0 (the "Prefill" mode of the pages), with a causal mask.
 *   x        [B][T][4096] bf16, the block input
 *   wq       [4096][4096] bf16 [out, in];  wk, wv [1024][4096];  wo [4096][4096]
 *   kcache, vcache   layouts above; rows 0..T-1 of each sequence are written
 *   T_max    rows per sequence in the caches and the table; T <= T_max
 *   rope     [T_max][64][2] fp32 from gqa_rope_table
 *   out      [B][T][4096] fp32, Delta_attn
 *   ws       workspace of ws_bytes >= gqa_workspace_bytes(B, T, T_max)
 *   probe    NULL, or [B][T][6144] fp32 receiving the post-RoPE Q | K and the V
 *            features exactly as computed before any rounding (for checking)
 * Aliasing: out, probe, ws and the caches must not overlap each other or the
 * inputs.
 */
int gqa_block_prefill(const gqa_bf16* x,
                      const gqa_bf16* wq, const gqa_bf16* wk,
                      const gqa_bf16* wv, const gqa_bf16* wo,
                      gqa_bf16* kcache, gqa_bf16* vcache, int T_max,
                      const float* rope, int B, int T,
                      float* out, void* ws, size_t ws_bytes, float* probe,
                      hipStream_t stream);

/*
 * gqa_block_prefill_from -- the block over T new tokens of B sequences at
 * positions start_pos .. start_pos+T-1, after start_pos rows already in the
 * caches (chunked prefill).  The page "Llama 3.1 8B . Grouped-query
 * attention" states the rule in the mask listing of its code section: with
 * start_pos cached positions, new token i sits at position start_pos + i and
 * attends to every key j <= start_pos + i, the cached rows included; RoPE
 * uses the same absolute positions.  start_pos = 0 is gqa_block_prefill.
 *   start_pos  0 .. T_max-T; rows 0 .. start_pos-1 of every sequence must
 *              hold the earlier tokens' keys and values; they are read, not
 *              written, and rows start_pos .. start_pos+T-1 are written
 *   ws         ws_bytes >= gqa_workspace_bytes_from(B, start_pos, T, T_max)
 *   other arguments as for gqa_block_prefill
 * Errors: as gqa_block_prefill; GQA_ERR_RANGE for start_pos < 0 or
 * start_pos + T > T_max.
 */
int gqa_block_prefill_from(const gqa_bf16* x,
                           const gqa_bf16* wq, const gqa_bf16* wk,
                           const gqa_bf16* wv, const gqa_bf16* wo,
                           gqa_bf16* kcache, gqa_bf16* vcache, int T_max,
                           const float* rope, int start_pos, int B, int T,
                           float* out, void* ws, size_t ws_bytes, float* probe,
                           hipStream_t stream);

/*
 * gqa_block_prefill_kv -- gqa_block_prefill_from for a model with n_kv_heads
 * key / value heads, each shared by 32 / n_kv_heads query heads (the n_rep of
 * the page "Llama 3.1 8B . Grouped-query attention", evidence "gqa": query
 * head h reads kv head h / n_rep; n_kv_heads = 32 is multi-head attention).
 *   n_kv_heads  8, 16 or 32 (8 behaves as gqa_block_prefill_from)
 *   wk, wv      [n_kv_heads*128][4096] bf16
 *   kcache      [B][n_kv_heads][T_max][128] bf16
 *   vcache      [B][n_kv_heads][T_max/32][128][32] bf16
 *   ws          ws_bytes >= gqa_workspace_bytes_kv(B, start_pos, T, T_max,
 *               n_kv_heads)
 *   probe       NULL or [B*T][4096 + 2*n_kv_heads*128] fp32
 *   events      NULL, or GQA_PREFILL_STAGES + 1 events recorded as by
 *               gqa_block_prefill_profiled
 *   other arguments as for gqa_block_prefill_from
 * Errors: as gqa_block_prefill_from; GQA_ERR_ARG for another n_kv_heads.
 */
int gqa_block_prefill_kv(const gqa_bf16* x,
                         const gqa_bf16* wq, const gqa_bf16* wk,
                         const gqa_bf16* wv, const gqa_bf16* wo,
                         gqa_bf16* kcache, gqa_bf16* vcache, int n_kv_heads,
                         int T_max, const float* rope, int start_pos, int B,
                         int T, float* out, void* ws, size_t ws_bytes,
                         float* probe, hipStream_t stream, hipEvent_t* events);

/*
 * Layer entry points: the block inside its residual branch, as the page
 * "Llama 3.1 8B . Grouped-query attention" shows it in its code section
 * (h = x + attention(attention_norm(x), ...), attention_norm an RMSNorm over
 * the 4096 features with eps = norm_eps, 1e-5 in the catalogue entry).  The
 * pages do not print the norm's body; it is taken as
 *   xn = x / sqrt(mean(x^2) + eps) * norm_w,
 * computed in fp32 and rounded once to bf16, the block's input dtype.
 * Outputs: h = x + Delta_attn(xn) in fp32, and for decode optionally its bf16
 * rounding (the next layer's input).
 *   x        bf16, [B][T][4096] (prefill) or [B][4096] (decode), the residual
 *            stream before the layer
 *   norm_w   bf16 [4096], the norm's gain
 *   eps      0 < eps < 1
 *   h        fp32, same shape as x; written, never read
 *   ws       ws_bytes >= gqa_layer_workspace_bytes(B, start_pos, T, T_max)
 *            for prefill, gqa_layer_workspace_bytes(B, 0, 1, T_max) for
 *            decode; the normalised input lives at its end
 *   other arguments as for gqa_block_prefill_from / gqa_block_decode
 * Errors: those of the block calls; GQA_ERR_ARG for eps; GQA_ERR_ALIAS when h
 * overlaps x, norm_w or ws.
 */
/*
 * gqa_vocab_logits -- the vocabulary projection of the page "Llama 3.1 8B .
 * Vocabulary projection": L = z W_out for one position of each of B
 * sequences, the weight stored [out, in] = [V][4096], no bias.  The page
 * casts the projection's output to float32 before returning it, so each
 * logit is the bf16 rounding (nearest even) of its fp32-accumulated dot
 * product, returned as fp32.  With norm_w non-NULL, z is the final norm of
 * the page's code (self.norm, an RMSNorm with norm_eps) applied to h, read as
 * in the layer pre-norm above; with NULL, z = h.
 *   h       [B][4096] bf16
 *   norm_w  NULL or [4096] bf16; eps as for the layers (ignored when NULL)
 *   w_out   [V][4096] bf16; V = 128256 for Llama 3.1 (1 .. GQA_MAX_VOCAB)
 *   logits  [B][V] fp32, written
 * One weight pass per 8 sequences.  No workspace.
 * Errors: GQA_ERR_NULL, GQA_ERR_SHAPE, GQA_ERR_ALIGN, GQA_ERR_ARG (eps),
 * GQA_ERR_ALIAS (logits overlapping an input), GQA_ERR_HIP.
 */
int gqa_vocab_logits(const gqa_bf16* h, const gqa_bf16* norm_w, float eps,
                     const gqa_bf16* w_out, int V, int B, float* logits,
                     hipStream_t stream);

size_t gqa_layer_workspace_bytes(int B, int start_pos, int T, int T_max);

int gqa_layer_prefill_from(const gqa_bf16* x, const gqa_bf16* norm_w, float eps,
                           const gqa_bf16* wq, const gqa_bf16* wk,
                           const gqa_bf16* wv, const gqa_bf16* wo,
                           gqa_bf16* kcache, gqa_bf16* vcache, int T_max,
                           const float* rope, int start_pos, int B, int T,
                           float* h, void* ws, size_t ws_bytes, float* probe,
                           hipStream_t stream);

int gqa_layer_decode(const gqa_bf16* x, const gqa_bf16* norm_w, float eps,
                     const gqa_bf16* wq, const gqa_bf16* wk,
                     const gqa_bf16* wv, const gqa_bf16* wo,
                     gqa_bf16* kcache, gqa_bf16* vcache, int T_max,
                     const float* rope, int start_pos, int B,
                     float* h, gqa_bf16* h_bf16,
                     void* ws, size_t ws_bytes, float* probe,
                     hipStream_t stream);

/*
 * gqa_layer_prefill_kv, gqa_layer_decode_kv, gqa_layer_workspace_bytes_kv --
 * the two layer entry points above for a model with n_kv_heads key/value
 * heads (the GQA map and the multi-head case of the page "Llama 3.1 8B .
 * Grouped-query attention", as for gqa_block_prefill_kv and
 * gqa_block_decode_kv); 8 behaves as gqa_layer_prefill_from /
 * gqa_layer_decode.
 *   n_kv_heads  8, 16 or 32
 *   wk, wv      [n_kv_heads*128][4096] bf16
 *   kcache      [B][n_kv_heads][T_max][128] bf16
 *   vcache      [B][n_kv_heads][T_max/32][128][32] bf16
 *   probe       NULL or [B*T][4096 + 2*n_kv_heads*128] fp32
 *   ws          ws_bytes >= gqa_layer_workspace_bytes_kv(B, start_pos, T,
 *               T_max, n_kv_heads) for prefill, (B, 0, 1, T_max, n_kv_heads)
 *               for decode, initialised once by gqa_workspace_init
 *   other arguments, ownership and asynchrony as for the 8-head entry points;
 *   decode other than 8 heads runs the three-launch schedule (GQA_ERR_ARG if
 *   GQA_DECODE_FUSED is forced)
 * Errors: as gqa_layer_prefill_from / gqa_layer_decode; GQA_ERR_ARG for
 * another n_kv_heads.  gqa_layer_workspace_bytes_kv returns 0 for shapes or
 * head counts that are not accepted.
 */
size_t gqa_layer_workspace_bytes_kv(int B, int start_pos, int T, int T_max,
                                    int n_kv_heads);

int gqa_layer_prefill_kv(const gqa_bf16* x, const gqa_bf16* norm_w, float eps,
                         const gqa_bf16* wq, const gqa_bf16* wk,
                         const gqa_bf16* wv, const gqa_bf16* wo,
                         gqa_bf16* kcache, gqa_bf16* vcache, int n_kv_heads,
                         int T_max, const float* rope, int start_pos, int B,
                         int T, float* h, void* ws, size_t ws_bytes,
                         float* probe, hipStream_t stream);

int gqa_layer_decode_kv(const gqa_bf16* x, const gqa_bf16* norm_w, float eps,
                        const gqa_bf16* wq, const gqa_bf16* wk,
                        const gqa_bf16* wv, const gqa_bf16* wo,
                        gqa_bf16* kcache, gqa_bf16* vcache, int n_kv_heads,
                        int T_max, const float* rope, int start_pos, int B,
                        float* h, gqa_bf16* h_bf16,
                        void* ws, size_t ws_bytes, float* probe,
                        hipStream_t stream);

/*
 * gqa_block_decode -- one new token per sequence at position start_pos (the
 * page's decode mode): writes cache row start_pos and attends over rows
 * 0..start_pos of each of the B sequences (one start_pos for all of them).
 *   x          [B][4096] bf16
 *   weights, caches, T_max, rope, ws, probe as for prefill (probe [B][6144])
 *   start_pos  0 .. T_max-1
 *   out        [B][4096] fp32: out = Delta when accumulate == 0,
 *              out += Delta when accumulate != 0 (the block residual
 *              h = x + attention(...), with the caller's fp32 residual in out)
 *   out_bf16   NULL, or [B][4096] bf16 receiving the bf16 rounding of out
 *              after the update (the next block's input in a stack of blocks)
 * Aliasing: out, out_bf16, probe, ws and the caches must not overlap each
 * other or the inputs.
 * Runs the schedule gqa_decode_schedule(B, start_pos, T_max) names; returns
 * GQA_ERR_ARG if that is an error.
 */
int gqa_block_decode(const gqa_bf16* x,
                     const gqa_bf16* wq, const gqa_bf16* wk,
                     const gqa_bf16* wv, const gqa_bf16* wo,
                     gqa_bf16* kcache, gqa_bf16* vcache, int T_max,
                     const float* rope, int start_pos, int B,
                     float* out, gqa_bf16* out_bf16, int accumulate,
                     void* ws, size_t ws_bytes, float* probe,
                     hipStream_t stream);

/*
 * gqa_block_decode_kv -- gqa_block_decode for a model with n_kv_heads key /
 * value heads shared by 32 / n_kv_heads query heads each (the n_rep of the
 * page "Llama 3.1 8B . Grouped-query attention", evidence "gqa": KV head g
 * serves query heads g*n_rep .. g*n_rep + n_rep - 1; n_rep = 1 is the
 * multi-head attention the page sizes beside GQA).  Llama 3.1 8B is
 * n_kv_heads = 8, where this equals gqa_block_decode.
 *   n_kv_heads  8, 16 or 32; other than 8 only with the three-launch
 *               schedule (GQA_ERR_ARG if GQA_DECODE_FUSED is forced); above 8
 *               tokens the projections run on the matrix cores for every
 *               head count
 *   wk, wv      [n_kv_heads*128][4096] bf16
 *   kcache      [B][n_kv_heads][T_max][128] bf16
 *   vcache      [B][n_kv_heads][T_max/32][128][32] bf16
 *   probe       NULL or [B][4096 + 2*n_kv_heads*128] fp32
 *   events      NULL, or GQA_DECODE_STAGES + 1 events recorded as by
 *               gqa_block_decode_profiled
 *   other arguments, ownership and workspace as for gqa_block_decode
 * Errors: as gqa_block_decode; GQA_ERR_ARG for another n_kv_heads.
 */
int gqa_block_decode_kv(const gqa_bf16* x,
                        const gqa_bf16* wq, const gqa_bf16* wk,
                        const gqa_bf16* wv, const gqa_bf16* wo,
                        gqa_bf16* kcache, gqa_bf16* vcache, int n_kv_heads,
                        int T_max, const float* rope, int start_pos, int B,
                        float* out, gqa_bf16* out_bf16, int accumulate,
                        void* ws, size_t ws_bytes, float* probe,
                        hipStream_t stream, hipEvent_t* events);

/*
 * Same as gqa_block_prefill / gqa_block_decode, and additionally records
 * events[0] on `stream` before the first kernel and events[i] after stage i
 * (GQA_PREFILL_STAGES / GQA_DECODE_STAGES stages), so that a caller can time
 * each kernel with hipEventElapsedTime.  events must hold that many + 1
 * created hipEvent_t handles.  Under the fused decode schedule the step is
 * one kernel: events[1] follows it and the later events are recorded
 * immediately after.
 */
int gqa_block_prefill_profiled(const gqa_bf16* x,
                               const gqa_bf16* wq, const gqa_bf16* wk,
                               const gqa_bf16* wv, const gqa_bf16* wo,
                               gqa_bf16* kcache, gqa_bf16* vcache, int T_max,
                               const float* rope, int B, int T,
                               float* out, void* ws, size_t ws_bytes, float* probe,
                               hipStream_t stream, hipEvent_t* events);

int gqa_block_decode_profiled(const gqa_bf16* x,
                              const gqa_bf16* wq, const gqa_bf16* wk,
                              const gqa_bf16* wv, const gqa_bf16* wo,
                              gqa_bf16* kcache, gqa_bf16* vcache, int T_max,
                              const float* rope, int start_pos, int B,
                              float* out, gqa_bf16* out_bf16, int accumulate,
                              void* ws, size_t ws_bytes, float* probe,
                              hipStream_t stream, hipEvent_t* events);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H */
