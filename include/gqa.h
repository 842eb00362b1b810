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
 *   gqa       KV head g serves query heads n_rep*g .. n_rep*g + n_rep-1,
 *             n_rep = 32 / n_kv_heads (4 for Llama 3.1 8B; n_kv_heads = 32 is
 *             the multi-head attention the page sizes beside it);
 *   scores    softmax over keys of Q K^T / sqrt(128), causal: query at
 *             position p sees keys 0..p;
 *   retrieval P V, heads merged to feature h*128 + d, Delta = O Wo^T.
 *
 * Conventions for every entry point:
 *   - All pointers are DEVICE pointers owned by the caller, contiguous, and
 *     16-byte aligned.  bf16 values are passed as their 16-bit patterns
 *     (gqa_bf16).  The library allocates no memory at run time.
 *   - Work is enqueued on `stream` (NULL = the null stream); calls return
 *     without synchronising.  Calls on different streams are safe when their
 *     buffers are disjoint.  Every choice (head count, decode schedule,
 *     events) is an argument of the call; the only state the library keeps
 *     is gqa_block_decode_noalloc's scratch array per GPU and its cached
 *     device address.
 *   - Every argument is validated on the host before any HIP call.  On an
 *     error nothing is launched and no buffer is modified.  No C++ exception
 *     crosses this interface.
 *   - Returns GQA_OK (0) or a negative gqa_status.
 *
 * KV cache layout (bf16, updated in place; n_kv = n_kv_heads; T_max = rows
 * per sequence, a multiple of 32):
 *   kcache [B][n_kv][T_max][128]        key of position t, kv head g, dim d at
 *                                       ((b*n_kv + g)*T_max + t)*128 + d
 *   vcache [B][n_kv][T_max/32][128][32] value of position t, kv head g, dim d at
 *                                       ((b*n_kv + g)*(T_max/32) + t/32)*4096
 *                                         + d*32 + t%32
 * Keys are head-major so that a run of positions of one head is contiguous.
 * Values come in blocks of 32 positions stored dimension-major, so the
 * positions that one probability multiplies are contiguous for the matrix
 * cores while a 32-position block stays one contiguous 8 KiB piece.  A call
 * writes exactly the rows start_pos .. start_pos+T-1 of sequences 0..B-1 and
 * leaves every other element bit-for-bit unchanged.  The appended values are
 * the post-RoPE keys and the values rounded to bf16 (nearest, ties to even);
 * attention reads the appended rows back in that rounded form.
 *
 * RoPE table layout: rope[T_max][64][2] fp32, (cos, sin) of position * f_i.
 *
 * Value range of prefill: its attention and output projection run on fp16
 * matrix-core operands (keys, values, Wo, and Q, P, O).  A key, value or Wo
 * entry beyond fp16's range (|v| > 65504, which bf16 can hold) is saturated
 * to +-65504, and the call sets GQA_WS_ERR_FP16_RANGE in its workspace's
 * error word; Delta is then not the exact block.  Decode has no such limit.
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

/* Leading bytes of every workspace: the synchronisation words of the decode
 * kernels, headed by an error word and a magic word, then the hand-off
 * buffers of the one-launch decode (gqa_workspace_init prepares both). */
#define GQA_SYNC_BYTES  540672

/* gqa_vocab_logits runs on the matrix cores from this many sequences on
 * (below, a GEMV with the norm fused); with a norm it then needs a
 * workspace for the normalised input. */
#define GQA_VOCAB_MFMA_MIN_B  6

/* Bits of the workspace error word (its first int). */
#define GQA_WS_ERR_WAIT        0x1   /* a bounded wait of the one-launch decode timed out */
#define GQA_WS_ERR_WO_WAIT     0x2   /* the same, in its output projection */
#define GQA_WS_ERR_INIT        0x4   /* a decode found the workspace uninitialised */
#define GQA_WS_ERR_FP16_RANGE  0x100 /* a prefill saturated an operand to +-65504 */

/* Decode schedules (the `schedule` argument of the decode calls). */
#define GQA_DECODE_AUTO   0             /* one launch where admitted and faster, else three */
#define GQA_DECODE_SPLIT  1             /* three launches: QKV, attention, wo */
#define GQA_DECODE_FUSED  2             /* one launch; shapes it does not admit fail */

/* Operations whose workspace gqa_workspace_bytes sizes. */
#define GQA_OP_PREFILL        0
#define GQA_OP_DECODE         1
#define GQA_OP_LAYER_PREFILL  2
#define GQA_OP_LAYER_DECODE   3
#define GQA_OP_VOCAB          4

/* Number of stages whose boundaries the `events` arguments record. */
#define GQA_DECODE_STAGES   3           /* QKV+RoPE+append, attention, wo */
#define GQA_PREFILL_STAGES  4           /* prep (wo to fp16, cached rows), QKV+RoPE+append,
                                           attention, wo */

typedef uint16_t gqa_bf16;

typedef enum {
    GQA_OK            = 0,
    GQA_ERR_NULL      = -1,  /* a required pointer is NULL */
    GQA_ERR_SHAPE     = -2,  /* B, T or T_max outside the supported range */
    GQA_ERR_RANGE     = -3,  /* start_pos < 0 or start_pos + T > T_max */
    GQA_ERR_ALIGN     = -4,  /* a pointer is not 16-byte aligned, or T_max % 32 != 0 */
    GQA_ERR_WORKSPACE = -5,  /* ws_bytes below gqa_workspace_bytes(...) */
    GQA_ERR_HIP       = -6,  /* a HIP call or kernel launch failed */
    GQA_ERR_ALIAS     = -7,  /* an output overlaps an input or another output */
    GQA_ERR_ARG       = -8   /* any other invalid argument (n_kv_heads, theta, flags,
                                schedule, or a schedule the shape does not admit) */
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
 * gqa_workspace_bytes -- device scratch needed by one call of operation `op`
 * with these arguments; 0 when they are out of range.
 *   op          GQA_OP_PREFILL (gqa_block_prefill), GQA_OP_DECODE
 *               (gqa_block_decode), GQA_OP_LAYER_PREFILL, GQA_OP_LAYER_DECODE,
 *               GQA_OP_VOCAB (gqa_vocab_logits: only B is used; the others
 *               must still be in range)
 *   n_kv_heads  8, 16 or 32
 *   B, T        sequences and new tokens per sequence (T = 1 for decode)
 *   start_pos   cached rows before the new tokens (prefill's fp16 key/value
 *               copies hold all start_pos + T keys; decode's scratch does not
 *               depend on it)
 *   T_max       rows per sequence of the caches
 * Decode needs the synchronisation region, Q, O and the attention partials
 * (about 1.5 MiB at B = 1); prefill adds fp16 copies of Q, O, the keys and
 * values and of Wo.  A workspace sized for one operation serves any smaller
 * one.  Calls that share a workspace must be ordered (one stream, or
 * events): they reuse its contents.
 */
size_t gqa_workspace_bytes(int op, int n_kv_heads, int B, int start_pos, int T, int T_max);

/*
 * gqa_workspace_init -- prepare a workspace of ws_bytes bytes (at least
 * GQA_SYNC_BYTES): zero its synchronisation words, write the magic word that
 * the decode kernels check and mark the one-launch decode's hand-off buffers
 * empty (one small fill kernel on stream, no host
 * synchronisation, no memset, so it can also sit in a captured graph).  Call
 * it once per workspace before its first decode, and again after the error
 * word turned nonzero.  Every decode leaves the synchronisation words as it
 * found them; prefill writes only GQA_WS_ERR_FP16_RANGE into the error word.
 * A decode on a workspace without the magic word writes NaN into its output
 * and sets GQA_WS_ERR_INIT.  The error word is the workspace's first int.
 * Errors: GQA_ERR_NULL, GQA_ERR_ALIGN, GQA_ERR_WORKSPACE, GQA_ERR_HIP.
 */
int gqa_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * gqa_decode_schedule -- the schedule a decode call with these arguments runs
 * when it asks for `schedule`: GQA_DECODE_SPLIT or GQA_DECODE_FUSED, or
 * GQA_ERR_ARG when the request is not one of the three schedules or is
 * GQA_DECODE_FUSED for a shape the one-launch schedule does not admit (the
 * decode call would fail with that code); GQA_ERR_SHAPE / GQA_ERR_RANGE for
 * invalid shapes.
 *
 * GQA_DECODE_SPLIT runs the three stages as three kernels.  GQA_DECODE_FUSED
 * runs the whole step as one kernel whose workgroups pass results to each
 * other through the workspace (Q/K/V -> attention -> wo), so that each
 * consumer's HBM reads overlap its producer's; it admits B <= 2 and
 * contexts that fit in at most 128 attention workgroups of at most 256
 * positions (the three-launch schedule's splits of 128 positions, fewer and
 * longer where they would be too many): start_pos + 1 <= 32768 / (n_kv_heads
 * * B), i.e. 4096 at 8 kv heads and B = 1, 2048 at 8 kv heads and B = 2 or
 * 16 and B = 1, 1024 at 16 and B = 2 or 32 and B = 1, 512 at 32 kv heads and
 * B = 2.  GQA_DECODE_AUTO takes the one-launch schedule
 * where it is admitted, except at B = 2 with 16 or 32 kv heads.  Where both
 * schedules split the positions alike (always below those lengths halved)
 * their results agree bit for bit; each is deterministic.
 */
int gqa_decode_schedule(int n_kv_heads, int B, int start_pos, int T_max, int schedule);

/*
 * gqa_wo_to_fp16 -- convert Wo [4096][4096] bf16 once into the fp16 copy that
 * prefill's output projection reads (entries beyond +-65504 saturate), so
 * that a caller running many prefills with one Wo does not pay the 32 MiB
 * conversion in every call.
 *   wo    [4096][4096] bf16 [out, in]
 *   wo16  [4096][4096] fp16, written (must not overlap wo)
 * Errors: GQA_ERR_NULL, GQA_ERR_ALIGN, GQA_ERR_ALIAS, GQA_ERR_HIP.
 */
int gqa_wo_to_fp16(const gqa_bf16* wo, uint16_t* wo16, hipStream_t stream);

/*
 * gqa_block_prefill -- the block over T new tokens of B sequences at
 * positions start_pos .. start_pos+T-1, with a causal mask.  start_pos = 0 is
 * the plain prefill; start_pos > 0 continues after start_pos rows already in
 * the caches (chunked prefill).  The page "Llama 3.1 8B . Grouped-query
 * attention" states the rule in the mask listing of its code section: new
 * token i sits at position start_pos + i and attends to every key
 * j <= start_pos + i, the cached rows included; RoPE uses the same absolute
 * positions.
 *   x          [B][T][4096] bf16, the block input
 *   wq         [4096][4096] bf16 [out, in]; wk, wv [n_kv_heads*128][4096];
 *              wo [4096][4096]
 *   wo16       NULL, or the fp16 copy of wo from gqa_wo_to_fp16 (then wo is
 *              not read; with NULL the call converts wo into the workspace)
 *   kcache, vcache   layouts above; rows 0 .. start_pos-1 of every sequence
 *              must hold the earlier tokens' keys and values (read, not
 *              written); rows start_pos .. start_pos+T-1 are written
 *   n_kv_heads 8, 16 or 32
 *   T_max      rows per sequence in the caches and the table
 *   rope       [T_max][64][2] fp32 from gqa_rope_table
 *   start_pos  0 .. T_max-T
 *   out        [B][T][4096] fp32, Delta_attn
 *   ws         workspace of ws_bytes >= gqa_workspace_bytes(GQA_OP_PREFILL,
 *              n_kv_heads, B, start_pos, T, T_max)
 *   probe      NULL, or [B][T][4096 + 2*n_kv_heads*128] fp32 receiving the
 *              post-RoPE Q | K and the V features exactly as computed before
 *              any rounding (for checking)
 *   events     NULL, or GQA_PREFILL_STAGES + 1 created hipEvent_t handles:
 *              events[0] is recorded on stream before the first kernel and
 *              events[i] after stage i, for timing each kernel
 * Aliasing: out, probe, ws and the caches must not overlap each other or the
 * inputs.
 * Errors: GQA_ERR_NULL, GQA_ERR_SHAPE, GQA_ERR_RANGE, GQA_ERR_ALIGN,
 * GQA_ERR_WORKSPACE, GQA_ERR_ALIAS, GQA_ERR_ARG (n_kv_heads), GQA_ERR_HIP.
 */
int gqa_block_prefill(const gqa_bf16* x,
                      const gqa_bf16* wq, const gqa_bf16* wk,
                      const gqa_bf16* wv, const gqa_bf16* wo, const uint16_t* wo16,
                      gqa_bf16* kcache, gqa_bf16* vcache, int n_kv_heads, int T_max,
                      const float* rope, int start_pos, int B, int T,
                      float* out, void* ws, size_t ws_bytes, float* probe,
                      hipEvent_t* events, hipStream_t stream);

/*
 * gqa_block_decode -- one new token per sequence at position start_pos (the
 * page's decode mode): writes cache row start_pos and attends over rows
 * 0..start_pos of each of the B sequences (one start_pos for all of them).
 *   x          [B][4096] bf16
 *   weights, caches, n_kv_heads, T_max, rope, probe ([B][4096 +
 *              2*n_kv_heads*128]) and events (GQA_DECODE_STAGES + 1; under
 *              the one-launch schedule events[1] follows its one kernel and
 *              the later events are recorded right after) as for prefill
 *   start_pos  0 .. T_max-1
 *   out        [B][4096] fp32: out = Delta when accumulate == 0,
 *              out += Delta when accumulate == 1 (the block residual
 *              h = x + attention(...), with the caller's fp32 residual in out)
 *   out_bf16   NULL, or [B][4096] bf16 receiving the bf16 rounding of out
 *              after the update (the next block's input in a stack of blocks)
 *   schedule   GQA_DECODE_AUTO, GQA_DECODE_SPLIT or GQA_DECODE_FUSED (see
 *              gqa_decode_schedule)
 *   ws         ws_bytes >= gqa_workspace_bytes(GQA_OP_DECODE, n_kv_heads, B,
 *              start_pos, 1, T_max), initialised once by gqa_workspace_init
 * Aliasing: out, out_bf16, probe, ws and the caches must not overlap each
 * other or the inputs.
 * Errors: as gqa_block_prefill; GQA_ERR_ARG for accumulate not 0/1 or a
 * schedule gqa_decode_schedule rejects.
 */
int gqa_block_decode(const gqa_bf16* x,
                     const gqa_bf16* wq, const gqa_bf16* wk,
                     const gqa_bf16* wv, const gqa_bf16* wo,
                     gqa_bf16* kcache, gqa_bf16* vcache, int n_kv_heads, int T_max,
                     const float* rope, int start_pos, int B,
                     float* out, gqa_bf16* out_bf16, int accumulate, int schedule,
                     void* ws, size_t ws_bytes, float* probe,
                     hipEvent_t* events, hipStream_t stream);

/*
 * gqa_block_decode_noalloc -- gqa_block_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid it): the same kernels, with the workspace taken from
 * the library's own scratch array instead of a ws argument.
 *   scratch    one array of GQA_NOALLOC_SCRATCH_BYTES (16 MiB) per GPU the
 *              library runs on, held until the process ends; its device
 *              address is looked up (hipGetSymbolAddress) on the first call on
 *              each device.  The call uses the CURRENT device's array, so
 *              `stream` must belong to the current device.
 *   limit      shapes whose decode workspace (gqa_workspace_bytes(
 *              GQA_OP_DECODE, ...)) exceeds the array fail with
 *              GQA_ERR_WORKSPACE before anything runs (B up to ~200 with 8 kv
 *              heads, ~64 with 32).
 *   other arguments as for gqa_block_decode (no ws, ws_bytes or events).
 * Each call first clears the array's synchronisation words with a small fill
 * kernel on `stream` (no memset), then runs the decode.  Every call on a GPU
 * shares that GPU's array, which keeps the last call's contents: calls that
 * overlap on one GPU (different streams without ordering) race and give
 * undefined results.  A timed-out wait shows only as NaN in `out` (the error
 * word is cleared by the next call).  Allocates nothing: no hipMalloc,
 * hipFree or allocating library routine.
 * Errors: as gqa_block_decode; GQA_ERR_WORKSPACE for shapes beyond the
 * scratch array; GQA_ERR_HIP when the device or the array's address cannot
 * be obtained.
 */
#define GQA_NOALLOC_SCRATCH_BYTES  (16u << 20)

int gqa_block_decode_noalloc(const gqa_bf16* x,
                             const gqa_bf16* wq, const gqa_bf16* wk,
                             const gqa_bf16* wv, const gqa_bf16* wo,
                             gqa_bf16* kcache, gqa_bf16* vcache, int n_kv_heads, int T_max,
                             const float* rope, int start_pos, int B,
                             float* out, gqa_bf16* out_bf16, int accumulate, int schedule,
                             float* probe, hipStream_t stream);

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
 *   ws       ws_bytes >= gqa_workspace_bytes(GQA_OP_LAYER_PREFILL or
 *            GQA_OP_LAYER_DECODE, ...); the normalised input lives at its end
 *   other arguments as for gqa_block_prefill / gqa_block_decode
 * Errors: those of the block calls; GQA_ERR_ARG for eps; GQA_ERR_ALIAS when h
 * overlaps x, norm_w or ws.
 */
int gqa_layer_prefill(const gqa_bf16* x, const gqa_bf16* norm_w, float eps,
                      const gqa_bf16* wq, const gqa_bf16* wk,
                      const gqa_bf16* wv, const gqa_bf16* wo, const uint16_t* wo16,
                      gqa_bf16* kcache, gqa_bf16* vcache, int n_kv_heads, int T_max,
                      const float* rope, int start_pos, int B, int T,
                      float* h, void* ws, size_t ws_bytes, float* probe,
                      hipStream_t stream);

int gqa_layer_decode(const gqa_bf16* x, const gqa_bf16* norm_w, float eps,
                     const gqa_bf16* wq, const gqa_bf16* wk,
                     const gqa_bf16* wv, const gqa_bf16* wo,
                     gqa_bf16* kcache, gqa_bf16* vcache, int n_kv_heads, int T_max,
                     const float* rope, int start_pos, int B,
                     float* h, gqa_bf16* h_bf16, int schedule,
                     void* ws, size_t ws_bytes, float* probe,
                     hipStream_t stream);

/*
 * gqa_vocab_logits -- the vocabulary projection of the page "Llama 3.1 8B .
 * Vocabulary projection": L = z W_out for one position of each of B
 * sequences, the weight stored [out, in] = [V][4096], no bias.  The page's
 * projection runs in the model's bf16 and its result is handed back as
 * float32, so each logit is the bf16 rounding (nearest even) of its
 * fp32-accumulated dot product, returned as fp32.  With norm_w non-NULL, z is
 * the final norm of the page's code (self.norm, an RMSNorm with norm_eps)
 * applied to h, read as in the layer pre-norm above; with NULL, z = h.
 *   h       [B][4096] bf16
 *   norm_w  NULL or [4096] bf16; eps as for the layers (ignored when NULL)
 *   w_out   [V][4096] bf16; V = 128256 for Llama 3.1 (1 .. GQA_MAX_VOCAB)
 *   logits  [B][V] fp32, written
 *   ws      needed only when B >= GQA_VOCAB_MFMA_MIN_B and norm_w is
 *           non-NULL (else it may be NULL, ws_bytes 0): ws_bytes >=
 *           gqa_workspace_bytes(GQA_OP_VOCAB, 8, B, 0, 1, 1); the normalised
 *           z is written after its synchronisation region, which is left
 *           untouched
 * Below GQA_VOCAB_MFMA_MIN_B sequences: a bandwidth GEMV over the weight
 * with the norm fused, one weight pass.  From there: the norm first (into
 * ws), then the matrix cores, one weight pass per 64 sequences.
 * Errors: GQA_ERR_NULL, GQA_ERR_SHAPE, GQA_ERR_ALIGN, GQA_ERR_ARG (eps),
 * GQA_ERR_WORKSPACE (ws missing or too small where needed), GQA_ERR_ALIAS
 * (logits or the used workspace overlapping an input or each other),
 * GQA_ERR_HIP.
 */
int gqa_vocab_logits(const gqa_bf16* h, const gqa_bf16* norm_w, float eps,
                     const gqa_bf16* w_out, int V, int B, float* logits,
                     void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H */
