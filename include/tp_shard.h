/*
 * tp_shard.h -- one rank's shard of a Megatron-style tensor-parallel
 * transformer layer, computed on one AMD Instinct MI355X (gfx950).
 *
 * The operation (undercodenews post 110319 on tensor parallelism in
 * transformers, section "the Original"; netray glossary "What Is Tensor
 * Parallelism?", section "Tensor Parallelism Explained"):
 *
 *   ATTN stage   n1 = RMSNorm(x)                        (replicated input)
 *                [q|k|v] = n1 * W_qkv,r^T                (column-parallel: rank r's heads)
 *                q,k rotated (RoPE); k,v stored in rank r's KV cache
 *                o = causal softmax(q k^T / sqrt(d)) v   (per local head, no communication)
 *                partial_attn = o * W_o[:, cols_r]^T     (row-parallel: one summand)
 *   reduce       h = x + sum_r partial_attn_r            (the all-reduce's sum)
 *   MLP stage    n2 = RMSNorm(h)
 *                act = SiLU(n2 W_gate,r^T) * (n2 W_up,r^T)   or GELU(n2 W_1,r^T)
 *                partial_mlp = act * W_down[:, F_r]^T    (row-parallel: one summand)
 *   reduce       y = h + sum_r partial_mlp_r
 *
 * Rank r owns contiguous blocks: query heads [r*H/t, (r+1)*H/t), KV heads
 * [r*Hkv/t, (r+1)*Hkv/t) and FFN columns [r*F/t, (r+1)*F/t).  Query head j
 * reads KV head floor(j / (H/Hkv)).  RoPE is rotate-half (pairs i, i+d/2),
 * theta_i = base^(-2i/d); prefill positions are 0..S-1, a decode token sits
 * at position L (the cache length before the call).  No biases.
 *
 * Conventions for every call:
 *  - Device pointers are HIP device addresses on the current device; host
 *    pointers are marked "host".  Activation, partial, residual and output
 *    pointers must be 16-byte aligned (TP_E_ARG otherwise).  Tensors are
 *    dense row-major, innermost dimension last.  Weight matrices are stored
 *    [out, in].
 *  - Element type: TP_BF16 (bfloat16 storage, fp32 arithmetic) or TP_F32,
 *    chosen at create time for activations, weights, KV cache and outputs.
 *    Partial sums are always fp32.
 *  - Ownership: the caller owns every pointer it passes and must keep the
 *    memory alive until the work enqueued on `stream` has completed.  The
 *    library owns the packed weight slices, the KV cache and its workspace
 *    and frees them in the matching *_destroy call.
 *  - Asynchrony: all device work is enqueued on `stream` (a hipStream_t;
 *    NULL means the null stream) and no call synchronises with the device,
 *    except that tp_shard_load_weights, tp_shard_reserve, tp_kv_create and
 *    the destroy calls may allocate or free device memory.
 *  - Errors: argument and state errors are detected on the host before any
 *    device work is enqueued and leave no side effects.  A failed HIP call
 *    returns TP_E_HIP; tp_status_string() then also reports the HIP error.
 *  - Handles are not thread-safe: use one handle from one host thread and
 *    one stream at a time.
 */
#ifndef TP_SHARD_H
#define TP_SHARD_H

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define TP_OK          0
#define TP_E_ARG      -1   /* bad pointer, size, layout or unsupported shape */
#define TP_E_DIVIDE   -2   /* heads, kv_heads or ffn not divisible by tp_degree, or tp_degree > heads */
#define TP_E_RANK     -3   /* rank outside [0, tp_degree) */
#define TP_E_NOMEM    -4   /* device or host allocation failed */
#define TP_E_HIP      -5   /* a HIP runtime call or kernel launch failed */
#define TP_E_KV_FULL  -6   /* the KV cache has no room for the tokens asked for */
#define TP_E_STATE    -7   /* call out of order (e.g. forward before weights are loaded) */
#define TP_E_SCRATCH  -8   /* the allocation-free entry point needs more than its static scratch */

/* element types */
#define TP_F32   0
#define TP_BF16  1

/* stages of a shard's forward pass */
#define TP_STAGE_ATTN  0
#define TP_STAGE_MLP   1
/* OR'ed into a stage: x is the already normalised stage input (the
 * sequence-parallel flow gathers the ranks' normalised rows, see
 * tp_shard_norm / tp_all_gather), so the stage skips its RMSNorm */
#define TP_STAGE_PRENORM 0x10

/* FFN activation */
#define TP_ACT_SWIGLU  0   /* act = SiLU(n W_gate^T) * (n W_up^T); three FFN matrices */
#define TP_ACT_GELU    1   /* act = GELU_erf(n W_up^T); two FFN matrices (w_gate unused) */

typedef struct tp_shard tp_shard;   /* opaque: one rank's packed weights + workspace */
typedef struct tp_kv    tp_kv;      /* opaque: K/V cache of one rank's KV heads      */

typedef struct {
    int   dtype;        /* TP_BF16 or TP_F32                                  */
    int   act;          /* TP_ACT_SWIGLU or TP_ACT_GELU                       */
    int   rmsnorm;      /* 1: RMSNorm (gamma g1/g2) before each stage; 0: none */
    float eps;          /* RMSNorm epsilon                                    */
    int   rope;         /* 1: rotate-half RoPE on q and k; 0: none            */
    float rope_theta;   /* RoPE base                                          */
    int   decode_fp8;   /* 1 (TP_BF16 only): also keep OCP E4M3 copies of the
                           four projection weights, one fp32 scale per row,
                           and decode one sequence (batch 1) from them      */
} tp_opts;

/* Full, unsharded layer weights (device pointers, element type = dtype):
 *   wq [heads*d, hidden], wk/wv [kv_heads*d, hidden], wo [hidden, heads*d],
 *   w_gate/w_up [ffn, hidden], w_down [hidden, ffn], g1/g2 [hidden].
 * Every rank is handed the same full weights and keeps only its slices
 * (column blocks of wq/wk/wv/w_gate/w_up, row-parallel column blocks of
 * wo/w_down).  w_gate is ignored for TP_ACT_GELU; g1/g2 for rmsnorm == 0. */
typedef struct {
    const void *wq, *wk, *wv, *wo, *w_gate, *w_up, *w_down, *g1, *g2;
} tp_weights;

/* tp_shard_create -- validate the partition and create rank `rank`'s shard
 * of a layer split `tp_degree` ways.  Host-only: no device call is made.
 * The split rules are the pages' (undercodenews post 110319, "the
 * Original": degree <= heads, heads % degree == 0, ffn % degree == 0) plus
 * kv_heads % degree == 0 so that KV heads split too (byteledger "Tensor
 * Parallelism: Splitting One Layer Across GPUs": the KV cache is split).
 * Violations return TP_E_DIVIDE; a rank outside [0, tp_degree) returns
 * TP_E_RANK.  Kernel limits return TP_E_ARG: hidden % heads == 0,
 * heads % kv_heads == 0, head_dim = hidden/heads in {64, 128},
 * hidden % 64 == 0, (ffn / degree) % 64 == 0.
 * opts == NULL selects {TP_BF16, TP_ACT_SWIGLU, rmsnorm 1, eps 1e-5, rope 1,
 * theta 10000, decode_fp8 0}.  decode_fp8 with TP_F32 returns TP_E_ARG.  *out receives the handle (host memory owned by the library). */
int tp_shard_create(int hidden, int heads, int kv_heads, int ffn,
                    int tp_degree, int rank, const tp_opts *opts,
                    tp_shard **out);

/* tp_shard_load_weights -- copy rank r's slices out of the full weights into
 * library-owned device memory, in the layout the kernels read (Q/K/V rows
 * of the rank's heads; gate/up rows of the rank's FFN columns interleaved
 * in 32-row blocks; the matching column blocks of wo and w_down).  Enqueued
 * on `stream`; the caller's weights may be freed once the stream has
 * drained.  May be called again to replace the weights.
 * With decode_fp8 it also quantises each packed matrix row by row: scale =
 * max|w| / 448 (1 for a zero row), code = the E4M3 value nearest to the
 * fp32 quotient w / scale (clamped to +-448), ties to the even code.  The
 * pages leave any quantisation open (netray glossary "What Is Tensor
 * Parallelism?", "In Practice": quantising as the alternative to
 * sharding); this per-row scheme is the library's. */
int tp_shard_load_weights(tp_shard *s, const tp_weights *full, void *stream);

/* tp_shard_reserve -- pre-size the workspace for calls of up to
 * `max_tokens` = batch * seq tokens (and decode batches up to that size),
 * so that later forward calls allocate nothing.  Forward calls grow the
 * workspace on demand otherwise (which frees the old one and therefore
 * waits for the device). */
int tp_shard_reserve(tp_shard *s, long long max_tokens);

/* tp_kv_create -- KV cache for this rank's kv_heads/t heads (the KV cache
 * is split across the devices like the heads: byteledger "Tensor
 * Parallelism: Splitting One Layer Across GPUs", "Interaction with the rest
 * of serving"):
 * K and V each [batch, kv_heads/t, max_seq, head_dim] in the shard's dtype,
 * zero-filled, length 0.  TP_F32 caches hold at most 16000 positions. */
int tp_kv_create(const tp_shard *s, int batch, int max_seq, tp_kv **out);

/* tp_kv_create_paged -- paged KV cache (TP_BF16 shards): K and V are pools
 * of `num_blocks` blocks, each [kv_heads/t, block_size, head_dim], and a
 * block table [batch, ceil(max_seq / block_size)] of block ids maps
 * position p of sequence b to block table[b][p / block_size], row
 * p % block_size.  The pages' serving context names paged attention as the
 * memory structure a tensor-parallel split applies to (byteledger "Tensor
 * Parallelism: Splitting One Layer Across GPUs", "Interaction with the rest
 * of serving"); this layout is the library's.  block_size is a power of two
 * in [16, 1024].  Until tp_kv_set_block_table, sequence b uses blocks
 * b * max_blocks + i (block 0 where that exceeds the pool).  Prefill writes
 * the prompt's K/V rows into the pages; decode appends and attends through
 * the table.  Zero-filled, length 0. */
int tp_kv_create_paged(const tp_shard *s, int batch, int max_seq, int block_size, int num_blocks,
                       tp_kv **out);

/* tp_kv_set_block_table -- copy a HOST table [batch, ceil(max_seq / block_size)]
 * of block ids in [0, num_blocks) to the cache (waits for the device first).
 * Sequences may share no block they write to.  TP_E_ARG for an id out of
 * range, TP_E_STATE for a contiguous cache. */
int tp_kv_set_block_table(tp_kv *kv, const int *host_table);

/* tp_kv_view -- device pointers to the K and V arrays (layout above; the
 * pools of a paged cache), e.g. to fill a cache with synthetic content.
 * Either output may be NULL. */
int tp_kv_view(tp_kv *kv, void **k, void **v);

/* tp_kv_set_len / tp_kv_get_len -- number of valid positions [0, len).
 * The length lives in device memory, where the kernels read and advance it
 * (so a decode call captured in a HIP graph stays correct on replay), next
 * to an overflow flag that a decode call raises when it finds the length at
 * max_seq and so appends nothing; the library also keeps a host copy of the
 * length for its capacity checks.  Both calls wait for the whole device
 * first (hipDeviceSynchronize: they are set-up and inspection calls, not
 * part of a step), then copy.  set_len also clears the overflow flag
 * (TP_E_ARG if len > max_seq); get_len refreshes the host copy, stores the
 * length in *len and returns TP_E_KV_FULL if the flag has been raised since
 * the last set_len or prefill (only replayed or host-stale calls can raise
 * it: an eager call on a full cache is refused up front). */
int tp_kv_set_len(tp_kv *kv, int len);
int tp_kv_get_len(const tp_kv *kv, int *len);

/* tp_kv_set_len_async / tp_kv_get_len_stream -- the same, ordered on
 * `stream` instead of waiting for the whole device.  set_len_async writes
 * the length and clears the overflow flag with a one-thread kernel on the
 * stream (no host wait; it may be captured in a HIP graph, which records a
 * kernel node, not a memset) and updates the host copy at once, so a
 * forward call queued after it on the same stream sees the new length;
 * TP_E_ARG as set_len.  get_len_stream copies the length on the stream and
 * waits for that stream only, then behaves as get_len.  The caller orders
 * other streams that use the cache. */
int tp_kv_set_len_async(tp_kv *kv, int len, void *stream);
int tp_kv_get_len_stream(const tp_kv *kv, int *len, void *stream);

/* tp_shard_forward_prefill -- one stage over a prompt batch.  The stages
 * are the pages' split of a layer (undercodenews post 110319 on tensor
 * parallelism in transformers, "the Original"): ATTN = the column-parallel
 * Q/K/V projection over the rank's own heads, attention per head with no
 * communication, and the row-parallel output projection whose result is a
 * partial sum; MLP = the column-parallel first FFN linear with its
 * activation and the row-parallel second linear, again a partial sum.  The
 * stage boundary is where the all-reduce of the partials must happen before
 * the layer can go on (byteledger "Tensor Parallelism: Splitting One Layer
 * Across GPUs", "Communication is the constraint").  A prompt runs the same
 * layer over many tokens at once (clusterbid "When Tensor Parallelism Makes
 * a Small Model Slower", the prefill paragraph).
 *   stage TP_STAGE_ATTN: x = layer input [batch, seq, hidden]; positions
 *     0..seq-1; K/V of the rank's heads are written to kv positions
 *     [0, seq) and the cache length becomes seq (kv may be NULL: K/V then
 *     live in the workspace only).  Requires seq <= max_seq.
 *   stage TP_STAGE_MLP: x = reduced h [batch, seq, hidden]; kv must be NULL.
 *   partial [batch, seq, hidden] fp32 receives this rank's summand. */
int tp_shard_forward_prefill(tp_shard *s, int stage, const void *x,
                             int batch, int seq, tp_kv *kv, float *partial,
                             void *stream);

/* tp_shard_forward_decode -- one stage for one new token per sequence.
 * Decode is a sequence of one-token steps through the same layer
 * (clusterbid "When Tensor Parallelism Makes a Small Model Slower", the
 * decode paragraph); each step's ATTN stage reads and extends the rank's
 * split of the KV cache (byteledger "Tensor Parallelism: Splitting One
 * Layer Across GPUs", "Interaction with the rest of serving").
 *   stage TP_STAGE_ATTN: x [batch, hidden] sits at position L = the cache
 *     length; its k, v are appended at slot L, the query attends to
 *     positions 0..L, and the cache length becomes L+1.  TP_E_KV_FULL if
 *     the host copy of L equals max_seq; batch must equal the cache's batch.
 *   stage TP_STAGE_MLP: x = reduced h [batch, hidden]; kv must be NULL.
 *     TP_E_STATE if no ATTN stage (prefill or decode) has run on this shard.
 *   partial [batch, hidden] fp32 receives this rank's summand.
 * Graph capture (TP_BF16 only): the kernels take L from the cache's device
 * length and advance it themselves, the attention grid and the workspace are
 * sized by max_seq, so a captured sequence of decode calls may be replayed;
 * each replay appends one token per captured ATTN call.  Make one eager call
 * of the same shape first (it sizes the workspace and the rotary table: no
 * allocation may happen during capture).  Capture leaves the host copy of
 * the length alone.  A replay past max_seq appends nothing, attends over the
 * first max_seq positions and raises the cache's overflow flag, which
 * tp_kv_get_len reports (TP_E_KV_FULL); the host copy of the length is
 * refreshed by tp_kv_get_len.  TP_F32 shards return TP_E_STATE on a
 * capturing stream. */
int tp_shard_forward_decode(tp_shard *s, int stage, const void *x, int batch,
                            tp_kv *kv, float *partial, void *stream);

/* tp_shard_forward_decode_noalloc -- tp_shard_forward_decode for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments, kernels,
 * results and errors, but no call to hipMalloc, hipFree or any allocating
 * routine: every intermediate (normalised input, q, attention output and
 * split-KV records, FFN activation, split-K partials) lives in one static
 * device array of TP_NOALLOC_SCRATCH_BYTES that the library holds on every
 * device it runs on until the process ends; its address on a device is
 * looked up at tp_shard_load_weights.  TP_BF16 shards only (TP_E_STATE for
 * TP_F32).  Returns TP_E_SCRATCH, before any launch, when the call's
 * workspace -- set by batch, the shard's widths and, for ATTN, the cache's
 * max_seq -- exceeds the array (e.g. 7B-shaped t=4: batch 1 up to ~1.8M
 * cached positions; 70B-shaped t=8, batch 1, up to ~250k positions).
 * Every call on a device shares that device's array and finds the previous
 * call's contents in it; no part of it needs to start at zero.  Calls that
 * overlap on one device (two streams, or two threads) race on it. */
#define TP_NOALLOC_SCRATCH_BYTES (32 << 20)
int tp_shard_forward_decode_noalloc(tp_shard *s, int stage, const void *x, int batch,
                                    tp_kv *kv, float *partial, void *stream);

/* tp_shard_forward_prefill_reduce -- tp_shard_forward_prefill followed by
 * tp_partial_reduce of its result with the other ranks' partials, as one
 * call.  Each stage of a layer ends with the all-reduce of the row-parallel
 * partials, and the next stage cannot start before it (byteledger "Tensor
 * Parallelism: Splitting One Layer Across GPUs", "Communication is the
 * constraint"; undercodenews post 110319, "the Original": the all-reduce
 * follows the row-parallel output projection and the FFN's second linear).
 * Here the sum is folded into the epilogue of the stage's row-parallel
 * projection (bf16 shards with tp_degree <= 8), so this rank's partial is
 * never stored; otherwise the partial goes to the workspace and the reduce
 * runs after it.
 *   out[i] = (sum_{r<t} P_r[i]) + residual[i], in rank order in fp32, then
 *   stored in the shard's dtype (bf16 rounds to nearest even), where
 *   P_rank is this call's own partial and P_r = partials[r] otherwise.
 * The result equals tp_shard_forward_prefill + tp_partial_reduce bit for bit.
 *   partials: HOST array of tp_degree device pointers, each [batch, seq,
 *     hidden] fp32, 16-byte aligned; entry `rank` is not read (may be NULL);
 *     a NULL entry for another rank (a lost rank) returns TP_E_ARG.
 *   residual: [batch, seq, hidden] in the shard's dtype, or NULL for none;
 *     may alias out.
 *   out: [batch, seq, hidden] in the shard's dtype; must not overlap x or
 *     another rank's partial (TP_E_ARG).
 * The next stage's norm is not applied (the stage that follows normalises
 * its input unless called with TP_STAGE_PRENORM).  Stages, cache handling
 * and errors as tp_shard_forward_prefill. */
int tp_shard_forward_prefill_reduce(tp_shard *s, int stage, const void *x, int batch, int seq, tp_kv *kv,
                                    const float *const *partials, const void *residual, void *out,
                                    void *stream);

/* tp_shard_forward_decode_reduce -- tp_shard_forward_decode followed by
 * tp_partial_reduce of its result with the other ranks' partials, as one
 * call.  Each decode step of a layer ends both stages with the all-reduce of
 * the row-parallel partials, and every rank waits on it before the next
 * projection (byteledger "Tensor Parallelism: Splitting One Layer Across
 * GPUs", "Communication is the constraint"; undercodenews post 110319, "the
 * Original": the all-reduce follows the row-parallel output projection and
 * the FFN's second linear).  Here the sum is folded into the epilogue of the
 * stage's row-parallel projection (batch 1..64 on bf16 shards with
 * tp_degree <= 8), so this rank's partial is never stored; otherwise the
 * partial goes to the workspace and the reduce runs after it.
 *   out[i] = (sum_{r<t} P_r[i]) + residual[i], in rank order in fp32, then
 *   stored in the shard's dtype (bf16 rounds to nearest even), where
 *   P_rank is this call's own partial and P_r = partials[r] otherwise.
 * The result equals tp_shard_forward_decode + tp_partial_reduce bit for bit.
 *   partials: HOST array of tp_degree device pointers, each [batch, hidden]
 *     fp32, 16-byte aligned; entry `rank` is not read (may be NULL); a NULL
 *     entry for another rank (a lost rank) returns TP_E_ARG.
 *   residual: [batch, hidden] in the shard's dtype, or NULL for none; may be
 *     x (the ATTN stage's residual is its input) and may alias out.
 *   out: [batch, hidden] in the shard's dtype; must not overlap x
 *     (TP_E_ARG) or any partial.
 * Stages, cache handling, graph capture and errors as tp_shard_forward_decode. */
int tp_shard_forward_decode_reduce(tp_shard *s, int stage, const void *x, int batch, tp_kv *kv,
                                   const float *const *partials, const void *residual, void *out,
                                   void *stream);

/* tp_partial_reduce -- the all-reduce's arithmetic on one device.  A
 * row-parallel linear leaves each rank with a partial result that an
 * all-reduce sums (undercodenews post 110319, "the Original"; netray
 * glossary "What Is Tensor Parallelism?", "Tensor Parallelism Explained");
 * here the t ranks' partials are resident on one device and summed by one
 * kernel:
 *   out[i] = (sum_{r=0..t-1} partials[r][i]) + residual[i]
 * summed in fp32 in rank order, then stored as out_dtype (TP_BF16 rounds to
 * nearest even).  `partials` is a HOST array of t device pointers, each to
 * n fp32 values; residual and out hold n elements of out_dtype (residual
 * may be NULL for none; out may alias residual).  1 <= t <= 64; a NULL
 * entry (a lost rank) returns TP_E_ARG.  n == 0 returns TP_OK and touches
 * no pointer. */
int tp_partial_reduce(const float *const *partials, int t,
                      const void *residual, void *out, long long n,
                      int out_dtype, void *stream);

/* tp_shard_reduce_norm -- the reduce of a stage's partials together with
 * the RMSNorm that the next stage applies to its result, in one pass over
 * `rows` rows of `hidden` values:
 *   out[i]      = (sum_{r<t} partials[r][i]) + residual[i]      (as tp_partial_reduce)
 *   norm_out[i] = RMSNorm(out[i]) * gain                       (as tp_shard_norm)
 * with the shard's gain g1 (which = 1: the input of an ATTN stage, e.g. the
 * next layer's) or g2 (which = 2: this layer's MLP stage); both stored in the
 * shard's dtype, the norm taken of the stored out.  The partials must be
 * combined before the layer can go on (byteledger "Tensor Parallelism:
 * Splitting One Layer Across GPUs", "Communication is the constraint"), and
 * the next stage's first step normalises exactly that result, so the two
 * share one read of it.  Feed norm_out to the next stage with
 * TP_STAGE_PRENORM.  bf16 shards with hidden <= 8192 take one fused kernel
 * whose results equal the two separate calls bit for bit; other shards run
 * those two calls.  Layout and alignment as tp_partial_reduce (partials: HOST
 * array of t device pointers to [rows, hidden] fp32; residual may be NULL);
 * TP_E_STATE before tp_shard_load_weights; rows == 0 touches nothing. */
int tp_shard_reduce_norm(tp_shard *s, int which, const float *const *partials, int t, const void *residual,
                         void *out, void *norm_out, long long rows, void *stream);

/* tp_shard_fp8_view -- device addresses of the E4M3 copy of a packed weight
 * (which = 0 Q/K/V [(heads+2 kv_heads)/t * d, hidden], 1 W_o block
 * [hidden, heads/t * d], 2 gate/up [2 ffn/t (ffn/t for GELU), hidden],
 * 3 W_down block [hidden, ffn/t]; rows in the packed order described at
 * tp_shard_load_weights), its per-row fp32 scales and its shape.
 * TP_E_STATE without decode_fp8 or before tp_shard_load_weights. */
int tp_shard_fp8_view(tp_shard *s, int which, void **codes, float **scales, int *rows, int *cols);

/* Sequence-parallel variant (undercodenews post 110319, "What Undercode
 * Say": tensor parallelism is paired with sequence parallelism).  Between
 * the stages the activations are split by token: rank r holds rows
 * [r T/t, (r+1) T/t) of the flattened [T = batch*seq, hidden] tensor.
 *
 * tp_partial_reduce_scatter -- rank `rank`'s rows of the reduce:
 *   out_rows[i] = (sum_{r<t} partials[r][rank * n + i]) + residual_rows[i],
 *   n = rows / t * cols, summed in fp32 in rank order, stored as out_dtype.
 *   partials: HOST array of t device pointers to [rows, cols] fp32;
 *   residual_rows (may be NULL) and out_rows: [rows / t, cols] of out_dtype.
 *   rows % t != 0 returns TP_E_DIVIDE; cols must be a multiple of 8.
 * tp_all_gather -- out [t * rows_per_rank, cols] = the t pieces (HOST array
 *   of device pointers, each [rows_per_rank, cols] of dtype) in rank order.
 *   cols * element size must be a multiple of 16.
 * tp_shard_norm -- out = RMSNorm(x) with the shard's gain g1 (which = 1) or
 *   g2 (which = 2) over `rows` rows of hidden values (a copy of x if the
 *   shard has no norm).  All pointers 16-byte aligned; enqueued on stream. */
int tp_partial_reduce_scatter(const float *const *partials, int t, int rank, const void *residual_rows,
                              void *out_rows, long long rows, int cols, int out_dtype, void *stream);
int tp_all_gather(const void *const *pieces, int t, long long rows_per_rank, int cols, int dtype, void *out,
                  void *stream);
int tp_shard_norm(tp_shard *s, int which, const void *x, long long rows, void *out, void *stream);

/* tp_shard_debug_view -- device address of a workspace tensor from the last
 * forward call, for diagnostics: which = 0 attention output o
 * [tokens, heads/t * d]; 1 FFN activation act [tokens, ffn/t]; 2 the
 * normalised stage input [tokens, hidden].  The contents are valid until
 * the next forward call on this shard. */
int tp_shard_debug_view(tp_shard *s, int which, void **ptr);

/* Kernel timer (diagnostics): while enabled, every kernel a forward call
 * launches is bracketed by two hipEvents recorded on the launch stream, and
 * the elapsed times are summed per kernel kind.  Recording adds a marker
 * between kernels, so time whole steps with the timer off.
 * tp_shard_timing(s, mask) enables and resets the sums (it creates the event
 * pool on first use): mask -1 brackets every kernel kind, any other nonzero
 * mask only the kinds k with bit (1 << k) set (TP_K_MASK), so that a timed
 * run can bracket just the kernel of interest; tp_shard_timing(s, 0) stops
 * recording.
 * tp_shard_timing_read waits for the recorded events and returns the total
 * milliseconds and launch count of one kernel kind (TP_K_*). */
#define TP_K_RMSNORM      0
#define TP_K_GEMM_QKV     1
#define TP_K_ATTN_PREFILL 2
#define TP_K_GEMM_OUT     3
#define TP_K_GEMM_UP      4
#define TP_K_GEMM_DOWN    5
#define TP_K_GEMV_QKV     6
#define TP_K_ATTN_DECODE  7
#define TP_K_GEMV_OUT     8
#define TP_K_GEMV_UP      9
#define TP_K_GEMV_DOWN    10
#define TP_K_REDUCE_NORM  11
#define TP_K_COUNT        12
#define TP_K_MASK(k)      (1 << (k))
int tp_shard_timing(tp_shard *s, int enable);
int tp_shard_timing_read(tp_shard *s, int kernel, double *total_ms, long long *launches);

/* tp_tune_set_gemm_config -- tuning hook: force the projection GEMM's tile
 * configuration for every later call in this process, or -1 to restore the
 * shape-based choice.  0..2: register-staged 256x128, 128x128, 128x256
 * output tiles; 3..10: direct-to-LDS rings 256x256 (K-step 64, 2 stages),
 * 256x256 (32, 4), 256x128 (64, 3), 128x128 (64, 4), 128x128 (64, 2),
 * 256x128 (32, 4), 128x384 (32, 4), 128x384 (32, 3); 11..13: register-
 * pipelined 256x256, 256x128 and 256x192 (K-step 64, eight waves); 14..16:
 * producer/consumer 256x256, 256x192 and 256x128 (eight MFMA waves, four
 * load waves); 17, 18: producer/consumer 256x192 and 256x128 with four MFMA
 * waves of 64x192 and 64x128.
 * A configuration that a projection cannot use (the 256x256 DMA rings and
 * configuration 17 with the rotary epilogue, the two-stage ring also with
 * the GELU and plain-store ones) falls back to the shape-based choice.
 * Process-wide, not thread-safe.
 * TP_E_ARG if out of range. */
int tp_tune_set_gemm_config(int cfg);

/* Projection kinds of the planner hooks below (the epilogue each applies). */
#define TP_PROJ_PARTIAL 0   /* out and down projections: fp32 partial   */
#define TP_PROJ_QKV     1   /* Q/K/V with the rotary epilogue           */
#define TP_PROJ_SWIGLU  2   /* gate/up with SwiGLU                      */
#define TP_PROJ_GELU    3   /* up projection with GELU                  */

/* tp_tune_gemm_plan -- host only, no device call: the launch plan that a
 * bf16 projection C[M, N] = A[M, K] B[N, K]^T of kind `proj` takes under the
 * current tuning hooks.  *parts receives 1 or 2 (launches over column
 * ranges), cfg[i] the tile configuration of launch i (the numbering of
 * tp_tune_set_gemm_config, -1 for no second launch) and ncols[i] its column
 * count (0 for none).  TP_E_ARG for non-positive sizes, a NULL output or an
 * unknown kind. */
int tp_tune_gemm_plan(int M, int N, int K, int proj, int *parts, int cfg[2], int ncols[2]);

/* tp_tune_set_gemm_split -- tuning and test hook: every later bf16
 * projection wider than cols0 columns runs as two launches, columns
 * [0, cols0) with tile configuration cfg0 and the others with cfg1 -- the
 * form the planner itself takes when a shape's last round of tiles would be
 * mostly idle.  cols0 = 0 restores the planner.  cols0 must be a multiple of
 * 64 (a rotary or gate/up column group never straddles the split); a
 * configuration that a projection cannot use leaves that projection to the
 * planner.  Process-wide, not thread-safe.  TP_E_ARG otherwise. */
int tp_tune_set_gemm_split(int cfg0, int cfg1, int cols0);

/* tp_tune_set_attn_groups -- tuning hook for prefill attention: 1 runs each
 * 128-query block with one group of four waves over all its key blocks, 2
 * with two groups over alternate key blocks whose softmax states merge at
 * the end (same result up to rounding order), 0 restores the choice by grid
 * size (two groups up to 512 work-groups).  Process-wide, not thread-safe.
 * TP_E_ARG outside 0..2. */
int tp_tune_set_attn_groups(int kg);

/* tp_tune_set_attn_kernel -- tuning hook for prefill attention: 1 runs the
 * kernel that stages each key block through registers into one LDS stage per
 * key group (two barriers per key block), 2 the software-pipelined kernel
 * (the default: K and V loaded straight into two LDS stages each, one barrier
 * per key block, the scores of the next block computed under the
 * exponentials of this one), 0 restores the default.  Same results up to
 * rounding order.  Process-wide, not thread-safe.  TP_E_ARG outside 0..2. */
int tp_tune_set_attn_kernel(int k);

/* tp_tune_set_decode_chunk -- tuning hook for bf16 decode attention: 16, 32
 * or 64 cached positions per chunk work-group (32 at least for head dim 64;
 * the split kernel for one query head per KV head always takes 64), or 0 to
 * restore the choice by grid size.  The workspace follows the chunk size on
 * the next call.  Process-wide, not thread-safe; TP_E_ARG for other values. */
int tp_tune_set_decode_chunk(int ch);

/* tp_tune_set_decode_attn -- tuning hook for bf16 decode attention:
 * 1 runs chunk work-groups that cover all query heads of a KV head, then a
 * merge launch; 2 runs one query head per chunk work-group and merges in
 * the same launch (the last chunk work-group of each sequence and head,
 * found with a device-scope release and an atomic count, merges the head's
 * chunks); 3 (also what 0, the default, restores) runs one query head per
 * chunk work-group, then a merge launch.  Same result up to rounding order.
 * Process-wide, not thread-safe; TP_E_ARG outside 0..3. */
int tp_tune_set_decode_attn(int mode);

void tp_shard_destroy(tp_shard *s);
void tp_kv_destroy(tp_kv *kv);

/* tp_status_string -- static text for a status code; for TP_E_HIP it names
 * the last HIP error seen by this library (thread-local). */
const char *tp_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* TP_SHARD_H */
