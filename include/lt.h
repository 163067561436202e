/*
 * lt.h -- C ABI of the LightTransfer-Test hot path on MI355X (gfx950).
 *
 * LightTransfer-Test converts a dense transformer into a hybrid one during
 * prefill: each layer's "lazy ratio" -- the softmax mass its last W queries
 * put on the S initial (sink) keys plus each query's R most recent keys -- is
 * measured as the layer runs, a priority queue keyed by that ratio keeps at
 * most C layers at full KV, and every layer the queue evicts has its KV cut
 * to the sink + recent slice and runs streaming attention from then on.
 * Sources, by page and section:
 *   [P1] Chinese write-up (xzbcqc.com): "problem 1 / solution 1" -- Flash
 *        Attention stores no attention weights; its LSE is the ratio's
 *        denominator and the numerator costs O(1) per query instead of an
 *        O(seq_len) recompute.  "problem 2 / solution 2" -- the priority
 *        queue that bounds peak prefill memory at 50% full KV + 50%
 *        streaming KV by evicting the highest-ratio layer on overflow.
 *   [P3] Press-release page (wuwenjie.xyz): "LightTransfer method" -- the
 *        lazy ratio sums the attention weights from queries to the initial
 *        and the recent keys; offline, the layers are measured on a set of
 *        prompts and the highest-ratio half replaced.
 *   [P4] LightTransfer project page: "Introduction" (lazy layers become
 *        streaming attention with a constant-size KV cache); Figure 2 caption
 *        (queue of (lazy ratio, layer index) updated after every layer; the
 *        evicted layer's KV cache is reduced).
 *
 * Conventions shared by every call
 *   Shapes: B batch, N sequence length (queries = keys, causal, aligned at
 *   position 0: key j is visible to query i iff j <= i), Hq query heads, Hkv
 *   KV heads with Hq % Hkv == 0 (query head h reads KV head h / (Hq/Hkv)),
 *   D head dim (64 or 128).  The recent set of query i is (i-R, i], the sink
 *   set [0, S); every call that takes them needs S >= 0, R >= 1 and
 *   S + R <= 2^30 (LT_ERR_SHAPE otherwise).
 *   Views: lt_view.data is a DEVICE pointer; sb, sh, sn are element strides of
 *   the batch, head and row dims; the head dim is contiguous.  Data pointers
 *   must be 16-byte aligned and strides multiples of 8 elements (bf16) or 4
 *   (f32), so 128-bit loads are legal; a row stride sn may not exceed 2^25
 *   elements (the attention kernels keep a lane's offset into a K/V tile in
 *   32 bits).  Sizes: N * (Hq/Hkv) must stay below 2^31 - 4096 and
 *   B * Hq * N at or below 2^38 (LT_ERR_SHAPE otherwise).
 *   Ownership: the caller owns every buffer (device memory and workspace);
 *   the library never allocates or frees device memory.
 *   Streams: device calls are asynchronous on the given stream, never
 *   synchronise, and write their outputs only; results are valid once the
 *   stream reaches that point.
 *   Errors: every argument is checked before anything is launched, so any
 *   status other than LT_ERR_HIP leaves every output untouched.  LT_ERR_HIP
 *   means the HIP runtime refused a launch; a call that launches several
 *   kernels (prefill with W > 0, decode) may then already have queued the
 *   earlier ones, so its outputs can be partly written.  A stale error left
 *   in the calling thread's HIP error state by unrelated earlier work is
 *   cleared before the first launch and not reported.  lt_last_error()
 *   returns the calling thread's last message.  Nothing throws or aborts.
 */
#ifndef LT_H
#define LT_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
    LT_OK = 0,
    LT_ERR_NULL = 1,      /* a required pointer is NULL */
    LT_ERR_SHAPE = 2,     /* sizes out of range or inconsistent */
    LT_ERR_DTYPE = 3,     /* unsupported dtype or head dim */
    LT_ERR_LAYOUT = 4,    /* misaligned pointer or stride */
    LT_ERR_WORKSPACE = 5, /* workspace too small */
    LT_ERR_HIP = 6,       /* the HIP runtime reported an error at launch */
    LT_ERR_VALUE = 7      /* bad value: NaN/inf score, capacity outside [0, L], layer out of order */
};

/* Element types. */
enum { LT_F32 = 0, LT_BF16 = 1 };

/* A strided [B, H, rows, D] tensor in device memory (element strides). */
typedef struct {
    void *data;
    int64_t sb, sh, sn;
} lt_view;

/* Prefill problem shape.  scale <= 0 selects 1/sqrt(D). */
typedef struct {
    int B, N, Hq, Hkv, D;
    int dtype; /* LT_F32 or LT_BF16; q, k, v and out share it */
    float scale;
} lt_shape;

/*
 * Causal GQA flash-attention prefill that also returns the per-row LSE and,
 * in the same call, each head's lazy ratio ([P1] solution 1, [P3] method).
 *   q [B,Hq,N,D], k/v [B,Hkv,N,D], out [B,Hq,N,D]: views as above.
 *   lse [B,Hq,N] fp32, contiguous, natural log: ln sum_{j<=i} exp(s_ij),
 *     s_ij = scale * q_i . k_j.  Required.
 *   W == 0: plain prefill; lazy_rows/lazy_ratio are ignored (may be NULL).
 *   W >= 1 (W <= N): lazy_rows [B,Hq,W] fp32 receives, for the last W
 *     queries i = N-W..N-1, r_i = sum over keys j <= i with j < S or
 *     j > i-R of exp(s_ij - lse_i); lazy_ratio [B,Hq] fp32 receives the mean
 *     of the W values, summed in row order.  Both required.  The numerator is
 *     summed in the main pass, on the sink and recent key steps of the
 *     observed rows only, next to the softmax sum that gives the LSE.
 *   Needs S >= 0, R >= 1.  bf16 runs on the matrix cores (fp32 accumulate,
 *   softmax weights rounded to bf16 for the P.V product); f32 runs in fp32.
 */
int lt_prefill_attn_lse_lazy(const lt_shape *shape, lt_view q, lt_view k, lt_view v,
                             lt_view out, float *lse, int S, int R, int W, float *lazy_rows,
                             float *lazy_ratio, hipStream_t stream);

/*
 * Streaming (sink + sliding-window) attention of converted layers ([P4]
 * introduction; [P1] training paragraph): query i attends only to keys
 * j <= i with j < S or j > i-R.  Same layouts as the prefill; lse [B,Hq,N]
 * fp32 may be NULL.  Needs S >= 0, R >= 1.
 */
int lt_streaming_attn(const lt_shape *shape, lt_view q, lt_view k, lt_view v, lt_view out,
                      float *lse, int S, int R, hipStream_t stream);

/*
 * Workspace for lt_hybrid_decode_attn at these sizes, in bytes: the split
 * partial states, (parts + B - 1) * Hq * (D + 2) fp32.  The number of parts
 * is chosen per (sequence, KV head) unit, so the size depends on Hkv as well
 * as on B, Hq, D and kv_len.  The same size also serves
 * lt_hybrid_decode_attn_varlen with max_kv_len = kv_len.  Host-only; no
 * device call.  Errors: LT_ERR_NULL, LT_ERR_SHAPE, LT_ERR_DTYPE (D).
 */
int lt_hybrid_decode_workspace_bytes(int B, int Hq, int Hkv, int D, int64_t kv_len,
                                     size_t *bytes);

/*
 * One decode step of one layer over its KV cache (full or streaming): the
 * KV reduction the pages report is realised here ([P1] training paragraph,
 * [P3] results).  q [B,Hq,D] contiguous (device), k_cache/v_cache views
 * [B,Hkv,>=kv_len,D]; every one of the kv_len rows is attended (the cache
 * includes the current token; row order is irrelevant).  A full layer passes
 * its whole context; a streaming layer passes its S+R-row cache.
 *   out [B,Hq,D] contiguous, same dtype as q; lse [B,Hq] fp32 or NULL.
 *   ws: device workspace of at least lt_hybrid_decode_workspace_bytes().
 */
int lt_hybrid_decode_attn(int B, int Hq, int Hkv, int D, int dtype, float scale, const void *q,
                          lt_view k_cache, lt_view v_cache, int64_t kv_len, void *out, float *lse,
                          void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * lt_hybrid_decode_attn without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments, outputs,
 * kernels and results as lt_hybrid_decode_attn (bit for bit); the split
 * partial states go to a fixed scratch array the library holds on each GPU
 * (LT_DECODE_NOALLOC_SCRATCH_BYTES, kept until the process ends).  Sizes
 * whose workspace (lt_hybrid_decode_workspace_bytes) exceeds that are
 * LT_ERR_WORKSPACE, checked before anything else touches the GPU.  Runs on
 * the current device (the stream must belong to it); the first call on a
 * device looks up that device's array (LT_ERR_HIP if that fails).  Nothing
 * is allocated and no memory is cleared (every partial state is written
 * before it is read).  Every call on one GPU shares that GPU's array: calls
 * that may overlap in time there (on different streams, or from different
 * threads without ordering) race and can give wrong results; calls on one
 * stream run one after the other and are safe.
 */
#define LT_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int lt_hybrid_decode_attn_noalloc(int B, int Hq, int Hkv, int D, int dtype, float scale,
                                  const void *q, lt_view k_cache, lt_view v_cache, int64_t kv_len,
                                  void *out, float *lse, hipStream_t stream);

/*
 * Switch a layer's KV to the streaming version ([P1] solution 2; [P4]
 * Figure 2): copy the rows of positions [0,S) and [N-R,N) of every (b, kv
 * head) of k_full / v_full [B,Hkv,N,D] into k_stream / v_stream
 * [B,Hkv,>=min(N,S+R),D]: position p < S into slot p, a recent position p
 * into slot S + (p-S) mod R (a ring of R slots, so that decode can append in
 * place with lt_stream_cache_append); when N <= S+R every row p goes to slot
 * p.  Attention over the cache does not depend on the slot order.  A byte
 * copy; the caller frees the full buffers afterwards.
 */
int lt_compact_kv_streaming(lt_view k_full, lt_view v_full, lt_view k_stream, lt_view v_stream,
                            int B, int Hkv, int N, int D, int dtype, int S, int R,
                            hipStream_t stream);

/*
 * Decode-time append to a streaming cache ([P4] Introduction: converted
 * layers keep attending to the sink and recent keys): write the new token's
 * K and V rows, k_new / v_new [B,Hkv,D] contiguous (device), for position
 * `pos` into slot pos (pos < S) or S + (pos-S) mod R of every (b, kv head)
 * of k_stream / v_stream [B,Hkv,>=min(pos+1,S+R),D] -- over the oldest recent
 * token once the ring is full.  The cache then holds the sink + recent set
 * of position pos; decode it with kv_len = min(pos+1, S+R).  Same slot rule
 * as lt_compact_kv_streaming.  Errors: LT_ERR_DTYPE, LT_ERR_SHAPE (S < 0,
 * R < 1, pos < 0), LT_ERR_NULL, LT_ERR_LAYOUT (16-byte alignment), LT_ERR_HIP.
 */
int lt_stream_cache_append(lt_view k_stream, lt_view v_stream, const void *k_new, const void *v_new,
                           int B, int Hkv, int D, int dtype, int S, int R, int64_t pos,
                           hipStream_t stream);

/*
 * Variable-length batches (padded layout).  Sequence b of a batch has its
 * own length, given per sequence in a DEVICE int32 array of B entries (so
 * that a captured HIP graph can be replayed with new lengths); its rows are
 * positions [0, len_b) of the padded tensors, and every method step runs on
 * each sequence as if it were alone: causal from its own position 0, its own
 * last W queries observed, its own sink + recent slice.  Lengths are read on
 * the device and cannot be checked there: a value below 0 counts as 0, one
 * above the padded size as the padded size.  Rows at or past len_b are
 * neither read (q, k, v) nor written (out, lse) -- their contents are left
 * as they were.  Everything else (views, validation, errors) is as in the
 * call without _varlen; a NULL length array is LT_ERR_NULL.
 *
 * Prefill: seq_lens [B]; shape->N is the padded length.  lse keeps its
 * [B,Hq,N] layout.  Lazy ratio: a sequence observes its last min(W, len_b)
 * queries; lazy_rows[b,h,k] holds row len_b - W + k, the W - len_b slots of
 * rows before position 0 (len_b < W) are set to NaN, and lazy_ratio is the
 * mean of the observed rows (NaN for an empty sequence).
 */
int lt_prefill_attn_lse_lazy_varlen(const lt_shape *shape, const int32_t *seq_lens, lt_view q,
                                    lt_view k, lt_view v, lt_view out, float *lse, int S, int R,
                                    int W, float *lazy_rows, float *lazy_ratio, hipStream_t stream);

/*
 * Prefill that also writes the layer's streaming slice ([P1] solution 2,
 * [P4] Figure 2: the KV of a layer that turns out lazy is cut to its sink +
 * recent rows; producing that slice in the prefill itself makes the later
 * switch a release of the full buffers, with no copy kernel).  Everything
 * lt_prefill_attn_lse_lazy (or, with seq_lens, its _varlen form) computes,
 * plus: k_stream / v_stream [B,Hkv,>=min(len,S+R),D] receive the K/V rows of
 * positions [0,S) and [len-R,len) of every (b, kv head) in the slot order of
 * lt_compact_kv_streaming, i.e. exactly what that call would write.
 * seq_lens: device int32 [B] or NULL (every sequence has N rows).  The two
 * views are checked like the others (LT_ERR_NULL, LT_ERR_LAYOUT).
 */
int lt_prefill_attn_lse_lazy_emit(const lt_shape *shape, const int32_t *seq_lens, lt_view q,
                                  lt_view k, lt_view v, lt_view out, float *lse, int S, int R,
                                  int W, float *lazy_rows, float *lazy_ratio, lt_view k_stream,
                                  lt_view v_stream, hipStream_t stream);

/* Streaming attention over a padded variable-length batch (seq_lens [B]). */
int lt_streaming_attn_varlen(const lt_shape *shape, const int32_t *seq_lens, lt_view q, lt_view k,
                             lt_view v, lt_view out, float *lse, int S, int R, hipStream_t stream);

/*
 * Decode over caches of different lengths: sequence b attends to rows
 * [0, kv_lens[b]) of its cache.  max_kv_len bounds every kv_lens[b] and sizes
 * the workspace (lt_hybrid_decode_workspace_bytes with kv_len = max_kv_len).
 * kv_lens[b] == 0 gives out = 0 and lse = -inf for that sequence.
 */
int lt_hybrid_decode_attn_varlen(int B, int Hq, int Hkv, int D, int dtype, float scale,
                                 const void *q, lt_view k_cache, lt_view v_cache,
                                 const int32_t *kv_lens, int64_t max_kv_len, void *out, float *lse,
                                 void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * lt_hybrid_decode_attn_varlen over a paged cache: the keys of every
 * sequence live in fixed-size pages of one pool, listed by a block table, so
 * contexts grow a page at a time without moving rows.
 *   k_pool / v_pool: views whose "batch" index is the pool page:
 *     data + page * sb + kv_head * sh + row * sn (row < page_size), d
 *     contiguous; num_pages pages (device memory the caller owns);
 *   page_size: a power of two in [16, 2^20];
 *   block_table [B, max_pages] int32 (device): key j of sequence b is row
 *     j % page_size of pool page block_table[b * max_pages + j / page_size];
 *     entries of pages past a sequence's context are not read, and an entry
 *     outside [0, num_pages) is clamped into it (a wrong table reads wrong
 *     rows, never outside the pool);
 *   kv_lens [B] int32 (device): sequence b attends to its keys
 *     [0, kv_lens[b]), kv_lens[b] clamped to [0, max_pages * page_size];
 *     0 gives out = 0 and lse = -inf;
 *   ws: at least lt_hybrid_decode_workspace_bytes(B, Hq, Hkv, D,
 *     max_pages * page_size) bytes.
 * q, out, lse, dtype and scale as for lt_hybrid_decode_attn.  The result
 * equals lt_hybrid_decode_attn_varlen over the gathered contiguous caches up
 * to rounding order.  Errors as for lt_hybrid_decode_attn_varlen, plus
 * LT_ERR_NULL (block_table), LT_ERR_LAYOUT (block_table or kv_lens not
 * 4-byte aligned) and LT_ERR_SHAPE (page_size, max_pages, num_pages).
 */
int lt_hybrid_decode_attn_paged(int B, int Hq, int Hkv, int D, int dtype, float scale,
                                const void *q, lt_view k_pool, lt_view v_pool, int page_size,
                                int num_pages, const int32_t *block_table, int max_pages,
                                const int32_t *kv_lens, void *out, float *lse, void *ws,
                                size_t ws_bytes, hipStream_t stream);

/*
 * Compaction of a padded variable-length batch: sequence b keeps positions
 * [0,S) and [len_b-R, len_b) of its own length, in the ring slot order of
 * lt_compact_kv_streaming (every row in order when len_b <= S+R); slots at or
 * past min(len_b, S+R) are left untouched.
 */
int lt_compact_kv_streaming_varlen(lt_view k_full, lt_view v_full, lt_view k_stream,
                                   lt_view v_stream, int B, int Hkv, int N, int D, int dtype, int S,
                                   int R, const int32_t *seq_lens, hipStream_t stream);

/*
 * Decode-time append with each sequence at its own position: pos [B] device
 * int32; sequence b's new rows go to the slot of pos[b] (same rule as
 * lt_stream_cache_append); a negative pos[b] writes nothing for b.  The
 * caches must hold S+R slots.
 */
int lt_stream_cache_append_varlen(lt_view k_stream, lt_view v_stream, const void *k_new,
                                  const void *v_new, int B, int Hkv, int D, int dtype, int S, int R,
                                  const int32_t *pos, hipStream_t stream);

/*
 * (full, streaming) KV bytes of one layer: 2*B*Hkv*N*D*e and
 * 2*B*Hkv*min(N,S+R)*D*e, e the element size.  Host-only.
 */
int lt_kv_bytes(int B, int Hkv, int64_t N, int D, int dtype, int S, int R, int64_t *full_bytes,
                int64_t *stream_bytes);

/*
 * The lazy-layer priority queue ([P1] solution 2; [P4] Figure 2), online
 * form: after layer `layer` finishes, push (score, layer); while the queue
 * holds more than C layers, the one with the highest score leaves (equal
 * scores: the lower layer index) and becomes a streaming layer.  *evicted
 * receives that layer or -1.  Layers must be pushed in order 0..L-1: a
 * layer out of order, or a push after layer L-1, is LT_ERR_VALUE and leaves
 * the queue unchanged.  Host memory is owned by the handle.
 */
typedef struct lt_lazy_queue lt_lazy_queue;
int lt_lazy_queue_create(int L, int C, lt_lazy_queue **out);

/*
 * When the queue evicts.  The pages give two timings ([P1] solution 2: a
 * layer leaves once more layers are queued than the threshold; [P4] Figure 2
 * caption: once the queue has reached its capacity, the laziest layer leaves,
 * freeing memory for the current one).
 *   LT_EVICT_AFTER_PUSH (the default of lt_lazy_queue_create and
 *     lt_select_lazy_layers): push, then evict while more than C are queued;
 *     the current layer may leave at its own step.
 *   LT_EVICT_BEFORE_PUSH: if C layers are already queued, evict the laziest
 *     of them, then push; the current layer always enters (with C == 0 no
 *     layer can be queued and each leaves at its own step).
 */
enum { LT_EVICT_AFTER_PUSH = 0, LT_EVICT_BEFORE_PUSH = 1 };
int lt_lazy_queue_create_policy(int L, int C, int policy, lt_lazy_queue **out);
int lt_lazy_queue_push(lt_lazy_queue *queue, int layer, double score, int *evicted);
void lt_lazy_queue_destroy(lt_lazy_queue *queue);

/*
 * Same push, with the layer's score computed here from its n per-(batch,
 * head) lazy ratios (head_ratio, host fp32, e.g. the lazy_ratio output of
 * lt_prefill_attn_lse_lazy copied to the host): their mean, summed in fp64
 * in index order.  *score (may be NULL) receives it.  Non-finite ratios
 * give LT_ERR_VALUE and leave the queue unchanged.
 */
int lt_lazy_queue_push_ratios(lt_lazy_queue *queue, int layer, const float *head_ratio, int n,
                              double *score, int *evicted);

/*
 * Batch form of the same queue.  head_ratio [L][n] host fp32: the n
 * per-(batch, head) lazy ratios of each layer.  A layer's score is their
 * mean, summed in fp64 in index order (written to layer_score [L] if not
 * NULL).  Then L pushes as above: evicted_at_step [L] (-1 = none) and
 * is_streaming [L] (0/1).  Host-only.
 */
int lt_select_lazy_layers(const float *head_ratio, int L, int n, int C, double *layer_score,
                          int *evicted_at_step, uint8_t *is_streaming);
/* The same with an eviction policy (LT_EVICT_AFTER_PUSH or _BEFORE_PUSH). */
int lt_select_lazy_layers_policy(const float *head_ratio, int L, int n, int C, int policy,
                                 double *layer_score, int *evicted_at_step, uint8_t *is_streaming);

/*
 * Offline lazy-layer selection ([P3] "LightTransfer method", steps 1-3: the
 * lazy ratio of every layer is measured on a set of prompts and the layers
 * with the highest ratios are replaced by streaming attention).
 * head_ratio [P][L][n] host fp32: the n per-(batch, head) lazy ratios of
 * layer l on prompt p (the lazy_ratio output of lt_prefill_attn_lse_lazy).
 * A layer's per-prompt score is the mean of its n ratios (fp64, index
 * order); its offline score the mean of those over the P prompts (fp64,
 * prompt order), written to layer_score [L] if not NULL.  The L - C layers
 * with the highest offline scores get is_streaming [L] = 1 (equal scores:
 * the lower layer index first), the other C stay full.  Host-only.  Errors:
 * LT_ERR_NULL, LT_ERR_SHAPE (P, L or n < 1), LT_ERR_VALUE (C outside
 * [0, L], a ratio not finite); outputs are untouched on error.
 */
int lt_select_offline(const float *head_ratio, int P, int L, int n, int C, double *layer_score,
                      uint8_t *is_streaming);

/*
 * KV bytes the prefill holds while it walks the layers ([P1] solution 2:
 * the queue bounds peak prefill memory at C full layers, the rest
 * streaming).  Every layer has the same sizes: full_bytes at full size,
 * stream_bytes once switched (lt_kv_bytes); with emit != 0 each prefill also
 * wrote its streaming slice (lt_prefill_attn_lse_lazy_emit), so a layer still
 * at full size holds full_bytes + stream_bytes and switching keeps the slice.
 * At step l (after layer l's push):
 *   transient[l]: layers 0..l-1 at their current size plus layer l at full
 *     size, before the queue's decision -- except that with
 *     LT_EVICT_BEFORE_PUSH an earlier layer evicted at this step is already
 *     switched (its memory is freed for layer l);
 *   retained[l]: every layer 0..l at its size after the decision.
 *
 * Online form: lt_lazy_queue_set_kv_bytes sets the sizes (before the first
 * push); after each push lt_lazy_queue_kv_bytes returns that step's pair.
 * Errors: LT_ERR_NULL; LT_ERR_VALUE (negative sizes, sizes not set, or no
 * layer pushed yet).
 */
int lt_lazy_queue_set_kv_bytes(lt_lazy_queue *queue, int64_t full_bytes, int64_t stream_bytes, int emit);
int lt_lazy_queue_kv_bytes(const lt_lazy_queue *queue, int64_t *retained, int64_t *transient);

/*
 * Batch form: the same pairs for a whole run from its evicted_at_step [L]
 * (as lt_select_lazy_layers_policy writes it, policy the same) into
 * retained [L] and transient [L].  Host-only.  Errors: LT_ERR_NULL,
 * LT_ERR_SHAPE (L < 1), LT_ERR_VALUE (unknown policy, negative sizes, an
 * entry that is not -1 or a layer 0..l, or a layer evicted twice); outputs
 * are untouched on error.
 */
int lt_kv_accounting(const int *evicted_at_step, int L, int policy, int64_t full_bytes,
                     int64_t stream_bytes, int emit, int64_t *retained, int64_t *transient);

/* Name of a status code, and the calling thread's last error message. */
const char *lt_status_str(int status);
const char *lt_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* LT_H */
