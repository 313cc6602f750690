/*
 * wmk -- sink + window KV-cache chunk attention for MI355X (gfx950).
 *
 * The hot path of a causal video DiT that generates latent-video chunks one
 * after another from cached history plus current inputs ("Mix Forcing: Causal
 * Pre-Training via Mixture Attention for Interactive World Models", Overview).
 * Per DiT layer the cache keeps the first frames as anchors ("sinks") for good
 * and a sliding window of the most recently finalized frames, evicting older
 * non-sink frames ("LingBot-World-Infinity: The Open-Source World Model That
 * Refuses to Forget", "The trick: treat video like a causal stream" and "How the
 * cache keeps the world alive").  The queries of the current chunk attend the
 * resident frames and the chunk itself -- 6 anchors + 8 recent + 4 current = 18
 * latent-frame slots in the native model ("Westlake AGI Lab's 'World in World'
 * Steers Frozen Video Models", second paragraph).  Training uses the MoBA mask:
 * a teacher-forcing mask plus an appended, fully bidirectional block
 * ("Infinite Worlds with Versatile Interactions", causal pretraining paragraph).
 *
 * Conventions for every call
 * --------------------------
 * - Token tensors are row-major [tokens][heads][head_dim], batch 1, in the
 *   dtype named by the descriptor (bf16 or fp32).  Softmax and accumulation are
 *   fp32 inside the kernels; bf16 outputs are rounded to nearest-even.
 * - All tensor pointers are device pointers owned by the caller and must be
 *   16-byte aligned.  The library never allocates or frees device memory and
 *   never synchronizes the device or a stream.
 * - Every call that does GPU work only enqueues it on the given stream and
 *   returns.  Calls on one cache must be issued on one stream (or ordered by
 *   the caller); host-side counters advance when the work is enqueued.
 * - A cache handle is host state without a lock: calls on one cache from
 *   several host threads must be serialized by the caller.  Calls on
 *   different caches, and the calls that take no cache, are independent.
 * - On any error nothing is enqueued, no state changes, and a message is
 *   available from wmk_last_error() on the calling thread.
 */
#ifndef WMK_H
#define WMK_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    WMK_OK = 0,
    WMK_ERR_NULL = 1,     /* a required pointer is NULL                              */
    WMK_ERR_SHAPE = 2,    /* a size, count or shape is out of its allowed set         */
    WMK_ERR_DTYPE = 3,    /* unsupported dtype, or dtype differs from the cache's     */
    WMK_ERR_RANGE = 4,    /* layer index or scale out of range                        */
    WMK_ERR_ALIGN = 5,    /* a device pointer is not 16-byte aligned                  */
    WMK_ERR_CAPACITY = 6, /* caller-provided buffer too small                         */
    WMK_ERR_HIP = 7       /* the HIP runtime refused a launch                         */
} wmk_status;

typedef enum { WMK_F32 = 0, WMK_BF16 = 1 } wmk_dtype;

/* Shape of a per-layer KV cache.  Sinks and window are counted in latent
 * frames; the window holds finalized non-sink frames and does not include the
 * chunk being generated. */
typedef struct {
    int32_t num_layers;       /* >= 1                                                  */
    int32_t num_heads;        /* 1 .. 4096                                             */
    int32_t head_dim;         /* 64 or 128                                             */
    int32_t tokens_per_frame; /* >= 1 (1508 for a 52x29 latent grid)                   */
    int32_t sink_frames;      /* S >= 0                                                */
    int32_t window_frames;    /* W >= 1                                                */
    int32_t chunk_frames;     /* frames per finalized chunk; >= 1 (informational)      */
    wmk_dtype dtype;          /* element type of K and V; stored bit-exactly           */
} wmk_cache_desc;

typedef struct wmk_cache wmk_cache; /* opaque host handle */

typedef struct {
    int32_t num_heads; /* 1 .. 4096 */
    int32_t head_dim;  /* 64 or 128 */
    wmk_dtype dtype;
} wmk_head_desc;

/* An extra span of keys/values, [tokens][heads][head_dim] each: the current
 * chunk's own K/V at a chunk step, or prompt K/V for cross-attention. */
typedef struct {
    const void* k;
    const void* v;
    int32_t tokens; /* >= 1 */
} wmk_kv_segment;

/* MoBA training sequence: [clean | noisy | bidirectional block], each part
 * `frames` latent frames of `tokens_per_frame` tokens; chunks of
 * `chunk_frames` frames (the last chunk of a part may be shorter). */
typedef struct {
    int32_t tokens_per_frame; /* >= 1 */
    int32_t frames;           /* >= 1, frames per part */
    int32_t chunk_frames;     /* >= 1 */
    int32_t bidir_block;      /* 1: append the bidirectional block; 0: clean + noisy only */
} wmk_moba_desc;

/* Chunk-causal cross-attention over a multi-chunk training sequence: queries
 * are `chunks` chunks of `chunk_q_tokens` tokens each (chunk i = rows
 * [i * chunk_q_tokens, (i + 1) * chunk_q_tokens)); keys/values are the shared
 * environment prompt followed by one local prompt per chunk,
 * [env_tokens | local_0 | local_1 | ...] with local_tokens tokens each. */
typedef struct {
    int32_t chunk_q_tokens; /* >= 1 */
    int32_t chunks;         /* >= 1 */
    int32_t env_tokens;     /* >= 0 */
    int32_t local_tokens;   /* >= 0; env_tokens + local_tokens >= 1 */
} wmk_xattn_desc;

/* Bytes of the K buffer (equal to the V buffer) for all layers of a cache with
 * descriptor d: num_layers * (S + W) * tokens_per_frame * heads * head_dim *
 * sizeof(dtype).  Layout [layer][slot][tokens_per_frame][heads][head_dim].
 * Returns 0 when d is NULL or invalid. */
size_t wmk_cache_bytes(const wmk_cache_desc* d);

/* Create a cache handle over caller-allocated K and V buffers of at least
 * capacity_bytes each (>= wmk_cache_bytes(d)).  Host-only: validates and
 * records the descriptor and sets every layer's frame counter to zero; the
 * buffers' contents are not touched (unfilled slots are never read).
 * Cache policy: sinks, then a window of W recent frames ("How the cache keeps
 * the world alive"); 18-slot layout of "World in World".
 * Errors: NULL d/k_dev/v_dev/out -> WMK_ERR_NULL; invalid descriptor ->
 * WMK_ERR_SHAPE or WMK_ERR_DTYPE; misaligned buffer -> WMK_ERR_ALIGN;
 * capacity_bytes too small -> WMK_ERR_CAPACITY.  On error *out is untouched. */
wmk_status wmk_cache_init(const wmk_cache_desc* d, void* k_dev, void* v_dev, size_t capacity_bytes,
                          wmk_cache** out);

/* Free the host handle (not the caller's buffers).  NULL is accepted. */
void wmk_cache_destroy(wmk_cache* c);

/* Append n_frames finalized frames to `layer` and evict in the same step:
 * the cache keeps its sink frames at the front for good and slides a window of
 * recent frames, discarding the oldest non-sink frame once the window is full
 * ("LingBot-World-Infinity: The Open-Source World Model That Refuses to
 * Forget", "How the cache keeps the world alive"; the simplified loop of "The
 * trick: treat video like a causal stream" -- evict old state, keep the
 * anchors, step, append -- with evict and append done here as one call after a
 * chunk is finalized).  In the native model the frames appended are the
 * recently finalized outputs the self-attention reads next to the initial
 * observation ("Westlake AGI Lab's 'World in World' Steers Frozen Video
 * Models", second paragraph).
 * k_new and v_new are [n_frames * tokens_per_frame][heads][head_dim] in the
 * cache dtype, device memory owned by the caller and only read here.  Frame f
 * (global append order) lands in slot f if f < S, else in slot
 * S + (f - S) mod W, overwriting -- and so evicting -- frame f - W.  Frames
 * that this same call would overwrite (only when n_frames > W) are not
 * written.  Bits are copied exactly.  The frame counter advances on enqueue.
 * Errors: NULL -> WMK_ERR_NULL; layer outside [0, num_layers) -> WMK_ERR_RANGE;
 * n_frames <= 0 -> WMK_ERR_SHAPE; misaligned -> WMK_ERR_ALIGN; launch refused
 * -> WMK_ERR_HIP (counter not advanced). */
wmk_status wmk_cache_append_evict(wmk_cache* c, int32_t layer, const void* k_new, const void* v_new,
                                  int32_t n_frames, hipStream_t stream);

/* wmk_cache_append_evict for n_layers consecutive layers [first_layer,
 * first_layer + n_layers) in one launch: the finalized chunk that every layer
 * of the model appends after it is generated (the same passages as
 * wmk_cache_append_evict: "How the cache keeps the world alive" of the
 * LingBot-World-Infinity page, and "World in World", second paragraph).  Each
 * layer's attention over the chunk reads its own K/V as a segment, so the
 * appends of all layers can wait for the end of the finalizing pass and go as
 * one call.
 * k_new and v_new are [n_layers][n_frames * tokens_per_frame][heads][head_dim]
 * in the cache dtype (layer first_layer + i at block i), device memory owned by
 * the caller and only read here.  The result equals n_layers calls of
 * wmk_cache_append_evict, bit for bit.  Every layer of the run must hold the
 * same frame count (a model keeps its layers in step).
 * Errors: NULL -> WMK_ERR_NULL; n_layers <= 0 or n_frames <= 0 ->
 * WMK_ERR_SHAPE; a layer outside [0, num_layers), or layers holding different
 * frame counts -> WMK_ERR_RANGE; misaligned -> WMK_ERR_ALIGN; launch refused ->
 * WMK_ERR_HIP.  On any error no counter advances and nothing is enqueued. */
wmk_status wmk_cache_append_evict_layers(wmk_cache* c, int32_t first_layer, int32_t n_layers, const void* k_new,
                                         const void* v_new, int32_t n_frames, hipStream_t stream);

/* Host-side view of a layer's slots, the bookkeeping of the sink + window
 * cache ("How the cache keeps the world alive": sinks kept at the front, the
 * window sliding behind them; "World in World", second paragraph: 6 anchor and
 * 8 recent-frame slots beside the 4 of the current chunk in the native model).
 * frame_of_slot[S + W] (a host array owned by the caller) receives the frame
 * held by each slot (-1 when empty) and *frames_appended the layer's counter
 * (either output pointer may be NULL).  Resident frames always fill the slot
 * prefix [0, valid).  No GPU work, no synchronization: computed from the host
 * counter alone.  Errors: NULL c -> WMK_ERR_NULL; layer out of range ->
 * WMK_ERR_RANGE. */
wmk_status wmk_cache_slots(const wmk_cache* c, int32_t layer, int64_t* frame_of_slot, int64_t* frames_appended);

/* Bytes of optional scratch that lets the attention calls below split the last,
 * partly filled round of work units over the whole GPU (a split-KV tail: the
 * pieces write fp32 partial results, a second small kernel on the same stream
 * merges them).  Passing less, NULL, or a pointer not 16-byte aligned is valid
 * and only disables that split.  q_tokens and heads are those of the call. */
size_t wmk_attention_workspace_bytes(const wmk_head_desc* hd, int32_t q_tokens);

/* Chunk attention at a denoising step: every query row of the current chunk
 * attends every resident frame of `layer` in cache c (if c is not NULL) and
 * every token of the n_seg extra segments (the current chunk's own K/V --
 * bidirectional inside the chunk -- or prompt K/V for cross-attention, where
 * chunk i passes the shared environment prompt and its own local prompt only,
 * "Mix Forcing", "Condition each chunk").  No other mask applies: every
 * resident frame is in the past, and causality lives in which frames are
 * resident.  out_i = softmax_j(scale * q_i . k_j) v_j per head.
 * q and out: [q_tokens][heads][head_dim], dtype of hd.  A row with no key at
 * all (empty cache and n_seg = 0) gets zeros.
 * Errors: NULL hd/q/out, or NULL seg with n_seg > 0 -> WMK_ERR_NULL; head_dim
 * not 64/128, q_tokens <= 0, n_seg outside [0, 4], a segment with tokens <= 0,
 * more than 2^31 - 1 keys, or hd not matching the cache -> WMK_ERR_SHAPE;
 * dtype -> WMK_ERR_DTYPE; layer out of range or scale not finite and > 0 ->
 * WMK_ERR_RANGE; misaligned -> WMK_ERR_ALIGN; launch refused -> WMK_ERR_HIP. */
wmk_status wmk_chunk_attention(const wmk_cache* c, int32_t layer, const wmk_head_desc* hd, const void* q,
                               int32_t q_tokens, const wmk_kv_segment* seg, int32_t n_seg, void* out, float scale,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* wmk_chunk_attention for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and the same split-tail plan as
 * wmk_chunk_attention given an ample workspace, but the split tail's scratch
 * is a device array the library holds -- one per GPU, 34,078,720 bytes, kept
 * until the process ends -- and the call allocates nothing.  Its address is
 * looked up on the first call on each device.  Every call on one GPU shares
 * that GPU's array: calls that overlap on one GPU (other streams, or other
 * threads without ordering) race and must not be issued.  Nothing in the
 * array needs clearing between calls.  Arguments, layout and ownership as
 * for wmk_chunk_attention.
 * Errors: as wmk_chunk_attention; a split tail needing more than the array
 * (more pieces than a 256-CU MI355X has resident attention workgroups: 256
 * pieces of 256 query rows, or 512 of 128 rows for short key walks) ->
 * WMK_ERR_CAPACITY; the array's address not available ->
 * WMK_ERR_HIP.  Nothing is enqueued on error. */
wmk_status wmk_chunk_attention_noalloc(const wmk_cache* c, int32_t layer, const wmk_head_desc* hd, const void* q,
                                       int32_t q_tokens, const wmk_kv_segment* seg, int32_t n_seg, void* out,
                                       float scale, hipStream_t stream);

/* Workspace bytes for wmk_chunk_attention_qk8 with q_tokens queries and up to
 * kv_tokens keys (cache part plus segments): the FP8 codes and scales of Q and
 * K, plus the optional split-tail scratch of wmk_attention_workspace_bytes.
 * 0 if hd is invalid, not bf16 or head_dim is not 128. */
size_t wmk_attention_qk8_workspace_bytes(const wmk_head_desc* hd, int32_t q_tokens, int64_t kv_tokens);

/* Chunk attention with a quantized QK^T: as wmk_chunk_attention, but the
 * scores S = Q K^T come from FP8 (OCP e4m3) operands with one fp32 scale per
 * block -- the precision variant of the attention step (LingBot-World 2.0
 * speed-up page, step table, "Attention" row: an INT8-QK^T SageAttention
 * kernel replaces FlashAttention-2; roofline table, "SageAttention" row; here
 * the operands are quantized to FP8 for the CDNA4 matrix cores).
 * Per head, Q is cut into blocks of 32 rows and the keys -- the resident
 * frames in time order (sinks, then the window, oldest first), then the
 * segments -- into tiles of 64, so the blocks depend only on which frames are
 * resident, not on where the ring has wrapped; per block, in fp32:
 * scale = max|x| / 448, code = e4m3(clamp(x * 448 / max|x|, +-448)), nearest
 * even (all zero: scale 0, codes 0).  Softmax, P (bf16) and P V (bf16, fp32
 * accumulate) are as in the plain path.
 * The workspace is required and holds, from its start (256-byte aligned), the
 * K codes ([tile][head][64][128] bytes, the 16-byte chunks of row r permuted
 * by XOR with (r / 2) % 8), the K scales ([tile][head] fp32), the Q codes
 * ([block][head][32][128] bytes, row-major) and the Q scales, each region
 * 256-byte aligned; any rest serves the split tail.  Contents are overwritten
 * on every call.  bf16 and head_dim 128 only.
 * Errors: as wmk_chunk_attention, plus dtype not bf16 -> WMK_ERR_DTYPE,
 * head_dim not 128 -> WMK_ERR_SHAPE, workspace NULL or smaller than
 * wmk_attention_qk8_workspace_bytes minus the split scratch ->
 * WMK_ERR_CAPACITY, workspace not 256-byte aligned -> WMK_ERR_ALIGN. */
wmk_status wmk_chunk_attention_qk8(const wmk_cache* c, int32_t layer, const wmk_head_desc* hd, const void* q,
                                   int32_t q_tokens, const wmk_kv_segment* seg, int32_t n_seg, void* out, float scale,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Chunk attention with variable retention: as wmk_chunk_attention, but of
 * the resident frames of `layer` only the n_keep listed in keep_frames (a
 * host array of global frame indices, any order, as reported by
 * wmk_cache_slots) are attended; the others stay in the cache, untouched, for
 * later calls.  This is the per-call choice of retained history of a dynamic
 * KV-cache scheduler ("Infinite Worlds with Versatile Interactions",
 * deployment paragraph: retained history adapted to the current control
 * signal).  Temporary auxiliary KV
 * blocks of the current chunk ("World in World", second paragraph: extra
 * evidence for the current chunk, dropped once it is finalized) are passed as
 * segments and never appended.  n_keep = 0 attends the segments only.  The
 * kept frames form one key span per run of adjacent slots; together with the
 * segments at most 16 spans.
 * Errors: c NULL, or keep_frames NULL with n_keep > 0 -> WMK_ERR_NULL;
 * n_keep < 0 -> WMK_ERR_SHAPE; a listed frame not resident in the layer, or
 * listed twice -> WMK_ERR_RANGE; more than 16 spans -> WMK_ERR_CAPACITY; the
 * rest as for wmk_chunk_attention.  Nothing is enqueued on error. */
wmk_status wmk_chunk_attention_retained(const wmk_cache* c, int32_t layer, const int64_t* keep_frames,
                                        int32_t n_keep, const wmk_head_desc* hd, const void* q, int32_t q_tokens,
                                        const wmk_kv_segment* seg, int32_t n_seg, void* out, float scale,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* MoBA-masked attention forward over one training sequence
 * [clean | noisy | block] ("Infinite Worlds with Versatile Interactions",
 * causal pretraining paragraph; "Mix Forcing", "Mix the training modes").
 * With k = chunk index of a token inside its part: clean rows see clean keys
 * of chunks <= k; noisy rows see clean keys of chunks < k and noisy keys of
 * chunk k; block rows see the whole block; nothing else is allowed.
 * q, k, v and out are [(2 + bidir_block) * frames * tokens_per_frame][heads]
 * [head_dim] in the dtype of hd.  Errors as for wmk_chunk_attention, plus
 * bidir_block outside {0, 1} or a non-positive field -> WMK_ERR_SHAPE. */
wmk_status wmk_moba_attention(const wmk_moba_desc* m, const wmk_head_desc* hd, const void* q, const void* k,
                              const void* v, void* out, float scale, hipStream_t stream);

/* MoBA forward for training: wmk_moba_attention plus the per-row log-sum-exp
 * the backward needs.  lse is [num_heads][n] fp32 (n = sequence length), lse =
 * log sum_j exp(scale q_i . k_j) over the keys row i is allowed (natural log;
 * -inf for a row with none).  bf16 only.  Errors as wmk_moba_attention, plus
 * NULL lse -> WMK_ERR_NULL, misaligned lse -> WMK_ERR_ALIGN, dtype not bf16
 * -> WMK_ERR_DTYPE. */
wmk_status wmk_moba_attention_train(const wmk_moba_desc* m, const wmk_head_desc* hd, const void* q, const void* k,
                                    const void* v, void* out, float* lse, float scale, hipStream_t stream);

/* Workspace bytes of wmk_moba_attention_backward (one fp32 per row and head);
 * 0 for an invalid descriptor. */
size_t wmk_moba_backward_workspace_bytes(const wmk_moba_desc* m, const wmk_head_desc* hd);

/* MoBA backward: the gradients dq, dk, dv of L = sum(dout * out) for out =
 * wmk_moba_attention(q, k, v) under the same mask (the training use of the
 * MoBA mask, "Infinite Worlds with Versatile Interactions", causal
 * pretraining paragraph), with the same skip of tiles no row allows.  With
 * P = exp(scale q k^T - lse) on allowed pairs, D_i = dout_i . out_i:
 * dv = P^T dout, dS = P (dout v^T - D), dq = scale dS k, dk = scale dS^T q.
 * out and lse are those of wmk_moba_attention_train on the same inputs.
 * q, k, v, out, dout, dq, dk, dv: [n][num_heads][128] bf16; the gradients
 * must not overlap the inputs.  workspace: at least
 * wmk_moba_backward_workspace_bytes (16-byte aligned), overwritten.
 * Errors as wmk_moba_attention, plus NULL dout/lse/dq/dk/dv -> WMK_ERR_NULL,
 * dtype not bf16 -> WMK_ERR_DTYPE, head_dim not 128 -> WMK_ERR_SHAPE,
 * misaligned -> WMK_ERR_ALIGN, workspace NULL or too small ->
 * WMK_ERR_CAPACITY. */
wmk_status wmk_moba_attention_backward(const wmk_moba_desc* m, const wmk_head_desc* hd, const void* q, const void* k,
                                       const void* v, const void* out, const void* dout, const float* lse, void* dq,
                                       void* dk, void* dv, float scale, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/* Chunk-causal cross-attention forward over a multi-chunk sequence (the
 * training form of the chunk-wise prompt conditioning: "Infinite Worlds with
 * Versatile Interactions", causal pretraining paragraph -- a causal
 * cross-attention mask keeps chunk-wise prompts from leaking future
 * semantics; "Mix Forcing", "Condition each chunk").  Query chunk i attends
 * the environment prompt and its own local prompt i, nothing else; the local
 * prompts of other chunks -- earlier or later -- are masked.
 * q and out: [chunks * chunk_q_tokens][heads][head_dim]; k and v:
 * [env_tokens + chunks * local_tokens][heads][head_dim]; dtype of hd.
 * workspace as for wmk_chunk_attention.  Errors as for wmk_chunk_attention,
 * plus a NULL descriptor -> WMK_ERR_NULL and a field out of its range, or more
 * than 2^31 - 1 query or key tokens -> WMK_ERR_SHAPE. */
wmk_status wmk_cross_attention_train(const wmk_xattn_desc* x, const wmk_head_desc* hd, const void* q,
                                     const void* k, const void* v, void* out, float scale, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/* Message of the last error on the calling thread ("" if none); valid until
 * the next wmk call on that thread. */
const char* wmk_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* WMK_H */
