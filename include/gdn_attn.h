/*
 * gdn_attn.h -- C ABI of the softmax block's attention over streaming chunks on MI355X (gfx950).
 *
 * The operation (SANA-Streaming pages, Chinese summary, "Core method": the hybrid DiT inserts
 * 5 softmax-attention blocks among its 15 GDN blocks; each attends over a sliding window plus
 * persistent sink tokens, which keeps its memory fixed while chunk boundaries keep token-level
 * correspondence; "Prerequisites": softmax attention forms token interactions from dot
 * products normalised by a softmax).  The pages give no sizes and no mask.  Readings: per
 * stream b and head h,
 *  - the sink holds the first `sink_tokens` tokens the stream produced, for the stream's life;
 *  - the window holds the newest `window_tokens` tokens produced after the sink;
 *  - every query of a chunk of T tokens attends over sink + window + all T tokens of the chunk
 *    (no mask inside the chunk), o_t = sum_j softmax_j(scale q_t.k_j) v_j;
 *  - a committed call then appends the chunk's k, v to the cache (filling the sink first, then
 *    the window, evicting its oldest tokens); GDN_NO_COMMIT leaves the cache unchanged (a
 *    denoising step that will be replayed).
 * The order of the cached tokens does not enter the result (a softmax over a set).
 *
 * Conventions are those of gdn_stream.h: GDN_OK or a negative GDN_E_* code, nothing enqueued
 * and the cache unchanged on error, gdn_last_error() for the message; device pointers are
 * caller-owned and not retained; work is enqueued asynchronously on `hip_stream` (a
 * hipStream_t, NULL = the null stream); one handle is one logical sequence of calls.
 * q, k, v, o are bf16 [B, T, H, head_dim] with (b, t, h) strides in elements, the feature
 * dimension contiguous, rows 16-byte aligned.  Scores and the softmax run in fp32; the
 * probabilities enter the value product as bf16; o is rounded to bf16 (nearest even).
 */
#ifndef GDN_ATTN_H
#define GDN_ATTN_H

#include "gdn_stream.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct gdn_attn_config {
    int32_t batch;          /* B independent streams, >= 1                               */
    int32_t heads;          /* H heads, >= 1                                             */
    int32_t head_dim;       /* d of q, k and v: 64, 112 or 128                           */
    int32_t sink_tokens;    /* sink capacity per (stream, head), >= 0                    */
    int32_t window_tokens;  /* window capacity per (stream, head), >= 0                  */
    int64_t max_tokens;     /* largest T of any call, >= 1; sink_tokens, window_tokens   */
                            /* and max_tokens times head_dim * 2 bytes stay below 2 GiB */
    float scale;            /* logit scale; 0 selects 1/sqrt(head_dim)                   */
} gdn_attn_config;

typedef struct gdn_attn_io {
    const void* q;          /* [B, T, H, d] bf16                                         */
    const void* k;          /* [B, T, H, d] bf16                                         */
    const void* v;          /* [B, T, H, d] bf16                                         */
    void* o;                /* [B, T, H, d] bf16, written                                */
    int64_t q_strides[3];   /* (b, t, h) strides in elements                             */
    int64_t k_strides[3];
    int64_t v_strides[3];
    int64_t o_strides[3];
} gdn_attn_io;

typedef struct gdn_attn gdn_attn;

/* Create a handle on `device`.  The library owns the cache: k and v of the sink and of the
 * window, bf16 [B, H, sink_tokens + window_tokens, d] each (2 * B * H * (sink + window) * d * 2
 * bytes), allocated here and never grown; it starts empty.  Errors: GDN_E_INVAL (NULL cfg or
 * out), GDN_E_SHAPE (sizes), GDN_E_NOMEM, GDN_E_HIP. */
GDN_API int gdn_attn_init(const gdn_attn_config* cfg, int device, gdn_attn** out);

/* Free the handle's memory (waits for the device to go idle).  NULL is a no-op. */
GDN_API int gdn_attn_destroy(gdn_attn* a);

/* Attention of one chunk of T tokens (0 <= T <= max_tokens; T = 0 does nothing) over the
 * cache and the chunk itself, written to io->o; then, unless `flags` has GDN_NO_COMMIT, the
 * chunk's k and v enter the cache.  Errors: GDN_E_INVAL (NULL handle/io/pointer, bad
 * alignment or strides, unknown flags), GDN_E_SHAPE (T), GDN_E_HIP. */
GDN_API int gdn_attn_chunk(gdn_attn* a, const gdn_attn_io* io, int64_t T, uint32_t flags, void* hip_stream);

/* Empty the cache (host-side bookkeeping only: nothing is enqueued). */
GDN_API int gdn_attn_reset(gdn_attn* a);

/* Tokens the cache holds now, per (stream, head): in the sink and in the window. */
GDN_API int gdn_attn_cache_len(const gdn_attn* a, int64_t* sink, int64_t* window);

/* Checkpoint and resume of the cache (the softmax block's counterpart of gdn_state_get/set).
 * The snapshot is the library's cache memory as it stands: k of the sink, v of the sink, k of
 * the window, v of the window, each bf16 [B, H, capacity, d] (gdn_attn_cache_bytes bytes in
 * all, device memory on the handle's device, 16-byte aligned), plus two counters: the tokens
 * in the sink and the tokens ever written to the window (its ring position).  Copies are
 * enqueued asynchronously on `hip_stream`; get takes the state after every call enqueued
 * before it.  set checks 0 <= sink_len <= sink_tokens, window_total >= 0 and window_total = 0
 * unless the sink is full (GDN_E_INVAL otherwise; nothing enqueued). */
GDN_API int gdn_attn_cache_bytes(const gdn_attn* a, int64_t* bytes);
GDN_API int gdn_attn_cache_get(gdn_attn* a, void* dst, int64_t* sink_len, int64_t* window_total, void* hip_stream);
GDN_API int gdn_attn_cache_set(gdn_attn* a, const void* src, int64_t sink_len, int64_t window_total,
                               void* hip_stream);

/* Optional timing of the attention kernel (not the cache append): with profiling on, every
 * launch is bracketed by hipEvents on the launch stream; gdn_attn_profile_read waits for them
 * and returns the summed milliseconds and the launch count, clearing them when `reset` != 0. */
GDN_API int gdn_attn_profile(gdn_attn* a, int enable);
GDN_API int gdn_attn_profile_read(gdn_attn* a, double* ms, int64_t* launches, int reset);

#ifdef __cplusplus
}
#endif

#endif /* GDN_ATTN_H */
