/*
 * gdn_stream.h -- C ABI of the MI355X (gfx950) Gated DeltaNet streaming core.
 *
 * The operation (SANA-Streaming pages: the Korean review, section 1 "Key
 * Terms", GDN entry -- a fixed-size state updated recursively from the previous
 * one; the Chinese summary, "Core method" -- GDN blocks carry global
 * information in a compact recurrent state; "Method steps" step 2 -- a chunk is
 * 3 latent frames, the streaming model runs a forward scan that starts from the
 * previous chunk's cache plus a backward scan inside the chunk).  The per-token
 * update is the published Gated DeltaNet rule, which the pages name but do not
 * print.  Per stream b and head h, with state S in R^{d_v x d_k}:
 *
 *     k^_t = k_t / sqrt(|k_t|^2 + eps),  q^_t likewise     (GDN_L2NORM_QK)
 *     S_t  = a_t S_{t-1} (I - beta_t k^_t k^_t^T) + beta_t v_t k^_t^T
 *     o_t  = scale * S_t q^_t
 *
 * gdn_chunk_forward runs t = 0..T-1 from the cached state of the handle and
 * (by default) stores S_{T-1} back into the cache, so consecutive calls stream
 * one long sequence in constant memory.  gdn_chunk_reverse runs t = T-1..0 from
 * a zero state (the future chunk does not exist yet) and never touches the
 * cache; o_t is stored at the token's own position.
 *
 * Conventions shared by every entry point
 *  - Return GDN_OK (0) or a negative GDN_E_* code.  On any error nothing has
 *    been enqueued and the cache is unchanged; gdn_last_error() gives a message
 *    (thread-local, valid until the next call from the same thread).
 *  - The kernels hand work between their wavefronts through bounded waits.  A
 *    wait that gives up (it never should) marks the handle's error word; the
 *    next call on the handle then returns GDN_E_HIP without enqueueing anything
 *    (the outputs of the earlier call are not valid) and clears the mark.  The
 *    bound is 2^22 polls, or the value of the environment variable
 *    GDN_SPIN_LIMIT when the handle was created.
 *  - Device pointers are caller-owned, must live on the handle's device, and
 *    are not retained after the call returns.  Work is enqueued asynchronously
 *    on `hip_stream` (a hipStream_t; NULL = the null stream); the caller
 *    synchronises.  A fault inside a kernel surfaces as GDN_E_HIP on a later
 *    call or at the caller's synchronisation.
 *  - One handle is one logical sequence: calls on a handle must not overlap in
 *    time (use one stream per handle).  Different handles are independent.
 *  - Strides are in elements, in the order (b, t, h); the feature dimension is
 *    contiguous.  q/k/v/o rows must be 16-byte aligned.
 */
#ifndef GDN_STREAM_H
#define GDN_STREAM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_API __attribute__((visibility("default")))

/* return codes */
#define GDN_OK        0
#define GDN_E_INVAL  -1   /* NULL handle/pointer, bad flag, bad alignment      */
#define GDN_E_SHAPE  -2   /* unsupported sizes, T outside [0, max_tokens], sizes
                             or strides whose products overflow                 */
#define GDN_E_DTYPE  -3   /* unknown io_dtype                                   */
#define GDN_E_NOMEM  -4   /* device allocation failed at init                   */
#define GDN_E_HIP    -5   /* a HIP runtime call failed (incl. earlier faults)   */

/* gdn_config.io_dtype: element type of q, k, v and o */
#define GDN_BF16 0
#define GDN_F32  1

/* gdn_config.flags */
#define GDN_L2NORM_QK   (1u << 0) /* normalise q and k per token (default on)     */
#define GDN_GATE_IS_LOG (1u << 1) /* io->a holds log a_t (<= 0) instead of a_t;
                                     the gradient da is then dL/d(log a_t)        */
#define GDN_POISON_WS   (1u << 2) /* debugging: fill the workspace with NaN bytes at
                                     init (the gradient workspaces when the first
                                     gradient call allocates them), so that a read
                                     of a workspace byte the kernels did not write
                                     shows up in the output */

/* per-call flags */
#define GDN_NO_COMMIT  (1u << 0)  /* forward: leave the cache unchanged; the final
                                     state goes to state_out (when non-NULL)      */
#define GDN_SEQUENTIAL (1u << 1)  /* use the token-sequential fp32 kernel instead
                                     of the chunked MFMA kernels                 */

typedef struct gdn_config {
    int32_t batch;       /* B independent streams, >= 1                          */
    int32_t heads;       /* H heads per stream, >= 1                             */
    int32_t d_k;         /* key/query width: multiple of 16, 16..128             */
    int32_t d_v;         /* value width (state rows): multiple of 16, 16..128;   */
                         /* the chunked kernels need d_v == d_k (16, 32, 64, 112, 128) */
    int64_t max_tokens;  /* largest T of any call, 1 .. 2^30; sizes the fixed    */
                         /* workspace                                          */
    int32_t subchunk;    /* chunked-kernel sub-chunk C: 0 (= 64), 16, 32 or 64  */
    int32_t io_dtype;    /* GDN_BF16 or GDN_F32.  With GDN_F32 the chunked       */
                         /* kernels stage q, k, v as bf16 (round to nearest    */
                         /* even; a workspace of 3*B*max_tokens*H*d_k*2 bytes   */
                         /* is added at init) and store o in fp32; the          */
                         /* sequential kernel stays in fp32 throughout          */
    uint32_t flags;      /* GDN_L2NORM_QK | GDN_GATE_IS_LOG | GDN_POISON_WS      */
    float l2_eps;        /* eps inside the L2 norm (1e-6 is the usual value)     */
    float scale;         /* output scale (1.0 when q is unit-norm)               */
} gdn_config;

typedef struct gdn_io {
    const void* q;        /* [B, T, H, d_k] io_dtype                           */
    const void* k;        /* [B, T, H, d_k] io_dtype                           */
    const void* v;        /* [B, T, H, d_v] io_dtype                           */
    void* o;              /* [B, T, H, d_v] io_dtype, written                  */
    const float* a;       /* [B, T, H] decay a_t in (0, 1] (log a_t with       */
                          /* GDN_GATE_IS_LOG); log-domain inside, clamped at -80 */
    const float* beta;    /* [B, T, H] write strength beta_t                    */
    int64_t q_strides[3]; /* (b, t, h) strides of q, in elements                */
    int64_t k_strides[3];
    int64_t v_strides[3];
    int64_t o_strides[3];
    int64_t g_strides[3]; /* shared by a and beta                               */
} gdn_io;

typedef struct gdn_stream gdn_stream;

/* Create a handle on `device`: allocates the state cache [B, H, d_v, d_k] fp32
 * (zeroed) plus a workspace sized by max_tokens.  Memory is fixed here and never
 * grows with the length of the stream.  Errors: GDN_E_INVAL (NULL cfg/out, bad
 * flags), GDN_E_SHAPE, GDN_E_DTYPE, GDN_E_NOMEM, GDN_E_HIP (bad device). */
GDN_API int gdn_stream_init(const gdn_config* cfg, int device, gdn_stream** out);

/* Free every allocation of the handle (waits for its device to go idle).
 * NULL is a no-op. */
GDN_API int gdn_stream_destroy(gdn_stream* s);

/* Causal forward scan of T tokens (0 <= T <= max_tokens) from the cached state;
 * writes o for every token.  Without GDN_NO_COMMIT the final state replaces the
 * cache; with it the cache is untouched and the final state goes to state_out
 * ([B, H, d_v, d_k] fp32 device memory, may be NULL).  T = 0 leaves everything
 * as it is (state_out, if given, receives the cached state). */
GDN_API int gdn_chunk_forward(gdn_stream* s, const gdn_io* io, int64_t T, uint32_t flags,
                              float* state_out, void* hip_stream);

/* The causal forward scan of gdn_chunk_forward, split in time (the three-stage pipeline of
 * the Chinese summary, "Method steps", step 4, in our reading: segment summaries, a serial
 * pass over them, then each segment from its start state).  The chunk's ceil(T / C) steps
 * are cut into `segments` consecutive segments of equal length (the last one shorter;
 * `segments` is lowered to the number of steps if larger, and to the smallest count of that
 * length with no empty segment).  Three launches after the prep: every segment from a zero
 * state (its state contribution D) and from the identity with v read as zero (the product P
 * of its transitions), all at once; per stream-head the start states S_{s+1} = S_s P_s + D_s
 * in fp32, serially over the segments from the cached state; every segment again from its
 * start state, writing o.  Same result as gdn_chunk_forward up to rounding, with about three
 * times its scan work spread over `segments` times as many workgroups: it pays when the
 * stream-heads B H are few and the chunk is long (the plain scan then leaves most of the chip
 * idle).  Arguments, flags (GDN_SEQUENTIAL is rejected with GDN_E_INVAL), cache handling and
 * state_out as for gdn_chunk_forward.  segments = 1, or a chunk of one step, runs
 * gdn_chunk_forward.  Workspace: 3 x segments states [B, H, d_v, d_k] fp32, allocated by the
 * first call that needs it (and again, after waiting for the device, by a call that needs
 * more).  Errors: as gdn_chunk_forward, GDN_E_INVAL for segments < 1, GDN_E_NOMEM. */
GDN_API int gdn_chunk_forward_split(gdn_stream* s, const gdn_io* io, int64_t T, int segments, uint32_t flags,
                                    float* state_out, void* hip_stream);

/* Backward scan inside the chunk: t = T-1 .. 0 from a zero state, each token
 * with its own a_t and beta_t.  Writes o; never reads or writes the cache.
 * state_out (may be NULL) receives the state after absorbing token 0. */
GDN_API int gdn_chunk_reverse(gdn_stream* s, const gdn_io* io, int64_t T, uint32_t flags,
                              float* state_out, void* hip_stream);

/* Both scans of one chunk in one pass (the pair the streaming model runs per
 * chunk): forward from the cache into o_fwd (committing unless GDN_NO_COMMIT,
 * then the final forward state goes to state_out) and reverse into o_rev.
 * `io->o` is o_fwd; o_rev has o's strides. */
GDN_API int gdn_chunk_bidir(gdn_stream* s, const gdn_io* io, void* o_rev, int64_t T,
                            uint32_t flags, float* state_out, void* hip_stream);

/* Allocation-free variant of gdn_chunk_bidir, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  It needs no handle and calls no hipMalloc, hipFree or
 * allocating library routine.  Runs on the current HIP device (the one that
 * hip_stream belongs to).
 *  - cfg: as for gdn_stream_init, except that io_dtype must be GDN_BF16
 *    (GDN_E_DTYPE otherwise), flags may hold GDN_L2NORM_QK and GDN_GATE_IS_LOG
 *    only, and max_tokens is not used (T bounds the call).
 *  - The forward scan starts from state_in ([B, H, d_v, d_k] fp32 device memory,
 *    NULL = zero) and writes o (io->o); its final state goes to state_out (same
 *    layout, may be NULL, may equal state_in).  The reverse scan starts from zero
 *    and writes o_rev (io->o's strides).  T = 0 copies state_in to state_out.
 *  - status: device-visible int (device memory or mapped host memory), not
 *    NULL.  The kernels set it to 1 when a wait gives up (spin limit as for a
 *    handle, read from GDN_SPIN_LIMIT at the first call); the outputs of that
 *    call are then not valid.  The library never clears it.
 *  - Workspace: the prep and scan items, 2 B H ceil(T / C) of chunk_item bytes
 *    (13312 bytes for C = 64 and d_k = 112: the 2640-token, 20-head chunk
 *    takes 22.4 MB),
 *    live in a static device array of GDN_NOALLOC_SCRATCH_BYTES, one per
 *    device, created when the library's code is loaded on that device and held
 *    until the process ends.  A call that needs more returns GDN_E_SHAPE.
 *  - Every call on a device uses that device's one array: calls that overlap
 *    in time on one device (different streams, no ordering between them) race
 *    and produce wrong outputs.  Calls on one stream are ordered and safe.
 * Errors: GDN_E_INVAL (NULL cfg, io or status, bad flags, alignment or
 * strides), GDN_E_SHAPE, GDN_E_DTYPE, GDN_E_HIP; on error nothing is enqueued. */
#define GDN_NOALLOC_SCRATCH_BYTES ((int64_t)64 << 20)
GDN_API int gdn_chunk_bidir_noalloc(const gdn_config* cfg, const gdn_io* io, void* o_rev, int64_t T,
                                    const float* state_in, float* state_out, int* status, void* hip_stream);

/* Asynchronous device-to-device copy of the cache [B, H, d_v, d_k] fp32 into
 * dst / from src (src NULL = zero the cache).  Checkpoint, resume and replay. */
GDN_API int gdn_state_get(gdn_stream* s, float* dst, void* hip_stream);
GDN_API int gdn_state_set(gdn_stream* s, const float* src, void* hip_stream);

/* Per-kernel timing for measurement.  While enabled, every launch of the handle
 * is bracketed by hipEvents recorded on the launch stream; gdn_profile_read
 * waits for them and returns, per kernel kind (GDN_KERNEL_*), the summed
 * duration in milliseconds and the launch count (arrays of GDN_KERNEL_COUNT;
 * either may be NULL), then clears the totals when `reset` is non-zero. */
#define GDN_KERNEL_PREP  0   /* chunk preparation (norms, gates, Gram, UT inverse) */
#define GDN_KERNEL_SCAN  1   /* chunk scan (state recurrence and outputs)          */
#define GDN_KERNEL_SEQ   2   /* token-sequential kernel                            */
#define GDN_KERNEL_BWD   3   /* gradient of one scan (both of its kernels)         */
#define GDN_KERNEL_COUNT 4
GDN_API int gdn_profile(gdn_stream* s, int enable);
GDN_API int gdn_profile_read(gdn_stream* s, double* ms, int64_t* launches, int reset);

/* Gradients of one scan, for training over streaming chunks (the Chinese summary,
 * "Method steps": bidirectional training on short clips and streaming training on
 * long ones).  The pages print no formula for this pass; it is the reverse-mode
 * derivative of the per-token rule, computed by a token-sequential fp32 path.
 * All pointers are device memory on the handle's device; gradients are written
 * in fp32, contiguous. */
typedef struct gdn_grad {
    const void* d_o;        /* [B, T, H, d_v] io_dtype, io->o_strides: dL/do of the scan   */
    const float* d_state;   /* [B, H, d_v, d_k] fp32: dL/d(final state), or NULL (zero)     */
    const float* state0;    /* [B, H, d_v, d_k] fp32: start state of a forward scan, or NULL
                               (zero); must be NULL for the reverse scan (it starts at zero) */
    float* dq;              /* [B, T, H, d_k] written                                       */
    float* dk;              /* [B, T, H, d_k] written                                       */
    float* dv;              /* [B, T, H, d_v] written                                       */
    float* da;              /* [B, T, H] written (gradient with respect to a_t)             */
    float* dbeta;           /* [B, T, H] written                                            */
    float* d_state0;        /* [B, H, d_v, d_k] written when non-NULL                       */
} gdn_grad;

/* Gradient of the forward scan (reverse = 0: t ascending from g->state0) or of the
 * reverse scan (reverse = 1: t descending from zero) over T tokens of io->q, k, v,
 * a, beta (io->o is not used; its strides give d_o's layout).  Never reads or
 * writes the cache.  Asynchronous on hip_stream.  The first call on a handle
 * allocates a backward workspace of 4 (B H (d_v/4)(ceil(max_tokens/8)+1
 * + ceil(max_tokens/64)) 4 d_k + B max_tokens H (d_v/4)(2 d_k + 4)) bytes (state
 * checkpoints every block of 8 tokens, adjoint checkpoints every 64 tokens, and
 * partial sums per block of 4 state rows), kept until gdn_stream_destroy
 * (GDN_E_NOMEM if that fails).  Errors: GDN_E_INVAL (NULL handle/io/g/output,
 * bad strides, state0 given with reverse), GDN_E_SHAPE (T outside [0, max_tokens]),
 * GDN_E_HIP; on error nothing is enqueued.  T = 0 writes d_state0 = d_state. */
GDN_API int gdn_chunk_backward(gdn_stream* s, const gdn_io* io, const gdn_grad* g, int64_t T, int reverse,
                               void* hip_stream);

/* Gradients of both scans of a gdn_chunk_bidir call, in one launch pair: g_fwd for the
 * forward scan (as gdn_chunk_backward with reverse = 0: g_fwd->state0 is its start
 * state) and g_rev for the intra-chunk reverse scan (as reverse = 1: g_rev->state0 must
 * be NULL).  Training on short clips needs both scans' gradients of every layer (the
 * Chinese summary, "Method steps", step 2: bidirectional training before streaming
 * training); the two are independent, so one launch runs them side by side.  The two
 * d_o tensors share io->o's strides.  Results are bitwise those of the two separate
 * calls.  The first call on a handle also allocates a second backward workspace of the
 * size given above (for the reverse scan), kept until gdn_stream_destroy.  Errors as
 * gdn_chunk_backward (GDN_E_INVAL also for a NULL g_fwd or g_rev); on error nothing is
 * enqueued.  T = 0 writes each d_state0 from its d_state. */
GDN_API int gdn_chunk_backward_bidir(gdn_stream* s, const gdn_io* io, const gdn_grad* g_fwd, const gdn_grad* g_rev,
                                     int64_t T, void* hip_stream);

/* Message for the last failing call on this thread ("" when none). */
GDN_API const char* gdn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_STREAM_H */
