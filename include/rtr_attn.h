/*
 * rtr_attn.h -- C ABI of librtr_attn.so: frame-block-causal attention and the
 * reference-anchored rolling KV cache of a streaming autoregressive video DiT,
 * for AMD Instinct MI355X (gfx950).
 *
 * Source of the method: web notes on "DiT as Real-Time Rerenderer: Streaming
 * Video Stylization with Autoregressive Diffusion Transformer" (RTR-DiT):
 *   - Key Designs 2, Attn equation: Attn(Q,K,V) = softmax(Q K^T / sqrt(d) + M) V
 *     with M_ij = 0 when floor(j/k) <= floor(i/k) and -inf otherwise; d is the
 *     head dimension and k the number of spatial tokens per latent frame.
 *   - Key Designs 1: the reference latent is prepended as one extra latent frame.
 *   - Key Designs 4: a rolling 3D-attention KV cache; new frames are appended,
 *     the oldest evicted once full; the reference tokens stay anchored at the
 *     front as a resident slot; on a condition switch the cache keeps the most
 *     recent frame and a new reference is anchored at the front.
 *
 * Conventions shared by every entry point
 *   - Layout: token-major [tokens, H, d], d contiguous; row stride H*d elements.
 *     Cache frames are [k, H, d] blocks; ring buffers hold W such frames and the
 *     reference buffer R_cap frames.
 *   - Memory: every device pointer is owned by the caller and must stay valid
 *     until the work enqueued on `stream` has finished.  The library allocates
 *     no device memory.  Device pointers must be 16-byte aligned.  Output
 *     buffers must not overlap inputs.
 *   - Asynchrony: device work is enqueued on `stream` (a hipStream_t; NULL is
 *     the default stream) and nothing waits for it.  Cache metadata lives on the
 *     host and changes at call time, so calls on one cache must be issued on
 *     one stream (or the caller orders the streams).
 *   - Errors: every argument is checked before anything is enqueued.  On error
 *     the call returns a negative rtr_status, records a message readable with
 *     rtr_last_error() (per thread), changes no state and enqueues nothing.
 *     A failed kernel launch returns RTR_EHIP.
 *   - Threads: a cache handle is not thread-safe.
 */
#ifndef RTR_ATTN_H
#define RTR_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RTR_OK = 0,
    RTR_EINVAL = -1,        /* bad argument (null, negative size, misaligned, overlap) */
    RTR_EUNSUPPORTED = -2,  /* valid request outside what the library implements */
    RTR_EHIP = -3,          /* HIP runtime or launch failure */
    RTR_ESTATE = -4         /* operation inconsistent with the cache state */
} rtr_status;

typedef enum { RTR_BF16 = 0, RTR_F32 = 1 } rtr_dtype;

/* Reference handling on a condition switch (Key Designs 4). */
typedef enum {
    RTR_REF_KEEP = 0,     /* text-only switch: reference slot unchanged */
    RTR_REF_REPLACE = 1,  /* anchor a new reference at the front */
    RTR_REF_CLEAR = 2     /* drop the reference (text-guided mode) */
} rtr_ref_mode;

typedef void *rtr_stream; /* hipStream_t */

#define RTR_MAX_WINDOW 64 /* window frames W */
#define RTR_MAX_REF 4     /* reference frames R (several anchored style references) */
#define RTR_MAX_CHUNK 16  /* frames per streaming chunk C */

typedef struct rtr_kv_cache rtr_kv_cache; /* opaque, host-side ring metadata */

/* Snapshot of a cache's metadata.  Window entries are in logical order, oldest
 * first: entry p lives in physical ring slot slot[p] = (head + p) mod
 * ring_slots and holds the frame with generation-order id frame_id[p]. */
typedef struct {
    int32_t window_frames;  /* W */
    int32_t count;          /* valid window frames, 0..W */
    int32_t head;           /* physical slot of the oldest valid frame */
    int32_t ref_frames;     /* reference frames currently anchored, 0..R_cap */
    int64_t ref_generation; /* incremented by every REPLACE */
    int64_t next_frame_id;  /* id the next appended frame receives */
    int32_t slot[RTR_MAX_WINDOW];
    int64_t frame_id[RTR_MAX_WINDOW];
    int32_t ring_slots;     /* physical ring slots N, W <= N <= RTR_MAX_WINDOW */
} rtr_kv_state;

/* ------------------------------------------------------------------------
 * Full-sequence form (training / teacher forcing).  Key Designs 2, Attn
 * equation, over one sequence of T tokens whose frame 0 may be the reference.
 *
 *   q, k, v : [T, H, d] device, dtype in_dtype
 *   o       : [T, H, d] device, dtype out_dtype (bf16 or f32 for bf16 input;
 *             f32 for f32 input)
 *   lse     : [H, T] device float32, natural-log softmax denominators
 *             (log-sum-exp of the scaled, masked logits), or NULL
 *   tokens_per_frame : k >= 1; k >= T gives the unmasked bidirectional teacher
 *   d       : 64 or 128
 *   scale   : logit scale; <= 0 selects 1/sqrt(d)
 *   workspace, workspace_bytes : split-K scratch (see rtr_attn_workspace_size)
 *             or NULL, 0
 * T == 0 is a no-op.  Returns RTR_OK or a negative rtr_status.
 * ---------------------------------------------------------------------- */
int rtr_attn_block_causal(const void *q, const void *k, const void *v, void *o, float *lse,
                          int64_t T, int32_t H, int32_t d, int64_t tokens_per_frame,
                          rtr_dtype in_dtype, rtr_dtype out_dtype, float scale,
                          void *workspace, size_t workspace_bytes, rtr_stream stream);

/* ------------------------------------------------------------------------
 * Split-K workspace.  Without one, each (head, block of query rows) is one
 * workgroup that walks all its visible keys, and the longest such unit bounds
 * the call.  With one (bf16 input, d == 128; otherwise it is accepted and
 * unused), the visible key tiles of all units are shared out evenly over the
 * GPU's compute units: a unit cut between two of them leaves unnormalised
 * partial results (fp32 O, exponent reference and row sum per query) in the
 * workspace, and a second kernel on the same stream merges them in a fixed
 * order, O = sum_s w_s O_s / sum_s w_s l_s with w_s the softmax weights of
 * the parts (the exact softmax over the union of their keys).  The result is
 * deterministic and equals the unsplit one up to fp32 rounding.
 *
 * rtr_attn_workspace_size stores in *bytes the size the current HIP device
 * needs (it depends on its compute-unit count, not on the token count; 0 when
 * the configuration never splits).  The workspace is caller-owned device
 * memory, 16-byte aligned, uninitialised on entry, clobbered on exit, and
 * must not overlap any input, output or cache buffer.  Calls that may run
 * concurrently need separate workspaces.  A workspace smaller than required
 * is RTR_EINVAL.
 * ---------------------------------------------------------------------- */
int rtr_attn_workspace_size(int32_t d, rtr_dtype in_dtype, size_t *bytes);

/* ------------------------------------------------------------------------
 * Gradients of the full-sequence form: dQ, dK, dV of Attn(Q,K,V) (Key
 * Designs 2 equation) for an upstream gradient dO -- the pass through which
 * the generator post-training of Key Designs 3 (Self Forcing + DMD) sends its
 * gradient.  With P = softmax(Q K^T * scale + M) recomputed from lse:
 *   dV = P^T dO,  dS = P * (dO V^T - rowsum(dO * O)),  dK = scale dS^T Q,
 *   dQ = scale dS K.
 *
 *   q, k, v : [T, H, d] device bf16, the forward's inputs
 *   o, lse  : the forward's output ([T, H, d] bf16) and natural-log LSE
 *             ([H, T] float32) for the same inputs, mask and scale, as
 *             written by rtr_attn_block_causal
 *   d_o     : [T, H, d] device bf16, gradient of the loss with respect to o
 *   dq, dk, dv : [T, H, d] device bf16 outputs (overwritten, not accumulated)
 *   tokens_per_frame, scale : as in the forward call
 *   d       : 128
 *   dtype   : RTR_BF16
 *   workspace, workspace_bytes : caller-owned device scratch of at least
 *             rtr_attn_bwd_workspace_size(T, H, d) bytes, 256-byte aligned,
 *             clobbered; it must not overlap any argument buffer, and calls
 *             that may run concurrently need separate workspaces
 * Limits: T * H * d < 2^31.  T == 0 is a no-op.  Returns RTR_OK or a negative
 * rtr_status (RTR_EUNSUPPORTED for another dtype or head dim).
 * ---------------------------------------------------------------------- */
int rtr_attn_block_causal_bwd(const void *q, const void *k, const void *v, const void *o,
                              const float *lse, const void *d_o, void *dq, void *dk, void *dv,
                              int64_t T, int32_t H, int32_t d, int64_t tokens_per_frame,
                              rtr_dtype dtype, float scale, void *workspace,
                              size_t workspace_bytes, rtr_stream stream);

/* Workspace bytes rtr_attn_block_causal_bwd (T tokens) and
 * rtr_attn_stream_step_bwd (T = chunk_frames * k query rows) need: per head
 * and 32-row tile, 256 bytes of row statistics and 16 KiB of transposed Q and
 * dO. */
int rtr_attn_bwd_workspace_size(int64_t T, int32_t H, int32_t d, size_t *bytes);

/* ------------------------------------------------------------------------
 * KV cache of one attention layer over caller-owned device buffers
 * (Key Designs 4).  k_ring, v_ring: [W, k, H, d]; k_ref, v_ref: [R_cap, k, H, d]
 * (may be NULL when R_cap == 0).  Starts empty: count 0, no reference,
 * generation 0, next frame id 0.  *out receives a handle to free with
 * rtr_kv_destroy.  0 <= W <= RTR_MAX_WINDOW (W = 0 keeps no history; the ring
 * pointers may then be NULL); 0 <= R_cap <= RTR_MAX_REF; d in {64, 128}.
 * ---------------------------------------------------------------------- */
int rtr_kv_create(rtr_kv_cache **out, void *k_ring, void *v_ring, void *k_ref, void *v_ref,
                  int32_t window_frames, int32_t ref_capacity_frames,
                  int64_t tokens_per_frame, int32_t H, int32_t d, rtr_dtype dtype);

/* The same cache over a ring of ring_slots >= W physical frame slots
 * (k_ring, v_ring: [ring_slots, k, H, d]; W <= ring_slots <= RTR_MAX_WINDOW);
 * rtr_kv_create is this with ring_slots = W.  The window is still the W
 * newest frames.  With ring_slots >= W + n, an append of n frames writes only
 * slots that the current window does not use (once the window is full, each
 * new frame goes to the slot after the newest and the oldest frame's slot is
 * freed), so it may run concurrently with a step that reads the current
 * window -- on another stream, after the previous step completes (which read
 * the slots this append overwrites) and before the next step starts -- and a
 * producer may write a chunk into the slots rtr_kv_next_slots reports before
 * the step that reads the chunk. */
int rtr_kv_create_slots(rtr_kv_cache **out, void *k_ring, void *v_ring, void *k_ref, void *v_ref,
                        int32_t window_frames, int32_t ring_slots, int32_t ref_capacity_frames,
                        int64_t tokens_per_frame, int32_t H, int32_t d, rtr_dtype dtype);
int rtr_kv_destroy(rtr_kv_cache *kv);

/* Commit n_frames newly generated frames, given as [n_frames, k, H, d] device
 * buffers k_new, v_new (Key Designs 4: appended in order; once the window is
 * full each append evicts the oldest frame; the reference slot is never
 * touched).  Only the newest min(n_frames, W) frames are copied; the copy is
 * enqueued on `stream`.  n_frames == 0 is a no-op.  With ring_slots = W the
 * copy overwrites the evicted frames' slots, which a step of the current
 * window reads: enqueue it after that step (same stream, or after it
 * completes). */
int rtr_kv_append_evict(rtr_kv_cache *kv, const void *k_new, const void *v_new,
                        int32_t n_frames, rtr_stream stream);

/* Physical ring slots the next n_frames appends would be written to, in
 * order; frames that the same append would evict again get -1.  Changes
 * nothing.  Lets a producer write K/V straight into the ring (zero-copy
 * append).  Order: once the window is full and ring_slots < W + n_frames,
 * some of these are slots of the oldest frames, which every step until the
 * commit still reads, so the producer writes them only after the last step
 * that reads the current window is enqueued, on the same stream (or after it
 * completes).  Slots outside the window (while it has free slots, or the
 * spare slots of a ring_slots > W cache) are not read by any step, and a
 * chunk may be written there first and passed to the step as its k, v.  A
 * step whose q, k or v overlaps a slot in use or the reference returns
 * RTR_EINVAL. */
int rtr_kv_next_slots(const rtr_kv_cache *kv, int32_t n_frames, int32_t *slots);

/* Metadata-only commit of n_frames frames that the caller has already written
 * into the slots reported by rtr_kv_next_slots (zero-copy append).  Same
 * state change as rtr_kv_append_evict; enqueues nothing. */
int rtr_kv_commit_inplace(rtr_kv_cache *kv, int32_t n_frames);

/* ------------------------------------------------------------------------
 * Streaming form for one chunk of C = chunk_frames latent frames.  The chunk
 * queries q ([C*k, H, d]) attend to the anchored reference frame(s), every
 * valid window frame in logical order, and the chunk's own keys k, v
 * ([C*k, H, d]) of chunk frames up to their own (the Attn mask with the chunk
 * placed after the cached frames).  The cache is only read; commit the chunk
 * afterwards with rtr_kv_append_evict.  o: [C*k, H, d] out_dtype; lse: [H, C*k]
 * float32 or NULL.  1 <= C <= RTR_MAX_CHUNK; scale <= 0 selects 1/sqrt(d).
 * workspace, workspace_bytes: split-K scratch as for rtr_attn_block_causal.
 * q, k and v may lie in ring slots that the window does not use (a chunk
 * written where rtr_kv_next_slots put it), never in a slot in use or in the
 * reference slot (RTR_EINVAL); o and lse overlap no input and no cache buffer.
 * ---------------------------------------------------------------------- */
int rtr_attn_stream_step(const rtr_kv_cache *kv, const void *q, const void *k, const void *v,
                         void *o, float *lse, int32_t chunk_frames, rtr_dtype out_dtype,
                         float scale, void *workspace, size_t workspace_bytes,
                         rtr_stream stream);

/* The same step with a coarser mask inside the chunk (chunk-level causality:
 * fixed-size chunks whose tokens see each other and every earlier token).  The
 * chunk's frames form blocks of block_frames frames; query row r sees every
 * cached key and the chunk keys of blocks <= its own, i.e. the frame mask with
 * block_frames * k tokens as its unit.  block_frames == 1 is
 * rtr_attn_stream_step; block_frames >= chunk_frames makes the whole chunk
 * mutually visible.  Other arguments and errors as rtr_attn_stream_step. */
int rtr_attn_stream_step_blocked(const rtr_kv_cache *kv, const void *q, const void *k, const void *v,
                                 void *o, float *lse, int32_t chunk_frames, int32_t block_frames,
                                 rtr_dtype out_dtype, float scale, void *workspace,
                                 size_t workspace_bytes, rtr_stream stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the
 * streaming step of rtr_attn_stream_step_blocked with its split-K scratch in a
 * static device array inside the library (34 MB per GPU, held from the first
 * call on that GPU until the process ends) instead of a caller workspace.  It
 * calls no device allocation routine.  The split planner keeps to that
 * scratch (256 partial-result slots); a problem that would need more runs
 * with fewer, longer pieces or unsplit, so no input size exceeds it.  Every
 * call on one GPU shares that GPU's scratch: calls that overlap in time on
 * one GPU (concurrent streams, or several host threads) race and must be
 * serialised by the caller.  Other arguments, results and errors as
 * rtr_attn_stream_step_blocked. */
int rtr_attn_stream_step_noalloc(const rtr_kv_cache *kv, const void *q, const void *k, const void *v,
                                 void *o, float *lse, int32_t chunk_frames, int32_t block_frames,
                                 rtr_dtype out_dtype, float scale, rtr_stream stream);

/* ------------------------------------------------------------------------
 * Gradients of one streaming step (Key Designs 2 and 4: the step's Attn over
 * [reference | window | chunk]; Key Designs 3 trains the causal generator by
 * rolling it out over this cache, so its gradient passes back through every
 * step).  kv must be as it was when the forward step ran, metadata and the
 * contents of the slots that step read: call this before the chunk is
 * committed with rtr_kv_append_evict (which may overwrite the oldest window
 * frame), or restore both the snapshot (rtr_kv_set_state) and the evicted
 * frames' data; q, k, v: the chunk's [C*k, H, d]; o and
 * lse: that forward step's output and its natural-log LSE [H, C*k] (from
 * rtr_attn_stream_step_blocked with the same chunk_frames, block_frames and
 * scale); d_o: upstream gradient [C*k, H, d].
 * Outputs (device, caller-owned, overwritten):
 *   dq, dk, dv : [C*k, H, d], the chunk's gradients
 *   dk_cache, dv_cache : [P, H, d], P = (ref_frames + count) * k, gradients
 *             of the cached keys and values in the order the step reads them
 *             (reference frames, then window frames oldest first); with a
 *             position-aware reference (rtr_kv_set_ref_rope) dk_cache's
 *             reference rows are with respect to the stored, unrotated keys.
 *             Both NULL: the cache is treated as constant and not
 *             differentiated (P == 0 writes nothing).
 * bf16 cache, d = 128 only.  workspace: rtr_attn_bwd_workspace_size(C*k, H,
 * d) bytes, 256-byte aligned, overlapping no argument.  No output may overlap
 * an input, the cache buffers or another output; q, k, v, o and d_o may not
 * overlap a window slot in use or the reference slot.  Limits: C*k * H * d < 2^31.
 * Returns RTR_OK or a negative rtr_status; every argument is checked before
 * anything is enqueued (a failing launch reports RTR_EHIP).
 * ---------------------------------------------------------------------- */
int rtr_attn_stream_step_bwd(const rtr_kv_cache *kv, const void *q, const void *k, const void *v,
                             const void *o, const float *lse, const void *d_o, int32_t chunk_frames,
                             int32_t block_frames, void *dq, void *dk, void *dv, void *dk_cache,
                             void *dv_cache, float scale, void *workspace, size_t workspace_bytes,
                             rtr_stream stream);

/* Condition switch (Key Designs 4).  First the reference: KEEP leaves it,
 * REPLACE anchors ref_frames (1..R_cap) new frames k_ref, v_ref
 * ([ref_frames, k, H, d] device; both NULL means the caller already wrote
 * them into the cache's reference buffers) and increments the generation,
 * CLEAR removes it.  Then the window keeps only its newest keep_recent frames
 * (-1 keeps all; the notes keep the most recent frame, keep_recent = 1).
 * Window trimming moves no data. */
int rtr_kv_reset_ref(rtr_kv_cache *kv, rtr_ref_mode mode, const void *k_ref, const void *v_ref,
                     int32_t ref_frames, int32_t keep_recent, rtr_stream stream);

/* ------------------------------------------------------------------------
 * Text cross-attention and its cache (Key Designs 1: text is encoded by T5 and
 * injected through cross attention; Key Designs 4: a fixed-length
 * cross-attention cache is initialised and, when a new text prompt arrives,
 * re-initialised so that the old condition is discarded).  The cache holds
 * the K/V of the current text condition for one layer, [n, H, d] with
 * 1 <= n <= capacity, in caller-owned device buffers k_buf, v_buf of
 * [capacity, H, d]; every chunk's queries attend to all n tokens (no mask):
 *   O = softmax(Q K_text^T * scale) V_text.
 * A reference-only switch leaves this cache untouched; a text switch resets
 * it (and, on the 3D cache, calls rtr_kv_reset_ref with RTR_REF_KEEP).
 * ---------------------------------------------------------------------- */
typedef struct rtr_text_cache rtr_text_cache; /* opaque, host-side metadata */

int rtr_text_cache_create(rtr_text_cache **out, void *k_buf, void *v_buf, int32_t capacity_tokens,
                          int32_t H, int32_t d, rtr_dtype dtype);
int rtr_text_cache_destroy(rtr_text_cache *tc);

/* Re-initialise with a new condition of n_tokens (1..capacity) tokens:
 * k_text, v_text are [n_tokens, H, d] device buffers copied into the cache on
 * `stream` (both NULL: the caller already wrote them into k_buf/v_buf).
 * n_tokens == 0 clears the cache (no condition).  Increments the generation
 * whenever a condition is set. */
int rtr_text_cache_reset(rtr_text_cache *tc, const void *k_text, const void *v_text,
                         int32_t n_tokens, rtr_stream stream);

/* Current token count and generation. */
int rtr_text_cache_state(const rtr_text_cache *tc, int32_t *n_tokens, int64_t *generation);

/* Cross-attention of Tq query rows ([Tq, H, d], the cache's dtype) to the
 * cache's tokens: o [Tq, H, d] out_dtype, lse [H, Tq] float32 or NULL,
 * scale <= 0 selects 1/sqrt(d), workspace as for rtr_attn_block_causal.
 * An empty cache is RTR_ESTATE. */
int rtr_attn_cross(const rtr_text_cache *tc, const void *q, void *o, float *lse, int64_t Tq,
                   rtr_dtype out_dtype, float scale, void *workspace, size_t workspace_bytes,
                   rtr_stream stream);

/* Gradients of that cross-attention (the generator's post-training, Key
 * Designs 3, back-propagates through the text injection of Key Designs 1 as
 * through the self-attention): for an upstream gradient d_o [Tq, H, d] and the
 * forward's o [Tq, H, d] and natural-log lse [H, Tq] (rtr_attn_cross with the
 * same scale and bf16 output), dq [Tq, H, d] and, when dk_text and dv_text are
 * given, the gradients of the current condition's text keys and values
 * [n, H, d] (both NULL: the text is treated as constant).  bf16 cache, d = 128
 * only; workspace: rtr_attn_cross_bwd_workspace_size(Tq, n, H, d) bytes with
 * text gradients (their fp32 partial sums when the few text key blocks are
 * split over the query rows), rtr_attn_bwd_workspace_size(Tq, H, d) without;
 * 256-byte aligned.  No output may overlap an input, the cache or another
 * output.
 * Limits: Tq * H * d < 2^31.  Tq == 0 is a no-op; an empty cache is
 * RTR_ESTATE. */
int rtr_attn_cross_bwd_workspace_size(int64_t Tq, int32_t n_text, int32_t H, int32_t d, size_t *bytes);
int rtr_attn_cross_bwd(const rtr_text_cache *tc, const void *q, const void *o, const float *lse,
                       const void *d_o, int64_t Tq, void *dq, void *dk_text, void *dv_text, float scale,
                       void *workspace, size_t workspace_bytes, rtr_stream stream);

/* Position-aware reference (rotary position encoding along time).  Rotary
 * encodings are baked into cached K, so in a rolling window the frames keep
 * their generation-time positions, which is exact for them (scores depend on
 * position differences only) -- but a reference anchored at the start would
 * drift ever further from the current frames.  With a view buffer set, every
 * streaming call first re-encodes the reference K into k_ref_view so that
 * the reference frames sit directly in front of the oldest frame the call
 * sees, as the reference frame sits in front of the first frame in the full
 * sequence, and the call reads the reference K from the view (V unchanged).
 * Conventions: the caller encodes each frame's Q and K at temporal position
 * frame_id + position_offset (frame ids count appended frames from 0, see
 * rtr_kv_state) and reference frame r at position r; the encoding rotates
 * element pairs (2i, 2i+1) of every head, i < rope_pairs, by position *
 * rope_base^(-i / rope_pairs).  The reference is re-encoded (one kernel, bytes
 * of the reference read and written once) only when that position, the
 * reference or the number of reference frames changes.  k_ref_view:
 * [R_cap, k, H, d] caller-owned device buffer, or NULL to switch this off. */
int rtr_kv_set_ref_rope(rtr_kv_cache *kv, void *k_ref_view, int32_t rope_pairs, float rope_base,
                        int64_t position_offset);

/* Metadata snapshot / restore (checkpoint-resume).  set_state validates the
 * snapshot against the cache's W, ring slots and R_cap and changes nothing on
 * error. */
int rtr_kv_get_state(const rtr_kv_cache *kv, rtr_kv_state *out);
int rtr_kv_set_state(rtr_kv_cache *kv, const rtr_kv_state *in);

/* Measurement helper (not part of the method): enqueues one single-lane
 * kernel that reads the shader-clock counter and the constant 100 MHz
 * counter until span_ticks (1..1e6) ticks of the latter have passed, and
 * writes the two differences to ticks[0] (shader clock) and ticks[1]
 * (100 MHz), a caller-owned device buffer of two 64-bit words.  The shader
 * clock over that interval is ticks[0] / ticks[1] * 100 MHz.  Returns
 * RTR_EINVAL for a NULL or misaligned buffer or a span out of range. */
int rtr_clock_sample(uint64_t *ticks, int64_t span_ticks, rtr_stream stream);

/* Diagnostics. */
const char *rtr_status_string(int code);
const char *rtr_last_error(void);
int rtr_version(void); /* major*10000 + minor*100 + patch */

#ifdef __cplusplus
}
#endif
#endif /* RTR_ATTN_H */
