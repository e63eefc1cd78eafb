/*
 * nha.h -- C ABI of the Native Hybrid Attention (NHA) layer operator for
 * AMD Instinct MI355X (gfx950).
 *
 * The operator (Paper-Notes page "Native Hybrid Attention for Efficient
 * Sequence Modeling", sections 整体框架 and 关键设计 > 层内混合; gist.science
 * page, "Mecanismo de Funcionamento"): per (batch, KV head) it keeps m
 * long-term key/value slots updated by a gated linear RNN,
 *     K_long <- Diag(alpha_t) K_long + (1 - alpha_t) (x) k,   V_long likewise,
 * where a token enters the slots only when it leaves the sliding window (token
 * shift: at step t >= w the token t - w is absorbed with gate alpha_t).  The
 * slots are concatenated with the w most recent exact tokens and ONE softmax,
 * scaled by 1/sqrt(d), runs over all m + w keys; RoPE (rotate-half, theta_i =
 * base^(-2i/d), absolute positions) is applied to the window query/keys only.
 * w = 0 is a pure gated-slot RNN; w >= T is causal softmax attention plus the m
 * never-written (zero) slots.
 *
 * Three calls follow the pages' statement of the problem:
 *   nha_fwd          chunkwise-parallel forward over a whole sequence (the
 *                    "Chunkwise 并行计算" section of the Paper-Notes page);
 *   nha_bwd          gradients dq, dk, dv, dalpha of the same forward
 *                    (training, ibid. 局限与展望: the chunk kernel serves training;
 *                    nha_bwd_after_fwd reuses the forward's workspace);
 *   nha_decode_step  one token of recurrent ("RNN mode") inference
 *                    (ibid. 局限与展望; ai.info page, "Why This Matters").
 *
 * ---------------------------------------------------------------- conventions
 * Pointers: every tensor argument is a DEVICE pointer (hipMalloc'd or from a
 * framework allocator) unless stated otherwise; the descriptor is a HOST
 * pointer.  Layouts are dense, row-major, in this dimension order:
 *     q, o, dO, dq   [B][T][H][d]          k, v, dk, dv  [B][T][Hkv][d]
 *     alpha          [B][T][Hkv][m]        dalpha        [B][T][Hkv][m] (float)
 *     lse            [B][H][T] (float)     natural-log sum-exp of the scaled
 *                                          logits over all m + n_w keys
 * Query head h reads KV head h / (H / Hkv) (grouped-query attention).
 * Element type of q, k, v, alpha, o, dO, dq, dk, dv is desc->dtype.
 * Pointers must be 16-byte aligned.
 *
 * Ownership: the caller allocates every buffer, including the workspace and
 * the decode state; the library never allocates device memory, frees it or
 * synchronises the host with the GPU.  Calls return before the GPU has run;
 * buffers must stay alive until the stream work completes.  Calls on distinct
 * buffers are thread-safe.  `stream` is a hipStream_t passed as void* (NULL =
 * the null stream).
 *
 * Library state, the whole of it:
 *   - a per-device cache of the compute-unit count (read once with
 *     hipDeviceGetAttribute; sizes persistent grids);
 *   - per calling thread and device, ONE side stream (default priority,
 *     hipStreamNonBlocking) and three events (timing disabled), created by the
 *     first nha_fwd, nha_fwd_s0, nha_bwd, nha_bwd_after_fwd or nha_bwd_s0 call
 *     of that thread on that device, kept until nha_release_side_streams().
 *     Those calls fork independent launches onto the side stream (the window
 *     branch -- RoPE, then band attention -- beside the gate products and the
 *     slot-state scan where the forward runs its two-kernel form, i.e. below
 *     256 state-scan waves, B * Hkv * d / 16; the window dq beside the
 *     adjoint scan and slot pass B, then (bf16) dalpha's exact carries at
 *     every 16th chunk once the adjoint scan is done; the dalpha carry beside
 *     the window dk/dv)
 *     after an event recorded on `stream`, and
 *     make `stream` wait for the side stream before they return, so each call
 *     still behaves as one operation ordered on `stream`.  If the side
 *     stream cannot be created, every launch goes on `stream`.  The *_timed
 *     calls with non-NULL events, the decode step and nha_fwd_noalloc never
 *     use it.  Results are bitwise the same either way.
 *
 * Graph capture: the calls enqueue kernel launches and event records / waits
 * only (no memset, no allocation, no host synchronisation), so a sequence of
 * them on `stream` can be captured into a HIP graph and replayed; the side
 * stream joins the capture through its event waits.  Tested: nha_fwd then
 * nha_bwd_after_fwd captured once and replayed, with eager calls in between,
 * bitwise equal to the eager results at every replay.
 *   - nha_fwd_noalloc's scratch array (see there).
 *
 * Errors: every argument check runs on the host before any HIP call and
 * returns a status; nothing throws across the ABI and nothing aborts.  A
 * failed launch returns NHA_ERR_HIP.  Faults inside a kernel surface at the
 * caller's next stream synchronisation, as usual in HIP.
 *
 * Determinism: no atomics are used; results are bitwise reproducible for the
 * same inputs, shapes and device.
 */
#ifndef NHA_H_
#define NHA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NHA_OK = 0,
  NHA_ERR_INVALID_ARG = 1, /* null pointer, negative size, H % Hkv != 0, misaligned pointer */
  NHA_ERR_UNSUPPORTED = 2, /* valid but not implemented (d, m, C, or tile budget) */
  NHA_ERR_WORKSPACE = 3,   /* ws_bytes smaller than the *_workspace_size() query */
  NHA_ERR_HIP = 4          /* a HIP launch failed (no device, bad stream, ...) */
} nha_status;

typedef enum { NHA_DTYPE_F32 = 0, NHA_DTYPE_BF16 = 1 } nha_dtype;

typedef struct {
  int32_t B;         /* batch, >= 1 */
  int32_t T;         /* sequence length, >= 1 (decode: ignored) */
  int32_t H;         /* query heads, >= 1 */
  int32_t Hkv;       /* KV heads, >= 1, H % Hkv == 0 */
  int32_t d;         /* head dim: 32, 64 or 128 */
  int32_t m;         /* long-term slots: 0 .. 64 (0: no slots, sliding-window
                        attention alone; then w >= 1 and alpha, dalpha may be
                        NULL) */
  int32_t w;         /* sliding window, >= 0; w >= T allowed (full attention) */
  int32_t C;         /* chunk length of the chunkwise form: 16, 32 or 64.
                        Results do not depend on C beyond rounding. */
  float rope_base;   /* > 0: RoPE base; 0: RoPE disabled */
  float scale;       /* softmax scale; 0 means 1/sqrt(d) */
  int32_t dtype;     /* nha_dtype of the tensor arguments */
  int32_t no_token_shift; /* 0: the method -- a token enters the slots when it
                        leaves the window (at step t + w); 1: the token-shift
                        ablation -- every token enters the slots at its own
                        step t while the window still holds it */
} nha_desc;

/* Workspace bytes that nha_fwd / nha_bwd need for this descriptor; 0 when the
 * descriptor is invalid or unsupported (call nha_check_desc for the reason).
 * nha_check_desc applies the forward's rules.  The backward has one limit
 * more: its fp32 tiles must fit the 160 KB of LDS of a workgroup, which rules
 * out fp32 at d = 128 (any m) and at d = 64 with m > 32; there
 * nha_bwd_workspace_size returns 0 although nha_check_desc returns NHA_OK,
 * and nha_bwd returns NHA_ERR_UNSUPPORTED.  (bf16 has no such limit; the fp32
 * forward is unsupported only at d = 128 with m > 32.) */
size_t nha_fwd_workspace_size(const nha_desc* desc);
size_t nha_bwd_workspace_size(const nha_desc* desc);

/* Validate a descriptor without touching the GPU. */
nha_status nha_check_desc(const nha_desc* desc);

/* Decode-state bytes for this descriptor (desc->T is ignored).  Layout, in
 * this order, each part starting at a 256-byte aligned offset:
 *   SK   float [B][Hkv][m][d]   long-term key slots
 *   SV   float [B][Hkv][m][d]   long-term value slots
 *   RK   dtype [B][Hkv][w][d]   ring of the last w raw (unrotated) keys;
 *                               position j lives at row j mod w
 *   RV   dtype [B][Hkv][w][d]   ring of the last w values
 *   RKR  dtype [B][Hkv][w][d]   the same keys with RoPE applied at their
 *                               positions (present only when rope_base > 0)
 *   pos  int64 [B][Hkv]         tokens consumed so far (all equal)
 *   part float [B*H][32][d+4]   scratch of one decode step (no meaning
 *                               between calls)
 * A zero-filled state is the state before the first token. */
size_t nha_decode_state_size(const nha_desc* desc);

/* Forward over the whole sequence.
 *   q, k, v, alpha  inputs (device), layouts above; alpha in [0, 1]
 *   o               output (device) [B][T][H][d], desc->dtype
 *   lse             output (device) [B][H][T] float; may be NULL
 *   state_out       may be NULL; else a decode state (nha_decode_state_size
 *                   bytes) that receives the state after token T-1, so that
 *                   nha_decode_step continues the sequence at position T
 *   ws, ws_bytes    device workspace of >= nha_fwd_workspace_size bytes
 *   stream          hipStream_t */
nha_status nha_fwd(const nha_desc* desc, const void* q, const void* k,
                   const void* v, const void* alpha, void* o, float* lse,
                   void* state_out, void* ws, size_t ws_bytes, void* stream);

/* Backward of nha_fwd.
 *   o, lse          the forward's outputs for the same inputs (lse required)
 *   dO              gradient of the loss w.r.t. o, [B][T][H][d]
 *   dq, dk, dv      outputs, desc->dtype, fully overwritten
 *   dalpha          output float [B][T][Hkv][m], fully overwritten;
 *                   dalpha_t = 0 for t < w (no absorption happens there).
 *                   Computed as (E_t - F_t) / alpha_t, so gates that round to
 *                   0 give large relative errors there. */
nha_status nha_bwd(const nha_desc* desc, const void* q, const void* k,
                   const void* v, const void* alpha, const void* o,
                   const float* lse, const void* dO, void* dq, void* dk,
                   void* dv, float* dalpha, void* ws, size_t ws_bytes,
                   void* stream);

/* nha_bwd for a workspace that still holds the forward's intermediates.
 * Precondition: `ws` is the workspace of the nha_fwd call that produced o
 * and lse for these same inputs and descriptor, and nothing has written to
 * it since (ws_bytes must still be >= nha_bwd_workspace_size).  The forward's
 * first stages -- RoPE of q and k, the per-chunk gate products and the slot
 * state at every chunk start -- are then read from the workspace instead of
 * being recomputed; results are bitwise identical to nha_bwd.  Violating the
 * precondition gives wrong gradients without an error. */
nha_status nha_bwd_after_fwd(const nha_desc* desc, const void* q,
                             const void* k, const void* v, const void* alpha,
                             const void* o, const float* lse, const void* dO,
                             void* dq, void* dk, void* dv, float* dalpha,
                             void* ws, size_t ws_bytes, void* stream);

/* One recurrent step at the position stored in the state (per (b, g)).
 *   q_t [B][H][d], k_t, v_t [B][Hkv][d], alpha_t [B][Hkv][m]  (desc->dtype)
 *   state           in/out decode state (see nha_decode_state_size)
 *   o_t             output [B][H][d]
 * At position t it absorbs the token leaving the window (t >= w) with
 * alpha_t, pushes (k_t, v_t), reads m slots + min(w, t+1) window tokens
 * through one softmax, writes o_t and advances the position by one.  The
 * result equals nha_fwd over the concatenated sequence at row t.  Two
 * launches: the keys of each (b, g) are split over several workgroups whose
 * partial softmax results a second launch merges.  m + w > 4096 returns
 * NHA_ERR_UNSUPPORTED. */
nha_status nha_decode_step(const nha_desc* desc, const void* q_t,
                           const void* k_t, const void* v_t,
                           const void* alpha_t, void* state, void* o_t,
                           void* stream);

/* ---------------------------------------------------------------- allocation-free forward
 * For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same result as nha_fwd (bitwise: the same kernels, every launch
 * on `stream`), with the workspace taken from a library-owned scratch array
 * of NHA_NOALLOC_SCRATCH_BYTES bytes that every GPU the library runs on holds
 * from module load until the process ends.  The call itself allocates
 * nothing (no hipMalloc, no stream or event creation); the first call on a
 * device looks the array's address up once (hipGetSymbolAddress).
 *   Arguments as for nha_fwd, without ws / ws_bytes.
 *   Limit: a descriptor whose nha_fwd_workspace_size exceeds
 *   NHA_NOALLOC_SCRATCH_BYTES returns NHA_ERR_WORKSPACE before any HIP call
 *   (e.g. d = 128, m = 64, H = 16, w = 512 fits up to about 2800 tokens of
 *   batch; use nha_fwd with a workspace beyond that).
 *   Every call on one GPU shares that GPU's array: calls that overlap on one
 *   GPU (different streams, or different host threads, without ordering
 *   between them) race and give wrong results.  The array keeps the last
 *   call's contents; nothing in it has to start at zero (each call writes
 *   every region before reading it). */
#define NHA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
nha_status nha_fwd_noalloc(const nha_desc* desc, const void* q, const void* k,
                           const void* v, const void* alpha, void* o,
                           float* lse, void* state_out, void* stream);

/* ---------------------------------------------------------------- initial slot states
 * Learnable initial memory-slot states (the ai.info page, "Future
 * Directions", item 1: parameter-efficient finetuning on slot initial
 * states).  The slots start from S0 instead of zero; as for the zero start a
 * state is only decayed by a step that absorbs a token, so S0 is unchanged
 * until t = w and is scaled by the product of alpha_u (w <= u <= t) after.
 *   s0k, s0v    device, float [B][Hkv][m][d] (S0 of the key and value slots),
 *               16-byte aligned, required (pass zeros for the zero start)
 * nha_fwd_s0: nha_fwd starting from S0 (state_out then holds the state after
 *   token T-1 of this segment, S0 decayed and all absorptions included).
 * nha_bwd_s0: nha_bwd of nha_fwd_s0 (recomputes the forward's prologue with
 *   S0), also writing
 *   ds0k, ds0v  device, float [B][Hkv][m][d]: gradients of the loss w.r.t.
 *               s0k, s0v (per batch row: a state shared over the batch gets
 *               the sum over b), fully overwritten.
 * Errors as for nha_fwd / nha_bwd; a NULL or misaligned s0k, s0v, ds0k or ds0v
 * returns NHA_ERR_INVALID_ARG. */
nha_status nha_fwd_s0(const nha_desc* desc, const void* q, const void* k,
                      const void* v, const void* alpha, const float* s0k,
                      const float* s0v, void* o, float* lse, void* state_out,
                      void* ws, size_t ws_bytes, void* stream);
nha_status nha_bwd_s0(const nha_desc* desc, const void* q, const void* k,
                      const void* v, const void* alpha, const float* s0k,
                      const float* s0v, const void* o, const float* lse,
                      const void* dO, void* dq, void* dk, void* dv,
                      float* dalpha, float* ds0k, float* ds0v, void* ws,
                      size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- chunked prefill
 * A segment of desc->T tokens that continues a decode state -- the state
 * nha_fwd(state_out), nha_decode_step or a previous segment left after pos0
 * tokens: its slot states, its ring of the last w keys and values, and the
 * absorptions those ring tokens still owe (the ai.info page, "Future
 * Directions", item 1: context carried across segments in the slot states).
 * nha_fwd over the whole sequence and nha_fwd_continue over its pieces give
 * the same o and lse up to rounding.
 *   pos0      tokens the state has consumed (its position counter; all
 *             (batch, KV head) units equal).  The library does not read the
 *             counter back: pass the value the state holds.
 *   state_in  device decode state (layout: nha_decode_state_size) -- read
 *             only; its slots SK, SV, ring RK, RV are used (RKR and the
 *             scratch part are not)
 *   state_out nullable; receives the state after the segment (pos0 + T
 *             tokens); may be state_in itself
 *   ws        device workspace of nha_continue_workspace_size bytes (serves
 *             both calls and every pos0; so the size applies the backward's
 *             LDS limit to both: with fp32 it is 0, and the calls return
 *             NHA_ERR_UNSUPPORTED, at d = 128 and at d = 64 with m > 32)
 * nha_bwd_continue: gradients of the segment's loss w.r.t. its inputs (dq,
 *   dk, dv, dalpha as nha_bwd), w.r.t. the state's slots (ds0k, ds0v float
 *   [B][Hkv][m][d]) and, nullable, w.r.t. its ring keys and values (drk, drv
 *   dtype [B][Hkv][w][d] in ring layout; rows holding no token are zero).  o
 *   and lse are the segment's forward outputs; state_in is the state the
 *   forward started from (keep a copy if the forward overwrote it).
 * The token-shift ablation (no_token_shift = 1) returns NHA_ERR_UNSUPPORTED;
 * pos0 < 0 returns NHA_ERR_INVALID_ARG; other errors as nha_fwd / nha_bwd. */
size_t nha_continue_workspace_size(const nha_desc* desc);
nha_status nha_fwd_continue(const nha_desc* desc, long long pos0,
                            const void* state_in, const void* q,
                            const void* k, const void* v, const void* alpha,
                            void* o, float* lse, void* state_out, void* ws,
                            size_t ws_bytes, void* stream);
nha_status nha_bwd_continue(const nha_desc* desc, long long pos0,
                            const void* state_in, const void* q,
                            const void* k, const void* v, const void* alpha,
                            const void* o, const float* lse, const void* dO,
                            void* dq, void* dk, void* dv, float* dalpha,
                            float* ds0k, float* ds0v, void* drk, void* drv,
                            void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- weighted fusion (ablation)
 * The variant the ai.info page's findings compare the method with ("Unified
 * softmax beats weighted fusion": a fixed-coefficient weighted sum, and a
 * learnable sequence-dependent coefficient) -- the separate-then-summed
 * intra-layer fusion of the Paper-Notes page's 现有痛点 paragraph: the m slot
 * logits and the window logits each get their OWN softmax, and per token t
 * and query head h
 *     o_t = lam_t o^slot_t + (1 - lam_t) o^window_t .
 * Slots, token shift, RoPE and gates are exactly as in nha_fwd (no_token_shift
 * applies too).  Needs m >= 1 and w >= 1 (else NHA_ERR_INVALID_ARG).
 *   lam     device float [B][T][H], the coefficient of the slot read (a fixed
 *           coefficient is a constant-filled tensor)
 *   ws      device workspace of nha_weighted_workspace_size bytes, shared by
 *           both calls (0 for an invalid descriptor or m = 0 or w = 0)
 * nha_fwd_weighted writes o [B][T][H][d] (desc->dtype) and, when lse2 is not
 *   NULL, lse2 [2][B][H][T] float: the slot softmax's lse, then the window's.
 * nha_bwd_weighted recomputes both reads and writes dq, dk, dv, dalpha as
 *   nha_bwd does, and dlam [B][T][H] float (= <dO_t, o^slot_t - o^window_t>;
 *   NULL: not wanted, e.g. a fixed coefficient).  Other errors as nha_fwd /
 *   nha_bwd. */
size_t nha_weighted_workspace_size(const nha_desc* desc);
nha_status nha_fwd_weighted(const nha_desc* desc, const void* q, const void* k,
                            const void* v, const void* alpha, const float* lam,
                            void* o, float* lse2, void* ws, size_t ws_bytes,
                            void* stream);
nha_status nha_bwd_weighted(const nha_desc* desc, const void* q, const void* k,
                            const void* v, const void* alpha, const float* lam,
                            const void* dO, void* dq, void* dk, void* dv,
                            float* dalpha, float* dlam, void* ws,
                            size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- timing
 * Kernel launches that one nha_fwd (backward = 0), nha_bwd (backward = 1) or
 * nha_bwd_after_fwd (backward = 2) call enqueues for this descriptor
 * (with_state: nha_fwd with a non-NULL
 * state_out), in launch order.  Up to `max` static names are stored in
 * `names` (nullable).  Returns the number of launches, or -1 for an invalid
 * descriptor. */
int nha_stage_names(const nha_desc* desc, int backward, int with_state,
                    const char** names, int max);

/* nha_fwd / nha_bwd that also record timing events: `events` holds n + 1
 * hipEvent_t handles (passed as void*), n = nha_stage_names(...); events[i]
 * is recorded on `stream` right before launch i and events[n] after the last
 * launch, so hipEventElapsedTime(events[i], events[i+1]) is the duration of
 * launch i.  The events are created and destroyed by the caller.  NULL events
 * behaves exactly like the untimed call. */
nha_status nha_fwd_timed(const nha_desc* desc, const void* q, const void* k,
                         const void* v, const void* alpha, void* o, float* lse,
                         void* state_out, void* ws, size_t ws_bytes,
                         void* stream, void* const* events);
nha_status nha_bwd_timed(const nha_desc* desc, const void* q, const void* k,
                         const void* v, const void* alpha, const void* o,
                         const float* lse, const void* dO, void* dq, void* dk,
                         void* dv, float* dalpha, void* ws, size_t ws_bytes,
                         void* stream, void* const* events);
nha_status nha_bwd_after_fwd_timed(const nha_desc* desc, const void* q,
                                   const void* k, const void* v,
                                   const void* alpha, const void* o,
                                   const float* lse, const void* dO, void* dq,
                                   void* dk, void* dv, float* dalpha, void* ws,
                                   size_t ws_bytes, void* stream,
                                   void* const* events);

/* Destroy the side stream and the three events that nha_fwd, nha_fwd_s0,
 * nha_bwd, nha_bwd_after_fwd and nha_bwd_s0 created for the CALLING thread
 * (on every device it used); the next such call creates them again.  Work
 * already enqueued on them completes normally (HIP releases the handles once
 * it has).  Call it before a thread exits, or after a device reset (the
 * cached handles are then stale).  Other threads' streams are untouched.
 * Returns NHA_OK, or NHA_ERR_HIP if a destroy call failed (the handles are
 * forgotten either way).  With nothing to release it makes no HIP call. */
nha_status nha_release_side_streams(void);

/* Static string for a status code. */
const char* nha_status_string(nha_status s);

#ifdef __cplusplus
}
#endif

#endif /* NHA_H_ */
