/*
 * gdn.h — C ABI of libgdn.so, the MI355X (gfx950) library for the Gated DeltaNet (GDN)
 * recurrent decode step.
 *
 * The operation. For each sequence b and head h the library keeps a state S of dv x dk values
 * (rows indexed by the value dimension, columns by the key dimension) and, for each of T new
 * tokens t in order, applies a gated rank-1 delta-rule update and reads the state out:
 *
 *     S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t (scale * q_t)
 *
 * "GDN tuning limits on Kunlun XPU" (buru.work), section 二 (背景), places this update in every
 * linear-attention layer (input projection -> short conv, kernel 4 -> gating -> recurrent update
 * of a 128x128 state per head -> output projection) and describes it as a rank-1 change of the
 * state plus a decay; the equation above is the gated delta rule, the reading used here.
 *
 * Conventions shared by every entry point:
 *  - Buffers. Every tensor is dense, row-major (last index fastest) and lives in device memory
 *    of the current HIP device. The caller owns every buffer; the library keeps no pointer
 *    after a call returns and holds no global state besides a thread-local error string and
 *    the fixed device scratch of gdn_prefill_noalloc.
 *  - Alignment. Every device pointer must be 16-byte aligned.
 *  - Streams. `stream` is a hipStream_t passed as void* (NULL = the null stream). Work is
 *    enqueued asynchronously: no host synchronisation, no allocation, no environment reads.
 *  - Errors. Arguments are validated on the host before anything is enqueued; on any error
 *    nothing is enqueued and no buffer changes. Launch failures return GDN_ERR_HIP with the
 *    HIP error text in gdn_last_error(). A fault inside a kernel surfaces at the caller's next
 *    synchronisation, as HIP reports it. No call aborts or throws across the ABI.
 *  - Empty work. B == 0 or T == 0 is a valid no-op (GDN_OK, nothing enqueued); pointers may
 *    then be NULL.
 *  - Shapes. dk == dv, one of 16, 32, 64, 128 (others return GDN_ERR_UNSUPPORTED);
 *    H >= 1; B * H < 2^31; B * H * 8 * dk < 2^32, i.e. fewer than 4,194,304 heads at dk = 128
 *    (every launch is one dispatch; GDN_ERR_UNSUPPORTED beyond).
 *  - Reentrancy. Calls on different buffers may run concurrently from any threads. Two calls
 *    that update the same state concurrently race.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad size, overlapping output */
    GDN_ERR_UNSUPPORTED = 2,      /* valid but not implemented (head dim, dtype combination) */
    GDN_ERR_OUT_OF_MEMORY = 3,    /* device allocation failed (gdn_state_alloc only) */
    GDN_ERR_HIP = 4               /* a HIP runtime call or kernel launch failed */
} gdn_status;

typedef enum {
    GDN_F32 = 0,  /* IEEE binary32 */
    GDN_BF16 = 1, /* bfloat16; every bf16 store rounds to nearest even */
    GDN_F16 = 2   /* IEEE binary16; every fp16 store rounds to nearest even (the reduced-
                     precision mode of "GDN tuning limits on Kunlun XPU", section 三.2) */
} gdn_dtype;

/*
 * gdn_state_alloc — allocate a zero-filled recurrent state of B sequences x H heads x dv x dk
 * elements of `state_dtype` on the current device (the per-head state of the section 二
 * chain). Synchronous. On success *state_out is a 256-byte aligned device pointer owned by the
 * caller (release it with gdn_state_free) and *bytes_out (if not NULL) its size in bytes.
 * Any dense device buffer of the same shape and dtype, e.g. a torch tensor, is an equally valid
 * state for the step functions.
 * Errors: GDN_ERR_INVALID_ARGUMENT (B < 1, H < 1, state_out NULL, bad dtype),
 *         GDN_ERR_UNSUPPORTED (dk != dv or not in {16,32,64,128}),
 *         GDN_ERR_OUT_OF_MEMORY (hipMalloc failed), GDN_ERR_HIP (other HIP failure).
 */
gdn_status gdn_state_alloc(int64_t B, int32_t H, int32_t dk, int32_t dv, gdn_dtype state_dtype,
                           void** state_out, size_t* bytes_out);

/* gdn_state_free — release a state from gdn_state_alloc (NULL is a no-op). Synchronous. */
gdn_status gdn_state_free(void* state);

/*
 * gdn_decode_step — one layer's recurrent step for T sequential tokens of every (b, h); the
 * operation above ("GDN tuning limits on Kunlun XPU", section 二: the recurrent update that
 * follows gating). Inputs arrive ready-made: q and k already L2-normalised, alpha and beta
 * already mapped to gate values.
 *
 *   q, k   act_dtype [B][T][H][dk]   read only (may alias each other)
 *   v      act_dtype [B][T][H][dv]   read only
 *   alpha  fp32      [B][T][H]       decay, one scalar per (b, t, h)
 *   beta   fp32      [B][T][H]       write strength, one scalar per (b, t, h)
 *   state  state_dtype [B][H][dv][dk]  read and updated IN PLACE: S_{t0-1} in, S_{t0+T-1} out
 *   o      act_dtype [B][T][H][dv]   written: o_t for every token; must not overlap any other
 *                                    argument (checked by address range)
 *   scale  multiplies q in the readout (1.0f = the plain definition)
 *
 * Arithmetic is fp32 (bf16 and fp16 inputs widen exactly); a 16-bit state is widened on load,
 * kept in fp32 across the T tokens of the call and rounded once when stored. With a bf16 state,
 * bf16 activations and 3 <= T <= 8 the call takes the chunk form of the same recurrence
 * (products with the loaded state, state updated once; section 三.3 of the same page names the
 * form): the same result up to the order of rounding. An fp16 state or
 * output saturates to infinity beyond 65504; keeping values in range is the caller's choice
 * of that dtype.
 * Errors: GDN_ERR_INVALID_ARGUMENT, GDN_ERR_UNSUPPORTED, GDN_ERR_HIP (see conventions).
 */
gdn_status gdn_decode_step(int64_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                           const void* q, const void* k, const void* v, gdn_dtype act_dtype,
                           const float* alpha, const float* beta,
                           void* state, gdn_dtype state_dtype,
                           void* o, float scale, void* stream);

/*
 * gdn_decode_verify — speculative / multi-token-prediction verify with a deferred commit of the
 * accepted prefix (for decoding that checks T drafted tokens in one pass and keeps only a
 * prefix of them; "GDN tuning limits on Kunlun XPU", sections 三.2 and 四, run GDN under MTP).
 * The pages do not define how the recurrent state drops rejected tokens; this is the reading:
 *
 *   1. `state` holds the committed state as of the start of the previous verify call. That call
 *      had Tp tokens; n_prev[b] (clamped to [0, Tp]) of them were accepted for sequence b. They
 *      are committed by replaying their updates, S <- alpha_t S + dk_t k_t^T for t < n_prev[b],
 *      from the previous call's keys, decays and emitted write coefficients; the result is
 *      stored in `state` (left untouched where the prefix is empty).
 *   2. The T new tokens run from that committed state as stored (rounded to state_dtype: the
 *      state the next call loads and replays their coefficients onto), as in gdn_decode_step,
 *      writing o for every token and their write coefficients dk_out
 *      (dk_t = beta_t (v_t - alpha_t S k_t), so that S_t = alpha_t S_{t-1} + dk_t k_t^T); the
 *      state after them is NOT stored.
 *
 * A first call passes Tp = 0; a final call that only commits passes T = 0. The caller keeps
 * each call's k, alpha and dk_out for the next call. One state read and at most one state
 * write per call, as for gdn_decode_step.
 *
 *   q, k, v, alpha, beta, o, scale  as gdn_decode_step, for the T new tokens
 *   state       state_dtype [B][H][dv][dk], read; written with the committed state
 *   Tp          tokens of the previous call (>= 0)
 *   n_prev      int32 [B], device; accepted prefix length per sequence (clamped to [0, Tp])
 *   k_prev      act_dtype [B][Tp][H][dk], the previous call's k
 *   alpha_prev  fp32 [B][Tp][H], the previous call's alpha
 *   dk_prev     fp32 [B][Tp][H][dv], the previous call's dk_out
 *   dk_out      fp32 [B][T][H][dv], written; must not overlap any other argument (nor o)
 * Pointers of an empty part (T == 0, or Tp == 0) may be NULL.
 * Errors: as gdn_decode_step.
 */
gdn_status gdn_decode_verify(int64_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                             const void* q, const void* k, const void* v, gdn_dtype act_dtype,
                             const float* alpha, const float* beta,
                             void* state, gdn_dtype state_dtype,
                             int32_t Tp, const int32_t* n_prev, const void* k_prev,
                             const float* alpha_prev, const float* dk_prev,
                             void* o, float* dk_out, float scale, void* stream);

/*
 * gdn_conv_gate_decode — the fused layer path of the same chain ("GDN tuning limits on Kunlun
 * XPU", section 二: short causal conv of kernel size 4, then gating, then the recurrent
 * update), for T sequential tokens:
 *   1. causal depthwise conv1d per channel c over (conv_state[c][0..2], x_0[c], x_1[c], ...):
 *        y_t[c] = sum_{i=0..3} conv_w[c][i] * u[t+i]  (+ conv_b[c]);  tap 3 = current input;
 *   2. SiLU on every channel, y * sigma(y);
 *   3. split into q, k, v; q and k scaled to unit length: x / sqrt(sum x^2 + l2_eps);
 *   4. beta = sigma(b_logit), alpha = exp(-softplus(a_logit));
 *   5. the recurrent step of gdn_decode_step on those values.
 *
 *   qkv        bf16 [B][T][C], C = H*dk + H*dk + H*dv, channel blocks ordered q | k | v, each
 *              block head-major with the head dimension fastest. Read only.
 *   conv_state bf16 [B][C][3], the last three raw inputs per channel, oldest first; updated IN
 *              PLACE to the last three inputs after token T-1 (a byte-exact move of inputs).
 *   conv_w     fp32 [C][4];  conv_b  fp32 [C] or NULL (no bias)
 *   a_logit, b_logit  fp32 [B][T][H]
 *   state      state_dtype [B][H][dv][dk], updated IN PLACE
 *   o          bf16 [B][T][H][dv], written; must not overlap any other argument
 * Errors: as gdn_decode_step; conv_state must not overlap state, qkv or o.
 */
gdn_status gdn_conv_gate_decode(int64_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                                const void* qkv, void* conv_state,
                                const float* conv_w, const float* conv_b,
                                const float* a_logit, const float* b_logit,
                                void* state, gdn_dtype state_dtype,
                                void* o, float scale, float l2_eps, void* stream);

/*
 * gdn_prefill_workspace_size — bytes of device workspace gdn_prefill needs for these sizes:
 * B * H * ceil(T / 16) * 2176 (one record per head and chunk of 16 tokens); 0 when B or T is 0.
 * Errors: GDN_ERR_INVALID_ARGUMENT (bytes NULL, bad size), GDN_ERR_UNSUPPORTED (head dims).
 */
gdn_status gdn_prefill_workspace_size(int64_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                                      size_t* bytes);

/*
 * gdn_prefill — the recurrent step of gdn_decode_step for a long run of T tokens (a prompt),
 * computed in the chunked form that "GDN tuning limits on Kunlun XPU", section 三.3, uses for
 * prefill: tokens are taken 16 at a time and the state is touched by dense products on the
 * matrix cores instead of one rank-1 update per token. The result is that of gdn_decode_step
 * on the same arguments up to fp32 rounding order (the state after the last token, and o for
 * every token); both read the state once and write it once. One difference for non-finite
 * inputs: a NaN or infinity in a token's k, q or v can also make the outputs of the earlier
 * tokens of its 16-token chunk non-finite (other heads, sequences and chunks are unaffected).
 *
 *   q, k, v, alpha, beta, state, o, scale, act_dtype, state_dtype  as gdn_decode_step
 *   workspace        device buffer of at least gdn_prefill_workspace_size(...) bytes, owned
 *                    by the caller; its contents on entry do not matter and on return are
 *                    unspecified. It must not overlap any other argument. Two calls in flight
 *                    at once need two workspaces.
 *   workspace_bytes  its size in bytes
 * Errors: as gdn_decode_step; GDN_ERR_INVALID_ARGUMENT also for a workspace smaller than
 * required; GDN_ERR_UNSUPPORTED when B * H * ceil(T / 16) * 64 >= 2^32 (the prep kernel's
 * single dispatch). Runs of fewer than 16 tokens take gdn_decode_step's kernel instead (the
 * same recurrence, faster there; the workspace is then not touched, and the non-finite caveat
 * above does not apply).
 */
gdn_status gdn_prefill(int64_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                       const void* q, const void* k, const void* v, gdn_dtype act_dtype,
                       const float* alpha, const float* beta,
                       void* state, gdn_dtype state_dtype,
                       void* o, float scale, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * gdn_prefill_noalloc — gdn_prefill for callers that cannot allocate or pass device memory of
 * their own: code being captured into a HIP graph, tight serving loops, and harnesses that
 * forbid allocation. Same arguments, results and errors as gdn_prefill, minus the workspace:
 * the chunk records go to a fixed scratch array that the library holds in device memory, 64 MiB
 * per GPU it runs on, for the life of the process. The call allocates nothing and calls no
 * allocating routine; the first call on each device looks the array's address up (make that
 * first call outside graph capture).
 * Limit: B * H * ceil(T / 16) * 2176 <= 67,108,864 bytes (30,840 head-chunks, e.g. one 48-head
 * sequence of up to 10,280 tokens); larger calls return GDN_ERR_UNSUPPORTED and enqueue
 * nothing (use gdn_prefill with a workspace). Every call on one GPU shares that GPU's array:
 * calls on one stream are ordered and safe; two calls in flight at once on one GPU (different
 * streams) race on it. The array's contents on entry do not matter (the prep kernel writes
 * every record the state kernel reads).
 */
gdn_status gdn_prefill_noalloc(int64_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                               const void* q, const void* k, const void* v, gdn_dtype act_dtype,
                               const float* alpha, const float* beta,
                               void* state, gdn_dtype state_dtype,
                               void* o, float scale, void* stream);

/*
 * gdn_lowrank_decode_step — T tokens of the recurrence on a sliding-window low-rank state, the
 * low-rank route of "GDN tuning limits on Kunlun XPU", section 三.3 (r = 16 or 32 there). That
 * page states that this state caches the most recent r rank-1 updates and is not a
 * factorisation of the full state; it prints no equations. Reading implemented: the state a
 * head stands for is the sum of the last r writes of the gated delta rule above, each decayed
 * by every gate since it was written, and each write is the full rule's write against that
 * windowed state. With r >= the tokens seen since an empty start this is exactly
 * gdn_decode_step; afterwards the oldest write leaves the window whole.
 *
 * Storage per (b, h): r slots; slot i holds a write vector U_i, its key K_i and a weight c_i,
 * and the state is S = sum_i c_i U_i K_i^T; pos is the slot the next token writes (the oldest
 * write once the window is full). Per token:
 *     delta = beta (v - alpha S k);  every c_i *= alpha;  slot pos <- (delta, k, 1);
 *     pos <- (pos + 1) mod r;        o = S_new (scale q)
 * An all-zero window (U, K, c and pos zero) is the empty state of a new sequence.
 *
 *   q, k, v, alpha, beta, o, act_dtype, scale   as gdn_decode_step
 *   r      window length: 8, 16 or 32 (GDN_ERR_UNSUPPORTED otherwise)
 *   U      state_dtype [B][H][r][dv]  write vectors, updated IN PLACE
 *   K      state_dtype [B][H][r][dk]  keys, updated IN PLACE (k rounded to state_dtype)
 *   c      fp32 [B][H][r]             weights, updated IN PLACE
 *   pos    int32 [B][H]               next slot, read modulo r as an unsigned value and
 *                                     written back as (pos + T) mod r
 * Within one call U, K and c stay fp32 in registers; only the slots the call wrote (one per
 * token, all r once T >= r), every weight and pos are stored. Stores to a 16-bit state round to
 * nearest even once per call. Non-finite inputs stay within their own (b, h); where a call on
 * a bf16 window (bf16 activations, D = 128, T >= 8 with T mod 8 in {0, 6, 7}) takes its tokens
 * in rounds of 8 in matrix form, a NaN or infinity in a token's k, q or v can also reach the
 * earlier outputs of its own round.
 * Errors: as gdn_decode_step; U, K, c and pos must not overlap each other or the inputs, and o
 * must not overlap any argument (GDN_ERR_INVALID_ARGUMENT).
 */
gdn_status gdn_lowrank_decode_step(int64_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                                   int32_t r, const void* q, const void* k, const void* v,
                                   gdn_dtype act_dtype, const float* alpha, const float* beta,
                                   void* U, void* K, gdn_dtype state_dtype, float* c,
                                   int32_t* pos, void* o, float scale, void* stream);

/* gdn_status_string — static name of a status code ("GDN_OK", ...; "unknown" otherwise). */
const char* gdn_status_string(gdn_status s);

/* gdn_last_error — detail of the calling thread's most recent failed call ("" if none).
 * The pointer stays valid until the thread's next library call. */
const char* gdn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
