/*
 * kda.h -- C ABI of the MI355X (gfx950) gated delta-rule / Kimi Delta
 * Attention library (libkda.so).
 *
 * The operator (one head, state S in R^{dk x dv}, row r = key channel r):
 *
 *   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *   o_t = S_t^T q_t,                      alpha_t = exp(g_t) per key channel.
 *
 * Equivalently, per token: fade the state by the per-channel gate, read the
 * faded state at the key, write beta times the difference to the value, then
 * read the output with the query after the write.  Sources on the pages:
 * dev.to "From GPT-2 to Kimi K3: How Language Models Learned to Manage
 * Memory", blocks 3-5 (read/compare/write; fade first; a retention factor per
 * key channel = per row of S); engineermaxxing "From GPT-2 to Kimi K3: one
 * memory, seven eviction policies", ch. 06b (per-channel decay inside the
 * delta rule) and ch. 05c (scalar gate = Gated DeltaNet; alpha = 1 =
 * DeltaNet); heqinghuang "From GPT2 to Kimi3, Explained", section 09 (output
 * read after the write, no normaliser, missing cache = zero state).
 *
 * Conventions shared by every entry point
 *  - All data pointers are DEVICE pointers (HIP device memory) except the
 *    kda_shape_t argument, which is a host pointer.  The caller owns every
 *    buffer; the library allocates no device memory and keeps no device state.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Every call only enqueues work on `stream` and returns; there is no
 *    implicit synchronisation.  Calls are reentrant: host threads may call
 *    concurrently on different streams.
 *  - Layouts are row-major and packed over tokens: q, k, g [T, H, dk];
 *    v, o [T, H, dv]; beta [T, H]; state pools [num_slots, H, dk, dv].
 *  - q, k, v, o have the I/O dtype (fp32 or bf16); g, beta and states are
 *    always fp32.  g = log(alpha) must be finite and <= 0 (alpha in (0, 1]);
 *    the library does not check values: NaN/Inf propagate, g > 0 is
 *    undefined.  q and k are used as given (callers L2-normalise them).
 *  - Arguments are validated on the host BEFORE any launch: on any error
 *    nothing is enqueued and nothing is written.  Values that live in device
 *    memory (cu_seqlens, slot indices) cannot be checked synchronously; the
 *    kernels never access memory out of bounds because of them: offsets are
 *    clamped to [0, total_tokens] and made nondecreasing, and entries whose
 *    slot lies outside [0, num_slots) are skipped (their outputs are left
 *    unwritten and no state is touched).
 *  - Launch failures return KDA_ERR_HIP; kda_last_error() then holds the HIP
 *    error text.  No C++ exception crosses this interface.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 3

typedef enum {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARGUMENT = 1,  /* bad pointer, shape, count or flag        */
  KDA_ERR_UNSUPPORTED = 2,       /* valid but not built: (dk, dv, chunk, io)  */
  KDA_ERR_WORKSPACE_TOO_SMALL = 3,
  KDA_ERR_HIP = 4                /* a HIP runtime call or launch failed       */
} kda_status_t;

typedef enum { KDA_FP32 = 0, KDA_BF16 = 1 } kda_dtype_t;  /* dtype of q, k, v, o */

typedef struct {
  int32_t num_heads;  /* H  >= 1 */
  int32_t dk;         /* key dimension (rows of S)      */
  int32_t dv;         /* value dimension (columns of S) */
  int32_t io_dtype;   /* kda_dtype_t                    */
} kda_shape_t;

/* flags of kda_chunk_fwd (bit-or); the last three also of kda_decode_step_ex.
 *
 * The variants are the special cases of the same recurrence that the pages
 * name (engineermaxxing ch. 05c: a scalar gate is Gated DeltaNet, alpha = 1 is
 * DeltaNet; heqinghuang section 07 and engineermaxxing ch. 02e-02g: without
 * the delta correction the write is additive, u = v, which is (gated) linear
 * attention).  They change what is read, not the layout of anything else. */
enum {
  KDA_READ_INITIAL_STATE = 1u,  /* start each sequence from states[slot]; else from 0 */
  KDA_WRITE_FINAL_STATE = 2u,   /* store each sequence's final state to states[slot]  */
  KDA_GATE_SCALAR = 4u,         /* g is [tokens, H]: one log-decay per token and head,
                                   the same for every key channel                      */
  KDA_GATE_NONE = 8u,           /* no decay (alpha = 1): g is not read and may be NULL  */
  KDA_ADDITIVE = 16u            /* u = v (no delta correction): beta is not read and
                                   may be NULL                                         */
};

/* Version of this interface (KDA_ABI_VERSION). */
int32_t kda_abi_version(void);

/* Static text for a status code. */
const char* kda_status_string(kda_status_t status);

/* Detail of the last failing call on the calling host thread ("" if none).
 * The pointer stays valid until the next failing call on this thread. */
const char* kda_last_error(void);

/* Whether (dk, dv, chunk, io_dtype) has a built prefill kernel (1) or not (0).
 * Supported: dk = dv in {16, 32, 64} with chunk in {16, 32, 64} for both
 * dtypes (fp32 arithmetic); dk = dv = 128 with chunk in {16, 32} for both
 * dtypes (fp32 arithmetic); dk = dv = 128, chunk = 64, bf16 (bf16 MFMA
 * products, fp32 state and accumulation). */
int32_t kda_chunk_fwd_supported(int32_t dk, int32_t dv, int32_t chunk, int32_t io_dtype);

/* Device workspace bytes that kda_chunk_fwd needs for up to `total_tokens`
 * tokens in up to `num_seqs` sequences (0 if none is needed).  Returns 0 for
 * invalid or unsupported arguments as well; kda_chunk_fwd reports those. */
size_t kda_chunk_fwd_workspace_bytes(const kda_shape_t* shape, int32_t chunk,
                                     int32_t total_tokens, int32_t num_seqs);

/* Chunkwise-parallel prefill over packed variable-length sequences.
 *
 * The result equals the token-by-token recurrence above (up to rounding):
 * the chunked form regroups it into in-chunk products and a triangular solve
 * plus a sequential pass over chunks (engineermaxxing ch. 04b-04f;
 * heqinghuang section 10, with the decay products of section 11).  `chunk`
 * changes cost, not semantics.
 *
 * cu_seqlens  device int32 [num_seqs + 1]; sequence n is tokens
 *             [cu_seqlens[n], cu_seqlens[n+1]); expected cu[0] = 0,
 *             nondecreasing, cu[num_seqs] = total_tokens.  Lengths need not
 *             be multiples of `chunk`; a zero-length sequence is allowed.
 * q, k        device [total_tokens, H, dk], io dtype, 16-byte aligned.
 * v           device [total_tokens, H, dv], io dtype, 16-byte aligned.
 * g           device fp32 [total_tokens, H, dk], log of the per-channel gate
 *             (16-byte aligned); [total_tokens, H] with KDA_GATE_SCALAR;
 *             unused (may be NULL) with KDA_GATE_NONE.
 * beta        device fp32 [total_tokens, H], write strengths; unused (may be
 *             NULL) with KDA_ADDITIVE.
 * states      device fp32 pool [num_slots, H, dk, dv], 16-byte aligned (may be
 *             NULL when neither state flag is set).  Read at the start of sequence n when
 *             KDA_READ_INITIAL_STATE is set, overwritten with its final state
 *             when KDA_WRITE_FINAL_STATE is set.
 * state_slots device int32 [num_seqs] (slot of sequence n), or NULL for slot n
 *             (then num_slots >= num_seqs is required).  Slots must be
 *             distinct within a call.
 * o           device [total_tokens, H, dv], io dtype, fully overwritten;
 *             16-byte aligned (rows are written in 16-byte pieces).
 * workspace   device scratch of at least kda_chunk_fwd_workspace_bytes()
 *             bytes, 256-byte aligned; contents on entry are ignored.
 * flags       KDA_READ_INITIAL_STATE | KDA_WRITE_FINAL_STATE | at most one of
 *             KDA_GATE_SCALAR, KDA_GATE_NONE | KDA_ADDITIVE; other bits, or
 *             both gate bits, are KDA_ERR_INVALID_ARGUMENT.
 * num_seqs == 0 is a no-op returning KDA_OK.  total_tokens == 0 makes every
 * sequence empty: each ends in the state it starts from (zero without an
 * initial state), so KDA_WRITE_FINAL_STATE without KDA_READ_INITIAL_STATE
 * zeroes each sequence's slot, every other flag setting leaves the pool as it
 * is, and nothing else is read or written. */
kda_status_t kda_chunk_fwd(const kda_shape_t* shape, int32_t chunk, int32_t total_tokens,
                           int32_t num_seqs, const int32_t* cu_seqlens, const void* q,
                           const void* k, const void* v, const float* g, const float* beta,
                           float* states, int32_t num_slots, const int32_t* state_slots,
                           uint32_t flags, void* o, void* workspace, size_t workspace_bytes,
                           void* stream);

/* One decode step: one new token per sequence against its resident state.
 *
 * For each b < batch and head h: S = states[slot(b), h] is faded by
 * exp(g[b,h,:]) per key channel, read at k, corrected by beta (v - read),
 * written back IN PLACE, and o[b,h,:] = S_new^T q (the recurrent form for
 * decode: heqinghuang section 10; engineermaxxing ch. 02b and 06b).
 *
 * q, k     device [batch, H, dk], io dtype;  v, o: device [batch, H, dv], io dtype.
 * g        device fp32 [batch, H, dk];       beta: device fp32 [batch, H].
 * states   device fp32 pool [num_slots, H, dk, dv], updated in place.
 * state_slots device int32 [batch] or NULL for slot b (num_slots >= batch).
 *          Slots must be distinct within a call (two tokens of one sequence
 *          are two calls).
 * batch == 0 is a no-op returning KDA_OK.  Supported: dk, dv in
 * {16, 32, 64, 128}, both dtypes. */
kda_status_t kda_decode_step(const kda_shape_t* shape, int32_t batch, const void* q,
                             const void* k, const void* v, const float* g, const float* beta,
                             float* states, int32_t num_slots, const int32_t* state_slots,
                             void* o, void* stream);

/* kda_decode_step for the variants: `flags` is a bit-or of at most one of
 * KDA_GATE_SCALAR (g is [batch, H]) and KDA_GATE_NONE (g unused, may be NULL),
 * and KDA_ADDITIVE (u = v; beta unused, may be NULL); flags == 0 is
 * kda_decode_step.  Other bits, or both gate bits, are
 * KDA_ERR_INVALID_ARGUMENT.  Same arguments, layouts and errors otherwise. */
kda_status_t kda_decode_step_ex(const kda_shape_t* shape, int32_t batch, const void* q,
                                const void* k, const void* v, const float* g,
                                const float* beta, float* states, int32_t num_slots,
                                const int32_t* state_slots, uint32_t flags, void* o,
                                void* stream);

/* Prefill that allocates nothing, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): kda_chunk_fwd with its scratch taken from a device array inside
 * the library instead of a caller workspace.  Every GPU the library runs on
 * holds that array, KDA_NOALLOC_SCRATCH_BYTES bytes, until the process ends; its
 * address is looked up on the first call on each device.
 *
 * Arguments, layouts, flags, results and errors are those of kda_chunk_fwd
 * without workspace / workspace_bytes.  A call that needs more scratch than the
 * array holds (kda_chunk_fwd_workspace_bytes() > KDA_NOALLOC_SCRATCH_BYTES: with
 * d = 128 and chunk 64, a chunk capacity (total_tokens / 64 + num_seqs) times H
 * above about 900) returns KDA_ERR_WORKSPACE_TOO_SMALL before anything is
 * enqueued.  The scratch's contents on entry are ignored, so nothing needs
 * clearing between calls.  All calls on one GPU share its array and it keeps the
 * last call's contents: calls that overlap in time on one GPU (different streams
 * or host threads) race on it, and the caller must order them.  No hipMalloc,
 * hipFree or allocating library routine is called. */
#define KDA_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
kda_status_t kda_chunk_fwd_noalloc(const kda_shape_t* shape, int32_t chunk, int32_t total_tokens,
                                   int32_t num_seqs, const int32_t* cu_seqlens, const void* q,
                                   const void* k, const void* v, const float* g,
                                   const float* beta, float* states, int32_t num_slots,
                                   const int32_t* state_slots, uint32_t flags, void* o,
                                   void* stream);

/* Prefill and decode from the raw projection outputs, with the input
 * preparation fused into the path (heqinghuang section 09: q and k pass through
 * SiLU and are scaled to unit length, beta is a sigmoid; engineermaxxing
 * ch. 06b: the per-channel decay is a sigmoid of its own projection; dev.to
 * block 5: K3 bounds the decay parameterisation for bf16 stability):
 *
 *   q = normalize(silu(q_raw)),  k = normalize(silu(k_raw))   over dk, per (token, head),
 *                                normalize(x) = x / max(|x|_2, 1e-12)
 *   beta = sigmoid(beta_logits)                               per (token, head)
 *   g = log(alpha) = max(log(sigmoid(gate_logits)), gate_min)  per key channel
 *
 * then exactly kda_chunk_fwd / kda_decode_step_ex on (q, k, v, g, beta).
 * Reading bf16 logits instead of fp32 log-decays moves 1,282 instead of 1,540
 * bytes per token and head.
 *
 * q_raw, k_raw  device bf16 [tokens, H, dk];  v: device bf16 [tokens, H, dv]; all
 *               three 16-byte aligned in the prefill (as q, k, v of kda_chunk_fwd).
 * gate_logits   device bf16 [tokens, H, dk] (8-byte aligned); [tokens, H] with
 *               KDA_GATE_SCALAR; unused (may be NULL) with KDA_GATE_NONE.
 * beta_logits   device bf16 [tokens, H]; unused (may be NULL) with KDA_ADDITIVE.
 * gate_min      floor of the log-decay (-INFINITY: none; NaN is an error).
 * Everything else (flags, states, slots, o, workspace, errors) as in
 * kda_chunk_fwd / kda_decode_step_ex.  Supported: io_dtype KDA_BF16; the
 * prefill for dk = dv = 128 with chunk 64 (else KDA_ERR_UNSUPPORTED), the
 * decode for the dims kda_decode_step supports. */
kda_status_t kda_chunk_fwd_raw(const kda_shape_t* shape, int32_t chunk, int32_t total_tokens,
                               int32_t num_seqs, const int32_t* cu_seqlens, const void* q_raw,
                               const void* k_raw, const void* v, const void* gate_logits,
                               const void* beta_logits, float gate_min, float* states,
                               int32_t num_slots, const int32_t* state_slots, uint32_t flags,
                               void* o, void* workspace, size_t workspace_bytes, void* stream);

kda_status_t kda_decode_step_raw(const kda_shape_t* shape, int32_t batch, const void* q_raw,
                                 const void* k_raw, const void* v, const void* gate_logits,
                                 const void* beta_logits, float gate_min, float* states,
                                 int32_t num_slots, const int32_t* state_slots, uint32_t flags,
                                 void* o, void* stream);

/* Device workspace bytes that kda_chunk_bwd needs (0 for invalid or
 * unsupported arguments; kda_chunk_bwd reports those). */
size_t kda_chunk_bwd_workspace_bytes(const kda_shape_t* shape, int32_t chunk,
                                     int32_t total_tokens, int32_t num_seqs);

/* Gradients of a scalar loss through kda_chunk_fwd (training).
 *
 * The chunked form exists for training (engineermaxxing ch. 04; heqinghuang
 * section 10); the pages give no gradient, so this is reverse-mode
 * differentiation of the same chunk algebra: a forward pass over the chunks
 * recomputes the state at every chunk start, a reverse pass carries dL/dS from
 * the last chunk to the first, and every (chunk, head) then forms its
 * gradients in parallel.  Results equal the gradients of the token-by-token
 * recurrence up to rounding.
 *
 * Inputs are those of the forward call (same layouts and variant flags): q, k,
 * v, g, beta, cu_seqlens, and with KDA_READ_INITIAL_STATE the initial
 * states[slot] (else zero).  g must be <= 0 (alpha <= 1), as for the forward.
 * q, k, v, states  16-byte aligned (read in 16-byte pieces).
 * d_o            device io dtype [total_tokens, H, dv]: dL/do (16-byte aligned).
 * d_final_state  device fp32 dense [num_seqs, H, dk, dv]: dL/dS_final, or NULL (0).
 * dq, dk         device io dtype [total_tokens, H, dk] (16-byte aligned);
 * dv             device io dtype [total_tokens, H, dv] (element-aligned);
 * dg             device fp32 [total_tokens, H, dk]; [total_tokens, H] with
 *                KDA_GATE_SCALAR (the gate is shared by the channels, so its gradient
 *                is their sum); not written (may be NULL) with KDA_GATE_NONE.
 * dbeta          device fp32 [total_tokens, H]; not written (may be NULL) with KDA_ADDITIVE.
 *                All written outputs are fully overwritten.
 * d_initial_state  device fp32 dense [num_seqs, H, dk, dv]: dL/dS0, or NULL (not formed).
 * flags          KDA_READ_INITIAL_STATE | at most one of KDA_GATE_SCALAR, KDA_GATE_NONE |
 *                KDA_ADDITIVE; KDA_WRITE_FINAL_STATE and unknown bits are
 *                KDA_ERR_INVALID_ARGUMENT.
 * workspace      device scratch of kda_chunk_bwd_workspace_bytes() bytes, 256-byte
 *                aligned (224.5 KiB per chunk and head of chunk capacity, the capacity
 *                being total_tokens / chunk + num_seqs chunks, plus a small header).
 * Supported: io_dtype KDA_BF16, dk = dv = 128, chunk 64 (else KDA_ERR_UNSUPPORTED).
 * num_seqs == 0 is a no-op returning KDA_OK.  total_tokens == 0 makes every
 * sequence empty, passing its state through unchanged: d_initial_state (when
 * given) is set to d_final_state, or to zero when that is NULL, and nothing
 * else is read or written. */
kda_status_t kda_chunk_bwd(const kda_shape_t* shape, int32_t chunk, int32_t total_tokens,
                           int32_t num_seqs, const int32_t* cu_seqlens, const void* q,
                           const void* k, const void* v, const float* g, const float* beta,
                           const float* states, int32_t num_slots, const int32_t* state_slots,
                           uint32_t flags, const void* d_o, const float* d_final_state, void* dq,
                           void* dk, void* dv, float* dg, float* dbeta, float* d_initial_state,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Gradients through kda_chunk_fwd_raw: the backward from raw projections.
 *
 * The preparation of kda_chunk_fwd_raw (q, k = normalize(SiLU(.)), beta =
 * sigmoid, g = max(log sigmoid, gate_min); heqinghuang section 09,
 * engineermaxxing ch. 06b) is recomputed, kda_chunk_bwd runs on the prepared
 * inputs, and the chain rule of the preparation maps the gradients back:
 * normalize's projection (I - y y^T)/|x| (I/1e-12 below its floor), SiLU's
 * derivative, sigmoid(-a) for the gate logit (0 where the floor is taken; a
 * scalar gate's logit receives the sum over channels) and s(1 - s) for the
 * write-strength logit.
 *
 * Inputs as kda_chunk_fwd_raw (bf16 raw q, k, gate and beta logits; v) plus d_o,
 * d_final_state as for kda_chunk_bwd.  Outputs (device bf16, fully overwritten):
 * dq_raw, dk_raw [tokens, H, dk] (16-byte aligned), dv [tokens, H, dv],
 * dgate_logits shaped like gate_logits (not written with KDA_GATE_NONE),
 * dbeta_logits [tokens, H] (not written with KDA_ADDITIVE); d_initial_state as
 * for kda_chunk_bwd.  workspace: kda_chunk_bwd_raw_workspace_bytes() bytes.
 * Supported: io_dtype KDA_BF16, dk = dv = 128, chunk 64. */
size_t kda_chunk_bwd_raw_workspace_bytes(const kda_shape_t* shape, int32_t chunk,
                                         int32_t total_tokens, int32_t num_seqs);
kda_status_t kda_chunk_bwd_raw(const kda_shape_t* shape, int32_t chunk, int32_t total_tokens,
                               int32_t num_seqs, const int32_t* cu_seqlens, const void* q_raw,
                               const void* k_raw, const void* v, const void* gate_logits,
                               const void* beta_logits, float gate_min, const float* states,
                               int32_t num_slots, const int32_t* state_slots, uint32_t flags,
                               const void* d_o, const float* d_final_state, void* dq_raw,
                               void* dk_raw, void* dv, void* dgate_logits, void* dbeta_logits,
                               float* d_initial_state, void* workspace, size_t workspace_bytes,
                               void* stream);

/* Composition of a segment's effect on its incoming state, for context-parallel
 * prefill of one long sequence split into segments (one per GPU):
 *
 *   S_out[i] = M[i] S_in[i] + B[i]      for i < n and every head,
 *
 * where a segment's M is its state-transition matrix, prod_t (I - beta_t k_t
 * k_t^T) Diag(alpha_t), and B the state it writes from the zero state; each
 * segment is affine in its incoming state because the state is all one chunk
 * passes to the next (heqinghuang section 10; engineermaxxing ch. 04f).  Both
 * come from kda_chunk_fwd on the segment (KDA_WRITE_FINAL_STATE): M with v = 0
 * from the identity (KDA_READ_INITIAL_STATE; needs dk = dv), B from the zero
 * state.  An exclusive scan of the segments' maps with this call gives every
 * segment its incoming state for the final kda_chunk_fwd; across GPUs the maps
 * (dk x dk + dk x dv fp32 per head) are what is exchanged.
 *
 * M     device fp32 dense [n, H, dk, dk];
 * S_in, B, S_out  device fp32 dense [n, H, dk, dv].  S_out may be B (in place)
 *       but must not overlap M or S_in.  fp32 arithmetic.  Supported: dk <= 256. */
kda_status_t kda_state_affine(const kda_shape_t* shape, int32_t n, const float* M,
                              const float* S_in, const float* B, float* S_out, void* stream);

/* The state pool.  Each (slot, head) holds one fp32 dk x dv state: the layer's
 * whole memory of its sequence, which is what the recurrent form carries from
 * one token to the next instead of a growing cache (heqinghuang "From GPT2 to
 * Kimi3, Explained", section 09: the forward pass takes an optional cache and
 * returns the updated state, and no cache means a zero state; engineermaxxing
 * ch. 02g: the decode step returns the state it was given, updated).  These
 * calls start sequences from zero and move states between the pool and dense
 * [n, H, dk, dv] buffers (for example to checkpoint, resume or migrate a
 * sequence).  Every buffer is device fp32, 16-byte aligned; H * dk * dv must be a
 * multiple of 4; bandwidth only, no arithmetic.
 *
 * kda_state_init: zero every state of a pool [num_slots, H, dk, dv]. */
kda_status_t kda_state_init(const kda_shape_t* shape, float* states, int32_t num_slots,
                            void* stream);

/* kda_state_load: copy n dense states src [n, H, dk, dv] into pool slots
 * slots[i] (device int32 [n], or i when slots is NULL, then num_slots >= n).
 * Entries with an out-of-range slot are skipped.  src and the pool must not
 * overlap.  n == 0 is a no-op. */
kda_status_t kda_state_load(const kda_shape_t* shape, float* states, int32_t num_slots,
                            const int32_t* slots, int32_t n, const float* src, void* stream);

/* kda_state_store: copy pool slots slots[i] (or i) into dense dst [n, H, dk, dv].
 * Entries with an out-of-range slot leave their dst rows unwritten.  n == 0 is
 * a no-op. */
kda_status_t kda_state_store(const kda_shape_t* shape, const float* states, int32_t num_slots,
                             const int32_t* slots, int32_t n, float* dst, void* stream);

/* ---------------------------------------------------------------- measurement
 * Per-launch timing of the library's own kernels, for benchmarks and profiles
 * (not part of the computation).  After kda_launch_timer_begin(stream), every
 * kernel launch that the library makes on the calling host thread records a
 * HIP event on `stream` right after itself; begin records the first.  All
 * library calls made before kda_launch_timer_end must use that same stream
 * (events on another stream would not bracket the launches).
 * kda_launch_timer_end waits for the last event and, for the i-th launch
 * (i < min(capacity, launches)), writes its elapsed time in milliseconds (the
 * previous event to its own) to ms[i] and its kernel name, a static string
 * owned by the library, to names[i]; *launches (if not NULL) receives the
 * number of launches recorded, at most KDA_LAUNCH_TIMER_MAX (later launches
 * are not timed).  ms and names are host arrays of `capacity` entries.
 * The timer creates HIP events (host-side runtime objects, no device memory)
 * and synchronises in end, so it must not be used under graph capture.
 * Errors: begin while a timer is active on the thread, end without one, or
 * capacity < 0 / NULL arrays with capacity > 0 -> KDA_ERR_INVALID_ARGUMENT
 * (end always stops the timer); event failures -> KDA_ERR_HIP. */
#define KDA_LAUNCH_TIMER_MAX 16
kda_status_t kda_launch_timer_begin(void* stream);
kda_status_t kda_launch_timer_end(float* ms, const char** names, int32_t capacity,
                                  int32_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
