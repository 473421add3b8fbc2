/*
 * gdn_beam.h — large-beam Gated DeltaNet decoding on one AMD Instinct MI355X (gfx950).
 *
 * One shared prefill state S_ctx per (request, head); every beam is a chain of
 * append-only GDN Transition Records r = (alpha, delta, k) in fixed slots, found
 * through an Ancestry Index.  No per-beam d_v x d_k state is ever built.
 *
 * Sources (the pages this follows):
 *   OneLA reading note (paper-archivist.com, "OneLA: Scaling Linear-Attention
 *   Decoding to Large Beams in Generative Recommendation"):
 *     section 1.2 eq. (3)   GDN recurrence and output o_t = S_t q_t
 *     section 2.1           logical / physical / index layers (S_ctx, GTR slots, ancestry)
 *     section 2.2 eq. (4-5) rank-1 form and the transition record r_t = (alpha_t, delta_t, k_t)
 *     section 2.3 eq. (6-8) projection replay along the ancestor chain, then delta_t and o_t
 *     section 2.4 eq. (9)   ancestry-index update h_t(b, j)
 *     section 2.5           fused shared-context kernel (S_ctx loaded once, reused across beams)
 *     section 1.1 eq. (1)   SID probability as a product of per-step conditionals
 *   RecoGEM (conceptio mirror, "RecoGEM: A Serving System for Production-Scale
 *   Generative Recommendation"), section 4.3: exact global top-K over a request's
 *   W x C candidates.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked "host".  Every device pointer must
 *     be 16-byte aligned.  Arrays are dense, row-major, last index fastest.
 *   - Calls are asynchronous on `stream` and never synchronise the host.
 *   - The library never allocates device memory: the caller owns the workspace.
 *   - Every check runs on the host before any launch; a rejected call changes no
 *     state and launches nothing.  Nothing aborts or prints.
 *   - One context serves one stream at a time; separate contexts are independent.
 *     Calls on one context must be issued in order: init, then for t = 0, 1, ...:
 *     step(t) then select(t).
 */
#ifndef GDN_BEAM_H
#define GDN_BEAM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN_OK = 0,
  GDN_ERR_INVALID_ARG = 1,  /* null or misaligned pointer, bad size or dtype */
  GDN_ERR_BAD_STATE = 2,    /* call out of order (e.g. select before step, wrong t) */
  GDN_ERR_CAPACITY = 3,     /* t >= T_max, W > W_max, V > V_max */
  GDN_ERR_WORKSPACE = 4,    /* workspace smaller than gdn_beam_workspace_bytes() */
  GDN_ERR_UNSUPPORTED = 5,  /* head dims or dtypes without a compiled kernel */
  GDN_ERR_HIP = 6           /* a HIP launch or copy failed; see gdn_beam_last_error() */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

typedef struct {
  int32_t R, H;        /* requests, GDN value heads per request                           */
  int32_t d_k, d_v;    /* head dims; supported (d_k, d_v): (16,16), (128,128), (128,256), */
                       /* (128,512), and with bf16 io (256,256), (256,512); d_v = 512   */
                       /* needs a bf16 codebook                                          */
  int32_t T_max;       /* SID decode steps (1..8)                                         */
  int32_t W_max;       /* peak beam width = GTR slots per step (1..1024)                  */
  int32_t V_max;       /* largest codebook passed to select (1..65536)                    */
  gdn_dtype io_dtype;  /* dtype of q, k, v; keys are stored in the GTR pool in it         */
  gdn_dtype wout_dtype;/* dtype of the codebook projection Wout                           */
  int32_t H_K;         /* key heads (0: H).  Grouped value heads: H = g * H_K, value head */
                       /* h uses q, k of key head h / g; S_ctx, v, gates, o and the      */
                       /* records' delta are per value head, q, k and keys per key head  */
} gdn_beam_config;

typedef struct gdn_beam_ctx gdn_beam_ctx;   /* opaque, host memory owned by the library */

/* Size in bytes of the workspace a context needs (host only, no GPU call).
 * Per request it is H*(4*d_v*d_k + T_max*W_max*(4 + 4*d_v + e*d_k)) plus
 * O(W_max*(T_max + d_v + V_max/32)) for ancestry, scores and selection scratch
 * (e = bytes per io element; the selection keeps one value per 32 codes of a
 * beam, never a W x V score matrix).  No term grows with d_v*d_k*W: this is the
 * persistent-capacity form of the OneLA reading note, section 2.2 (eq. 5) and
 * section 4.3 (b), against W*d_v*d_k for one state per beam. */
gdn_status gdn_beam_workspace_bytes(const gdn_beam_config* cfg, size_t* bytes /* host */);

/* Start a decode.  S_ctx [R,H,d_v,d_k] fp32 is the shared prefill state of each
 * (request, head) (section 2.1, logical layer); it is read only by the launch this
 * call makes and may be freed once `stream` has passed it.  W0 beams start at
 * t = 0, all children of S_ctx with cumulative score 0.  `workspace` (device,
 * >= gdn_beam_workspace_bytes, 256-byte aligned) must outlive the context.
 * On success *out (host) receives a new context. */
gdn_status gdn_beam_init(const gdn_beam_config* cfg, const float* S_ctx, int32_t W0,
                         void* workspace, size_t workspace_bytes, hipStream_t stream,
                         gdn_beam_ctx** out /* host */);

/* One SID step t for all R*H*W_t beams (W_t = beams alive at step t).
 * Inputs: q, k [R,H_K,W_t,d_k] and v [R,H,W_t,d_v] in io_dtype; alpha, beta
 * [R,H,W_t] fp32.  For each beam: u_q = S_ctx q_t and u_k = S_ctx k_t, replayed
 * along the beam's ancestor records by eqs. (6)-(7); then eq. (8):
 * delta_t = beta (v - alpha u_k), o_t = alpha u_q + delta_t (k_t . q_t).
 * Output: o [R,H,W_t,d_v] fp32.  The record (alpha_t, delta_t, k_t) is written
 * once into slot (t, b) of the GTR pool (section 2.2 eq. 5, section 2.5 step 3).
 * Valid after init (t = 0) or after select(t-1).  Re-issuing step(t) before
 * select(t) rewrites the same slots with the same values. */
gdn_status gdn_beam_step(gdn_beam_ctx* ctx, int32_t t,
                         const void* q, const void* k, const void* v,
                         const float* alpha, const float* beta,
                         float* o, hipStream_t stream);

/* Score step t's beams and choose the W_next beams of step t+1.
 * o [R,H,W_t,d_v] fp32 is the output of step(t).  Wout [d_v,V] in wout_dtype is
 * the codebook projection shared by all heads.  Per request: z_b = sum_h o_b,
 * logit_bc = z_b . Wout[:,c], and candidate (b, c) scores
 * cum_b + (logit_bc - logsumexp_c logit_b)  (log form of eq. 1).
 * Logits are computed with fp32 precision: z (fp32) enters the matrix cores as three bf16
 * terms against a bf16 codebook, or, for selections of at least 2^33 multiply-adds
 * (R*W_t*V*d_v; the environment variable GDN_BEAM_F16_MIN_MACS, read per call, changes
 * the threshold), as two fp16 terms against the codebook rescaled exactly into fp16 tile
 * by tile, where every 32-code tile's nonzero entries span at most 32 binades.
 * The environment variable GDN_BEAM_LOGITS_GPB (1..8, read per call) sets how many code
 * groups one logits block takes in turn; results do not depend on it (for tests).
 * The exact top-W_next over the request's W_t*V candidates, ordered by score
 * descending then flat index b*V + c ascending, is written to parent, token
 * [R,W_next] int32 and score [R,W_next] fp32 (RecoGEM section 4.3).
 * If forced_parent and forced_token [R,W_next] int32 are both non-NULL, the
 * beams follow them instead and carry the score of the forced candidate; the
 * top-W is still computed into parent/token/score.  Forced entries out of range
 * are clamped and flagged in the status word (gdn_beam_export GDN_EXPORT_STATUS).
 * Then the ancestry is remapped by eq. (9) (section 2.4): only indices move,
 * never records.  A NaN score ranks below every number (a NaN in o_t makes every
 * score of that beam NaN).  Requires W_next <= W_max, V <= V_max, W_next <= W_t*V. */
gdn_status gdn_beam_select(gdn_beam_ctx* ctx, int32_t t, const float* o,
                           const void* Wout, int32_t V, int32_t W_next,
                           const int32_t* forced_parent, const int32_t* forced_token,
                           int32_t* parent, int32_t* token, float* score,
                           hipStream_t stream);

/* Size of the static selection scratch gdn_beam_select_static uses, per GPU. */
#define GDN_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

/* For callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments, results, errors and
 * state machine as gdn_beam_select, and the same kernels; only the selection's per-call
 * scratch (head sums, operand fragments, transposed codebook, tile maxima, candidate
 * lists, refined keys) lives in a static device array of GDN_STATIC_SCRATCH_BYTES
 * instead of the context's workspace (the beam state, ancestry and status stay there).
 * The call allocates nothing.  Each GPU the library runs on holds its own copy of the
 * array from this call's first use on it until the process ends; the device of
 * `stream` must be the current device.  The scratch a configuration needs grows as
 * R * W_max * (V_max / 8 + 6 d_v + ...) bytes (about 10 MiB for R = 32, W_max = 256,
 * V_max = 1024, d_v = 128); a context that needs more than the array is refused with
 * GDN_ERR_CAPACITY before any other check, and gdn_beam_last_error() states the size
 * needed.  Every call on one GPU shares that GPU's array and leaves its contents
 * there: calls that overlap on one GPU (other streams, other threads, other contexts)
 * race and must be serialised by the caller.  Nothing in the array needs to start at
 * zero: every call writes what it reads. */
gdn_status gdn_beam_select_static(gdn_beam_ctx* ctx, int32_t t, const float* o,
                                  const void* Wout, int32_t V, int32_t W_next,
                                  const int32_t* forced_parent, const int32_t* forced_token,
                                  int32_t* parent, int32_t* token, float* score,
                                  hipStream_t stream);

/* Bytes of the state buffer gdn_fullstate_step needs (host only):
 * 2 * R*H*W_max*d_v*d_k*4, two generations of one fp32 d_v x d_k state per
 * (request, head, beam). */
gdn_status gdn_fullstate_bytes(const gdn_beam_config* cfg, size_t* bytes /* host */);

/* The FullState baseline of the OneLA reading note (section 1.3, Fig. 2; eq. 4 of
 * section 2.2): every beam carries its own state, copied on reorder.  Same inputs,
 * output and state machine as gdn_beam_step, in its place (select(t) follows):
 * beam b reads its parent's state P (S_ctx at t = 0, else the state this call wrote
 * at step t-1 for slot pi_t(b), from the ancestry the selection left), and writes
 * S_{t,b} = alpha P + delta k^T with delta = beta (v - alpha P k), and
 * o = S_{t,b} q [R,H,W_t,d_v] fp32.  It writes no transition records, so a decode
 * uses either this call or gdn_beam_step for all its steps (mixing them is
 * GDN_ERR_BAD_STATE).
 * states: device, >= gdn_fullstate_bytes, 16-byte aligned, owned by the caller, the
 * same buffer for every step of the decode (steps alternate its two halves).
 * S_ctx [R,H,d_v,d_k] fp32 (device) is read at t = 0 only (may be NULL later).
 * Errors as gdn_beam_step; a short buffer is GDN_ERR_WORKSPACE. */
gdn_status gdn_fullstate_step(gdn_beam_ctx* ctx, int32_t t, const float* S_ctx,
                              const void* q, const void* k, const void* v,
                              const float* alpha, const float* beta, float* o,
                              void* states, size_t states_bytes, hipStream_t stream);

/* Copy internal state to a caller buffer (device) for tests and debugging. */
typedef enum {
  GDN_EXPORT_ANCESTRY = 0,  /* [R,W_max,T_max] int32: h_t(b,j) of the coming step        */
  GDN_EXPORT_TOKENS = 1,    /* [R,W_max,T_max] int32: SID prefix of each live beam       */
  GDN_EXPORT_CUM = 2,       /* [R,W_max] fp32: cumulative score of each live beam        */
  GDN_EXPORT_GTR_ALPHA = 3, /* [R,H,T_max,W_max] fp32                                    */
  GDN_EXPORT_GTR_DELTA = 4, /* [R,H,T_max,W_max,d_v] fp32                                */
  GDN_EXPORT_GTR_KEY = 5,   /* [R,H_K,T_max,W_max,d_k] io_dtype                          */
  GDN_EXPORT_STATUS = 6     /* [1] int32, bits set by select since init:                 */
                            /*   bit 0 (1): a forced parent/token was out of range       */
                            /*   (clamped);  bit 1 (2): a selection found fewer than     */
                            /*   W_next candidates (possible only with NaN outputs);     */
                            /*   the missing ranks are filled with beam 0, token 0;      */
                            /*   bit 2 (4): a selection in the two-term fp16 form fell   */
                            /*   back to three bf16 terms, a code tile's exponents       */
                            /*   spanning more than fp16 can hold                        */
} gdn_export_what;
gdn_status gdn_beam_export(const gdn_beam_ctx* ctx, int32_t what, void* dst,
                           size_t dst_bytes, hipStream_t stream);

/* Bytes gdn_beam_export writes for `what` (host only). */
gdn_status gdn_beam_export_bytes(const gdn_beam_ctx* ctx, int32_t what, size_t* bytes /* host */);

/* Beams alive at the coming step and the step index expected next (host only). */
gdn_status gdn_beam_query(const gdn_beam_ctx* ctx, int32_t* t_next, int32_t* W_cur /* host */);

/* Free a context (host memory only; the workspace stays the caller's). NULL is a no-op. */
void gdn_beam_destroy(gdn_beam_ctx* ctx);

/* Measurement, not an operation of the method: kernel time of the step launches as
 * they run in a stream of decodes.  gdn_beam_time_steps(capacity) creates 2 * capacity
 * HIP events on the current device (host call, no device memory) and makes each of
 * the next `capacity` gdn_beam_step / gdn_fullstate_step launches of the process, on
 * that device and whatever their context, record its own start and end on a pair of
 * them: the dispatch stamps them itself, so nothing is added to the stream between
 * launches.  capacity = 0 releases the events; calling it again restarts the count.
 * Errors: capacity outside 0..65536 (INVALID_ARG), event creation failing (HIP). */
gdn_status gdn_beam_time_steps(int32_t capacity);

/* Waits for the timed launches recorded since the last call and writes the first
 * min(recorded, cap) durations in milliseconds, in launch order, to ms (host); *n
 * (host) receives the number recorded.  The count then starts over (the events are
 * reused for the next launches). */
gdn_status gdn_beam_step_times(float* ms /* host */, int32_t cap, int32_t* n /* host */);

/* Measurement, not an operation of the method: MFMA activity of the S_ctx projection
 * inside the fused step (OneLA reading note, section 2.5 step 2: the accumulators start as
 * S_ctx q_t and S_ctx k_t).  Arms the next gdn_beam_step launch of the process to write
 * one 32-byte record per (workgroup, wave, 32-beam chunk) into buf (device, 16-byte
 * aligned, caller-owned, `bytes` long; records past it are dropped), then disarms.  Record
 * ((wid * NW) + wave) * ceil(W_t / 32) + chunk, wid the work item (request * H + head,
 * times the row blocks of a head: one per 256 rows of d_v), NW = min(d_v, 256) / 32 waves;
 * words (uint32): shader-clock cycle (s_memtime) before the chunk's first projection MFMA,
 * lo and hi; the cycle after a VALU operation read its last results, lo and hi; HW_ID;
 * XCC_ID; MFMA flops of the phase; the bits of the value read.  With stamps on, that
 * launch waits for the projection before the chunk's dot products; its outputs are
 * unchanged.  buf = NULL disarms.  Errors: misaligned buf or bytes < 32 (INVALID_ARG). */
gdn_status gdn_beam_stamp_projection(void* buf, size_t bytes);

/* Measurement, not an operation of the method: the device's streaming rate, the
 * reference against which HBM-bound launches are read.  mode 0 copies `bytes` from src
 * to dst; mode 1 reads src and writes at most one 4-byte word at dst; mode 2 only
 * writes dst (src unused, may be NULL), as 512-byte rows in the fused step's store
 * pattern (each row in four 128-byte pieces from four waves, eight rows per store;
 * floor(bytes / 16384) groups of 32 rows).  Pointers are device, caller-owned, 16-byte
 * aligned, bytes a multiple of 16 (not overlapping for mode 0); 16-byte accesses
 * (non-temporal for modes 0 and 1), four 256-thread workgroups per compute unit,
 * grid-strided, on `stream`.  Errors: null or misaligned pointers, bytes not a multiple
 * of 16, mode outside 0..2 (INVALID_ARG); a launch failure (HIP). */
gdn_status gdn_beam_stream_probe(void* dst, const void* src, size_t bytes, int32_t mode,
                                 hipStream_t stream);

/* Static description of a status code. */
const char* gdn_beam_status_str(gdn_status s);

/* Text of the last GDN_ERR_HIP on the calling thread, or of a static-scratch capacity
 * refusal of gdn_beam_select_static ("" if none). */
const char* gdn_beam_last_error(void);

/* Prefill (eq. 3, section 1.2): S_out[r,h] = the state after request r's prompt,
 * starting from zero.  Prompt tokens of all requests are stacked:
 * k [N,H_K,d_k] (H_K = 0: H), v [N,H,d_v], alpha, beta [N,H] fp32, request r owning rows
 * offsets[r] .. offsets[r+1]-1, with offsets [R+1] int32 (device), nondecreasing,
 * offsets[R] = N.  Offsets are clamped to [0, N] on the device (decreasing offsets give
 * unspecified states, never an access outside the arrays).  S_out [R,H,d_v,d_k] fp32.
 * Same head dims as the decode.
 *
 * workspace = NULL: eq. (3) token by token in fp32 (no scratch memory).
 * workspace != NULL (256-byte aligned, workspace_bytes >= gdn_beam_prefill_workspace_bytes):
 * the chunked form of eq. (3) (32-token chunks; within a chunk the update vectors solve a
 * unit lower-triangular system, whose inverse a first kernel forms for every chunk in
 * parallel; a second kernel applies the chunks of each (request, head) in order as matrix
 * products on MFMA, operands split into bf16 hi + lo parts, fp32 accumulation).  Chunks are
 * 32-token blocks of the stacked array; a block shared by two prompts is split between
 * them.  The caller owns the workspace; its contents are scratch.  d_k = 16 has only the
 * token-sequential form and ignores the workspace.  A short workspace is GDN_ERR_WORKSPACE. */
size_t gdn_beam_prefill_workspace_bytes(int32_t H, int32_t d_k, int32_t d_v, int64_t N);
gdn_status gdn_beam_prefill(int32_t R, int32_t H, int32_t H_K, int32_t d_k, int32_t d_v, int64_t N,
                            const float* k, const float* v, const float* alpha,
                            const float* beta, const int32_t* offsets,
                            float* S_out, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* GDN_BEAM_H */
