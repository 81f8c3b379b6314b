/*
 * int4vh.h -- C ABI of the MI355X (gfx950) int4 lm_head verification library
 * (libint4vh.so).
 *
 * The operation.  A verify block of final hidden states is projected through
 * a calibrated int4 output head, each position is reduced to its greedy
 * argmax, and the number of leading drafted tokens that agree with those
 * argmaxes is counted:
 *
 *   logit[r, v]   = sum_h  f32(hidden[r, h]) * f32(scales[h]) * q[v, h]
 *   argmax_ids[r] = the v with the largest logit[r, v]; lowest v on ties
 *   logits_max[r] = logit[r, argmax_ids[r]]
 *   n_accepted[i] = largest k <= T-1 with draft_ids[i, t] == argmax_ids[i*T + t]
 *                   for every t < k
 *
 * Sources: the int4 head with one scale per hidden channel and values in
 * [-7, 7] is the requantised lm_head of "Qwen3.8-27B on a Single RTX 3090:
 * How Calibrated Quantization and Speculative Decoding Hit 1,000 tok/s",
 * Technical Insight (requantisation listing), also "HyperQwen: 1,000 tok/s on
 * a Single RTX 3090 Through Aggressive Recurrent-State Speculation", Technical
 * Insight (lm_head paragraph: only the ordering of logits matters).  Greedy
 * verification with an accepted prefix is the verify step of the same
 * "Qwen3.8-27B ..." page, Technical Insight (split-KV verify listing), and a
 * block of up to 16 positions (7 drafted, up to 8 copied from the context, 1
 * bonus) is from "HyperQwen on one RTX 3090: a first-time developer's guide to
 * the 381-token claim", "What actually became faster?".
 *
 * Data layout (all row-major, all device memory owned by the caller):
 *   hidden     binary16 [M, H], M = R*T rows (request i owns rows i*T..i*T+T-1)
 *   packed_w   uint8 [V, H/2]: two int4 values per byte, low nibble = even
 *              hidden channel h, high nibble = h+1, two's-complement nibbles.
 *              Only [-7, 7] is legal; nibble 0x8 is a precondition violation
 *              that the verify calls do not check (see *_check_weights).
 *   scales     binary16 [H], one scale per hidden channel
 *   draft_ids  int32 [R, T-1]; NULL allowed only when T == 1.  Ids outside
 *              [0, V) are legal and never match.
 *   logits_max float32 [M]; argmax_ids int32 [M]; n_accepted int32 [R]
 *   logits_out optional float32 [M, V] (every logit; NULL to skip)
 *
 * Numerics.  For each row, hidden*scale (exact in binary32) is rounded to a
 * 24-bit fixed-point code with a power-of-two step chosen from the row's
 * largest |hidden*scale| (the step is at most 2^-22 of it; round to nearest
 * even).  Each code is split into three signed bytes, the int4 weights enter
 * the int8 matrix cores exactly, the int32 partial sums are exact and are
 * combined exactly in 64-bit integers, and each logit is rounded to
 * binary32 once.  The absolute error of a logit is below
 *   2^-23 * max_h|hidden*scale| * sum_h|q[v,h]|   (+ the final rounding),
 * far inside the 2e-3 * max_v|logit| parity tolerance.  Every result is
 * bit-for-bit reproducible and independent of the launch shape: a row gives
 * the same logits, argmax and maximum whether it runs alone, in a block of
 * up to 16 rows (the weight-stream kernel) or in a batch of up to 4096 rows
 * (the MFMA-bound batch kernel).
 *
 * Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL is
 * the null stream).  Results are valid once the caller synchronises that
 * stream.  The verify calls allocate nothing and never synchronise.
 *
 * Workspace.  Every verify call needs a caller-owned device workspace of at
 * least verify_lm_head_int4_workspace_bytes(R, T, V, H) bytes, 256-byte
 * aligned, initialised once with verify_lm_head_int4_workspace_init.  A
 * call leaves the workspace ready for the next call.  Two calls that are in
 * flight at the same time must not share a workspace.  After a call that
 * returned INT4VH_EHIP, initialise the workspace again.
 *
 * Errors.  Every entry point returns a status code; nothing is thrown across
 * the ABI.  Arguments are validated on the host before anything is launched
 * (no GPU call happens when validation fails):
 *   INT4VH_EINVAL       T outside [1, 16]; R < 1; R*T > 4096
 *                       (INT4VH_MAX_ROWS); V < 1; H < 32 or H % 32 != 0; a
 *                       required pointer is NULL
 *   INT4VH_EALIGN       a tensor pointer is not 16-byte aligned (workspace:
 *                       256-byte aligned)
 *   INT4VH_EWORKSPACE   workspace smaller than required
 *   INT4VH_EUNSUPPORTED a shape beyond this build's limits (H > 8192,
 *                       V*H/2 >= 2^40 bytes)
 *   INT4VH_EHIP         a HIP runtime error; the text is in
 *                       verify_lm_head_int4_last_error()
 *   INT4VH_ESCRATCH     (verify_lm_head_int4_batch_noalloc only) the shape
 *                       needs more workspace than its static scratch holds
 */
#ifndef INT4VH_H
#define INT4VH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    INT4VH_OK = 0,
    INT4VH_EINVAL = -1,
    INT4VH_EALIGN = -2,
    INT4VH_EWORKSPACE = -3,
    INT4VH_EHIP = -4,
    INT4VH_EUNSUPPORTED = -5,
    INT4VH_ESCRATCH = -6
};

/* Largest hidden size of this build. */
#define INT4VH_MAX_H 8192
/* Largest T (verify positions per request). */
#define INT4VH_MAX_T 16
/* Largest number of rows R*T of one call. */
#define INT4VH_MAX_ROWS 4096

/* Bytes of workspace a verify call with these sizes needs (0 if the sizes are
 * invalid).  Pure host function. */
size_t verify_lm_head_int4_workspace_bytes(int R, int T, int V, int H);

/* Bytes of workspace verify_lm_head_int4_sampled (and its _timed variant)
 * needs: the same as verify_lm_head_int4_workspace_bytes up to 64 rows; above,
 * that plus the call's logits, R*T*V*4 bytes, and the rows' best keys per
 * vocabulary tile of 128 rows, R*T*ceil(V/128)*8 bytes (areas rounded to
 * 256).  0 if the sizes are invalid.  Pure host function. */
size_t verify_lm_head_int4_sampled_workspace_bytes(int R, int T, int V, int H);

/* Zero the workspace's control words on `stream` (a small fill kernel, no
 * memset node, so it may be captured in a graph).  Call once after
 * allocation.  Returns INT4VH_EINVAL for NULL, INT4VH_EALIGN if not 256-byte
 * aligned, INT4VH_EWORKSPACE if ws_bytes is below the minimum for any call. */
int verify_lm_head_int4_workspace_init(void *workspace, size_t workspace_bytes, void *stream);

/* One request: the verify block of T <= 16 positions (R = 1). */
int verify_lm_head_int4(const void *hidden, const uint8_t *packed_w, const void *scales,
                        const int32_t *draft_ids, int T, int V, int H,
                        float *logits_max, int32_t *argmax_ids, int32_t *n_accepted,
                        float *logits_out, void *workspace, size_t workspace_bytes,
                        void *stream);

/* R independent requests of T positions each, sharing one head.  Rows of
 * request i are hidden[i*T .. i*T+T-1]; its drafts are draft_ids[i*(T-1) ..].
 * Per-request acceptance goes to n_accepted[i].  Up to 64 rows the call runs
 * the weight-stream kernels (in token groups of 16 beyond 16 rows); beyond,
 * up to INT4VH_MAX_ROWS rows, it runs a GEMM on the int8 matrix cores.  The
 * workspace grows with R*T (verify_lm_head_int4_workspace_bytes).  The batch
 * mode of the HyperQwen README, "The numbers behind that", serves 64 requests
 * at once: 64 x 4 = 256 rows.  Results are identical either way. */
int verify_lm_head_int4_batch(const void *hidden, const uint8_t *packed_w, const void *scales,
                              const int32_t *draft_ids, int R, int T, int V, int H,
                              float *logits_max, int32_t *argmax_ids, int32_t *n_accepted,
                              float *logits_out, void *workspace, size_t workspace_bytes,
                              void *stream);

/* The batch call, instrumented: event_before and event_after (hipEvent_t
 * handles owned by the caller, created on the stream's device; either may be
 * NULL) take the start and end timestamps of the main verify kernel's own
 * dispatch (the staging kernel runs before it, untimed), so that
 * hipEventElapsedTime gives the main kernel's duration alone, as a kernel
 * trace measures it.  Same arguments, results and errors as
 * verify_lm_head_int4_batch; a failed launch returns INT4VH_EHIP.  For
 * measuring the weight stream (or the matrix cores) against its roofline;
 * under HIP graph capture call it with both events NULL (or call
 * verify_lm_head_int4_batch), since events attached to a dispatch are not
 * part of the capturable API. */
int verify_lm_head_int4_batch_timed(const void *hidden, const uint8_t *packed_w,
                                    const void *scales, const int32_t *draft_ids, int R, int T,
                                    int V, int H, float *logits_max, int32_t *argmax_ids,
                                    int32_t *n_accepted, float *logits_out, void *workspace,
                                    size_t workspace_bytes, void *stream, void *event_before,
                                    void *event_after);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the batch
 * call with no workspace argument.  The library keeps one scratch array of
 * INT4VH_SCRATCH_BYTES (16 MiB) per device in static device memory, created
 * when the library's code object is loaded on that device and held until the
 * process ends; this call allocates nothing and calls no allocating routine.
 * Its control words are zeroed once per device by a small fill kernel on
 * `stream` (under stream capture the fill is recorded into the graph, and the
 * next uncaptured call issues it again); every call leaves them zeroed.
 * Every call on one device shares that device's array, which keeps the last
 * call's contents: calls that overlap in time on one GPU (two streams, two
 * host threads, two graphs in flight) race and must be serialised by the
 * caller.  Same arguments (minus the workspace), results and errors as
 * verify_lm_head_int4_batch, plus INT4VH_ESCRATCH, returned before any GPU
 * call, when the shape needs more workspace than the scratch holds
 * (verify_lm_head_int4_workspace_bytes(R, T, V, H) > INT4VH_SCRATCH_BYTES:
 * every call of up to 16 rows fits; at H = 5120, up to 1024 rows).  After an
 * INT4VH_EHIP the next call zeroes the control words again. */
#define INT4VH_SCRATCH_BYTES (16u << 20)
int verify_lm_head_int4_batch_noalloc(const void *hidden, const uint8_t *packed_w, const void *scales,
                                      const int32_t *draft_ids, int R, int T, int V, int H,
                                      float *logits_max, int32_t *argmax_ids, int32_t *n_accepted,
                                      float *logits_out, void *stream);

/* A head whose rows are a subset of the vocabulary: the draft vocabulary of
 * "HyperQwen: 1,000 tok/s on a Single RTX 3090 Through Aggressive
 * Recurrent-State Speculation", Technical Insight (speculation configuration:
 * the drafter's vocabulary is cut to the 8192 tokens actually observed, out of
 * about 152k), and the 40k-token draft vocabulary of the HyperQwen README
 * ("Roadmap").  vocab_ids (device int32 [V], required) gives the token id of
 * each head row and must be strictly increasing and non-negative (checked by
 * verify_lm_head_int4_check_vocab_map, not by this call).  The argmax is taken
 * over the head's rows exactly as in verify_lm_head_int4_batch (the lowest row
 * wins ties, which is the lowest token id for an increasing map); argmax_ids
 * then holds vocab_ids[row], and the drafts are compared with those token ids.
 * logits_out, when given, is indexed by head row.  Other arguments, results
 * and errors as verify_lm_head_int4_batch; INT4VH_EINVAL if vocab_ids is NULL,
 * INT4VH_EALIGN if it is not 4-byte aligned. */
int verify_lm_head_int4_mapped(const void *hidden, const uint8_t *packed_w, const void *scales,
                               const int32_t *vocab_ids, const int32_t *draft_ids, int R, int T,
                               int V, int H, float *logits_max, int32_t *argmax_ids,
                               int32_t *n_accepted, float *logits_out, void *workspace,
                               size_t workspace_bytes, void *stream);

/* Sampled (non-greedy) verification for R*T <= 4096 rows (R requests of T
 * positions).  Up to 64 rows the sampling epilogue is fused into the weight
 * stream (beyond 16 rows in token groups of 16 sharing the tile stream, like
 * the greedy call); above, the batch kernels write the call's logits into the
 * workspace and one workgroup per row takes its top-k, log-sum-exp and p(d)
 * from them (same formulas and ties; the workspace is then
 * verify_lm_head_int4_sampled_workspace_bytes).  The int4 head suffices
 * because top-k
 * sampling needs only the ordering of the logits ("HyperQwen: 1,000 tok/s on
 * a Single RTX 3090 Through Aggressive Recurrent-State Speculation",
 * Technical Insight, lm_head paragraph).  Per row r:
 *   lse[r]         log sum_v exp(logit[r, v] / temperature) over the whole
 *                  vocabulary (optional output, NULL to skip)
 *   topk_ids[r, j], topk_logits[r, j]  for top_k >= 1: the top_k largest
 *                  logits, best first (equal logits: lower row first)
 *   argmax_ids[r], logits_max[r]        the greedy outputs
 * and per drafted position t < T-1 of request i, with d = draft_ids[i, t]:
 *   p_draft[i, t]  the target probability of d: for top_k >= 1, top-k
 *                  sampling, exp(l_d / tau) / sum_j exp(l_j / tau) over the k
 *                  logits (0 if d is not among them); for top_k == 0,
 *                  sampling over the whole vocabulary, exp(l_d / tau - lse)
 *                  (0 if d is outside [0, V)); binary32
 *   accepted       uniforms[i, t] * draft_probs[i, t] < p_draft[i, t]
 *                  (draft_probs: the drafter's probability of d, 1 for a
 *                  token copied from the context; uniforms in [0, 1) drawn
 *                  by the caller)
 *   n_accepted[i]  the number of leading accepted drafts (speculative
 *                  sampling; the caller draws the replacement or bonus token
 *                  from the top-k outputs).
 * draft_probs, uniforms, p_draft: device float32 [R, T-1] (may be NULL only
 * when T == 1); topk_ids int32 / topk_logits float32 [R*T, top_k] (may be
 * NULL when top_k == 0); lse float32 [R*T] or NULL.
 * Errors as verify_lm_head_int4_batch (INT4VH_EWORKSPACE against
 * verify_lm_head_int4_sampled_workspace_bytes), plus INT4VH_EINVAL for top_k
 * outside [0, min(16, V)], a temperature that is not finite and > 0, or a
 * missing sampled buffer. */
int verify_lm_head_int4_sampled(const void *hidden, const uint8_t *packed_w, const void *scales,
                                const int32_t *draft_ids, const float *draft_probs,
                                const float *uniforms, int R, int T, int V, int H, int top_k,
                                float temperature, float *logits_max, int32_t *argmax_ids,
                                int32_t *topk_ids, float *topk_logits, float *lse, float *p_draft,
                                int32_t *n_accepted, void *workspace, size_t workspace_bytes,
                                void *stream);

/* The sampled call, instrumented like verify_lm_head_int4_batch_timed:
 * event_before / event_after (caller-owned hipEvent_t, either may be NULL)
 * take the start and end timestamps of the main verify kernel's dispatch
 * (the batch kernel above 64 rows; the selection and acceptance kernels
 * after it are untimed). */
int verify_lm_head_int4_sampled_timed(const void *hidden, const uint8_t *packed_w,
                                      const void *scales, const int32_t *draft_ids,
                                      const float *draft_probs, const float *uniforms, int R, int T,
                                      int V, int H, int top_k, float temperature,
                                      float *logits_max, int32_t *argmax_ids, int32_t *topk_ids,
                                      float *topk_logits, float *lse, float *p_draft,
                                      int32_t *n_accepted, void *workspace, size_t workspace_bytes,
                                      void *stream, void *event_before, void *event_after);

/* Count the positions i of a row -> token map (device int32 [V]) where it is
 * not strictly increasing and non-negative (vocab_ids[0] < 0, or
 * vocab_ids[i] <= vocab_ids[i-1]) into *n_bad_out (device int32,
 * overwritten).  Asynchronous on `stream`. */
int verify_lm_head_int4_check_vocab_map(const int32_t *vocab_ids, int V, int32_t *n_bad_out,
                                        void *stream);

/* Count illegal nibbles (0x8) of a packed head into *n_bad_out (device int32,
 * overwritten).  Asynchronous on `stream`. */
int verify_lm_head_int4_check_weights(const uint8_t *packed_w, int V, int H,
                                      int32_t *n_bad_out, void *stream);

/* Static text for a status code. */
const char *verify_lm_head_int4_status_string(int status);

/* Text of the last INT4VH_EHIP error raised on the calling thread ("" if
 * none).  Valid until the next call on that thread. */
const char *verify_lm_head_int4_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* INT4VH_H */
