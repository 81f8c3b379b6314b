/*
 * int4vh_drafter.h -- C ABI of the context-copy (prompt lookup) drafter that
 * fills verify positions 7-14 from the request's own prompt (same library,
 * libint4vh.so; status codes and error text as in int4vh.h).
 *
 * The operation: "Qwen3.8-27B on a Single RTX 3090: How Calibrated
 * Quantization and Speculative Decoding Hit 1,000 tok/s", Technical Insight
 * (the draft-from-context optimisation copies positions 7-14 of the verify
 * block from the prompt), and "HyperQwen on one RTX 3090: a first-time
 * developer's guide to the 381-token claim", "What actually became faster?"
 * (a lookup proposes further tokens straight from the context).  For request
 * r with prompt P (length L) and key = the last n_max tokens of its sequence
 * (committed tokens then the 7 drafted ones):
 *   l(e)  for 1 <= e <= L-1: the number of key tokens matching P backwards
 *         from e (P[e-1-i] == key[n_max-1-i] for i < l(e), l(e) <= min(n_max, e))
 *   match the largest l(e) >= n_min; among equal lengths the largest e
 *   out   P[e .. e + count), count = min(n_out, L - e); no match: count 0
 *
 * Layout (device memory owned by the caller):
 *   prompts        int32, all prompts back to back
 *   prompt_offsets int64 [R+1]: prompt r is prompts[offsets[r] .. offsets[r+1])
 *   keys           int32 [R, n_max]
 *   out_tokens     int32 [R, n_out]: the proposal, -1 past count
 *   out_count, out_match_end (-1 if none), out_match_len (0 if none): int32 [R]
 * Integer work only; results are exact.  One workgroup per request.
 *
 * Errors (host validation before any launch): INT4VH_EINVAL for R < 1, n_max
 * outside [1, 64], n_min outside [1, n_max], n_out outside [1, 64] or a NULL
 * pointer; INT4VH_EALIGN for int32 arrays not 4-byte or offsets not 8-byte
 * aligned; INT4VH_EHIP for a launch failure.  Offsets must be non-decreasing
 * with each prompt shorter than 2^31 tokens (a precondition).
 */
#ifndef INT4VH_DRAFTER_H
#define INT4VH_DRAFTER_H

#include <stddef.h>
#include <stdint.h>

#include "int4vh.h"

#ifdef __cplusplus
extern "C" {
#endif

int context_copy_propose(const int32_t *prompts, const int64_t *prompt_offsets, int R,
                         const int32_t *keys, int n_max, int n_min, int n_out, int32_t *out_tokens,
                         int32_t *out_count, int32_t *out_match_end, int32_t *out_match_len,
                         void *stream);

/* The call instrumented for measurement: event_before / event_after
 * (caller-owned hipEvent_t, either may be NULL) take the start and end
 * timestamps of the kernel's own dispatch; not for use under HIP graph
 * capture. */
int context_copy_propose_timed(const int32_t *prompts, const int64_t *prompt_offsets, int R,
                               const int32_t *keys, int n_max, int n_min, int n_out,
                               int32_t *out_tokens, int32_t *out_count, int32_t *out_match_end,
                               int32_t *out_match_len, void *stream, void *event_before,
                               void *event_after);

#ifdef __cplusplus
}
#endif

#endif /* INT4VH_DRAFTER_H */
