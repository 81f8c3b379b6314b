/*
 * int4vh_requant.h -- C ABI of the offline requantisation of the output head
 * into the calibrated int4 format that the verify calls of int4vh.h read
 * (same library, libint4vh.so; status codes and error text as in int4vh.h).
 *
 * The operation is the requantisation of "Qwen3.8-27B on a Single RTX 3090:
 * How Calibrated Quantization and Speculative Decoding Hit 1,000 tok/s",
 * Technical Insight (requantisation listing), also described in "HyperQwen:
 * 1,000 tok/s on a Single RTX 3090 Through Aggressive Recurrent-State
 * Speculation", Technical Insight (lm_head paragraph):
 *
 *   amax[h]   = max over calibration rows n of |acts[n, h]|        (exact)
 *   scales[h] = binary16( amax[h] / 7 )   division in binary32, then rounded
 *                                         to binary16 (nearest, ties to even)
 *   q[v, h]   = clamp( round_half_even( W[v, h] / scales[h] ), -7, 7 )
 *               with the quotient in binary32; q = 0 where scales[h] is 0 or
 *               infinite
 *   packed    = q packed two per byte, [V, H/2], low nibble = even channel,
 *               high nibble = odd channel, two's-complement nibbles: the head
 *               layout of verify_lm_head_int4.
 *
 * The calibration statistics (activations of the model on representative
 * prompts) come from the caller; they need the model and a dataset.
 *
 * Results are bit-exact: the integer codes equal those of the binary32
 * definition above for every finite input.  The kernels compute W * (1/s)
 * and round it, after snapping it to a multiple of 2^-14, to the nearest
 * integer: for binary16 or bfloat16 weights and binary16 scales this gives
 * the definition's code for every input pair, exact ties included.
 *
 * Element types: dtype INT4VH_F16 (IEEE binary16) or INT4VH_BF16 (bfloat16)
 * for the weights and the activations; scales are always binary16.  Inputs
 * must be finite, a precondition that the kernels do not check (results for
 * NaN or infinite inputs are unspecified).
 *
 * Calls are asynchronous on `stream` (a hipStream_t passed as void*), allocate
 * nothing and never synchronise.  Arguments are validated on the host before
 * any launch (no GPU call on failure):
 *   INT4VH_EINVAL  N < 1, V < 1, H < 32 or H % 32 != 0, unknown dtype, a NULL
 *                  pointer
 *   INT4VH_EALIGN  acts, W, scales or packed not 16-byte aligned; amax not
 *                  4-byte aligned
 *   INT4VH_EUNSUPPORTED  V*H/32 >= 2^31 or N*H >= 2^40 elements
 *   INT4VH_EHIP    a launch failed (text in verify_lm_head_int4_last_error)
 */
#ifndef INT4VH_REQUANT_H
#define INT4VH_REQUANT_H

#include <stddef.h>
#include <stdint.h>

#include "int4vh.h"

#ifdef __cplusplus
extern "C" {
#endif

enum { INT4VH_F16 = 0, INT4VH_BF16 = 1 };

/* Running per-channel maximum of |acts| over a batch of N calibration rows:
 *   acts   device [N, H] of `dtype`, row-major
 *   amax   device float32 [H], read and written: on return
 *          amax[h] = max(amax[h], max_n |acts[n, h]|) if accumulate != 0,
 *          or max_n |acts[n, h]| if accumulate == 0 (amax is cleared first).
 * Call once per batch of calibration rows (accumulate = 0 for the first) to
 * reduce a whole calibration set.  amax values are >= 0. */
int requant_lm_head_int4_amax(const void *acts, int dtype, int N, int H, float *amax,
                              int accumulate, void *stream);

/* scales[h] = binary16(amax[h] / 7) for h < H (device float32 [H] in,
 * device binary16 [H] out).  amax must be >= 0. */
int requant_lm_head_int4_scales(const float *amax, int H, void *scales, void *stream);

/* Quantise and pack the head: W device [V, H] of `dtype`, scales device
 * binary16 [H], packed device uint8 [V, H/2] (written in full). */
int requant_lm_head_int4_pack(const void *W, int dtype, int V, int H, const void *scales,
                              uint8_t *packed, void *stream);

/* The three steps in order for one calibration batch: amax (cleared first,
 * caller-owned device float32 [H] scratch that holds the statistics on
 * return), scales, packed. */
int requant_lm_head_int4(const void *W, int w_dtype, int V, int H, const void *acts,
                         int acts_dtype, int N, float *amax, void *scales, uint8_t *packed,
                         void *stream);

/* The pack step, instrumented for measurement: event_before and event_after
 * (caller-owned hipEvent_t handles, either may be NULL) take the start and
 * end timestamps of the quantise-and-pack kernel's own dispatch
 * (hipExtLaunchKernel); not for use under HIP graph capture. */
int requant_lm_head_int4_pack_timed(const void *W, int dtype, int V, int H, const void *scales,
                                    uint8_t *packed, void *stream, void *event_before,
                                    void *event_after);

#ifdef __cplusplus
}
#endif

#endif /* INT4VH_REQUANT_H */
