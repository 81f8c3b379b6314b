/*
 * int4vh_probe.h -- a measurement kernel of libint4vh.so: a plain read-only
 * stream over a device buffer, the "achievable HBM bandwidth" reference for
 * the verify path's weight stream.
 *
 * The int4 head is read once per verify call; the method's point is moving
 * a quarter of the fp16 head's bytes ("Qwen3.8-27B on a Single RTX 3090: How
 * Calibrated Quantization and Speculative Decoding Hit 1,000 tok/s",
 * Technical Insight: the 4-bit verification head cuts memory bandwidth by
 * 75%).  How fast the same number of bytes can be read at all, with no
 * arithmetic, bounds what the verify kernel can reach on a given GPU.
 */
#ifndef INT4VH_PROBE_H
#define INT4VH_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define INT4VH_PROBE_EINVAL (-1)
/* Words of the `out` buffer of int4vh_stream_read. */
#define INT4VH_PROBE_OUT_WORDS 8192

/* Read `bytes` bytes of the device buffer `buf` once, asynchronously on
 * `stream` (a hipStream_t as void*), one persistent workgroup per compute
 * unit.  mode 0: 16-byte loads into registers, folded by xor; mode 1: 16-byte
 * per lane copies straight into LDS (global_load_lds_dwordx4, the verify
 * kernel's load), nothing read back.  out (device uint32
 * [INT4VH_PROBE_OUT_WORDS], caller-owned) receives one word per wave: in mode
 * 0 the xor of every 32-bit word the wave read (so the xor of all of `out`
 * is the xor of the whole buffer), in mode 1 zero.  event_before /
 * event_after (hipEvent_t, either may be NULL) take the start and end
 * timestamps of the kernel's own dispatch.  Returns 0, INT4VH_PROBE_EINVAL (NULL pointer, bytes 0 or not a
 * multiple of 1024, buf not 16-byte aligned, out not 4-byte aligned, mode not
 * 0 or 1), or INT4VH_EHIP (-4) with the text in
 * verify_lm_head_int4_last_error(). */
int int4vh_stream_read(const void *buf, size_t bytes, int mode, uint32_t *out, void *stream,
                       void *event_before, void *event_after);

#ifdef __cplusplus
}
#endif

#endif /* INT4VH_PROBE_H */
