/*
 * photon_probe.h - bandwidth probes: what one MI355X delivers for the
 * memory traffic of a decode call, with no attention arithmetic.
 *
 * The decode kernels read K/V through block tables over ragged contexts
 * (README "Technical details -> Paged attention": a block-level KV cache,
 * per-sequence cache offsets).  These two kernels read the same kind of
 * bytes and do nothing with them but fold them into a checksum, so their
 * time is a ceiling for the decode kernels at the same size:
 *
 *   - photon_probe_stream_read reads one contiguous buffer;
 *   - photon_probe_gather reads exactly the K and V rows a decode call over
 *     the same block tables and context lengths reads (every valid row of
 *     every (sequence, KV head) once, through the tables), split evenly
 *     over its wavefronts the way the decode kernel splits its work.
 *
 * Each wavefront XORs every 32-bit word it reads and stores the result to
 * sink[wavefront], so the XOR over sink[0 .. waves) equals the XOR of every
 * word read (a CPU check that the right bytes were read).  Conventions as in
 * photon_decode.h: device pointers owned by the caller, asynchronous on
 * stream, validation before any HIP call, status codes.
 */
#ifndef PHOTON_PROBE_H
#define PHOTON_PROBE_H

#include "photon_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read bytes (a positive multiple of 16) of buf, 16-byte aligned, with
 * `waves` wavefronts (a positive multiple of 4, at most 2^20), each taking a
 * contiguous, equal share in 16 KiB batches of 16-byte loads.
 *   sink  [waves] uint32, written
 */
PHOTON_API photon_status photon_probe_stream_read(const void *buf, size_t bytes, int32_t waves,
                                                  uint32_t *sink, void *stream);

/*
 * Read every valid K and V row of the decode call described by desc
 * (rows t < context_lens[b] of sequence b under every KV head, through
 * block_tables), with `waves` wavefronts (a positive multiple of 4, at most
 * 2^20), each taking an equal share of the list of (sequence, KV head,
 * block) tiles, sequence-major.  desc->num_seqs must be at most 64 (the
 * tile prefix sums are held in one wavefront's registers); desc->num_q_heads
 * and desc->flags are not used.  Arguments otherwise as for
 * photon_paged_attn_decode.
 *   sink  [waves] uint32, written
 */
PHOTON_API photon_status photon_probe_gather(const void *k_cache, const void *v_cache,
                                             const int32_t *block_tables,
                                             const int32_t *context_lens,
                                             const photon_decode_desc *desc, int32_t waves,
                                             uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PHOTON_PROBE_H */
