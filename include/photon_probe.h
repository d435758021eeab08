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

/*
 * The rows of photon_probe_gather, with the list of (sequence, KV head,
 * block) tiles split evenly over `workgroups` workgroups of four
 * wavefronts (1 to 2^18).  A workgroup's wavefronts take its tiles in turn;
 * each keeps ring_tiles tiles (2, 4 or 8) in flight in its own part of LDS,
 * written by the loads themselves, and reads each back once it has landed.
 * The ring of a workgroup (4 x ring_tiles x 32 x row bytes) must fit in
 * 128 KiB: 8 tiles for 128-byte rows, 4 for 256, 2 for 512; other sizes are
 * PHOTON_ERR_UNSUPPORTED.  Other arguments as for photon_probe_gather.
 *   sink  [4 * workgroups] uint32, written
 */
PHOTON_API photon_status photon_probe_gather_staged(const void *k_cache, const void *v_cache,
                                                    const int32_t *block_tables,
                                                    const int32_t *context_lens,
                                                    const photon_decode_desc *desc,
                                                    int32_t workgroups, int32_t ring_tiles,
                                                    uint32_t *sink, void *stream);

/*
 * The rows of photon_probe_gather.  The first static_permille thousandths
 * (0 to 1000) of the tile list are split evenly over the wavefronts; the
 * rest is cut into pieces of piece_tiles tiles (1 to 64) that wavefronts
 * draw at run time: each draws tickets from *queue with an agent-scope
 * atomic add until it draws one past the last piece.
 *   queue  one uint64, device memory, 8-byte aligned, read and written.  It
 *          must hold zero when the call starts; the wavefront that draws the
 *          call's last ticket stores zero back, so calls that complete leave
 *          it ready for the next.  After a call that did not complete, clear
 *          it.  A non-zero start makes the call skip pieces (a wrong
 *          checksum), never read out of bounds or loop without end.  Calls
 *          that share one queue must not overlap.
 *   sink   [waves] uint32, written
 * Other arguments as for photon_probe_gather.
 */
PHOTON_API photon_status photon_probe_gather_queue(const void *k_cache, const void *v_cache,
                                                   const int32_t *block_tables,
                                                   const int32_t *context_lens,
                                                   const photon_decode_desc *desc, int32_t waves,
                                                   int32_t static_permille, int32_t piece_tiles,
                                                   uint64_t *queue, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PHOTON_PROBE_H */
