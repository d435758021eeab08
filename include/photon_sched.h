/*
 * photon_sched.h - C ABI of the host-side block manager and two-phase step
 * scheduler that produce the inputs of the decode path (block tables,
 * context lengths, slot mappings, positions).
 *
 * What it follows (PhotonInfer README):
 *   - "Technical details -> Paged attention": a block-level KV cache with
 *     allocation free of fragmentation (here: a FIFO free list of fixed-size
 *     physical blocks) and per-sequence cache offsets (here: block tables);
 *   - "Technical details -> Continuous-batching scheduler": two phases per
 *     step, first every running request continues, then waiting requests
 *     are admitted into the capacity that is left; requests go waiting ->
 *     running -> finished, with preemption; num_computed_tokens records
 *     exactly where a request resumes;
 *   - "Key features -> vLLM-style continuous batching": requests join while
 *     others are generating, at token granularity.
 *
 * Rules (the same in the CPU reference the tests compare against):
 *   - A request has prompt_len tokens and generates max_new_tokens.  Its
 *     known tokens are the prompt plus the tokens generated so far;
 *     num_computed counts the known tokens whose K/V are in the cache.
 *   - schedule(), phase 1: running requests in running order each get
 *     n = min(known - num_computed, budget_left - R) new tokens, R being the
 *     number of running requests after it (each of which must still get at
 *     least one), so no running request is ever skipped.  The blocks to
 *     hold num_computed + n tokens are taken from the front of the free
 *     list; while too few are free, the last running request is preempted:
 *     its blocks go to the back of the free list in table order, its
 *     num_computed becomes 0 and it goes to the front of the waiting queue
 *     (it may be the request being scheduled, which then gets no tokens).
 *   - schedule(), phase 2: while requests wait, fewer than max_seqs are
 *     scheduled and token budget is left, the first waiting request gets
 *     n = min(known - num_computed, budget_left) tokens if the free list
 *     holds the blocks for them; it then joins the end of the running list.
 *     Otherwise admission stops for this step (phase 2 never preempts).
 *   - update() (after the step ran): each scheduled request adds its n to
 *     num_computed; a request whose known tokens are then all computed
 *     generates one token; a request that has generated max_new_tokens
 *     finishes and its blocks go to the back of the free list.
 *   - The batch lists phase-1 requests in running order, then phase-2
 *     requests in admission order.  Request b's new tokens are at
 *     positions num_computed .. num_computed + n - 1, its slots follow from
 *     its block table (slot = block * block_size + position % block_size),
 *     and context_lens[b] = num_computed + n (the tokens attended to after
 *     the step's cache write).
 *
 * Memory: the scheduler owns its host state (created and destroyed through
 * this API).  photon_sched_schedule writes into host arrays the caller
 * provides, sized by the limits given at creation.  Not thread-safe: one
 * thread at a time per scheduler.  Errors are returned as photon_status
 * (see photon_decode.h) with a message from photon_last_error_detail().
 */
#ifndef PHOTON_SCHED_H
#define PHOTON_SCHED_H

#include <stdint.h>

#include "photon_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct photon_sched photon_sched; /* opaque */

typedef struct photon_sched_config {
    int32_t num_blocks;          /* physical blocks in the pool, > 0               */
    int32_t block_size;          /* tokens per block, > 0 (the kernels use 16)     */
    int32_t max_seqs;            /* requests per step, > 0                         */
    int32_t max_tokens_per_step; /* new tokens per step, >= max_seqs               */
    int32_t max_blocks_per_seq;  /* row length of the block tables, > 0            */
} photon_sched_config;

/* One scheduled step.  The caller sets the pointers (host arrays of the
 * stated capacities); schedule() fills them and the counts. */
typedef struct photon_sched_batch {
    int32_t num_seqs;       /* out: B                                               */
    int32_t num_tokens;     /* out: T = sum of new tokens                           */
    int32_t num_preempted;  /* out: requests preempted during this schedule call    */
    int32_t reserved;
    int64_t *request_ids;   /* [max_seqs]                                           */
    int32_t *query_start;   /* [max_seqs + 1]: request b's tokens are
                               query_start[b] .. query_start[b+1] - 1               */
    int32_t *context_lens;  /* [max_seqs]                                           */
    int32_t *block_tables;  /* [max_seqs * max_blocks_per_seq], -1 past the table   */
    int32_t *slot_mapping;  /* [max_tokens_per_step]                                */
    int32_t *positions;     /* [max_tokens_per_step]                                */
    int64_t *preempted_ids; /* [max_seqs] or NULL: ids preempted, in order          */
} photon_sched_batch;

/* Per-request counters, for inspection. */
typedef struct photon_sched_request_info {
    int32_t state;          /* 0 waiting, 1 running, 2 finished                     */
    int32_t num_computed;   /* known tokens with K/V in the cache                   */
    int32_t num_known;      /* prompt + generated                                   */
    int32_t num_generated;
    int32_t num_blocks;     /* blocks held                                          */
    int32_t num_preemptions;
} photon_sched_request_info;

PHOTON_API photon_status photon_sched_create(const photon_sched_config *config, photon_sched **out);
PHOTON_API void photon_sched_destroy(photon_sched *sched);

/* Queue a new request (waiting, behind the requests already waiting).  Ids
 * must be unique.  prompt_len >= 1, max_new_tokens >= 1, and the most tokens
 * it can cache, prompt_len + max_new_tokens - 1, must fit in
 * max_blocks_per_seq and in the pool. */
PHOTON_API photon_status photon_sched_add_request(photon_sched *sched, int64_t request_id,
                                                  int32_t prompt_len, int32_t max_new_tokens);

/* Phase 1 and phase 2 of one step; fills *batch.  A second schedule() before
 * update() is an error.  A step with nothing to run returns num_seqs = 0. */
PHOTON_API photon_status photon_sched_schedule(photon_sched *sched, photon_sched_batch *batch);

/* Apply the step last scheduled (see the rules above).  *num_finished (if
 * not NULL) receives how many requests finished; their ids go to
 * finished_ids (if not NULL, capacity max_seqs). */
PHOTON_API photon_status photon_sched_update(photon_sched *sched, int32_t *num_finished,
                                             int64_t *finished_ids);

/* Counts of the scheduler: waiting, running, finished requests, free blocks. */
PHOTON_API photon_status photon_sched_counts(const photon_sched *sched, int32_t *num_waiting,
                                             int32_t *num_running, int32_t *num_finished,
                                             int32_t *num_free_blocks);

PHOTON_API photon_status photon_sched_request(const photon_sched *sched, int64_t request_id,
                                              photon_sched_request_info *info);

#ifdef __cplusplus
}
#endif

#endif /* PHOTON_SCHED_H */
