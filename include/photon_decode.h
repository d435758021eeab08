/*
 * photon_decode.h - C ABI of the MI355X (gfx950) batched paged-attention
 * decode library.
 *
 * The operations are the two steps of a decode step that the PhotonInfer
 * README describes:
 *   - "Technical details -> Paged attention": a block-level KV cache, per
 *     sequence cache offsets (here: block tables), and one kernel that writes
 *     the K/V of many sequences at once (here: a per-token slot mapping);
 *   - "GPU-optimised kernels": batched paged attention with a numerically
 *     stable softmax, and batched RoPE among the fused operations (applied
 *     to q and k in the same kernel as the cache write).
 *
 * Conventions shared by every entry point
 *   - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *     never allocates, frees or keeps a pointer past the call (the README's
 *     "C++20 architecture" section asks for zero-copy views; these are they).
 *   - Tensors are dense, row-major.  The K and V pools share one layout,
 *     [num_blocks, num_kv_heads, block_size, head_dim]; the row of token
 *     position t of sequence b under KV head g is
 *     pool[block_tables[b][t / block_size]][g][t % block_size][:].
 *   - A slot is physical_block * block_size + offset_in_block (int32).
 *   - stream is a hipStream_t (NULL = the legacy default stream).  Work is
 *     enqueued asynchronously; PHOTON_OK means "validated and launched".  A
 *     fault inside a kernel surfaces at the caller's next synchronisation.
 *   - Errors are returned, never thrown (the README's "C++20 architecture"
 *     section: errors propagate explicitly as values).  All argument checks
 *     run before any HIP call, so they behave the same with or without a GPU.
 *     On failure nothing is launched and photon_last_error_detail() returns a
 *     message for the calling thread.
 *   - Device-resident indices (slot_mapping, block_tables, context_lens) are
 *     NOT range-checked by the kernels: out-of-range values are a caller
 *     error and may fault the GPU.
 *   - Functions may be called from several threads.  The library's only
 *     state is a process-wide call counter (see "Workspaces" below).
 *   - Workspaces.  Calls that split work over several wavefronts take a
 *     caller-provided workspace for partial results and per-segment arrival
 *     counters.  Its contents before a call do not matter: it need not be
 *     cleared, ever.  Each counter is a 64-bit word whose upper half is
 *     tagged with the number the library gives every call, and a call
 *     replaces any value tagged otherwise before counting on it (so neither
 *     uninitialised memory nor a call that never finished can corrupt a
 *     later call; a stale value is missed only if its tag happens to equal
 *     the new call's number, one chance in 2^32).  A call that finishes
 *     leaves every counter at 0.  Calls that may run at the same time (on
 *     different streams) need workspaces of their own.
 */
#ifndef PHOTON_DECODE_H
#define PHOTON_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PHOTON_ABI_VERSION 7

#if defined(__GNUC__)
#define PHOTON_API __attribute__((visibility("default")))
#else
#define PHOTON_API
#endif

typedef enum photon_status {
    PHOTON_OK = 0,
    PHOTON_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment, bad enum */
    PHOTON_ERR_UNSUPPORTED = 2, /* valid but not built: head_dim, block_size, group */
    PHOTON_ERR_WORKSPACE = 3,   /* workspace smaller than photon_paged_attn_workspace_bytes */
    PHOTON_ERR_HIP = 4          /* the HIP runtime refused a launch */
} photon_status;

/* Storage type of q, the K/V pools, new K/V rows and (unless
 * PHOTON_DECODE_OUT_F32 is set) the output.  Scores, softmax and
 * accumulation are always fp32.  PHOTON_BF16 is bfloat16 (the upper 16 bits
 * of a binary32), the half-precision type the README's roadmap names next to
 * FP16. */
typedef enum photon_dtype {
    PHOTON_F32 = 0,
    PHOTON_F16 = 1,
    PHOTON_BF16 = 2
} photon_dtype;

/* photon_decode_desc.flags */
enum {
    /* Write the decode output as fp32 whatever kv.dtype is (a no-op for
     * PHOTON_F32): the output row is then the fp32 accumulation, normalised,
     * without a final rounding to 16 bits. */
    PHOTON_DECODE_OUT_F32 = 1
};

/* Shape of one KV block pool (K and V pools have the same shape). */
typedef struct photon_kv_desc {
    int32_t num_blocks;   /* physical blocks in each pool, > 0                  */
    int32_t num_kv_heads; /* > 0                                                 */
    int32_t block_size;   /* tokens per block; 16 is built                      */
    int32_t head_dim;     /* 64 or 128 are built                                */
    int32_t dtype;        /* photon_dtype                                       */
} photon_kv_desc;

/* Shape of one decode call. */
typedef struct photon_decode_desc {
    int32_t num_seqs;           /* B, >= 0                                       */
    int32_t num_q_heads;        /* Hq, a multiple of kv.num_kv_heads; the group
                                   Hq / Hkv must be 1, 2, 4 or 8                 */
    int32_t max_blocks_per_seq; /* row length of block_tables, > 0               */
    int32_t max_context_len;    /* >= every context_lens[b], and
                                   <= max_blocks_per_seq * block_size; sizes the
                                   grid and the workspace                        */
    int32_t partition_tokens;   /* 0 = automatic (enough wavefronts for about
                                   64 KiB of K/V reads in flight per CU,
                                   counting the two chunks a wavefront keeps
                                   in flight, one with eight query heads per
                                   KV head; at least one per SIMD);
                                   otherwise the most tokens one wavefront
                                   handles when every sequence is at
                                   max_context_len, a positive multiple of
                                   photon_paged_attn_partition_quantum(); the
                                   actual batch is always split evenly over
                                   the wavefronts this implies, but over no
                                   more than one per five quanta of it (a
                                   slice is never much shorter than five)
                                   unless that leaves fewer than 256; in a
                                   batch of 768 quanta or more, a wavefront
                                   whose slice moves on to another (sequence,
                                   KV head) is charged two quanta for the
                                   change                                     */
    photon_kv_desc kv;
    int32_t flags;              /* PHOTON_DECODE_* bits, 0 = none; other bits
                                   are PHOTON_ERR_INVALID_ARG                    */
} photon_decode_desc;

/*
 * Slot-mapped KV cache write (README "Technical details -> Paged attention":
 * one kernel writes K/V rows of many sequences).
 *
 * For every token i < num_tokens with slot_mapping[i] >= 0 and every KV head
 * h, copies the raw bytes of k[i][h][:] into
 * k_cache[slot / block_size][h][slot % block_size][:], and the same for v.
 * Tokens whose slot is negative are skipped (padding).  No conversion: k, v
 * and the pools share kv->dtype, and the copy is bit-exact.
 *
 *   k, v          [num_tokens, num_kv_heads, head_dim]   kv->dtype, 16-byte aligned
 *   slot_mapping  [num_tokens] int32, each >= 0 slot distinct and
 *                 < num_blocks * block_size (two tokens with one slot: the
 *                 stored row is unspecified)
 *   k_cache, v_cache  pools, updated in place, 16-byte aligned
 *
 * num_tokens == 0 launches nothing and returns PHOTON_OK.
 */
PHOTON_API photon_status photon_kv_cache_write(const void *k, const void *v, const int32_t *slot_mapping,
                                    int32_t num_tokens, void *k_cache, void *v_cache,
                                    const photon_kv_desc *kv, void *stream);

/* Shape of one multi-query call. */
typedef struct photon_multi_query_desc {
    int32_t num_seqs;           /* B, >= 0 (at most 65535 / num_kv_heads)         */
    int32_t num_tokens;         /* T = query_start[B], rows of q and out, >= 0    */
    int32_t num_q_heads;        /* Hq, a multiple of kv.num_kv_heads; the group
                                   Hq / Hkv must be 1, 2, 4 or 8                  */
    int32_t max_blocks_per_seq; /* row length of block_tables, > 0                */
    int32_t max_query_len;      /* >= every query_start[b+1] - query_start[b];
                                   sizes the grid                                 */
    int32_t max_context_len;    /* >= every context_lens[b], <= max_blocks_per_seq
                                   * block_size; sizes the KV splits              */
    int32_t split_tokens;       /* 0 = automatic (about 1024 workgroups); else the
                                   KV tokens one workgroup scans for a tile of 16
                                   query rows, a positive multiple of 64          */
    int32_t flags;              /* PHOTON_DECODE_OUT_F32 or 0                     */
    photon_kv_desc kv;
} photon_multi_query_desc;

/*
 * Workspace bytes photon_paged_attn_multi_query needs for desc: 0 when no
 * tile's KV range is split, else one 64-bit arrival counter per tile of 16
 * query rows (padded to 256 bytes), then one fp32 record of
 * 16 * (head_dim + 2) floats per tile and split.  Its contents before a call
 * do not matter (see "Workspaces" above).
 */
PHOTON_API photon_status photon_paged_attn_multi_query_workspace_bytes(
    const photon_multi_query_desc *desc, size_t *bytes);

/*
 * Multi-query paged attention with a causal tail: several new tokens of each
 * sequence attend at once (chunked prefill, and the verification step of
 * speculative decoding on the README's roadmap), over the same block-level
 * cache and block tables as photon_paged_attn_decode (README "GPU-optimised
 * kernels": batched paged attention).  Sequence b owns query rows
 * query_start[b] .. query_start[b+1] - 1, which are the last
 * n_b = query_start[b+1] - query_start[b] of its context_lens[b] tokens
 * (already written to the cache).  Row j of sequence b is at position
 * p = context_lens[b] - n_b + j and, for query head h and KV head
 * g = h / (Hq / Hkv), gets
 *
 *   out = sum_{t <= p} exp(s_t - max s) V_t / sum_{t <= p} exp(s_t - max s),
 *   s_t = scale * <q_row_h, K_t>.
 *
 * Scores and products run on the matrix cores: fp32 storage in fp32
 * (16x16x4 MFMA), 16-bit storage with exact products and fp32 sums (16x16x16
 * MFMA); softmax weights are applied as a 16-bit value plus its 16-bit
 * rounding residual, so they carry about fp32 accuracy.
 *
 *   q             [num_tokens, num_q_heads, head_dim]     kv.dtype, 16-byte aligned
 *   k_cache, v_cache  pools (read only), 16-byte aligned
 *   block_tables  [num_seqs, max_blocks_per_seq] int32
 *   context_lens  [num_seqs] int32, n_b <= ctx <= max_blocks_per_seq * block_size
 *   query_start   [num_seqs + 1] int32, query_start[0] = 0, non-decreasing,
 *                 query_start[num_seqs] = num_tokens
 *   out           [num_tokens, num_q_heads, head_dim]     kv.dtype (fp32 with
 *                 PHOTON_DECODE_OUT_F32), 16-byte aligned
 *
 *   workspace     device scratch of at least the size the workspace query
 *                 returns (may be NULL when that is 0), 16-byte aligned
 *
 * A tile of 16 query rows whose causal range spans several splits is
 * reduced by the last of its workgroups to finish, in split order, so
 * results are deterministic.  Device-resident indices are not range-checked
 * (caller error).  num_seqs == 0 or num_tokens == 0 launches nothing.
 */
PHOTON_API photon_status photon_paged_attn_multi_query(const void *q, const void *k_cache,
                                                       const void *v_cache,
                                                       const int32_t *block_tables,
                                                       const int32_t *context_lens,
                                                       const int32_t *query_start, float scale,
                                                       const photon_multi_query_desc *desc,
                                                       void *out, void *workspace,
                                                       size_t workspace_bytes, void *stream);

/* Rotary embedding parameters of photon_rope_kv_cache_write. */
typedef struct photon_rope_desc {
    double base;            /* frequency base, finite and > 0 (10000 in the RoFormer
                               paper, 500000 for Llama 3, 1000000 for Qwen3)        */
    int32_t adjacent_pairs; /* 0: pair j is (x_j, x_{j+D/2}), the rotate-half layout
                               of Llama and GPT-NeoX; 1: pair j is (x_{2j}, x_{2j+1}),
                               the layout of the RoFormer paper and GPT-J            */
    int32_t reserved;       /* must be 0                                            */
} photon_rope_desc;

/*
 * Fused rotary position embedding and slot-mapped KV cache write (README
 * "GPU-optimised kernels": batched RoPE among the fused operations;
 * "Technical details -> Paged attention": one kernel writes the K/V rows of
 * many sequences).  For every token i at position p = positions[i] and
 * every pair j < D/2 of each head row of q and k, with
 * angle = p * base^(-2j/D) (formed in double, then rounded to fp32):
 *
 *   x'_a = x_a cos(angle) - x_b sin(angle),  x'_b = x_a sin(angle) + x_b cos(angle)
 *
 * Rotated q rows go to q_out; when slot_mapping[i] >= 0 the rotated k rows
 * and the raw v rows go to pool row (slot / block_size, h, slot % block_size)
 * of k_cache and v_cache.  The rotation is fp32 and the result is rounded to
 * nearest even in kv->dtype; v is copied bit-exactly.
 *
 *   q, q_out      [num_tokens, num_q_heads, head_dim]   kv->dtype, 16-byte aligned;
 *                 q_out may equal q (in place), must not overlap it otherwise
 *   k, v          [num_tokens, num_kv_heads, head_dim]  kv->dtype, 16-byte aligned
 *   positions     [num_tokens] int32, >= 0
 *   slot_mapping  [num_tokens] int32, as for photon_kv_cache_write
 *   k_cache, v_cache  pools, updated in place, 16-byte aligned
 *
 * num_q_heads must be > 0.  num_tokens == 0 launches nothing.  Errors as for
 * photon_kv_cache_write, plus PHOTON_ERR_INVALID_ARG for a bad rope
 * descriptor.
 */
PHOTON_API photon_status photon_rope_kv_cache_write(const void *q, void *q_out, const void *k,
                                                    const void *v, const int32_t *positions,
                                                    const int32_t *slot_mapping, int32_t num_tokens,
                                                    int32_t num_q_heads, void *k_cache,
                                                    void *v_cache, const photon_kv_desc *kv,
                                                    const photon_rope_desc *rope, void *stream);

/*
 * Token granularity of partition_tokens: the tokens of one unit of work (a
 * chunk of whole KV blocks of one sequence and KV head) for this shape.
 * Returns 0 and sets the detail message if desc is invalid or unsupported.
 */
PHOTON_API int32_t photon_paged_attn_partition_quantum(const photon_decode_desc *desc);

/*
 * Tokens per wavefront a call with this descriptor will use for the largest
 * batch it allows (resolves partition_tokens == 0).  Returns 0 if desc is
 * invalid or unsupported.
 */
PHOTON_API int32_t photon_paged_attn_partition_tokens(const photon_decode_desc *desc);

/*
 * Workspace bytes photon_paged_attn_decode needs for desc: 0 when num_seqs
 * is 0 or max_context_len is at most one partition quantum (no context is
 * then ever split), else one 64-bit arrival counter per (sequence, KV head),
 * padded to 256 bytes, then two fp32 partial records per wavefront (the
 * unnormalised output rows of the query heads of a group, then their running
 * maxima and exponential sums).  Its contents before a call do not matter
 * (see "Workspaces" above): the same workspace serves later calls of any
 * shape it is large enough for, without clearing.
 */
PHOTON_API photon_status photon_paged_attn_workspace_bytes(const photon_decode_desc *desc,
                                                           size_t *bytes);

/*
 * Batched paged-attention decode with grouped-query heads (README "GPU-
 * optimised kernels": batched paged attention, stable softmax).  For each
 * sequence b and query head h, with g = h / (Hq / Hkv), ctx = context_lens[b]
 * and K_t, V_t the rows of logical position t under KV head g:
 *
 *   s_t        = scale * <q[b][h], K_t>            for t < ctx
 *   out[b][h]  = sum_t exp(s_t - max s) V_t / sum_t exp(s_t - max s)
 *
 * A sequence with ctx == 0 gets an all-zero row.  Table entries at or past
 * ceil(ctx / block_size) and pool slots at or past ctx in the last block are
 * never read.  One kernel is launched: it splits the batch's K/V reads
 * evenly over its wavefronts, whatever the mix of context lengths; a
 * (sequence, KV head) split over several wavefronts is merged by the last of
 * them to finish, in a fixed order, so results are deterministic run to run.
 * num_seqs is at most 2048, and num_seqs * num_kv_heads * (units of
 * max_context_len + 2) at most INT32_MAX, where a unit is the kernel's
 * 16- or 32-token chunk (PHOTON_ERR_UNSUPPORTED above either).
 *
 *   q             [num_seqs, num_q_heads, head_dim]        kv.dtype, 16-byte aligned
 *   k_cache, v_cache  pools (read only), 16-byte aligned
 *   block_tables  [num_seqs, max_blocks_per_seq] int32, entries < kv.num_blocks
 *   context_lens  [num_seqs] int32, 0 <= ctx <= max_context_len (a longer
 *                 context is a caller error: with no workspace it may fault)
 *   out           [num_seqs, num_q_heads, head_dim]        kv.dtype (fp32 with
 *                 PHOTON_DECODE_OUT_F32), 16-byte aligned
 *   workspace     device scratch of workspace_bytes >= the size the workspace
 *                 query returns, 16-byte aligned, any contents; may be NULL
 *                 when that size is 0
 */
PHOTON_API photon_status photon_paged_attn_decode(const void *q, const void *k_cache, const void *v_cache,
                                       const int32_t *block_tables, const int32_t *context_lens,
                                       float scale, const photon_decode_desc *desc, void *out,
                                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * Size of the device array photon_paged_attn_decode_noalloc uses as its
 * workspace (one copy per GPU the library runs on, held until the process
 * ends).
 */
#define PHOTON_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * photon_paged_attn_decode without a workspace argument and without any
 * allocation, for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid it.  Same
 * operation, arguments, kernels and results as photon_paged_attn_decode;
 * the workspace is a static device array of PHOTON_NOALLOC_SCRATCH_BYTES
 * (32 MiB) per GPU, whose address is looked up once per device (on the
 * first call that needs it, with that device current).
 *
 *   - stream must belong to the current device.
 *   - A call whose workspace need (photon_paged_attn_workspace_bytes)
 *     exceeds PHOTON_NOALLOC_SCRATCH_BYTES returns PHOTON_ERR_WORKSPACE and
 *     launches nothing; every shape with automatic partitioning and
 *     num_seqs * num_kv_heads up to a million fits.
 *   - Every call on one GPU shares that GPU's array: calls that may overlap
 *     in time on one GPU (other streams, other threads) race and give wrong
 *     results.  Calls on one stream are ordered and safe.  Nothing in the
 *     array needs clearing between calls (see "Workspaces" above).
 */
PHOTON_API photon_status photon_paged_attn_decode_noalloc(const void *q, const void *k_cache,
                                                          const void *v_cache,
                                                          const int32_t *block_tables,
                                                          const int32_t *context_lens, float scale,
                                                          const photon_decode_desc *desc,
                                                          void *out, void *stream);

/*
 * One decode step in one launch: the cache write of each sequence's new
 * token fused with photon_paged_attn_decode (README "Technical details ->
 * Paged attention" and "GPU-optimised kernels").  For every sequence b with
 * ctx = context_lens[b] > 0, the rows k_new[b][h][:] and v_new[b][h][:] are
 * stored at the sequence's position ctx - 1, i.e. pool row
 * (block_tables[b][(ctx-1) / block_size], h, (ctx-1) % block_size), and the
 * output is then exactly that of photon_paged_attn_decode over the ctx
 * tokens, new one included.  This equals photon_kv_cache_write with
 * slot_mapping[b] = block_tables[b][(ctx-1)/bs] * bs + (ctx-1) % bs followed
 * by photon_paged_attn_decode, bit for bit.
 *
 *   k_new, v_new  [num_seqs, num_kv_heads, head_dim]   kv.dtype, 16-byte aligned
 *   k_cache, v_cache  pools, updated in place
 *   other arguments as for photon_paged_attn_decode
 *
 * Precondition (not checked): the block holding position ctx - 1 of a
 * sequence is read by no other sequence of the call (it is the block being
 * appended to).
 */
PHOTON_API photon_status photon_paged_attn_decode_step(const void *q, const void *k_new,
                                                       const void *v_new, void *k_cache,
                                                       void *v_cache, const int32_t *block_tables,
                                                       const int32_t *context_lens, float scale,
                                                       const photon_decode_desc *desc, void *out,
                                                       void *workspace, size_t workspace_bytes,
                                                       void *stream);

/* Static name of a status code. */
PHOTON_API const char *photon_status_str(photon_status status);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
PHOTON_API const char *photon_last_error_detail(void);

/* PHOTON_ABI_VERSION of the loaded library. */
PHOTON_API int32_t photon_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PHOTON_DECODE_H */
