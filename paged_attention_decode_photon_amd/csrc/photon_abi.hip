// C ABI of the decode library: argument validation, partition sizing,
// workspace sizing and launches.  Declarations and the contract of every
// entry point are in include/photon_decode.h.
//
// Every check runs before the first HIP call, so invalid arguments return
// the same status with or without a GPU, and nothing is enqueued.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "launch.h"
#include "photon_decode.h"
#include "status.h"

namespace photon {

namespace {
thread_local char g_detail[256] = "";
}  // namespace

photon_status fail(photon_status st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_detail, sizeof g_detail, fmt, ap);
    va_end(ap);
    return st;
}

photon_status ok()
{
    g_detail[0] = '\0';
    return PHOTON_OK;
}

const char *last_detail() { return g_detail; }

namespace {
std::atomic<uint32_t> g_calls{0};
}  // namespace

// Number of this call, never 0: it tags the workspace arrival counters, so
// whatever a workspace held before a call is never counted by it.  This
// process-wide counter is the library's only state.
uint32_t next_epoch()
{
    uint32_t e;
    do {
        e = g_calls.fetch_add(1, std::memory_order_relaxed) + 1;
    } while (e == 0);
    return e;
}

}  // namespace photon

namespace {

using photon::fail;
using photon::ok;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int elem_bytes_of(int32_t dtype)
{
    switch (dtype) {
    case PHOTON_F32: return 4;
    case PHOTON_F16: return 2;
    case PHOTON_BF16: return 2;
    default: return 0;
    }
}
static_assert(PHOTON_F32 == photon::kDtypeF32 && PHOTON_F16 == photon::kDtypeF16 &&
                  PHOTON_BF16 == photon::kDtypeBF16,
              "dtype codes");
constexpr int32_t kKnownDecodeFlags = PHOTON_DECODE_OUT_F32;

// Default number of decode wavefronts: enough per compute unit of an MI355X
// (256 CUs) that the chunks in flight, counting every chunk a wave keeps in
// flight, add up to 64 KiB per CU, and at least four (one per SIMD).  Each
// wave takes an equal share of the batch's units.  Counting one chunk per
// wave instead put two waves on every SIMD for 16-bit rows with two chunks
// in flight; one per SIMD is faster there (ragged f16 batch of 64:
// 27.1 -> 25.6 us), while with one chunk in flight (eight query heads per
// KV head) two per SIMD stay faster (32.2 against 34.6 us).
constexpr int64_t kComputeUnits = 256;
constexpr int64_t kBytesInFlightPerCu = 64 * 1024;
constexpr int64_t kMinWavesPerCu = 4;
// Upper bound on wavefronts, which bounds the workspace.
constexpr int64_t kMaxWaves = 1 << 20;

photon_status check_kv(const photon_kv_desc *kv)
{
    if (!kv)
        return fail(PHOTON_ERR_INVALID_ARG, "kv descriptor is NULL");
    if (kv->num_blocks <= 0 || kv->num_kv_heads <= 0 || kv->block_size <= 0 || kv->head_dim <= 0)
        return fail(PHOTON_ERR_INVALID_ARG,
                    "kv sizes must be positive (num_blocks=%d num_kv_heads=%d block_size=%d "
                    "head_dim=%d)",
                    kv->num_blocks, kv->num_kv_heads, kv->block_size, kv->head_dim);
    if (elem_bytes_of(kv->dtype) == 0)
        return fail(PHOTON_ERR_INVALID_ARG, "unknown dtype %d", kv->dtype);
    if ((int64_t)kv->num_blocks * kv->block_size > INT32_MAX)
        return fail(PHOTON_ERR_INVALID_ARG, "num_blocks * block_size exceeds the int32 slot range");
    if (kv->block_size != photon::kBlockTokens)
        return fail(PHOTON_ERR_UNSUPPORTED, "block_size %d not built (16 is)", kv->block_size);
    if (kv->head_dim != 64 && kv->head_dim != 128)
        return fail(PHOTON_ERR_UNSUPPORTED, "head_dim %d not built (64, 128 are)", kv->head_dim);
    if (kv->num_kv_heads > 65535)
        return fail(PHOTON_ERR_UNSUPPORTED, "num_kv_heads %d above the grid limit", kv->num_kv_heads);
    return PHOTON_OK;
}

struct Plan {
    int group;
    int elem_bytes;
    int quantum;      // tokens per chunk (unit of work)
    int part_tokens;  // chunk-aligned tokens per wave slice for the upper-bound batch
    int num_waves;
    size_t count_bytes;  // arrival counters, one 64-bit word per (sequence, KV head)
    size_t ws_bytes;     // total
};

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

photon_status plan_decode(const photon_decode_desc *d, Plan *plan)
{
    if (!d)
        return fail(PHOTON_ERR_INVALID_ARG, "decode descriptor is NULL");
    photon_status st = check_kv(&d->kv);
    if (st != PHOTON_OK)
        return st;
    if (d->num_seqs < 0 || d->num_q_heads <= 0 || d->max_blocks_per_seq <= 0 ||
        d->max_context_len < 0 || d->partition_tokens < 0)
        return fail(PHOTON_ERR_INVALID_ARG,
                    "bad sizes (num_seqs=%d num_q_heads=%d max_blocks_per_seq=%d "
                    "max_context_len=%d partition_tokens=%d)",
                    d->num_seqs, d->num_q_heads, d->max_blocks_per_seq, d->max_context_len,
                    d->partition_tokens);
    if (d->flags & ~kKnownDecodeFlags)
        return fail(PHOTON_ERR_INVALID_ARG, "unknown decode flags 0x%x", (unsigned)d->flags);
    if (d->num_q_heads % d->kv.num_kv_heads != 0)
        return fail(PHOTON_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d",
                    d->num_q_heads, d->kv.num_kv_heads);
    if ((int64_t)d->max_context_len > (int64_t)d->max_blocks_per_seq * d->kv.block_size)
        return fail(PHOTON_ERR_INVALID_ARG,
                    "max_context_len %d exceeds max_blocks_per_seq * block_size = %lld",
                    d->max_context_len, (long long)d->max_blocks_per_seq * d->kv.block_size);
    const int group = d->num_q_heads / d->kv.num_kv_heads;
    if (group != 1 && group != 2 && group != 4 && group != 8)
        return fail(PHOTON_ERR_UNSUPPORTED, "query heads per KV head %d not built (1, 2, 4, 8 are)",
                    group);
    if (d->num_seqs > photon::kMaxDecodeSeqs)
        return fail(PHOTON_ERR_UNSUPPORTED, "num_seqs %d above %d", d->num_seqs,
                    photon::kMaxDecodeSeqs);

    Plan p{};
    p.group = group;
    p.elem_bytes = elem_bytes_of(d->kv.dtype);
    p.quantum = photon::decode_chunk_tokens(p.elem_bytes, d->kv.head_dim, group);
    // Units of the largest batch this descriptor allows (every sequence at
    // max_context_len); the kernel splits the actual units evenly over the
    // waves, so the slice a wave gets is at most part_tokens.
    const int64_t chunks = ((int64_t)d->max_context_len + p.quantum - 1) / p.quantum;
    const int64_t upper = (int64_t)d->num_seqs * d->kv.num_kv_heads * chunks;
    if (upper + (int64_t)photon::kDecodeBoundaryUnits * d->num_seqs * d->kv.num_kv_heads > INT32_MAX)
        return fail(PHOTON_ERR_UNSUPPORTED,
                    "%lld units of work (num_seqs * num_kv_heads * chunks of max_context_len) "
                    "exceed the kernel's 32-bit indexing",
                    (long long)upper);
    int64_t waves;
    if (d->partition_tokens > 0) {
        if (d->partition_tokens % p.quantum != 0)
            return fail(PHOTON_ERR_INVALID_ARG, "partition_tokens %d is not a multiple of %d",
                        d->partition_tokens, p.quantum);
        const int64_t per_wave = d->partition_tokens / p.quantum;
        waves = (upper + per_wave - 1) / per_wave;
    } else {
        const int64_t unit_bytes = 2LL * p.quantum * d->kv.head_dim * p.elem_bytes;  // K + V
        int64_t per_cu = kBytesInFlightPerCu / (unit_bytes * photon::decode_chunks_in_flight(group));
        per_cu = per_cu < kMinWavesPerCu ? kMinWavesPerCu : per_cu;
        const int64_t auto_waves = kComputeUnits * per_cu;
        waves = upper < auto_waves ? upper : auto_waves;
    }
    if (waves > kMaxWaves)
        return fail(PHOTON_ERR_UNSUPPORTED, "%lld wavefronts needed, at most %lld",
                    (long long)waves, (long long)kMaxWaves);
    if (waves < 1)
        waves = 1;
    waves = (waves + photon::kDecodeWaves - 1) / photon::kDecodeWaves * photon::kDecodeWaves;
    p.num_waves = (int)waves;
    const int64_t per_wave = upper > 0 ? (upper + waves - 1) / waves : 1;
    p.part_tokens = (int)(per_wave * p.quantum);
    // A segment of one unit is never split, so calls whose contexts all fit
    // in one unit need no workspace.
    if (d->num_seqs > 0 && chunks > 1) {
        const size_t rec = (size_t)photon::decode_record_floats(d->kv.head_dim, group) * sizeof(float);
        p.count_bytes = align256((size_t)d->num_seqs * d->kv.num_kv_heads * sizeof(uint64_t));
        p.ws_bytes = p.count_bytes + (size_t)waves * 2 * rec;
    }
    *plan = p;
    return PHOTON_OK;
}

struct MqPlan {
    int group;
    int max_tiles;
    int split_blocks;
    int num_splits;
    size_t count_bytes;
    size_t ws_bytes;
};

// Automatic KV splitting of the multi-query kernel aims at this many
// workgroups (four per compute unit of an MI355X).
constexpr int64_t kMqTargetGroups = 1024;
// ... but no split shorter than 32 blocks: each wave then runs at least four
// blocks, two at a time (measured best for 16-bit 4-token verification at
// batch 16) ...
constexpr int64_t kMqMinSplitBlocks = 32;
// ... or 16 blocks for fp32 storage in the per-tile kernel, whose blocks take
// twice the bytes (4-token verification at batch 16: 26.5 -> 25.5 us).
constexpr int64_t kMqMinSplitBlocksF32 = 16;
// ... and none longer than 64 blocks (1024 tokens): a long prompt chunk at a
// long context is then spread over several workgroups.
constexpr int64_t kMqMaxSplitBlocks = 64;

photon_status plan_multi_query(const photon_multi_query_desc *d, MqPlan *plan)
{
    if (!d)
        return fail(PHOTON_ERR_INVALID_ARG, "multi-query descriptor is NULL");
    photon_status st = check_kv(&d->kv);
    if (st != PHOTON_OK)
        return st;
    if (d->num_seqs < 0 || d->num_tokens < 0 || d->num_q_heads <= 0 || d->max_blocks_per_seq <= 0 ||
        d->max_query_len < 0 || d->max_context_len < 0 || d->split_tokens < 0)
        return fail(PHOTON_ERR_INVALID_ARG,
                    "bad sizes (num_seqs=%d num_tokens=%d num_q_heads=%d max_blocks_per_seq=%d "
                    "max_query_len=%d max_context_len=%d split_tokens=%d)",
                    d->num_seqs, d->num_tokens, d->num_q_heads, d->max_blocks_per_seq,
                    d->max_query_len, d->max_context_len, d->split_tokens);
    if (d->flags & ~kKnownDecodeFlags)
        return fail(PHOTON_ERR_INVALID_ARG, "unknown flags 0x%x", (unsigned)d->flags);
    if (d->num_q_heads % d->kv.num_kv_heads != 0)
        return fail(PHOTON_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d",
                    d->num_q_heads, d->kv.num_kv_heads);
    const int group = d->num_q_heads / d->kv.num_kv_heads;
    if (group != 1 && group != 2 && group != 4 && group != 8)
        return fail(PHOTON_ERR_UNSUPPORTED, "query heads per KV head %d not built (1, 2, 4, 8 are)",
                    group);
    if ((int64_t)d->num_seqs * d->kv.num_kv_heads > 65535)
        return fail(PHOTON_ERR_UNSUPPORTED, "num_seqs * num_kv_heads %lld above 65535",
                    (long long)d->num_seqs * d->kv.num_kv_heads);
    if (d->max_query_len > d->num_tokens)
        return fail(PHOTON_ERR_INVALID_ARG, "max_query_len %d exceeds num_tokens %d",
                    d->max_query_len, d->num_tokens);
    if ((int64_t)d->max_context_len > (int64_t)d->max_blocks_per_seq * d->kv.block_size)
        return fail(PHOTON_ERR_INVALID_ARG,
                    "max_context_len %d exceeds max_blocks_per_seq * block_size = %lld",
                    d->max_context_len, (long long)d->max_blocks_per_seq * d->kv.block_size);
    if (d->split_tokens % 64 != 0)
        return fail(PHOTON_ERR_INVALID_ARG, "split_tokens %d is not a multiple of 64",
                    d->split_tokens);
    MqPlan p{};
    p.group = group;
    p.max_tiles = (int)(((int64_t)d->max_query_len * group + 15) / 16);
    const int64_t tiles = (int64_t)d->num_seqs * d->kv.num_kv_heads * p.max_tiles;
    const int64_t max_nblk = ((int64_t)d->max_context_len + d->kv.block_size - 1) / d->kv.block_size;
    int64_t sb;
    if (d->split_tokens > 0) {
        sb = d->split_tokens / d->kv.block_size;
    } else {
        const int64_t want = tiles > 0 ? (kMqTargetGroups + tiles - 1) / tiles : 1;
        sb = want > 1 ? (max_nblk + want - 1) / want : max_nblk;
        // whole steps: every wave of a workgroup two blocks
        const int64_t step = 2 * (p.max_tiles < photon::kWideTiles ? photon::kMqTileWaves : 4);
        sb = (sb + step - 1) / step * step;
        const int64_t min_sb = elem_bytes_of(d->kv.dtype) == 4 && p.max_tiles < photon::kWideTiles
                                   ? kMqMinSplitBlocksF32
                                   : kMqMinSplitBlocks;
        sb = sb < min_sb ? min_sb : sb;
        sb = sb > kMqMaxSplitBlocks ? kMqMaxSplitBlocks : sb;
    }
    const int64_t splits = max_nblk > sb ? (max_nblk + sb - 1) / sb : 1;
    if (splits > 65535)
        return fail(PHOTON_ERR_UNSUPPORTED, "%lld KV splits, at most 65535", (long long)splits);
    p.split_blocks = (int)(sb > INT32_MAX ? INT32_MAX : sb);
    p.num_splits = (int)splits;
    if (splits > 1 && tiles > 0) {
        const size_t rec = (size_t)16 * (d->kv.head_dim + 2) * sizeof(float);
        p.count_bytes = align256((size_t)tiles * sizeof(uint64_t));
        p.ws_bytes = p.count_bytes + (size_t)tiles * splits * rec;
    }
    *plan = p;
    return PHOTON_OK;
}

}  // namespace

extern "C" {

photon_status photon_kv_cache_write(const void *k, const void *v, const int32_t *slot_mapping,
                                    int32_t num_tokens, void *k_cache, void *v_cache,
                                    const photon_kv_desc *kv, void *stream)
{
    photon_status st = check_kv(kv);
    if (st != PHOTON_OK)
        return st;
    if (num_tokens < 0)
        return fail(PHOTON_ERR_INVALID_ARG, "num_tokens %d is negative", num_tokens);
    if (num_tokens == 0)
        return ok();
    if (!k || !v || !slot_mapping || !k_cache || !v_cache)
        return fail(PHOTON_ERR_INVALID_ARG, "NULL data pointer");
    if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
        return fail(PHOTON_ERR_INVALID_ARG, "k, v and the pools must be 16-byte aligned");
    if (!aligned4(slot_mapping))
        return fail(PHOTON_ERR_INVALID_ARG, "slot_mapping must be 4-byte aligned");
    const int row_bytes = kv->head_dim * elem_bytes_of(kv->dtype);
    hipError_t err = photon::launch_kv_cache_write(k, v, slot_mapping, num_tokens, k_cache, v_cache,
                                                   kv->num_kv_heads, kv->block_size, row_bytes,
                                                   (hipStream_t)stream);
    if (err != hipSuccess)
        return fail(PHOTON_ERR_HIP, "kv cache write launch: %s", hipGetErrorString(err));
    return ok();
}

photon_status photon_paged_attn_multi_query_workspace_bytes(const photon_multi_query_desc *d,
                                                           size_t *bytes)
{
    if (!bytes)
        return fail(PHOTON_ERR_INVALID_ARG, "bytes is NULL");
    MqPlan p;
    photon_status st = plan_multi_query(d, &p);
    if (st != PHOTON_OK)
        return st;
    *bytes = p.ws_bytes;
    return ok();
}

photon_status photon_paged_attn_multi_query(const void *q, const void *k_cache, const void *v_cache,
                                           const int32_t *block_tables, const int32_t *context_lens,
                                           const int32_t *query_start, float scale,
                                           const photon_multi_query_desc *d, void *out,
                                           void *workspace, size_t workspace_bytes, void *stream)
{
    MqPlan p;
    photon_status st = plan_multi_query(d, &p);
    if (st != PHOTON_OK)
        return st;
    if (!std::isfinite(scale))
        return fail(PHOTON_ERR_INVALID_ARG, "scale is not finite");
    if (d->num_seqs == 0 || d->num_tokens == 0 || d->max_query_len == 0)
        return ok();
    if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start || !out)
        return fail(PHOTON_ERR_INVALID_ARG, "NULL data pointer");
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
        return fail(PHOTON_ERR_INVALID_ARG, "q, the pools and out must be 16-byte aligned");
    if (!aligned4(block_tables) || !aligned4(context_lens) || !aligned4(query_start))
        return fail(PHOTON_ERR_INVALID_ARG, "index arrays must be 4-byte aligned");
    if (workspace_bytes < p.ws_bytes)
        return fail(PHOTON_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes,
                    p.ws_bytes);
    if (p.ws_bytes && (!workspace || !aligned16(workspace)))
        return fail(PHOTON_ERR_INVALID_ARG, "workspace must be non-NULL and 16-byte aligned");
    photon::MultiQueryArgs a{};
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.query_start = query_start;
    a.out = out;
    a.num_seqs = d->num_seqs;
    a.num_kv_heads = d->kv.num_kv_heads;
    a.group = p.group;
    a.head_dim = d->kv.head_dim;
    a.max_blocks = d->max_blocks_per_seq;
    a.max_tiles = p.max_tiles;
    a.split_blocks = p.split_blocks;
    a.num_splits = p.num_splits;
    char *ws = static_cast<char *>(workspace);
    a.ws_count = p.ws_bytes ? reinterpret_cast<uint64_t *>(ws) : nullptr;
    a.ws_rec = p.ws_bytes ? reinterpret_cast<float *>(ws + p.count_bytes) : nullptr;
    a.dtype = d->kv.dtype;
    a.out_f32 = (d->flags & PHOTON_DECODE_OUT_F32) ? 1 : 0;
    a.qscale = (float)((double)scale * 1.4426950408889634);  // log2(e)
    a.epoch = photon::next_epoch();
    hipError_t err = photon::launch_paged_multi_query(a, (hipStream_t)stream);
    if (err != hipSuccess)
        return fail(PHOTON_ERR_HIP, "multi-query launch: %s", hipGetErrorString(err));
    return ok();
}

photon_status photon_rope_kv_cache_write(const void *q, void *q_out, const void *k, const void *v,
                                         const int32_t *positions, const int32_t *slot_mapping,
                                         int32_t num_tokens, int32_t num_q_heads, void *k_cache,
                                         void *v_cache, const photon_kv_desc *kv,
                                         const photon_rope_desc *rope, void *stream)
{
    photon_status st = check_kv(kv);
    if (st != PHOTON_OK)
        return st;
    if (!rope)
        return fail(PHOTON_ERR_INVALID_ARG, "rope descriptor is NULL");
    if (!std::isfinite(rope->base) || !(rope->base > 0.0))
        return fail(PHOTON_ERR_INVALID_ARG, "rope base %g must be finite and positive", rope->base);
    if ((rope->adjacent_pairs != 0 && rope->adjacent_pairs != 1) || rope->reserved != 0)
        return fail(PHOTON_ERR_INVALID_ARG, "rope adjacent_pairs must be 0 or 1, reserved 0");
    if (num_tokens < 0 || num_q_heads <= 0)
        return fail(PHOTON_ERR_INVALID_ARG, "num_tokens %d must be >= 0, num_q_heads %d > 0",
                    num_tokens, num_q_heads);
    if (num_tokens == 0)
        return ok();
    if (!q || !q_out || !k || !v || !positions || !slot_mapping || !k_cache || !v_cache)
        return fail(PHOTON_ERR_INVALID_ARG, "NULL data pointer");
    if (!aligned16(q) || !aligned16(q_out) || !aligned16(k) || !aligned16(v) ||
        !aligned16(k_cache) || !aligned16(v_cache))
        return fail(PHOTON_ERR_INVALID_ARG, "q, q_out, k, v and the pools must be 16-byte aligned");
    if (!aligned4(positions) || !aligned4(slot_mapping))
        return fail(PHOTON_ERR_INVALID_ARG, "positions and slot_mapping must be 4-byte aligned");
    const size_t q_bytes = (size_t)num_tokens * num_q_heads * kv->head_dim * elem_bytes_of(kv->dtype);
    const char *qb = static_cast<const char *>(q), *ob = static_cast<const char *>(q_out);
    if (qb != ob && qb < ob + q_bytes && ob < qb + q_bytes)
        return fail(PHOTON_ERR_INVALID_ARG, "q_out overlaps q without being equal to it");
    photon::RopeArgs a{};
    a.q = q;
    a.q_out = q_out;
    a.k = k;
    a.v = v;
    a.positions = positions;
    a.slot_mapping = slot_mapping;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.base = rope->base;
    a.num_tokens = num_tokens;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = kv->num_kv_heads;
    a.head_dim = kv->head_dim;
    a.block_size = kv->block_size;
    a.dtype = kv->dtype;
    a.adjacent_pairs = rope->adjacent_pairs;
    hipError_t err = photon::launch_rope_kv_cache_write(a, (hipStream_t)stream);
    if (err != hipSuccess)
        return fail(PHOTON_ERR_HIP, "rope cache write launch: %s", hipGetErrorString(err));
    return ok();
}

int32_t photon_paged_attn_partition_quantum(const photon_decode_desc *desc)
{
    Plan p;
    return plan_decode(desc, &p) == PHOTON_OK ? p.quantum : 0;
}

int32_t photon_paged_attn_partition_tokens(const photon_decode_desc *desc)
{
    Plan p;
    return plan_decode(desc, &p) == PHOTON_OK ? p.part_tokens : 0;
}

photon_status photon_paged_attn_workspace_bytes(const photon_decode_desc *desc, size_t *bytes)
{
    if (!bytes)
        return fail(PHOTON_ERR_INVALID_ARG, "bytes is NULL");
    Plan p;
    photon_status st = plan_decode(desc, &p);
    if (st != PHOTON_OK)
        return st;
    *bytes = p.ws_bytes;
    return ok();
}

}  // extern "C"

// Workspace of photon_paged_attn_decode_noalloc: a fixed device array, one
// copy per GPU, held until the process ends.  Host code never uses this name
// as an address (on the host it is only a stand-in for the device symbol);
// the device address of each GPU's copy comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[PHOTON_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 256;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxScratchDevices];  // device address of `scratch` per device, once known

// Device address of the current device's copy of `scratch`, looked up once
// per device with that device current.
photon_status current_device_scratch(void **ptr)
{
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return fail(PHOTON_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(err));
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(PHOTON_ERR_UNSUPPORTED, "device %d above the %d the scratch table holds", dev,
                    kMaxScratchDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess || !p)
            return fail(PHOTON_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        hipGetErrorString(err));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return PHOTON_OK;
}

photon_status decode_impl(const void *q, const void *k_new, const void *v_new, const void *k_cache,
                          const void *v_cache, const int32_t *block_tables,
                          const int32_t *context_lens, float scale, const photon_decode_desc *desc,
                          void *out, void *workspace, size_t workspace_bytes, void *stream,
                          bool static_scratch = false)
{
    Plan p;
    photon_status st = plan_decode(desc, &p);
    if (st != PHOTON_OK)
        return st;
    if (desc->num_seqs == 0)
        return ok();
    if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out)
        return fail(PHOTON_ERR_INVALID_ARG, "NULL data pointer");
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
        return fail(PHOTON_ERR_INVALID_ARG, "q, the pools and out must be 16-byte aligned");
    if (!aligned4(block_tables) || !aligned4(context_lens))
        return fail(PHOTON_ERR_INVALID_ARG, "block_tables and context_lens must be 4-byte aligned");
    if (!std::isfinite(scale))
        return fail(PHOTON_ERR_INVALID_ARG, "scale is not finite");
    if (static_scratch) {
        if (p.ws_bytes > (size_t)PHOTON_NOALLOC_SCRATCH_BYTES)
            return fail(PHOTON_ERR_WORKSPACE,
                        "this call needs %zu bytes of workspace, the static scratch holds %zu",
                        p.ws_bytes, (size_t)PHOTON_NOALLOC_SCRATCH_BYTES);
        workspace = nullptr;
        workspace_bytes = 0;
        if (p.ws_bytes) {  // first HIP call of the path, after every check
            st = current_device_scratch(&workspace);
            if (st != PHOTON_OK)
                return st;
            workspace_bytes = PHOTON_NOALLOC_SCRATCH_BYTES;
        }
    }
    if (workspace_bytes < p.ws_bytes)
        return fail(PHOTON_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes,
                    p.ws_bytes);
    if (p.ws_bytes && (!workspace || !aligned16(workspace)))
        return fail(PHOTON_ERR_INVALID_ARG, "workspace must be non-NULL and 16-byte aligned");

    photon::DecodeArgs a{};
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.k_new = k_new;
    a.v_new = v_new;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.out = out;
    char *ws = static_cast<char *>(workspace);
    a.ws_count = p.ws_bytes ? reinterpret_cast<uint64_t *>(ws) : nullptr;
    a.ws_rec = p.ws_bytes ? reinterpret_cast<float *>(ws + p.count_bytes) : nullptr;
    a.num_seqs = desc->num_seqs;
    a.num_kv_heads = desc->kv.num_kv_heads;
    a.group = p.group;
    a.head_dim = desc->kv.head_dim;
    a.elem_bytes = p.elem_bytes;
    a.dtype = desc->kv.dtype;
    a.out_f32 = (desc->flags & PHOTON_DECODE_OUT_F32) ? 1 : 0;
    a.max_blocks = desc->max_blocks_per_seq;
    a.num_waves = p.num_waves;
    a.qscale = (float)((double)scale * 1.4426950408889634);  // log2(e)
    a.epoch = photon::next_epoch();
    hipError_t err = photon::launch_paged_decode(a, (hipStream_t)stream);
    if (err != hipSuccess)
        return fail(PHOTON_ERR_HIP, "decode launch: %s", hipGetErrorString(err));
    return ok();
}

}  // namespace

extern "C" {

photon_status photon_paged_attn_decode(const void *q, const void *k_cache, const void *v_cache,
                                       const int32_t *block_tables, const int32_t *context_lens,
                                       float scale, const photon_decode_desc *desc, void *out,
                                       void *workspace, size_t workspace_bytes, void *stream)
{
    return decode_impl(q, nullptr, nullptr, k_cache, v_cache, block_tables, context_lens, scale,
                       desc, out, workspace, workspace_bytes, stream);
}

photon_status photon_paged_attn_decode_noalloc(const void *q, const void *k_cache,
                                               const void *v_cache, const int32_t *block_tables,
                                               const int32_t *context_lens, float scale,
                                               const photon_decode_desc *desc, void *out,
                                               void *stream)
{
    return decode_impl(q, nullptr, nullptr, k_cache, v_cache, block_tables, context_lens, scale,
                       desc, out, nullptr, 0, stream, true);
}

photon_status photon_paged_attn_decode_step(const void *q, const void *k_new, const void *v_new,
                                            void *k_cache, void *v_cache,
                                            const int32_t *block_tables,
                                            const int32_t *context_lens, float scale,
                                            const photon_decode_desc *desc, void *out,
                                            void *workspace, size_t workspace_bytes, void *stream)
{
    if (desc && desc->num_seqs > 0) {
        if (!k_new || !v_new)
            return fail(PHOTON_ERR_INVALID_ARG, "k_new and v_new must not be NULL");
        if (!aligned16(k_new) || !aligned16(v_new))
            return fail(PHOTON_ERR_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
    }
    return decode_impl(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale, desc,
                       out, workspace, workspace_bytes, stream);
}

const char *photon_status_str(photon_status status)
{
    switch (status) {
    case PHOTON_OK: return "PHOTON_OK";
    case PHOTON_ERR_INVALID_ARG: return "PHOTON_ERR_INVALID_ARG";
    case PHOTON_ERR_UNSUPPORTED: return "PHOTON_ERR_UNSUPPORTED";
    case PHOTON_ERR_WORKSPACE: return "PHOTON_ERR_WORKSPACE";
    case PHOTON_ERR_HIP: return "PHOTON_ERR_HIP";
    }
    return "PHOTON_UNKNOWN_STATUS";
}

const char *photon_last_error_detail(void) { return photon::last_detail(); }

int32_t photon_abi_version(void) { return PHOTON_ABI_VERSION; }

}  // extern "C"
