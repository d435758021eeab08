// Internal launch interface between the C ABI (photon_abi.hip) and the kernel
// translation units.  Not installed; the public interface is photon_decode.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace photon {

// Build-time tuning knobs of the decode kernel (defaults are the tuned values).
#ifndef PHOTON_DECODE_WAVES
#define PHOTON_DECODE_WAVES 4    // wavefronts per decode workgroup
#endif
#ifndef PHOTON_K_LOAD_AUX
#define PHOTON_K_LOAD_AUX 0      // cache-policy bits of the decode K loads
#endif
#ifndef PHOTON_V_LOAD_AUX
#define PHOTON_V_LOAD_AUX 2      // ... and of the V loads (2: the nt bit, see below)
#endif
#ifndef PHOTON_DECODE_CHUNK_BLOCKS
#define PHOTON_DECODE_CHUNK_BLOCKS 0  // KV blocks per unit of work; 0: shape rule below
#endif

// Storage types (the values of photon_dtype).
constexpr int kDtypeF32 = 0;
constexpr int kDtypeF16 = 1;
constexpr int kDtypeBF16 = 2;

constexpr int kBlockTokens = 16;     // tokens per KV block the decode kernels are built for
constexpr int kDecodeWaves = PHOTON_DECODE_WAVES;

// KV blocks one decode wavefront loads per loop step.  Two blocks while the
// per-lane partial scores stay at <= 32 registers and a row is <= 256 bytes,
// else one.
constexpr int decode_chunk_blocks(int elem_bytes, int head_dim, int group)
{
    return PHOTON_DECODE_CHUNK_BLOCKS > 0 ? PHOTON_DECODE_CHUNK_BLOCKS
           : (head_dim * elem_bytes <= 256 && (head_dim * elem_bytes / 64) * group <= 16) ? 2
                                                                                           : 1;
}

// Chunks a decode wavefront keeps in flight: two register sets alternate
// (the next chunk loads while the current one is used), except with eight
// query heads per KV head, where a second set would cost occupancy.
constexpr int decode_chunks_in_flight(int group) { return group < 8 ? 2 : 1; }

// Cache-policy bits of the decode kernel's K and V loads: V non-temporal
// (the nt bit), K default.  Measured per call (fused step, both orders): nt
// on V alone is 1-8% faster on every shape tried (f32 and 16-bit, head_dim
// 64 and 128, two to eight query heads per KV head, batch 1 to 8 x 32K
// tokens); nt on K as well gains a little more with four query heads per
// KV head at f32 and loses 10-30% with two.
constexpr int kDecodeKLoadAux = PHOTON_K_LOAD_AUX;
constexpr int kDecodeVLoadAux = PHOTON_V_LOAD_AUX;

// Tokens one decode wavefront handles per loop step (the partition quantum).
constexpr int decode_chunk_tokens(int elem_bytes, int head_dim, int group)
{
    return decode_chunk_blocks(elem_bytes, head_dim, group) * kBlockTokens;
}

// Floats of one partial record: the unnormalised output rows of the group's
// query heads, then the running max and the exponential sum of each; padded
// to a multiple of four floats.
constexpr int decode_record_floats(int head_dim, int group)
{
    return (2 * group + group * head_dim + 3) & ~3;
}

// Multi-query calls whose longest query run spans at least this many
// 16-row tiles use the wide kernel (four tiles per workgroup sharing each
// K/V block through LDS); shorter ones the per-tile kernel.
#ifndef PHOTON_MQ_WIDE_TILES
#define PHOTON_MQ_WIDE_TILES 4
#endif
constexpr int kWideTiles = PHOTON_MQ_WIDE_TILES;
// Wavefronts per workgroup of the per-tile multi-query kernel (each takes
// every kMqTileWaves-th block of the workgroup's split).  Four-token
// verification at batch 16 at its best split, fp32 / bf16: 1 wave 29.8 /
// 23.7 us, 2 waves 26.5 / 19.1 us, 4 waves 25.0 / 16.7 us.
#ifndef PHOTON_MQ_TILE_WAVES
#define PHOTON_MQ_TILE_WAVES 4
#endif
constexpr int kMqTileWaves = PHOTON_MQ_TILE_WAVES;

// Sequences per call: the decode kernel keeps per-sequence prefix sums in LDS.
constexpr int kMaxDecodeSeqs = 2048;

// Empty units charged at the start of each non-empty segment in the decode
// kernel's split of larger calls (the kernel explains the choice).  The
// charged list of units is indexed with 32-bit integers.
constexpr int kDecodeBoundaryUnits = 2;

struct DecodeArgs {
    const void *q;
    const void *k_cache;
    const void *v_cache;
    const void *k_new;  // fused decode step: rows appended at position ctx-1; NULL otherwise
    const void *v_new;
    const int32_t *block_tables;
    const int32_t *context_lens;
    void *out;
    uint64_t *ws_count;  // [B][Hkv] epoch-tagged arrival counters (arrival.h)
    float *ws_rec;  // [num_waves][2] partial records of decode_record_floats each
    int num_seqs;
    int num_kv_heads;
    int group;
    int head_dim;
    int elem_bytes;
    int dtype;      // kDtype* of q and the pools
    int out_f32;    // 1: out is fp32 whatever the storage type
    int max_blocks;
    int num_waves;  // wavefronts launched; a multiple of kDecodeWaves
    float qscale;   // scale * log2(e)
    uint32_t epoch; // this call's number (never 0): tags the arrival counters
};

// One decode launch on stream (partitions merge inside the same kernel).
hipError_t launch_paged_decode(const DecodeArgs &a, hipStream_t stream);

struct MultiQueryArgs {
    const void *q;
    const void *k_cache;
    const void *v_cache;
    const int32_t *block_tables;
    const int32_t *context_lens;
    const int32_t *query_start;
    void *out;
    int num_seqs;
    int num_kv_heads;
    int group;
    int head_dim;
    int max_blocks;
    int max_tiles;  // ceil(max_query_len * group / 16): grid x
    int split_blocks;  // KV blocks per split of a tile's causal range
    int num_splits;    // grid z: splits of the longest range
    uint64_t *ws_count;  // [B * Hkv * max_tiles] epoch-tagged arrival counters (arrival.h)
    float *ws_rec;     // [B * Hkv * max_tiles * num_splits] records of 16 * (D + 2) floats
    int dtype;
    int out_f32;
    float qscale;   // scale * log2(e)
    uint32_t epoch; // this call's number (never 0): tags the arrival counters
};

// Multi-query paged attention with a causal tail, one launch.
hipError_t launch_paged_multi_query(const MultiQueryArgs &a, hipStream_t stream);

struct RopeArgs {
    const void *q;
    void *q_out;  // may equal q
    const void *k;
    const void *v;
    const int32_t *positions;
    const int32_t *slot_mapping;
    void *k_cache;
    void *v_cache;
    double base;
    int num_tokens;
    int num_q_heads;
    int num_kv_heads;
    int head_dim;
    int block_size;
    int dtype;
    int adjacent_pairs;  // 1: pairs (2j, 2j+1); 0: pairs (j, j + D/2)
};

// Rotary embedding of q and k, then the slot-mapped write of rotated k and v.
hipError_t launch_rope_kv_cache_write(const RopeArgs &a, hipStream_t stream);

hipError_t launch_kv_cache_write(const void *k, const void *v, const int32_t *slots,
                                 int num_tokens, void *k_cache, void *v_cache, int num_kv_heads,
                                 int block_size, int row_bytes, hipStream_t stream);

}  // namespace photon
