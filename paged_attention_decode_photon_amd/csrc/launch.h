// Internal launch interface between the C ABI (photon_abi.hip) and the kernel
// translation units.  Not installed; the public interface is photon_decode.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace photon {

constexpr int kBlockTokens = 16;     // tokens per KV block the decode kernels are built for
constexpr int kDecodeWaves = 4;      // wavefronts per decode workgroup

// KV blocks one decode wavefront loads per loop step.  Two blocks while the
// per-lane partial scores stay at <= 32 registers and a row is <= 256 bytes,
// else one.
constexpr int decode_chunk_blocks(int elem_bytes, int head_dim, int group)
{
    return (head_dim * elem_bytes <= 256 && (head_dim * elem_bytes / 64) * group <= 16) ? 2 : 1;
}

// Tokens one decode wavefront handles per loop step (the partition quantum).
constexpr int decode_chunk_tokens(int elem_bytes, int head_dim, int group)
{
    return decode_chunk_blocks(elem_bytes, head_dim, group) * kBlockTokens;
}

struct DecodeArgs {
    const void *q;
    const void *k_cache;
    const void *v_cache;
    const int32_t *block_tables;
    const int32_t *context_lens;
    void *out;
    float *ws_ml;  // [B][Hq][max_parts][2] (running max in log2 units, exp sum)
    float *ws_o;   // [B][Hq][max_parts][D] unnormalised partial outputs
    int num_seqs;
    int num_kv_heads;
    int group;
    int head_dim;
    int elem_bytes;
    int max_blocks;
    int part_tokens;
    int max_parts;
    float qscale;  // scale * log2(e)
};

// Partition kernel (and, when max_parts > 1, the merge kernel) on stream.
hipError_t launch_paged_decode(const DecodeArgs &a, hipStream_t stream);

hipError_t launch_kv_cache_write(const void *k, const void *v, const int32_t *slots,
                                 int num_tokens, void *k_cache, void *v_cache, int num_kv_heads,
                                 int block_size, int row_bytes, hipStream_t stream);

}  // namespace photon
