// Slot-mapped KV cache write for gfx950 (PhotonInfer README, "Technical
// details -> Paged attention": one kernel writes the K/V rows of many
// sequences into the block-level cache).
//
// Token i with slot s >= 0 writes row k[i][h][:] to pool row
// (s / block_size, h, s % block_size) for every KV head h, and the same for
// v.  Each thread moves one 16-byte chunk of one row with integer loads and
// stores, so the copy is bit-exact (NaN payloads and subnormals included).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace photon {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void kv_cache_write_kernel(
    const u32x4 *__restrict__ k, const u32x4 *__restrict__ v, const int32_t *__restrict__ slots,
    int64_t total_chunks, u32x4 *__restrict__ k_cache, u32x4 *__restrict__ v_cache,
    int num_kv_heads, int block_size, int chunks_per_row)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total_chunks)
        return;
    const int chunk = (int)(idx % chunks_per_row);
    const int64_t row = idx / chunks_per_row;  // = token * num_kv_heads + head
    const int h = (int)(row % num_kv_heads);
    const int64_t token = row / num_kv_heads;
    const int32_t slot = slots[token];
    if (slot < 0)
        return;
    const int64_t blk = slot / block_size;
    const int64_t off = slot % block_size;
    const int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * chunks_per_row + chunk;
    k_cache[dst] = k[idx];
    v_cache[dst] = v[idx];
}

}  // namespace

hipError_t launch_kv_cache_write(const void *k, const void *v, const int32_t *slots,
                                 int num_tokens, void *k_cache, void *v_cache, int num_kv_heads,
                                 int block_size, int row_bytes, hipStream_t stream)
{
    const int chunks_per_row = row_bytes / 16;
    const int64_t total = (int64_t)num_tokens * num_kv_heads * chunks_per_row;
    const int threads = 256;
    const int64_t blocks = (total + threads - 1) / threads;
    hipLaunchKernelGGL(kv_cache_write_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                       (const u32x4 *)k, (const u32x4 *)v, slots, total, (u32x4 *)k_cache,
                       (u32x4 *)v_cache, num_kv_heads, block_size, chunks_per_row);
    return hipGetLastError();
}

}  // namespace photon
