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
    u32x4 *__restrict__ k_cache, u32x4 *__restrict__ v_cache, int num_kv_heads, int block_size,
    int chunks_per_row)
{
    // Block x = token (so its slot is a wave-uniform scalar load); y and the
    // thread index cover that token's (head, 16-byte chunk) pairs.
    const int64_t token = blockIdx.x;
    const int i = blockIdx.y * blockDim.x + threadIdx.x;
    const int per_token = num_kv_heads * chunks_per_row;
    if (i >= per_token)
        return;
    const int64_t src = token * per_token + i;
    const u32x4 kr = k[src];
    const u32x4 vr = v[src];
    const int32_t slot = slots[token];
    // Keep the row loads in flight together with the slot load rather than
    // letting the compiler sink them below the slot test.
    asm volatile("" ::"v"(kr), "v"(vr), "s"(slot));
    if (slot < 0)
        return;
    const int h = i / chunks_per_row;
    const int chunk = i - h * chunks_per_row;
    const int64_t blk = slot / block_size;
    const int64_t off = slot - blk * block_size;
    const int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * chunks_per_row + chunk;
    k_cache[dst] = kr;
    v_cache[dst] = vr;
}

}  // namespace

hipError_t launch_kv_cache_write(const void *k, const void *v, const int32_t *slots,
                                 int num_tokens, void *k_cache, void *v_cache, int num_kv_heads,
                                 int block_size, int row_bytes, hipStream_t stream)
{
    const int chunks_per_row = row_bytes / 16;
    const int threads = 256;
    const int per_token = num_kv_heads * chunks_per_row;
    const dim3 grid((unsigned)num_tokens, (unsigned)((per_token + threads - 1) / threads));
    hipLaunchKernelGGL(kv_cache_write_kernel, grid, dim3(threads), 0, stream, (const u32x4 *)k,
                       (const u32x4 *)v, slots, (u32x4 *)k_cache, (u32x4 *)v_cache, num_kv_heads,
                       block_size, chunks_per_row);
    return hipGetLastError();
}

}  // namespace photon
