// Bandwidth probes for gfx950: a contiguous streaming read, and a bare
// gather of the K/V rows of a paged decode call (PhotonInfer README,
// "Technical details -> Paged attention": block-level cache read through
// per-sequence tables).  Neither does any attention arithmetic: every 32-bit
// word read is XOR-folded into one value per wavefront, so their durations
// bound what a decode kernel reading the same bytes can reach.
//
// Both use the decode kernel's memory instructions (16-byte raw buffer
// loads, range-checked descriptors) and keep 16 KiB of loads in flight per
// wavefront (two alternating 8 KiB register sets).  The gather splits the
// sequence-major list of (sequence, KV head, block) tiles evenly over the
// wavefronts, like the decode kernel's balanced split, and resolves up to
// 64 tiles at a time with one table load per lane.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "elem.h"
#include "lane_ops.h"
#include "photon_probe.h"
#include "status.h"

namespace photon {
namespace {

constexpr int kRawBufferWord3 = 0x00020000;  // raw, unswizzled buffer (gfx9 family)
constexpr int kProbeWaves = 4;               // wavefronts per workgroup
constexpr int kSetLoads = 8;                 // 16-byte loads per lane per register set (8 KiB/wave)
constexpr int kMaxProbeSeqs = 64;
constexpr int64_t kMaxProbeWaves = 1 << 20;

__device__ __forceinline__ uint32_t fold(const u32x4 &v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

__device__ __forceinline__ void store_wave_xor(uint32_t acc, uint32_t *sink, int wave)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        acc ^= __shfl_xor(acc, m, 64);
    if ((threadIdx.x & 63) == 0)
        sink[wave] = acc;
}

__global__ __launch_bounds__(kProbeWaves * 64) void stream_read_kernel(const char *buf,
                                                                       uint64_t chunks,
                                                                       int num_waves,
                                                                       uint32_t *sink)
{
    const int lane = threadIdx.x & 63;
    const int wave = blockIdx.x * kProbeWaves + (threadIdx.x >> 6);
    // The wave's contiguous share of the 16-byte chunks; loads past its end
    // return zero (the descriptor's range), so no tail handling is needed.
    const uint64_t c0 = (uint64_t)wave * chunks / num_waves;
    const uint64_t c1 = (uint64_t)(wave + 1) * chunks / num_waves;
    const uint32_t bytes = (uint32_t)((c1 - c0) * 16);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void *)(buf + c0 * 16), (short)0, bytes, kRawBufferWord3);
    constexpr uint32_t kSetBytes = kSetLoads * 64 * 16;
    u32x4 a[kSetLoads], b[kSetLoads];
    uint32_t acc = 0;
    auto issue = [&](uint32_t off, u32x4(&d)[kSetLoads]) {
#pragma unroll
        for (int i = 0; i < kSetLoads; ++i)
            d[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off + (i * 64 + lane) * 16, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto consume = [&](const u32x4(&d)[kSetLoads]) {
#pragma unroll
        for (int i = 0; i < kSetLoads; ++i)
            acc ^= fold(d[i]);
    };
    if (bytes > 0)
        issue(0, a);
    for (uint32_t off = 0; off < bytes;) {
        if (off + kSetBytes < bytes)
            issue(off + kSetBytes, b);
        consume(a);
        off += kSetBytes;
        if (off >= bytes)
            break;
        if (off + kSetBytes < bytes)
            issue(off + kSetBytes, a);
        consume(b);
        off += kSetBytes;
    }
    store_wave_xor(acc, sink, wave);
}

struct GatherArgs {
    const char *k_cache;
    const char *v_cache;
    const int32_t *block_tables;
    const int32_t *context_lens;
    uint32_t *sink;
    int num_seqs;
    int num_kv_heads;
    int max_blocks;
    int num_waves;
};

// RB: bytes of one K/V row.  A 16-row tile is TL = RB / 64 wave-wide
// 16-byte loads; a register set holds TS = kSetLoads / (2 TL) tiles of K and
// V (or half a tile when RB = 512).
template <int RB>
__global__ __launch_bounds__(kProbeWaves * 64) void gather_kernel(GatherArgs a)
{
    constexpr int TL = RB / 64;                       // loads per tile, each of K and V
    constexpr int TS = kSetLoads / (2 * TL) > 0 ? kSetLoads / (2 * TL) : 1;  // tiles per set
    constexpr int SL = TS * 2 * TL;                   // loads per set
    const int lane = threadIdx.x & 63;
    const int wave = blockIdx.x * kProbeWaves + (threadIdx.x >> 6);
    const int B = a.num_seqs;
    const int hkv = a.num_kv_heads;

    // Tiles per sequence (Hkv * blocks), prefix-summed across lanes.
    const int cl = lane < B ? a.context_lens[lane] : 0;
    const int nb = (cl + 15) / 16;
    const int end = wave_inclusive_sum(hkv * nb);
    const int total = B > 0 ? __builtin_amdgcn_readlane(end, B - 1) : 0;
    const int u0 = (int)((int64_t)wave * total / a.num_waves);
    const int u1 = (int)((int64_t)(wave + 1) * total / a.num_waves);

    uint32_t acc = 0;
    for (int base = u0; base < u1; base += 64) {
        // Lane i resolves tile base + i: its sequence, KV head, block and rows.
        const int uu = base + lane;
        const bool valid = uu < u1;
        int bl = 0;
        for (int j = 0; j < B; ++j)
            bl += __builtin_amdgcn_readlane(end, j) <= uu ? 1 : 0;
        bl = bl < B ? bl : B - 1;
        // every lane takes part in each shuffle (a shuffle inside a branch
        // would read inactive lanes)
        const int prev_end = __shfl(end, bl > 0 ? bl - 1 : 0, 64);
        const int start = bl > 0 ? prev_end : 0;
        const int nb_b = __shfl(nb, bl, 64);
        const int ctx_b = __shfl(cl, bl, 64);
        int tile = 0, rows = 0;
        if (valid) {
            const int r = uu - start;
            const int g = r / nb_b;
            const int n = r - g * nb_b;
            rows = ctx_b - 16 * n;
            rows = rows > 16 ? 16 : rows;
            const int blk = a.block_tables[(size_t)bl * a.max_blocks + n];
            tile = blk * hkv + g;
        }
        const int count = u1 - base < 64 ? u1 - base : 64;

        u32x4 s0[SL], s1[SL];
        auto issue = [&](int t0, u32x4(&d)[SL]) {
#pragma unroll
            for (int t = 0; t < TS; ++t) {
                const int ti = t0 + t < count ? t0 + t : count - 1;
                const int tt = __builtin_amdgcn_readlane(tile, ti);
                const int rr = t0 + t < count ? __builtin_amdgcn_readlane(rows, ti) : 0;
                const size_t off = (size_t)tt * 16 * RB;
                const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
                    (void *)(a.k_cache + off), (short)0, rr * RB, kRawBufferWord3);
                const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
                    (void *)(a.v_cache + off), (short)0, rr * RB, kRawBufferWord3);
#pragma unroll
                for (int i = 0; i < TL; ++i) {
                    d[(2 * t) * TL + i] =
                        __builtin_amdgcn_raw_buffer_load_b128(rk, (i * 64 + lane) * 16, 0, 0);
                    d[(2 * t + 1) * TL + i] =
                        __builtin_amdgcn_raw_buffer_load_b128(rv, (i * 64 + lane) * 16, 0, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        auto consume = [&](const u32x4(&d)[SL]) {
#pragma unroll
            for (int i = 0; i < SL; ++i)
                acc ^= fold(d[i]);
        };
        issue(0, s0);
        for (int t = 0; t < count;) {
            if (t + TS < count)
                issue(t + TS, s1);
            consume(s0);
            t += TS;
            if (t >= count)
                break;
            if (t + TS < count)
                issue(t + TS, s0);
            consume(s1);
            t += TS;
        }
    }
    store_wave_xor(acc, a.sink, wave);
}

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

photon_status check_waves(int32_t waves, const uint32_t *sink)
{
    if (waves <= 0 || waves % kProbeWaves != 0 || waves > kMaxProbeWaves)
        return fail(PHOTON_ERR_INVALID_ARG, "waves %d must be a positive multiple of %d, at most %lld",
                    waves, kProbeWaves, (long long)kMaxProbeWaves);
    if (!sink || !aligned(sink, 4))
        return fail(PHOTON_ERR_INVALID_ARG, "sink must be non-NULL and 4-byte aligned");
    return PHOTON_OK;
}

}  // namespace
}  // namespace photon

using photon::fail;
using photon::ok;

extern "C" {

photon_status photon_probe_stream_read(const void *buf, size_t bytes, int32_t waves, uint32_t *sink,
                                       void *stream)
{
    photon_status st = photon::check_waves(waves, sink);
    if (st != PHOTON_OK)
        return st;
    if (!buf || !photon::aligned(buf, 16))
        return fail(PHOTON_ERR_INVALID_ARG, "buf must be non-NULL and 16-byte aligned");
    if (bytes == 0 || bytes % 16 != 0)
        return fail(PHOTON_ERR_INVALID_ARG, "bytes %zu must be a positive multiple of 16", bytes);
    if (bytes / (size_t)waves >= ((size_t)1 << 32) - 16)
        return fail(PHOTON_ERR_UNSUPPORTED, "%zu bytes per wavefront exceed a buffer descriptor",
                    bytes / (size_t)waves);
    hipLaunchKernelGGL(photon::stream_read_kernel, dim3((unsigned)(waves / photon::kProbeWaves)),
                       dim3(photon::kProbeWaves * 64), 0, (hipStream_t)stream,
                       static_cast<const char *>(buf), (uint64_t)(bytes / 16), (int)waves, sink);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return fail(PHOTON_ERR_HIP, "stream read launch: %s", hipGetErrorString(err));
    return ok();
}

photon_status photon_probe_gather(const void *k_cache, const void *v_cache,
                                  const int32_t *block_tables, const int32_t *context_lens,
                                  const photon_decode_desc *desc, int32_t waves, uint32_t *sink,
                                  void *stream)
{
    photon_status st = photon::check_waves(waves, sink);
    if (st != PHOTON_OK)
        return st;
    if (!desc)
        return fail(PHOTON_ERR_INVALID_ARG, "decode descriptor is NULL");
    const photon_kv_desc &kv = desc->kv;
    const int eb = kv.dtype == PHOTON_F32 ? 4 : (kv.dtype == PHOTON_F16 || kv.dtype == PHOTON_BF16) ? 2 : 0;
    if (eb == 0)
        return fail(PHOTON_ERR_INVALID_ARG, "unknown dtype %d", kv.dtype);
    if (desc->num_seqs < 0 || desc->num_seqs > photon::kMaxProbeSeqs)
        return fail(PHOTON_ERR_UNSUPPORTED, "num_seqs %d: the gather probe takes 0 to %d",
                    desc->num_seqs, photon::kMaxProbeSeqs);
    if (kv.num_blocks <= 0 || kv.num_kv_heads <= 0 || desc->max_blocks_per_seq <= 0 ||
        desc->max_context_len < 0 ||
        (int64_t)desc->max_context_len > (int64_t)desc->max_blocks_per_seq * kv.block_size)
        return fail(PHOTON_ERR_INVALID_ARG, "bad sizes");
    if (kv.block_size != 16)
        return fail(PHOTON_ERR_UNSUPPORTED, "block_size %d (16 is built)", kv.block_size);
    const int rb = kv.head_dim * eb;
    if (rb != 128 && rb != 256 && rb != 512)
        return fail(PHOTON_ERR_UNSUPPORTED, "row of %d bytes (128, 256 or 512 are built)", rb);
    if ((int64_t)kv.num_blocks * kv.num_kv_heads > INT32_MAX)
        return fail(PHOTON_ERR_UNSUPPORTED, "num_blocks * num_kv_heads above the int32 range");
    if (!k_cache || !v_cache || !block_tables || !context_lens)
        return fail(PHOTON_ERR_INVALID_ARG, "NULL data pointer");
    if (!photon::aligned(k_cache, 16) || !photon::aligned(v_cache, 16) ||
        !photon::aligned(block_tables, 4) || !photon::aligned(context_lens, 4))
        return fail(PHOTON_ERR_INVALID_ARG, "misaligned pointer");
    photon::GatherArgs a{};
    a.k_cache = static_cast<const char *>(k_cache);
    a.v_cache = static_cast<const char *>(v_cache);
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.sink = sink;
    a.num_seqs = desc->num_seqs;
    a.num_kv_heads = kv.num_kv_heads;
    a.max_blocks = desc->max_blocks_per_seq;
    a.num_waves = waves;
    const dim3 grid((unsigned)(waves / photon::kProbeWaves)), block(photon::kProbeWaves * 64);
    switch (rb) {
    case 128: hipLaunchKernelGGL(photon::gather_kernel<128>, grid, block, 0, (hipStream_t)stream, a); break;
    case 256: hipLaunchKernelGGL(photon::gather_kernel<256>, grid, block, 0, (hipStream_t)stream, a); break;
    default: hipLaunchKernelGGL(photon::gather_kernel<512>, grid, block, 0, (hipStream_t)stream, a); break;
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return fail(PHOTON_ERR_HIP, "gather launch: %s", hipGetErrorString(err));
    return ok();
}

}  // extern "C"
