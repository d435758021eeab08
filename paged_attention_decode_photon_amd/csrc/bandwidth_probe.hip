// Bandwidth probes for gfx950: a contiguous streaming read, and a bare
// gather of the K/V rows of a paged decode call (PhotonInfer README,
// "Technical details -> Paged attention": block-level cache read through
// per-sequence tables).  Neither does any attention arithmetic: every 32-bit
// word read is XOR-folded into one value per wavefront, so their durations
// bound what a decode kernel reading the same bytes can reach.
//
// All use the decode kernel's memory instructions (16-byte raw buffer
// loads, range-checked descriptors, V rows loaded non-temporal).  The gathers walk the sequence-major
// list of (sequence, KV head, block) tiles and resolve up to 64 tiles at a
// time with one table load per lane.  Three ways of handing out the list:
//   - gather_kernel: an even split over wavefronts, like the decode kernel's
//     balanced split, 16 KiB in flight per wavefront (two alternating 8 KiB
//     register sets);
//   - gather_staged_kernel: an even split over workgroups of four
//     wavefronts that take the workgroup's tiles in turn, each keeping a
//     ring of tiles in flight in LDS (loads that write LDS directly);
//   - gather_queue_kernel: part of the list split evenly, the rest handed
//     out at run time in fixed pieces through one agent-scope atomic counter.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "elem.h"
#include "lane_ops.h"
#include "photon_probe.h"
#include "status.h"

namespace photon {
namespace {

constexpr int kRawBufferWord3 = 0x00020000;  // raw, unswizzled buffer (gfx9 family)
constexpr int kVLoadAux = 2;                 // nt bit on V loads, K plain (the decode kernel's policy)
constexpr int kProbeWaves = 4;               // wavefronts per workgroup
constexpr int kSetLoads = 8;                 // 16-byte loads per lane per register set (8 KiB/wave)
constexpr int kMaxProbeSeqs = 64;
constexpr int kStagedWaves = 4;                 // one per SIMD of a CU
constexpr int kStagedLdsBytes = 128 * 1024;     // LDS ring of a staged-gather workgroup, at most
constexpr int64_t kMaxProbeWaves = 1 << 20;

__device__ __forceinline__ uint32_t fold(const u32x4 &v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

__device__ __forceinline__ unsigned long long first_lane_u64(unsigned long long v)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((unsigned long long)hi << 32) | lo;
}

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

// Tile-list bookkeeping shared by the gathers.  Lane b holds sequence b's
// context length, block count and the inclusive prefix sum of Hkv * blocks.
struct TileList {
    int B, hkv, cl, nb, end;
    __device__ explicit TileList(const GatherArgs &a)
    {
        const int lane = threadIdx.x & 63;
        B = a.num_seqs;
        hkv = a.num_kv_heads;
        cl = lane < B ? a.context_lens[lane] : 0;
        nb = (cl + 15) / 16;
        end = wave_inclusive_sum(hkv * nb);
    }
    __device__ int total() const { return B > 0 ? __builtin_amdgcn_readlane(end, B - 1) : 0; }
    // Lane i resolves list entry uu (valid: in range): the tile's index in
    // the pool ((block * Hkv + head)) and its valid rows.
    __device__ void resolve(const GatherArgs &a, int uu, bool valid, int &tile, int &rows) const
    {
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
        tile = 0;
        rows = 0;
        if (valid) {
            const int r = uu - start;
            const int g = r / nb_b;
            const int n = r - g * nb_b;
            rows = ctx_b - 16 * n;
            rows = rows > 16 ? 16 : rows;
            const int blk = a.block_tables[(size_t)bl * a.max_blocks + n];
            tile = blk * hkv + g;
        }
    }
};

// RB: bytes of one K/V row.  A 16-row tile is TL = RB / 64 wave-wide
// 16-byte loads, each of K and V; a register set holds TS = kSetLoads /
// (2 TL) tiles of K and V (or half a tile when RB = 512).
template <int RB>
struct RegisterGather {
    static constexpr int TL = RB / 64;
    static constexpr int TS = kSetLoads / (2 * TL) > 0 ? kSetLoads / (2 * TL) : 1;
    static constexpr int SL = TS * 2 * TL;
    const GatherArgs &a;
    const TileList &list;
    uint32_t acc = 0;
    __device__ RegisterGather(const GatherArgs &a_, const TileList &l) : a(a_), list(l) {}

    // Read list entries [u0, u1).
    __device__ void range(int u0, int u1)
    {
        const int lane = threadIdx.x & 63;
        for (int base = u0; base < u1; base += 64) {
            int tile, rows;
            list.resolve(a, base + lane, base + lane < u1, tile, rows);
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
                        d[(2 * t + 1) * TL + i] = __builtin_amdgcn_raw_buffer_load_b128(
                            rv, (i * 64 + lane) * 16, 0, kVLoadAux);
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
    }
};

template <int RB>
__global__ __launch_bounds__(kProbeWaves * 64) void gather_kernel(GatherArgs a)
{
    const int wave = blockIdx.x * kProbeWaves + (threadIdx.x >> 6);
    const TileList list(a);
    RegisterGather<RB> g(a, list);
    const int total = list.total();
    g.range((int)((int64_t)wave * total / a.num_waves),
            (int)((int64_t)(wave + 1) * total / a.num_waves));
    store_wave_xor(g.acc, a.sink, wave);
}

// The first static_permille thousandths of the list are split evenly over
// the wavefronts; the rest is cut into pieces of `piece` entries, handed
// out by *queue.  Every wavefront draws tickets (agent-scope atomic add on
// one 64-bit word) until it draws one past the last piece, so the call
// draws exactly pieces + waves tickets, and the wavefront holding the last
// of them (no other draw can follow it) stores zero back.  The first draw is
// issued before the static share's loads so its latency hides behind them.
template <int RB>
__global__ __launch_bounds__(kProbeWaves * 64) void gather_queue_kernel(GatherArgs a,
                                                                        unsigned long long *queue,
                                                                        int static_permille,
                                                                        int piece)
{
    const int lane = threadIdx.x & 63;
    const int wave = blockIdx.x * kProbeWaves + (threadIdx.x >> 6);
    const TileList list(a);
    RegisterGather<RB> g(a, list);
    const int total = list.total();
    const int S = (int)((int64_t)total * static_permille / 1000);
    const unsigned long long pieces = (unsigned long long)((total - S + piece - 1) / piece);
    unsigned long long got = 0;
    if (lane == 0)
        got = __hip_atomic_fetch_add(queue, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    g.range((int)((int64_t)wave * S / a.num_waves), (int)((int64_t)(wave + 1) * S / a.num_waves));
    unsigned long long t = first_lane_u64(got);
    while (t < pieces) {
        if (lane == 0)
            got = __hip_atomic_fetch_add(queue, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int u0 = S + (int)t * piece;
        g.range(u0, u0 + piece < total ? u0 + piece : total);
        t = first_lane_u64(got);
    }
    if (t == pieces + (unsigned long long)a.num_waves - 1 && lane == 0)
        __hip_atomic_store(queue, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    store_wave_xor(g.acc, a.sink, wave);
}

typedef __attribute__((address_space(3))) void lds_void;

// The list split evenly over workgroups of kStagedWaves wavefronts; a
// workgroup's wavefronts take its tiles in turn.  Each wavefront keeps RING
// tiles in flight in its own part of LDS: the loads write LDS directly (a
// wave-wide 16-byte load fills 1 KiB), the wavefront waits until the oldest
// tile has landed (vmcnt counts these loads too, in issue order), reads it
// back and refills the slot with the tile RING - 1 places further on.
// Entries past the wavefront's list get empty descriptors (no memory
// access), so the wait count is the same on every step.
template <int RB, int RING>
__global__ __launch_bounds__(kStagedWaves * 64) void gather_staged_kernel(GatherArgs a,
                                                                          int num_workgroups)
{
    constexpr int TL = RB / 64;        // 1 KiB loads per tile, each of K and V
    constexpr int LPT = 2 * TL;        // loads per tile
    constexpr int TILE = 32 * RB;      // bytes of K and V of one 16-row tile
    constexpr int NV = LPT * (RING - 1);
    static_assert(NV <= 63, "vmcnt range");
    static_assert(kStagedWaves * RING * TILE <= kStagedLdsBytes, "LDS");
    __shared__ __attribute__((aligned(16))) char lds[kStagedWaves * RING * TILE];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    char *ring = lds + wv * RING * TILE;  // uniform, as the LDS address of these loads must be
    const TileList list(a);
    const int total = list.total();
    const int w0 = (int)((int64_t)blockIdx.x * total / num_workgroups);
    const int w1 = (int)((int64_t)(blockIdx.x + 1) * total / num_workgroups);
    // this wavefront's entries: w0 + wv + kStagedWaves * k, k < n
    const int n = w1 - w0 > wv ? (w1 - w0 - wv + kStagedWaves - 1) / kStagedWaves : 0;
    uint32_t acc = 0;
    for (int base = 0; base < n; base += 64) {
        int tile, rows;
        list.resolve(a, w0 + wv + kStagedWaves * (base + lane), base + lane < n, tile, rows);
        const int count = n - base < 64 ? n - base : 64;
        auto issue = [&](int t) {
            const int ti = t < count ? t : count - 1;
            const int tt = __builtin_amdgcn_readlane(tile, ti);
            const int rr = t < count ? __builtin_amdgcn_readlane(rows, ti) : 0;
            const size_t off = (size_t)tt * 16 * RB;
            const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(a.k_cache + off), (short)0, rr * RB, kRawBufferWord3);
            const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(a.v_cache + off), (short)0, rr * RB, kRawBufferWord3);
            char *slot = ring + (t % RING) * TILE;
#pragma unroll
            for (int i = 0; i < TL; ++i) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void *)(slot + i * 1024), 16,
                                                         (i * 64 + lane) * 16, 0, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(slot + (TL + i) * 1024),
                                                         16, (i * 64 + lane) * 16, 0, 0, kVLoadAux);
            }
        };
#pragma unroll
        for (int t = 0; t < RING - 1; ++t)
            issue(t);
        for (int t = 0; t < count; ++t) {
            issue(t + RING - 1);
            // vmcnt(NV): at most the RING - 1 newer tiles' loads are pending
            __builtin_amdgcn_s_waitcnt((NV & 15) | ((NV >> 4) << 14) | 0x0f70);
            asm volatile("" ::: "memory");
            const char *slot = ring + (t % RING) * TILE;
#pragma unroll
            for (int i = 0; i < LPT; ++i)
                acc ^= fold(*reinterpret_cast<const u32x4 *>(slot + i * 1024 + lane * 16));
            // lgkmcnt(0): the slot's reads are done before a load refills it
            __builtin_amdgcn_s_waitcnt(0xc07f);
            asm volatile("" ::: "memory");
        }
        // vmcnt(0): the empty loads past the list have landed before the
        // ring is reused
        __builtin_amdgcn_s_waitcnt(0x0f70);
        asm volatile("" ::: "memory");
    }
    store_wave_xor(acc, a.sink, blockIdx.x * kStagedWaves + wv);
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

// Validation shared by the gathers; fills the kernel arguments (num_waves
// excepted) and the row size in bytes.
photon_status gather_args(const void *k_cache, const void *v_cache, const int32_t *block_tables,
                          const int32_t *context_lens, const photon_decode_desc *desc,
                          uint32_t *sink, GatherArgs &a, int &rb)
{
    if (!desc)
        return fail(PHOTON_ERR_INVALID_ARG, "decode descriptor is NULL");
    const photon_kv_desc &kv = desc->kv;
    const int eb = kv.dtype == PHOTON_F32 ? 4 : (kv.dtype == PHOTON_F16 || kv.dtype == PHOTON_BF16) ? 2 : 0;
    if (eb == 0)
        return fail(PHOTON_ERR_INVALID_ARG, "unknown dtype %d", kv.dtype);
    if (desc->num_seqs < 0 || desc->num_seqs > kMaxProbeSeqs)
        return fail(PHOTON_ERR_UNSUPPORTED, "num_seqs %d: the gather probes take 0 to %d",
                    desc->num_seqs, kMaxProbeSeqs);
    if (kv.num_blocks <= 0 || kv.num_kv_heads <= 0 || desc->max_blocks_per_seq <= 0 ||
        desc->max_context_len < 0 ||
        (int64_t)desc->max_context_len > (int64_t)desc->max_blocks_per_seq * kv.block_size)
        return fail(PHOTON_ERR_INVALID_ARG, "bad sizes");
    if (kv.block_size != 16)
        return fail(PHOTON_ERR_UNSUPPORTED, "block_size %d (16 is built)", kv.block_size);
    rb = kv.head_dim * eb;
    if (rb != 128 && rb != 256 && rb != 512)
        return fail(PHOTON_ERR_UNSUPPORTED, "row of %d bytes (128, 256 or 512 are built)", rb);
    if ((int64_t)kv.num_blocks * kv.num_kv_heads > INT32_MAX)
        return fail(PHOTON_ERR_UNSUPPORTED, "num_blocks * num_kv_heads above the int32 range");
    if (!k_cache || !v_cache || !block_tables || !context_lens)
        return fail(PHOTON_ERR_INVALID_ARG, "NULL data pointer");
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(block_tables, 4) ||
        !aligned(context_lens, 4))
        return fail(PHOTON_ERR_INVALID_ARG, "misaligned pointer");
    if (!sink || !aligned(sink, 4))
        return fail(PHOTON_ERR_INVALID_ARG, "sink must be non-NULL and 4-byte aligned");
    a = GatherArgs{};
    a.k_cache = static_cast<const char *>(k_cache);
    a.v_cache = static_cast<const char *>(v_cache);
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.sink = sink;
    a.num_seqs = desc->num_seqs;
    a.num_kv_heads = kv.num_kv_heads;
    a.max_blocks = desc->max_blocks_per_seq;
    return PHOTON_OK;
}

photon_status launched(const char *what)
{
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return fail(PHOTON_ERR_HIP, "%s launch: %s", what, hipGetErrorString(err));
    return ok();
}

template <int RB>
void launch_staged(const GatherArgs &a, int workgroups, int ring, hipStream_t stream)
{
    const dim3 grid((unsigned)workgroups), block(kStagedWaves * 64);
    if constexpr (RB * 2 <= kStagedLdsBytes / (32 * kStagedWaves)) {
        if (ring == 2) {
            hipLaunchKernelGGL((gather_staged_kernel<RB, 2>), grid, block, 0, stream, a, workgroups);
            return;
        }
    }
    if constexpr (RB * 4 <= kStagedLdsBytes / (32 * kStagedWaves)) {
        if (ring == 4) {
            hipLaunchKernelGGL((gather_staged_kernel<RB, 4>), grid, block, 0, stream, a, workgroups);
            return;
        }
    }
    if constexpr (RB * 8 <= kStagedLdsBytes / (32 * kStagedWaves)) {
        if (ring == 8) {
            hipLaunchKernelGGL((gather_staged_kernel<RB, 8>), grid, block, 0, stream, a, workgroups);
            return;
        }
    }
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
    return photon::launched("stream read");
}

photon_status photon_probe_gather(const void *k_cache, const void *v_cache,
                                  const int32_t *block_tables, const int32_t *context_lens,
                                  const photon_decode_desc *desc, int32_t waves, uint32_t *sink,
                                  void *stream)
{
    photon_status st = photon::check_waves(waves, sink);
    if (st != PHOTON_OK)
        return st;
    photon::GatherArgs a;
    int rb;
    if ((st = photon::gather_args(k_cache, v_cache, block_tables, context_lens, desc, sink, a, rb)) !=
        PHOTON_OK)
        return st;
    a.num_waves = waves;
    const dim3 grid((unsigned)(waves / photon::kProbeWaves)), block(photon::kProbeWaves * 64);
    switch (rb) {
    case 128: hipLaunchKernelGGL(photon::gather_kernel<128>, grid, block, 0, (hipStream_t)stream, a); break;
    case 256: hipLaunchKernelGGL(photon::gather_kernel<256>, grid, block, 0, (hipStream_t)stream, a); break;
    default: hipLaunchKernelGGL(photon::gather_kernel<512>, grid, block, 0, (hipStream_t)stream, a); break;
    }
    return photon::launched("gather");
}

photon_status photon_probe_gather_staged(const void *k_cache, const void *v_cache,
                                         const int32_t *block_tables, const int32_t *context_lens,
                                         const photon_decode_desc *desc, int32_t workgroups,
                                         int32_t ring_tiles, uint32_t *sink, void *stream)
{
    if (workgroups <= 0 || workgroups > photon::kMaxProbeWaves / photon::kStagedWaves)
        return fail(PHOTON_ERR_INVALID_ARG, "workgroups %d: 1 to %lld", workgroups,
                    (long long)(photon::kMaxProbeWaves / photon::kStagedWaves));
    photon::GatherArgs a;
    int rb;
    photon_status st = photon::gather_args(k_cache, v_cache, block_tables, context_lens, desc, sink, a, rb);
    if (st != PHOTON_OK)
        return st;
    if ((ring_tiles != 2 && ring_tiles != 4 && ring_tiles != 8) ||
        (int64_t)photon::kStagedWaves * ring_tiles * 32 * rb > photon::kStagedLdsBytes)
        return fail(PHOTON_ERR_UNSUPPORTED,
                    "ring of %d tiles of %d-byte rows (2, 4 or 8 tiles, at most %d KiB per workgroup)",
                    ring_tiles, rb, photon::kStagedLdsBytes / 1024);
    a.num_waves = workgroups * photon::kStagedWaves;
    switch (rb) {
    case 128: photon::launch_staged<128>(a, workgroups, ring_tiles, (hipStream_t)stream); break;
    case 256: photon::launch_staged<256>(a, workgroups, ring_tiles, (hipStream_t)stream); break;
    default: photon::launch_staged<512>(a, workgroups, ring_tiles, (hipStream_t)stream); break;
    }
    return photon::launched("staged gather");
}

photon_status photon_probe_gather_queue(const void *k_cache, const void *v_cache,
                                        const int32_t *block_tables, const int32_t *context_lens,
                                        const photon_decode_desc *desc, int32_t waves,
                                        int32_t static_permille, int32_t piece_tiles,
                                        uint64_t *queue, uint32_t *sink, void *stream)
{
    photon_status st = photon::check_waves(waves, sink);
    if (st != PHOTON_OK)
        return st;
    if (static_permille < 0 || static_permille > 1000)
        return fail(PHOTON_ERR_INVALID_ARG, "static_permille %d: 0 to 1000", static_permille);
    if (piece_tiles < 1 || piece_tiles > 64)
        return fail(PHOTON_ERR_INVALID_ARG, "piece_tiles %d: 1 to 64", piece_tiles);
    if (!queue || !photon::aligned(queue, 8))
        return fail(PHOTON_ERR_INVALID_ARG, "queue must be non-NULL and 8-byte aligned");
    photon::GatherArgs a;
    int rb;
    if ((st = photon::gather_args(k_cache, v_cache, block_tables, context_lens, desc, sink, a, rb)) !=
        PHOTON_OK)
        return st;
    a.num_waves = waves;
    unsigned long long *q = reinterpret_cast<unsigned long long *>(queue);
    const dim3 grid((unsigned)(waves / photon::kProbeWaves)), block(photon::kProbeWaves * 64);
    switch (rb) {
    case 128:
        hipLaunchKernelGGL(photon::gather_queue_kernel<128>, grid, block, 0, (hipStream_t)stream, a, q,
                           (int)static_permille, (int)piece_tiles);
        break;
    case 256:
        hipLaunchKernelGGL(photon::gather_queue_kernel<256>, grid, block, 0, (hipStream_t)stream, a, q,
                           (int)static_permille, (int)piece_tiles);
        break;
    default:
        hipLaunchKernelGGL(photon::gather_queue_kernel<512>, grid, block, 0, (hipStream_t)stream, a, q,
                           (int)static_permille, (int)piece_tiles);
        break;
    }
    return photon::launched("queue gather");
}

}  // extern "C"
