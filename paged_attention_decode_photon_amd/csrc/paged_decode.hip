// Batched paged-attention decode for gfx950 (CDNA4), one kernel per call.
//
// Operation (PhotonInfer README, "GPU-optimised kernels": batched paged
// attention with a stable softmax; "Technical details -> Paged attention":
// block-level KV cache addressed through per-sequence block tables): for
// sequence b, query head h and KV head g = h / G,
//   out[b][h] = sum_t exp(s_t - m) V_t / sum_t exp(s_t - m),
//   s_t = scale * <q[b][h], K_t>,  m = max_t s_t,  t < context_lens[b].
//
// Work decomposition (balanced split of the whole batch).  A "segment" is one
// (sequence b, KV head g) pair together with the G query heads that read it,
// so every K/V byte is fetched from HBM once.  A segment is cut into chunks
// of CT = 16 U tokens; the chunks of all segments, sequence-major then
// KV-head-major, form one list of U_tot units.  In the list the waves
// split, each non-empty segment is preceded by C empty entries (C = 2 for
// batches of 768 units or more, else 0); of the wavefronts launched,
// NW = min(launched, max(ceil(L / 5), min(U_tot, 256))) take part, for L
// list entries, and wave s takes entries [s L / NW, (s+1) L / NW): every wave gets
// the same amount of work however ragged the contexts are, a slice that
// changes segment being charged two units for it, which keeps all compute
// units busy until the end.  Context lengths live on the device, so the
// kernel first forms the prefix sums of per-sequence unit counts and of
// non-empty sequences: each wave in its own registers for up to 64
// sequences, else each workgroup in LDS; every wave then finds its first
// sequence with one or two wave-wide ballots.
// Each wave keeps two chunks in flight (up to four query heads per KV head;
// with eight the second register set would cost occupancy).
//
// A wave's slice covers pieces of one or more segments.  A piece that holds
// a whole segment writes its normalised output directly.  Otherwise the
// piece's (max, sum, unnormalised rows) go to a workspace record and the
// wave adds the piece's unit count to the segment's arrival counter (tagged
// with the call's epoch, so whatever the workspace held before the call is
// never counted; arrival.h); the wave that completes the count merges all
// pieces of the segment in slice order (deterministic whichever wave that
// is) and resets the counter to zero.  Waves of one segment may run on different XCDs, whose L2 caches are
// not coherent with each other; rather than agent-scope fences (an L2
// write-back or invalidate, far too slow here) only the partial results
// travel coherently, as device-scope (sc1) stores and loads, and a wave's
// stores complete before it counts its arrival with an agent-scope atomic.
// No workgroup barrier is used after the prefix sum: waves never wait for
// each other.
//
// Lane layout.  A K/V row is RB = D * sizeof(T) bytes, i.e. L = RB / 16
// lanes of one 16-byte load each; one wave-wide load covers RPI = 64 / L
// rows and a 16-token block takes NIB = 16 / RPI loads.  Lane (r, c) with
// r = lane / L, c = lane % L always holds byte chunk c of some row; the 16
// bytes of each quad of lanes are contiguous.
//
// Scores without select-heavy reductions.  Per chunk a lane forms NS = NU*G
// partial dot products (NU = U*NIB loads, G heads), each over its own chunk
// c of the row.  They are summed over the L lanes of a row by a butterfly
// reduce-scatter in which lane c keeps slot j for "item" j ^ phi(c)
// (item = load * G + head, phi(c) = low CP bits of c).  A lane therefore
// loads row ((load % NIB) ^ (phi >> log2 G)) of its block and multiplies by
// query head (head ^ (phi % G)); after each pairing step the partner's
// register j ^ mask already holds the item this lane keeps, so every step is
// one add with a DPP or swizzle operand.  The permutation never leaves a
// block, so the buffer descriptor of each load stays wave-uniform.
// Remaining lane bits (when CP < log2 L) are summed with plain pairings.
//
// Masking.  Every block tile is read through a raw buffer descriptor whose
// size is the number of valid rows; rows past the context length and whole
// blocks past it return zero without touching memory, and their scores are
// set to -inf, so pool padding (even NaN) never reaches the arithmetic.
//
// Dot products.  fp32 rows: q is widened once per piece, pre-multiplied by
// scale * log2 e, and each partial product is a chain of FMAs.  16-bit rows:
// q stays packed and K is never widened; each partial product is a chain of
// two-element dot instructions (v_dot2_f32_f16 / v_dot2_f32_bf16, fp32
// accumulation), half the instructions and no conversions, and the reduced
// score is multiplied by scale * log2 e.
//
// Softmax.  Scores are kept in log2 units and use v_exp_f32.  Each wave
// keeps an online maximum and sum per head over its piece.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "arrival.h"
#include "elem.h"
#include "lane_ops.h"
#include "launch.h"

namespace photon {
namespace {

// Fourth descriptor word of a raw (unswizzled, stride 0) buffer on gfx9-family.
constexpr int kRawBufferWord3 = 0x00020000;
// Fewest units a wavefront's slice holds while more than kMinWaves waves
// would take part: measured best among 1-6 on the batch-16 (fp32 and bf16),
// ragged batch-64 and long-context workloads.  Small calls keep kMinWaves
// waves (or one per unit), since there the latency of a wave's chain of
// chunks dominates: batch 1 at 512 tokens takes 10.5 us with one unit per
// wave against 14.3 us with five.  128 rather than 256: fewer slices per
// segment, so fewer records to merge (batch 1 at 2048 tokens 13.4 -> 11.9 us,
// batch 2 f32 13.9 -> 12.2 us, bf16 11.2 -> 9.3 us; batch 1 at 512 tokens,
// batch 4 and up unchanged).
constexpr int kMinUnitsPerWave = 5;
constexpr int kMinWaves = 128;
// Work a wavefront is charged for starting on a segment, in units: a piece
// change costs a record, an arrival and a fresh first round trip, so in a
// batch of at least kChargeFromUnits units each non-empty segment is counted
// as this many units longer (empty units at its start).  A slice that spans
// a segment change then holds that many fewer chunks.  Two was measured
// best among one to three (ragged batch-64: 29.6 -> 28.2 us).  From
// 3 * kMinWaves units on, every slice holds at least three list entries, so
// at least one unit of work (batch 4: 14.8 -> 13.6 us at fp32).
constexpr int kBoundaryUnits = kDecodeBoundaryUnits;
constexpr int kChargeFromUnits = 3 * kMinWaves;

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }
constexpr int cmin(int a, int b) { return a < b ? a : b; }

template <typename T, int D, int G>
struct Shape {
    static constexpr int EB = sizeof(T);
    static constexpr int E = 16 / EB;                 // elements per lane chunk
    static constexpr int RB = D * EB;                 // bytes per row
    static constexpr int L = RB / 16;                 // lanes per row
    static constexpr int LOG2L = ilog2(L);
    static constexpr int RPI = 64 / L;                // rows per wave-wide load
    static constexpr int NIB = kBlockTokens / RPI;    // loads per block
    static constexpr int LOG2G = ilog2(G);
    static constexpr int U = decode_chunk_blocks(EB, D, G);
    static constexpr int CT = U * kBlockTokens;       // tokens per chunk
    static constexpr int NU = U * NIB;                // loads per chunk (each of K, V)
    static constexpr int NS = NU * G;                 // partial-score slots
    static constexpr int CP = cmin(LOG2G + ilog2(NIB), LOG2L);  // reduce-scatter steps
    static constexpr int NK = NS >> CP;               // scores per lane after the butterfly
    static constexpr int REC = decode_record_floats(D, G);  // floats per partial record
    static_assert(L * E == D, "row split");
    static_assert(L >= G && L >= 8 && L <= 32, "lane layout");
    static_assert(CT == decode_chunk_tokens(EB, D, G), "chunk size");
};

// Partial records travel between waves that may sit on different XCDs,
// whose L2 caches are not coherent with each other.  They are written and
// read with device-scope (sc1) buffer accesses, which write through and read
// past the per-XCD L2, so no cache-wide fence is needed.
constexpr int kDeviceScope = 16;  // cache-policy bits: sc1

__device__ __forceinline__ __amdgpu_buffer_rsrc_t record_rsrc(float *rec, int floats)
{
    return __builtin_amdgcn_make_buffer_rsrc(rec, (short)0, floats * 4, kRawBufferWord3);
}
// Wait until every vector memory operation this wave issued has completed
// (stores included); the memory clobber keeps the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void wait_vector_memory()
{
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}
// Compiler-only barrier for memory accesses.
__device__ __forceinline__ void compiler_memory_barrier()
{
    asm volatile("" ::: "memory");
}

// Mask of the reduce-scatter step that halves slot bit k.  The mask has bit
// k set and no higher bit, so it maps live slots onto live slots.
constexpr int rs_mask(int k) { return k == 0 ? 1 : k == 1 ? 2 : k == 2 ? 7 : k == 3 ? 8 : 16; }

template <int NS, int CP, int K>
__device__ __forceinline__ void reduce_scatter(float (&part)[NS])
{
    if constexpr (K >= 0) {
        constexpr int M = rs_mask(K);
        constexpr int live = (1 << (CP - K)) - 1;  // bits K..CP-1 must be zero afterwards
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            if (((j >> K) & live) == 0)
                part[j] += xor_partner<M>(part[j ^ M]);
        }
        reduce_scatter<NS, CP, K - 1>(part);
    }
}

struct KernelArgs {
    const void *q;
    const void *k_cache;  // written only by the fused decode step (store_new_token)
    const void *v_cache;
    const void *k_new;    // fused decode step: [B][Hkv][D] rows to append; NULL otherwise
    const void *v_new;
    const int32_t *block_tables;
    void *out;
    uint64_t *ws_count;  // epoch-tagged arrival counters (arrival.h)
    float *ws_rec;
    int num_kv_heads;
    int max_blocks;
    int num_waves;
    float qscale;
    uint32_t epoch;  // this call's number, never 0
};

// floor(n / d) for wave-uniform integers 0 <= n < 2^53 and 0 < d < 2^31,
// held exactly in doubles.  A 64-bit integer division compiles to several
// hundred scalar instructions (about 0.2 us of a wave's time, on the path
// of every slice's start and every merge); this is a dozen vector ones.
// Exact: when n / d is not an integer it lies at least 1 / d below the next
// one, while the correctly rounded quotient is off by at most
// (n / d) 2^-53 < 1 / d.
__device__ __forceinline__ int floor_div(double n, double d)
{
    return __builtin_amdgcn_readfirstlane((int)__builtin_floor(n / d));
}
// First list entry of slice s (slices split [0, total) as evenly as integers
// allow).  s <= nw <= 2^20 and total < 2^31 (the host checks both), so the
// products below are exact doubles under 2^51.
__device__ __forceinline__ int slice_start(int s, int total, int nw)
{
    return floor_div((double)s * total, nw);
}
// Slice that holds list entry u: the largest s with slice_start(s) <= u.
__device__ __forceinline__ int slice_of(int u, int total, int nw)
{
    return floor_div((double)(u + 1) * nw - 1.0, total);
}

// The slices holding a segment's records, in merge order.  The segment's
// units are entries [su0, su1) of the slice list, after its empty units,
// which start at sv0: a slice that starts at or after sv0 has the segment as
// its first piece (record role 0), else as its second (role 1).
struct SegmentSlices {
    int first, last, first_role;
};
__device__ __forceinline__ SegmentSlices segment_slices(int sv0, int su0, int su1, int total, int nw)
{
    SegmentSlices ss;
    ss.first = slice_of(su0, total, nw);
    ss.last = slice_of(su1 - 1, total, nw);
    ss.first_role = slice_start(ss.first, total, nw) >= sv0 ? 0 : 1;
    return ss;
}

template <typename T, typename O, int D, int G>
struct WaveDecoder {
    using S = Shape<T, D, G>;
    static constexpr int E = S::E, L = S::L, RPI = S::RPI, NIB = S::NIB, CT = S::CT;
    static constexpr int NU = S::NU, NS = S::NS, CP = S::CP, NK = S::NK, RB = S::RB;

    const KernelArgs &a;
    float (*p_lds)[G];  // this wave's [CT][G] softmax weights
    int lane, c, r, phi, row_x, head_x, my_head;
    int k_off[NIB], v_off[NIB];

    // state of the current piece
    int b, g, ctx;
    int new_pos;         // fused step: position of the appended token, else -1
    u32x4 knew, vnew;    // fused step: this lane's column of the new K and V rows
    // Lane 0: what the claim of the piece's arrival counter found, when
    // run_chunks made the claim (see early_claim in the kernel).
    uint64_t claim_seen = 0;
    bool append_pending = false;  // the new rows are loaded but not yet stored
    bool append_settled = true;   // a chunk loaded after the stores has been used
    int nblk;      // blocks holding the sequence's context
    int win0;      // first block index of the table window
    int tbl_win;   // lane i: block_tables[b][win0 + i] (0 past the context)
    // Query rows of the piece, this lane's chunk of each head.  fp32 storage:
    // widened and pre-multiplied by the scale (qf).  16-bit storage: kept
    // packed (qpk) for two-element dot instructions; the scale then goes on
    // the reduced score.
    static constexpr bool kPackedQ = S::EB == 2;
    float qf[G][E];
    u32x4 qpk[G];
    float m_run, l_run;
    float o_acc[G][E];

    __device__ WaveDecoder(const KernelArgs &args, float (*lds)[G]) : a(args), p_lds(lds)
    {
        lane = threadIdx.x & 63;
        c = lane & (L - 1);
        r = lane >> S::LOG2L;
        phi = c & ((1 << CP) - 1);
        row_x = phi >> S::LOG2G;
        head_x = phi & (G - 1);
        my_head = c & (G - 1);
#pragma unroll
        for (int i = 0; i < NIB; ++i) {
            k_off[i] = (((i ^ row_x) * RPI + r) * RB) + c * 16;
            v_off[i] = ((i * RPI + r) * RB) + c * 16;
        }
    }

    // Load 64 block-table entries starting at block n0, one per lane, so the
    // K/V loads of the following units need no dependent table read.
    __device__ void load_table_window(int n0)
    {
        win0 = n0;
        const int n = n0 + lane;
        tbl_win = n < nblk ? a.block_tables[(size_t)b * a.max_blocks + n] : 0;
    }

    // Make the window hold blocks [n_first, n_last] (n_last - n_first < 64).
    // A refreshed window is waited for right here.  The load is conditional,
    // so without this wait the compiler counts the window register as
    // possibly pending wherever it is read and waits for every load in
    // flight before each block lookup, the chunk in flight included: the
    // next chunk would only be issued once the current one had arrived.
    __device__ void cover_blocks(int n_first, int n_last)
    {
        if (n_last - win0 >= 64) {
            load_table_window(n_first);
        }
    }

    __device__ int block_at(int n) const { return __builtin_amdgcn_readlane(tbl_win, n - win0); }

    __device__ void begin_piece(int b_, int g_, int ctx_, int ch0)
    {
        b = b_;
        g = g_;
        ctx = ctx_;
        nblk = (ctx + kBlockTokens - 1) / kBlockTokens;
        load_table_window(ch0 * S::U);
        const int hq = a.num_kv_heads * G;
        const T *q = (const T *)a.q;
#pragma unroll
        for (int hs = 0; hs < G; ++hs) {
            const T *row = q + ((size_t)b * hq + (size_t)g * G + (hs ^ head_x)) * D + c * E;
            if constexpr (kPackedQ) {
                qpk[hs] = *reinterpret_cast<const u32x4 *>(row);
            } else {
                Elem<T>::unpack(*reinterpret_cast<const u32x4 *>(row), qf[hs]);
#pragma unroll
                for (int e = 0; e < E; ++e)
                    qf[hs][e] *= a.qscale;
            }
        }
        // The window (and the query rows, in the same round trip) before the
        // piece's first loads; see cover_blocks.
        new_pos = -1;
        m_run = -INFINITY;
        l_run = 0.0f;
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < E; ++e)
                o_acc[h][e] = 0.0f;
    }

    // Issue the K and V loads of chunk ch (U blocks) of the current segment.
    // A block past the context gets an empty descriptor: its loads return
    // zeros without touching memory.
    // live == false (wave-uniform): every descriptor is empty, so the loads
    // return zeros without touching memory.
    __device__ void load_chunk(int ch, u32x4 (&kd)[NU], u32x4 (&vd)[NU], bool live = true) const
    {
        const size_t tile_stride = (size_t)kBlockTokens * RB;
        __amdgpu_buffer_rsrc_t rk[S::U], rv[S::U];
#pragma unroll
        for (int u = 0; u < S::U; ++u) {
            const int n = ch * S::U + u;
            int rows = live ? ctx - n * kBlockTokens : 0;
            rows = rows > kBlockTokens ? kBlockTokens : rows;
            int blk = 0;
            if (rows > 0)
                blk = block_at(n);
            else
                rows = 0;
            const size_t tile = ((size_t)blk * a.num_kv_heads + g) * tile_stride;
            rk[u] = __builtin_amdgcn_make_buffer_rsrc((void *)((const char *)a.k_cache + tile),
                                                      (short)0, rows * RB, kRawBufferWord3);
            rv[u] = __builtin_amdgcn_make_buffer_rsrc((void *)((const char *)a.v_cache + tile),
                                                      (short)0, rows * RB, kRawBufferWord3);
        }
#pragma unroll
        for (int i = 0; i < NU; ++i)
            kd[i] = __builtin_amdgcn_raw_buffer_load_b128(rk[i / NIB], k_off[i % NIB], 0,
                                                          kDecodeKLoadAux);
#pragma unroll
        for (int i = 0; i < NU; ++i)
            vd[i] = __builtin_amdgcn_raw_buffer_load_b128(rv[i / NIB], v_off[i % NIB], 0,
                                                          kDecodeVLoadAux);
        // Keep every K and V load of the chunk ahead of the math (the
        // scheduler otherwise sinks part of V behind the scores, which costs
        // a second round trip per chunk).
        __builtin_amdgcn_sched_barrier(0);
    }

    // Scores, online softmax update and P.V for chunk ch.
    __device__ void consume_chunk(int ch, const u32x4 (&kd)[NU], const u32x4 (&vd)[NU])
    {
        const int ct0 = ch * CT;
        // Partial dot products over this lane's chunk: slot (i, hs) pairs the
        // lane's load i with query head hs ^ head_x.
        float part[NS];
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            if constexpr (kPackedQ) {
#pragma unroll
                for (int hs = 0; hs < G; ++hs) {
                    float acc = 0.0f;
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        // Copy the dwords out of the vectors before the bit
                        // cast inside dot2 (see Elem<_Float16>::unpack).
                        const uint32_t qw = qpk[hs][w];
                        const uint32_t kw = kd[i][w];
                        acc = Elem<T>::dot2(qw, kw, acc);
                    }
                    part[i * G + hs] = acc;
                }
            } else {
                float kf[E];
                Elem<T>::unpack(kd[i], kf);
#pragma unroll
                for (int hs = 0; hs < G; ++hs) {
                    float acc = 0.0f;
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        acc = __builtin_fmaf(qf[hs][e], kf[e], acc);
                    part[i * G + hs] = acc;
                }
            }
        }
        reduce_scatter<NS, CP, CP - 1>(part);

        // Scores: slot n << CP now holds item (n << CP) | phi, summed over the
        // CP permuted lane bits; the remaining row bits are summed directly.
        float s[NK];
        int s_tok[NK];
        float cmax = -INFINITY;
#pragma unroll
        for (int n = 0; n < NK; ++n) {
            float v = allreduce_bits<CP, S::LOG2L, OpSum>(part[n << CP]);
            if constexpr (kPackedQ)
                v *= a.qscale;
            const int item = (n << CP) | phi;
            const int ld = item >> S::LOG2G;
            const int tok = (ld / NIB) * kBlockTokens + (ld % NIB) * RPI + r;
            s_tok[n] = tok;
            v = (ct0 + tok < ctx) ? v : -INFINITY;
            s[n] = v;
            cmax = fmaxf(cmax, v);
        }
        // Maximum over every lane that holds the same head.
        cmax = allreduce_bits<S::LOG2G, 6, OpMax>(cmax);
        const float m_new = fmaxf(m_run, cmax);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        float psum = 0.0f;
#pragma unroll
        for (int n = 0; n < NK; ++n) {
            const float pv = __builtin_amdgcn_exp2f(s[n] - m_new);
            psum += pv;
            p_lds[s_tok[n]][my_head] = pv;
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;

        // Rescale the running output rows of every head (lane h holds head h).
        float alpha_h[G];
#pragma unroll
        for (int h = 0; h < G; ++h)
            alpha_h[h] = read_lane(alpha, h);
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < E; ++e)
                o_acc[h][e] *= alpha_h[h];

        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // P.V over this lane's chunk of V rows.
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            float vf[E];
            Elem<T>::unpack(vd[i], vf);
            const int tok = (i / NIB) * kBlockTokens + (i % NIB) * RPI + r;
            float pw[G];
#pragma unroll
            for (int h = 0; h < G; ++h)
                pw[h] = p_lds[tok][h];
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < E; ++e)
                    o_acc[h][e] = __builtin_fmaf(pw[h], vf[e], o_acc[h][e]);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        append_settled = true;  // this chunk's loads are done, and so are older stores
    }

    // live == false: a chunk past the piece's end, issued with empty
    // descriptors (see run_chunks).
    __device__ void issue_chunk(int ch, u32x4 (&kd)[NU], u32x4 (&vd)[NU], bool live = true)
    {
        if (live) {
            cover_blocks(ch * S::U, (ch + 1) * S::U - 1);
            if (append_pending) {  // the piece's first chunk: store the new row now
                store_new_token();
                append_pending = false;
                append_settled = false;
            }
            // The chunk that holds the new row must see it: the stores are
            // done once any chunk issued after them has been used, else wait.
            if (new_pos >= ch * CT && new_pos < (ch + 1) * CT && !append_settled)
                wait_vector_memory();
        }
        load_chunk(ch, kd, vd, live);
    }

    // Chunks [ch0, ch1) of the current segment, two in flight: the next
    // chunk is loaded before the current one is used (two register sets,
    // alternating).  With eight query heads per KV head the second set would
    // take the kernel past 256 VGPRs, i.e. below the two waves per SIMD the
    // automatic plan launches for 16-bit storage; those go one at a time.
    //
    // Inside the loop the next chunk's loads are issued on every iteration,
    // past the piece's last chunk with empty descriptors (no memory access):
    // with an issue that only some paths make, the compiler's waits for the
    // current chunk count as if the next one were not in flight and wait for
    // it as well.  A one-chunk piece takes a path of its own, so that it
    // issues no empty chunk.
    //
    // ctr: when not null, the piece's arrival counter, claimed right after the
    // first chunk's loads (one place in the code, so the compiler keeps the
    // result where the swap left it).
    __device__ void run_chunks(int ch0, int ch1, uint64_t *ctr)
    {
        auto claim = [&]() {
            claim_seen = 0;
            if (ctr != nullptr && lane == 0)
                claim_seen = claim_counter(ctr, a.epoch);
        };
        if constexpr (decode_chunks_in_flight(G) == 2) {
            u32x4 ka[NU], va[NU], kb[NU], vb[NU];
            issue_chunk(ch0, ka, va);
            claim();
            if (ch0 + 1 >= ch1)
                consume_chunk(ch0, ka, va);
            else
                for (int ch = ch0;;) {
                    issue_chunk(ch + 1, kb, vb, ch + 1 < ch1);
                    consume_chunk(ch, ka, va);
                    if (++ch >= ch1)
                        break;
                    issue_chunk(ch + 1, ka, va, ch + 1 < ch1);
                    consume_chunk(ch, kb, vb);
                    if (++ch >= ch1)
                        break;
                }
        } else {
            {
                u32x4 kd[NU], vd[NU];
                issue_chunk(ch0, kd, vd);
                claim();
                consume_chunk(ch0, kd, vd);
            }
            for (int ch = ch0 + 1; ch < ch1; ++ch) {
                u32x4 kd[NU], vd[NU];
                issue_chunk(ch, kd, vd);
                consume_chunk(ch, kd, vd);
            }
        }
    }

    // Fused decode step.  The segment's new K and V rows belong at position
    // ctx - 1, inside the segment's last chunk, which only this wave reads.
    // Each lane takes its 16-byte column of both rows from k_new / v_new when
    // the piece starts and stores them to the pool just before the piece's
    // first chunk is loaded.  Stores and loads complete in order, so once a
    // chunk loaded after the stores has been used the stores are done; the
    // chunk holding the position waits for them only if none has (a piece of
    // one or two chunks).
    __device__ void prepare_new_token()
    {
        const size_t src = ((size_t)b * a.num_kv_heads + g) * D + c * E;
        knew = *reinterpret_cast<const u32x4 *>((const T *)a.k_new + src);
        vnew = *reinterpret_cast<const u32x4 *>((const T *)a.v_new + src);
        new_pos = ctx - 1;
        append_pending = true;
    }

    __device__ void store_new_token() const
    {
        const int n = new_pos / kBlockTokens;
        const int blk = n - win0 < 64 ? block_at(n)
                                      : __builtin_amdgcn_readfirstlane(
                                            a.block_tables[(size_t)b * a.max_blocks + n]);
        if (r == 0) {  // lanes 0 .. L-1: one 16-byte column of the row each
            const size_t dst =
                (((size_t)blk * a.num_kv_heads + g) * kBlockTokens + new_pos % kBlockTokens) * D +
                c * E;
            *reinterpret_cast<u32x4 *>((T *)const_cast<void *>(a.k_cache) + dst) = knew;
            *reinterpret_cast<u32x4 *>((T *)const_cast<void *>(a.v_cache) + dst) = vnew;
        }
    }

    // Values of the flattened [G][E] output rows a lane keeps after
    // reduce_piece: G * D / 64 (one to sixteen).
    static constexpr int kOut = G * D / 64;
    static_assert(kOut >= 1 && (G * E) % kOut == 0, "scatter width");
    __device__ float &acc_at(int i) { return o_acc[i / E][i % E]; }

    // One reduce-scatter step over lane bit K on the first 2n flattened
    // values: lanes with the bit clear keep the sums of values [0, n), lanes
    // with it set those of [n, 2n), in slots [0, n).  The swap instructions
    // exchange two registers between the lane halves in one instruction, so
    // a step costs one swap and one add per value kept.
    template <int K, int n>
    __device__ void scatter_step()
    {
#pragma unroll
        for (int i = 0; i < n; ++i) {
            const float x = acc_at(i), y = acc_at(i + n);
            if constexpr (K == 5 || K == 4) {
                const auto p =
                    K == 5 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y),
                                                              false, false)
                           : __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y),
                                                              false, false);
                acc_at(i) = __uint_as_float(p[0]) + __uint_as_float(p[1]);
            } else {
                static_assert(K == 3, "row bits start at lane bit 3");
                const bool hi = (lane >> 3) & 1;
                acc_at(i) = (hi ? y : x) + xor_partner<8>(hi ? x : y);
            }
        }
    }

    // Reduce the piece's per-lane state to per-head totals.  Every lane ends
    // with the exponential sum of head my_head in l_run.  The output rows
    // are reduce-scattered over the row bits of the lane index (LOG2L..5,
    // highest first): lane (c, r) ends with kOut sums in o_acc's first
    // flattened slots, those of flattened indices [r kOut, (r + 1) kOut) of
    // column chunk c.  An all-reduce would cost two instructions per value at
    // every step (plus a copy per swap); this costs two per value kept.
    __device__ void reduce_piece()
    {
        // Lanes that differ only in directly-summed row bits hold copies of
        // the same scores; count each score once.
        const float l_once = ((c >> CP) == 0) ? l_run : 0.0f;
        l_run = allreduce_bits<S::LOG2G, 6, OpSum>(l_once);
        constexpr int steps = 6 - S::LOG2L;
        if constexpr (steps >= 1)
            scatter_step<5, G * E / 2>();
        if constexpr (steps >= 2)
            scatter_step<4, G * E / 4>();
        if constexpr (steps >= 3)
            scatter_step<3, G * E / 8>();
    }

    __device__ O *out_rows(int b_, int g_) const
    {
        return (O *)a.out + ((size_t)b_ * a.num_kv_heads * G + (size_t)g_ * G) * D;
    }

    // Flattened index i of chunk c, as an offset into [G][D] rows.
    __device__ int row_offset(int i) const { return (i / E) * D + c * E + i % E; }

    __device__ void write_output()
    {
        O *dst = out_rows(b, g);
        float inv_l[G];
#pragma unroll
        for (int h = 0; h < G; ++h)
            inv_l[h] = 1.0f / read_lane(l_run, h);
        // Groups of consecutive values inside one head.
        constexpr int kGrp = kOut < E ? kOut : E;
#pragma unroll
        for (int j0 = 0; j0 < kOut; j0 += kGrp) {
            const int i0 = r * kOut + j0;
            const int h = i0 / E;
            float inv = inv_l[0];
#pragma unroll
            for (int hh = 1; hh < G; ++hh)
                inv = h == hh ? inv_l[hh] : inv;
            float v[kGrp];
#pragma unroll
            for (int j = 0; j < kGrp; ++j)
                v[j] = acc_at(j0 + j) * inv;
            store_out_n<O, kGrp>(dst + row_offset(i0), v);
        }
    }

    // Record layout (fp32): o[G][D] unnormalised rows, then (m, l) of each
    // head; REC floats per record (a multiple of four).  Every lane stores
    // its kOut values, in 16-byte pieces where it holds four or more.
    __device__ void store_record(float *rec)
    {
        const __amdgpu_buffer_rsrc_t rs = record_rsrc(rec, S::REC);
        constexpr int kGrp = kOut < 4 ? kOut : 4;
#pragma unroll
        for (int j0 = 0; j0 < kOut; j0 += kGrp) {
            const int off = row_offset(r * kOut + j0) * 4;
            if constexpr (kGrp == 4) {
                const u32x4 v{__float_as_uint(acc_at(j0)), __float_as_uint(acc_at(j0 + 1)),
                              __float_as_uint(acc_at(j0 + 2)), __float_as_uint(acc_at(j0 + 3))};
                __builtin_amdgcn_raw_buffer_store_b128(v, rs, off, 0, kDeviceScope);
            } else if constexpr (kGrp == 2) {
                const u32x2 v{__float_as_uint(acc_at(j0)), __float_as_uint(acc_at(j0 + 1))};
                __builtin_amdgcn_raw_buffer_store_b64(v, rs, off, 0, kDeviceScope);
            } else {
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc_at(j0)), rs, off, 0,
                                                      kDeviceScope);
            }
        }
        if (lane < G)
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(m_run), __float_as_uint(l_run)},
                                                  rs, (G * D + 2 * lane) * 4, 0, kDeviceScope);
    }

    // Fold the records of slices [s_first, s_last] into one lane's running
    // (m, lsum, o) for outputs i .. i+3 of head h, kBatch records per round
    // trip.  Slots past s_last load zeros without touching memory, and with
    // m = -inf they add exact zeros, so a call takes the same values whatever
    // kBatch covers it in one pass.
    template <int kBatch>
    __device__ void fold_records(int s_first, int s_last, int first_role, int i, int h, float &m,
                                 float &lsum, float (&o)[4]) const
    {
        for (int s0 = s_first; s0 <= s_last; s0 += kBatch) {
            // One descriptor over the batch's records (two per slice, role 0
            // then role 1), offsets in the vector operand so that the range
            // check covers them: slots past s_last fall outside and load zeros.
            const int nrec = 2 * (min(s_last + 1, s0 + kBatch) - s0);
            const __amdgpu_buffer_rsrc_t rs =
                record_rsrc(a.ws_rec + (size_t)s0 * 2 * S::REC, nrec * S::REC);
            float mj[kBatch], lj[kBatch];
            u32x4 oj[kBatch];
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                const int s = s0 + k;
                const bool in = s <= s_last;
                const int role = s == s_first ? first_role : 0;
                const int rec = (2 * k + role) * S::REC * 4;
                oj[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, rec + i * 4, 0, kDeviceScope);
                const u32x2 ml = __builtin_amdgcn_raw_buffer_load_b64(rs, rec + (G * D + 2 * h) * 4, 0,
                                                                      kDeviceScope);
                mj[k] = in ? __uint_as_float(ml[0]) : -INFINITY;
                lj[k] = __uint_as_float(ml[1]);
            }
            float m_new = m;
#pragma unroll
            for (int k = 0; k < kBatch; ++k)
                m_new = fmaxf(m_new, mj[k]);
            const float rescale = __builtin_amdgcn_exp2f(m - m_new);
            lsum *= rescale;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o[e] *= rescale;
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                const float f = __builtin_amdgcn_exp2f(mj[k] - m_new);
                lsum = __builtin_fmaf(f, lj[k], lsum);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    o[e] = __builtin_fmaf(f, __uint_as_float(oj[k][e]), o[e]);
            }
            m = m_new;
        }
    }

    // Merge the records of every piece of segment (sb, sg), units [su0, su1),
    // in slice order, and write the normalised output.  Each lane folds four
    // consecutive outputs of one head.  Up to eight records (every segment
    // of the batch-16 workloads) are loaded in one pass of eight, more in
    // passes of sixteen (one round trip for the 16 one-unit pieces of a
    // batch-1 segment of 512 tokens; the registers of the chunk loop are free
    // here).
    __device__ void merge_segment(int sb, int sg, const SegmentSlices &ss) const
    {
        const int s_first = ss.first, s_last = ss.last, first_role = ss.first_role;
        O *dst = out_rows(sb, sg);
        compiler_memory_barrier();
        for (int v = lane; v < G * D / 4; v += 64) {
            const int i = 4 * v;  // first of this lane's four outputs
            const int h = i / D;
            float m = -INFINITY, lsum = 0.0f, o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if (s_last - s_first < 8)
                fold_records<8>(s_first, s_last, first_role, i, h, m, lsum, o);
            else
                fold_records<16>(s_first, s_last, first_role, i, h, m, lsum, o);
            const float inv = 1.0f / lsum;
            float r4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                r4[e] = o[e] * inv;
            store_out_n<O, 4>(dst + i, r4);
        }
    }
};

// Inclusive prefix sums of two values per thread over the workgroup.
__device__ int2 block_inclusive_scan2(int2 v, int2 *wave_totals)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    v.x = wave_inclusive_sum(v.x);
    v.y = wave_inclusive_sum(v.y);
    if (lane == 63)
        wave_totals[wave] = v;
    __syncthreads();
    int2 before = make_int2(0, 0);
    for (int w = 0; w < wave; ++w) {
        before.x += wave_totals[w].x;
        before.y += wave_totals[w].y;
    }
    __syncthreads();
    return make_int2(v.x + before.x, v.y + before.y);
}

// The context lengths and the batch size come first, as arguments of their
// own: the library builds this kernel with them preloaded into scalar
// registers at dispatch, so the context-length load, the first link of the
// kernel's chain of dependent loads, is issued without waiting for a load of
// the kernel arguments (the other arguments are loaded meanwhile).
template <typename T, typename O, int D, int G>
__global__ __launch_bounds__(kDecodeWaves * 64) void paged_decode_kernel(
    const int32_t *context_lens, int num_seqs, KernelArgs a)
{
    using S = Shape<T, D, G>;
    constexpr int CT = S::CT;
    constexpr int WAVES = kDecodeWaves;
    constexpr int NT = WAVES * 64;

    __shared__ int unit_end[kMaxDecodeSeqs];  // inclusive prefix of units per sequence
    __shared__ int ne_end[kMaxDecodeSeqs];    // inclusive count of non-empty sequences
    __shared__ int ctx_lds[kMaxDecodeSeqs];
    __shared__ int2 wave_totals[WAVES];
    __shared__ __attribute__((aligned(16))) float p_lds[WAVES][CT][G];
    constexpr bool kEarlyClaimRows = S::EB == 2 && D == 64;

    const int B = num_seqs;
    const int hkv = a.num_kv_heads;

    // Per sequence: its context length, and the inclusive prefix sums of
    // units (Hkv * chunks) and of non-empty sequences.  Up to 64 sequences,
    // every wave computes them for itself in registers (lane b holds
    // sequence b; a wave-wide scan, no workgroup barrier and no LDS).  Larger
    // batches scan over the workgroup into LDS, each thread owning a
    // contiguous run of sequences.
    const int lane = threadIdx.x & 63;
    const bool small = B <= 64;
    int r_ctx = 0, r_end = 0, r_ne = 0;
    if (small) {
        const int cl = lane < B ? context_lens[lane] : 0;
        r_ctx = cl;
        r_end = wave_inclusive_sum(hkv * ((cl + CT - 1) / CT));
        r_ne = wave_inclusive_sum(cl > 0 ? 1 : 0);
    } else {
        // Each thread owns `per` consecutive sequences; their lengths are
        // all loaded before any is used (one round trip, not `per`).
        constexpr int kMaxPer = (kMaxDecodeSeqs + NT - 1) / NT;
        const int per = (B + NT - 1) / NT;
        const int first = threadIdx.x * per;
        int cls[kMaxPer];
#pragma unroll
        for (int j = 0; j < kMaxPer; ++j)
            cls[j] = (j < per && first + j < B) ? context_lens[first + j] : 0;
        int2 mine = make_int2(0, 0);
#pragma unroll
        for (int j = 0; j < kMaxPer; ++j) {
            const int bb = first + j;
            if (j < per && bb < B) {
                const int cl = cls[j];
                ctx_lds[bb] = cl;
                mine.x += hkv * ((cl + CT - 1) / CT);
                mine.y += cl > 0 ? 1 : 0;
            }
        }
        int2 run = block_inclusive_scan2(mine, wave_totals);
        run.x -= mine.x;
        run.y -= mine.y;
#pragma unroll
        for (int j = 0; j < kMaxPer; ++j) {
            const int bb = first + j;
            if (j < per && bb < B) {
                const int cl = cls[j];
                run.x += hkv * ((cl + CT - 1) / CT);
                run.y += cl > 0 ? 1 : 0;
                unit_end[bb] = run.x;
                ne_end[bb] = run.y;
            }
        }
        __syncthreads();
    }
    // Accessors for a wave-uniform sequence index.  Values read from LDS are
    // the same in every lane, but the compiler cannot know that;
    // readfirstlane keeps everything derived from them in scalar registers
    // (a divergent buffer descriptor would wrap each load in a waterfall
    // loop).
    auto ctx_of = [&](int bb) -> int {
        return small ? __builtin_amdgcn_readlane(r_ctx, bb)
                     : __builtin_amdgcn_readfirstlane(ctx_lds[bb]);
    };
    auto end_of = [&](int bb) -> int {
        return small ? __builtin_amdgcn_readlane(r_end, bb)
                     : __builtin_amdgcn_readfirstlane(unit_end[bb]);
    };
    auto ne_of = [&](int bb) -> int {
        return small ? __builtin_amdgcn_readlane(r_ne, bb)
                     : __builtin_amdgcn_readfirstlane(ne_end[bb]);
    };

    const int total = end_of(B - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int s = blockIdx.x * WAVES + wave;

    // Sequences with an empty context have no units; their rows are zero.
    for (int bb = s; bb < B; bb += a.num_waves) {
        if (ctx_of(bb) == 0) {
            O *row = (O *)a.out + (size_t)bb * hkv * G * D;
            for (int i = lane; i < hkv * G * D; i += 64)
                row[i] = Elem<O>::from_float(0.0f);
        }
    }
    // Slices split the list in which every non-empty segment starts with C
    // empty units (none for small calls, whose slices would hold one or two
    // entries).  At most one wavefront per kMinUnitsPerWave entries of that
    // list, but no fewer than kMinWaves (or one per unit): a wave's fixed
    // costs (prefix, first table window and round trip, record, arrival,
    // merge) are paid once per slice, and fewer, longer slices also mean
    // fewer records and arrivals per segment, until too few waves are left
    // to hide memory latency.  Slices hold at least three list entries when
    // C > 0, so every slice holds work, and every slice between two others
    // holds a record of any segment spanning them.
    const int C = total >= kChargeFromUnits ? kBoundaryUnits : 0;
    const int total_v = total + C * hkv * ne_of(B - 1);
    const int nw = min(a.num_waves, max((total_v + kMinUnitsPerWave - 1) / kMinUnitsPerWave,
                                        min(total, kMinWaves)));
    if (s >= nw)
        return;
    const int v_begin = slice_start(s, total_v, nw);
    const int v_end = slice_start(s + 1, total_v, nw);
    // End of sequence bb's entries in that list (any lane's bb; LDS path).
    auto seq_end_lds = [&](int bb) { return unit_end[bb] + C * hkv * ne_end[bb]; };

    WaveDecoder<T, O, D, G> w(a, p_lds[wave]);

    // First sequence whose entries reach past v_begin (the ends are
    // non-decreasing and the last, total_v, exceeds v_begin): one ballot
    // over the registers of a small batch; for larger ones two ballots
    // instead of a binary search of dependent LDS reads (lane i first tests
    // the last entry of group i of `step` sequences; then lane j tests entry
    // j of the first group that reaches past v_begin).
    int b;
    if (small) {
        b = __builtin_ctzll(__builtin_amdgcn_ballot_w64(lane < B && r_end + C * hkv * r_ne > v_begin));
        b = b < B ? b : B - 1;  // (v_begin < total_v, so some lane qualifies)
    } else {
        const int step = (B + 63) / 64;
        const int grp = __builtin_ctzll(__builtin_amdgcn_ballot_w64(
            lane * step < B && seq_end_lds(min(B - 1, lane * step + step - 1)) > v_begin));
        b = grp * step + __builtin_ctzll(__builtin_amdgcn_ballot_w64(
            lane < step && grp * step + lane < B && seq_end_lds(min(B - 1, grp * step + lane)) > v_begin));
    }
    int v = v_begin;
    bool first_piece = true;
    // A first piece that ends inside the slice leaves its arrival pending:
    // it is counted once the next piece's first loads are on their way, so
    // the record stores complete during that round trip instead of stalling
    // the wave, and the count's result is only read at the end (merging
    // then, should this wave have completed the segment).
    bool pend = false, pend_count_now = false;
    int pend_b = 0, pend_g = 0, pend_nch = 0, pend_units = 0, pend_old = 0;
    SegmentSlices pend_slices{0, 0, 0};
    uint64_t pend_seen = 0;  // lane 0: what the pending piece's claim found
    while (true) {
        const int seq_end = end_of(b) + C * hkv * ne_of(b);
        const int ctx = ctx_of(b);
        const int nch = (ctx + CT - 1) / CT;  // > 0: v lies inside sequence b
        const int stride = nch + C;           // list entries per segment
        const int seq_begin = seq_end - hkv * stride;
        const int g = (v - seq_begin) / stride;
        const int seg_v0 = seq_begin + g * stride;  // first entry of segment (b, g)
        const int r0 = max(v, seg_v0 + C);
        if (r0 >= v_end)  // only empty units left in this slice
            break;
        const int r1 = min(v_end, seg_v0 + stride);
        const int ch0 = r0 - seg_v0 - C;
        const int ch1 = r1 - seg_v0 - C;

        w.begin_piece(b, g, ctx, ch0);
        const bool appends = a.k_new != nullptr && ch1 == nch;
        if (appends)
            w.prepare_new_token();
        if (pend_count_now) {
            // the record stores before, this piece's window and query loads
            // after: one wait covers both, then the arrival counts
            wait_vector_memory();
            int old = 0;
            if (lane == 0)
                old = (int)arrive_counter(&a.ws_count[(size_t)pend_b * hkv + pend_g], a.epoch,
                                          pend_seen, pend_units);
            pend_old = old;
            pend_count_now = false;
        }
        // Where a piece that is not a whole segment claims its arrival
        // counter: with the first chunk's loads for 16-bit rows of 64
        // elements and for one-chunk pieces, else with the record stores.
        // An early claim takes the swap out of the tail, where it returns
        // after the stores (bf16 batch 16: 15.1 -> 14.2 us, batch 1: 9.1 ->
        // 8.3 us), but loads issued after it complete behind it, which costs
        // more than that when a wave keeps 32 KiB in flight over several
        // chunks (fp32 batch 16: 18.9 -> 19.3 us, long context: +0.4 us).
        const bool whole = ch0 == 0 && ch1 == nch;
        const bool early_claim = !whole && (kEarlyClaimRows || ch1 - ch0 == 1);
        w.run_chunks(ch0, ch1, early_claim ? &a.ws_count[(size_t)b * hkv + g] : nullptr);
        w.reduce_piece();
        if (whole) {
            w.write_output();
        } else {
            const int role = first_piece ? 0 : 1;
            w.store_record(a.ws_rec + ((size_t)s * 2 + role) * S::REC);
            // Otherwise claim the segment's counter now; the wait for the
            // record stores below also covers the swap.
            uint64_t seen = 0;
            if (early_claim)
                seen = w.claim_seen;
            else if (lane == 0)
                seen = claim_counter(&a.ws_count[(size_t)b * hkv + g], a.epoch);
            if (first_piece && r1 + C < v_end) {  // another piece follows in this slice
                pend = pend_count_now = true;
                pend_seen = seen;
                pend_b = b;
                pend_g = g;
                pend_slices = segment_slices(seg_v0, seg_v0 + C, seg_v0 + stride, total_v, nw);
                pend_nch = nch;
                pend_units = ch1 - ch0;
            } else {
                // The merge's slice bounds, in the shadow of the stores and the count.
                const SegmentSlices ss = segment_slices(seg_v0, seg_v0 + C, seg_v0 + stride, total_v, nw);
                wait_vector_memory();
                int done = 0;
                if (lane == 0)
                    done = (int)arrive_counter(&a.ws_count[(size_t)b * hkv + g], a.epoch, seen,
                                               ch1 - ch0);
                done = __builtin_amdgcn_readfirstlane(done) + (ch1 - ch0);
                if (done == nch) {
                    w.merge_segment(b, g, ss);
                    if (lane == 0)
                        release_counter(&a.ws_count[(size_t)b * hkv + g]);
                }
            }
        }
        first_piece = false;
        v = r1;
        if (v >= v_end)
            break;
        if (v == seq_end) {  // move on to the next sequence that has units
            ++b;
            while (b < B && end_of(b) == end_of(b - 1))
                ++b;
        }
    }
    if (pend && __builtin_amdgcn_readfirstlane(pend_old) + pend_units == pend_nch) {
        w.merge_segment(pend_b, pend_g, pend_slices);
        if (lane == 0)
            release_counter(&a.ws_count[(size_t)pend_b * hkv + pend_g]);
    }
}

template <typename T, typename O, int D, int G>
hipError_t launch_typed(const DecodeArgs &d, hipStream_t stream)
{
    KernelArgs a;
    a.q = d.q;
    a.k_cache = d.k_cache;
    a.v_cache = d.v_cache;
    a.k_new = d.k_new;
    a.v_new = d.v_new;
    a.block_tables = d.block_tables;
    a.out = d.out;
    a.ws_count = d.ws_count;
    a.ws_rec = d.ws_rec;
    a.num_kv_heads = d.num_kv_heads;
    a.max_blocks = d.max_blocks;
    a.num_waves = d.num_waves;
    a.qscale = d.qscale;
    a.epoch = d.epoch;
    hipLaunchKernelGGL((paged_decode_kernel<T, O, D, G>), dim3(d.num_waves / kDecodeWaves),
                       dim3(kDecodeWaves * 64), 0, stream, d.context_lens, d.num_seqs, a);
    return hipGetLastError();
}

template <typename T, typename O, int D>
hipError_t launch_group(const DecodeArgs &a, hipStream_t stream)
{
    switch (a.group) {
    case 1: return launch_typed<T, O, D, 1>(a, stream);
    case 2: return launch_typed<T, O, D, 2>(a, stream);
    case 4: return launch_typed<T, O, D, 4>(a, stream);
    case 8: return launch_typed<T, O, D, 8>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

template <typename T, typename O>
hipError_t launch_dim(const DecodeArgs &a, hipStream_t stream)
{
    switch (a.head_dim) {
    case 64: return launch_group<T, O, 64>(a, stream);
    case 128: return launch_group<T, O, 128>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

// 16-bit storage with the output in its own type or in fp32.
template <typename T>
hipError_t launch_out(const DecodeArgs &a, hipStream_t stream)
{
    return a.out_f32 ? launch_dim<T, float>(a, stream) : launch_dim<T, T>(a, stream);
}

}  // namespace

hipError_t launch_paged_decode(const DecodeArgs &a, hipStream_t stream)
{
    switch (a.dtype) {
    case kDtypeF32: return launch_dim<float, float>(a, stream);
    case kDtypeF16: return launch_out<_Float16>(a, stream);
    case kDtypeBF16: return launch_out<__bf16>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace photon
