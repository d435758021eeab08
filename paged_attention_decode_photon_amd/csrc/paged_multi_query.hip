// Multi-query paged attention with a causal tail, for gfx950 matrix cores.
//
// Operation (PhotonInfer README: "GPU-optimised kernels", batched paged
// attention over the block-level KV cache; the roadmap's speculative
// decoding and the scheduler's chunked admission both need several new
// tokens of a sequence attended at once): sequence b owns query rows
// query_start[b] .. query_start[b+1]-1, the last n_b of its context_lens[b]
// tokens; row j of b, at position p = ctx - n_b + j, attends to the tokens
// t <= p of its sequence through the block table:
//   out = sum_{t<=p} exp(s_t - m) V_t / sum_{t<=p} exp(s_t - m),
//   s_t = scale * <q, K_t>, with KV head g = h / G for query head h.
//
// Work decomposition.  The n_b * G query rows of one (sequence, KV head)
// are ordered token-major (row = j * G + head offset) and cut into tiles of
// 16 rows.  A tile's causal range of KV blocks is cut into splits of
// split_blocks blocks (grid z); a workgroup of four waves takes one split of
// one tile, each wave taking every fourth block with two in flight, and the
// four partial softmax states are merged through LDS.  (Long query runs use
// the wide variant below: four tiles per workgroup sharing each K/V block.)
// A tile with one split writes its
// rows directly.  Otherwise each workgroup stores its (max, sum, unnormalised
// rows) record with device-scope stores, waits for them, and counts its
// arrival on the tile's counter; the workgroup that completes the count
// merges the records in split order (deterministic) and resets the counter.
// Records cross XCDs, whose L2 caches are not coherent with each other, so
// they are written and read with device-scope (sc1) buffer accesses rather
// than behind cache-wide fences.
//
// Matrix-core mapping (16x16 MFMA: K = 4 for fp32; K = 16 or, in the wide
// variant and for P.V, K = 32 for 16-bit storage).  Per KV block the wave
// forms S^T = K Q^T (16 tokens x 16 rows): lane l supplies token l % 16 of K
// and row l % 16 of Q, both over the same quarter D/4 * (l / 16) .. of the
// head dimension, since a contraction may visit the head dimension in any
// order as long as both operands agree; each lane then holds
// S^T[4 (l/16) + i][l % 16], i.e. four tokens of its own row, which is
// exactly the B-operand layout of O^T = V^T P^T.  The V^T operand (four
// consecutive tokens of one column per lane) comes from an LDS tile: fp32 V
// is stored transposed, 16-bit V row-major and read back with the gfx950
// transposing read.  For 16-bit storage P is split into a rounded part and
// its rounding residual, which keeps the weights as accurate as fp32.
// Masked tokens (past a row's position, or
// past the context in the last block) get -inf scores and zero K/V rows
// (raw buffer loads past the valid rows return zero), so pool padding never
// reaches the arithmetic.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "arrival.h"
#include "elem.h"
#include "lane_ops.h"
#include "launch.h"

namespace photon {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short lds_i16x4 __attribute__((ext_vector_type(4)));

constexpr int kMqWaves = 4;
constexpr int kSc1 = 16;  // cache-policy bits of device-scope record accesses

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rec_rsrc(float *rec, int floats)
{
    return __builtin_amdgcn_make_buffer_rsrc(rec, (short)0, floats * 4, 0x00020000);
}
constexpr int kRawWord3 = 0x00020000;
constexpr int kTile = 16;  // query rows per tile, tokens per KV block

__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Round four fp32 values to the 16-bit storage type (nearest even), as raw bits.
template <typename T>
__device__ __forceinline__ u32x2 round4(const float (&p)[4])
{
    u32x2 r;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        typedef T t2 __attribute__((ext_vector_type(2)));
        t2 v;
        v[0] = (T)p[2 * k];
        v[1] = (T)p[2 * k + 1];
        const uint32_t w = __builtin_bit_cast(uint32_t, v);
        r[k] = w;
    }
    return r;
}

template <typename T>
__device__ __forceinline__ void widen4(const u32x2 &w, float (&f)[4])
{
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        typedef T t2 __attribute__((ext_vector_type(2)));
        const uint32_t word = w[k];
        const t2 v = __builtin_bit_cast(t2, word);
        f[2 * k] = (float)v[0];
        f[2 * k + 1] = (float)v[1];
    }
}

// One 16x16x32 MFMA on raw 16-bit operands (eight values per lane; gfx950).
// Lane l holds A[m = l % 16][k = 8 (l / 16) + i] and B[k][n = l % 16] for
// i < 8, and receives D[4 (l / 16) + i][l % 16] as the 16x16x16 form does
// (checked with an in-bounds probe).
template <typename T>
__device__ __forceinline__ f32x4 mfma32(const u32x4 &a, const u32x4 &b, f32x4 c)
{
    if constexpr (__is_same(T, _Float16)) {
        typedef _Float16 h8 __attribute__((ext_vector_type(8)));
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a),
                                                      __builtin_bit_cast(h8, b), c, 0, 0, 0);
    } else {
        typedef __bf16 b8 __attribute__((ext_vector_type(8)));
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, a),
                                                       __builtin_bit_cast(b8, b), c, 0, 0, 0);
    }
}

// widen4 written on the packed bits: bfloat16 widens by a shift or a mask
// of the word it was packed in (so the compiler does not re-round the fp32
// source); binary16 converts each half.
template <typename T>
__device__ __forceinline__ void widen_packed(const u32x2 &w, float (&f)[4])
{
    if constexpr (__is_same(T, __bf16)) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            uint32_t word = w[k];
            // hide the word's origin: otherwise the compiler re-rounds the
            // low half's source value instead of shifting the packed word
            asm("" : "+v"(word));
            f[2 * k] = __uint_as_float(word << 16);
            f[2 * k + 1] = __uint_as_float(word & 0xffff0000u);
        }
    } else {
        widen4<T>(w, f);
    }
}

// One 16x16x16 MFMA on raw 16-bit operands (four values per lane).
template <typename T>
__device__ __forceinline__ f32x4 mfma16(const u32x2 &a, const u32x2 &b, f32x4 c)
{
    if constexpr (sizeof(T) == 2 && __is_same(T, _Float16))
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                     __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                         __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}

// Transposing LDS read of 16-bit data (gfx950).  Within each group of 16
// lanes, lane i returns element i % 4 of the 8 bytes read by lane
// 4 k + i / 4, for k = 0..3: when lane w of the group points at row w / 4
// (4 consecutive elements starting at column 4 (w % 4)) of a row-major
// tile, lane i receives column i of those 4 rows, i.e. one column of the
// tile across 4 consecutive rows.
__device__ __forceinline__ u32x2 lds_read_transposed(const void *p)
{
    const lds_i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) lds_i16x4 *)p);
    return __builtin_bit_cast(u32x2, v);
}

// The online-softmax state of one wave's 16 query rows (lane l: row l % 16)
// and the three per-block steps both kernels share.
template <typename T, int D>
struct TileState {
    static constexpr int EB = sizeof(T);
    static constexpr int QD = D / 4;           // head-dimension elements per lane
    static constexpr int NW = QD * EB / 4;     // dwords of them
    static constexpr int MT = D / 16;          // 16-wide output column tiles
    static constexpr int VS = kTile + 4;       // LDS row stride of a transposed V tile

    float m_run = -INFINITY, l_lane = 0.0f;
    f32x4 o_acc[MT];

    __device__ TileState()
    {
#pragma unroll
        for (int t = 0; t < MT; ++t)
            o_acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }

    // S^T = K Q^T over one 16-token block: lane l gets tokens 4 (l/16) + i of row l % 16.
    __device__ static f32x4 scores(const uint32_t (&kw)[NW], const uint32_t (&qw)[NW])
    {
        f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (EB == 4) {
#pragma unroll
            for (int k = 0; k < QD; ++k)
                s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kw[k]),
                                                         __uint_as_float(qw[k]), s, 0, 0, 0);
        } else {
#pragma unroll
            for (int k = 0; k < QD / 4; ++k)
                s = mfma16<T>(u32x2{kw[2 * k], kw[2 * k + 1]}, u32x2{qw[2 * k], qw[2 * k + 1]}, s);
        }
        return s;
    }

    // Scores of NB blocks at once, the blocks' MFMA chains interleaved so
    // that no MFMA waits on the one before it.
    template <int NB>
    __device__ static void scores_blocks(const uint32_t (&kw)[NB][NW], const uint32_t (&qw)[NW],
                                         f32x4 (&s)[NB])
    {
#pragma unroll
        for (int bi = 0; bi < NB; ++bi)
            s[bi] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (EB == 4) {
#pragma unroll
            for (int k = 0; k < QD; ++k)
#pragma unroll
                for (int bi = 0; bi < NB; ++bi)
                    s[bi] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kw[bi][k]),
                                                                 __uint_as_float(qw[k]), s[bi], 0, 0, 0);
        } else {
            // K = 32 per MFMA: a lane's head-dimension elements 8 c .. 8 c + 7
            // of its quarter feed MFMA c, the same ones from K and from Q.
#pragma unroll
            for (int c = 0; c < QD / 8; ++c)
#pragma unroll
                for (int bi = 0; bi < NB; ++bi)
                    s[bi] = mfma32<T>(u32x4{kw[bi][4 * c], kw[bi][4 * c + 1], kw[bi][4 * c + 2],
                                            kw[bi][4 * c + 3]},
                                      u32x4{qw[4 * c], qw[4 * c + 1], qw[4 * c + 2], qw[4 * c + 3]},
                                      s[bi]);
        }
    }

    // One softmax update over NB blocks n0 .. n0 + NB - 1 (those with
    // live[bi]): scores in log2 units, tokens past my_pos (or any token of a
    // padding row) masked, unless `unmasked` says every token of the blocks
    // lies at or before every row's position (wave-uniform); p receives the
    // weights.  One maximum reduction per call, however many blocks.
    //
    // The accumulators are rescaled lazily: the reference maximum m_run only
    // moves (and o, l are rescaled) when some row of the wave sees a score
    // more than kSlack above it; otherwise the weights are formed against
    // the old reference and stay below 2^kSlack.  o and l always share one
    // reference, so the normalised result is the same up to rounding.
    static constexpr float kSlack = 8.0f;

    template <int NB>
    __device__ void update(const f32x4 (&s)[NB], const bool (&live)[NB], bool unmasked, int n0,
                           bool row_ok, int my_pos, float qscale, int gq, float (&p)[NB][4])
    {
        if (qscale > 0.0f)  // wave-uniform
            update_impl<NB, true>(s, live, unmasked, n0, row_ok, my_pos, qscale, gq, p);
        else
            update_impl<NB, false>(s, live, unmasked, n0, row_ok, my_pos, qscale, gq, p);
    }

    template <int NB, bool kPos>
    __device__ void update_impl(const f32x4 (&s)[NB], const bool (&live)[NB], bool unmasked,
                                int n0, bool row_ok, int my_pos, float qscale, int gq,
                                float (&p)[NB][4])
    {
        // Token 4 gq + i of block bi is kept while 4 gq + i <= lim_b: lim
        // is this row's last visible position relative to the step's first
        // token (no limit when unmasked, none visible for a padding row), so
        // masking is one compare and one select per score, without branches.
        // With qscale > 0 (every usual scale) the scores stay unscaled until
        // the exponent, where the scale and the maximum fold into one FMA;
        // any other scale multiplies first and exponentiates at scale 1.
        const float post = kPos ? qscale : 1.0f;
        const int big = NB * kTile;
        const int lim = row_ok ? min(my_pos - n0 * kTile, big) : -1;
        float bmax = -INFINITY;
#pragma unroll
        for (int bi = 0; bi < NB; ++bi)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                p[bi][i] = kPos ? s[bi][i] : s[bi][i] * qscale;
        if (!unmasked) {  // wave-uniform; most steps of a long run need no mask
#pragma unroll
            for (int bi = 0; bi < NB; ++bi) {
                const int lim_b = (live[bi] ? lim : -1) - bi * kTile - 4 * gq;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    p[bi][i] = i <= lim_b ? p[bi][i] : -INFINITY;
            }
        }
#pragma unroll
        for (int bi = 0; bi < NB; ++bi)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                bmax = fmaxf(bmax, p[bi][i]);
        bmax = allreduce_pair<16, OpMax>(bmax);
        bmax = allreduce_pair<32, OpMax>(bmax);
        if constexpr (kPos)
            bmax *= qscale;
        if (__builtin_amdgcn_ballot_w64(bmax > m_run + kSlack) != 0) {
            const float m_new = fmaxf(m_run, bmax);
            const float m_use = m_new == -INFINITY ? 0.0f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
            m_run = m_new;
            l_lane *= alpha;
#pragma unroll
            for (int t = 0; t < MT; ++t)
                o_acc[t] *= alpha;
        }
        const float m_use = m_run == -INFINITY ? 0.0f : m_run;
#pragma unroll
        for (int bi = 0; bi < NB; ++bi)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                p[bi][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(p[bi][i], post, -m_use));
        float psum = p[0][0];
#pragma unroll
        for (int bi = 0; bi < NB; ++bi)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (bi != 0 || i != 0)
                    psum += p[bi][i];
        l_lane += psum;
    }

    // O^T += V^T P^T with V row-major in LDS (16 tokens x D, row stride
    // ks), 16-bit storage only: the A operand (column d = 16 t + lr of
    // tokens 4 gq .. 4 gq + 3) comes from one transposing read per tile.
    __device__ void pv_rows(const T *v, int ks, int lr, int gq, const float (&p)[4])
    {
        static_assert(EB == 2, "transposing LDS reads are 16-bit");
        const u32x2 p_hi = round4<T>(p);
        float hi[4], lo[4];
        widen_packed<T>(p_hi, hi);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            lo[i] = p[i] - hi[i];
        const u32x2 p_lo = round4<T>(lo);
        const T *src = &v[(4 * gq + (lr >> 2)) * ks + 4 * (lr & 3)];
        u32x2 va[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t)
            va[t] = lds_read_transposed(src + 16 * t);
        // One K = 32 MFMA per tile takes both parts of the weights: k = 4 g + i
        // pairs token 4 g + i with its rounded weight, k = 4 g + 4 + i with
        // its residual, so the A operand is the same four V values twice.
        const u32x4 pb{p_hi[0], p_hi[1], p_lo[0], p_lo[1]};
#pragma unroll
        for (int t = 0; t < MT; ++t)
            o_acc[t] = mfma32<T>(u32x4{va[t][0], va[t][1], va[t][0], va[t][1]}, pb, o_acc[t]);
    }

    // The same for two blocks at once (v1 = the second block's tile): K = 32
    // pairs k = 4 g + i with token 4 g + i of the first block and
    // k = 4 g + 4 + i with that of the second, so each tile's A operand is
    // two transposing reads side by side; rounded weights and residuals
    // take one MFMA each.
    __device__ void pv_rows2(const T *v0, const T *v1, int ks, int lr, int gq, const float (&p0)[4],
                             const float (&p1)[4])
    {
        static_assert(EB == 2, "transposing LDS reads are 16-bit");
        u32x2 hi[2], lo[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float(&p)[4] = j == 0 ? p0 : p1;
            hi[j] = round4<T>(p);
            float h[4], l[4];
            widen_packed<T>(hi[j], h);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                l[i] = p[i] - h[i];
            lo[j] = round4<T>(l);
        }
        const int off = (4 * gq + (lr >> 2)) * ks + 4 * (lr & 3);
        u32x4 va[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const u32x2 a0 = lds_read_transposed(v0 + off + 16 * t);
            const u32x2 a1 = lds_read_transposed(v1 + off + 16 * t);
            va[t] = u32x4{a0[0], a0[1], a1[0], a1[1]};
        }
        const u32x4 bh{hi[0][0], hi[0][1], hi[1][0], hi[1][1]};
        const u32x4 bl{lo[0][0], lo[0][1], lo[1][0], lo[1][1]};
#pragma unroll
        for (int t = 0; t < MT; ++t)
            o_acc[t] = mfma32<T>(va[t], bh, o_acc[t]);
#pragma unroll
        for (int t = 0; t < MT; ++t)
            o_acc[t] = mfma32<T>(va[t], bl, o_acc[t]);
    }

    // O^T += V^T P^T for fp32 storage with the A operand loaded straight
    // from memory: v[4 t + i] is V[token 4 gq + i][column 16 t + lr].
    __device__ void pv_direct(const uint32_t (&v)[NW], const float (&p)[4])
    {
        static_assert(EB == 4 && NW == 4 * MT, "one dword per tile and token");
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int t = 0; t < MT; ++t)
                o_acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v[4 * t + i]), p[i],
                                                                o_acc[t], 0, 0, 0);
    }

    // O^T += V^T P^T with V^T (D x 16 tokens, row stride VS) in LDS (fp32
    // storage; 16-bit V goes through pv_rows / pv_rows2).
    __device__ void pv(const T *vt, int lr, int gq, const float (&p)[4])
    {
        static_assert(EB == 4, "16-bit V is read through the transposing LDS read");
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const f32x4 va = *reinterpret_cast<const f32x4 *>(&vt[(16 * t + lr) * VS + 4 * gq]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                o_acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(va[i], p[i], o_acc[t], 0, 0, 0);
        }
    }
};

// Workgroup-level running max and exponential sum of tile row r, from the
// W waves' statistics (the same values every lane forms in the merge).
template <int W>
__device__ __forceinline__ float m_all_row(const float (&sm)[W][kTile], int r)
{
    float m = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w)
        m = fmaxf(m, sm[w][r]);
    return m;
}
template <int W>
__device__ __forceinline__ float l_all_row(const float (&sm)[W][kTile], const float (&sl)[W][kTile],
                                           int r)
{
    const float m = m_all_row(sm, r);
    const float mu = m == -INFINITY ? 0.0f : m;
    float l = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w)
        l += sl[w][r] * __builtin_amdgcn_exp2f(sm[w][r] - mu);
    return l;
}

template <typename T, typename O, int D, int G>
__global__ __launch_bounds__(kMqTileWaves * 64) void paged_mq_kernel(MultiQueryArgs a)
{
    constexpr int EB = sizeof(T);
    constexpr int QD = D / 4;              // head-dimension elements per lane
    constexpr int NL = QD * EB / 16;       // 16-byte loads per lane per K (or V) row part
    constexpr int NW = QD * EB / 4;        // dwords per lane per row part
    constexpr int MT = D / 16;             // 16-wide output column tiles
    // One wave's V tile for 16-bit storage: row-major (16 x D, row stride
    // VRS), read back through the transposing LDS read.  fp32 V is loaded
    // straight into the MFMA operand layout and needs none.
    constexpr int VRS = D + 16 / EB;
    constexpr int VT_BYTES = EB == 4 ? 0 : kTile * VRS * EB;
    constexpr int OB_BYTES = kTile * D * 4;
    constexpr int W = kMqTileWaves;
    constexpr int SMEM = (W * VT_BYTES > W * OB_BYTES) ? W * VT_BYTES : W * OB_BYTES;
    __shared__ __attribute__((aligned(16))) char smem[SMEM];
    __shared__ float stat_m[W][kTile], stat_l[W][kTile];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int gq = lane >> 4;   // lane group: head-dimension quarter, token quad
    const int lr = lane & 15;   // this lane's row (Q, S^T column) and K token
    const int hkv = a.num_kv_heads;
    const int b = blockIdx.y / hkv;
    const int g = blockIdx.y - b * hkv;
    const int tile = blockIdx.x;
    const int q0 = a.query_start[b];
    const int nq = a.query_start[b + 1] - q0;
    const int rows = nq * G;
    if (tile * kTile >= rows)
        return;  // the whole workgroup leaves together
    const int ctx = a.context_lens[b];
    const int first_pos = ctx - nq;
    const int last_row = min(tile * kTile + kTile - 1, rows - 1);
    const int scan_end = first_pos + last_row / G + 1;  // tokens [0, scan_end)
    const int nblk = (scan_end + kTile - 1) / kTile;
    const int nsplit = (nblk + a.split_blocks - 1) / a.split_blocks;
    const int z = blockIdx.z;
    if (z >= nsplit)
        return;  // this tile's range has fewer splits
    const int n_begin = z * a.split_blocks;
    const int n_end = min(nblk, n_begin + a.split_blocks);

    const int r = tile * kTile + lr;  // this lane's row
    const bool row_ok = r < rows;
    const int rj = r / G;
    const int my_pos = first_pos + rj;
    const int hq = hkv * G;

    // Q operand: row r over head-dimension quarter gq (zero for padding rows,
    // which read the tile's last real row instead of past the query rows).
    uint32_t qw[NW];
    {
        const int cr = row_ok ? r : rows - 1;
        const int cj = cr / G, ch = cr - (cr / G) * G;
        const T *qrow = (const T *)a.q + ((size_t)(q0 + cj) * hq + (size_t)g * G + ch) * D + gq * QD;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            u32x4 v = reinterpret_cast<const u32x4 *>(qrow)[i];
            if (!row_ok)
                v = u32x4{0, 0, 0, 0};
#pragma unroll
            for (int k = 0; k < 4; ++k)
                qw[4 * i + k] = v[k];
        }
    }

    using TS = TileState<T, D>;
    TS st;
    T *vt = reinterpret_cast<T *>(smem + wave * VT_BYTES);
    const int tile_first_pos = first_pos + (tile * kTile) / G;  // the tile's earliest row
    const size_t tile_elems = (size_t)kTile * D;

    // Issue the K and V loads of block n (rows past scan_end read as zero).
    auto load_block = [&](int n, uint32_t (&kw)[NW], uint32_t (&vw)[NW]) {
        const int blk = __builtin_amdgcn_readfirstlane(a.block_tables[(size_t)b * a.max_blocks + n]);
        const int valid = min(kTile, scan_end - n * kTile);
        const size_t base = ((size_t)blk * hkv + g) * tile_elems;
        const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)((const T *)a.k_cache + base), (short)0, valid * D * EB, kRawWord3);
        const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)((const T *)a.v_cache + base), (short)0, valid * D * EB, kRawWord3);
        const int off = (lr * D + gq * QD) * EB;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const u32x4 kv = __builtin_amdgcn_raw_buffer_load_b128(krs, off + 16 * i, 0, 0);
#pragma unroll
            for (int k = 0; k < 4; ++k)
                kw[4 * i + k] = kv[k];
        }
        if constexpr (EB == 4) {
            // V straight into the A operand of O^T += V^T P^T: dword 4 t + i
            // is V[token 4 gq + i][column 16 t + lr] (four 64-byte runs per
            // load; the block's 4 KiB are read once over the 16 loads).
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    vw[4 * t + i] = __builtin_amdgcn_raw_buffer_load_b32(
                        vrs, ((4 * gq + i) * D + 16 * t + lr) * EB, 0, 0);
        } else {
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                const u32x4 vv = __builtin_amdgcn_raw_buffer_load_b128(vrs, off + 16 * i, 0, 0);
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    vw[4 * i + k] = vv[k];
            }
        }
    };

    // Scores, softmax update and P.V of block n from its loaded K and V.
    auto compute_block = [&](int n, const uint32_t (&kw)[NW], const uint32_t (&vw)[NW]) {
        const f32x4 sc = TS::scores(kw, qw);
        if constexpr (EB == 2) {
            // V row lr, this lane's quarter, as it is (16-byte stores).
#pragma unroll
            for (int i = 0; i < NL; ++i)
                *reinterpret_cast<u32x4 *>(&vt[lr * VRS + gq * QD + 8 * i]) =
                    u32x4{vw[4 * i], vw[4 * i + 1], vw[4 * i + 2], vw[4 * i + 3]};
        }
        float p[1][4];
        const f32x4 sv[1] = {sc};
        const bool live[1] = {true};
        st.template update<1>(sv, live, (n + 1) * kTile - 1 <= tile_first_pos, n, row_ok, my_pos,
                              a.qscale, gq, p);
        if constexpr (EB == 4) {
            st.pv_direct(vw, p[0]);  // V was loaded in the operand layout
        } else {
            wave_sync();  // the V tile is complete
            st.pv_rows(vt, VRS, lr, gq, p[0]);
            wave_sync();  // reads of the V tile are done before the next block overwrites it
        }
    };

    // This wave's blocks n_begin + wave + W j, two in flight at all times:
    // each block's registers are refilled with the block after next as soon
    // as the block has been used.
    {
        constexpr int S = W;
        uint32_t ka[NW], va[NW], kb[NW], vb[NW];
        int n = n_begin + wave;
        if (n < n_end)
            load_block(n, ka, va);
        if (n + S < n_end)
            load_block(n + S, kb, vb);
        while (n < n_end) {
            compute_block(n, ka, va);
            if (n + 2 * S < n_end)
                load_block(n + 2 * S, ka, va);
            n += S;
            if (n >= n_end)
                break;
            compute_block(n, kb, vb);
            if (n + 2 * S < n_end)
                load_block(n + 2 * S, kb, vb);
            n += S;
        }
    }

    // Merge the W waves' partial states of each row.
    float l_row = allreduce_pair<16, OpSum>(st.l_lane);
    l_row = allreduce_pair<32, OpSum>(l_row);
    const float m_run = st.m_run;
    if (gq == 0) {
        stat_m[wave][lr] = m_run;
        stat_l[wave][lr] = l_row;
    }
    __syncthreads();  // also ends every wave's use of the V tiles
    const float m_all = m_all_row(stat_m, lr);
    const float l_all = l_all_row(stat_m, stat_l, lr);
    // With one split every real row has token 0 in range, so m_all is finite
    // and l_all > 0; with several, a split's rows may all be masked (m_all =
    // -inf, l_all = 0): the record carries that and the merge weighs it 0.
    const float m_use = m_all == -INFINITY ? 0.0f : m_all;
    const float f = __builtin_amdgcn_exp2f(m_run - m_use) / (nsplit == 1 ? l_all : 1.0f);
    float *ob = reinterpret_cast<float *>(smem) + wave * kTile * D;
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            ob[lr * D + 16 * t + 4 * gq + i] = st.o_acc[t][i] * f;
    __syncthreads();

    // Sum the W partial rows: thread -> (row, D / (4 W) columns).
    constexpr int TPR = 4 * W;  // threads per row
    constexpr int PER = D / TPR;
    static_assert(PER % 4 == 0, "whole 16-byte pieces per thread");
    const int orow = threadIdx.x / TPR;
    const int c0 = (threadIdx.x % TPR) * PER;
    const int rr = tile * kTile + orow;
    float v[PER];
    {
        const float *o0 = reinterpret_cast<const float *>(smem);
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            float acc = 0.0f;
#pragma unroll
            for (int w = 0; w < W; ++w)
                acc += o0[(w * kTile + orow) * D + c0 + e];
            v[e] = acc;
        }
    }
    O *dst = (O *)a.out + ((size_t)(q0 + (rr / G)) * hq + (size_t)g * G + (rr % G)) * D + c0;
    if (nsplit == 1) {
        if (rr < rows) {
#pragma unroll
            for (int e = 0; e < PER; ++e)
                dst[e] = Elem<O>::from_float(v[e]);
        }
        return;
    }

    // Several splits: record = o[16][D] (unnormalised), m[16], l[16].
    constexpr int REC = kTile * D + 2 * kTile;
    const size_t tile_id = ((size_t)blockIdx.y * gridDim.x + tile);
    {
        float *rec = a.ws_rec + (tile_id * gridDim.z + z) * REC;
        const __amdgpu_buffer_rsrc_t rs = rec_rsrc(rec, REC);
#pragma unroll
        for (int k = 0; k < PER / 4; ++k)
            __builtin_amdgcn_raw_buffer_store_b128(
                u32x4{__float_as_uint(v[4 * k]), __float_as_uint(v[4 * k + 1]),
                      __float_as_uint(v[4 * k + 2]), __float_as_uint(v[4 * k + 3])},
                rs, (orow * D + c0 + 4 * k) * 4, 0, kSc1);
        if (threadIdx.x % TPR == 0) {
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m_all_row(stat_m, orow)), rs,
                                                  (kTile * D + orow) * 4, 0, kSc1);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l_all_row(stat_m, stat_l, orow)),
                                                  rs, (kTile * D + kTile + orow) * 4, 0, kSc1);
        }
    }
    // Claim the tile's counter for this call (arrival.h); the wait for the
    // record stores also covers the swap.
    uint64_t seen = 0;
    if (threadIdx.x == 0)
        seen = claim_counter(&a.ws_count[tile_id], a.epoch);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's record stores are done
    __syncthreads();                                   // ... and every thread's
    __shared__ int arrived;
    if (threadIdx.x == 0)
        arrived = (int)arrive_counter(&a.ws_count[tile_id], a.epoch, seen, 1) + 1;
    __syncthreads();
    if (arrived != nsplit)
        return;

    // Last arrival: merge the splits in order.
    asm volatile("" ::: "memory");
    if (rr < rows) {
        float mz_max = -INFINITY;
        for (int zz = 0; zz < nsplit; ++zz) {
            const __amdgpu_buffer_rsrc_t rs = rec_rsrc(a.ws_rec + (tile_id * gridDim.z + zz) * REC, REC);
            mz_max = fmaxf(mz_max, __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                                       rs, (kTile * D + orow) * 4, 0, kSc1)));
        }
        float lsum = 0.0f, acc[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e)
            acc[e] = 0.0f;
        for (int zz = 0; zz < nsplit; ++zz) {
            const __amdgpu_buffer_rsrc_t rs = rec_rsrc(a.ws_rec + (tile_id * gridDim.z + zz) * REC, REC);
            const float mz = __uint_as_float(
                __builtin_amdgcn_raw_buffer_load_b32(rs, (kTile * D + orow) * 4, 0, kSc1));
            const float lz = __uint_as_float(
                __builtin_amdgcn_raw_buffer_load_b32(rs, (kTile * D + kTile + orow) * 4, 0, kSc1));
            const float wz = mz == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mz - mz_max);
            lsum = __builtin_fmaf(wz, lz, lsum);
#pragma unroll
            for (int k = 0; k < PER / 4; ++k) {
                const u32x4 oz = __builtin_amdgcn_raw_buffer_load_b128(rs, (orow * D + c0 + 4 * k) * 4,
                                                                      0, kSc1);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[4 * k + e] = __builtin_fmaf(wz, __uint_as_float(oz[e]), acc[4 * k + e]);
            }
        }
        const float inv = 1.0f / lsum;
#pragma unroll
        for (int e = 0; e < PER; ++e)
            dst[e] = Elem<O>::from_float(acc[e] * inv);
    }
    if (threadIdx.x == 0)
        release_counter(&a.ws_count[tile_id]);
}

// Wide variant for long query runs (chunked prefill): a workgroup takes four
// consecutive tiles of one (sequence, KV head), one wave per tile, and
// walks the KV blocks of its split once: each 16-token block of K and V is
// loaded by the whole workgroup into LDS (K row-major, V transposed;
// double-buffered, the next block's loads in flight during the current
// block's math) and read by all four waves, so K/V are fetched once per 64
// query rows instead of once per 16.  A wave skips blocks wholly past its
// rows' positions.  Each wave finishes its own tile: directly with one
// split, else through the per-tile records and arrival counter.
template <typename T, typename O, int D, int G>
__global__ __launch_bounds__(kMqWaves * 64) void paged_mq_wide_kernel(MultiQueryArgs a)
{
    using TS = TileState<T, D>;
    constexpr int EB = sizeof(T);
    constexpr int QD = TS::QD, NW = TS::NW, MT = TS::MT, VS = TS::VS;
    constexpr int NL = QD * EB / 16;           // 16-byte loads per lane per row part
    constexpr int EC = 16 / EB;                // elements per 16-byte chunk
    constexpr int CH = D / EC;                 // chunks per row
    constexpr int KS = D + EC;                 // LDS row stride of K (one chunk of padding)
    constexpr int NCH = 2 * kTile * CH;        // chunks of one K block plus one V block
    static_assert((kTile * CH) % 64 == 0, "each wave loads K chunks only or V chunks only");
    constexpr int PER = (NCH + kMqWaves * 64 - 1) / (kMqWaves * 64);
    // KV blocks per step: as many as keep the whole workgroup at 16 bytes of
    // K/V per thread per step (one round trip to memory per step).
    constexpr int NB = PER >= 4 ? 1 : 4 / PER;
    // 16-bit V stays row-major (like K) and is read back through the
    // transposing LDS read; fp32 V is stored transposed.
    constexpr bool kRowV = EB == 2;
    constexpr int VKS = KS;  // row stride of a row-major V tile
    constexpr int VBLK = kRowV ? kTile * VKS : D * VS;  // LDS elements of one V block
    __shared__ __attribute__((aligned(16))) T kl[2][NB * kTile * KS];
    __shared__ __attribute__((aligned(16))) T vtl[2][NB * VBLK];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int gq = lane >> 4;
    const int lr = lane & 15;
    const int hkv = a.num_kv_heads;
    const int b = blockIdx.y / hkv;
    const int g = blockIdx.y - b * hkv;
    const int q0 = a.query_start[b];
    const int nq = a.query_start[b + 1] - q0;
    const int rows = nq * G;
    const int tile0 = blockIdx.x * kMqWaves;
    if (tile0 * kTile >= rows)
        return;  // the whole workgroup leaves together
    const int ctx = a.context_lens[b];
    const int first_pos = ctx - nq;
    const int wg_last_row = min((tile0 + kMqWaves) * kTile - 1, rows - 1);
    const int scan_end = first_pos + wg_last_row / G + 1;
    const int nblk = (scan_end + kTile - 1) / kTile;
    const int nsplit = (nblk + a.split_blocks - 1) / a.split_blocks;
    const int z = blockIdx.z;
    if (z >= nsplit)
        return;
    const int n_begin = z * a.split_blocks;
    const int n_end = min(nblk, n_begin + a.split_blocks);

    const int tile = tile0 + wave;
    const bool has_rows = tile * kTile < rows;   // wave-uniform
    const int r = tile * kTile + lr;
    const bool row_ok = r < rows;
    const int my_pos = first_pos + r / G;
    const int wave_last_pos = first_pos + min(tile * kTile + kTile - 1, rows - 1) / G;
    const int wave_first_pos = first_pos + (tile * kTile) / G;
    const int hq = hkv * G;

    uint32_t qw[NW];
    {
        const int cr = row_ok ? r : rows - 1;
        const int cj = cr / G, ch = cr - (cr / G) * G;
        const T *qrow = (const T *)a.q + ((size_t)(q0 + cj) * hq + (size_t)g * G + ch) * D + gq * QD;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            u32x4 v = reinterpret_cast<const u32x4 *>(qrow)[i];
            if (!row_ok)
                v = u32x4{0, 0, 0, 0};
#pragma unroll
            for (int k = 0; k < 4; ++k)
                qw[4 * i + k] = v[k];
        }
    }

    // Whole-workgroup loads of the NB blocks starting at n0: chunk c of
    // this thread covers K (first half of the chunks) or V, row c / CH,
    // 16-byte column c % CH; blocks at or past n_end read as zero rows.
    const size_t tile_elems = (size_t)kTile * D;
    // Block-table window: lane i holds the entry of block win0 + i (0 past
    // the split), so a step's block ids need no dependent memory access.
    int win0 = n_begin, tbl_win = 0;
    auto load_window = [&](int n) {
        win0 = n;
        tbl_win = n + lane < n_end ? a.block_tables[(size_t)b * a.max_blocks + n + lane] : 0;
    };
    load_window(n_begin);
    // Each wave loads one contiguous quarter of the step's chunks, which lies
    // inside one block (K part or V part), so a wave sets up one block's
    // descriptors per step: lane l takes chunk c0 + 64 i + l.
    constexpr int CPW = NB * NCH / kMqWaves;  // chunks per wave per step
    constexpr int PW = CPW / 64;              // 16-byte loads per lane per step
    static_assert(CPW % 64 == 0 && NCH % CPW == 0, "a wave's chunks lie in one block");
    const int c0 = wave * CPW;
    const int wbi = c0 / NCH;  // the wave's block within the step
    auto gload = [&](int n0, u32x4 (&regs)[PW]) {
        if (n0 + NB - 1 - win0 >= 64)
            load_window(n0);
        const int n = n0 + wbi;
        const bool live = n < n_end;
        const int blk = __builtin_amdgcn_readlane(tbl_win, (live ? n : n0) - win0);
        const int valid = live ? min(kTile, scan_end - n * kTile) : 0;
        const size_t base = ((size_t)blk * hkv + g) * tile_elems;
        const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)((const T *)a.k_cache + base), (short)0, valid * D * EB, kRawWord3);
        const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)((const T *)a.v_cache + base), (short)0, valid * D * EB, kRawWord3);
#pragma unroll
        for (int i = 0; i < PW; ++i) {
            const int cc = c0 % NCH + i * 64;  // wave-uniform; K and V split at a multiple of 64
            const bool is_k = cc < kTile * CH;
            const int rc = cc % (kTile * CH) + lane;
            regs[i] = __builtin_amdgcn_raw_buffer_load_b128(is_k ? krs : vrs, rc * 16, 0, 0);
        }
    };
    auto lstore = [&](int buf, const u32x4 (&regs)[PW]) {
        T *kb = &kl[buf][wbi * kTile * KS];
        T *vb = &vtl[buf][wbi * VBLK];
#pragma unroll
        for (int i = 0; i < PW; ++i) {
            const int cc = c0 % NCH + i * 64;
            const int rc = cc % (kTile * CH) + lane;
            const int row = rc / CH, col = rc % CH;
            if (cc < kTile * CH) {
                *reinterpret_cast<u32x4 *>(&kb[row * KS + col * EC]) = regs[i];
            } else if constexpr (kRowV) {
                *reinterpret_cast<u32x4 *>(&vb[row * VKS + col * EC]) = regs[i];
            } else {
                const u32x4 w = regs[i];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t word = w[k];
                    if constexpr (EB == 4) {
                        vb[(col * EC + k) * VS + row] = __builtin_bit_cast(T, word);
                    } else {
                        typedef T t2 __attribute__((ext_vector_type(2)));
                        const t2 pair = __builtin_bit_cast(t2, word);
                        vb[(col * EC + 2 * k) * VS + row] = pair[0];
                        vb[(col * EC + 2 * k + 1) * VS + row] = pair[1];
                    }
                }
            }
        }
    };

    TS st;
    u32x4 regs[PW];
    if (n_begin < n_end) {
        gload(n_begin, regs);
        lstore(0, regs);
    }
    __syncthreads();
    for (int n0 = n_begin; n0 < n_end; n0 += NB) {
        const int buf = ((n0 - n_begin) / NB) & 1;
        const bool more = n0 + NB < n_end;
        if (more)
            gload(n0 + NB, regs);  // in flight while these blocks are used
        if (has_rows && n0 * kTile <= wave_last_pos) {
            // Scores of all the step's blocks, one softmax update, then
            // P.V.  Blocks that no row of this wave reaches (past its last
            // position, or past the split: zero rows in LDS) are computed
            // too, without branches; their weights are exactly zero.
            f32x4 sc[NB];
            bool live[NB];
            uint32_t kw[NB][NW];
#pragma unroll
            for (int bi = 0; bi < NB; ++bi) {
                const int n = n0 + bi;
                live[bi] = n < n_end && n * kTile <= wave_last_pos;  // wave-uniform
                const T *krow = &kl[buf][(bi * kTile + lr) * KS + gq * QD];
#pragma unroll
                for (int i = 0; i < NL; ++i) {
                    const u32x4 v = reinterpret_cast<const u32x4 *>(krow)[i];
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        kw[bi][4 * i + k] = v[k];
                }
            }
            TS::template scores_blocks<NB>(kw, qw, sc);
            float p[NB][4];
            bool all_live = true;
#pragma unroll
            for (int bi = 0; bi < NB; ++bi)
                all_live = all_live && live[bi];
            const bool unmasked = all_live && (n0 + NB) * kTile - 1 <= wave_first_pos;
            st.template update<NB>(sc, live, unmasked, n0, row_ok, my_pos, a.qscale, gq, p);
            if constexpr (kRowV) {
                static_assert(NB % 2 == 0, "16-bit steps hold whole block pairs");
#pragma unroll
                for (int bi = 0; bi < NB; bi += 2)
                    st.pv_rows2(&vtl[buf][bi * VBLK], &vtl[buf][(bi + 1) * VBLK], VKS, lr, gq,
                                p[bi], p[bi + 1]);
            } else {
#pragma unroll
                for (int bi = 0; bi < NB; ++bi)
                    st.pv(&vtl[buf][bi * VBLK], lr, gq, p[bi]);
            }
        }
        if (more)
            lstore(buf ^ 1, regs);
        __syncthreads();  // the next buffer is filled; this one is no longer read
    }
    if (!has_rows)
        return;

    // This wave's tile: lane holds O^T[16 t + 4 gq + i][row lr].
    float l_row = allreduce_pair<16, OpSum>(st.l_lane);
    l_row = allreduce_pair<32, OpSum>(l_row);
    const int oj = r / G, oh = r - (r / G) * G;
    O *dst = (O *)a.out + ((size_t)(q0 + oj) * hq + (size_t)g * G + oh) * D + 4 * gq;
    if (nsplit == 1) {
        if (row_ok) {
            const float inv = 1.0f / l_row;
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dst[16 * t + i] = Elem<O>::from_float(st.o_acc[t][i] * inv);
        }
        return;
    }
    constexpr int REC = kTile * D + 2 * kTile;
    const size_t tile_id = (size_t)blockIdx.y * a.max_tiles + tile;
    {
        const __amdgpu_buffer_rsrc_t rs = rec_rsrc(a.ws_rec + (tile_id * gridDim.z + z) * REC, REC);
#pragma unroll
        for (int t = 0; t < MT; ++t)
            __builtin_amdgcn_raw_buffer_store_b128(
                u32x4{__float_as_uint(st.o_acc[t][0]), __float_as_uint(st.o_acc[t][1]),
                      __float_as_uint(st.o_acc[t][2]), __float_as_uint(st.o_acc[t][3])},
                rs, (lr * D + 16 * t + 4 * gq) * 4, 0, kSc1);
        if (gq == 0) {
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(st.m_run), rs, (kTile * D + lr) * 4,
                                                  0, kSc1);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l_row), rs,
                                                  (kTile * D + kTile + lr) * 4, 0, kSc1);
        }
    }
    // Claim the tile's counter for this call (arrival.h); the wait for the
    // record stores also covers the swap.
    uint64_t seen = 0;
    if (lane == 0)
        seen = claim_counter(&a.ws_count[tile_id], a.epoch);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the whole wave's record is stored
    int arrived = 0;
    if (lane == 0)
        arrived = (int)arrive_counter(&a.ws_count[tile_id], a.epoch, seen, 1) + 1;
    arrived = __builtin_amdgcn_readfirstlane(arrived);
    if (arrived != nsplit)
        return;
    asm volatile("" ::: "memory");
    float mz_max = -INFINITY;
    for (int zz = 0; zz < nsplit; ++zz) {
        const __amdgpu_buffer_rsrc_t rs = rec_rsrc(a.ws_rec + (tile_id * gridDim.z + zz) * REC, REC);
        mz_max = fmaxf(mz_max, __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                                   rs, (kTile * D + lr) * 4, 0, kSc1)));
    }
    float lsum = 0.0f;
    f32x4 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
        acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int zz = 0; zz < nsplit; ++zz) {
        const __amdgpu_buffer_rsrc_t rs = rec_rsrc(a.ws_rec + (tile_id * gridDim.z + zz) * REC, REC);
        const float mz = __uint_as_float(
            __builtin_amdgcn_raw_buffer_load_b32(rs, (kTile * D + lr) * 4, 0, kSc1));
        const float lz = __uint_as_float(
            __builtin_amdgcn_raw_buffer_load_b32(rs, (kTile * D + kTile + lr) * 4, 0, kSc1));
        const float wz = mz == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mz - mz_max);
        lsum = __builtin_fmaf(wz, lz, lsum);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const u32x4 oz = __builtin_amdgcn_raw_buffer_load_b128(rs, (lr * D + 16 * t + 4 * gq) * 4,
                                                                  0, kSc1);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[t][i] = __builtin_fmaf(wz, __uint_as_float(oz[i]), acc[t][i]);
        }
    }
    if (row_ok) {
        const float inv = 1.0f / lsum;
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dst[16 * t + i] = Elem<O>::from_float(acc[t][i] * inv);
    }
    if (lane == 0)
        release_counter(&a.ws_count[tile_id]);
}

template <typename T, typename O, int D>
hipError_t launch_mq_group(const MultiQueryArgs &a, hipStream_t stream)
{
    const dim3 block(kMqWaves * 64);
    const unsigned yz = (unsigned)(a.num_seqs * a.num_kv_heads);
    if (a.max_tiles >= kWideTiles) {
        const dim3 grid((unsigned)((a.max_tiles + kMqWaves - 1) / kMqWaves), yz, (unsigned)a.num_splits);
        switch (a.group) {
        case 1: hipLaunchKernelGGL((paged_mq_wide_kernel<T, O, D, 1>), grid, block, 0, stream, a); break;
        case 2: hipLaunchKernelGGL((paged_mq_wide_kernel<T, O, D, 2>), grid, block, 0, stream, a); break;
        case 4: hipLaunchKernelGGL((paged_mq_wide_kernel<T, O, D, 4>), grid, block, 0, stream, a); break;
        case 8: hipLaunchKernelGGL((paged_mq_wide_kernel<T, O, D, 8>), grid, block, 0, stream, a); break;
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    const dim3 grid((unsigned)a.max_tiles, yz, (unsigned)a.num_splits);
    const dim3 tile_block(kMqTileWaves * 64);
    switch (a.group) {
    case 1: hipLaunchKernelGGL((paged_mq_kernel<T, O, D, 1>), grid, tile_block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((paged_mq_kernel<T, O, D, 2>), grid, tile_block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((paged_mq_kernel<T, O, D, 4>), grid, tile_block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((paged_mq_kernel<T, O, D, 8>), grid, tile_block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, typename O>
hipError_t launch_mq_dim(const MultiQueryArgs &a, hipStream_t stream)
{
    switch (a.head_dim) {
    case 64: return launch_mq_group<T, O, 64>(a, stream);
    case 128: return launch_mq_group<T, O, 128>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t launch_mq_out(const MultiQueryArgs &a, hipStream_t stream)
{
    return a.out_f32 ? launch_mq_dim<T, float>(a, stream) : launch_mq_dim<T, T>(a, stream);
}

}  // namespace

hipError_t launch_paged_multi_query(const MultiQueryArgs &a, hipStream_t stream)
{
    switch (a.dtype) {
    case kDtypeF32: return launch_mq_dim<float, float>(a, stream);
    case kDtypeF16: return launch_mq_out<_Float16>(a, stream);
    case kDtypeBF16: return launch_mq_out<__bf16>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace photon
