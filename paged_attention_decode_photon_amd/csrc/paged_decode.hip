// Batched paged-attention decode for gfx950: split-context partition kernel
// and the kernel that merges partitions.
//
// Operation (PhotonInfer README, "GPU-optimised kernels": batched paged
// attention with a stable softmax; "Technical details -> Paged attention":
// block-level KV cache addressed through per-sequence block tables): for
// sequence b, query head h and KV head g = h / G,
//   out[b][h] = sum_t exp(s_t - m) V_t / sum_t exp(s_t - m),
//   s_t = scale * <q[b][h], K_t>,  m = max_t s_t,  t < context_lens[b].
//
// Work decomposition.  One workgroup of kDecodeWaves wavefronts owns one
// (context partition p, KV head g, sequence b) and all G query heads that
// read KV head g, so every K/V byte is fetched from HBM exactly once.  A
// wavefront walks its partition in chunks of U blocks (CT = 16 U tokens).
//
// Lane layout.  A K/V row is RB = D * sizeof(T) bytes, i.e. L = RB / 16
// lanes of one 16-byte load each; one wave-wide load covers RPI = 64 / L
// rows and a 16-token block takes NIB = 16 / RPI loads.  Lane (r, c) with
// r = lane / L, c = lane % L always holds byte chunk c of some row; each 16
// bytes a quad of lanes loads are contiguous.
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
// Softmax.  Scores are kept in log2 units (q is pre-multiplied by
// scale * log2 e) and use v_exp_f32.  Each wave keeps an online maximum and
// sum per head; the waves of a workgroup are merged through LDS.  When the
// sequence has one partition the workgroup writes the normalised output,
// otherwise (max, sum, unnormalised row) go to the workspace and
// paged_decode_merge combines partitions in index order.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "lane_ops.h"
#include "launch.h"

namespace photon {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// Fourth descriptor word of a raw (unswizzled, stride 0) buffer on gfx9-family.
constexpr int kRawBufferWord3 = 0x00020000;

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }
constexpr int cmin(int a, int b) { return a < b ? a : b; }

template <typename T>
struct Elem;

template <>
struct Elem<float> {
    __device__ static void unpack(const u32x4 &v, float (&f)[4])
    {
        f[0] = __uint_as_float(v[0]);
        f[1] = __uint_as_float(v[1]);
        f[2] = __uint_as_float(v[2]);
        f[3] = __uint_as_float(v[3]);
    }
    __device__ static float to_float(float x) { return x; }
    __device__ static float from_float(float x) { return x; }
};

template <>
struct Elem<_Float16> {
    __device__ static void unpack(const u32x4 &v, float (&f)[8])
    {
        // Copy each dword out of the vector before the bit cast: a bit cast of
        // the vector element itself reads the vector's first dword.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t word = v[i];
            half2_t h = __builtin_bit_cast(half2_t, word);
            f[2 * i] = (float)h[0];
            f[2 * i + 1] = (float)h[1];
        }
    }
    __device__ static float to_float(_Float16 x) { return (float)x; }
    __device__ static _Float16 from_float(float x) { return (_Float16)x; }
};

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
    static_assert(L * E == D, "row split");
    static_assert(L >= G && L >= 8 && L <= 32, "lane layout");
    static_assert(CT == decode_chunk_tokens(EB, D, G), "chunk size");
};

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

template <typename T, int D, int G>
__global__ __launch_bounds__(kDecodeWaves * 64) void paged_decode_partition(
    const T *__restrict__ q, const T *__restrict__ k_cache, const T *__restrict__ v_cache,
    const int32_t *__restrict__ block_tables, const int32_t *__restrict__ context_lens,
    T *__restrict__ out, float *__restrict__ ws_ml, float *__restrict__ ws_o, int num_kv_heads,
    int max_blocks, int part_tokens, int max_parts, float qscale)
{
    using S = Shape<T, D, G>;
    constexpr int E = S::E, L = S::L, RPI = S::RPI, NIB = S::NIB, CT = S::CT, NU = S::NU;
    constexpr int NS = S::NS, CP = S::CP, NK = S::NK, RB = S::RB;
    constexpr int WAVES = kDecodeWaves;

    __shared__ __attribute__((aligned(16))) float p_lds[WAVES][CT][G];
    __shared__ float red_m[WAVES][G];
    __shared__ float red_l[WAVES][G];
    __shared__ __attribute__((aligned(16))) float red_o[WAVES][G][D];

    const int p = blockIdx.x;
    const int g = blockIdx.y;
    const int b = blockIdx.z;
    const int hq = num_kv_heads * G;
    const int ctx = context_lens[b];
    const int t0 = p * part_tokens;
    T *out_rows = out + ((size_t)b * hq + (size_t)g * G) * D;

    if (t0 >= ctx) {
        if (p == 0) {  // empty context: the row is defined as zero
            for (int i = threadIdx.x; i < G * D; i += WAVES * 64)
                out_rows[i] = Elem<T>::from_float(0.0f);
        }
        return;
    }

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nparts = (ctx + part_tokens - 1) / part_tokens;
    const int tok_end = min(ctx, t0 + part_tokens);
    const int nchunks = (tok_end - t0 + CT - 1) / CT;

    const int c = lane & (L - 1);         // byte chunk of the row
    const int r = lane >> S::LOG2L;       // row inside a wave-wide load
    const int phi = c & ((1 << CP) - 1);  // slot permutation of this lane
    const int row_x = phi >> S::LOG2G;    // load-index xor (stays inside a block)
    const int head_x = phi & (G - 1);     // head xor
    const int my_head = c & (G - 1);      // head of the scores this lane ends with

    // q rows of the group, in this lane's head order, pre-scaled to log2 units.
    float qf[G][E];
#pragma unroll
    for (int hs = 0; hs < G; ++hs) {
        const T *row = q + ((size_t)b * hq + (size_t)g * G + (hs ^ head_x)) * D + c * E;
        Elem<T>::unpack(*reinterpret_cast<const u32x4 *>(row), qf[hs]);
#pragma unroll
        for (int e = 0; e < E; ++e)
            qf[hs][e] *= qscale;
    }

    int k_off[NIB], v_off[NIB];
#pragma unroll
    for (int i = 0; i < NIB; ++i) {
        k_off[i] = (((i ^ row_x) * RPI + r) * RB) + c * 16;
        v_off[i] = ((i * RPI + r) * RB) + c * 16;
    }

    float m_run = -INFINITY;  // running maximum (log2 units) of head my_head
    float l_run = 0.0f;       // this lane's share of the exponential sum
    float o_acc[G][E];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < E; ++e)
            o_acc[h][e] = 0.0f;

    const int32_t *table = block_tables + (size_t)b * max_blocks;
    const size_t tile_stride = (size_t)kBlockTokens * RB;

    for (int ch = wave; ch < nchunks; ch += WAVES) {
        const int ct0 = t0 + ch * CT;
        __amdgpu_buffer_rsrc_t rk[S::U], rv[S::U];
#pragma unroll
        for (int u = 0; u < S::U; ++u) {
            const int n = (ct0 / kBlockTokens) + u;
            int rows = ctx - n * kBlockTokens;
            rows = rows > kBlockTokens ? kBlockTokens : rows;
            int blk = 0;
            if (rows > 0)
                blk = table[n];
            else
                rows = 0;
            const size_t tile = ((size_t)blk * num_kv_heads + g) * tile_stride;
            rk[u] = __builtin_amdgcn_make_buffer_rsrc((void *)((const char *)k_cache + tile), (short)0,
                                                      rows * RB, kRawBufferWord3);
            rv[u] = __builtin_amdgcn_make_buffer_rsrc((void *)((const char *)v_cache + tile), (short)0,
                                                      rows * RB, kRawBufferWord3);
        }

        u32x4 kd[NU], vd[NU];
#pragma unroll
        for (int i = 0; i < NU; ++i)
            kd[i] = __builtin_amdgcn_raw_buffer_load_b128(rk[i / NIB], k_off[i % NIB], 0, 0);
#pragma unroll
        for (int i = 0; i < NU; ++i)
            vd[i] = __builtin_amdgcn_raw_buffer_load_b128(rv[i / NIB], v_off[i % NIB], 0, 0);

        // Partial dot products over this lane's chunk: slot (i, hs) pairs the
        // lane's load i with query head hs ^ head_x.
        float part[NS];
#pragma unroll
        for (int i = 0; i < NU; ++i) {
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
        reduce_scatter<NS, CP, CP - 1>(part);

        // Scores: slot n << CP now holds item (n << CP) | phi, summed over the
        // CP permuted lane bits; the remaining row bits are summed directly.
        float s[NK];
        int s_tok[NK];
        float cmax = -INFINITY;
#pragma unroll
        for (int n = 0; n < NK; ++n) {
            float v = allreduce_bits<CP, S::LOG2L, OpSum>(part[n << CP]);
            const int item = (n << CP) | phi;
            const int ld = item >> S::LOG2G;
            const int tok = (ld / NIB) * kBlockTokens + (ld % NIB) * RPI + r;
            s_tok[n] = tok;
            v = (ct0 + tok < tok_end) ? v : -INFINITY;
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
            p_lds[wave][s_tok[n]][my_head] = pv;
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
                pw[h] = p_lds[wave][tok][h];
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < E; ++e)
                    o_acc[h][e] = __builtin_fmaf(pw[h], vf[e], o_acc[h][e]);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // Per-wave totals.  Lanes that differ only in directly-summed row bits
    // hold copies of the same scores; count each score once.
    float l_once = ((c >> CP) == 0) ? l_run : 0.0f;
    l_once = allreduce_bits<S::LOG2G, 6, OpSum>(l_once);
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < E; ++e)
            o_acc[h][e] = allreduce_bits<S::LOG2L, 6, OpSum>(o_acc[h][e]);

    if (lane < G) {
        red_m[wave][lane] = m_run;
        red_l[wave][lane] = l_once;
    }
    if (r == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < E; ++e)
                red_o[wave][h][c * E + e] = o_acc[h][e];
    }
    __syncthreads();

    for (int i = threadIdx.x; i < G * D; i += WAVES * 64) {
        const int h = i / D;
        const int dim = i % D;
        float m = red_m[0][h];
#pragma unroll
        for (int w = 1; w < WAVES; ++w)
            m = fmaxf(m, red_m[w][h]);
        float lsum = 0.0f, o = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            const float f = __builtin_amdgcn_exp2f(red_m[w][h] - m);
            lsum = __builtin_fmaf(f, red_l[w][h], lsum);
            o = __builtin_fmaf(f, red_o[w][h][dim], o);
        }
        if (nparts == 1) {
            out_rows[i] = Elem<T>::from_float(o / lsum);
        } else {
            const size_t slot = ((size_t)b * hq + (size_t)g * G + h) * max_parts + p;
            ws_o[slot * D + dim] = o;
            if (dim == 0) {
                ws_ml[slot * 2] = m;
                ws_ml[slot * 2 + 1] = lsum;
            }
        }
    }
}

// Merge the partitions of every (sequence, query head) that has more than one:
// out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p with M = max_p m_p,
// accumulated in partition order.
template <typename T, int D>
__global__ __launch_bounds__(D) void paged_decode_merge(T *__restrict__ out,
                                                         const float *__restrict__ ws_ml,
                                                         const float *__restrict__ ws_o,
                                                         const int32_t *__restrict__ context_lens,
                                                         int num_q_heads, int part_tokens,
                                                         int max_parts)
{
    const int h = blockIdx.x;
    const int b = blockIdx.y;
    const int dim = threadIdx.x;
    const int ctx = context_lens[b];
    const int nparts = (ctx + part_tokens - 1) / part_tokens;
    if (nparts <= 1)
        return;
    const size_t base = ((size_t)b * num_q_heads + h) * max_parts;
    const float *ml = ws_ml + base * 2;
    float m = -INFINITY;
    for (int i = 0; i < nparts; ++i)
        m = fmaxf(m, ml[2 * i]);
    float lsum = 0.0f, o = 0.0f;
    for (int i = 0; i < nparts; ++i) {
        const float f = __builtin_amdgcn_exp2f(ml[2 * i] - m);
        lsum = __builtin_fmaf(f, ml[2 * i + 1], lsum);
        o = __builtin_fmaf(f, ws_o[(base + i) * D + dim], o);
    }
    out[((size_t)b * num_q_heads + h) * D + dim] = Elem<T>::from_float(o / lsum);
}

template <typename T, int D, int G>
hipError_t launch_typed(const DecodeArgs &a, hipStream_t stream)
{
    const dim3 grid(a.max_parts, a.num_kv_heads, a.num_seqs);
    hipLaunchKernelGGL((paged_decode_partition<T, D, G>), grid, dim3(kDecodeWaves * 64), 0,
                       stream, (const T *)a.q, (const T *)a.k_cache, (const T *)a.v_cache,
                       a.block_tables, a.context_lens, (T *)a.out, a.ws_ml, a.ws_o,
                       a.num_kv_heads, a.max_blocks, a.part_tokens, a.max_parts, a.qscale);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || a.max_parts <= 1)
        return err;
    hipLaunchKernelGGL((paged_decode_merge<T, D>), dim3(a.num_kv_heads * G, a.num_seqs), dim3(D),
                       0, stream, (T *)a.out, a.ws_ml, a.ws_o, a.context_lens,
                       a.num_kv_heads * G, a.part_tokens, a.max_parts);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_group(const DecodeArgs &a, hipStream_t stream)
{
    switch (a.group) {
    case 1: return launch_typed<T, D, 1>(a, stream);
    case 2: return launch_typed<T, D, 2>(a, stream);
    case 4: return launch_typed<T, D, 4>(a, stream);
    case 8: return launch_typed<T, D, 8>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t launch_dim(const DecodeArgs &a, hipStream_t stream)
{
    switch (a.head_dim) {
    case 64: return launch_group<T, 64>(a, stream);
    case 128: return launch_group<T, 128>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_paged_decode(const DecodeArgs &a, hipStream_t stream)
{
    if (a.elem_bytes == 4)
        return launch_dim<float>(a, stream);
    if (a.elem_bytes == 2)
        return launch_dim<_Float16>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace photon
