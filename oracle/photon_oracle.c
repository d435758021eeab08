/*
 * CPU oracle for batched paged-attention decode.  TEST INFRASTRUCTURE ONLY:
 * the parity tests, the smoke check and the benchmark's CPU-baseline leg are
 * its only callers.  It shares no code, header or constant with the HIP
 * library; both sides see only the same seeded inputs.
 *
 * What it follows (PhotonInfer README, zh-CN / fr / ja translations):
 *   - "GPU-optimised kernels": batched paged attention over a block-level KV
 *     cache, a numerically stable softmax, and batched RoPE among the fused
 *     operations;
 *   - "Technical details -> Paged attention": a block-level KV cache, per
 *     sequence cache offsets (read as block tables), and one batched K/V
 *     write for many sequences (read as a per-token slot mapping).
 * The pages print no formula; the attention computed here is the textbook
 * single-query decode step, out = softmax(scale * q K^T) V, with grouped-query
 * heads: q head h reads KV head floor(h / (Hq/Hkv)).
 *
 * Layout (shared by K and V pools): [num_blocks, num_kv_heads, block_size,
 * head_dim], contiguous.  slot = physical_block * block_size + offset.
 *
 * Arithmetic: every element is widened exactly to double, scores, maximum,
 * exponentials, sums and the weighted sum of V are all formed in double, with
 * one plain pass per output and no blocking or rescaling.  Sums run in token
 * order, dot products in element order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum {
    ORACLE_OK = 0,
    ORACLE_ERR_ARG = 1,         /* bad sizes, dtype or null pointers        */
    ORACLE_ERR_SLOT_RANGE = 2,  /* slot < -1 or slot >= num_blocks*bs        */
    ORACLE_ERR_SLOT_DUP = 3,    /* two tokens write the same slot            */
    ORACLE_ERR_BLOCK_RANGE = 4, /* a block id the sequence uses is out of range */
    ORACLE_ERR_CTX = 5,         /* context length < 0 or > max_blocks*bs     */
    ORACLE_ERR_HEADS = 6        /* num_q_heads not a multiple of num_kv_heads */
};

enum { ORACLE_F32 = 0, ORACLE_F16 = 1, ORACLE_BF16 = 2 };

/* IEEE 754 binary16 -> double, from the format's definition: 1 sign bit,
 * 5 exponent bits (bias 15), 10 fraction bits; exponent 0 encodes zero and
 * subnormals (fraction * 2^-24), exponent 31 encodes inf / NaN. */
double oracle_half_to_double(uint16_t bits)
{
    const int sign = bits >> 15;
    const int expo = (bits >> 10) & 0x1f;
    const int frac = bits & 0x3ff;
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -24);
    else if (expo == 31)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexp((double)(frac | 0x400), expo - 25);
    return sign ? -mag : mag;
}

/* bfloat16 -> double, from the format's definition: 1 sign bit, 8 exponent
 * bits (bias 127, as binary32), 7 fraction bits; exponent 0 encodes zero and
 * subnormals (fraction * 2^-133), exponent 255 encodes inf / NaN. */
double oracle_bfloat16_to_double(uint16_t bits)
{
    const int sign = bits >> 15;
    const int expo = (bits >> 7) & 0xff;
    const int frac = bits & 0x7f;
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -133);
    else if (expo == 255)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexp((double)(frac | 0x80), expo - 134);
    return sign ? -mag : mag;
}

static double widen(const void *base, int64_t idx, int dtype)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)base)[idx];
    if (dtype == ORACLE_F16)
        return oracle_half_to_double(((const uint16_t *)base)[idx]);
    return oracle_bfloat16_to_double(((const uint16_t *)base)[idx]);
}

/* Cache write: for each token i with slot >= 0, copy the raw bytes of
 * k[i, h, :] and v[i, h, :] into row (slot / bs, h, slot % bs) of the pools,
 * for every KV head h.  Bytes are copied, never converted. */
int oracle_kv_cache_write(const void *k, const void *v, const int32_t *slot_mapping,
                          int64_t num_tokens, void *k_cache, void *v_cache,
                          int64_t num_blocks, int64_t num_kv_heads, int64_t block_size,
                          int64_t head_dim, int64_t elem_bytes)
{
    if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0 || block_size <= 0 ||
        head_dim <= 0 || (elem_bytes != 2 && elem_bytes != 4))
        return ORACLE_ERR_ARG;
    if (num_tokens == 0)
        return ORACLE_OK;
    if (!k || !v || !slot_mapping || !k_cache || !v_cache)
        return ORACLE_ERR_ARG;

    const int64_t nslots = num_blocks * block_size;
    unsigned char *seen = (unsigned char *)calloc((size_t)nslots, 1);
    if (!seen)
        return ORACLE_ERR_ARG;
    for (int64_t i = 0; i < num_tokens; ++i) {
        const int64_t s = slot_mapping[i];
        if (s < -1 || s >= nslots) {
            free(seen);
            return ORACLE_ERR_SLOT_RANGE;
        }
        if (s >= 0) {
            if (seen[s]) {
                free(seen);
                return ORACLE_ERR_SLOT_DUP;
            }
            seen[s] = 1;
        }
    }
    free(seen);

    const int64_t row_bytes = head_dim * elem_bytes;
    for (int64_t i = 0; i < num_tokens; ++i) {
        const int64_t s = slot_mapping[i];
        if (s < 0)
            continue;
        const int64_t blk = s / block_size;
        const int64_t off = s % block_size;
        for (int64_t h = 0; h < num_kv_heads; ++h) {
            const int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * row_bytes;
            const int64_t src = (i * num_kv_heads + h) * row_bytes;
            memcpy((char *)k_cache + dst, (const char *)k + src, (size_t)row_bytes);
            memcpy((char *)v_cache + dst, (const char *)v + src, (size_t)row_bytes);
        }
    }
    return ORACLE_OK;
}

/* Paged decode attention.
 *   q            [B, Hq, D]           dtype
 *   k/v_cache    [NB, Hkv, bs, D]     dtype
 *   block_tables [B, max_blocks]      int32 (entries past ceil(ctx/bs) ignored)
 *   context_lens [B]                  int32
 *   out          [B, Hq, D]           double
 *   probs        [B, Hq, max_blocks*bs] double or NULL: softmax weights,
 *                zero past the context length
 * A sequence with context length 0 gets an all-zero output row. */
int oracle_paged_attn_decode(const void *q, const void *k_cache, const void *v_cache,
                             const int32_t *block_tables, const int32_t *context_lens,
                             int64_t num_seqs, int64_t num_q_heads, int64_t num_kv_heads,
                             int64_t head_dim, int64_t block_size, int64_t num_blocks,
                             int64_t max_blocks, int dtype, double scale, double *out,
                             double *probs, int num_threads)
{
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || num_blocks <= 0 || max_blocks <= 0 ||
        (dtype != ORACLE_F32 && dtype != ORACLE_F16 && dtype != ORACLE_BF16))
        return ORACLE_ERR_ARG;
    if (num_q_heads % num_kv_heads != 0)
        return ORACLE_ERR_HEADS;
    if (num_seqs == 0)
        return ORACLE_OK;
    if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out)
        return ORACLE_ERR_ARG;

    for (int64_t b = 0; b < num_seqs; ++b) {
        const int64_t ctx = context_lens[b];
        if (ctx < 0 || ctx > max_blocks * block_size)
            return ORACLE_ERR_CTX;
        const int64_t nblk = (ctx + block_size - 1) / block_size;
        for (int64_t n = 0; n < nblk; ++n) {
            const int64_t id = block_tables[b * max_blocks + n];
            if (id < 0 || id >= num_blocks)
                return ORACLE_ERR_BLOCK_RANGE;
        }
    }

    const int64_t group = num_q_heads / num_kv_heads;
    const int64_t max_tokens = max_blocks * block_size;
    const int64_t pairs = num_seqs * num_q_heads;
    int rc = ORACLE_OK;
#ifdef _OPENMP
    if (num_threads <= 0)
        num_threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(num_threads)
#else
    (void)num_threads;
#endif
    for (int64_t pair = 0; pair < pairs; ++pair) {
        const int64_t b = pair / num_q_heads;
        const int64_t h = pair % num_q_heads;
        const int64_t g = h / group; /* KV head read by q head h */
        const int64_t ctx = context_lens[b];
        double *o = out + pair * head_dim;
        double *p = probs ? probs + pair * max_tokens : NULL;
        if (p)
            memset(p, 0, sizeof(double) * (size_t)max_tokens);
        if (ctx == 0) {
            memset(o, 0, sizeof(double) * (size_t)head_dim);
            continue;
        }
        double *s = (double *)malloc(sizeof(double) * (size_t)ctx);
        if (!s) {
            rc = ORACLE_ERR_ARG;
            continue;
        }
        /* pass 1: scores s_t = scale * <q, K_t> and their maximum */
        double m = -INFINITY;
        for (int64_t t = 0; t < ctx; ++t) {
            const int64_t blk = block_tables[b * max_blocks + t / block_size];
            const int64_t row = ((blk * num_kv_heads + g) * block_size + t % block_size) * head_dim;
            double dot = 0.0;
            for (int64_t j = 0; j < head_dim; ++j)
                dot += widen(q, pair * head_dim + j, dtype) * widen(k_cache, row + j, dtype);
            s[t] = scale * dot;
            if (s[t] > m)
                m = s[t];
        }
        /* pass 2: e_t = exp(s_t - m), l = sum e_t, o = sum e_t V_t / l */
        double l = 0.0;
        for (int64_t j = 0; j < head_dim; ++j)
            o[j] = 0.0;
        for (int64_t t = 0; t < ctx; ++t) {
            const int64_t blk = block_tables[b * max_blocks + t / block_size];
            const int64_t row = ((blk * num_kv_heads + g) * block_size + t % block_size) * head_dim;
            const double e = exp(s[t] - m);
            s[t] = e;
            l += e;
            for (int64_t j = 0; j < head_dim; ++j)
                o[j] += e * widen(v_cache, row + j, dtype);
        }
        for (int64_t j = 0; j < head_dim; ++j)
            o[j] /= l;
        if (p)
            for (int64_t t = 0; t < ctx; ++t)
                p[t] = s[t] / l;
        free(s);
    }
    return rc;
}

/* Multi-query paged attention with a causal tail (chunked prefill and
 * speculative verification: several new tokens of a sequence attend at
 * once).  Sequence b owns query rows query_start[b] .. query_start[b+1]-1;
 * with n_b = query_start[b+1] - query_start[b] and ctx = context_lens[b]
 * (which counts the new tokens), query row j of b is the token at position
 * p = ctx - n_b + j and attends to the cached tokens t <= p.  Each (row,
 * query head) is the single-query step of oracle_paged_attn_decode with the
 * context cut at p + 1: two passes in double, sums in token order.
 *   q, out  [T, Hq, D] (out in double), T = query_start[B]
 * Preconditions (errors, not undefined behaviour): query_start starts at 0
 * and never decreases, n_b <= ctx_b <= max_blocks * block_size, used block
 * ids in range. */
int oracle_paged_attn_multi_query(const void *q, const void *k_cache, const void *v_cache,
                                  const int32_t *block_tables, const int32_t *context_lens,
                                  const int32_t *query_start, int64_t num_seqs,
                                  int64_t num_q_heads, int64_t num_kv_heads, int64_t head_dim,
                                  int64_t block_size, int64_t num_blocks, int64_t max_blocks,
                                  int dtype, double scale, double *out, int num_threads)
{
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || num_blocks <= 0 || max_blocks <= 0 ||
        (dtype != ORACLE_F32 && dtype != ORACLE_F16 && dtype != ORACLE_BF16))
        return ORACLE_ERR_ARG;
    if (num_q_heads % num_kv_heads != 0)
        return ORACLE_ERR_HEADS;
    if (num_seqs == 0)
        return ORACLE_OK;
    if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start || !out)
        return ORACLE_ERR_ARG;
    if (query_start[0] != 0)
        return ORACLE_ERR_ARG;
    for (int64_t b = 0; b < num_seqs; ++b) {
        const int64_t n = (int64_t)query_start[b + 1] - query_start[b];
        const int64_t ctx = context_lens[b];
        if (n < 0 || ctx < n || ctx > max_blocks * block_size)
            return ORACLE_ERR_CTX;
        const int64_t nblk = (ctx + block_size - 1) / block_size;
        for (int64_t i = 0; i < nblk; ++i) {
            const int64_t id = block_tables[b * max_blocks + i];
            if (id < 0 || id >= num_blocks)
                return ORACLE_ERR_BLOCK_RANGE;
        }
    }
    const int64_t group = num_q_heads / num_kv_heads;
    const int64_t rows = (int64_t)query_start[num_seqs] * num_q_heads;
    int rc = ORACLE_OK;
#ifdef _OPENMP
    if (num_threads <= 0)
        num_threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(num_threads)
#else
    (void)num_threads;
#endif
    for (int64_t row = 0; row < rows; ++row) {
        const int64_t tok = row / num_q_heads; /* query row (token) index */
        const int64_t h = row % num_q_heads;
        const int64_t g = h / group;
        int64_t b = 0;
        while (query_start[b + 1] <= tok)
            ++b;
        const int64_t n = (int64_t)query_start[b + 1] - query_start[b];
        const int64_t j = tok - query_start[b];
        const int64_t p = (int64_t)context_lens[b] - n + j; /* this token's position */
        const int64_t len = p + 1;                          /* tokens it attends to */
        double *o = out + row * head_dim;
        double *s = (double *)malloc(sizeof(double) * (size_t)len);
        if (!s) {
            rc = ORACLE_ERR_ARG;
            continue;
        }
        double m = -INFINITY;
        for (int64_t t = 0; t < len; ++t) {
            const int64_t blk = block_tables[b * max_blocks + t / block_size];
            const int64_t kr = ((blk * num_kv_heads + g) * block_size + t % block_size) * head_dim;
            double dot = 0.0;
            for (int64_t d = 0; d < head_dim; ++d)
                dot += widen(q, row * head_dim + d, dtype) * widen(k_cache, kr + d, dtype);
            s[t] = scale * dot;
            if (s[t] > m)
                m = s[t];
        }
        double l = 0.0;
        for (int64_t d = 0; d < head_dim; ++d)
            o[d] = 0.0;
        for (int64_t t = 0; t < len; ++t) {
            const int64_t blk = block_tables[b * max_blocks + t / block_size];
            const int64_t vr = ((blk * num_kv_heads + g) * block_size + t % block_size) * head_dim;
            const double e = exp(s[t] - m);
            l += e;
            for (int64_t d = 0; d < head_dim; ++d)
                o[d] += e * widen(v_cache, vr + d, dtype);
        }
        for (int64_t d = 0; d < head_dim; ++d)
            o[d] /= l;
        free(s);
    }
    return rc;
}

/* Rotary position embedding (the README's "GPU-optimised kernels" section
 * lists batched RoPE among its fused operations; the rotation itself is the
 * textbook one of RoFormer).  Each head row x of token i is split into D/2
 * pairs; pair j is rotated by the angle positions[i] * base^(-2j/D):
 *   x'_a = x_a cos(angle) - x_b sin(angle),  x'_b = x_a sin(angle) + x_b cos(angle).
 * Pair j is (x_j, x_{j+D/2}) when interleaved == 0 (the rotate-half layout of
 * Llama / GPT-NeoX), and (x_{2j}, x_{2j+1}) when interleaved == 1 (the layout
 * of the RoFormer paper and GPT-J).
 *   x    [T, H, D] dtype (widened exactly)
 *   out  [T, H, D] double
 * Angles, sines, cosines and the rotation are all formed in double. */
int oracle_rope(const void *x, const int32_t *positions, int64_t num_tokens, int64_t num_heads,
                int64_t head_dim, int dtype, double base, int interleaved, double *out)
{
    if (num_tokens < 0 || num_heads <= 0 || head_dim <= 0 || head_dim % 2 != 0 ||
        !(base > 0.0) || (interleaved != 0 && interleaved != 1) ||
        (dtype != ORACLE_F32 && dtype != ORACLE_F16 && dtype != ORACLE_BF16))
        return ORACLE_ERR_ARG;
    if (num_tokens == 0)
        return ORACLE_OK;
    if (!x || !positions || !out)
        return ORACLE_ERR_ARG;
    const int64_t half = head_dim / 2;
    for (int64_t i = 0; i < num_tokens; ++i) {
        if (positions[i] < 0)
            return ORACLE_ERR_ARG;
        for (int64_t j = 0; j < half; ++j) {
            const double angle = (double)positions[i] * pow(base, -2.0 * (double)j / (double)head_dim);
            const double c = cos(angle), s = sin(angle);
            const int64_t ia = interleaved ? 2 * j : j;
            const int64_t ib = interleaved ? 2 * j + 1 : j + half;
            for (int64_t h = 0; h < num_heads; ++h) {
                const int64_t row = (i * num_heads + h) * head_dim;
                const double xa = widen(x, row + ia, dtype);
                const double xb = widen(x, row + ib, dtype);
                out[row + ia] = xa * c - xb * s;
                out[row + ib] = xa * s + xb * c;
            }
        }
    }
    return ORACLE_OK;
}

/* Exact double values of n storage elements. */
int oracle_widen(const void *x, int64_t n, int dtype, double *out)
{
    if (n < 0 || (dtype != ORACLE_F32 && dtype != ORACLE_F16 && dtype != ORACLE_BF16) ||
        (n > 0 && (!x || !out)))
        return ORACLE_ERR_ARG;
    for (int64_t i = 0; i < n; ++i)
        out[i] = widen(x, i, dtype);
    return ORACLE_OK;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
