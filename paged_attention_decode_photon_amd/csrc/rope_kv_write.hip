// Fused rotary position embedding and slot-mapped KV cache write for gfx950
// (PhotonInfer README: "GPU-optimised kernels" lists batched RoPE among the
// fused operations; "Technical details -> Paged attention" describes one
// kernel writing the K/V rows of many sequences into the block-level cache).
//
// For token i at position p = positions[i], pair j of every q and k head row
// is rotated by the angle p * base^(-2j/D):
//   x'_a = x_a cos - x_b sin,   x'_b = x_a sin + x_b cos,
// with pair j = (x_j, x_{j+D/2}) (rotate-half layout) or (x_{2j}, x_{2j+1})
// (adjacent pairs).  Rotated q goes to q_out; rotated k and the raw v row go
// to pool row (slot / block_size, h, slot % block_size) when slot >= 0.
//
// One workgroup per token: the D/2 angles are formed once, in double
// (position times base^(-2j/D), then sin and cos), rounded to fp32 into LDS,
// and every thread then rotates 16-byte chunks with fp32 multiply-adds.  The
// v rows are copied as raw bits.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "elem.h"
#include "launch.h"

namespace photon {
namespace {

constexpr int kRopeThreads = 256;

template <typename T, int D, bool ADJACENT>
__global__ __launch_bounds__(kRopeThreads) void rope_kv_cache_write_kernel(RopeArgs a)
{
    constexpr int E = 16 / sizeof(T);                 // elements per 16-byte chunk
    constexpr int HALF = D / 2;
    constexpr int CPR = D / E;                        // chunks per row
    constexpr int IPR = ADJACENT ? CPR : CPR / 2;     // rotation items per row
    __shared__ float cos_t[HALF], sin_t[HALF];

    const int64_t tok = blockIdx.x;
    const int pos = a.positions[tok];
    const int slot = a.slot_mapping[tok];
    for (int j = threadIdx.x; j < HALF; j += kRopeThreads) {
        const double angle = (double)pos * pow(a.base, -2.0 * (double)j / (double)D);
        double s, c;
        sincos(angle, &s, &c);
        cos_t[j] = (float)c;
        sin_t[j] = (float)s;
    }
    __syncthreads();

    const int hq = a.num_q_heads, hkv = a.num_kv_heads;
    const int nq = hq * IPR, nk = hkv * IPR, nv = hkv * CPR;
    const int64_t blk = slot / a.block_size;
    const int64_t off = slot - blk * a.block_size;
    for (int i = threadIdx.x; i < nq + nk + nv; i += kRopeThreads) {
        if (i >= nq && slot < 0)
            break;  // k and v items only go to the cache
        if (i < nq + nk) {
            const bool is_q = i < nq;
            const int r = is_q ? i : i - nq;
            const int h = r / IPR, c = r - (r / IPR) * IPR;
            const u32x4 *src = is_q ? (const u32x4 *)a.q + (tok * hq + h) * CPR
                                    : (const u32x4 *)a.k + (tok * hkv + h) * CPR;
            u32x4 *dst = is_q ? (u32x4 *)a.q_out + (tok * hq + h) * CPR
                              : (u32x4 *)a.k_cache + ((blk * hkv + h) * a.block_size + off) * CPR;
            if constexpr (ADJACENT) {
                float x[E];
                Elem<T>::unpack(src[c], x);
#pragma unroll
                for (int p = 0; p < E / 2; ++p) {
                    const int j = c * (E / 2) + p;
                    const float xa = x[2 * p], xb = x[2 * p + 1];
                    x[2 * p] = __builtin_fmaf(xa, cos_t[j], -xb * sin_t[j]);
                    x[2 * p + 1] = __builtin_fmaf(xa, sin_t[j], xb * cos_t[j]);
                }
                dst[c] = Elem<T>::pack(x);
            } else {
                float xa[E], xb[E];
                Elem<T>::unpack(src[c], xa);
                Elem<T>::unpack(src[c + CPR / 2], xb);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int j = c * E + e;
                    const float ya = __builtin_fmaf(xa[e], cos_t[j], -xb[e] * sin_t[j]);
                    const float yb = __builtin_fmaf(xa[e], sin_t[j], xb[e] * cos_t[j]);
                    xa[e] = ya;
                    xb[e] = yb;
                }
                dst[c] = Elem<T>::pack(xa);
                dst[c + CPR / 2] = Elem<T>::pack(xb);
            }
        } else {
            const int r = i - nq - nk;
            const int h = r / CPR, c = r - (r / CPR) * CPR;
            ((u32x4 *)a.v_cache)[((blk * hkv + h) * a.block_size + off) * CPR + c] =
                ((const u32x4 *)a.v)[(tok * hkv + h) * CPR + c];
        }
    }
}

template <typename T, int D>
hipError_t launch_layout(const RopeArgs &a, hipStream_t stream)
{
    if (a.adjacent_pairs)
        hipLaunchKernelGGL((rope_kv_cache_write_kernel<T, D, true>), dim3((unsigned)a.num_tokens),
                           dim3(kRopeThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((rope_kv_cache_write_kernel<T, D, false>), dim3((unsigned)a.num_tokens),
                           dim3(kRopeThreads), 0, stream, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_rope_dim(const RopeArgs &a, hipStream_t stream)
{
    switch (a.head_dim) {
    case 64: return launch_layout<T, 64>(a, stream);
    case 128: return launch_layout<T, 128>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_rope_kv_cache_write(const RopeArgs &a, hipStream_t stream)
{
    switch (a.dtype) {
    case kDtypeF32: return launch_rope_dim<float>(a, stream);
    case kDtypeF16: return launch_rope_dim<_Float16>(a, stream);
    case kDtypeBF16: return launch_rope_dim<__bf16>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace photon
