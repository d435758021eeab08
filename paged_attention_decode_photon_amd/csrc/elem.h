// Storage element types of the HIP kernels: widening of 16-byte chunks to
// fp32 and narrowing back (round to nearest even).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace photon {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

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
    __device__ static u32x4 pack(const float (&f)[4])
    {
        return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                     __float_as_uint(f[3])};
    }
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
    __device__ static u32x4 pack(const float (&f)[8])
    {
        u32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            half2_t h;
            h[0] = (_Float16)f[2 * i];
            h[1] = (_Float16)f[2 * i + 1];
            const uint32_t word = __builtin_bit_cast(uint32_t, h);
            v[i] = word;
        }
        return v;
    }
    __device__ static _Float16 from_float(float x) { return (_Float16)x; }
    __device__ static uint32_t pack2(float lo, float hi)
    {
        half2_t h;
        h[0] = (_Float16)lo;
        h[1] = (_Float16)hi;
        return __builtin_bit_cast(uint32_t, h);
    }
    // acc + x.lo * y.lo + x.hi * y.hi over two packed elements, in fp32
    // (v_dot2_f32_f16; the products of two halves are exact in fp32).
    __device__ static float dot2(uint32_t x, uint32_t y, float acc)
    {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, x),
                                      __builtin_bit_cast(half2_t, y), acc, false);
    }
};

// bfloat16 is the upper half of a binary32, so widening is a shift; narrowing
// rounds to nearest even (v_cvt_pk_bf16_f32 on gfx950).
template <>
struct Elem<__bf16> {
    __device__ static void unpack(const u32x4 &v, float (&f)[8])
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t word = v[i];
            f[2 * i] = __uint_as_float(word << 16);
            f[2 * i + 1] = __uint_as_float(word & 0xffff0000u);
        }
    }
    __device__ static u32x4 pack(const float (&f)[8])
    {
        u32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            bf162_t h;
            h[0] = (__bf16)f[2 * i];
            h[1] = (__bf16)f[2 * i + 1];
            const uint32_t word = __builtin_bit_cast(uint32_t, h);
            v[i] = word;
        }
        return v;
    }
    __device__ static __bf16 from_float(float x) { return (__bf16)x; }
    __device__ static uint32_t pack2(float lo, float hi)
    {
        bf162_t h;
        h[0] = (__bf16)lo;
        h[1] = (__bf16)hi;
        return __builtin_bit_cast(uint32_t, h);
    }
    // acc + x.lo * y.lo + x.hi * y.hi in fp32 (v_dot2_f32_bf16).
    __device__ static float dot2(uint32_t x, uint32_t y, float acc)
    {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, x),
                                               __builtin_bit_cast(bf162_t, y), acc, false);
    }
};

// Store N consecutive outputs of type O (N a power of two up to 8; dst
// aligned to N * sizeof(O) bytes, at most 16).
template <typename O, int N>
__device__ __forceinline__ void store_out_n(O *dst, const float (&v)[N])
{
    if constexpr (sizeof(O) == 4) {
        if constexpr (N >= 4) {
#pragma unroll
            for (int k = 0; k < N / 4; ++k)
                *reinterpret_cast<u32x4 *>(dst + 4 * k) =
                    u32x4{__float_as_uint(v[4 * k]), __float_as_uint(v[4 * k + 1]),
                          __float_as_uint(v[4 * k + 2]), __float_as_uint(v[4 * k + 3])};
        } else if constexpr (N == 2) {
            *reinterpret_cast<u32x2 *>(dst) = u32x2{__float_as_uint(v[0]), __float_as_uint(v[1])};
        } else {
            *dst = v[0];
        }
    } else if constexpr (N == 8) {
        *reinterpret_cast<u32x4 *>(dst) = Elem<O>::pack(v);
    } else if constexpr (N == 4) {
        *reinterpret_cast<u32x2 *>(dst) =
            u32x2{Elem<O>::pack2(v[0], v[1]), Elem<O>::pack2(v[2], v[3])};
    } else if constexpr (N == 2) {
        *reinterpret_cast<uint32_t *>(dst) = Elem<O>::pack2(v[0], v[1]);
    } else {
        *dst = Elem<O>::from_float(v[0]);
    }
}

}  // namespace photon
