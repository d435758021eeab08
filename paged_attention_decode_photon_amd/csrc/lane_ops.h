// Cross-lane primitives for wave64 on gfx950 (CDNA4).
//
// Pairings used by the decode kernels, each one instruction:
//   xor 1, xor 2   DPP quad_perm          (inside 4-lane quads)
//   xor 7          DPP row_half_mirror    (lane i <-> 7-i inside 8-lane halves)
//   xor 8          DPP row_ror:8          (inside 16-lane rows)
//   xor 4, xor 16  ds_swizzle bit mode    (inside 32-lane halves, no LDS memory)
// Symmetric all-reductions across 16- and 32-lane halves use the gfx950
// v_permlane16_swap / v_permlane32_swap pair exchange.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace photon {

// DPP control words (GCN3+ encoding).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowRor8 = 0x128;

// ds_swizzle bit mode: and_mask = 0x1f, or_mask = 0, xor_mask in bits 14:10.
constexpr int swizzle_xor(int m) { return 0x1f | (m << 10); }

template <int kCtrl>
__device__ __forceinline__ float dpp(float v)
{
    return __builtin_amdgcn_update_dpp(0.0f, v, kCtrl, 0xf, 0xf, true);
}

// Value held by lane (lane ^ M) for the pairings listed above.
template <int M>
__device__ __forceinline__ float xor_partner(float v)
{
    if constexpr (M == 1) {
        return dpp<kDppQuadXor1>(v);
    } else if constexpr (M == 2) {
        return dpp<kDppQuadXor2>(v);
    } else if constexpr (M == 7) {
        return dpp<kDppRowHalfMirror>(v);
    } else if constexpr (M == 8) {
        return dpp<kDppRowRor8>(v);
    } else if constexpr (M == 4 || M == 16) {
        return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), swizzle_xor(M)));
    } else {
        static_assert(M == 1, "unsupported lane pairing");
        return v;
    }
}

struct OpSum {
    __device__ static float apply(float a, float b) { return a + b; }
};
struct OpMax {
    __device__ static float apply(float a, float b) { return fmaxf(a, b); }
};

// op(v, value of lane ^ M) in every lane.
template <int M, class Op>
__device__ __forceinline__ float allreduce_pair(float v)
{
    if constexpr (M == 32) {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        return Op::apply(__uint_as_float(r[0]), __uint_as_float(r[1]));
    } else if constexpr (M == 16) {
        auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        return Op::apply(__uint_as_float(r[0]), __uint_as_float(r[1]));
    } else {
        return Op::apply(v, xor_partner<M>(v));
    }
}

// op over the lanes that differ from this one only in lane-index bits [LO, HI).
template <int LO, int HI, class Op>
__device__ __forceinline__ float allreduce_bits(float v)
{
    if constexpr (LO < HI) {
        v = allreduce_pair<(1 << LO), Op>(v);
        return allreduce_bits<LO + 1, HI, Op>(v);
    } else {
        return v;
    }
}

__device__ __forceinline__ float read_lane(float v, int lane)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// DPP controls of the wave-wide scan below (gfx9-family encodings).
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142;  // lane 15 of each row -> the next row
constexpr int kDppRowBcast31 = 0x143;  // lane 31 -> rows 2 and 3

// Inclusive prefix sum over the 64 lanes of a wave.  Inside each 16-lane
// row a log-step scan with row_shr 1, 2, 4, 8 (a lane with no source in its
// row adds 0); then row_bcast:15 adds the total of row r to row r + 1 (rows
// 1 and 3 written), and row_bcast:31 adds the total of rows 0-1 to rows 2
// and 3.  Six DPP adds and no LDS traffic, where a shuffle-based scan costs
// six serialised LDS permutes.
__device__ __forceinline__ int wave_inclusive_sum(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr1, 0xf, 0xf, true);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr2, 0xf, 0xf, true);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr4, 0xf, 0xf, true);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr8, 0xf, 0xf, true);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast15, 0xa, 0xf, false);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast31, 0xc, 0xf, false);
    return v;
}

}  // namespace photon
