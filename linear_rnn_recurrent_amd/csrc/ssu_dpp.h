// Cross-lane sums with DPP (data-parallel primitives): no LDS traffic.
#pragma once

#include <hip/hip_runtime.h>

namespace ssu {

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float a)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, a),
                                                                CTRL, 0xF, 0xF, false));
}

// dpp_f32 with a fill value: lanes whose source lies outside their row of 16
// get `fill` (row shifts leave the first lanes of a row without a source).
template <int CTRL>
__device__ __forceinline__ float dpp_f32_fill(float fill, float a)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, fill),
                                                                __builtin_bit_cast(int, a), CTRL,
                                                                0xF, 0xF, false));
}

// Inclusive running product along each row of 16 lanes (lane i of a row gets
// the product of lanes 0..i): four row shifts, Hillis-Steele.
__device__ __forceinline__ float row_prefix_prod16(float v)
{
    v *= dpp_f32_fill<0x111>(1.0f, v);  // row_shr:1
    v *= dpp_f32_fill<0x112>(1.0f, v);  // row_shr:2
    v *= dpp_f32_fill<0x114>(1.0f, v);  // row_shr:4
    v *= dpp_f32_fill<0x118>(1.0f, v);  // row_shr:8
    return v;
}

// Inclusive prefix and suffix sums along each row of 16 lanes (row shifts
// with zero fill, Hillis-Steele).
__device__ __forceinline__ float row_prefix_sum16(float v)
{
    v += dpp_f32_fill<0x111>(0.0f, v);  // row_shr:1
    v += dpp_f32_fill<0x112>(0.0f, v);  // row_shr:2
    v += dpp_f32_fill<0x114>(0.0f, v);  // row_shr:4
    v += dpp_f32_fill<0x118>(0.0f, v);  // row_shr:8
    return v;
}
__device__ __forceinline__ float row_suffix_sum16(float v)
{
    v += dpp_f32_fill<0x101>(0.0f, v);  // row_shl:1
    v += dpp_f32_fill<0x102>(0.0f, v);  // row_shl:2
    v += dpp_f32_fill<0x104>(0.0f, v);  // row_shl:4
    v += dpp_f32_fill<0x108>(0.0f, v);  // row_shl:8
    return v;
}

// Sum over aligned groups of W lanes (W = 4, 8 or 16): quad permutations, then
// the half-row and row mirrors; every lane of a group gets the group's sum.
template <int W>
__device__ __forceinline__ float row_group_sum(float v)
{
    v += dpp_f32<0xB1>(v);  // quad_perm [1,0,3,2]
    v += dpp_f32<0x4E>(v);  // quad_perm [2,3,0,1]
    if constexpr (W >= 8)
        v += dpp_f32<0x141>(v);  // row_half_mirror: lane i <- lane 7 - i of its half row
    if constexpr (W >= 16)
        v += dpp_f32<0x140>(v);  // row_mirror: lane i <- lane 15 - i
    return v;
}

// Sum over the whole 64-lane wave, returned wave-uniform: row sums by DPP,
// then the four rows' sums read from lanes 0, 16, 32 and 48.
__device__ __forceinline__ float wave_sum(float v)
{
    v = row_group_sum<16>(v);
    const int u = __builtin_bit_cast(int, v);
    return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 0)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 16))) +
           (__builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 32)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 48)));
}

}  // namespace ssu
